"""Page-pool packing (host logic, no GPU): page sizes against the pages' page
formula, bucket packing, arena layout, and the allocator against a plain
Python model of the same policy under random operation sequences."""

import ctypes
import json
import os
import random

import pytest

import decode_attention_compressed_amd as hca
from oracle import paging

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
STACK = [(4, 512, "fp8"), (128, 512, "fp8"), (1, 512, "fp8"), (4, 128, "fp4")]  # c4a, c128a, window, indexer


def test_page_bytes_follow_the_page_formula():
    # [V4-vLLM] 3.1.3: page size = block size x compress ratio x bytes per element
    for m in (1, 2, 4, 64, 128, 256):
        for d in (64, 128, 512, 5120):
            assert hca.page_bytes(m, d, "bf16") == (paging.page_bytes(m, d, 2), 0)
            assert hca.page_bytes(m, d, "fp8") == (paging.page_bytes(m, d, 1), 4)
            if d % 32 == 0:
                assert hca.page_bytes(m, d, "fp4") == (paging.page_bytes(m, d, 0.5), (256 // m) * (d // 32))
    gold = json.load(open(os.path.join(GOLDEN, "pages_worked_numbers.json")))
    for e in gold["page_bytes_bf16_5120"]:
        assert hca.page_bytes(e["m"], 5120, "bf16")[0] == e["bytes"], e["cite"]
    with pytest.raises(hca.HcaError):
        hca.page_bytes(3, 512, "fp8")
    with pytest.raises(hca.HcaError):
        hca.page_bytes(4, 100, "fp4")


def test_buckets_and_arena_layout():
    kinds = STACK + [(4, 128, "fp8"), (1, 128, "fp8"), (2, 256, "fp8")]  # the last two share the c4a page size
    pool = hca.PagePool(kinds, [7, 5, 3, 11, 13])
    assert pool.kind_bucket == [0, 1, 2, 3, 4, 0, 0] and pool.n_buckets == 5
    caps = [7, 5, 3, 11, 13]
    regions = []
    for b in range(5):
        k = pool.kind_bucket.index(b)
        cb, sb = hca.page_bytes(*kinds[k])
        free, cached, held, co, so = pool.stats(b)
        assert (free, cached, held) == (caps[b], 0, 0)
        assert co % 256 == 0 and so % 256 == 0
        regions += [(co, co + cb * caps[b]), (so, so + sb * caps[b])]
    regions.sort()
    for (a0, a1), (b0, b1) in zip(regions, regions[1:]):
        assert a1 <= b0  # no overlap
    assert regions[-1][1] <= pool.arena_bytes


class Model:
    """The allocator's policy, plainly: a free stack (page 0 on top at start),
    reference counts, keys, and released keyed pages cached oldest first."""

    def __init__(self, cap):
        self.free = list(range(cap - 1, -1, -1))
        self.refs = [0] * cap
        self.key = {}
        self.by_key = {}
        self.cached = []

    def alloc(self, n):
        if n > len(self.free) + len(self.cached):
            return None
        out = []
        for _ in range(n):
            if not self.free:
                p = self.cached.pop(0)
                del self.by_key[self.key.pop(p)]
                self.free.append(p)
            p = self.free.pop()
            self.refs[p] = 1
            out.append(p)
        return out

    def release(self, pages):
        for p in pages:
            self.refs[p] -= 1
            if self.refs[p] == 0:
                (self.cached if p in self.key else self.free).append(p)

    def lookup(self, key):
        p = self.by_key.get(key, -1)
        if p >= 0:
            if p in self.cached:
                self.cached.remove(p)
            self.refs[p] += 1
        return p


def test_allocator_matches_model_random_ops():
    rnd = random.Random(5)
    for trial in range(20):
        cap = rnd.choice([1, 3, 16, 64])
        pool = hca.PagePool([(4, 128, "fp8")], [cap])
        mod = Model(cap)
        held = []  # references we hold, one entry per reference
        for step in range(300):
            op = rnd.random()
            if op < 0.3:
                n = rnd.randint(0, 4)
                want = mod.alloc(n)
                if want is None:
                    with pytest.raises(hca.HcaError):
                        pool.alloc(0, n)
                else:
                    assert pool.alloc(0, n) == want
                    held += want
            elif op < 0.55 and held:
                k = rnd.randint(1, min(3, len(held)))
                rel = [held.pop(rnd.randrange(len(held))) for _ in range(k)]
                pool.release(0, rel)
                mod.release(rel)
            elif op < 0.65 and held:
                p = rnd.choice(held)
                pool.share(0, [p])
                mod.refs[p] += 1
                held.append(p)
            elif op < 0.8 and held:
                p = rnd.choice(held)
                key = rnd.randint(0, 40)
                other = mod.by_key.get(key)
                if other is not None and other != p:
                    with pytest.raises(hca.HcaError):
                        pool.publish(0, p, key)
                else:
                    pool.publish(0, p, key)
                    if p in mod.key and mod.key[p] != key:
                        del mod.by_key[mod.key[p]]
                    mod.key[p] = key
                    mod.by_key[key] = p
            else:
                key = rnd.randint(0, 40)
                want = mod.lookup(key)
                assert pool.lookup(0, key) == want
                if want >= 0:
                    held.append(want)
            free, cached, nheld, _, _ = pool.stats(0)
            assert (free, cached) == (len(mod.free), len(mod.cached)), (trial, step)
            assert nheld == cap - free - cached == sum(1 for r in mod.refs if r > 0)


def test_invalid_calls_change_nothing():
    pool = hca.PagePool([(4, 128, "fp8")], [4])
    a = pool.alloc(0, 2)
    before = pool.stats(0)
    L = hca.lib()
    arr = (ctypes.c_int32 * 3)(a[0], 9, a[1])
    assert L.hca_pool_release(pool._h, 0, arr, 3) == 1  # page 9 does not exist
    arr = (ctypes.c_int32 * 2)(a[0], a[0])
    assert L.hca_pool_release(pool._h, 0, arr, 2) == 1  # released twice, held once
    free = [p for p in range(4) if p not in a]
    arr = (ctypes.c_int32 * 1)(free[0])
    assert L.hca_pool_share(pool._h, 0, arr, 1) == 1  # a free page cannot be shared
    assert L.hca_pool_publish(pool._h, 0, free[0], 7) == 1  # nor published
    assert L.hca_pool_alloc(pool._h, 1, 1, arr) == 1  # no bucket 1
    assert L.hca_pool_alloc(pool._h, 0, -1, arr) == 1
    assert pool.stats(0) == before
    kinds = (hca.CKvKind * 1)(hca.CKvKind(3, 128, 1))
    out = ctypes.c_void_p(0)
    nbytes = ctypes.c_size_t(0)
    caps = (ctypes.c_int32 * 1)(4)
    assert L.hca_pool_create(kinds, 1, caps, ctypes.byref(nbytes), ctypes.byref(out)) == 1 and not out.value
    pc = hca.CPagedCache()
    assert L.hca_pool_view(pool._h, 0, ctypes.c_void_p(0x1010), ctypes.byref(pc)) == 1  # arena not 256-aligned
    assert L.hca_pool_view(pool._h, 0, ctypes.c_void_p(0x1000), ctypes.byref(pc)) == 0
    assert pc.num_pages == 4 and pc.epp == 64 and pc.dim == 128 and pc.dtype == 1
