"""CPU checks of libhca: it loads, exports every declared symbol, validates
arguments on the host, and its encoders (the kernels' own source, compiled for
the host) round exactly like the oracle's codecs."""

import ctypes
import os
import re

import numpy as np
import pytest

import decode_attention_compressed_amd as hca
from oracle import codecs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(hca.LIB_PATH), reason="libhca.so not built")


def _declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)) - {"defined"}


def test_every_declared_symbol_is_exported():
    L = hca.lib()
    names = _declared("hca.h") | _declared("hca_testing.h")
    assert {"kv_compress", "kv_quantize_page", "indexer_topk", "paged_hybrid_decode", "kv_gather"} <= names
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(hca.EXPORTS)
    assert hca.version().startswith("hca ")
    for s in range(5):
        assert L.hca_status_string(s)


def test_debug_build_exports_every_declared_symbol():
    # libhca_debug.so: the same kernels with index checks (-DHCA_DEBUG); loaded
    # beside the release library, no device call made
    path = os.path.join(os.path.dirname(hca.__file__), "libhca_debug.so")
    assert os.path.exists(path), "build it with `python -m decode_attention_compressed_amd.build --debug`"
    D = ctypes.CDLL(path)
    for n in _declared("hca.h") | _declared("hca_testing.h"):
        assert hasattr(D, n), n
    D.hca_version.restype = ctypes.c_char_p
    assert D.hca_version().decode().endswith(" debug")


def test_release_build_debug_status_is_unsupported():
    # the release build records nothing: HCA_ERR_UNSUPPORTED, bits 0, no device call
    assert hca.debug_status() == (2, 0)
    assert hca.lib().hca_debug_status(None) == 2


def _host_encode(fn, x, out_dtype):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape, dtype=out_dtype)
    rc = fn(x.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p), x.size)
    assert rc == 0
    return out


def _probe_values(table, n_random, rng):
    pos = table[np.isfinite(table) & (table >= 0)]
    pos = np.unique(pos)
    mids = (pos[:-1] + pos[1:]) / 2
    v = np.concatenate([pos, mids]).astype(np.float32)
    near = np.concatenate([np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(-np.inf))])
    extra = np.array([0.0, 1e-30, 1e30, 448.0, 464.0, 480.0, 6.0, 6.5, 7.0, 2.0 ** -10, 2.0 ** -9], np.float32)
    rnd = np.concatenate([rng.normal(0, 1, n_random), rng.normal(0, 100, n_random // 4),
                          np.ldexp(rng.uniform(0, 1, n_random // 4), -8)]).astype(np.float32)
    x = np.concatenate([v, near, extra, rnd])
    return np.concatenate([x, -x])


def test_host_e4m3_encoder_matches_oracle():
    rng = np.random.default_rng(21)
    x = _probe_values(codecs.E4M3_TABLE, 2_000_000, rng)
    # every binary32 pattern with the 12 low mantissa bits clear, over the whole finite range
    sweep = (np.arange(0, 0x7F800000 >> 12, dtype=np.uint32) << 12).view(np.float32)
    x = np.concatenate([x, sweep, -sweep])
    got = _host_encode(hca.lib().hca_host_e4m3_encode, x, np.uint8)
    assert np.array_equal(got, codecs.e4m3_encode(x))


def test_host_e2m1_encoder_matches_oracle():
    rng = np.random.default_rng(22)
    x = _probe_values(codecs.E2M1_TABLE, 1_000_000, rng)
    sweep = (np.arange(0, 0x7F800000 >> 12, dtype=np.uint32) << 12).view(np.float32)
    x = np.concatenate([x, sweep, -sweep])
    got = _host_encode(hca.lib().hca_host_e2m1_encode, x, np.uint8)
    assert np.array_equal(got, codecs.e2m1_encode(x))


def test_host_bf16_encoder_matches_oracle():
    rng = np.random.default_rng(23)
    x = np.concatenate([rng.normal(0, 10, 1_000_000), rng.normal(0, 1e-3, 100_000)]).astype(np.float32)
    u = ((rng.integers(0, 2, 50000) << 31) | (rng.integers(1, 250, 50000) << 23) |
         (rng.integers(0, 128, 50000) << 16) | 0x8000).astype(np.uint32)
    x = np.concatenate([x, u.view(np.float32)])
    got = _host_encode(hca.lib().hca_host_bf16_encode, x, np.uint16)
    assert np.array_equal(got, codecs.bf16_encode(x))


# ----------------------------------------------------------------- host validation
FAKE = ctypes.c_void_p(0x1000)  # any non-null, 256-byte aligned address: nothing is launched on failure


def _cache(dtype=1, epp=64, dim=128, pages=4, codes=FAKE, scales=FAKE):
    return hca.CPagedCache(codes.value if codes else 0, scales.value if scales else 0, pages, epp, dim, dtype)


def test_validation_kv_compress():
    L = hca.lib()
    ok = dict(x=FAKE, xs=4096 * 8, z=FAKE, zs=4096, beta=FAKE, pos0=FAKE, ntok=FAKE, B=2, mx=4096, d=128, m=4,
              ov=0, theta=1e6, gam=None, eps=1e-6, out=FAKE, os=1024 * 128)

    def call(**kw):
        a = dict(ok, **kw)
        return L.kv_compress(a["x"], a["xs"], a["z"], a["zs"], a["beta"], a["pos0"], a["ntok"], a["B"], a["mx"],
                             a["d"], a["m"], a["ov"], a["theta"], a["gam"], a["eps"], a["out"], a["os"], None)

    assert call(m=3) == 1 and call(m=512) == 1 and call(m=0) == 1
    assert call(d=12) == 1 and call(d=4096) == 2
    assert call(theta=0.0) == 1 and call(theta=float("nan")) == 1
    assert call(x=None) == 1 and call(out=None) == 1 and call(ntok=None) == 1
    assert call(xs=100) == 1 and call(os=16) == 1
    assert call(B=-1) == 1
    assert call(B=0) == 0 and call(mx=0) == 0  # nothing to do, nothing launched
    # normalisation: an aligned gain vector and a finite eps > 0
    assert call(gam=FAKE, eps=0.0) == 1 and call(gam=FAKE, eps=float("inf")) == 1
    assert call(gam=ctypes.c_void_p(0x1004)) == 1
    assert call(gam=FAKE, B=0) == 0 and call(gam=None, eps=0.0, B=0) == 0
    # overlapping windows: 0 .. m, and only for groups of at most 16
    assert call(ov=-1) == 1 and call(ov=5) == 1 and call(m=32, ov=4) == 2
    assert call(ov=4, B=0) == 0 and call(m=16, ov=16, B=0) == 0


def test_validation_kv_prefill_pages():
    L = hca.lib()
    ok = dict(x=FAKE, xs=4096 * 128, z=FAKE, zs=4096, beta=FAKE, pos0=FAKE, ntok=FAKE, B=2, mx=4096, m=4, ov=0,
              theta=1e6, gam=None, eps=1e-6, bt=FAKE, bts=16, dst=_cache())

    def call(**kw):
        a = dict(ok, **kw)
        return L.kv_prefill_pages(a["x"], a["xs"], a["z"], a["zs"], a["beta"], a["pos0"], a["ntok"], a["B"], a["mx"],
                                  a["m"], a["ov"], a["theta"], a["gam"], a["eps"], a["bt"], a["bts"], a["dst"], None)

    assert call(B=0) == 0 and call(mx=0) == 0  # nothing to do, nothing launched
    assert call(m=3) == 1 and call(m=8) == 1  # m = 8 does not match the pool's 64 entries a page
    assert call(bts=0) == 1 and call(B=-1) == 1
    assert call(theta=0.0) == 1 and call(gam=FAKE, eps=0.0) == 1
    assert call(ov=5) == 1 and call(ov=4, B=0) == 0
    assert call(x=None) == 1 and call(bt=None) == 1 and call(ntok=None) == 1
    assert call(xs=100) == 1
    # page formats the fused kernels write, and pages that fit one block
    assert call(dst=_cache(dtype=2)) == 2  # fp4
    assert call(m=1, dst=_cache(epp=256, dim=512)) == 2  # 256 rows of 512 dims
    assert call(m=4, dst=_cache(epp=64, dim=512), B=0) == 0
    assert call(m=128, dst=_cache(epp=2, dim=2048), B=0) == 0 and call(m=32, dst=_cache(epp=8, dim=2048)) == 2


def test_validation_kv_compress_insert():
    L = hca.lib()
    ok = dict(x=FAKE, xs=4 * 128, z=FAKE, zs=4, beta=FAKE, pos0=FAKE, ntok=FAKE, B=2, m=4, ov=0, theta=1e6,
              gam=None, eps=1e-6, st=FAKE, ss=64 * 128, e0=FAKE, bt=FAKE, bts=16, dst=_cache(), app=0, fs=None,
              fss=0)

    def call(**kw):
        a = dict(ok, **kw)
        return L.kv_compress_insert(a["x"], a["xs"], a["z"], a["zs"], a["beta"], a["pos0"], a["ntok"], a["B"],
                                    a["m"], a["ov"], a["theta"], a["gam"], a["eps"], a["st"], a["ss"], a["e0"],
                                    a["bt"], a["bts"], a["dst"], a["app"], a["fs"], a["fss"], None)

    assert call(m=3) == 1 and call(m=8) == 1  # the pool's epp must be 256 / m
    assert call(dst=_cache(dim=4096)) == 2
    assert call(dst=_cache(dtype=7)) == 1 and call(dst=_cache(scales=None)) == 1
    assert call(app=2) == 1 and call(bts=0) == 1 and call(theta=0.0) == 1
    assert call(x=None) == 1 and call(st=None) == 1 and call(e0=None) == 1 and call(bt=None) == 1
    assert call(xs=100) == 1 and call(ss=16) == 1 and call(zs=3) == 1
    assert call(B=-1) == 1
    assert call(gam=FAKE, eps=-1.0) == 1 and call(gam=ctypes.c_void_p(0x1008)) == 1
    assert call(ov=8) == 1 and call(ov=-2) == 1
    # update states: aligned, a page header of 4 floats, + two fold states of 4 + d floats when m > 16
    c128 = dict(m=128, xs=128 * 128, zs=128, ss=2 * 128, dst=_cache(epp=2))
    assert call(fs=ctypes.c_void_p(0x1004), fss=4 + 2 * 132, **c128) == 1
    assert call(fs=FAKE, fss=2 * 132, **c128) == 1 and call(fs=FAKE, fss=4 + 2 * 132 + 2, **c128) == 1
    assert call(fs=FAKE, fss=4 + 2 * 132, B=0, **c128) == 0
    assert call(fs=FAKE, fss=2) == 1 and call(fs=ctypes.c_void_p(0x1004), fss=4) == 1  # m = 4: the header
    assert call(fs=FAKE, fss=4, B=0) == 0
    assert call(B=0) == 0 and call(gam=FAKE, B=0) == 0  # nothing to do, nothing launched


def test_validation_kv_compress_insert_jobs():
    L = hca.lib()

    def job(**kw):
        a = dict(x=FAKE.value, xs=4 * 128, z=FAKE.value, zs=4, beta=FAKE.value, pos0=FAKE.value, ntok=FAKE.value,
                 m=4, ov=0, theta=1e6, gam=None, eps=1e-6, st=FAKE.value, ss=64 * 128, e0=FAKE.value,
                 bt=FAKE.value, bts=16, dst=_cache(), app=0)
        a.update(kw)
        return hca.CInsertJob(a["x"], a["xs"], a["z"], a["zs"], a["beta"], a["pos0"], a["ntok"], a["m"], a["ov"],
                              a["theta"], a["gam"], a["eps"], a["st"], a["ss"], a["e0"], a["bt"], a["bts"], a["dst"], a["app"])

    def call(jobs, B=2):
        arr = (hca.CInsertJob * max(len(jobs), 1))(*jobs)
        return L.kv_compress_insert_jobs(arr, len(jobs), B, None)

    assert call([job(), job(m=3)]) == 1  # every job is checked before anything is launched
    assert call([job(), job(dst=_cache(dim=4096))]) == 2
    assert call([job()] * 5) == 2  # at most four jobs
    assert call([job(x=None, z=None, beta=None, ntok=None, st=None)]) == 1  # no fold, but a staging row is needed
    assert call([job()], B=-1) == 1
    assert call([job(), job(app=3)]) == 1
    assert call([], B=2) == 0 and call([job()], B=0) == 0  # nothing to do, nothing launched
    assert call([job(), job(gam=FAKE.value, eps=0.0)]) == 1
    # without a fold the norm and overlap arguments are not used
    assert call([job(x=None, gam=FAKE.value, eps=0.0, ov=9)], B=0) == 0
    assert call([job(), job(ov=5)]) == 1


def test_validation_quantize_and_gather():
    L = hca.lib()
    assert L.kv_quantize_page(FAKE, 8192, FAKE, FAKE, 2, 64, FAKE, 16, _cache(dtype=7), None, 0, None) == 1
    assert L.kv_quantize_page(FAKE, 8192, FAKE, FAKE, 2, 64, FAKE, 16, _cache(epp=3), None, 0, None) == 1
    assert L.kv_quantize_page(FAKE, 8192, FAKE, FAKE, 2, 64, FAKE, 16, _cache(dtype=2, dim=48), None, 0, None) == 1
    assert L.kv_quantize_page(FAKE, 8192, FAKE, FAKE, 2, 64, FAKE, 16, _cache(scales=None), None, 0, None) == 1
    assert L.kv_quantize_page(None, 8192, FAKE, FAKE, 2, 64, FAKE, 16, _cache(), None, 0, None) == 1
    assert L.kv_quantize_page(FAKE, 8192, FAKE, FAKE, 2, 64, FAKE, 0, _cache(), None, 0, None) == 1
    assert L.kv_quantize_page(FAKE, 8192, FAKE, FAKE, 0, 64, FAKE, 16, _cache(), None, 0, None) == 0
    # a workspace smaller than kv_quantize_page_workspace(...) is rejected before any launch
    need = L.kv_quantize_page_workspace(2, 64, _cache())
    assert need > 0 and need % 256 == 0
    assert L.kv_quantize_page(FAKE, 8192, FAKE, FAKE, 2, 64, FAKE, 16, _cache(), FAKE, need - 1, None) == 1
    assert L.kv_quantize_page_workspace(2, 64, _cache(dtype=2, dim=64)) == 0  # fp4: no workspace
    assert L.kv_gather(_cache(), FAKE, 1, FAKE, 2, 65, FAKE, FAKE, None) == 1  # table too narrow for 65 rows
    assert L.kv_gather(_cache(), FAKE, 2, FAKE, 2, 65, FAKE, None, None) == 1  # fp8 needs scales out
    assert L.kv_gather(_cache(), FAKE, 2, FAKE, 0, 65, FAKE, FAKE, None) == 0


def test_validation_indexer_and_attention():
    L = hca.lib()
    ws_need = L.indexer_topk_workspace(2, 4096, 4, 256)
    assert ws_need > 0 and L.indexer_topk_workspace(2, 4096, 3, 256) == 0

    def idx(**kw):
        a = dict(q=FAKE, w=FAKE, HI=16, keys=_cache(dtype=1, epp=64, dim=128), bt=FAKE, bts=16, lens=FAKE, B=2,
                 L=4096, m=4, k=256, out=FAKE, n=FAKE, ws=FAKE, wsb=ws_need)
        a.update(kw)
        return L.indexer_topk(a["q"], a["w"], a["HI"], a["keys"], a["bt"], a["bts"], a["lens"], a["B"], a["L"],
                              a["m"], a["k"], a["out"], a["n"], a["ws"], a["wsb"], None)

    assert idx(HI=17) == 2 and idx(HI=0) == 1
    assert idx(k=0) == 1 and idx(k=9000) == 2
    assert idx(keys=_cache(dtype=1, epp=2, dim=128)) == 1  # epp must be 256/m
    assert idx(keys=_cache(dtype=1, epp=64, dim=96)) == 2
    assert idx(bts=15) == 1  # 15*256 < 4096
    assert idx(wsb=ws_need - 1) == 3 and idx(ws=None) == 3
    assert idx(out=None) == 1
    assert idx(B=0) == 0

    ws_att = L.paged_hybrid_decode_workspace(2, 64, 512, 4096, 4, 128, 256)
    assert ws_att > 0

    def att(**kw):
        a = dict(q=FAKE, H=64, kv=_cache(dtype=1, epp=64, dim=512), bt=FAKE, bts=16,
                 win=_cache(dtype=1, epp=256, dim=512), wbt=FAKE, wbts=16, lens=FAKE, B=2, L=4096, m=4, W=128,
                 sel=FAKE, seln=FAKE, k=256, scale=0.04, theta=1e6, out=FAKE, lse=None, o8=None, o8s=None, ws=FAKE,
                 wsb=ws_att)
        a.update(kw)
        return L.paged_hybrid_decode(a["q"], a["H"], a["kv"], a["bt"], a["bts"], a["win"], a["wbt"], a["wbts"],
                                     a["lens"], a["B"], a["L"], a["m"], a["W"], a["sel"], a["seln"], a["k"],
                                     a["scale"], a["theta"], a["out"], a["lse"], a["o8"], a["o8s"], a["ws"], a["wsb"],
                                     None)

    assert att(H=129) == 2 and att(H=0) == 1
    assert att(kv=_cache(dtype=1, epp=64, dim=384)) == 2
    assert att(kv=_cache(dtype=2, epp=64, dim=512)) == 2
    assert att(W=300) == 1 and att(win=_cache(dtype=1, epp=64, dim=512)) == 1
    assert att(win=_cache(dtype=1, epp=256, dim=256)) == 1
    assert att(seln=None) == 1 and att(k=0) == 1
    assert att(scale=float("inf")) == 1
    assert att(wsb=ws_att - 1) == 3
    assert att(m=5) == 1
    # the fp8 output needs its scales and 2-byte alignment; one of the two outputs is required
    assert att(out=None) == 1 and att(o8=FAKE) == 1 and att(out=None, o8=ctypes.c_void_p(0x1001), o8s=FAKE) == 1
    assert att(out=None, o8=FAKE, o8s=FAKE, wsb=ws_att - 1) == 3  # valid outputs; only the workspace is short
    assert att(B=0) == 0


def test_validation_indexer_topk_with_updates():
    L = hca.lib()
    ws_need = L.indexer_topk_workspace(2, 4096, 4, 256)
    OTHER = ctypes.c_void_p(0x2000)

    def job(dst):
        return hca.CInsertJob(FAKE.value, 4 * 128, FAKE.value, 4, FAKE.value, FAKE.value, FAKE.value, 4, 0, 1e6, None,
                              1e-6, FAKE.value, 64 * 128, FAKE.value, FAKE.value, 16, dst, 0)

    def call(jobs, B=2, HI=16, keys=None):
        keys = keys or _cache(dtype=2, epp=64, dim=128, codes=FAKE)
        arr = (hca.CInsertJob * max(len(jobs), 1))(*jobs)
        return L.indexer_topk_with_updates(FAKE, FAKE, HI, keys, FAKE, 16, FAKE, B, 4096, 4, 256, FAKE, FAKE, FAKE,
                                           ws_need, arr, len(jobs), None)

    ok = job(_cache(dtype=1, epp=64, dim=128, codes=OTHER))
    assert call([ok], B=0) == 0  # valid, nothing to do
    # a job writing the keys being scored is accepted (it runs before the score pass)
    assert call([ok, job(_cache(dtype=1, epp=64, dim=128, codes=FAKE))], B=0) == 0
    assert call([ok] * 5, B=0) == 2  # at most four jobs
    assert call([ok, job(_cache(dtype=1, epp=3, dim=128, codes=OTHER))]) == 1  # every job checked, nothing launched
    assert call([ok], HI=17) == 2 and call([ok], B=-1) == 1  # the indexer arguments as for indexer_topk
    assert call([], B=0) == 0
