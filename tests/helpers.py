"""Shared helpers of the GPU tests: build oracle pools on the host, upload them,
and compare with the tolerances the checks use.

Tolerances (floating point), per the problem statement of this build:
  attention out: for every (sequence, head), max|gpu - ref| / max|ref| <= 2e-3
  compressed entries (before quantization): per entry, max|gpu - ref| / max|ref| <= 1e-3
Bit-exact: codes and scales of valid page slots, top-k index sets, gathers.
"""

import math

import numpy as np
import torch

import synth
from oracle import codecs, compressor, indexer, paging, pipeline
from synth import gen

ATTN_TOL = 2e-3
ENTRY_TOL = 1e-3
MARGIN = 1e-4


def flush(msg):
    print(msg, flush=True)


def rel_err_rows(got, ref):
    """max over rows of max|got-ref| / max|ref| (rows = all leading axes)."""
    got = np.asarray(got, np.float64).reshape(-1, np.shape(got)[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    num = np.abs(got - ref).max(axis=1)
    den = np.abs(ref).max(axis=1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def upload_pool(pool: paging.Pool):
    import decode_attention_compressed_amd as hca

    if pool.dtype == "bf16":
        codes = to_dev(pool.codes.view(np.int16))
        scales = None
    else:
        codes = to_dev(pool.codes)
        scales = to_dev(pool.scales)
    return hca.PagedCache(codes, scales, pool.epp, pool.d, pool.dtype)


def download_pool(pc, like: paging.Pool) -> paging.Pool:
    out = paging.Pool(like.dtype, like.num_pages, like.epp, like.d)
    if like.dtype == "bf16":
        out.codes = pc.codes.cpu().numpy().view(np.uint16)
    else:
        out.codes = pc.codes.cpu().numpy()
        out.scales = pc.scales.cpu().numpy()
    return out


# E2M1 magnitudes by code (sign in bit 3): the format's eight values
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
_E2M1 = np.concatenate([_E2M1, -_E2M1])


def _f8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def decode_page_rows(dtype, codes, scales):
    """Rows of one page as stored by the GPU, decoded without the oracle (torch's
    float8_e4m3fn and bfloat16 casts, the E2M1 value list; fp4: element 2c in
    the low nibble, one E4M3 scale per 32 elements)."""
    if dtype == "fp8":
        return _f8(codes) * np.float64(scales)
    if dtype == "bf16":
        bits = np.ascontiguousarray(codes).view(np.int16)
        return torch.from_numpy(bits).view(torch.bfloat16).to(torch.float64).numpy()
    v = np.empty(codes.shape[:-1] + (2 * codes.shape[-1],))
    v[..., 0::2] = _E2M1[codes & 0xF]
    v[..., 1::2] = _E2M1[codes >> 4]
    return v * np.repeat(_f8(scales), 32, axis=-1)


def quantized_rows_close(dtype, codes, scales, ref_rows, tol=ENTRY_TOL):
    """Stored page rows against fp64 reference rows.  The kernel quantizes its
    own fp32 rows, which may differ from the reference by tol * (row's max|ref|),
    so each element may be off by that plus half a code step at the stored
    scale (fp8: the E4M3 step at its binade, subnormal below 2^-6; fp4: at
    most one scale unit, the half step between 4 and 6 and the saturation of
    a rounded block scale; bf16: 2^-8 relative).  An fp8 page scale must be
    within 2 tol of amax/448 of the reference rows."""
    ref = np.asarray(ref_rows, np.float64)
    dec = decode_page_rows(dtype, codes, scales)
    dev = tol * np.abs(ref).max(axis=-1, keepdims=True)
    if dtype == "fp8":
        s = float(scales)
        amax = float(np.abs(ref).max())
        if amax > 0 and abs(s - amax / 448.0) > 2 * tol * amax / 448.0:
            return False
        y = (np.abs(ref) + dev) / s
        e = np.maximum(np.floor(np.log2(np.maximum(y, 2.0 ** -12))), -6)
        half = 0.5 * 2.0 ** (e - 3) * s
    elif dtype == "fp4":
        half = np.repeat(_f8(scales), 32, axis=-1)
    else:
        half = (np.abs(ref) + dev) * 2.0 ** -8
    return bool((np.abs(dec - ref) <= (dev + half) * (1 + 1e-9) + 1e-30).all())


def bf16_to_f64(bits):
    return codecs.bf16_decode(bits)


class SeqData:
    """Host-side inputs of one layer for a batch: tokens, logits, bias, queries,
    block tables, and the oracle-built pools."""

    def __init__(self, w: synth.Workload, layer_idx: int, lens, seed=0, build_pools=True, kind=None):
        self.w = w
        self.kind = kind if kind is not None else w.layers[layer_idx]
        self.layer = layer_idx
        self.lens = np.asarray(lens, np.int32)
        self.B = len(self.lens)
        self.members = gen.shared_members(w, self.lens, seed)
        self.table, self.num_pages, self.wtable, self.num_wpages = gen.block_tables(w, self.lens, seed)
        self.spec = pipeline.LayerSpec(m=self.kind.m, d=w.d, H=w.H, window=w.window, topk=self.kind.topk,
                                       kv_dtype=w.kv_dtype, idx_dtype=self.kind.idx_dtype, d_idx=self.kind.d_idx,
                                       h_idx=self.kind.h_idx, theta=w.theta, overlap=self.kind.overlap)
        self.x = [gen.tokens(w, layer_idx, b, int(L), self.members, seed) for b, L in enumerate(self.lens)]
        self.z = [gen.logits(w, layer_idx, b, int(L), self.members, seed) for b, L in enumerate(self.lens)]
        self.beta = gen.slot_bias(w, layer_idx, self.kind.slots, seed)
        self.q = gen.queries(w, layer_idx, seed)[: self.B]
        self.entries = None
        if self.kind.topk is not None:
            self.qi = gen.index_queries(w, layer_idx, self.kind.h_idx, self.kind.d_idx, seed)[: self.B]
            self.wi = gen.index_weights(w, layer_idx, self.kind.h_idx, seed)[: self.B]
            self.keys = [gen.index_keys(w, layer_idx, b, int(compressor.n_entries(L, self.kind.m)), self.kind.d_idx,
                                        self.kind.m, self.members, seed) for b, L in enumerate(self.lens)]
        if build_pools:
            self.build_pools()

    def build_pools(self):
        s = self.spec
        self.kv = paging.Pool(s.kv_dtype, self.num_pages, s.epp, s.d)
        self.win = paging.Pool(s.kv_dtype, max(1, self.num_wpages), 256, s.d)
        self.entries = []
        done_shared = False
        for b in range(self.B):
            xb = bf16_to_f64(self.x[b])
            e = pipeline.fill_entries(s, self.kv, self.table[b], xb, self.z[b], self.beta)
            self.entries.append(e)
            pipeline.fill_window(s, self.win, self.wtable[b], xb, int(self.lens[b]))
        if self.kind.topk is not None:
            self.idx = paging.Pool(self.kind.idx_dtype, self.num_pages, s.epp, self.kind.d_idx)
            for b in range(self.B):
                paging.write_run(self.idx, self.table[b], 0, self.keys[b])
        del done_shared

    def oracle_scores(self, b):
        N = int(compressor.n_entries(int(self.lens[b]), self.kind.m))
        keys = paging.decode_rows(self.idx, self.table[b], np.arange(N))
        return indexer.scores(bf16_to_f64(self.qi[b]), self.wi[b].astype(np.float64), keys)

    def enforce_margin(self, seed=0, max_rounds=50):
        """Re-draw indexer keys near the top-k cut until every sequence's k-th score
        is at least MARGIN away from its neighbour across the cut."""
        k = self.kind.topk
        for b in range(self.B):
            if b in set(self.members.tolist()):
                continue  # shared-prefix keys stay shared; their margins are checked below
            for attempt in range(max_rounds):
                s = self.oracle_scores(b)
                N = len(s)
                if k >= N:
                    break
                srt = np.sort(s)[::-1]
                cut = 0.5 * (srt[k - 1] + srt[k])
                near = np.nonzero(np.abs(s - cut) < MARGIN)[0]
                if len(near) == 0 and indexer.kth_margin(s, k) >= MARGIN:
                    break
                if len(near) == 0:
                    near = np.nonzero(np.abs(s - srt[k - 1]) < 2 * MARGIN)[0]
                self.keys[b][near] = gen.redraw_keys(self.w, self.layer, b, near, self.kind.d_idx, attempt)
                paging.write_run(self.idx, self.table[b], 0, self.keys[b])
        return [indexer.kth_margin(self.oracle_scores(b), k) for b in range(self.B)]

    def oracle_select(self, b):
        if self.kind.topk is None:
            return np.arange(int(compressor.n_entries(int(self.lens[b]), self.kind.m)))
        return indexer.topk(self.oracle_scores(b), self.kind.topk)

    def oracle_attend(self, b, sel):
        q = bf16_to_f64(self.q[b])
        return pipeline.attend(self.spec, int(self.lens[b]), q, self.kv, self.table[b], self.win, self.wtable[b], sel)

    # device copies
    def dev_common(self):
        return dict(table=to_dev(self.table), wtable=to_dev(self.wtable), lens=to_dev(self.lens),
                    q=to_dev(self.q.view(np.int16)))


def max_len(lens):
    return int(np.max(lens))


def scale_for(d):
    return 1.0 / math.sqrt(d)
