"""Full-size workloads in the benchmark's launch configuration, checked on
sampled outputs.

Each case builds one layer's caches on the GPU the way the benchmark does
(kv_compress with the entries' RMSNorm + kv_quantize_page over the whole
context, the window pages, the indexer keys, all drawn with the same seeded
device generator), runs indexer_topk and paged_hybrid_decode with workspaces
sized for the full workload (so the split plan and grids are the
benchmark's), and compares with the fp64 oracle.  The oracle takes only the
workload's inputs (raw tokens, logits, slot biases, gains, indexer keys and
queries, block tables), never a GPU result: for each sampled sequence it folds
the entries of the pages it needs itself and quantizes them into its own
pools.  Checked:

- compressed entries of sampled groups, to 1e-3;
- sampled stored pages: the GPU's decoded rows within 1e-3 plus half a code
  step of the oracle's rows (the quantizer alone is bit-exact against the
  oracle's in the kv_quantize_page tests);
- the window rows of sampled sequences, and their pages, likewise;
- indexer pages bit for bit (both sides quantize the same fp32 keys);
- the top-k set of sampled sequences, exactly, after the keys near the cut are
  re-drawn until no oracle score is within 1e-4 of it;
- every head's attention output of sampled sequences, to 2e-3, and its fp8
  form to 2e-3 plus half an E4M3 step: the oracle attends over its own pools
  with its own selection, and the pages the GPU attention reads for those
  sequences are replaced by the oracle's beforehand (where the GPU's fold and
  the oracle's fall on either side of a rounding boundary, their codes differ
  by one E4M3 step, which in a row of some weight moves the output by more
  than the tolerance; the GPU's own pages are checked above).
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import codecs, compressor, indexer, paging, pipeline
from synth import gen

from tests import helpers as H

pytestmark = pytest.mark.gpu

BLOCK = 256


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class FullLayer:
    """One layer of a fixed-length workload, built on the GPU."""

    def __init__(self, hca, w, li):
        kind = w.layers[li]
        self.w, self.li, self.kind = w, li, kind
        B, L, d, W = w.B, w.L, w.d, w.window
        m = kind.m
        self.m, self.epp, self.N = m, BLOCK // m, -(-L // m)
        self.lens_np = np.full((B,), L, np.int32)
        self.table, self.P, self.wtable, self.PW = gen.block_tables(w, self.lens_np)
        self.lens = _dev(self.lens_np)
        zeros = _dev(np.zeros(B, np.int32))
        # raw tokens and logits (seeded device draws, as the benchmark)
        self.x = torch.empty((B, L, d), dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            self.x[b] = gen.device_normal((L, d), 1.0, (0, w.cid, li, gen.S_TOK, b), dtype=torch.bfloat16)
        self.z = gen.device_normal((B, L), 1.0, (0, w.cid, li, gen.S_LOGIT))
        self.beta_np = gen.slot_bias(w, li, kind.slots)
        self.gamma_np = gen.norm_gain(w, li, d)
        xi = self.x.view(torch.int16)
        # prefill: entries, their pages
        self.ent = torch.empty((B, self.N, d), dtype=torch.float32, device="cuda")
        hca.kv_compress(xi, self.z, _dev(self.beta_np), zeros, self.lens, m, w.theta, self.ent, L,
                        norm_gamma=_dev(self.gamma_np), norm_eps=1e-6, overlap=kind.overlap)
        self.kv = hca.PagedCache.empty(self.P, self.epp, d, w.kv_dtype)
        hca.kv_quantize_page(self.ent, zeros, _dev(np.full(B, self.N, np.int32)), self.N, _dev(self.table), self.kv)
        # window pages: every token of the blocks that overlap [L-W, L)
        self.t0 = (max(0, L - W) // BLOCK) * BLOCK
        nw = L - self.t0
        self.wrows = torch.empty((B, nw, d), dtype=torch.float32, device="cuda")
        hca.kv_compress(xi[:, self.t0:], self.z[:, self.t0:], _dev(np.zeros(1, np.float32)),
                        _dev(np.full(B, self.t0, np.int32)), _dev(np.full(B, nw, np.int32)), 1, w.theta, self.wrows, nw)
        self.win = hca.PagedCache.empty(self.PW, BLOCK, d, w.kv_dtype)
        hca.kv_quantize_page(self.wrows, _dev(np.full(B, self.t0, np.int32)), _dev(np.full(B, nw, np.int32)), nw,
                             _dev(self.wtable), self.win)
        self.q_np = gen.queries(w, li)
        self.q = _dev(self.q_np.view(np.int16))
        if kind.topk is not None:
            self.keys = gen.device_normal((B, self.N, kind.d_idx), 1.0, (0, w.cid, li, gen.S_IDXK))
            self.idx = hca.PagedCache.empty(self.P, self.epp, kind.d_idx, kind.idx_dtype)
            hca.kv_quantize_page(self.keys, zeros, _dev(np.full(B, self.N, np.int32)), self.N, _dev(self.table),
                                 self.idx)
            self.qi_np = gen.index_queries(w, li, kind.h_idx, kind.d_idx)
            self.wi_np = gen.index_weights(w, li, kind.h_idx)
        torch.cuda.synchronize()

    def spec(self):
        w, k = self.w, self.kind
        return pipeline.LayerSpec(m=k.m, d=w.d, H=w.H, window=w.window, topk=k.topk, kv_dtype=w.kv_dtype,
                                  idx_dtype=k.idx_dtype, d_idx=k.d_idx, h_idx=k.h_idx, theta=w.theta,
                                  gamma=self.gamma_np, eps=1e-6, overlap=k.overlap)

    def gpu_page(self, pc, phys):
        """Codes and scale(s) of one physical page of a GPU pool, on the host."""
        codes = pc.codes[phys].cpu().numpy()
        if pc.dtype == "bf16":
            return codes.view(np.uint16), None
        return codes, pc.scales[phys].cpu().numpy()


class OracleSeq:
    """The oracle's side of one sequence of a FullLayer, built from the inputs
    only: the raw tokens and logits (copied from the seeded device draws), the
    slot biases and gains, the indexer keys, the block tables."""

    def __init__(self, lay, b):
        w = lay.w
        self.lay, self.b = lay, b
        self.x = lay.x[b].view(torch.int16).cpu().numpy().view(np.uint16)
        self.z = lay.z[b].cpu().numpy()
        self.spec = lay.spec()
        self.kv = paging.Pool(w.kv_dtype, lay.P, lay.epp, w.d)
        self.rows = {}  # logical page -> the oracle's fp64 entries of that page

    def fold_pages(self, pages, run=64):
        """Fold the entries of the given logical pages (runs of consecutive
        pages in one call) and quantize them into the oracle's pool."""
        lay, w = self.lay, self.lay.w
        todo = sorted(set(int(p) for p in pages) - set(self.rows))
        k = 0
        while k < len(todo):
            p0 = todo[k]
            p1 = p0 + 1
            while k + 1 < len(todo) and todo[k + 1] == p1 and p1 - p0 < run:
                k += 1
                p1 += 1
            k += 1
            e0, e1 = p0 * lay.epp, min(lay.N, p1 * lay.epp)
            t0, t1 = e0 * lay.m, min(w.L, e1 * lay.m)
            o = lay.kind.overlap
            if o > 0:
                e = compressor.compress_overlap(codecs.bf16_decode(self.x[t0:t1]), self.z[t0:t1], lay.beta_np,
                                                lay.m, o, w.theta, pos0=t0,
                                                x_prev=codecs.bf16_decode(self.x[max(0, t0 - o): t0]),
                                                z_prev=self.z[max(0, t0 - o): t0], gamma=lay.gamma_np, eps=1e-6)
            else:
                e = compressor.compress(codecs.bf16_decode(self.x[t0:t1]), self.z[t0:t1], lay.beta_np, lay.m,
                                        w.theta, pos0=t0, gamma=lay.gamma_np, eps=1e-6)
            paging.write_run(self.kv, lay.table[self.b], e0, e.astype(np.float32))
            for p in range(p0, p1):
                self.rows[p] = e[(p - p0) * lay.epp: (p - p0 + 1) * lay.epp]

    def entry(self, j):
        self.fold_pages([j // self.lay.epp])
        return self.rows[j // self.lay.epp][j % self.lay.epp]

    def window(self):
        """The window rows (every token of the blocks overlapping [L-W, L)) and
        the oracle's window pool."""
        lay, w = self.lay, self.lay.w
        rows = compressor.window_rows(codecs.bf16_decode(self.x[lay.t0:]), lay.t0, w.theta)
        pool = paging.Pool(w.kv_dtype, lay.PW, BLOCK, w.d)
        paging.write_run(pool, lay.wtable[self.b], lay.t0, rows.astype(np.float32))
        return rows, pool


def _check_entries(lay, orc, rng):
    w, m, N = lay.w, lay.m, lay.N
    js = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 22)]))
    got = lay.ent[orc.b, torch.from_numpy(js).cuda()].cpu().numpy()
    for r, j in enumerate(js):
        assert H.rel_err_rows(got[r][None], orc.entry(int(j))[None]) <= H.ENTRY_TOL, (orc.b, int(j))


def _check_pages_close(lay, pc, table_row, rows_of_page, pages, dtype):
    """GPU pages against the oracle's rows of the same logical pages."""
    for p in pages:
        ref = rows_of_page(p)
        codes, sc = lay.gpu_page(pc, int(table_row[p]))
        n = ref.shape[0]
        scale = sc if dtype == "fp8" else (sc[:n] if dtype == "fp4" else None)
        assert H.quantized_rows_close(dtype, codes[:n], scale, ref), p


def _upload_pages(pc, pool, phys):
    """Copy physical pages of an oracle pool into the same pages of a GPU pool."""
    idx = torch.from_numpy(np.asarray(phys, np.int64)).cuda()
    codes = pool.codes[np.asarray(phys)]
    pc.codes[idx] = torch.from_numpy(codes.view(np.int16) if pool.dtype == "bf16" else codes).cuda()
    if pool.dtype != "bf16":
        pc.scales[idx] = torch.from_numpy(pool.scales[np.asarray(phys)]).cuda()
    torch.cuda.synchronize()


def _enforce_margin(hca, lay, b, keys_b, idx_ref, max_rounds=20):
    """Re-draw the keys of entries near the top-k cut of sequence b (the same
    new fp32 keys on the GPU and in the oracle's pool) until the oracle's k-th
    score is clear by 1e-4.  Returns the oracle's scores."""
    k, kind = lay.kind.topk, lay.kind
    qi = codecs.bf16_decode(lay.qi_np[b])
    wi = lay.wi_np[b].astype(np.float64)
    ent_idx = np.arange(lay.N)
    for attempt in range(max_rounds):
        s = indexer.scores(qi, wi, paging.decode_rows(idx_ref, lay.table[b], ent_idx))
        if indexer.kth_margin(s, k) >= H.MARGIN:
            return s
        srt = np.sort(s)[::-1]
        cut = 0.5 * (srt[k - 1] + srt[k])
        near = np.nonzero(np.abs(s - cut) < 4 * H.MARGIN)[0]
        new = gen.redraw_keys(lay.w, lay.li, b, near, kind.d_idx, attempt)
        keys_b[near] = new
        lay.keys[b, torch.from_numpy(near).cuda()] = torch.from_numpy(new).cuda()
        one = _dev(np.zeros(1, np.int32))
        hca.kv_quantize_page(lay.keys[b:b + 1], one, _dev(np.array([lay.N], np.int32)), lay.N,
                             _dev(lay.table[b:b + 1]), lay.idx)
        paging.write_run(idx_ref, lay.table[b], 0, keys_b)
        torch.cuda.synchronize()
    pytest.fail(f"could not clear the top-k margin of sequence {b}")


CASES = [
    # (workload id, layer index, sampled sequences, compressor overlap: None as the workload)
    pytest.param(4, 0, (0, 3), None, id="stack1m-c4a-fp4"),
    pytest.param(4, 30, (1, 2), None, id="stack1m-c128a"),  # the stack lists its 30 c4a layers first
    pytest.param(2, 0, (0, 9, 15), None, id="c4a-128k-b16-fp8"),
    pytest.param(1, 0, (0, 7), None, id="c128a-64k-b8"),
    # the plain c4a compressor: a softmax over the 4 slots of non-overlapping
    # groups, on the 1M-token stack's c4a layer shape
    pytest.param(4, 0, (1, 2), 0, id="stack1m-c4a-fp4-no-overlap"),
]


@pytest.mark.parametrize("cid,li,bs,overlap", CASES)
def test_full_workload_sampled(cid, li, bs, overlap):
    import dataclasses

    import decode_attention_compressed_amd as hca

    w = synth.workload(cid)
    if overlap is not None:
        layers = list(w.layers)
        layers[li] = dataclasses.replace(layers[li], overlap=overlap)
        w = dataclasses.replace(w, layers=layers)
    kind = w.layers[li]
    assert kind.name == ("c128a" if "c128a" in w.name or li >= 30 else "c4a")
    H.flush(f"full workload {w.name} layer {li} ({kind.name}, overlap {kind.overlap}) B={w.B} L={w.L} sampled {bs}")
    rng = np.random.default_rng(1000 + 10 * cid + li)
    lay = FullLayer(hca, w, li)
    B, L, d, W, Hq = w.B, w.L, w.d, w.window, w.H
    n_pages = -(-lay.N // lay.epp)
    orcs = {}
    win_ref = {}
    for b in bs:
        orc = orcs[b] = OracleSeq(lay, b)
        _check_entries(lay, orc, rng)
        pages = np.unique(np.concatenate([[0, n_pages - 1], rng.integers(0, n_pages, 3)]))
        orc.fold_pages(pages)
        _check_pages_close(lay, lay.kv, lay.table[b], lambda p: orc.rows[p], pages, w.kv_dtype)
        # window rows against the oracle's rotation of the raw tokens, then their pages
        wrows, win_ref[b] = orc.window()
        assert H.rel_err_rows(lay.wrows[b].cpu().numpy(), wrows) <= H.ENTRY_TOL, b
        wpages = np.arange(lay.t0 // BLOCK, -(-L // BLOCK))
        _check_pages_close(lay, lay.win, lay.wtable[b],
                           lambda p: wrows[p * BLOCK - lay.t0: min(L, (p + 1) * BLOCK) - lay.t0], wpages, w.kv_dtype)

    sel = sel_n = None
    sel_host = {}
    if kind.topk is not None:
        for b in bs:
            keys_b = lay.keys[b].cpu().numpy()
            idx_ref = paging.Pool(kind.idx_dtype, lay.P, lay.epp, kind.d_idx)
            paging.write_run(idx_ref, lay.table[b], 0, keys_b)
            for p in np.unique(np.concatenate([[0, n_pages - 1], rng.integers(0, n_pages, 3)])):
                phys = int(lay.table[b][p])
                codes, sc = lay.gpu_page(lay.idx, phys)
                n = min(lay.epp, lay.N - p * lay.epp)
                assert np.array_equal(codes[:n], idx_ref.codes[phys, :n]), p
                if kind.idx_dtype == "fp8":
                    assert sc == idx_ref.scales[phys], p
                elif kind.idx_dtype == "fp4":
                    assert np.array_equal(sc[:n], idx_ref.scales[phys, :n]), p
            s = _enforce_margin(hca, lay, b, keys_b, idx_ref)
            sel_host[b] = indexer.topk(s, kind.topk)
        ws = hca.workspace(hca.indexer_topk_workspace(B, L, kind.m, kind.topk))
        sel = torch.full((B, kind.topk), -7, dtype=torch.int32, device="cuda")
        sel_n = torch.zeros((B,), dtype=torch.int32, device="cuda")
        hca.indexer_topk(_dev(lay.qi_np.view(np.int16)), _dev(lay.wi_np), lay.idx, _dev(lay.table), lay.lens, L,
                         kind.m, kind.topk, sel, sel_n, ws)
        torch.cuda.synchronize()
        got_sel, got_n = sel.cpu().numpy(), sel_n.cpu().numpy()
        for b in bs:
            want = sel_host[b]
            assert got_n[b] == len(want), b
            assert np.array_equal(got_sel[b, : got_n[b]], want), b
    else:
        for b in bs:
            sel_host[b] = np.arange(lay.N)

    # the attention reads the oracle's pages: the sampled sequences' pages that
    # it reads are replaced by the oracle's own (one E4M3 step between a GPU
    # code and the oracle's at a rounding boundary would otherwise move the
    # output by more than the tolerance), so both sides attend over the same
    # stored rows
    for b in bs:
        orc = orcs[b]
        need = np.unique(sel_host[b] // lay.epp)
        orc.fold_pages(need)
        _upload_pages(lay.kv, orc.kv, lay.table[b][need])
        _upload_pages(lay.win, win_ref[b], lay.wtable[b][np.arange(lay.t0 // BLOCK, -(-L // BLOCK))])
    wsa = hca.workspace(hca.paged_hybrid_decode_workspace(B, Hq, d, L, kind.m, W, kind.topk or 0))
    out = torch.zeros((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
    o8 = torch.zeros((B, Hq, d), dtype=torch.uint8, device="cuda")
    o8s = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
    hca.paged_hybrid_decode(lay.q, lay.kv, _dev(lay.table), lay.win, _dev(lay.wtable), lay.lens, L, kind.m, W,
                            sel, sel_n, 1.0 / math.sqrt(d), w.theta, out, lse, wsa, out_fp8=o8, out_scale=o8s)
    torch.cuda.synchronize()
    got, got_lse = out.cpu().numpy(), lse.cpu().numpy()
    got8, got8s = o8.cpu().numpy(), o8s.cpu().numpy()
    for b in bs:
        orc = orcs[b]
        q = codecs.bf16_decode(lay.q_np[b])
        ref, ref_lse, _ = pipeline.attend(orc.spec, L, q, orc.kv, lay.table[b], win_ref[b], lay.wtable[b],
                                          sel_host[b])
        err = H.rel_err_rows(got[b], ref)
        H.flush(f"  sequence {b}: attention rel err {err:.2e}")
        assert err <= H.ATTN_TOL, b
        assert np.allclose(got_lse[b], ref_lse, rtol=0, atol=1e-3), b
        for h in range(Hq):
            assert H.quantized_rows_close("fp8", got8[b, h], got8s[b, h], ref[h], tol=H.ATTN_TOL), (b, h)
    del lay
    torch.cuda.empty_cache()
