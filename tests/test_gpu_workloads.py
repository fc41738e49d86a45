"""Full-size workloads in the benchmark's launch configuration, checked on
sampled outputs.

Each case builds one layer's caches on the GPU the way the benchmark does
(kv_compress + kv_quantize_page over the whole context, the window pages, the
indexer keys, all drawn with the same seeded device generator), runs
indexer_topk and paged_hybrid_decode with workspaces sized for the full
workload (so the split plan and grids are the benchmark's), and compares with
the fp64 oracle:

- compressed entries of sampled groups (oracle fold of the downloaded raw
  tokens of those groups), to 1e-3;
- codes and scales of sampled pages, bit for bit (oracle quantization of the
  GPU's own fp32 rows);
- the window rows of sampled sequences, and their page codes;
- the top-k set of sampled sequences, exactly, after the keys near the cut are
  re-drawn until no score is within 1e-4 of it (oracle scores over the
  downloaded indexer pool);
- every head's attention output of sampled sequences, to 2e-3 (oracle over the
  downloaded pools, with the oracle's own selection).
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
        self.beta_np = gen.slot_bias(w, li, m)
        xi = self.x.view(torch.int16)
        # prefill: entries, their pages
        self.ent = torch.empty((B, self.N, d), dtype=torch.float32, device="cuda")
        hca.kv_compress(xi, self.z, _dev(self.beta_np), zeros, self.lens, m, w.theta, self.ent, L)
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

    # host mirrors of the GPU pools (the oracle reads these)
    def host_pool(self, pc, dtype, num_pages, epp, dim):
        like = paging.Pool(dtype, num_pages, epp, dim)
        return H.download_pool(pc, like)

    def spec(self):
        w, k = self.w, self.kind
        return pipeline.LayerSpec(m=k.m, d=w.d, H=w.H, window=w.window, topk=k.topk, kv_dtype=w.kv_dtype,
                                  idx_dtype=k.idx_dtype, d_idx=k.d_idx, h_idx=k.h_idx, theta=w.theta)


def _check_entries(lay, bs, rng):
    w, m, N = lay.w, lay.m, lay.N
    for b in bs:
        js = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 22)]))
        for j in js:
            t0, t1 = j * m, min(w.L, (j + 1) * m)
            xg = lay.x[b, t0:t1].view(torch.int16).cpu().numpy().view(np.uint16)
            zg = lay.z[b, t0:t1].cpu().numpy()
            ref = compressor.compress(codecs.bf16_decode(xg), zg, lay.beta_np, m, w.theta, pos0=int(t0))
            got = lay.ent[b, j].cpu().numpy()[None]
            assert H.rel_err_rows(got, ref) <= H.ENTRY_TOL, (b, int(j))


def _check_pages(pool_host, rows_dev, table_row, epp, dtype, pages, first_entry=0):
    for p in pages:
        rows = rows_dev[p * epp - first_entry: (p + 1) * epp - first_entry].cpu().numpy()
        codes, scales = paging.quantize_page(rows, dtype, epp)
        phys = int(table_row[p])
        n = rows.shape[0]
        assert np.array_equal(pool_host.codes[phys, :n], codes[:n]), p
        if dtype == "fp8":
            assert pool_host.scales[phys] == scales, p
        elif dtype == "fp4":
            assert np.array_equal(pool_host.scales[phys, :n], scales[:n]), p


def _enforce_margin(hca, lay, idx_host, b, max_rounds=20):
    """Re-draw the keys of entries near the top-k cut of sequence b (on the
    GPU, then re-quantize its pages) until the k-th score is clear by 1e-4."""
    k, kind = lay.kind.topk, lay.kind
    qi = codecs.bf16_decode(lay.qi_np[b])
    wi = lay.wi_np[b].astype(np.float64)
    ent_idx = np.arange(lay.N)
    for attempt in range(max_rounds):
        keys = paging.decode_rows(idx_host, lay.table[b], ent_idx)
        s = indexer.scores(qi, wi, keys)
        if indexer.kth_margin(s, k) >= H.MARGIN:
            return s
        srt = np.sort(s)[::-1]
        cut = 0.5 * (srt[k - 1] + srt[k])
        near = np.nonzero(np.abs(s - cut) < 4 * H.MARGIN)[0]
        new = gen.redraw_keys(lay.w, lay.li, b, near, kind.d_idx, attempt)
        lay.keys[b, torch.from_numpy(near).cuda()] = torch.from_numpy(new).cuda()
        # re-quantize the pages of sequence b, then refresh their host copy
        one = _dev(np.zeros(1, np.int32))
        hca.kv_quantize_page(lay.keys[b:b + 1], one, _dev(np.array([lay.N], np.int32)), lay.N,
                             _dev(lay.table[b:b + 1]), lay.idx)
        torch.cuda.synchronize()
        pages = np.unique(lay.table[b][: -(-lay.N // lay.epp)])
        idx_host.codes[pages] = lay.idx.codes[torch.from_numpy(pages).cuda().long()].cpu().numpy()
        if idx_host.dtype != "bf16":
            idx_host.scales[pages] = lay.idx.scales[torch.from_numpy(pages).cuda().long()].cpu().numpy()
    pytest.fail(f"could not clear the top-k margin of sequence {b}")


CASES = [
    # (workload id, layer index, sampled sequences)
    pytest.param(4, 0, (0, 3), id="stack1m-c4a-fp4"),
    pytest.param(4, 30, (1, 2), id="stack1m-c128a"),  # the stack lists its 30 c4a layers first
    pytest.param(2, 0, (0, 9, 15), id="c4a-128k-b16-fp8"),
    pytest.param(1, 0, (0, 7), id="c128a-64k-b8"),
]


@pytest.mark.parametrize("cid,li,bs", CASES)
def test_full_workload_sampled(cid, li, bs):
    import decode_attention_compressed_amd as hca

    w = synth.workload(cid)
    kind = w.layers[li]
    assert kind.name == ("c128a" if "c128a" in w.name or li >= 30 else "c4a")
    H.flush(f"full workload {w.name} layer {li} ({kind.name}) B={w.B} L={w.L} sampled {bs}")
    rng = np.random.default_rng(1000 + 10 * cid + li)
    lay = FullLayer(hca, w, li)
    B, L, d, W, Hq = w.B, w.L, w.d, w.window, w.H
    _check_entries(lay, bs, rng)
    kv_host = lay.host_pool(lay.kv, w.kv_dtype, lay.P, lay.epp, d)
    win_host = lay.host_pool(lay.win, w.kv_dtype, lay.PW, BLOCK, d)
    n_pages = -(-lay.N // lay.epp)
    for b in bs:
        pages = np.unique(np.concatenate([[0, n_pages - 1], rng.integers(0, n_pages, 3)]))
        _check_pages(kv_host, lay.ent[b], lay.table[b], lay.epp, w.kv_dtype, pages)
        # window rows against the oracle's rotation of the raw tokens, then their pages
        xw = lay.x[b, lay.t0:].view(torch.int16).cpu().numpy().view(np.uint16)
        ref = compressor.window_rows(codecs.bf16_decode(xw), lay.t0, w.theta)
        assert H.rel_err_rows(lay.wrows[b].cpu().numpy(), ref) <= H.ENTRY_TOL, b
        wpages = np.arange(lay.t0 // BLOCK, -(-L // BLOCK))
        _check_pages(win_host, lay.wrows[b], lay.wtable[b], BLOCK, w.kv_dtype, wpages, first_entry=lay.t0)

    sel = sel_n = None
    sel_host = {}
    if kind.topk is not None:
        idx_host = lay.host_pool(lay.idx, kind.idx_dtype, lay.P, lay.epp, kind.d_idx)
        for b in bs:
            _check_pages(idx_host, lay.keys[b], lay.table[b], lay.epp, kind.idx_dtype,
                         np.unique(np.concatenate([[0, n_pages - 1], rng.integers(0, n_pages, 3)])))
            s = _enforce_margin(hca, lay, idx_host, b)
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

    wsa = hca.workspace(hca.paged_hybrid_decode_workspace(B, Hq, d, L, kind.m, W, kind.topk or 0))
    out = torch.zeros((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
    hca.paged_hybrid_decode(lay.q, lay.kv, _dev(lay.table), lay.win, _dev(lay.wtable), lay.lens, L, kind.m, W,
                            sel, sel_n, 1.0 / math.sqrt(d), w.theta, out, lse, wsa)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    got_lse = lse.cpu().numpy()
    spec = lay.spec()
    for b in bs:
        q = codecs.bf16_decode(lay.q_np[b])
        ref, ref_lse, _ = pipeline.attend(spec, L, q, kv_host, lay.table[b], win_host, lay.wtable[b], sel_host[b])
        err = H.rel_err_rows(got[b], ref)
        H.flush(f"  sequence {b}: attention rel err {err:.2e}")
        assert err <= H.ATTN_TOL, b
        assert np.allclose(got_lse[b], ref_lse, rtol=0, atol=1e-3), b
    del lay
    torch.cuda.empty_cache()
