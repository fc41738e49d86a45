"""The mixed paged batch at full size: 64 sequences of log-uniform lengths in
[256, 131072] (none block-aligned), 16 of them sharing an 8-block prefix whose
pages are aliased in the block table, one c4a layer (8-token windows at stride
4, fp8 indexer keys, top-2048) and one c128a layer, fp8 KV of 512 dims, 64
query heads, a 128-token window.

The caches are built on the GPU as the benchmark builds them (the shared
prefix's pages written once, by the first sequence that holds them), the
indexer and the attention run with workspaces sized for the whole batch (the
benchmark's launch configuration, whose work list cuts every sequence's rows
into splits sized from all the lengths), and the oracle, from the inputs
alone, checks sampled sequences: the entries of sampled groups (1e-3), the
top-k set exactly (keys near the cut re-drawn outside the shared prefix), and
every head's attention output (2e-3) over the oracle's own pages and
selection.  Every sequence of the batch is also checked against the same
attention launched for that sequence alone (2e-3), which covers the work list
for all 64 lengths.
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


class MixedLayer:
    """One layer of the mixed batch, built on the GPU."""

    def __init__(self, hca, w, li):
        kind = w.layers[li]
        self.w, self.li, self.kind = w, li, kind
        B, d, W = w.B, w.d, w.window
        m = kind.m
        self.m, self.epp = m, BLOCK // m
        self.lens_np = gen.lengths(w)
        self.Lmax = int(self.lens_np.max())
        self.N = -(-self.lens_np // m)
        self.members = [int(b) for b in gen.shared_members(w, self.lens_np)]
        assert len(self.members) == w.shared_prefix_seqs
        self.npre_tok = w.shared_prefix_blocks * BLOCK
        self.npre = self.npre_tok // m
        self.table, self.P, self.wtable, self.PW = gen.block_tables(w, self.lens_np)
        for b in self.members[1:]:  # the prefix's pages are aliased
            assert np.array_equal(self.table[b, : w.shared_prefix_blocks],
                                  self.table[self.members[0], : w.shared_prefix_blocks])
        self.lens = _dev(self.lens_np)
        rest = self.members[1:]
        own = [b for b in range(B) if b not in rest]
        self.x = torch.empty((B, self.Lmax, d), dtype=torch.bfloat16, device="cuda")
        for b in range(B):
            self.x[b] = gen.device_normal((self.Lmax, d), 1.0, (0, w.cid, li, gen.S_TOK, b), dtype=torch.bfloat16)
        self.z = gen.device_normal((B, self.Lmax), 1.0, (0, w.cid, li, gen.S_LOGIT))
        for b in rest:
            self.x[b, : self.npre_tok] = self.x[self.members[0], : self.npre_tok]
            self.z[b, : self.npre_tok] = self.z[self.members[0], : self.npre_tok]
        self.beta_np = gen.slot_bias(w, li, kind.slots)
        self.gamma_np = gen.norm_gain(w, li, d)
        xi = self.x.view(torch.int16)
        Nmax = int(self.N.max())
        self.ent = torch.empty((B, Nmax, d), dtype=torch.float32, device="cuda")
        hca.kv_compress(xi, self.z, _dev(self.beta_np), _dev(np.zeros(B, np.int32)), self.lens, m, w.theta, self.ent,
                        self.Lmax, norm_gamma=_dev(self.gamma_np), norm_eps=1e-6, overlap=kind.overlap)
        self.kv = hca.PagedCache.empty(self.P, self.epp, d, w.kv_dtype)
        self._quantize(hca, self.ent, self.kv, own, rest, Nmax)
        # window pages: every token of the blocks that overlap [L-W, L)
        self.t0 = (np.maximum(0, self.lens_np - W) // BLOCK) * BLOCK
        nw = self.lens_np - self.t0
        nwmax = int(nw.max())
        xw = torch.zeros((B, nwmax, d), dtype=torch.int16, device="cuda")
        zw = torch.zeros((B, nwmax), dtype=torch.float32, device="cuda")
        for b in range(B):
            xw[b, : nw[b]] = xi[b, self.t0[b]: self.lens_np[b]]
            zw[b, : nw[b]] = self.z[b, self.t0[b]: self.lens_np[b]]
        self.wrows = torch.empty((B, nwmax, d), dtype=torch.float32, device="cuda")
        t0d, nwd = _dev(self.t0.astype(np.int32)), _dev(nw.astype(np.int32))
        hca.kv_compress(xw, zw, _dev(np.zeros(1, np.float32)), t0d, nwd, 1, w.theta, self.wrows, nwmax)
        self.win = hca.PagedCache.empty(self.PW, BLOCK, d, w.kv_dtype)
        hca.kv_quantize_page(self.wrows, t0d, nwd, nwmax, _dev(self.wtable), self.win)
        self.q_np = gen.queries(w, li)
        self.q = _dev(self.q_np.view(np.int16))
        if kind.topk is not None:
            self.keys = gen.device_normal((B, Nmax, kind.d_idx), 1.0, (0, w.cid, li, gen.S_IDXK))
            for b in rest:
                self.keys[b, : self.npre] = self.keys[self.members[0], : self.npre]
            self.idx = hca.PagedCache.empty(self.P, self.epp, kind.d_idx, kind.idx_dtype)
            self._quantize(hca, self.keys, self.idx, own, rest, Nmax)
            self.qi_np = gen.index_queries(w, li, kind.h_idx, kind.d_idx)
            self.wi_np = gen.index_weights(w, li, kind.h_idx)
        torch.cuda.synchronize()

    def _quantize(self, hca, src, pool, own, rest, Nmax):
        # every page once: the shared prefix's pages by the first member only
        sub = torch.tensor(own, dtype=torch.long, device="cuda")
        hca.kv_quantize_page(src[sub], _dev(np.zeros(len(own), np.int32)), _dev(self.N[own].astype(np.int32)), Nmax,
                             _dev(self.table[own]), pool)
        if rest:
            sr = torch.tensor(rest, dtype=torch.long, device="cuda")
            hca.kv_quantize_page(src[sr][:, self.npre:].contiguous(), _dev(np.full(len(rest), self.npre, np.int32)),
                                 _dev((self.N[rest] - self.npre).astype(np.int32)), Nmax - self.npre,
                                 _dev(self.table[rest]), pool)

    def spec(self):
        w, k = self.w, self.kind
        return pipeline.LayerSpec(m=k.m, d=w.d, H=w.H, window=w.window, topk=k.topk, kv_dtype=w.kv_dtype,
                                  idx_dtype=k.idx_dtype, d_idx=k.d_idx, h_idx=k.h_idx, theta=w.theta,
                                  gamma=self.gamma_np, eps=1e-6, overlap=k.overlap)


def _oracle_entries(lay, b, e0, e1):
    """The oracle's entries e0 .. e1-1 of sequence b from its raw tokens."""
    w, m, o = lay.w, lay.m, lay.kind.overlap
    L = int(lay.lens_np[b])
    x = lay.x[b].view(torch.int16).cpu().numpy().view(np.uint16)
    z = lay.z[b].cpu().numpy()
    t0, t1 = e0 * m, min(L, e1 * m)
    if o > 0:
        return compressor.compress_overlap(codecs.bf16_decode(x[t0:t1]), z[t0:t1], lay.beta_np, m, o, w.theta,
                                           pos0=t0, x_prev=codecs.bf16_decode(x[max(0, t0 - o): t0]),
                                           z_prev=z[max(0, t0 - o): t0], gamma=lay.gamma_np, eps=1e-6)
    return compressor.compress(codecs.bf16_decode(x[t0:t1]), z[t0:t1], lay.beta_np, m, w.theta, pos0=t0,
                               gamma=lay.gamma_np, eps=1e-6)


def _attend_batch(hca, lay, sel, sel_n, rows=None):
    """paged_hybrid_decode over the whole batch (rows: None) or over the listed
    sequences one launch each; returns fp32 outputs and lse."""
    w, B = lay.w, lay.w.B
    d, Hq = w.d, w.H
    k = lay.kind.topk or 0
    out = torch.zeros((B, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, Hq), dtype=torch.float32, device="cuda")
    tab, wtab = _dev(lay.table), _dev(lay.wtable)
    if rows is None:
        ws = hca.workspace(hca.paged_hybrid_decode_workspace(B, Hq, d, lay.Lmax, lay.m, w.window, k))
        hca.paged_hybrid_decode(lay.q, lay.kv, tab, lay.win, wtab, lay.lens, lay.Lmax, lay.m, w.window, sel, sel_n,
                                1.0 / math.sqrt(d), w.theta, out, lse, ws)
    else:
        for b in rows:
            Lb = int(lay.lens_np[b])
            ws = hca.workspace(hca.paged_hybrid_decode_workspace(1, Hq, d, Lb, lay.m, w.window, k))
            hca.paged_hybrid_decode(lay.q[b: b + 1], lay.kv, tab[b: b + 1], lay.win, wtab[b: b + 1],
                                    lay.lens[b: b + 1], Lb, lay.m, w.window,
                                    None if sel is None else sel[b: b + 1], None if sel_n is None else sel_n[b: b + 1],
                                    1.0 / math.sqrt(d), w.theta, out[b: b + 1], lse[b: b + 1], ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("li", [0, 1], ids=["c4a", "c128a"])
def test_mixed_batch(li):
    import decode_attention_compressed_amd as hca

    w = synth.workload(3)
    kind = w.layers[li]
    lay = MixedLayer(hca, w, li)
    lens, B = lay.lens_np, w.B
    assert (lens % BLOCK != 0).all() and lens.min() >= 256 and lens.max() <= 131072
    order = np.argsort(lens)
    others = [b for b in range(B) if b not in lay.members]
    sample = sorted({int(order[0]), int(order[-1]), lay.members[0], lay.members[-1], others[len(others) // 2],
                     int(order[B // 3])})
    H.flush(f"mixed batch {kind.name}: lens {int(lens.min())}..{int(lens.max())}, members {lay.members}, "
            f"sampled {sample}")
    rng = np.random.default_rng(3003 + li)
    # entries of sampled groups (the prefix's among them for the members)
    for b in sample:
        N = int(lay.N[b])
        js = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 10)]))
        got = lay.ent[b, torch.from_numpy(js).cuda()].cpu().numpy()
        for r, j in enumerate(js):
            ref = _oracle_entries(lay, b, int(j), int(j) + 1)
            assert H.rel_err_rows(got[r][None], ref) <= H.ENTRY_TOL, (b, int(j))

    # the oracle's pools for the sampled sequences (the prefix pages of the
    # members are the same physical pages, with the same contents)
    spec = lay.spec()
    kv_ref = paging.Pool(w.kv_dtype, lay.P, lay.epp, w.d)
    win_ref = paging.Pool(w.kv_dtype, lay.PW, BLOCK, w.d)
    for b in sample:
        L, N = int(lens[b]), int(lay.N[b])
        paging.write_run(kv_ref, lay.table[b], 0, _oracle_entries(lay, b, 0, N).astype(np.float32))
        xw = lay.x[b, lay.t0[b]: L].view(torch.int16).cpu().numpy().view(np.uint16)
        rows = compressor.window_rows(codecs.bf16_decode(xw), int(lay.t0[b]), w.theta)
        paging.write_run(win_ref, lay.wtable[b], int(lay.t0[b]), rows.astype(np.float32))

    sel = sel_n = None
    sel_ref = {}
    if kind.topk is not None:
        k = kind.topk
        idx_ref = paging.Pool(kind.idx_dtype, lay.P, lay.epp, kind.d_idx)
        clean = []
        for b in sample:
            N = int(lay.N[b])
            keys_b = lay.keys[b, :N].cpu().numpy()
            paging.write_run(idx_ref, lay.table[b], 0, keys_b)
            qi, wi = codecs.bf16_decode(lay.qi_np[b]), lay.wi_np[b].astype(np.float64)
            ok = False
            for attempt in range(20):
                s = indexer.scores(qi, wi, paging.decode_rows(idx_ref, lay.table[b], np.arange(N)))
                if k >= N or indexer.kth_margin(s, k) >= H.MARGIN:
                    ok = True
                    break
                srt = np.sort(s)[::-1]
                near = np.nonzero(np.abs(s - 0.5 * (srt[k - 1] + srt[k])) < 4 * H.MARGIN)[0]
                if (near < lay.npre).any() and b in lay.members:
                    break  # a shared key near the cut: left as is, this sequence's set is not compared
                new = gen.redraw_keys(w, li, b, near, kind.d_idx, attempt)
                keys_b[near] = new
                lay.keys[b, torch.from_numpy(near).cuda()] = torch.from_numpy(new).cuda()
                paging.write_run(idx_ref, lay.table[b], 0, keys_b)
            # the GPU pages of this sequence from its (possibly re-drawn) keys
            e0 = lay.npre if (b in lay.members and b != lay.members[0]) else 0
            hca.kv_quantize_page(lay.keys[b: b + 1, e0:N].contiguous(), _dev(np.array([e0], np.int32)),
                                 _dev(np.array([N - e0], np.int32)), N - e0, _dev(lay.table[b: b + 1]), lay.idx)
            sel_ref[b] = indexer.topk(s, k)
            if ok:
                clean.append(b)
        torch.cuda.synchronize()
        ws = hca.workspace(hca.indexer_topk_workspace(B, lay.Lmax, kind.m, k))
        sel = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
        sel_n = torch.zeros((B,), dtype=torch.int32, device="cuda")
        hca.indexer_topk(_dev(lay.qi_np.view(np.int16)), _dev(lay.wi_np), lay.idx, _dev(lay.table), lay.lens,
                         lay.Lmax, kind.m, k, sel, sel_n, ws)
        torch.cuda.synchronize()
        got_sel, got_n = sel.cpu().numpy(), sel_n.cpu().numpy()
        assert (got_n == np.minimum(k, lay.N)).all()
        assert len(clean) >= len(sample) - 2, clean
        for b in clean:
            want = sel_ref[b]
            assert got_n[b] == len(want) and np.array_equal(got_sel[b, : got_n[b]], want), b
        # the attention takes the oracle's selection for the sampled sequences
        sel_h = got_sel.copy()
        for b in sample:
            sel_h[b] = -1
            sel_h[b, : len(sel_ref[b])] = sel_ref[b]
        sel = _dev(sel_h)
        sel_n = _dev(np.array([np.count_nonzero(r >= 0) for r in sel_h], np.int32))
    else:
        for b in sample:
            sel_ref[b] = np.arange(int(lay.N[b]))

    # the batch against each sequence alone (GPU pages), every sequence
    got_b, lse_b = _attend_batch(hca, lay, sel, sel_n)
    got_1, lse_1 = _attend_batch(hca, lay, sel, sel_n, rows=range(B))
    for b in range(B):
        assert H.rel_err_rows(got_b[b], got_1[b]) <= H.ATTN_TOL, b
        assert np.allclose(lse_b[b], lse_1[b], rtol=0, atol=1e-3), b

    # sampled sequences against the oracle: the GPU reads the oracle's pages
    for b in sample:
        need = np.unique(np.concatenate([sel_ref[b] // lay.epp]))
        phys = lay.table[b][need]
        lay.kv.codes[torch.from_numpy(phys.astype(np.int64)).cuda()] = torch.from_numpy(kv_ref.codes[phys]).cuda()
        lay.kv.scales[torch.from_numpy(phys.astype(np.int64)).cuda()] = torch.from_numpy(kv_ref.scales[phys]).cuda()
        wp = lay.wtable[b][np.arange(int(lay.t0[b]) // BLOCK, -(-int(lens[b]) // BLOCK))]
        lay.win.codes[torch.from_numpy(wp.astype(np.int64)).cuda()] = torch.from_numpy(win_ref.codes[wp]).cuda()
        lay.win.scales[torch.from_numpy(wp.astype(np.int64)).cuda()] = torch.from_numpy(win_ref.scales[wp]).cuda()
    torch.cuda.synchronize()
    got, got_lse = _attend_batch(hca, lay, sel, sel_n)
    for b in sample:
        q = codecs.bf16_decode(lay.q_np[b])
        ref, ref_lse, _ = pipeline.attend(spec, int(lens[b]), q, kv_ref, lay.table[b], win_ref, lay.wtable[b],
                                          sel_ref[b])
        err = H.rel_err_rows(got[b], ref)
        H.flush(f"  sequence {b} (L={int(lens[b])}): attention rel err {err:.2e}")
        assert err <= H.ATTN_TOL, b
        assert np.allclose(got_lse[b], ref_lse, rtol=0, atol=1e-3), b
    del lay
    torch.cuda.empty_cache()
