"""Many decode steps through the fused update, as a decode loop runs it.

Two layers (c4a: 8-token windows at stride 4, RMSNorm, fp8 entries, fp8
indexer keys; c128a: 128-token groups with a running fold state) start from a
GPU prefill and then take one token per step for a few hundred steps, crossing
group, page and window-block boundaries: per step one kv_compress_insert_jobs
launch per layer (window insert, the open entry, the open indexer page), the
rings and update states kept the way a caller keeps them.  Every step's open
entry must match the oracle's one-shot fold of the whole context, and at the
end every page the steps wrote must hold the oracle's rows (within the entry
tolerance plus half a code step), the indexer pages bit-exactly the oracle's
quantization of the same keys."""

import numpy as np
import pytest
import torch

from oracle import codecs, compressor, paging
from synth import gen

from tests import helpers as H

pytestmark = pytest.mark.gpu

BLOCK = 256


def _oracle_entries(x, z, beta, m, o, gamma, L):
    if o > 0:
        return compressor.compress_overlap(x[:L], z[:L], beta, m, o, 1e6, gamma=gamma, eps=1e-6)
    return compressor.compress(x[:L], z[:L], beta, m, 1e6, gamma=gamma, eps=1e-6)


@pytest.mark.parametrize("m,o", [(4, 4), (128, 0)])
def test_decode_loop_matches_one_shot(m, o):
    import decode_attention_compressed_amd as hca

    H.flush(f"decode loop m={m} overlap={o}")
    rng = np.random.default_rng(91 + m)
    B, d, di, steps = 2, 128, 64, 300
    L0 = np.array([BLOCK * 3 - 37, 1000 + (m - 5 if m > 4 else 1)], np.int64)  # crosses a page start / a group start
    Lmax = int(L0.max()) + steps
    nb = Lmax // BLOCK + 2
    epp = BLOCK // m
    table = rng.permutation(B * nb).reshape(B, nb).astype(np.int32)
    wtable = rng.permutation(B * nb).reshape(B, nb).astype(np.int32)
    # the whole contexts' inputs, drawn up front (the oracle folds them one-shot)
    xs = gen.to_bf16_bits(rng.standard_normal((B, Lmax, d)).astype(np.float32))
    zs = rng.standard_normal((B, Lmax)).astype(np.float32)
    keys = rng.standard_normal((B, Lmax // m + 2, di)).astype(np.float32)
    beta = (rng.standard_normal(m + o) * 0.1).astype(np.float32)
    gam = rng.uniform(0.5, 1.5, d).astype(np.float32)
    xf = codecs.bf16_decode(xs)
    dev = H.to_dev
    kv = hca.PagedCache.empty(B * nb, epp, d, "fp8")
    win = hca.PagedCache.empty(B * nb, BLOCK, d, "fp8")
    idx = hca.PagedCache.empty(B * nb, epp, di, "fp8")
    # prefill: every entry, window block and key page of the starting contexts
    pre_ent, pre_win = [], []
    for b in range(B):
        L = int(L0[b])
        N = -(-L // m)
        ent = torch.zeros((1, N, d), dtype=torch.float32, device="cuda")
        hca.kv_compress(dev(xs[b:b + 1, :L].view(np.int16)), dev(zs[b:b + 1, :L]), dev(beta), dev(np.zeros(1, np.int32)),
                        dev(np.array([L], np.int32)), m, 1e6, ent, L, norm_gamma=dev(gam), overlap=o)
        hca.kv_quantize_page(ent, dev(np.zeros(1, np.int32)), dev(np.array([N], np.int32)), N, dev(table[b:b + 1]), kv)
        pre_ent.append(ent)
        hca.kv_quantize_page(dev(keys[b:b + 1, :N]), dev(np.zeros(1, np.int32)), dev(np.array([N], np.int32)), N,
                             dev(table[b:b + 1]), idx)
        t0 = BLOCK * ((L - 1) // BLOCK)
        wr = torch.zeros((1, L - t0, d), dtype=torch.float32, device="cuda")
        hca.kv_compress(dev(xs[b:b + 1, t0:L].view(np.int16)), dev(zs[b:b + 1, t0:L]), dev(np.zeros(1, np.float32)),
                        dev(np.array([t0], np.int32)), dev(np.array([L - t0], np.int32)), 1, 1e6, wr, L - t0)
        hca.kv_quantize_page(wr, dev(np.array([t0], np.int32)), dev(np.array([L - t0], np.int32)), L - t0,
                             dev(wtable[b:b + 1]), win)
        pre_win.append(wr)
    # the caller's decode state: the open pages' staging (the rows the prefill
    # quantized them from), rings, update state
    stage = torch.zeros((B, epp, d), dtype=torch.float32, device="cuda")
    istage = torch.zeros((B, epp, di), dtype=torch.float32, device="cuda")
    wstage = torch.zeros((B, BLOCK, d), dtype=torch.float32, device="cuda")
    for b in range(B):
        L = int(L0[b])
        j = (L - 1) // m
        e0 = epp * (j // epp)
        stage[b, : j - e0 + 1] = pre_ent[b][0, e0: j + 1]
        istage[b, : j - e0 + 1] = dev(keys[b, e0: j + 1])
        wstage[b, : pre_win[b].shape[1]] = pre_win[b][0]
    state = torch.zeros((B, 4 + (2 * (4 + d) if m > 16 else 0)), dtype=torch.float32, device="cuda")
    tab, wtab, beta_d, gam_d = dev(table), dev(wtable), dev(beta), dev(gam)
    L = L0.copy()
    for step in range(steps):
        L += 1
        p0 = (m * ((L - 1) // m)).astype(np.int32)
        ntok = (L - p0).astype(np.int32)
        j = p0 // m
        e0 = (epp * (j // epp)).astype(np.int32)
        we0 = (BLOCK * ((L - 1) // BLOCK)).astype(np.int32)
        ring = np.zeros((B, o + m, d), np.uint16)
        ringz = np.zeros((B, o + m), np.float32)
        for b in range(B):
            lo = max(0, int(p0[b]) - o)
            ring[b, o - (int(p0[b]) - lo): o + ntok[b]] = xs[b, lo: L[b]]
            ringz[b, o - (int(p0[b]) - lo): o + ntok[b]] = zs[b, lo: L[b]]
            if ntok[b] == 1:  # a new entry: its key row joins the open indexer page
                if j[b] % epp == 0:
                    istage[b].zero_()
                istage[b, j[b] - e0[b]] = dev(keys[b, j[b]])
            if (L[b] - 1) % BLOCK == 0:
                wstage[b].zero_()
        # every tensor a job names stays referenced until the launch is enqueued
        a = dict(rd=dev(ring.view(np.int16)), rz=dev(ringz),
                 xl=dev(xs[np.arange(B), L - 1][:, None].view(np.int16).copy()),
                 zl=dev(zs[np.arange(B), L - 1][:, None].copy()), wpos=dev((L - 1).astype(np.int32)), we0=dev(we0),
                 zero1=dev(np.zeros(1, np.float32)), one=dev(np.ones(B, np.int32)), p0=dev(p0), e0=dev(e0),
                 ntok=dev(ntok))
        jobs = [hca.insert_job(wstage, a["wpos"], a["we0"], wtab, win, 1, x=a["xl"], gate_logit=a["zl"],
                               pos_bias=a["zero1"], ntok=a["one"], rope_theta=1e6, append=True),
                hca.insert_job(stage, a["p0"], a["e0"], tab, kv, m, x=a["rd"][:, o:], gate_logit=a["rz"][:, o:],
                               pos_bias=beta_d, ntok=a["ntok"], rope_theta=1e6, append=True, norm_gamma=gam_d,
                               overlap=o, fold_state=state),
                hca.insert_job(istage, a["p0"], a["e0"], tab, idx, m, append=True)]
        hca.kv_compress_insert_jobs(jobs, B)
        torch.cuda.synchronize()
        if step % 7 == 0 or step == steps - 1:
            sf = stage.cpu().numpy()
            for b in range(B):
                want = _oracle_entries(xf[b], zs[b], beta, m, o, gam, int(L[b]))[j[b]]
                assert H.rel_err_rows(sf[b, j[b] - e0[b]][None], want[None]) <= H.ENTRY_TOL, (step, b)
    torch.cuda.synchronize()
    # every page the loop wrote holds the oracle's rows; indexer pages are bit-exact
    kvh = H.download_pool(kv, paging.Pool("fp8", B * nb, epp, d))
    wh = H.download_pool(win, paging.Pool("fp8", B * nb, BLOCK, d))
    ih = H.download_pool(idx, paging.Pool("fp8", B * nb, epp, di))
    iref = paging.Pool("fp8", B * nb, epp, di)
    for b in range(B):
        Lb = int(L[b])
        N = -(-Lb // m)
        ent = _oracle_entries(xf[b], zs[b], beta, m, o, gam, Lb)
        paging.write_run(iref, table[b], 0, keys[b, :N])
        for lb in range(int(L0[b]) // BLOCK, -(-Lb // BLOCK)):  # the blocks the loop reached
            r0, r1 = lb * epp, min(N, (lb + 1) * epp)
            if r1 <= r0:
                continue
            ph = int(table[b, lb])
            assert H.quantized_rows_close("fp8", kvh.codes[ph, : r1 - r0], kvh.scales[ph], ent[r0:r1]), (b, lb)
            assert np.array_equal(ih.codes[ph, : r1 - r0], iref.codes[ph, : r1 - r0]) and ih.scales[ph] == iref.scales[ph]
            t0, t1 = lb * BLOCK, min(Lb, (lb + 1) * BLOCK)
            wrows = compressor.window_rows(xf[b, t0:t1], t0, 1e6)
            pw = int(wtable[b, lb])
            if lb >= (Lb - 1) // BLOCK - 1:  # the window blocks the loop kept whole
                assert H.quantized_rows_close("fp8", wh.codes[pw, : t1 - t0], wh.scales[pw], wrows), (b, lb)
    if m > 16:
        return  # c128a: a running fold state; its pages are checked against the oracle above
    # c4a has no fold state: each entry is refolded from its tokens, so every
    # page the loop wrote must hold the same bytes as the GPU's one-shot prefill
    # of the final context, both the two-launch form (kv_compress +
    # kv_quantize_page) and the fused kv_prefill_pages; the window pages as the
    # one-shot fold of their tokens (m = 1) quantized whole
    kv1 = hca.PagedCache.empty(B * nb, epp, d, "fp8")
    kv2 = hca.PagedCache.empty(B * nb, epp, d, "fp8")
    win1 = hca.PagedCache.empty(B * nb, BLOCK, d, "fp8")
    for b in range(B):
        Lb = int(L[b])
        N = -(-Lb // m)
        ent = torch.zeros((1, N, d), dtype=torch.float32, device="cuda")
        xb, zb = dev(xs[b:b + 1, :Lb].view(np.int16)), dev(zs[b:b + 1, :Lb])
        z1, n1 = dev(np.zeros(1, np.int32)), dev(np.array([Lb], np.int32))
        hca.kv_compress(xb, zb, beta_d, z1, n1, m, 1e6, ent, Lb, norm_gamma=gam_d, overlap=o)
        hca.kv_quantize_page(ent, z1, dev(np.array([N], np.int32)), N, dev(table[b:b + 1]), kv1)
        hca.kv_prefill_pages(xb, zb, beta_d, z1, n1, m, 1e6, Lb, dev(table[b:b + 1]), kv2, norm_gamma=gam_d, overlap=o)
        for lb in range((int(L0[b]) - 1) // BLOCK, -(-Lb // BLOCK)):
            t0, t1 = lb * BLOCK, min(Lb, (lb + 1) * BLOCK)
            wr = torch.zeros((1, t1 - t0, d), dtype=torch.float32, device="cuda")
            p0w, nw = dev(np.array([t0], np.int32)), dev(np.array([t1 - t0], np.int32))
            hca.kv_compress(dev(xs[b:b + 1, t0:t1].view(np.int16)), dev(zs[b:b + 1, t0:t1]), dev(np.zeros(1, np.float32)),
                            p0w, nw, 1, 1e6, wr, t1 - t0)
            hca.kv_quantize_page(wr, p0w, nw, t1 - t0, dev(wtable[b:b + 1]), win1)
    torch.cuda.synchronize()
    k1 = H.download_pool(kv1, paging.Pool("fp8", B * nb, epp, d))
    k2 = H.download_pool(kv2, paging.Pool("fp8", B * nb, epp, d))
    w1 = H.download_pool(win1, paging.Pool("fp8", B * nb, BLOCK, d))
    for b in range(B):
        Lb = int(L[b])
        N = -(-Lb // m)
        for lb in range(int(L0[b]) // BLOCK, -(-Lb // BLOCK)):
            r0, r1 = lb * epp, min(N, (lb + 1) * epp)
            if r1 <= r0:
                continue
            ph = int(table[b, lb])
            for ref, what in ((k1, "kv_compress + kv_quantize_page"), (k2, "kv_prefill_pages")):
                assert np.array_equal(kvh.codes[ph, : r1 - r0], ref.codes[ph, : r1 - r0]), (b, lb, what)
                assert kvh.scales[ph] == ref.scales[ph], (b, lb, what)
        for lb in range((int(L0[b]) - 1) // BLOCK, -(-Lb // BLOCK)):
            t0, t1 = lb * BLOCK, min(Lb, (lb + 1) * BLOCK)
            pw = int(wtable[b, lb])
            assert np.array_equal(wh.codes[pw, : t1 - t0], w1.codes[pw, : t1 - t0]), (b, lb, "window")
            assert wh.scales[pw] == w1.scales[pw], (b, lb, "window")
