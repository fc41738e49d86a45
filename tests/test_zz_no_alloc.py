"""paged_hybrid_decode_noalloc (the library's static per-GPU scratch instead of a
workspace) against paged_hybrid_decode on the same inputs, through the C ABI:
two calls in a row, the second with a smaller input, and a shape past the
scratch's size rejected before any launch."""

import numpy as np
import pytest
import torch

import decode_attention_compressed_amd as hca
import synth
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _inputs(kind, lens, d=512, Hh=64, window=128):
    w = synth.Workload(111, "noalloc", len(lens), None, d, Hh, window, "fp8", [kind])
    sd = H.SeqData(w, 0, lens)
    if kind.topk is not None:
        assert min(sd.enforce_margin()) >= H.MARGIN
        sel_list = [sd.oracle_select(b) for b in range(sd.B)]
        k = max(1, max(len(s) for s in sel_list))
        sel = np.full((sd.B, k), -1, np.int32)
        for b, s in enumerate(sel_list):
            sel[b, : len(s)] = s
        sel_d, seln_d = H.to_dev(sel), H.to_dev(np.array([len(s) for s in sel_list], np.int32))
    else:
        sel_list, k, sel_d, seln_d = None, 0, None, None
    dev = dict(q=H.to_dev(sd.q.view(np.int16)), kv=H.upload_pool(sd.kv), win=H.upload_pool(sd.win),
               table=H.to_dev(sd.table), wtable=H.to_dev(sd.wtable), lens=H.to_dev(sd.lens), sel=sel_d, sel_n=seln_d)
    return sd, sel_list, k, dev


def _call(fn, sd, k, dev, ws=None):
    B, d, Hh = sd.B, sd.w.d, sd.w.H
    out = torch.full((B, Hh, d), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hh), 7.0, dtype=torch.float32, device="cuda")
    o8 = torch.full((B, Hh, d), 0x55, dtype=torch.uint8, device="cuda")
    o8s = torch.full((B, Hh), -1.0, dtype=torch.float32, device="cuda")
    args = (dev["q"], dev["kv"], dev["table"], dev["win"], dev["wtable"], dev["lens"], H.max_len(sd.lens), sd.kind.m,
            sd.w.window, dev["sel"], dev["sel_n"], H.scale_for(d), sd.w.theta, out, lse)
    if ws is None:
        fn(*args, out_fp8=o8, out_scale=o8s)
    else:
        fn(*args, ws, out_fp8=o8, out_scale=o8s)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy(), o8.cpu().numpy(), o8s.cpu().numpy()


def test_noalloc_matches_workspace_entry_point_twice():
    c4a = synth.LayerKind("c4a", 4, 2048, "fp8", 128, 16, overlap=0)
    c128a = synth.LayerKind("c128a", 128, None)
    cases = [(c4a, [70001, 9000, 3001, 20000]), (c128a, [65536, 1000])]  # the second call is smaller
    for kind, lens in cases:
        H.flush(f"noalloc {kind.name} lens={lens}")
        sd, sel_list, k, dev = _inputs(kind, lens)
        need = hca.paged_hybrid_decode_workspace(sd.B, sd.w.H, sd.w.d, H.max_len(lens), kind.m, sd.w.window, k)
        assert 0 < need <= hca.paged_hybrid_decode_noalloc_max_bytes()
        ws = hca.workspace(need)
        ref = _call(hca.paged_hybrid_decode, sd, k, dev, ws)
        got = _call(hca.paged_hybrid_decode_noalloc, sd, k, dev)
        # the same kernels and plan: identical bytes in every output
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)
        # and the oracle's result within the attention tolerance
        for b in range(sd.B):
            sel = sel_list[b] if sel_list is not None else sd.oracle_select(b)
            o_ref, lse_ref, _ = sd.oracle_attend(b, sel)
            assert H.rel_err_rows(got[0][b], o_ref) <= H.ATTN_TOL, b
            assert np.allclose(got[1][b], lse_ref, rtol=0, atol=1e-3), b


def test_noalloc_rejects_shapes_past_its_scratch():
    cap = hca.paged_hybrid_decode_noalloc_max_bytes()
    B, Hh, d, L = 64, 128, 512, 1 << 20
    assert hca.paged_hybrid_decode_workspace(B, Hh, d, L, 128, 128, 0) > cap
    q = torch.zeros((B, Hh, d), dtype=torch.int16, device="cuda")
    kv = hca.PagedCache.empty(4, 2, d, "fp8")
    win = hca.PagedCache.empty(4, 256, d, "fp8")
    tab = torch.zeros((B, L // 256), dtype=torch.int32, device="cuda")
    lens = torch.full((B,), L, dtype=torch.int32, device="cuda")
    out = torch.zeros((B, Hh, d), dtype=torch.float32, device="cuda")
    with pytest.raises(hca.HcaError) as e:
        hca.paged_hybrid_decode_noalloc(q, kv, tab, win, tab, lens, L, 128, 128, None, None, 0.04, 1e6, out, None)
    assert e.value.status == 3  # HCA_ERR_WORKSPACE
    torch.cuda.synchronize()
