"""GPU parity of every entry point against the CPU oracle (needs an MI355X).

Stage-isolated: each kernel gets inputs the oracle built (pages, selections)
and is compared with the oracle's result for them.  Sizes span several tiles
and blocks with ragged tails; the full workload sizes are covered in
test_gpu_workloads.py.
"""

import numpy as np
import pytest
import torch

import synth
from oracle import codecs, compressor, indexer, paging
from synth import gen
from tests import helpers as H

pytestmark = pytest.mark.gpu

hca = pytest.importorskip("decode_attention_compressed_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    hca.lib()


# ----------------------------------------------------------------- hardware layout probes


@pytest.mark.parametrize("kind", [0, 1])
def test_probe_mfma_16x16x32_layout(kind):
    H.flush(f"probe mfma kind={kind}")
    rng = np.random.default_rng(31)
    A = rng.integers(-4, 5, (16, 32)).astype(np.float32)
    B = rng.integers(-4, 5, (32, 16)).astype(np.float32)
    if kind == 0:
        a16 = torch.from_numpy(A).half().view(torch.int16)
        b16 = torch.from_numpy(B).half().view(torch.int16)
    else:
        a16 = torch.from_numpy(A).bfloat16().view(torch.int16)
        b16 = torch.from_numpy(B).bfloat16().view(torch.int16)
    D = torch.zeros((16, 16), dtype=torch.float32, device="cuda")
    a_d, b_d = a16.cuda(), b16.cuda()
    assert hca.lib().hca_probe_mfma(a_d.data_ptr(), b_d.data_ptr(), D.data_ptr(), kind, None) == 0
    torch.cuda.synchronize()
    assert np.array_equal(D.cpu().numpy(), A @ B)


def test_probe_hw_decoders_are_exact():
    H.flush("probe decode fp8/fp4")
    codes = np.arange(256, dtype=np.uint8)
    out = torch.zeros(256, dtype=torch.float32, device="cuda")
    assert hca.lib().hca_probe_decode(H.to_dev(codes).data_ptr(), out.data_ptr(), 256, 0, None) == 0
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    finite = np.isfinite(codecs.E4M3_TABLE)
    assert np.array_equal(got[finite], codecs.E4M3_TABLE[finite])
    out4 = torch.zeros(512, dtype=torch.float32, device="cuda")
    assert hca.lib().hca_probe_decode(H.to_dev(codes).data_ptr(), out4.data_ptr(), 512, 1, None) == 0
    torch.cuda.synchronize()
    got4 = out4.cpu().numpy().astype(np.float64)
    want = np.empty(512)
    want[0::2] = codecs.E2M1_TABLE[codes & 0xF]
    want[1::2] = codecs.E2M1_TABLE[codes >> 4]
    assert np.array_equal(got4, want)


def test_probe_hw_e4m3_encoder_equals_exact_encoder_everywhere():
    # every binary32 value (NaNs aside) through the hardware E4M3 conversion
    # after its saturating clamp and through the exact-step encoder, which the
    # host tests pin against the oracle over the same sweep: the kernels use
    # the hardware one
    H.flush("probe e4m3 encoders, all binary32 values")
    res = torch.zeros(2, dtype=torch.int32, device="cuda")
    for part in range(4):
        assert hca.lib().hca_probe_e4m3_sweep(part << 30, 1 << 30, res.data_ptr(), None) == 0
    torch.cuda.synchronize()
    bad, last = (int(v) & 0xFFFFFFFF for v in res.cpu().numpy())
    assert bad == 0, (bad, hex(last))


# ----------------------------------------------------------------- kv_quantize_page


@pytest.mark.parametrize("use_ws", [False, True])
@pytest.mark.parametrize("dtype,epp,dim", [("fp8", 64, 512), ("fp8", 2, 512), ("fp8", 256, 128), ("fp4", 64, 128),
                                           ("bf16", 64, 128), ("fp4", 64, 64), ("fp8", 64, 136), ("fp8", 256, 512),
                                           ("fp4", 64, 256)])
def test_quantize_pages_bit_exact(dtype, epp, dim, use_ws):
    H.flush(f"quantize {dtype} epp={epp} dim={dim} ws={use_ws}")
    rng = np.random.default_rng(41)
    lens = np.array([epp * 5 + 7, epp * 3, 1, epp * 2 - 1])
    B = len(lens)
    max_ne = int(lens.max())
    nb = -(-max_ne // epp)
    perm = rng.permutation(B * nb + 3)
    table = perm[: B * nb].reshape(B, nb).astype(np.int32)
    src = (rng.standard_normal((B, max_ne, dim)) * rng.uniform(0.01, 3, (B, 1, 1))).astype(np.float32)
    src[1, : epp] = 0.0  # an all-zero page: fp8 scale 1, fp4 scale codes 0
    src[2, 0, :5] = [448 * 3, -1e-9, 0.0, -0.0, 2.0 ** -12]
    ref = paging.Pool(dtype, B * nb + 3, epp, dim)
    for b in range(B):
        paging.write_run(ref, table[b], 0, src[b, : lens[b]])
    dst = hca.PagedCache.empty(B * nb + 3, epp, dim, dtype)
    dst.codes.fill_(0x5A)  # slots past the valid rows must come back zeroed
    ws = None
    if use_ws:
        nws = hca.kv_quantize_page_workspace(B, max_ne, dst)
        assert (nws > 0) == (dtype == "fp8")
        ws = torch.full((max(nws, 1),), 0xC3, dtype=torch.uint8, device="cuda")  # no initial contents needed
    hca.kv_quantize_page(H.to_dev(src), H.to_dev(np.zeros(B, np.int32)), H.to_dev(lens.astype(np.int32)), max_ne,
                         H.to_dev(table), dst, ws=ws)
    torch.cuda.synchronize()
    got = H.download_pool(dst, ref)
    for b in range(B):
        for p in range(-(-lens[b] // epp)):
            phys = table[b, p]
            nv = min(epp, lens[b] - p * epp)
            assert np.array_equal(got.codes[phys, :nv], ref.codes[phys, :nv]), (b, p)
            assert not got.codes[phys, nv:].any(), (b, p)
            if dtype == "fp8":
                assert got.scales[phys] == ref.scales[phys], (b, p)
            elif dtype == "fp4":
                assert np.array_equal(got.scales[phys, :nv], ref.scales[phys, :nv]), (b, p)


@pytest.mark.parametrize("use_ws", [False, True])
def test_quantize_fp8_values_at_rounding_midpoints(use_ws):
    # the page encoder divides by the page scale through a reciprocal and takes
    # the exact quotient only near E4M3's rounding points: here every value of
    # a page is within a few units in the last place of s times an E4M3
    # midpoint (every midpoint of the normal range, both signs), for scales of
    # several magnitudes and mantissas, and the codes must equal the oracle's
    # RNE(fl32(x / s)) bit for bit
    H.flush(f"quantize fp8 at rounding midpoints ws={use_ws}")
    rng = np.random.default_rng(43)
    epp, dim = 64, 512
    mids = []
    for e in range(-6, 9):
        for mant in range(8):
            lo = 2.0 ** e * (1 + mant / 8)
            mids.append(lo * (1 + 1 / 16))  # halfway to the next E4M3 value
    mids = np.array([m for m in mids if m < 448], np.float64)
    pages = []
    for amax in [448.0, 1.0, 3.0e-4, 7.77, 1234.5678, 0.1]:
        s = np.float32(np.float32(amax) / np.float32(448))
        vals = []
        for m in mids:
            for k in range(-10, 11):  # x / s from about 11 units below the midpoint to 11 above, the midpoint itself among them
                vals.append(np.float32(m) * s * np.float32(1 + k * 2.0 ** -23))
        vals = np.array(vals, np.float32)
        vals = vals * rng.choice([-1, 1], vals.shape).astype(np.float32)
        flat = np.zeros(epp * dim, np.float32)
        flat[0] = np.float32(amax)  # the page's amax
        flat[1: 1 + min(len(vals), epp * dim - 1)] = vals[: epp * dim - 1]
        pages.append(flat.reshape(epp, dim))
    B = len(pages)
    src = np.stack(pages)  # [B, epp, dim]: one page per sequence
    table = np.arange(B, dtype=np.int32).reshape(B, 1)
    ref = paging.Pool("fp8", B, epp, dim)
    for b in range(B):
        paging.write_run(ref, table[b], 0, src[b])
    assert (np.abs(src).max(axis=(1, 2)) == np.array([448.0, 1.0, 3.0e-4, 7.77, 1234.5678, 0.1], np.float32)).all()
    dst = hca.PagedCache.empty(B, epp, dim, "fp8")
    ws = None
    if use_ws:
        ws = torch.zeros((max(hca.kv_quantize_page_workspace(B, epp, dst), 1),), dtype=torch.uint8, device="cuda")
    lens = np.full(B, epp, np.int32)
    hca.kv_quantize_page(H.to_dev(src), H.to_dev(np.zeros(B, np.int32)), H.to_dev(lens), epp, H.to_dev(table), dst, ws=ws)
    torch.cuda.synchronize()
    got = H.download_pool(dst, ref)
    for b in range(B):
        assert got.scales[b] == ref.scales[b], b
        bad = np.nonzero(got.codes[b] != ref.codes[b])
        assert bad[0].size == 0, (b, bad[0][:5], bad[1][:5])


@pytest.mark.parametrize("use_ws", [False, True])
def test_quantize_open_page_run(use_ws):
    # a run that starts at a later page (the decode update's open page), e0 > 0
    H.flush(f"quantize open page ws={use_ws}")
    rng = np.random.default_rng(42)
    epp, dim = 64, 512
    table = np.array([[5, 2, 7, 0], [1, 3, 4, 6]], np.int32)
    rows = rng.standard_normal((2, 40, dim)).astype(np.float32)
    e0 = np.array([128, 64], np.int32)
    ne = np.array([40, 17], np.int32)
    ref = paging.Pool("fp8", 8, epp, dim)
    for b in range(2):
        paging.write_run(ref, table[b], int(e0[b]), rows[b, : ne[b]])
    dst = hca.PagedCache.empty(8, epp, dim, "fp8")
    ws = hca.workspace(hca.kv_quantize_page_workspace(2, 40, dst)) if use_ws else None
    hca.kv_quantize_page(H.to_dev(rows), H.to_dev(e0), H.to_dev(ne), 40, H.to_dev(table), dst, ws=ws)
    got = H.download_pool(dst, ref)
    assert np.array_equal(got.codes[7, :40], ref.codes[7, :40]) and got.scales[7] == ref.scales[7]
    assert np.array_equal(got.codes[3, :17], ref.codes[3, :17]) and got.scales[3] == ref.scales[3]


# ----------------------------------------------------------------- kv_compress


# groups0 sets the first sequence's full groups; a large-m fold takes its row
# group's tokens in batches of 16, so m = 256 (64 tokens per row group at d =
# 128) spans several batches; d = 136 leaves threads of the block idle.
@pytest.mark.parametrize("m,d,groups0", [(4, 512, 37), (128, 512, 37), (4, 128, 37), (1, 512, 37), (16, 64, 37),
                                         (256, 128, 37), (128, 512, 140), (64, 136, 37), (32, 256, 1)])
def test_compress_entries(m, d, groups0):
    H.flush(f"compress m={m} d={d} groups0={groups0}")
    rng = np.random.default_rng(51)
    T = [m * groups0 + (m // 2 + 1 if m > 1 else 0), 3, m * 9, 1]
    B = len(T)
    Tm = max(T)
    x32 = rng.standard_normal((B, Tm, d)).astype(np.float32)
    xb = gen.to_bf16_bits(x32)
    z = rng.standard_normal((B, Tm)).astype(np.float32)
    beta = (rng.standard_normal(m) * 0.1).astype(np.float32)
    pos0 = np.array([0, m * 1000, m * 262143, m * 5], np.int32)
    ntok = np.array(T, np.int32)
    n_out = -(-Tm // m)
    out = torch.zeros((B, n_out, d), dtype=torch.float32, device="cuda")
    hca.kv_compress(H.to_dev(xb.view(np.int16)), H.to_dev(z), H.to_dev(beta), H.to_dev(pos0), H.to_dev(ntok), m, 1e6,
                    out, Tm)
    got = out.cpu().numpy()
    for b in range(B):
        ref = compressor.compress(codecs.bf16_decode(xb[b, : T[b]]), z[b, : T[b]], beta, m, 1e6, pos0=int(pos0[b]))
        assert H.rel_err_rows(got[b, : ref.shape[0]], ref) <= H.ENTRY_TOL, b


# RMS-normalised entries: the row's sum of squares is reduced by an xor
# butterfly inside a wave (d <= 512), across waves (d = 1024, 2048), through
# LDS (d = 136: 17 threads a row), or over the block (m > 16)
@pytest.mark.parametrize("m,d", [(4, 512), (1, 512), (128, 512), (4, 136), (2, 1024), (16, 2048), (256, 128),
                                 (64, 136), (4, 64)])
def test_compress_entries_normalised(m, d):
    H.flush(f"compress normalised m={m} d={d}")
    rng = np.random.default_rng(52)
    T = [m * 37 + (m // 2 + 1 if m > 1 else 0), 3, m * 9, 1]
    B, Tm = len(T), max(T)
    x32 = rng.standard_normal((B, Tm, d)).astype(np.float32) * rng.uniform(0.01, 10.0, (B, Tm, 1)).astype(np.float32)
    xb = gen.to_bf16_bits(x32)
    z = rng.standard_normal((B, Tm)).astype(np.float32)
    beta = (rng.standard_normal(m) * 0.1).astype(np.float32)
    gam = rng.uniform(0.5, 1.5, d).astype(np.float32)
    pos0 = np.array([0, m * 1000, m * 262143, m * 5], np.int32)
    ntok = np.array(T, np.int32)
    out = torch.zeros((B, -(-Tm // m), d), dtype=torch.float32, device="cuda")
    hca.kv_compress(H.to_dev(xb.view(np.int16)), H.to_dev(z), H.to_dev(beta), H.to_dev(pos0), H.to_dev(ntok), m, 1e6,
                    out, Tm, norm_gamma=H.to_dev(gam), norm_eps=1e-6)
    got = out.cpu().numpy()
    for b in range(B):
        ref = compressor.compress(codecs.bf16_decode(xb[b, : T[b]]), z[b, : T[b]], beta, m, 1e6, pos0=int(pos0[b]),
                                  gamma=gam, eps=1e-6)
        assert H.rel_err_rows(got[b, : ref.shape[0]], ref) <= H.ENTRY_TOL, b


# Overlapping windows: each entry also folds the o tokens before its group,
# read at rows -o .. -1 of the run (the buffer holds them before the view
# passed in; for pos0 = 0 those rows hold NaNs, which must never be read).
@pytest.mark.parametrize("m,o,d,norm", [(4, 4, 512, False), (4, 4, 512, True), (4, 4, 136, True), (2, 1, 64, False),
                                        (16, 16, 128, False), (4, 2, 1024, True), (1, 1, 256, False)])
def test_compress_entries_overlap(m, o, d, norm):
    H.flush(f"compress overlap m={m} o={o} d={d} norm={norm}")
    rng = np.random.default_rng(53)
    T = [m * 37 + (m // 2 + 1 if m > 1 else 0), 3, m * 9, 1, 2 * m]
    pos0 = np.array([0, m * 1000, m * 262143, 0, m], np.int32)
    B, Tm = len(T), max(T)
    x32 = rng.standard_normal((B, o + Tm, d)).astype(np.float32)
    xb = gen.to_bf16_bits(x32)
    z = rng.standard_normal((B, o + Tm)).astype(np.float32)
    for b in range(B):
        if pos0[b] == 0:  # positions below 0: never read
            xb[b, :o] = 0x7FC0
            z[b, :o] = np.nan
    beta = (rng.standard_normal(m + o) * 0.1).astype(np.float32)
    gam = rng.uniform(0.5, 1.5, d).astype(np.float32) if norm else None
    xd, zd = H.to_dev(xb.view(np.int16)), H.to_dev(z)
    out = torch.zeros((B, -(-Tm // m), d), dtype=torch.float32, device="cuda")
    hca.kv_compress(xd[:, o:], zd[:, o:], H.to_dev(beta), H.to_dev(pos0), H.to_dev(np.array(T, np.int32)), m, 1e6,
                    out, Tm, norm_gamma=None if gam is None else H.to_dev(gam), overlap=o)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    for b in range(B):
        xs = codecs.bf16_decode(xb[b, o: o + T[b]])
        ref = compressor.compress_overlap(xs, z[b, o: o + T[b]], beta, m, o, 1e6, pos0=int(pos0[b]),
                                          x_prev=codecs.bf16_decode(xb[b, :o]), z_prev=z[b, :o], gamma=gam)
        assert H.rel_err_rows(got[b, : ref.shape[0]], ref) <= H.ENTRY_TOL, b


# ----------------------------------------------------------------- kv_prefill_pages


# The fused prefill against kv_compress + kv_quantize_page on the same inputs
# (identical bytes in every page written) and against the oracle.  Runs start
# at a page (pos0 a multiple of 256, some > 0 with the overlap's tokens before
# them), end mid-page or mid-group, and one is empty.  The shapes take the
# small-group path with a row sum by xor butterfly (d = 128, 256, 512), across
# the LDS (d = 136) and the large-group path (m = 64, 128, 256).
@pytest.mark.parametrize("m,o,d,dtype,norm", [
    (4, 4, 512, "fp8", True), (128, 0, 512, "fp8", True), (4, 0, 128, "bf16", False), (16, 16, 128, "fp8", False),
    (4, 2, 136, "fp8", True), (2, 1, 256, "fp8", False), (64, 0, 136, "fp8", True), (256, 0, 128, "bf16", False),
    (4, 4, 512, "bf16", True)])
def test_prefill_pages_matches_two_calls_and_oracle(m, o, d, dtype, norm):
    H.flush(f"prefill pages m={m} o={o} d={d} {dtype} norm={norm}")
    rng = np.random.default_rng(71 + m + d)
    epp = 256 // m
    T = [256 * 3 + 5 * m + (m // 2 + 1 if m > 1 else 0), 256 - 1, 0, 256 * 2, 37]
    pos0 = np.array([0, 256 * 7, 256, 256 * 4000, 0], np.int32)
    B, Tm = len(T), max(T)
    ntok = np.array(T, np.int32)
    x32 = rng.standard_normal((B, o + Tm, d)).astype(np.float32) * rng.uniform(0.1, 4, (B, 1, 1)).astype(np.float32)
    xb = gen.to_bf16_bits(x32)
    z = rng.standard_normal((B, o + Tm)).astype(np.float32)
    beta = (rng.standard_normal(m + o) * 0.1).astype(np.float32)
    gam = rng.uniform(0.5, 1.5, d).astype(np.float32) if norm else None
    nb = int((pos0.astype(np.int64) + Tm).max()) // 256 + 2
    P = B * nb
    table = rng.permutation(P).reshape(B, nb).astype(np.int32)
    xd, zd = H.to_dev(xb.view(np.int16)), H.to_dev(z)
    gd = None if gam is None else H.to_dev(gam)
    args = dict(norm_gamma=gd, overlap=o)
    fused = hca.PagedCache.empty(P, epp, d, dtype)
    fused.codes.fill_(0x5A)  # slots past the valid rows must come back zeroed
    hca.kv_prefill_pages(xd[:, o:], zd[:, o:], H.to_dev(beta), H.to_dev(pos0), H.to_dev(ntok), m, 1e6, Tm,
                         H.to_dev(table), fused, **args)
    n_out = -(-Tm // m)
    ent = torch.zeros((B, n_out, d), dtype=torch.float32, device="cuda")
    hca.kv_compress(xd[:, o:], zd[:, o:], H.to_dev(beta), H.to_dev(pos0), H.to_dev(ntok), m, 1e6, ent, Tm, **args)
    two = hca.PagedCache.empty(P, epp, d, dtype)
    ne = (-(-ntok // m)).astype(np.int32)
    hca.kv_quantize_page(ent, H.to_dev((pos0 // m).astype(np.int32)), H.to_dev(ne), n_out, H.to_dev(table), two)
    torch.cuda.synchronize()
    got_e = ent.cpu().numpy()
    for b in range(B):
        lb0 = int(pos0[b]) // 256
        for p in range(-(-int(ne[b]) // epp)):
            phys = int(table[b, lb0 + p])
            nv = min(epp, int(ne[b]) - p * epp)
            assert torch.equal(fused.codes[phys, :nv], two.codes[phys, :nv]), (b, p)
            assert not fused.codes[phys, nv:].any(), (b, p)
            if dtype == "fp8":
                assert torch.equal(fused.scales[phys], two.scales[phys]), (b, p)
        if ne[b] == 0:
            continue
        # the oracle's entries, and the fused pages decoded against them
        xs = codecs.bf16_decode(xb[b, o: o + T[b]])
        if o > 0:
            ref = compressor.compress_overlap(xs, z[b, o: o + T[b]], beta, m, o, 1e6, pos0=int(pos0[b]),
                                              x_prev=codecs.bf16_decode(xb[b, :o]), z_prev=z[b, :o], gamma=gam)
        else:
            ref = compressor.compress(xs, z[b, : T[b]], beta, m, 1e6, pos0=int(pos0[b]), gamma=gam)
        assert H.rel_err_rows(got_e[b, : ref.shape[0]], ref) <= H.ENTRY_TOL, b
        for p in range(-(-int(ne[b]) // epp)):
            phys = int(table[b, lb0 + p])
            rows = ref[p * epp: (p + 1) * epp]
            codes = fused.codes[phys, : rows.shape[0]].cpu().numpy()
            sc = fused.scales[phys].item() if dtype == "fp8" else None
            assert H.quantized_rows_close(dtype, codes.view(np.uint16) if dtype == "bf16" else codes, sc, rows), (b, p)


def test_prefill_pages_rejects_unsupported_shapes():
    kv = hca.PagedCache.empty(4, 256, 512, "fp8")  # m = 1, 512 dims: a page is more rows than a block holds
    x = torch.zeros((1, 256, 512), dtype=torch.int16, device="cuda")
    z = torch.zeros((1, 256), dtype=torch.float32, device="cuda")
    one = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(hca.HcaError) as e:
        hca.kv_prefill_pages(x, z, torch.zeros(1, device="cuda"), one, one + 256, 1, 1e6, 256,
                             torch.zeros((1, 1), dtype=torch.int32, device="cuda"), kv)
    assert e.value.status == 2  # HCA_ERR_UNSUPPORTED
    fp4 = hca.PagedCache.empty(4, 64, 128, "fp4")
    with pytest.raises(hca.HcaError) as e:
        hca.kv_prefill_pages(x[:, :, :128].contiguous(), z, torch.zeros(4, device="cuda"), one, one + 256, 4, 1e6,
                             256, torch.zeros((1, 1), dtype=torch.int32, device="cuda"), fp4)
    assert e.value.status == 2


# ----------------------------------------------------------------- kv_compress_insert


# Decode steps of one pool: each step adds one token; the fused call must leave
# the same staging rows and page bytes as kv_compress + kv_quantize_page on the
# open page, and those must match the oracle (fold within the entry tolerance,
# page codes bit-exact for the GPU staging rows).  The runs cross a page start
# (the new page's first row), grow an fp8 page scale with a large token, and
# start one page from all-zero rows (scale 1.0, which append mode must not
# trust).  With norm, every folded entry is RMS-normalised before its rotation.
@pytest.mark.parametrize("m,dtype,d,append,norm,o", [
    (1, "fp8", 512, True, False, 0), (1, "fp8", 512, False, False, 0), (4, "fp8", 512, False, False, 0),
    (4, "fp8", 512, True, False, 0), (128, "fp8", 512, True, False, 0), (128, "fp8", 512, False, False, 0),
    (2, "fp8", 136, False, False, 0), (2, "fp8", 512, True, False, 0), (4, "fp4", 128, False, False, 0),
    (1, "fp4", 128, True, False, 0), (4, "bf16", 128, False, False, 0), (1, "bf16", 64, True, False, 0),
    (4, "fp8", 512, True, True, 0), (128, "fp8", 512, True, True, 0), (1, "fp8", 512, True, True, 0),
    (2, "fp8", 136, False, True, 0), (4, "fp4", 128, True, True, 0),
    (4, "fp8", 512, True, True, 4), (4, "fp8", 512, False, False, 4), (4, "fp4", 128, True, False, 4),
    (2, "bf16", 64, False, False, 2), (4, "fp8", 136, True, True, 2)])
def test_compress_insert_matches_two_calls_and_oracle(m, dtype, d, append, norm, o):
    H.flush(f"compress_insert m={m} {dtype} d={d} append={append} norm={norm} overlap={o}")
    rng = np.random.default_rng(61 + m)
    gam = rng.uniform(0.5, 1.5, d).astype(np.float32) if norm else None
    gam_d = H.to_dev(gam) if norm else None
    epp = 256 // m
    B, steps, theta = 3, 7, 1e6
    # lengths before the first step: seq 0 three tokens before a page start,
    # seq 1 empty, seq 2 mid-page (its page begins with all-zero rows)
    L = np.array([256 * 2 - 3, 0, 256 * 5 + 9 * m + 1], np.int64)
    nb = int(L.max() + steps) // 256 + 2
    table = rng.permutation(B * nb + 2)[: B * nb].reshape(B, nb).astype(np.int32)
    P = B * nb + 2
    beta = (rng.standard_normal(m + o) * 0.1).astype(np.float32)
    stage_f = torch.zeros((B, epp, d), dtype=torch.float32, device="cuda")
    pool_f = hca.PagedCache.empty(P, epp, d, dtype)
    pool_f.codes.fill_(0)
    if pool_f.scales is not None:
        pool_f.scales.fill_(0)
    # history of each open page: its earlier rows, quantized as they would have been
    hist = np.zeros((B, epp, d), np.float32)
    for b in range(B):
        j = (L[b]) // m if L[b] % m == 0 else L[b] // m  # the next step's entry
        row = j % epp
        hist[b, :row] = rng.standard_normal((row, d)).astype(np.float32)
        if b == 2:
            hist[b, :row] = 0.0
        stage_f[b] = H.to_dev(hist[b])
        if row > 0:
            e0 = np.array([j - row], np.int32)
            hca.kv_quantize_page(stage_f[b:b + 1], H.to_dev(e0), H.to_dev(np.array([row], np.int32)), epp,
                                 H.to_dev(table[b:b + 1]), pool_f)
    torch.cuda.synchronize()
    ref_rows = hist.astype(np.float64)  # the open pages' rows as the oracle has them
    # append runs keep an update state (the page header: its closed rows' amax)
    state = torch.zeros((B, 4 + (2 * (4 + d) if m > 16 else 0)), dtype=torch.float32, device="cuda") if append else None
    stage_u = stage_f.clone()
    pool_u = hca.PagedCache(pool_f.codes.clone(), None if pool_f.scales is None else pool_f.scales.clone(), epp, d,
                            dtype)
    # the ring of the open group's window: rows 0 .. o-1 the overlap (the tokens
    # before the group: drawn for the starting state, then carried), rows o ..
    # the open group
    ring_x = np.zeros((B, o + m, d), np.float32)
    ring_z = np.zeros((B, o + m), np.float32)
    ring_x[:, :o] = rng.standard_normal((B, o, d))
    ring_z[:, :o] = rng.standard_normal((B, o))
    for step in range(steps):
        L += 1
        pos0 = (m * ((L - 1) // m)).astype(np.int32)
        ntok = (L - pos0).astype(np.int32)
        for b in range(B):
            t = int(ntok[b]) - 1
            if t == 0:
                if step > 0 and o > 0:  # the closed group's last o tokens become the overlap
                    ring_x[b, :o] = ring_x[b, m: m + o].copy()
                    ring_z[b, :o] = ring_z[b, m: m + o].copy()
                ring_x[b, o:] = 0.0
                ring_z[b, o:] = 0.0
            scale = 40.0 if (b == 2 and step == 3) else (0.0 if (b == 2 and step == 0) else 1.0)
            ring_x[b, o + t] = rng.standard_normal(d) * scale
            ring_z[b, o + t] = rng.standard_normal()
        xb = gen.to_bf16_bits(ring_x)
        j = pos0 // m
        e0 = (epp * (j // epp)).astype(np.int32)
        row = j - e0
        xr, zr = H.to_dev(xb.view(np.int16)), H.to_dev(ring_z)
        xd, zd = xr[:, o:], zr[:, o:]  # rows -o .. -1: the overlap
        hca.kv_compress_insert(xd, zd, H.to_dev(beta), H.to_dev(pos0), H.to_dev(ntok), m, theta, stage_f,
                               H.to_dev(e0), H.to_dev(table), pool_f, append=append, norm_gamma=gam_d, overlap=o,
                               fold_state=state if m <= 16 else None)
        for b in range(B):  # the two-call path, one sequence at a time (rows differ)
            hca.kv_compress(xd[b:b + 1], zd[b:b + 1], H.to_dev(beta), H.to_dev(pos0[b:b + 1]),
                            H.to_dev(ntok[b:b + 1]), m, theta, stage_u[b:b + 1, int(row[b]):], m, norm_gamma=gam_d,
                            overlap=o)
            hca.kv_quantize_page(stage_u[b:b + 1], H.to_dev(e0[b:b + 1]), H.to_dev(row[b:b + 1] + 1), epp,
                                 H.to_dev(table[b:b + 1]), pool_u)
        torch.cuda.synchronize()
        sf, su = stage_f.cpu().numpy(), stage_u.cpu().numpy()
        ref_pool = paging.Pool(dtype, P, epp, d)
        got_f = H.download_pool(pool_f, ref_pool)
        got_u = H.download_pool(pool_u, ref_pool)
        for b in range(B):
            r = int(row[b])
            assert np.array_equal(sf[b, : r + 1].view(np.uint32), su[b, : r + 1].view(np.uint32)), (step, b)
            if o > 0:
                ent = compressor.compress_overlap(codecs.bf16_decode(xb[b, o: o + ntok[b]]), ring_z[b, o: o + ntok[b]],
                                                  beta, m, o, theta, pos0=int(pos0[b]),
                                                  x_prev=codecs.bf16_decode(xb[b, :o]), z_prev=ring_z[b, :o],
                                                  gamma=gam, eps=1e-6)
            else:
                ent = compressor.compress(codecs.bf16_decode(xb[b, : ntok[b]]), ring_z[b, : ntok[b]], beta, m, theta,
                                          pos0=int(pos0[b]), gamma=gam, eps=1e-6)
            assert H.rel_err_rows(sf[b, r : r + 1], ent[-1:]) <= H.ENTRY_TOL, (step, b)
            if r == 0:
                ref_rows[b] = 0.0  # a new page
            ref_rows[b, r] = ent[-1]
            phys = int(table[b, e0[b] // epp])
            assert np.array_equal(got_f.codes[phys], got_u.codes[phys]), (step, b)
            if dtype != "bf16":
                assert np.array_equal(got_f.scales[phys], got_u.scales[phys]), (step, b)
            # the stored page against the oracle's rows (its codes are bit-exact
            # against the oracle's quantizer in the kv_quantize_page tests)
            sc = got_f.scales[phys] if dtype == "fp8" else (got_f.scales[phys, : r + 1] if dtype == "fp4" else None)
            assert H.quantized_rows_close(dtype, got_f.codes[phys, : r + 1], sc, ref_rows[b, : r + 1]), (step, b)


# Running fold states (groups of more than 16 tokens): each call folds only the
# newest token into the state it reads and writes the next state; a group's
# first token, a zero-filled state, or a state the caller did not keep make
# it re-fold the whole group.  The staging row must match the oracle's entry,
# the page bytes must be kv_quantize_page's on the same staging rows, and a
# repeated call must change nothing.
@pytest.mark.parametrize("m,dtype,d,norm", [(128, "fp8", 512, True), (128, "fp8", 512, False), (32, "bf16", 136, True),
                                            (64, "fp4", 128, False), (256, "fp8", 256, True)])
def test_compress_insert_fold_state(m, dtype, d, norm):
    H.flush(f"compress_insert fold state m={m} {dtype} d={d} norm={norm}")
    rng = np.random.default_rng(81 + m)
    epp = 256 // m
    B, steps, theta = 3, 12, 1e6
    # seq 0 crosses a group start at its 6th step; seq 1 starts empty; seq 2 mid-group
    L = np.array([m * 40 - 5, 0, m * 7 + 3], np.int64)
    nb = int(L.max() + steps) // 256 + 2
    P = B * nb + 2
    table = rng.permutation(P)[: B * nb].reshape(B, nb).astype(np.int32)
    beta = (rng.standard_normal(m) * 0.1).astype(np.float32)
    gam = rng.uniform(0.5, 1.5, d).astype(np.float32) if norm else None
    gam_d = H.to_dev(gam) if norm else None
    stage = torch.zeros((B, epp, d), dtype=torch.float32, device="cuda")
    pool = hca.PagedCache.empty(P, epp, d, dtype)
    pool.codes.fill_(0)
    if pool.scales is not None:
        pool.scales.fill_(0)
    state = torch.zeros((B, 4 + 2 * (4 + d)), dtype=torch.float32, device="cuda")  # page header, two fold states
    # the open groups' tokens so far (their earlier tokens drawn for the starting state)
    grp_x = [list(rng.standard_normal((int(L[b]) % m, d)).astype(np.float32)) for b in range(B)]
    grp_z = [list(rng.standard_normal(int(L[b]) % m).astype(np.float32)) for b in range(B)]
    # earlier rows of each open page: drawn, in staging and quantized into the page
    ref_rows = np.zeros((B, epp, d))
    for b in range(B):
        row = (int(L[b]) // m) % epp
        if row > 0:
            h = rng.standard_normal((row, d)).astype(np.float32)
            ref_rows[b, :row] = h
            stage[b, :row] = H.to_dev(h)
            hca.kv_quantize_page(stage[b:b + 1], H.to_dev(np.array([int(L[b]) // m - row], np.int32)),
                                 H.to_dev(np.array([row], np.int32)), epp, H.to_dev(table[b:b + 1]), pool)
    check = hca.PagedCache.empty(P, epp, d, dtype)
    for step in range(steps):
        L += 1
        pos0 = (m * ((L - 1) // m)).astype(np.int32)
        ntok = (L - pos0).astype(np.int32)
        for b in range(B):
            if ntok[b] == 1:
                grp_x[b], grp_z[b] = [], []
            grp_x[b].append(rng.standard_normal(d).astype(np.float32) * (30.0 if step == 4 else 1.0))
            grp_z[b].append(np.float32(rng.standard_normal() + (4.0 if step == 9 else 0.0)))  # a new running max
        ring = np.zeros((B, m, d), np.float32)
        ring_z = np.zeros((B, m), np.float32)
        for b in range(B):
            ring[b, : ntok[b]] = np.stack(grp_x[b])
            ring_z[b, : ntok[b]] = np.array(grp_z[b])
        xb = gen.to_bf16_bits(ring)
        j = pos0 // m
        e0 = (epp * (j // epp)).astype(np.int32)
        row = j - e0
        args = (H.to_dev(xb.view(np.int16)), H.to_dev(ring_z), H.to_dev(beta), H.to_dev(pos0), H.to_dev(ntok), m, theta,
                stage, H.to_dev(e0), H.to_dev(table), pool)
        hca.kv_compress_insert(*args, append=True, norm_gamma=gam_d, fold_state=state)
        torch.cuda.synchronize()
        if step == 7:  # the same call again: nothing changes
            snap = (stage.clone(), pool.codes.clone(), None if pool.scales is None else pool.scales.clone(),
                    state.clone())
            hca.kv_compress_insert(*args, append=True, norm_gamma=gam_d, fold_state=state)
            torch.cuda.synchronize()
            assert torch.equal(stage, snap[0]) and torch.equal(pool.codes, snap[1]) and torch.equal(state, snap[3])
            if pool.scales is not None:
                assert torch.equal(pool.scales, snap[2])
        # kv_quantize_page on the same staging rows gives the same page bytes
        hca.kv_quantize_page(stage, H.to_dev(e0), H.to_dev((row + 1).astype(np.int32)), epp, H.to_dev(table), check)
        torch.cuda.synchronize()
        sf = stage.cpu().numpy()
        ref_pool = paging.Pool(dtype, P, epp, d)
        got = H.download_pool(pool, ref_pool)
        want = H.download_pool(check, ref_pool)
        for b in range(B):
            r = int(row[b])
            ent = compressor.compress(codecs.bf16_decode(xb[b, : ntok[b]]), ring_z[b, : ntok[b]], beta, m, theta,
                                      pos0=int(pos0[b]), gamma=gam, eps=1e-6)
            assert H.rel_err_rows(sf[b, r: r + 1], ent[-1:]) <= H.ENTRY_TOL, (step, b)
            if r == 0:
                ref_rows[b] = 0.0
            ref_rows[b, r] = ent[-1]
            phys = int(table[b, e0[b] // epp])
            assert np.array_equal(got.codes[phys, : r + 1], want.codes[phys, : r + 1]), (step, b)
            sc = None
            if dtype == "fp8":
                assert got.scales[phys] == want.scales[phys], (step, b)
                sc = got.scales[phys]
            elif dtype == "fp4":
                assert np.array_equal(got.scales[phys, : r + 1], want.scales[phys, : r + 1]), (step, b)
                sc = got.scales[phys, : r + 1]
            assert H.quantized_rows_close(dtype, got.codes[phys, : r + 1], sc, ref_rows[b, : r + 1]), (step, b)
        # the state holds the open groups' token counts
        st = state.cpu().numpy()
        for b in range(B):
            assert st[b, 4 + (int(ntok[b]) % 2) * (4 + d)] == ntok[b], (step, b)


def test_compress_insert_jobs_one_launch():
    # a layer's decode update as one launch: window insert (m = 1, fp8), the
    # open c4a entry (m = 4, fp8) and its open fp4 indexer page (no fold: the
    # row is in staging); the same as the three single calls
    H.flush("compress_insert_jobs")
    rng = np.random.default_rng(71)
    B, d, di, theta = 3, 512, 128, 1e6
    L = np.array([1000, 4097, 300], np.int64)
    nb = int(L.max()) // 256 + 2
    table = rng.permutation(B * nb).reshape(B, nb).astype(np.int32)
    wtable = rng.permutation(B * nb).reshape(B, nb).astype(np.int32)
    pos_w = (L - 1).astype(np.int32)
    e0_w = (256 * ((L - 1) // 256)).astype(np.int32)
    pos_c = (4 * ((L - 1) // 4)).astype(np.int32)
    ntok_c = (L - pos_c).astype(np.int32)
    e0_c = (64 * ((pos_c // 4) // 64)).astype(np.int32)
    xw = gen.to_bf16_bits(rng.standard_normal((B, 1, d)).astype(np.float32))
    zw = rng.standard_normal((B, 1)).astype(np.float32)
    xc = gen.to_bf16_bits(rng.standard_normal((B, 8, d)).astype(np.float32))  # the 8-token window's ring
    zc = rng.standard_normal((B, 8)).astype(np.float32)
    beta = (rng.standard_normal(8) * 0.1).astype(np.float32)
    gam = H.to_dev(rng.uniform(0.5, 1.5, d).astype(np.float32))  # the entries are RMS-normalised
    stages = (rng.standard_normal((B, 256, d)).astype(np.float32), rng.standard_normal((B, 64, d)).astype(np.float32),
              rng.standard_normal((B, 64, di)).astype(np.float32))
    outs = []
    for fused in (True, False):
        wst, cst, ist = (H.to_dev(a) for a in stages)
        win = hca.PagedCache.empty(B * nb, 256, d, "fp8")
        kv = hca.PagedCache.empty(B * nb, 64, d, "fp8")
        idx = hca.PagedCache.empty(B * nb, 64, di, "fp4")
        xwd, zwd, xcd, zcd = H.to_dev(xw.view(np.int16)), H.to_dev(zw), H.to_dev(xc.view(np.int16))[:, 4:], \
            H.to_dev(zc)[:, 4:]
        args = dict(pos_w=H.to_dev(pos_w), e0_w=H.to_dev(e0_w), pos_c=H.to_dev(pos_c), ntok_c=H.to_dev(ntok_c),
                    e0_c=H.to_dev(e0_c), one=H.to_dev(np.ones(B, np.int32)), zero1=H.to_dev(np.zeros(1, np.float32)),
                    beta=H.to_dev(beta), tab=H.to_dev(table), wtab=H.to_dev(wtable))
        if fused:
            jobs = [hca.insert_job(wst, args["pos_w"], args["e0_w"], args["wtab"], win, 1, x=xwd, gate_logit=zwd,
                                   pos_bias=args["zero1"], ntok=args["one"], rope_theta=theta),
                    hca.insert_job(cst, args["pos_c"], args["e0_c"], args["tab"], kv, 4, x=xcd, gate_logit=zcd,
                                   pos_bias=args["beta"], ntok=args["ntok_c"], rope_theta=theta, norm_gamma=gam,
                                   overlap=4),
                    hca.insert_job(ist, args["pos_c"], args["e0_c"], args["tab"], idx, 4)]
            hca.kv_compress_insert_jobs(jobs, B)
        else:
            hca.kv_compress_insert(xwd, zwd, args["zero1"], args["pos_w"], args["one"], 1, theta, wst, args["e0_w"],
                                   args["wtab"], win)
            hca.kv_compress_insert(xcd, zcd, args["beta"], args["pos_c"], args["ntok_c"], 4, theta, cst, args["e0_c"],
                                   args["tab"], kv, norm_gamma=gam, overlap=4)
            rows = H.to_dev(((pos_c // 4) - e0_c + 1).astype(np.int32))
            hca.kv_quantize_page(ist, args["e0_c"], rows, 64, args["tab"], idx)
        torch.cuda.synchronize()
        outs.append((wst, cst, ist, win, kv, idx))
    (wf, cf, if_, winf, kvf, idxf), (wu, cu, iu, winu, kvu, idxu) = outs
    assert torch.equal(wf, wu) and torch.equal(cf, cu) and torch.equal(if_, iu)
    for b in range(B):
        pw, pc = int(wtable[b, e0_w[b] // 256]), int(table[b, e0_c[b] // 64])
        nw, nc = int(pos_w[b] - e0_w[b] + 1), int(pos_c[b] // 4 - e0_c[b] + 1)
        assert torch.equal(winf.codes[pw, :nw], winu.codes[pw, :nw]) and torch.equal(winf.scales[pw], winu.scales[pw])
        assert torch.equal(kvf.codes[pc, :nc], kvu.codes[pc, :nc]) and torch.equal(kvf.scales[pc], kvu.scales[pc])
        assert torch.equal(idxf.codes[pc, :nc], idxu.codes[pc, :nc])
        assert torch.equal(idxf.scales[pc, :nc], idxu.scales[pc, :nc])


# ----------------------------------------------------------------- indexer_topk


def _idx_workload(dtype, d_idx, k, B=3):
    kind = synth.LayerKind("c4a", 4, k, dtype, d_idx, 16)
    return synth.Workload(100, f"idx-{dtype}", B, None, 128, 8, 128, "fp8", [kind])


@pytest.mark.parametrize("dtype,d_idx,k,lens", [
    ("fp8", 128, 256, [40000, 4097, 1025]),
    ("fp4", 128, 2048, [70001, 8193, 9000]),
    ("bf16", 64, 256, [4096, 1023, 2000]),
    ("fp8", 64, 300, [1200, 1201, 1199]),  # N = 300 ~ k: k-1, k, k+1 entries
    ("fp4", 32, 17, [100000, 640, 65]),
    ("fp4", 64, 500, [30000, 257, 64]),     # two scale blocks per key
    ("fp4", 256, 1000, [20000, 4096, 100]),  # eight scale blocks per key
    ("fp8", 32, 300, [2200000, 3000]),      # 550,000 entries: past the LDS bitmap, separate compaction
    ("fp4", 128, 64, [(i * 1499) % 5000 + 1 for i in range(70)]),  # 70 sequences, some with N < k
])
def test_indexer_topk_sets(dtype, d_idx, k, lens):
    H.flush(f"indexer {dtype} dI={d_idx} k={k} lens={lens}")
    w = _idx_workload(dtype, d_idx, k, len(lens))
    sd = H.SeqData(w, 0, lens, build_pools=False)
    sd.idx = paging.Pool(dtype, sd.num_pages, 64, d_idx)
    for b in range(sd.B):
        paging.write_run(sd.idx, sd.table[b], 0, sd.keys[b])
    margins = sd.enforce_margin()
    assert min(margins) >= H.MARGIN
    Lmax = H.max_len(lens)
    ws = hca.workspace(hca.indexer_topk_workspace(sd.B, Lmax, 4, k))
    out_idx = torch.full((sd.B, k), -7, dtype=torch.int32, device="cuda")
    out_n = torch.zeros(sd.B, dtype=torch.int32, device="cuda")
    keys = H.upload_pool(sd.idx)
    for rep in range(2):  # the second call needs the counters and histogram the first left zeroed
        hca.indexer_topk(H.to_dev(sd.qi.view(np.int16)), H.to_dev(sd.wi), keys, H.to_dev(sd.table), H.to_dev(sd.lens),
                         Lmax, 4, k, out_idx, out_n, ws)
        torch.cuda.synchronize()
        got, n = out_idx.cpu().numpy(), out_n.cpu().numpy()
        for b in range(sd.B):
            want = sd.oracle_select(b)
            assert n[b] == len(want), (rep, b)
            assert np.array_equal(got[b, : n[b]], want), (rep, b)
            assert (got[b, n[b]:] == -1).all()


# Every score of the scoring pass against the oracle's, element by element.
# The GPU forms q_h . k_j with bf16 MFMA over exactly decoded keys (products
# exact in fp32, sums rounded in fp32, the fp4 block scale or fp8 page scale
# applied in fp32), then sum_h w_h max(0, .) in fp32: a forward error of at
# most about (d_I + H_I + 2) u times the absolute score
# A_j = sum_h |w_h| sum_i |q_hi k_ji| (u = 2^-24, ReLU is 1-Lipschitz).  The
# test allows 4 (d_I + H_I) u A_j: a scale error, a dropped block scale, a
# wrong head weight or a transposed key fails it.
@pytest.mark.parametrize("dtype,d_idx,lens", [
    ("fp4", 128, [70001, 8193, 257]),   # the V4 layers' indexer: pages of 64 entries
    ("fp8", 128, [40000, 4097, 1025]),
    ("fp4", 64, [30000, 257, 64]),      # two scale blocks per key
    ("fp4", 256, [20000, 4096, 100]),   # eight scale blocks per key
    ("bf16", 64, [4096, 1023, 2000]),
])
def test_indexer_scores_elementwise(dtype, d_idx, lens):
    H.flush(f"indexer scores {dtype} dI={d_idx} lens={lens}")
    k = 256
    w = _idx_workload(dtype, d_idx, k, len(lens))
    sd = H.SeqData(w, 0, lens, build_pools=False)
    sd.idx = paging.Pool(dtype, sd.num_pages, 64, d_idx)
    for b in range(sd.B):
        paging.write_run(sd.idx, sd.table[b], 0, sd.keys[b])
    Lmax = H.max_len(lens)
    ws = hca.workspace(hca.indexer_topk_workspace(sd.B, Lmax, 4, k))
    hca.indexer_score(H.to_dev(sd.qi.view(np.int16)), H.to_dev(sd.wi), H.upload_pool(sd.idx), H.to_dev(sd.table),
                      H.to_dev(sd.lens), Lmax, 4, k, ws)
    torch.cuda.synchronize()
    # the scores lie at the workspace's start: a row of 2048 * ceil(n_max / 2048) per sequence
    n_max = -(-Lmax // 4)
    n_pad = -(-n_max // 2048) * 2048
    got = ws[: sd.B * n_pad * 4].view(torch.float32).reshape(sd.B, n_pad).cpu().numpy()
    u = 2.0 ** -24
    for b in range(sd.B):
        N = int(compressor.n_entries(int(sd.lens[b]), 4))
        keys = paging.decode_rows(sd.idx, sd.table[b], np.arange(N))
        q = codecs.bf16_decode(sd.qi[b]).astype(np.float64)
        wgt = sd.wi[b].astype(np.float64)
        want = indexer.scores(q, wgt, keys)
        absolute = np.abs(keys) @ np.abs(q).T @ np.abs(wgt)
        tol = 4 * (d_idx + len(wgt)) * u * absolute
        err = np.abs(got[b, :N].astype(np.float64) - want)
        assert (err <= tol).all(), (b, int(np.argmax(err - tol)), float(err.max()))
        assert np.isfinite(want).all() and (np.abs(want) > 0).mean() > 0.5  # ReLU keeps a score for most entries


@pytest.mark.parametrize("dtype,d_idx,k,lens,back", [
    ("fp4", 128, 2048, [70001, 8193, 9000], 0),
    ("fp4", 128, 2048, [70001, 8193, 9000], 1),  # the staged row is not its page's last valid row
    ("fp8", 32, 300, [1200, 1201, 1199], 0),  # N = 300 ~ k
])
def test_indexer_topk_with_updates_matches_two_calls(dtype, d_idx, k, lens, back):
    # a c4a layer's window insert, open-entry update and the re-encoding of one
    # indexer row (entry N-1-back) with the indexer.  The row's staged key is a
    # fresh draw, and the uploaded pool holds zeros in its place, so the update
    # must write it and the score pass must score the new bytes: the selection
    # is the oracle's over the new keys, the indexer pool equals the oracle's,
    # and every staging row and page the jobs write has the same bytes as the
    # update call followed by the indexer
    H.flush(f"indexer with updates {dtype} dI={d_idx} k={k} lens={lens} back={back}")
    w = _idx_workload(dtype, d_idx, k, len(lens))
    sd = H.SeqData(w, 0, lens, build_pools=False)
    L = np.array(lens, np.int64)
    N = -(-L // 4)
    e_open = N - 1 - back
    fresh = np.random.default_rng(91).standard_normal((sd.B, d_idx)).astype(np.float32)
    for b in range(sd.B):
        sd.keys[b][e_open[b]] = fresh[b]
    sd.idx = paging.Pool(dtype, sd.num_pages, 64, d_idx)
    for b in range(sd.B):
        paging.write_run(sd.idx, sd.table[b], 0, sd.keys[b])
    assert min(sd.enforce_margin()) >= H.MARGIN
    stale = paging.Pool(dtype, sd.num_pages, 64, d_idx)
    stale.codes, stale.scales = sd.idx.codes.copy(), sd.idx.scales.copy()
    for b in range(sd.B):
        ph, sl = int(sd.table[b][e_open[b] // 64]), int(e_open[b] % 64)
        stale.codes[ph, sl] = 0
        if dtype == "fp4":  # per-row block scales (fp8: one scale per page, left as it is)
            stale.scales[ph, sl] = 0
        assert not np.array_equal(stale.codes[ph], sd.idx.codes[ph])
    Lmax = H.max_len(lens)
    B, d, theta = sd.B, 512, 1e6
    rng = np.random.default_rng(73)
    nb = int(L.max()) // 256 + 2
    table = rng.permutation(B * nb).reshape(B, nb).astype(np.int32)
    wtable = rng.permutation(B * nb).reshape(B, nb).astype(np.int32)
    pos_w = (L - 1).astype(np.int32)
    e0_w = (256 * ((L - 1) // 256)).astype(np.int32)
    pos_c = (4 * ((L - 1) // 4)).astype(np.int32)
    ntok_c = (L - pos_c).astype(np.int32)
    e0_c = (64 * ((pos_c // 4) // 64)).astype(np.int32)
    xw = gen.to_bf16_bits(rng.standard_normal((B, 1, d)).astype(np.float32))
    zw = rng.standard_normal((B, 1)).astype(np.float32)
    xc = gen.to_bf16_bits(rng.standard_normal((B, 8, d)).astype(np.float32))
    zc = rng.standard_normal((B, 8)).astype(np.float32)
    beta = (rng.standard_normal(8) * 0.1).astype(np.float32)
    gam = H.to_dev(rng.uniform(0.5, 1.5, d).astype(np.float32))
    stages = (rng.standard_normal((B, 256, d)).astype(np.float32), rng.standard_normal((B, 64, d)).astype(np.float32))
    dev = {n: H.to_dev(v) for n, v in dict(pos_w=pos_w, e0_w=e0_w, pos_c=pos_c, ntok_c=ntok_c, e0_c=e0_c,
                                            one=np.ones(B, np.int32), zero1=np.zeros(1, np.float32), beta=beta,
                                            tab=table, wtab=wtable).items()}
    qi, wi = H.to_dev(sd.qi.view(np.int16)), H.to_dev(sd.wi)
    ws = hca.workspace(hca.indexer_topk_workspace(B, Lmax, 4, k))
    # the re-encoded indexer row: entry e_open of each sequence, staged in f32
    # as the oracle's (new) key, with the rest of its page staged too
    pos_i, e0_i = (4 * e_open).astype(np.int32), (64 * (e_open // 64)).astype(np.int32)
    istage = np.zeros((B, 64, d_idx), np.float32)
    for bb in range(B):
        e1 = min(N[bb], e0_i[bb] + 64)  # the page's valid rows
        istage[bb, : e1 - e0_i[bb]] = sd.keys[bb][e0_i[bb]: e1]
    outs = []
    for fused in (True, False):
        keys = H.upload_pool(stale)
        ist = H.to_dev(istage)
        wst, cst = (H.to_dev(a) for a in stages)
        win = hca.PagedCache.empty(B * nb, 256, d, "fp8")
        kv = hca.PagedCache.empty(B * nb, 64, d, "fp8")
        xwd, zwd = H.to_dev(xw.view(np.int16)), H.to_dev(zw)
        xcd, zcd = H.to_dev(xc.view(np.int16))[:, 4:], H.to_dev(zc)[:, 4:]
        jobs = [hca.insert_job(wst, dev["pos_w"], dev["e0_w"], dev["wtab"], win, 1, x=xwd, gate_logit=zwd,
                               pos_bias=dev["zero1"], ntok=dev["one"], rope_theta=theta),
                hca.insert_job(cst, dev["pos_c"], dev["e0_c"], dev["tab"], kv, 4, x=xcd, gate_logit=zcd,
                               pos_bias=dev["beta"], ntok=dev["ntok_c"], rope_theta=theta, norm_gamma=gam,
                               overlap=4),
                hca.insert_job(ist, H.to_dev(pos_i), H.to_dev(e0_i), H.to_dev(sd.table), keys, 4, append=True)]
        out_idx = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
        out_n = torch.zeros(B, dtype=torch.int32, device="cuda")
        if fused:
            hca.indexer_topk_with_updates(qi, wi, keys, H.to_dev(sd.table), H.to_dev(sd.lens), Lmax, 4, k, out_idx,
                                          out_n, ws, jobs)
        else:
            hca.kv_compress_insert_jobs(jobs, B)
            hca.indexer_topk(qi, wi, keys, H.to_dev(sd.table), H.to_dev(sd.lens), Lmax, 4, k, out_idx, out_n, ws)
        torch.cuda.synchronize()
        outs.append((out_idx, out_n, wst, cst, win, kv, keys))
    (of, nf, wf, cf, winf, kvf, kf), (ou, nu, wu, cu, winu, kvu, ku) = outs
    assert torch.equal(of, ou) and torch.equal(nf, nu)
    assert torch.equal(kf.codes, ku.codes) and torch.equal(kf.scales, ku.scales)  # the whole indexer pool
    if dtype == "fp4":  # one row re-encoded: the pool is the oracle's, byte for byte
        assert np.array_equal(kf.codes.cpu().numpy(), sd.idx.codes)
        assert np.array_equal(kf.scales.cpu().numpy(), sd.idx.scales)
    else:  # the open page is re-quantized whole (one scale per page): compare its valid rows
        for b in range(B):
            ph = int(sd.table[b][e_open[b] // 64])
            nv = int(min(64, N[b] - 64 * (e_open[b] // 64)))
            assert np.array_equal(kf.codes[ph, :nv].cpu().numpy(), sd.idx.codes[ph, :nv])
            assert kf.scales[ph].item() == sd.idx.scales[ph]
    got, n = of.cpu().numpy(), nf.cpu().numpy()
    for b in range(B):
        want = sd.oracle_select(b)
        assert n[b] == len(want) and np.array_equal(got[b, : n[b]], want), b
    assert torch.equal(wf, wu) and torch.equal(cf, cu)
    for b in range(B):
        pw, pc = int(wtable[b, e0_w[b] // 256]), int(table[b, e0_c[b] // 64])
        nw, nc = int(pos_w[b] - e0_w[b] + 1), int(pos_c[b] // 4 - e0_c[b] + 1)
        assert torch.equal(winf.codes[pw, :nw], winu.codes[pw, :nw]) and torch.equal(winf.scales[pw], winu.scales[pw])
        assert torch.equal(kvf.codes[pc, :nc], kvu.codes[pc, :nc]) and torch.equal(kvf.scales[pc], kvu.scales[pc])


# ----------------------------------------------------------------- paged_hybrid_decode


def _attn_workload(kv_dtype, d, Hh, window, kind, B=3):
    return synth.Workload(101, "attn", B, None, d, Hh, window, kv_dtype, [kind])


def _run_attn(sd, sel_list, window, ws=None, table=None, wtable=None, kv=None, win=None, fp8=None):
    """fp8: None (fp32 output only), "both" (fp32 and fp8 outputs) or "only"
    (fp8 output alone); with fp8 the fp8 codes and scales are returned too."""
    B, d, Hh = sd.B, sd.w.d, sd.w.H
    Lmax = H.max_len(sd.lens)
    m = sd.kind.m
    if sel_list is not None:
        k = max(1, max(len(s) for s in sel_list))
        sel = np.full((B, k), -1, np.int32)
        for b, s in enumerate(sel_list):
            sel[b, : len(s)] = s
        sel_n = np.array([len(s) for s in sel_list], np.int32)
        sel_d, seln_d = H.to_dev(sel), H.to_dev(sel_n)
    else:
        k, sel_d, seln_d = 0, None, None
    if ws is None:
        ws = hca.workspace(hca.paged_hybrid_decode_workspace(B, Hh, d, Lmax, m, window, k))
    out = torch.zeros((B, Hh, d), dtype=torch.float32, device="cuda") if fp8 != "only" else None
    lse = torch.zeros((B, Hh), dtype=torch.float32, device="cuda")
    o8 = torch.full((B, Hh, d), 0x55, dtype=torch.uint8, device="cuda") if fp8 else None
    o8s = torch.full((B, Hh), -1.0, dtype=torch.float32, device="cuda") if fp8 else None
    hca.paged_hybrid_decode(H.to_dev(sd.q.view(np.int16)), kv or H.upload_pool(sd.kv),
                            H.to_dev(sd.table if table is None else table), win or H.upload_pool(sd.win),
                            H.to_dev(sd.wtable if wtable is None else wtable), H.to_dev(sd.lens), Lmax, m, window,
                            sel_d, seln_d, H.scale_for(d), sd.w.theta, out, lse, ws, out_fp8=o8, out_scale=o8s)
    torch.cuda.synchronize()
    res = (None if out is None else out.cpu().numpy(), lse.cpu().numpy())
    return res + ((o8.cpu().numpy(), o8s.cpu().numpy()) if fp8 else ())


@pytest.mark.parametrize("case", [
    dict(kv="fp8", d=512, H=64, W=128, m=4, topk=256, lens=[9000, 300, 2500]),
    dict(kv="fp8", d=512, H=64, W=128, m=128, topk=None, lens=[65536, 1000, 20000]),
    dict(kv="bf16", d=128, H=8, W=128, m=4, topk=256, lens=[4096, 129, 1000]),
    dict(kv="fp8", d=256, H=96, W=0, m=4, topk=64, lens=[3000, 50, 700]),
    dict(kv="fp8", d=64, H=20, W=256, m=128, topk=None, lens=[700, 1, 257]),
    dict(kv="fp8", d=512, H=128, W=128, m=1, topk=None, lens=[100, 33, 1]),
    # the paired 512-dim kernel with a partial head group (40 = 2 x 16 + 8),
    # a sequence shorter than the window and top-k above its entry count
    dict(kv="fp8", d=512, H=40, W=128, m=4, topk=300, lens=[5000, 64, 3333]),
    # and without a window: every row a compressed entry, one partial tile
    dict(kv="fp8", d=512, H=16, W=0, m=128, topk=None, lens=[129, 4229]),
    # more than 64 sequences: the work list spans two 64-lane chunks of lengths
    dict(kv="fp8", d=512, H=16, W=128, m=128, topk=None, lens=[(i * 997) % 3000 + 1 for i in range(70)]),
    dict(kv="fp8", d=512, H=16, W=128, m=4, topk=64, lens=[(i * 1499) % 2500 + 1 for i in range(70)]),
])
def test_paged_hybrid_decode(case):
    H.flush(f"attention {case}")
    kind = synth.LayerKind("c4a" if case["topk"] else "c128a", case["m"], case["topk"], "fp8" if case["topk"] else None,
                           128 if case["topk"] else 0)
    w = _attn_workload(case["kv"], case["d"], case["H"], case["W"], kind, len(case["lens"]))
    sd = H.SeqData(w, 0, case["lens"])
    if case["topk"]:
        # a valid selection per sequence: the oracle's own top-k
        sel = [sd.oracle_select(b) for b in range(sd.B)]
    else:
        sel = None
    out, lse, o8, o8s = _run_attn(sd, sel, case["W"], fp8="both")
    for b in range(sd.B):
        s = sel[b] if sel is not None else np.arange(int(compressor.n_entries(int(sd.lens[b]), case["m"])))
        ref_out, ref_lse, p = sd.oracle_attend(b, s)
        assert np.allclose(p.sum(axis=1), 1.0)
        err = H.rel_err_rows(out[b], ref_out)
        assert err <= H.ATTN_TOL, (b, err)
        assert np.allclose(lse[b], ref_lse, rtol=0, atol=2e-3), b
        # the fused fp8 form of the output (inverse RoPE, then per-row E4M3)
        for h in range(case["H"]):
            assert H.quantized_rows_close("fp8", o8[b, h], o8s[b, h], ref_out[h], tol=H.ATTN_TOL), (b, h)
        _check_fp8_rows_of(out[b], o8[b], o8s[b])
    # the fp8 output alone: the same bytes
    _, lse2, o8b, o8sb = _run_attn(sd, sel, case["W"], fp8="only")
    assert np.array_equal(o8b, o8) and np.array_equal(o8sb.view(np.uint32), o8s.view(np.uint32))
    assert np.array_equal(lse2.view(np.uint32), lse.view(np.uint32))


def _check_fp8_rows_of(out32, codes, scales):
    """The fp8 rows against the same call's fp32 rows: scale = fl32(amax/448)
    (1 for a zero row), the largest element at code 0x7E, every element within
    half an E4M3 step (decoded by torch's float8_e4m3fn cast)."""
    amax = np.abs(out32).max(axis=-1).astype(np.float32)
    want = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    assert np.array_equal(scales.view(np.uint32), want.view(np.uint32))
    dec = H.decode_page_rows("fp8", codes, 1.0)
    y = np.abs(out32.astype(np.float64)) / scales[:, None]
    e = np.maximum(np.floor(np.log2(np.maximum(y, 2.0 ** -12))), -6)
    assert (np.abs(dec - out32 / scales[:, None]) <= 0.5 * 2.0 ** (e - 3) * (1 + 1e-6)).all()
    for h in range(out32.shape[0]):
        if amax[h] > 0:
            assert ((codes[h][np.abs(out32[h]) == amax[h]] & 0x7F) == 0x7E).all()
        else:
            assert (codes[h] == 0).all()


def test_attention_layout_invariance_bitwise():
    # the same logical content through relocated pages, and through a table whose
    # shared-prefix blocks alias one set of pages: outputs must be bit-identical
    H.flush("attention layout invariance")
    kind = synth.LayerKind("c4a", 4, 512, "fp8", 128)
    w = synth.Workload(102, "alias", 2, None, 512, 64, 128, "fp8", [kind], shared_prefix_seqs=2,
                       shared_prefix_blocks=8)
    sd = H.SeqData(w, 0, [6000, 4100])
    assert len(sd.members) == 2 and (sd.table[0, :8] == sd.table[1, :8]).all()
    sel = [sd.oracle_select(b) for b in range(sd.B)]
    base_out, base_lse = _run_attn(sd, sel, 128)
    for b in range(sd.B):
        ref_out, _, _ = sd.oracle_attend(b, sel[b])
        assert H.rel_err_rows(base_out[b], ref_out) <= H.ATTN_TOL
    rng = np.random.default_rng(61)
    for trial in range(3):
        # relocate every page of both pools (trial 2 also un-aliases: sequence 1 gets its own copies)
        extra = 8 if trial == 2 else 0
        P = sd.num_pages + 5 + extra
        perm = rng.permutation(P)
        kv2 = paging.Pool("fp8", P, sd.kv.epp, sd.kv.d)
        kv2.codes[perm[: sd.num_pages]] = sd.kv.codes
        kv2.scales[perm[: sd.num_pages]] = sd.kv.scales
        t2 = np.where(sd.table >= 0, perm[np.maximum(sd.table, 0)], -1).astype(np.int32)
        if trial == 2:
            for i in range(8):
                fresh = perm[sd.num_pages + 5 + i]
                kv2.codes[fresh] = kv2.codes[t2[1, i]]
                kv2.scales[fresh] = kv2.scales[t2[1, i]]
                t2[1, i] = fresh
        wperm = rng.permutation(sd.num_wpages + 2)
        win2 = paging.Pool("fp8", sd.num_wpages + 2, 256, sd.win.d)
        win2.codes[wperm[: sd.num_wpages]] = sd.win.codes[: sd.num_wpages]
        win2.scales[wperm[: sd.num_wpages]] = sd.win.scales[: sd.num_wpages]
        wt2 = np.where(sd.wtable >= 0, wperm[np.maximum(sd.wtable, 0)], -1).astype(np.int32)
        out, lse = _run_attn(sd, sel, 128, table=t2, wtable=wt2, kv=H.upload_pool(kv2), win=H.upload_pool(win2))
        assert np.array_equal(out, base_out) and np.array_equal(lse, base_lse), trial


@pytest.mark.parametrize("d", [128, 512])
def test_attention_skips_invalid_indices_and_empty_sequences(d):
    H.flush(f"attention invalid / empty d={d}")
    kind = synth.LayerKind("c4a", 4, 64, "fp8", 128)
    w = _attn_workload("fp8", d, 16, 0, kind, 2)
    sd = H.SeqData(w, 0, [1000, 1])
    good = np.arange(0, 250, 5)
    sel = [np.concatenate([good, [-3, 250, 10 ** 6]]), np.zeros(0, np.int64)]
    out, lse, o8, o8s = _run_attn(sd, sel, 0, fp8="both")
    ref_out, ref_lse, _ = sd.oracle_attend(0, good)
    assert H.rel_err_rows(out[0], ref_out) <= H.ATTN_TOL
    assert not out[1].any() and np.all(np.isneginf(lse[1]))
    # a sequence with no rows: zero codes and scale 1 in the fp8 output
    assert not o8[1].any() and (o8s[1] == 1.0).all()


# ----------------------------------------------------------------- kv_gather


@pytest.mark.parametrize("dtype,epp,dim", [("fp8", 64, 512), ("fp4", 64, 128), ("bf16", 2, 128)])
def test_gather_bit_exact(dtype, epp, dim):
    H.flush(f"gather {dtype}")
    rng = np.random.default_rng(71)
    B, n = 3, epp * 4 + 3
    nb = -(-n // epp)
    table = rng.permutation(B * nb).reshape(B, nb).astype(np.int32)
    pool = paging.Pool(dtype, B * nb, epp, dim)
    rows = rng.standard_normal((B, n, dim)).astype(np.float32)
    for b in range(B):
        paging.write_run(pool, table[b], 0, rows[b])
    pc = H.upload_pool(pool)
    nrows = np.array([n, n - 5, 1], np.int32)
    rb = {"fp8": dim, "fp4": dim // 2, "bf16": 2 * dim}[dtype]
    codes = torch.zeros((B, n, rb), dtype=torch.uint8, device="cuda")
    scales = {"fp8": torch.zeros((B, n), dtype=torch.float32, device="cuda"),
              "fp4": torch.zeros((B, n, dim // 32), dtype=torch.uint8, device="cuda"), "bf16": None}[dtype]
    hca.kv_gather(pc, H.to_dev(table), H.to_dev(nrows), n, codes, scales)
    torch.cuda.synchronize()
    gc = codes.cpu().numpy()
    for b in range(B):
        rc, rs = paging.gather_bytes(pool, table[b], int(nrows[b]))
        assert np.array_equal(gc[b, : nrows[b]], rc.view(np.uint8).reshape(nrows[b], rb))
        if dtype != "bf16":
            assert np.array_equal(scales.cpu().numpy()[b, : nrows[b]], rs)


# ----------------------------------------------------------------- page-pool packing


def test_indexer_and_attention_over_pool_pages():
    # the pools of one c4a layer (entries, window, indexer keys) live in one
    # device arena cut by PagePool into size buckets; the block tables are the
    # allocator's pages, two sequences naming the same prefix pages (found by
    # key), and the top-k sets and attention equal the oracle's and are
    # bit-identical to the same contents in plain per-kind pools
    H.flush("indexer + attention over pool pages")
    kind = synth.LayerKind("c4a", 4, 512, "fp8", 128)
    w = synth.Workload(103, "pool", 3, None, 512, 64, 128, "fp8", [kind], shared_prefix_seqs=2,
                       shared_prefix_blocks=8)
    sd = H.SeqData(w, 0, [6000, 4100, 2500])
    assert len(sd.members) == 2
    sd.idx = paging.Pool("fp8", sd.num_pages, 64, 128)
    for b in range(sd.B):
        paging.write_run(sd.idx, sd.table[b], 0, sd.keys[b])
    sd.enforce_margin()
    kinds = [(4, 512, "fp8"), (1, 512, "fp8"), (4, 128, "fp8")]
    nblk = [-(-int(L) // 256) for L in sd.lens]
    pool = hca.PagePool(kinds, [sum(nblk) + 3, 2 * sd.B + 3, sum(nblk) + 3])
    arena = torch.zeros(pool.arena_bytes, dtype=torch.uint8, device="cuda")
    kv, win, idx = (pool.view(i, arena) for i in range(3))
    bkv, bwin, bidx = (pool.bucket_of(i) for i in range(3))
    T = np.full(sd.table.shape, -1, np.int32)
    TI = np.full(sd.table.shape, -1, np.int32)
    TW = np.full(sd.wtable.shape, -1, np.int32)
    first = int(sd.members[0])
    for b in range(sd.B):
        lb0 = 0
        if b in sd.members.tolist() and b != first:  # the prefix pages come from the first member, by key
            for lb in range(8):
                T[b, lb] = pool.lookup(bkv, 1000 + lb)
                TI[b, lb] = pool.lookup(bidx, 1000 + lb)
            assert (T[b, :8] == T[first, :8]).all() and (TI[b, :8] == TI[first, :8]).all()
            lb0 = 8
        T[b, lb0: nblk[b]] = pool.alloc(bkv, nblk[b] - lb0)
        TI[b, lb0: nblk[b]] = pool.alloc(bidx, nblk[b] - lb0)
        if b == first:
            for lb in range(8):
                pool.publish(bkv, int(T[b, lb]), 1000 + lb)
                pool.publish(bidx, int(TI[b, lb]), 1000 + lb)
        wl = np.nonzero(sd.wtable[b] >= 0)[0]
        TW[b, wl] = pool.alloc(bwin, len(wl))
    assert pool.stats(bkv)[2] == sum(nblk) - 8  # the prefix pages are held once, by two sequences
    # the oracle's page contents, placed where the allocator put them
    for b in range(sd.B):
        for lb in range(nblk[b]):
            for src, dst, tt in ((sd.kv, kv, T), (sd.idx, idx, TI)):
                dst.codes[int(tt[b, lb])] = H.to_dev(src.codes[int(sd.table[b, lb])])
                dst.scales[int(tt[b, lb])] = float(src.scales[int(sd.table[b, lb])])
        for lb in np.nonzero(sd.wtable[b] >= 0)[0]:
            win.codes[int(TW[b, lb])] = H.to_dev(sd.win.codes[int(sd.wtable[b, lb])])
            win.scales[int(TW[b, lb])] = float(sd.win.scales[int(sd.wtable[b, lb])])
    torch.cuda.synchronize()
    Lmax, k = H.max_len(sd.lens), kind.topk
    res = []
    for (kvp, winp, idxp, t, ti, tw) in ((kv, win, idx, T, TI, TW),
                                         (H.upload_pool(sd.kv), H.upload_pool(sd.win), H.upload_pool(sd.idx),
                                          sd.table, sd.table, sd.wtable)):
        ws = hca.workspace(hca.indexer_topk_workspace(sd.B, Lmax, 4, k))
        sel = torch.full((sd.B, k), -7, dtype=torch.int32, device="cuda")
        sel_n = torch.zeros(sd.B, dtype=torch.int32, device="cuda")
        hca.indexer_topk(H.to_dev(sd.qi.view(np.int16)), H.to_dev(sd.wi), idxp, H.to_dev(ti), H.to_dev(sd.lens), Lmax, 4,
                         k, sel, sel_n, ws)
        wsa = hca.workspace(hca.paged_hybrid_decode_workspace(sd.B, w.H, w.d, Lmax, 4, 128, k))
        out = torch.zeros((sd.B, w.H, w.d), dtype=torch.float32, device="cuda")
        lse = torch.zeros((sd.B, w.H), dtype=torch.float32, device="cuda")
        hca.paged_hybrid_decode(H.to_dev(sd.q.view(np.int16)), kvp, H.to_dev(t), winp, H.to_dev(tw), H.to_dev(sd.lens),
                                Lmax, 4, 128, sel, sel_n, H.scale_for(w.d), w.theta, out, lse, wsa)
        torch.cuda.synchronize()
        res.append((sel.cpu().numpy(), sel_n.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()))
    (sel_p, n_p, out_p, lse_p), (sel_u, n_u, out_u, lse_u) = res
    assert np.array_equal(sel_p, sel_u) and np.array_equal(n_p, n_u)
    assert np.array_equal(out_p.view(np.uint32), out_u.view(np.uint32))
    assert np.array_equal(lse_p.view(np.uint32), lse_u.view(np.uint32))
    for b in range(sd.B):
        want = sd.oracle_select(b)
        assert n_p[b] == len(want) and np.array_equal(sel_p[b, : n_p[b]], want), b
        ref_out, ref_lse, _ = sd.oracle_attend(b, want)
        assert H.rel_err_rows(out_p[b], ref_out) <= H.ATTN_TOL, b
    # the second member lets go: its prefix pages stay held by the first
    second = int(sd.members[1])
    pool.release(bkv, [int(p) for p in T[second, : nblk[second]]])
    assert pool.stats(bkv)[2] == sum(nblk) - 8 - (nblk[second] - 8)
