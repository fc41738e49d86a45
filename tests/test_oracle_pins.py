"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what it pins: closed forms, brute force written a different
way, library routines, invariants the pages state, and the pages' worked
numbers (tests/golden).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, codecs, compressor, indexer, norm, paging, pipeline
from oracle.rope import rope

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- codecs


def test_e4m3_table_anchor_values():
    # field definition: bias 7, 3 mantissa bits, S.1111.111 = NaN
    t = codecs.E4M3_TABLE
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x38] == 1.0  # exponent field 7, mantissa 0
    assert t[0x08] == 2.0 ** -6  # smallest normal
    assert t[0x01] == 2.0 ** -9  # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9  # largest subnormal
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t).sum() == 254
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)  # monotone in the code


def test_e2m1_table():
    assert list(codecs.E2M1_TABLE[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(codecs.E2M1_TABLE[8:]) == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_codec_round_trip_every_code(fmt):
    enc = codecs.e4m3_encode if fmt == "e4m3" else codecs.e2m1_encode
    tab = codecs.E4M3_TABLE if fmt == "e4m3" else codecs.E2M1_TABLE
    codes = [c for c in range(len(tab)) if np.isfinite(tab[c])]
    back = enc(tab[codes].astype(np.float32))
    assert list(back) == codes


def _brute_nearest_even(values, a, max_value):
    # nearest finite non-negative value by exhaustive search; ties -> even code
    a = min(abs(a), max_value)
    best = None
    for code, v in enumerate(values):
        dist = abs(v - a)
        if best is None or dist < best[0] or (dist == best[0] and code % 2 == 0):
            best = (dist, code)
    return best[1]


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_codec_matches_brute_force_on_midpoints_and_edges(fmt):
    if fmt == "e4m3":
        enc, pos, mx, sb = codecs.e4m3_encode, list(codecs.E4M3_TABLE[:0x7F]), 448.0, 7
    else:
        enc, pos, mx, sb = codecs.e2m1_encode, list(codecs.E2M1_TABLE[:8]), 6.0, 3
    probes = []
    for lo, hi in zip(pos[:-1], pos[1:]):
        mid = (lo + hi) / 2
        probes += [lo, mid, np.nextafter(np.float32(mid), np.float32(0)), np.nextafter(np.float32(mid), np.float32(1e9)), hi]
    probes += [mx * 1.01, mx * 100, 1e30, 0.0]
    for a in probes:
        a32 = np.float32(a)
        want = _brute_nearest_even(pos, float(a32), mx)
        assert enc(a32) == want, (fmt, a)
        assert enc(-a32) == want | (1 << sb), (fmt, -a)


def test_e4m3_matches_torch_in_range():
    g = np.random.default_rng(1)
    x = np.concatenate([
        g.uniform(-448, 448, 200000), g.normal(0, 1, 200000), g.normal(0, 1e-2, 100000),
        np.ldexp(g.uniform(-1, 1, 50000), -8),
    ]).astype(np.float32)
    ours = codecs.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_bf16_matches_torch():
    g = np.random.default_rng(2)
    x = g.normal(0, 10, 500000).astype(np.float32)
    # exact halfway cases in both tie directions
    n = 20000
    u = ((g.integers(0, 2, n) << 31) | (g.integers(100, 150, n) << 23) | (g.integers(0, 128, n) << 16) | 0x8000).astype(np.uint32)
    x = np.concatenate([x, u.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(codecs.bf16_encode(x), ref)
    assert np.array_equal(codecs.bf16_decode(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().double().numpy())


# ----------------------------------------------------------------- paging


def test_fp8_page_quantization_error_bound_and_scale():
    g = np.random.default_rng(3)
    rows = g.normal(0, 0.5, (37, 64)).astype(np.float32)
    codes, s = paging.quantize_page(rows, "fp8", 64)
    amax = np.abs(rows).max()
    assert s == np.float32(amax) / np.float32(448)
    dec = codecs.e4m3_decode(codes[:37]) * np.float64(s)
    # E4M3 keeps 3 mantissa bits: relative error <= 2^-4 above the smallest normal,
    # absolute error <= half the subnormal spacing below it
    err = np.abs(dec - rows)
    bound = np.maximum(np.abs(rows) * 2.0 ** -4, 0.5 * 2.0 ** -9 * s) * (1 + 1e-6)
    assert np.all(err <= bound)
    assert np.abs(dec).max() == pytest.approx(amax, rel=1e-6)  # the page max maps to 448
    z, sz = paging.quantize_page(np.zeros((3, 64), np.float32), "fp8", 64)
    assert sz == 1.0 and not z.any()


def test_fp4_key_quantization_block_scales():
    g = np.random.default_rng(4)
    rows = g.normal(0, 1, (5, 128)).astype(np.float32)
    rows[2, 32:64] = 0.0  # an all-zero block: scale code 0, codes 0
    pool = paging.Pool("fp4", 1, 64, 128)
    paging.write_run(pool, [0], 0, rows)
    dec = paging.decode_rows(pool, [0], np.arange(5))
    blocks = rows.reshape(5, 4, 32)
    sc = codecs.e4m3_decode(pool.scales[0, :5])
    for r in range(5):
        for b in range(4):
            amax = np.abs(blocks[r, b]).max()
            if amax == 0:
                assert sc[r, b] == 0 and not dec[r, 32 * b: 32 * b + 32].any()
                continue
            # scale is the E4M3 rounding of amax/6
            assert sc[r, b] == codecs.E4M3_TABLE[codecs.e4m3_encode(np.float32(amax) / np.float32(6))]
            # every decoded value is a multiple of the block scale by an E2M1 magnitude
            ratio = dec[r, 32 * b: 32 * b + 32] / sc[r, b]
            assert set(np.abs(ratio).tolist()) <= set(codecs.E2M1_TABLE[:8].tolist())
    # nibble packing: element 2c in the low nibble of byte c
    lo = pool.codes[0, 0, 0] & 0xF
    assert codecs.E2M1_TABLE[lo] * sc[0, 0] == dec[0, 0]


def _fraction(s):
    if "/" in s:
        n, d = s.split("/")
        return float(n) / float(d)
    return float(s)


def test_fp4_key_block_hand_example():
    # tests/golden: two 32-element blocks worked by hand from the bit fields
    # (scale code, the divided values, the nibbles, the packed bytes, the
    # decoded values); the second block is the first halved
    with open(os.path.join(GOLDEN, "fp4_key_block_hand_example.json")) as f:
        g = json.load(f)
    b0, b1 = g["blocks"]
    x = np.array(b0["x"], np.float32)
    row = np.concatenate([x, x * np.float32(0.5)])[None, :]
    assert np.abs(row[0, 32:]).max() == b1["amax"]
    assert np.float32(np.float32(b0["amax"]) / np.float32(6)) == np.float32(b0["amax_over_6"])
    assert np.float32(np.float32(b1["amax"]) / np.float32(6)) == np.float32(b1["amax_over_6"])
    codes, scales = paging.quantize_page(row, "fp4", 64)
    assert list(scales[0]) == [b0["scale_code"], b1["scale_code"]]
    assert codecs.E4M3_TABLE[b0["scale_code"]] == b0["scale"] and codecs.E4M3_TABLE[b1["scale_code"]] == b1["scale"]
    # the divided values as the hand computation states them
    y = x / np.float32(b0["scale"])
    assert np.allclose(y, [_fraction(s) for s in b0["y"]], rtol=0, atol=5e-5)
    assert list(codes[0, :16]) == b0["bytes"] and list(codes[0, 16:32]) == b0["bytes"]
    assert not codes[1:].any() and not scales[1:].any()  # slots past the valid rows
    nib = np.empty(64, np.int64)
    nib[0::2], nib[1::2] = codes[0] & 0xF, codes[0] >> 4
    assert list(nib[:32]) == b0["codes"]
    pool = paging.Pool("fp4", 1, 64, 64)
    pool.codes[0], pool.scales[0] = codes, scales
    dec = paging.decode_rows(pool, [0], [0])[0]
    want = np.array(b0["decoded"], np.float64)
    assert np.array_equal(dec[:32], want) and np.array_equal(dec[32:], want * 0.5)
    assert np.array_equal(np.signbit(dec[:32]), np.signbit(want))  # -0.25 rounds to a signed zero


def _e2m1_half_step(a):
    # half the E2M1 spacing around magnitude a (a <= 6): 0.25 below 2, 0.5 below 4, 1 up to 6
    return np.where(a < 2.0, 0.25, np.where(a < 4.0, 0.5, 1.0))


def test_fp4_key_quantization_half_step_bound():
    # every decoded element lies within half an E2M1 step (at the magnitude of
    # x / decoded scale) of x, times the decoded scale; the block's largest
    # element maps into [4, 6] times the scale.  Dividing by the unrounded
    # amax/6 instead of the decoded scale breaks this bound.
    g = np.random.default_rng(41)
    for spread in (1e-3, 4e-3, 1.0, 37.0):
        rows = (g.standard_normal((64, 128)) * spread).astype(np.float32)
        rows[5, :32] *= 1e-3  # one block much smaller than its neighbours
        codes, scales = paging.quantize_page(rows, "fp4", 64)
        pool = paging.Pool("fp4", 1, 64, 128)
        pool.codes[0], pool.scales[0] = codes, scales
        dec = paging.decode_rows(pool, [0], np.arange(64))
        sdec = np.repeat(codecs.e4m3_decode(scales), 32, axis=1)
        x = rows.astype(np.float64)
        zero = sdec == 0  # amax/6 below half the smallest E4M3 subnormal 2^-9: every code 0
        assert np.all(dec[zero] == 0) and np.all(np.abs(x[zero]) <= 6 * 2.0 ** -10 * (1 + 1e-6))
        s = np.where(zero, 1.0, sdec)
        a = np.abs(x) / s
        normal = ~zero & (sdec >= 2.0 ** -6)
        assert np.all(a[normal] <= 6.0 * (1 + 2.0 ** -4) * (1 + 1e-6))  # sc = amax/6 up to one E4M3 rounding
        err = np.abs(dec - x)
        inside = ~zero & (a <= 6.0)
        assert np.all(err[inside] <= (_e2m1_half_step(a) * s)[inside] * (1 + 1e-6))
        sat = ~zero & (a > 6.0)  # saturated: coded as +-6 with x's sign
        assert np.all(dec[sat] == np.sign(x[sat]) * 6.0 * sdec[sat])
        # with a normal scale the block's largest element is coded at 4 or 6 times it
        sc4 = codecs.e4m3_decode(scales)
        top = np.abs(dec.reshape(64, 4, 32)).max(axis=2) / np.where(sc4 > 0, sc4, 1.0)
        assert np.all((top >= 4.0) | (sc4 < 2.0 ** -6))
    # the plausible mistake the bound catches: codes from x / fl32(amax/6)
    x = np.array([6.5, 2.75] + [0.0] * 30, np.float32)
    sc = codecs.e4m3_decode(codecs.e4m3_encode(np.float32(6.5) / np.float32(6)))
    wrong = codecs.e2m1_decode(codecs.e2m1_encode(x / (np.float32(6.5) / np.float32(6)))) * sc
    assert abs(wrong[1] - 2.75) > _e2m1_half_step(2.75 / sc) * sc


def test_paged_equals_contiguous_under_permutation_and_aliasing():
    # the same logical rows through three different tables read back bit-identically
    g = np.random.default_rng(5)
    rows = g.normal(0, 1, (300, 32)).astype(np.float32)
    for dtype in ("fp8", "bf16", "fp4"):
        outs = []
        for trial in range(3):
            pool = paging.Pool(dtype, 10, 64, 32)
            table = g.permutation(10)[:5] if trial else np.arange(5)
            paging.write_run(pool, table, 0, rows)
            outs.append(paging.decode_rows(pool, table, np.arange(300)))
            outs.append(paging.gather_bytes(pool, table, 300)[0].astype(np.float64))
        assert np.array_equal(outs[0], outs[2]) and np.array_equal(outs[0], outs[4])
        assert np.array_equal(outs[1], outs[3]) and np.array_equal(outs[1], outs[5])
    # aliasing: two sequences whose first two blocks name the same pages
    pool = paging.Pool("fp8", 8, 64, 32)
    t0 = np.array([5, 6, 0, 1, 2])
    t1 = np.array([5, 6, 3, 4, 7])
    paging.write_run(pool, t0, 0, rows)
    paging.write_run(pool, t1, 0, np.concatenate([rows[:128], rows[128:] * 2]))
    assert np.array_equal(paging.decode_rows(pool, t0, np.arange(128)), paging.decode_rows(pool, t1, np.arange(128)))


# ----------------------------------------------------------------- worked numbers


def test_pages_worked_numbers():
    gold = json.load(open(os.path.join(GOLDEN, "pages_worked_numbers.json")))
    for e in gold["entry_counts"]:
        assert int(compressor.n_entries(e["L"], e["m"])) == e["N"], e["cite"]
    for e in gold["entries_per_block"]:
        assert paging.entries_per_page(e["m"]) == e["epp"], e["cite"]
    for e in gold["page_bytes_bf16_5120"]:
        assert paging.page_bytes(e["m"], 5120, 2) == e["bytes"], e["cite"]
    for e in gold["layer_bytes_bf16_5120"]:
        assert e["N"] * 5120 * 2 == e["bytes"], e["cite"]
    # the ceil(L/m) rule at the 2^20 contexts of the long-context workload
    assert compressor.n_entries(1 << 20, 4) == 262144 and compressor.n_entries(1 << 20, 128) == 8192


# ----------------------------------------------------------------- rope


def _rotation_matrix(d, pos, theta):
    # block-diagonal 2x2 rotations, built entry by entry
    R = np.zeros((d, d))
    for i in range(d // 2):
        ang = pos * theta ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        R[2 * i, 2 * i], R[2 * i, 2 * i + 1] = c, -s
        R[2 * i + 1, 2 * i], R[2 * i + 1, 2 * i + 1] = s, c
    return R


def test_rope_is_block_rotation_and_inverse():
    g = np.random.default_rng(6)
    v = g.normal(size=(16,))
    for pos in (0, 1, 7, 1000, 1 << 20):
        R = _rotation_matrix(16, pos, 1e6)
        assert np.allclose(rope(v, pos, 1e6), R @ v, atol=1e-12)
        assert np.allclose(rope(rope(v, pos, 1e6), pos, 1e6, inverse=True), v, atol=1e-12)
    assert np.allclose(rope(rope(v, 3, 1e4), 5, 1e4), rope(v, 8, 1e4), atol=1e-12)


# ----------------------------------------------------------------- compressor


def test_compressor_mean_pooling_and_identity():
    g = np.random.default_rng(7)
    x = g.normal(size=(37, 8))
    e = compressor.compress(x, np.zeros(37), np.zeros(4), 4, None)
    assert e.shape == (10, 8)
    for j in range(10):
        assert np.allclose(e[j], np.mean(x[4 * j: 4 * j + 4], axis=0), atol=1e-14)
    # m = 1 is the identity before rotation, and RoPE(x_t, t) with it
    assert np.allclose(compressor.compress(x, g.normal(size=37), g.normal(size=1), 1, None), x, atol=1e-15)
    assert np.allclose(compressor.compress(x, g.normal(size=37), g.normal(size=1), 1, 1e4),
                       compressor.window_rows(x, 0, 1e4), atol=1e-13)


def test_compressor_dominant_logit_and_weights_sum_to_one():
    g = np.random.default_rng(8)
    x = g.normal(size=(256, 8))
    z = g.normal(size=256)
    z[130] = 1e4  # dominates group 1 (tokens 128..255) of m = 128
    e = compressor.compress(x, z, g.normal(0, 0.1, 128), 128, None)
    assert np.allclose(e[1], x[130], atol=1e-12)
    w = compressor.group_weights(g.normal(size=203), g.normal(0, 0.1, 4), 4)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)
    assert (w[-1, 3:] == 0).all()  # partial last group: 203 = 50*4 + 3


def test_compressor_partial_group_is_the_running_residual():
    # the partial group equals a running fold over its tokens (max, sum exp, sum w*x),
    # i.e. the softmax renormalized over the available slots
    g = np.random.default_rng(9)
    x = g.normal(size=(7, 6))
    z = g.normal(size=7)
    beta = g.normal(0, 0.1, 4)
    e = compressor.compress(x, z, beta, 4, None)
    mx, se, acc = -np.inf, 0.0, np.zeros(6)
    for i in range(3):
        a = z[4 + i] + beta[i]
        nm = max(mx, a)
        se = se * math.exp(mx - nm) + math.exp(a - nm)
        acc = acc * math.exp(mx - nm) + math.exp(a - nm) * x[4 + i]
        mx = nm
    assert np.allclose(e[1], acc / se, atol=1e-14)


def test_incremental_equals_one_shot():
    # prefill L-1 tokens, then re-fold only the open group with the new token:
    # the same entries as compressing all L tokens at once
    g = np.random.default_rng(10)
    m, L, d = 4, 1031, 8
    x, z, beta = g.normal(size=(L, d)), g.normal(size=L), g.normal(0, 0.1, m)
    full = compressor.compress(x, z, beta, m, 1e6)
    pre = compressor.compress(x[: L - 1], z[: L - 1], beta, m, 1e6)
    gopen = (L - 1) // m
    upd = compressor.compress(x[gopen * m: L], z[gopen * m: L], beta, m, 1e6, pos0=gopen * m)
    inc = np.concatenate([pre[:gopen], upd], axis=0)
    assert np.array_equal(full, inc)


# ----------------------------------------------------------------- indexer


def test_indexer_scores_against_loop_and_relu_identity():
    g = np.random.default_rng(11)
    q, w, k = g.normal(size=(16, 32)), g.normal(size=16), g.normal(size=(50, 32))
    s = indexer.scores(q, w, k)
    for j in range(50):
        ref = math.fsum(w[h] * max(0.0, math.fsum(q[h, c] * k[j, c] for c in range(32))) for h in range(16))
        assert s[j] == pytest.approx(ref, abs=1e-11)
    # relu(x) - relu(-x) = x: the ReLU is present and the key sign enters linearly
    diff = indexer.scores(q, w, k) - indexer.scores(q, w, -k)
    assert np.allclose(diff, (k @ q.T) @ w, atol=1e-11)
    # basis keys pick one coordinate of every head
    s_basis = indexer.scores(q, w, np.eye(32)[:5])
    assert np.allclose(s_basis, (np.maximum(q[:, :5], 0) * w[:, None]).sum(axis=0), atol=1e-13)


def test_topk_against_stable_argsort_with_ties():
    g = np.random.default_rng(12)
    for trial in range(50):
        N = int(g.integers(1, 60))
        s = g.integers(0, 6, N).astype(np.float64)  # many ties
        k = int(g.integers(1, 70))
        got = indexer.topk(s, k)
        order = np.argsort(-s, kind="stable")  # stable: equal scores keep index order
        want = np.sort(order[: min(k, N)])
        assert np.array_equal(got, want)
    assert np.array_equal(indexer.topk(np.ones(5), 9), np.arange(5))


# ----------------------------------------------------------------- attention


def test_attention_reduces_to_sdpa_without_rope():
    # m = 1, no window, no top-k, rotation switched off: standard single-KV-head attention
    g = np.random.default_rng(13)
    H, d, L = 4, 16, 40
    x, q = g.normal(size=(L, d)), g.normal(size=(H, d))
    e = compressor.compress(x, g.normal(size=L), g.normal(size=1), 1, None)
    out, lse, p = attention.attend(q, e, L, 1 / math.sqrt(d), None)
    kv = torch.from_numpy(x)[None, None]
    qt = torch.from_numpy(q).reshape(1, H, 1, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kv.expand(1, H, L, d), kv.expand(1, H, L, d))
    assert np.allclose(out, ref[0, :, 0].numpy(), atol=1e-12)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
    logits = (q @ x.T) / math.sqrt(d)
    assert np.allclose(lse, np.log(np.exp(logits).sum(axis=1)), atol=1e-12)


def test_attention_with_rope_brute_force_rotation_matrices():
    # out_h = sum_t p_t R(t-(L-1)) x_t with logits q_h^T R(t-(L-1)) x_t
    g = np.random.default_rng(14)
    H, d, L, theta = 3, 8, 24, 100.0
    x, q = g.normal(size=(L, d)), g.normal(size=(H, d))
    rows = compressor.window_rows(x, 0, theta)
    out, _, _ = attention.attend(q, rows, L, 0.3, theta)
    for h in range(H):
        logit = np.array([q[h] @ _rotation_matrix(d, t - (L - 1), theta) @ x[t] for t in range(L)]) * 0.3
        p = np.exp(logit - logit.max())
        p /= p.sum()
        ref = sum(p[t] * (_rotation_matrix(d, t - (L - 1), theta) @ x[t]) for t in range(L))
        assert np.allclose(out[h], ref, atol=1e-12)


def test_attention_translation_invariance():
    # shifting every stored position and the query position by the same amount
    # leaves the output unchanged: only relative position survives
    g = np.random.default_rng(15)
    H, d, n = 4, 32, 50
    x, q = g.normal(size=(n, d)), g.normal(size=(H, d))
    pos = np.sort(g.choice(5000, n, replace=False))
    L = int(pos[-1]) + 1
    ref, _, _ = attention.attend(q, rope(x, pos, 1e6), L, 0.2, 1e6)
    for shift in (4, 128, 12345 * 4, (1 << 20) - L):
        got, _, _ = attention.attend(q, rope(x, pos + shift, 1e6), L + shift, 0.2, 1e6)
        assert np.allclose(got, ref, atol=1e-9)
    # without the inverse rotation on the output the result would move with the shift
    qt = rope(q, L - 1, 1e6)
    assert not np.allclose(qt, rope(q, L - 1 + 128, 1e6), atol=1e-3)


def test_attention_empty_rows():
    out, lse, _ = attention.attend(np.ones((2, 8)), np.zeros((0, 8)), 5, 1.0, 1e6)
    assert not out.any() and np.all(np.isneginf(lse))


# ----------------------------------------------------------------- pipeline


def test_window_blocks_and_pipeline_paging_invariance():
    assert pipeline.window_blocks(300, 128) == [0, 1]
    assert pipeline.window_blocks(256, 128) == [0]
    assert pipeline.window_blocks(257, 128) == [0, 1]
    assert pipeline.window_blocks(100, 0) == []
    g = np.random.default_rng(16)
    spec = pipeline.LayerSpec(m=4, d=32, H=4, window=16, topk=20, kv_dtype="fp8", idx_dtype="fp4", d_idx=32)
    L = 700
    x, z, beta = g.normal(size=(L, 32)), g.normal(size=L), g.normal(0, 0.1, 4)
    keys = g.normal(size=(175, 32)).astype(np.float32)
    q, qi, wi = g.normal(size=(4, 32)), g.normal(size=(16, 32)), g.normal(size=16)
    results = []
    for trial in range(3):
        perm = g.permutation(6) if trial else np.arange(6)
        wperm = g.permutation(3) if trial else np.arange(3)
        table, wtable = perm[:3], np.full(3, -1)
        for i, blk in enumerate(pipeline.window_blocks(L, spec.window)):
            wtable[blk] = wperm[i]
        kv, idx, win = paging.Pool("fp8", 6, 64, 32), paging.Pool("fp4", 6, 64, 32), paging.Pool("fp8", 3, 256, 32)
        pipeline.fill_entries(spec, kv, table, x, z, beta)
        pipeline.fill_window(spec, win, wtable, x, L)
        pipeline.fill_index_keys(idx, table, keys)
        sel, _ = pipeline.select(spec, L, idx, table, qi, wi)
        results.append(pipeline.attend(spec, L, q, kv, table, win, wtable, sel)[0])
    assert np.array_equal(results[0], results[1]) and np.array_equal(results[0], results[2])


def test_entry_rotated_at_first_token_position():
    # reading: entry j is rotated at position j*m
    g = np.random.default_rng(17)
    x = g.normal(size=(16, 8))
    e = compressor.compress(x, np.zeros(16), np.zeros(4), 4, 1e4)
    for j in range(4):
        assert np.allclose(e[j], _rotation_matrix(8, 4 * j, 1e4) @ np.mean(x[4 * j: 4 * j + 4], axis=0), atol=1e-13)


def test_page_and_slot_addressing():
    # entry e of a sequence lives in physical page table[e // epp], slot e % epp
    g = np.random.default_rng(18)
    rows = g.normal(size=(130, 16)).astype(np.float32)
    table = np.array([4, 1, 3])
    pool = paging.Pool("bf16", 5, 64, 16)
    paging.write_run(pool, table, 0, rows)
    for e in (0, 63, 64, 100, 129):
        assert np.array_equal(pool.codes[table[e // 64], e % 64], codecs.bf16_encode(rows[e]))
    # a run that starts at a later page (the open page of a decode update)
    pool2 = paging.Pool("fp8", 5, 2, 16)
    paging.write_run(pool2, [0, 2, 4], 2, rows[:3])
    assert np.array_equal(pool2.codes[2, :2], paging.quantize_page(rows[:2], "fp8", 2)[0])
    assert np.array_equal(pool2.codes[4, :1], paging.quantize_page(rows[2:3], "fp8", 2)[0][:1])


# ----------------------------------------------------------------- fused epilogues


def test_rms_norm_and_out_fp8_hand_examples():
    gold = json.load(open(os.path.join(GOLDEN, "fused_epilogue_hand_examples.json")))
    for e in gold["rms_norm"]:
        y = norm.rms_norm(np.array(e["c"]), np.array(e["gamma"]), e["eps"])
        assert np.allclose(y, e["y"], rtol=0, atol=1e-14), e["cite"]
    for e in gold["out_fp8"]:
        codes, s = attention.quantize_out_fp8(np.array(e["x"]))
        assert codes.tolist() == e["codes"], e["cite"]
        if "scale" in e:
            assert float(s) == e["scale"], e["cite"]


def test_compressor_norm_before_rope_closed_form():
    # one token, one pair, gains (2, 1/2), position 1 (angle 1 rad for pair 0):
    # the gains act before the rotation, so the rotated pair is R(1) (6, 2) sqrt(2)/5
    y0, y1 = 6 * math.sqrt(2) / 5, 2 * math.sqrt(2) / 5
    want = [y0 * math.cos(1.0) - y1 * math.sin(1.0), y0 * math.sin(1.0) + y1 * math.cos(1.0)]
    for fn in (lambda x: compressor.compress(x, np.zeros(1), np.zeros(1), 1, 1e6, pos0=1, gamma=[2.0, 0.5], eps=0.0),
               lambda x: compressor.window_rows(x, 1, 1e6, gamma=[2.0, 0.5], eps=0.0)):
        got = fn(np.array([[3.0, 4.0]]))
        assert np.allclose(got[0], want, rtol=0, atol=1e-14)
    # gains applied after the rotation would differ
    wrong = [2.0 * (3 * math.cos(1.0) - 4 * math.sin(1.0)), 0.5 * (3 * math.sin(1.0) + 4 * math.cos(1.0))]
    assert not np.allclose(np.array(wrong) / math.sqrt(12.5), want, atol=1e-3)


def test_compressor_norm_invariants():
    g = np.random.default_rng(31)
    T, d = 43, 16
    x, z, beta = g.normal(size=(T, d)), g.normal(size=T), g.normal(0, 0.1, 4)
    ones = np.ones(d)
    # unit gains, no eps: every entry (partial last one included) has mean square 1
    # after the rotation, which keeps pair norms
    e = compressor.compress(x, z, beta, 4, 1e4, gamma=ones, eps=0.0)
    assert np.allclose(np.mean(e * e, axis=1), 1.0, atol=1e-13)
    # no eps: invariant to a positive scale of the tokens, odd in their sign
    assert np.allclose(compressor.compress(7.5 * x, z, beta, 4, 1e4, gamma=ones, eps=0.0), e, atol=1e-13)
    assert np.allclose(compressor.compress(-x, z, beta, 4, 1e4, gamma=ones, eps=0.0), -e, atol=1e-13)
    # gains scale the unrotated entry dimension by dimension
    gam = g.uniform(0.5, 1.5, d)
    u1 = compressor.compress(x, z, beta, 4, None, gamma=ones, eps=1e-6)
    ug = compressor.compress(x, z, beta, 4, None, gamma=gam, eps=1e-6)
    assert np.allclose(ug, u1 * gam, atol=1e-13)
    # normalising never changes the direction of the unrotated entry
    raw = compressor.compress(x, z, beta, 4, None)
    cosang = np.sum(raw * u1, axis=1) / np.linalg.norm(raw, axis=1) / np.linalg.norm(u1, axis=1)
    assert np.allclose(cosang, 1.0, atol=1e-13)
    # eps: a row of mean square eps is scaled by 1/sqrt(2)
    c = np.full((1, d), 1e-3)
    assert np.allclose(norm.rms_norm(c, ones, 1e-6), c / math.sqrt(2e-6), atol=1e-14)


def test_out_fp8_bound_and_saturation():
    g = np.random.default_rng(32)
    q, rows = g.normal(size=(8, 64)), g.normal(size=(300, 64))
    out, _, _ = attention.attend(q, rows, 300, 0.125, 1e6)
    out[3] = 0.0
    codes, s = attention.quantize_out_fp8(out)
    assert codes.shape == out.shape and s.shape == (8,) and s.dtype == np.float32
    assert s[3] == 1.0 and (codes[3] == 0).all()
    dec = codecs.e4m3_decode(codes) * s[:, None].astype(np.float64)
    assert np.isfinite(dec).all()
    o32 = out.astype(np.float32).astype(np.float64)
    for h in range(8):
        if h == 3:
            continue
        amax = np.abs(o32[h]).max()
        assert s[h] == np.float32(np.float32(amax) / np.float32(448.0))
        # the largest element takes the largest finite code
        assert (codes[h][np.abs(o32[h]) == amax] & 0x7F == 0x7E).all()
        # each element within half an E4M3 step (at its binade, subnormal below 2^-6) of x
        y = np.abs(o32[h]) / s[h]
        e = np.maximum(np.floor(np.log2(np.maximum(y, 1e-30))), -6)
        assert (np.abs(dec[h] - o32[h]) <= 0.5 * 2.0 ** (e - 3) * s[h] * (1 + 1e-6) + 1e-300).all()


# ----------------------------------------------------------------- overlapping windows


def test_overlap_zero_is_the_plain_compressor():
    # two implementations of one definition: the group-at-a-time fold and the
    # entry-by-entry window fold with no overlap
    g = np.random.default_rng(41)
    for m, T in ((4, 37), (1, 9), (16, 100)):
        x, z, beta = g.normal(size=(T, 8)), g.normal(size=T), g.normal(0, 0.1, m)
        a = compressor.compress(x, z, beta, m, 1e4, gamma=np.linspace(0.5, 1.5, 8))
        b = compressor.compress_overlap(x, z, beta, m, 0, 1e4, gamma=np.linspace(0.5, 1.5, 8))
        assert np.allclose(a, b, atol=1e-13)


def test_overlap_windows_by_pooling_slot_bias_and_dominant_token():
    g = np.random.default_rng(42)
    T = 37
    x = g.normal(size=(T, 8))
    # uniform weights: entry j is the mean of positions [4j-4, 4j+4) within [0, T)
    e = compressor.compress_overlap(x, np.zeros(T), np.zeros(8), 4, 4, None)
    assert e.shape == (10, 8)
    assert np.allclose(e[0], x[0:4].mean(axis=0), atol=1e-14)
    for j in range(1, 9):
        assert np.allclose(e[j], x[4 * j - 4: 4 * j + 4].mean(axis=0), atol=1e-14)
    assert np.allclose(e[9], x[32:37].mean(axis=0), atol=1e-14)  # partial: 32..36
    # slot 0 (the oldest token of the window) dominant: entry j >= 1 is x[4j-4];
    # entry 0's slots 0..3 lie before position 0, so it falls back to its own group
    beta = np.zeros(8)
    beta[0] = 1e4
    e = compressor.compress_overlap(x, np.zeros(T), beta, 4, 4, None)
    assert np.allclose(e[0], x[0:4].mean(axis=0), atol=1e-14)
    for j in range(1, 10):
        assert np.allclose(e[j], x[4 * j - 4], atol=1e-12)
    # a dominant token at t is the whole of the two entries whose windows hold it
    z = g.normal(size=T)
    z[13] = 1e4
    e = compressor.compress_overlap(x, z, g.normal(0, 0.1, 8), 4, 4, None)
    hit = [j for j in range(10) if np.allclose(e[j], x[13], atol=1e-12)]
    assert hit == [3, 4]


def test_overlap_runs_split_anywhere_and_decode_refold():
    # a run that starts at pos0 > 0 with the o tokens before it equals the same
    # entries of one run from 0; re-folding the open group every step from the
    # last o + m tokens gives the one-shot entries (the 8-token compressor state)
    g = np.random.default_rng(43)
    T, d = 203, 16
    x, z, beta = g.normal(size=(T, d)), g.normal(size=T), g.normal(0, 0.1, 8)
    gam = g.uniform(0.5, 1.5, d)
    full = compressor.compress_overlap(x, z, beta, 4, 4, 1e6, gamma=gam)
    for p0 in (4, 64, 200):
        part = compressor.compress_overlap(x[p0:], z[p0:], beta, 4, 4, 1e6, pos0=p0, x_prev=x[p0 - 4: p0],
                                           z_prev=z[p0 - 4: p0], gamma=gam)
        assert np.allclose(part, full[p0 // 4:], atol=1e-12)
    for L in range(1, T + 1):
        j = (L - 1) // 4
        p0 = 4 * j
        open_e = compressor.compress_overlap(x[p0:L], z[p0:L], beta, 4, 4, 1e6, pos0=p0,
                                             x_prev=x[max(0, p0 - 4): p0], z_prev=z[max(0, p0 - 4): p0], gamma=gam)
        ref = compressor.compress_overlap(x[:L], z[:L], beta, 4, 4, 1e6, gamma=gam)
        assert np.allclose(open_e[0], ref[j], atol=1e-12)
    assert compressor.compress_overlap(x[:1], z[:1], beta, 4, 4, None).shape == (1, d)
