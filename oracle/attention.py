"""Hybrid decode attention over the selected compressed entries plus the raw
window (fp64).

[V4-vLLM] 2.1: keys and values are one shared, RoPE-rotated vector; the
attention output is rotated back by inverse RoPE so only relative position
remains.  c128a layers attend to all of their entries; c4a layers to the
entries the indexer selects ([V4-vLLM] 2.2).  [V4-vLLM] 2.3: every layer also
attends to an uncompressed sliding window of the most recent tokens (usually
128).

Readings adopted: the decode query is the last token of the context, at
position L-1 (the current token is already in the cache); selected entries and
window tokens enter one softmax, with no de-duplication of tokens that are seen
both raw and compressed; the logit scale is passed in (1/sqrt(d) in the
workloads); window = 0 means no window rows.
"""

import numpy as np

from . import codecs
from .rope import rope


def attend(q, rows, L: int, scale: float, theta):
    """q: [H, d] unrotated queries; rows: [R, d] decoded, already-rotated shared
    K=V rows.  Returns (out [H, d], lse [H], p [H, R]) where
    out_h = RoPE^-1(sum_r p_hr rows_r, L-1), p_h = softmax(scale * RoPE(q_h, L-1) . rows)."""
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    H, d = q.shape
    if rows.shape[0] == 0:
        return np.zeros((H, d)), np.full((H,), -np.inf), np.zeros((H, 0))
    qt = rope(q, L - 1, theta)
    logits = scale * (qt @ rows.T)  # [H, R]
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    tot = e.sum(axis=1, keepdims=True)
    p = e / tot
    o = p @ rows
    out = rope(o, L - 1, theta, inverse=True)
    lse = mx[:, 0] + np.log(tot[:, 0])
    return out, lse, p


def window_positions(L: int, window: int) -> np.ndarray:
    """Token positions of the raw window: [max(0, L-W), L)."""
    return np.arange(max(0, L - window), L, dtype=np.int64)


def quantize_out_fp8(out):
    """The attention output's fp8 form for the next projection ([V4-vLLM]
    3.2.1: inverse RoPE and fp8 quantisation of the attention output are one
    fused step ahead of the fp8 o_lora GEMM).

    Reading adopted (the pages give no granularity): one scale per output row,
    i.e. per (token, head) vector of d values, with the same rule as the fp8
    pages: s = fl32(amax/448) (1 when the row is all zero), codes
    E4M3(fl32(x/s)).  The row is taken in fp32, the precision the attention
    output is delivered in.  out: [..., d].  Returns (codes uint8 [..., d],
    scales float32 [...])."""
    o32 = np.asarray(out, dtype=np.float64).astype(np.float32)
    amax = np.abs(o32).max(axis=-1)
    s = np.where(amax > 0, (amax / np.float32(codecs.E4M3_MAX)).astype(np.float32), np.float32(1))
    s = s.astype(np.float32)
    y = (o32 / s[..., None]).astype(np.float32)
    return codecs.e4m3_encode(y), s
