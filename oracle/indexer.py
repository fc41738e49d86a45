"""Indexer scoring and top-k selection for c4a layers (fp64).

[V4-vLLM] 2.2: c4a layers get a separate, smaller indexer KV cache that tells a
query which compressed entries to look in, instead of a brute-force search over
the main KV; its pages are stored like the c4a main KV and quantized too.  The
pages give no scoring formula.

Readings adopted (the problem statement of this build: "16 heads x dim 128 fp8
keys, per-head ReLU-weighted score sum, top-k"):
* one indexer key k_j (dim d_I) per compressed entry j, shared by H_I query
  heads; score s_j = sum_h w_h * max(0, q_h . k_j), no extra scale, no RoPE;
* top-k keeps the k largest scores, ties broken toward the lower index, and
  returns the kept indices in ascending order; if k >= N every entry is kept.
"""

import numpy as np


def scores(q, w, keys) -> np.ndarray:
    """q: [H_I, d_I], w: [H_I], keys: [N, d_I] decoded keys; returns s [N] (fp64)."""
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    dots = keys @ q.T  # [N, H_I]
    return np.maximum(dots, 0.0) @ w


def topk(s, k: int) -> np.ndarray:
    """Indices of the k best scores (score descending, index ascending on ties),
    returned in ascending index order."""
    s = np.asarray(s, dtype=np.float64)
    N = s.shape[0]
    if k >= N:
        return np.arange(N, dtype=np.int64)
    order = np.lexsort((np.arange(N), -s))  # primary: -s, secondary: index
    return np.sort(order[:k])


def kth_margin(s, k: int) -> float:
    """Distance from the k-th best score to the nearest score on the other side of
    the cut (inf when everything is kept).  Inputs whose margin is below a
    threshold are re-drawn by the tests so that the selected set does not hinge
    on rounding."""
    s = np.asarray(s, dtype=np.float64)
    N = s.shape[0]
    if k >= N:
        return float("inf")
    srt = np.sort(s)[::-1]
    return float(srt[k - 1] - srt[k])
