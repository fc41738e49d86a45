"""Rotary position embedding and its inverse (fp64).

[V4-vLLM] 2.1: keys and values share one vector; RoPE is applied on the key use
and, because the same rotated vector is also the value, the attention output is
rotated back by the query's position (inverse RoPE), which leaves only the
relative position in the result.  [V4-vLLM] 3.2.1 applies RoPE before cache
insertion, so stored rows are already rotated.  [vLLM-0.7.2] 4.3 gives the base
1e6.

Reading adopted: adjacent pairs (2i, 2i+1) rotate by angle p * theta**(-2i/d),
i < d/2, over all d dimensions:
    (v[2i], v[2i+1]) -> (v[2i] cos - v[2i+1] sin, v[2i] sin + v[2i+1] cos);
the inverse uses the negated angle.
"""

import numpy as np


def inv_freq(d: int, theta: float) -> np.ndarray:
    i = np.arange(d // 2, dtype=np.float64)
    return np.float64(theta) ** (-2.0 * i / d)


def rope(v, pos, theta: float, inverse: bool = False) -> np.ndarray:
    """Rotate the last axis of ``v`` (fp64, even length d) by position(s) ``pos``
    (broadcast against v's leading axes).  ``theta=None`` returns ``v``
    unchanged (used only to pin attention against a rotation-free library
    routine)."""
    v = np.asarray(v, dtype=np.float64)
    if theta is None:
        return v.copy()
    d = v.shape[-1]
    pos = np.asarray(pos, dtype=np.float64)
    phi = pos[..., None] * inv_freq(d, theta)
    if inverse:
        phi = -phi
    c, s = np.cos(phi), np.sin(phi)
    v0, v1 = v[..., 0::2], v[..., 1::2]
    out = np.empty(np.broadcast_shapes(v.shape, phi.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = v0 * c - v1 * s
    out[..., 1::2] = v0 * s + v1 * c
    return out
