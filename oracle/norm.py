"""RMS normalisation of a compressed entry (fp64).

[V4-vLLM] 3.2.1 lists, for the c4a decode path, one fused kernel made of the
compressor, an RMSNorm, RoPE and the cache insertion, in that order: the
compressed vector is normalised, then rotated, then stored.

The pages do not write RMSNorm out; the usual definition is taken: with a
learned per-dimension gain gamma and a small eps,
    y_i = gamma_i * c_i / sqrt(mean_j c_j**2 + eps),   i, j < d.
The real gamma and eps are model parameters the pages do not give; they are
inputs here (synthetic gamma in the tests, eps = 1e-6 by default).
"""

import numpy as np


def rms_norm(c, gamma, eps: float = 1e-6) -> np.ndarray:
    """Normalise the last axis of ``c`` by its root mean square and scale it by
    ``gamma`` (length d)."""
    c = np.asarray(c, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    ms = np.mean(c * c, axis=-1, keepdims=True)
    return c / np.sqrt(ms + np.float64(eps)) * gamma
