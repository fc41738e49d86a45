"""The compressor: m consecutive token vectors -> one shared K=V entry (fp64).

[V4-vLLM] 2.1: c4a layers fold every few raw tokens, c128a layers every 128,
into one entry by a learned weighted sum with a positional bias (not a plain
average); a 1M-token context gives 1,000,000/128 ~= 7,813 c128a entries and
1,000,000/4 = 250,000 c4a entries.  [V4-vLLM] 3.1.2: compression is not
one-shot; the part of the context not yet folded is carried as a rolling
residual whose state is kept like sliding-window KV.  [V4-vLLM] 3.2.1: RoPE is
applied to the compressed vector before it is inserted into the cache.

Readings adopted:
* groups are the non-overlapping runs [jm, jm+m) (m = 4 for c4a, 128 for
  c128a); entry count N = ceil(L/m);
* the weights are a softmax over the group's slots of (token logit z_t +
  per-slot bias beta_i);
* a partial last group (r < m tokens) is an entry whose softmax runs over its r
  available slots; this is exactly the state a running (max, sum exp, sum w*x)
  residual holds after r tokens, and equals the full entry once r = m;
* the entry is rotated at the position of its first token, jm;
* with a gain gamma, the entry is RMS-normalised before it is rotated
  ([V4-vLLM] 3.2.1: compressor, then RMSNorm, then RoPE, then insertion); a
  partial group's entry is normalised as it stands.

Overlapping windows ([V4-vLLM] 2.1 describes c4a as folding every 8 tokens
into one entry at a ratio of 1/4; 3.1.2 gives c4a an 8-token compressor
state): with an overlap o, entry j folds the o + m tokens of positions
[jm - o, jm + m), its own group and the last o tokens of the group before; one
softmax runs over the window's slots i = 0 .. o+m-1 (slot bias beta_i, slot 0
the oldest token); slots at positions below 0 or at or past the context's end
are absent.  The entry count stays ceil(L/m) and the entry is still rotated at
jm.  c4a's window is o = m = 4.
"""

import numpy as np

from .norm import rms_norm
from .rope import rope


def n_entries(L, m):
    """N = ceil(L/m)."""
    L = np.asarray(L, dtype=np.int64)
    return -(-L // m)


def group_weights(z, beta, m):
    """Softmax weights of every group.  z: [T] logits for tokens 0..T-1 of a run
    that starts at a group boundary; returns w [N, m] with zeros in the slots
    past the end of a partial last group."""
    z = np.asarray(z, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T = z.shape[0]
    N = int(n_entries(T, m))
    a = np.full((N, m), -np.inf)
    a.reshape(-1)[:T] = z
    a = a + beta[None, :m]
    valid = np.arange(N * m).reshape(N, m) < T
    a = np.where(valid, a, -np.inf)
    amax = a.max(axis=1, keepdims=True)
    e = np.exp(a - amax)
    return e / e.sum(axis=1, keepdims=True)


def compress(x, z, beta, m, theta, pos0=0, chunk_groups=1 << 14, gamma=None, eps=1e-6):
    """Entries of a run of tokens.

    x: [T, d] token vectors of positions pos0 .. pos0+T-1 (pos0 a multiple of m),
    z: [T] logits, beta: [m] slot biases.  Returns e [ceil(T/m), d] fp64, entry j
    rotated at position pos0 + j*m.  With ``gamma`` ([d]) each entry is
    RMS-normalised (gain gamma, offset eps) before the rotation.  Processed in
    chunks of groups so that long contexts fit in memory; chunking does not
    change any value."""
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    assert pos0 % m == 0
    N = int(n_entries(T, m))
    out = np.empty((N, d), dtype=np.float64)
    for g0 in range(0, N, chunk_groups):
        g1 = min(N, g0 + chunk_groups)
        t0, t1 = g0 * m, min(T, g1 * m)
        w = group_weights(z[t0:t1], beta, m)  # [g1-g0, m]
        xs = np.zeros(((g1 - g0) * m, d))
        xs[: t1 - t0] = x[t0:t1]
        c = np.einsum("gi,gid->gd", w, xs.reshape(g1 - g0, m, d))
        if gamma is not None:
            c = rms_norm(c, gamma, eps)
        pos = pos0 + m * np.arange(g0, g1, dtype=np.float64)
        out[g0:g1] = rope(c, pos, theta)
    return out


def window_rows(x_block, first_pos, theta, gamma=None, eps=1e-6):
    """Sliding-window rows ([V4-vLLM] 2.3: raw, uncompressed recent tokens, kept in
    every layer): token t is stored as RoPE(x_t, t).  This is the compressor with
    m = 1 (one slot, weight 1), with the same optional RMS normalisation."""
    x_block = np.asarray(x_block, dtype=np.float64)
    if gamma is not None:
        x_block = rms_norm(x_block, gamma, eps)
    pos = first_pos + np.arange(x_block.shape[0], dtype=np.float64)
    return rope(x_block, pos, theta)


def compress_overlap(x, z, beta, m, o, theta, pos0=0, x_prev=None, z_prev=None, gamma=None, eps=1e-6):
    """Entries of a run of tokens with overlapping windows of o + m tokens.

    x: [T, d], z: [T] for positions pos0 .. pos0+T-1 (pos0 a multiple of m);
    x_prev: [o, d], z_prev: [o] the o tokens before pos0 (ignored, and may be
    None, where pos0 = 0: those positions do not exist); beta: [o + m].
    Entry j (j < ceil(T/m)) folds the valid slots of positions
    [pos0 + jm - o, pos0 + jm + m); returns e [ceil(T/m), d] fp64, entry j
    rotated at pos0 + jm.  Written entry by entry from the definition."""
    x = np.asarray(x, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    T, d = x.shape
    assert pos0 % m == 0 and beta.shape[0] == o + m
    if o > 0 and pos0 > 0:
        xr = np.concatenate([np.asarray(x_prev, dtype=np.float64).reshape(o, d), x])
        zr = np.concatenate([np.asarray(z_prev, dtype=np.float64).reshape(o), z])
    else:  # rows of the (absent) positions before 0 are never read
        xr = np.concatenate([np.zeros((o, d)), x])
        zr = np.concatenate([np.zeros(o), z])
    N = int(n_entries(T, m))
    out = np.empty((N, d), dtype=np.float64)
    for j in range(N):
        pos = pos0 + j * m - o + np.arange(o + m)  # the window's positions
        valid = (pos >= 0) & (pos < pos0 + T)
        rows = j * m + np.arange(o + m)  # their rows in xr / zr
        a = np.where(valid, zr[np.minimum(rows, o + T - 1)] + beta, -np.inf)
        w = np.exp(a - a.max())
        w = w / w.sum()
        c = w[valid] @ xr[rows[valid]]
        if gamma is not None:
            c = rms_norm(c, gamma, eps)
        out[j] = rope(c, pos0 + j * m, theta)
    return out
