"""Seeded draws for the workloads in ``configs``.

Every array comes from its own NumPy PCG64 stream keyed by
SeedSequence([seed, config, layer, stream, sequence]), so any one sequence of
any one layer can be drawn without drawing the rest.  Stream ids: 0 block
table, 1 lengths, 2 tokens, 3 logits, 4 slot bias, 5 queries, 6 indexer keys,
7 indexer queries, 8 indexer head weights, 9 indexer-key re-draws, 10 the
entries' RMSNorm gain.

Distributions: tokens, logits, queries, indexer keys and queries and head
weights ~ N(0, 1); slot biases ~ N(0, 0.1) (0.1 is the standard deviation);
RMSNorm gains ~ U(0.5, 1.5) (fp32);
bf16 tensors are fp32 draws rounded to nearest even by torch's CPU cast.

For the largest workloads the benchmark draws tensors on the GPU with torch's
seeded device generator instead (``device_normal``); those values are inputs
like any other and can be copied back to the host for checking.
"""

import numpy as np

from .configs import Workload

BLOCK = 256
S_TABLE, S_LEN, S_TOK, S_LOGIT, S_BETA, S_Q, S_IDXK, S_IDXQ, S_IDXW, S_REDRAW, S_GAIN = range(11)
SHARED = 1 << 20  # sub-key of the shared-prefix draws


def rng(seed, cid, layer, stream, sub=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cid, layer, stream, sub])))


def to_bf16_bits(a) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def lengths(w: Workload, seed=0) -> np.ndarray:
    if w.L is not None:
        return np.full((w.B,), w.L, np.int32)
    lo, hi = w.L_range
    out = np.empty((w.B,), np.int32)
    for b in range(w.B):
        g = rng(seed, w.cid, 0, S_LEN, b)
        while True:
            L = int(np.exp(g.uniform(np.log(lo), np.log(hi))))
            if L % BLOCK != 0 and lo <= L <= hi:
                break
        out[b] = L
    return out


def shared_members(w: Workload, lens, seed=0) -> np.ndarray:
    """Sequences whose first ``shared_prefix_blocks`` blocks are the same tokens and
    share physical pages (drawn among those long enough to have the whole prefix
    plus a window that does not reach into it)."""
    if w.shared_prefix_seqs == 0:
        return np.zeros((0,), np.int64)
    need = w.shared_prefix_blocks * BLOCK + BLOCK
    elig = np.nonzero(np.asarray(lens) > need)[0]
    g = rng(seed, w.cid, 0, S_TABLE, 1)
    k = min(w.shared_prefix_seqs, len(elig))
    return np.sort(g.choice(elig, size=k, replace=False))


def block_tables(w: Workload, lens, seed=0):
    """Block tables of the compressed pools (one table serves every compressed
    pool of every layer) and of the window pool.

    Returns (table [B, nb] int32, num_pages, wtable [B, nb] int32, num_wpages);
    unmapped blocks are -1.  Only window blocks that overlap [L-W, L) are mapped."""
    lens = np.asarray(lens, np.int64)
    B = len(lens)
    nb = int(-(-lens.max() // BLOCK))
    members = set(shared_members(w, lens, seed).tolist())
    nshared = w.shared_prefix_blocks if members else 0
    # logical (sequence, block) slots that need a page of their own
    slots = []
    for b in range(B):
        nblk = int(-(-lens[b] // BLOCK))
        for i in range(nblk):
            if b in members and i < nshared:
                continue
            slots.append((b, i))
    total = len(slots) + nshared
    if w.table == "identity":
        perm = np.arange(total)
    else:
        perm = rng(seed, w.cid, 0, S_TABLE, 0).permutation(total)
    table = np.full((B, nb), -1, np.int32)
    for (b, i), p in zip(slots, perm[: len(slots)]):
        table[b, i] = p
    for b in members:
        table[b, :nshared] = perm[len(slots) :]
    # window pool
    wslots = []
    for b in range(B):
        L = int(lens[b])
        if w.window > 0 and L > 0:
            for i in range(max(0, L - w.window) // BLOCK, (L - 1) // BLOCK + 1):
                wslots.append((b, i))
    wperm = np.arange(len(wslots)) if w.table == "identity" else rng(seed, w.cid, 0, S_TABLE, 2).permutation(len(wslots))
    wtable = np.full((B, nb), -1, np.int32)
    for (b, i), p in zip(wslots, wperm):
        wtable[b, i] = p
    return table, total, wtable, len(wslots)


def _normal(g, shape, std=1.0):
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _with_prefix(w, seed, layer, stream, b, members, n_total, n_prefix, shape_tail, std=1.0):
    x = _normal(rng(seed, w.cid, layer, stream, b), (n_total,) + shape_tail, std)
    if b in members and n_prefix > 0:
        x[:n_prefix] = _normal(rng(seed, w.cid, layer, stream, SHARED), (n_prefix,) + shape_tail, std)
    return x


def tokens_f32(w: Workload, layer, b, L, members=(), seed=0, t0=0, t1=None):
    """Token vectors of sequence b, positions [t0, t1) (fp32 before the bf16 cast)."""
    x = _with_prefix(w, seed, layer, S_TOK, b, set(members), L, w.shared_prefix_blocks * BLOCK, (w.d,), w.token_std)
    return x[t0:t1]


def tokens(w: Workload, layer, b, L, members=(), seed=0):
    """bf16 bit patterns [L, d] of sequence b's tokens."""
    return to_bf16_bits(tokens_f32(w, layer, b, L, members, seed))


def logits(w: Workload, layer, b, L, members=(), seed=0):
    return _with_prefix(w, seed, layer, S_LOGIT, b, set(members), L, w.shared_prefix_blocks * BLOCK, ())


def slot_bias(w: Workload, layer, m, seed=0):
    return _normal(rng(seed, w.cid, layer, S_BETA), (m,), w.beta_std)


def norm_gain(w: Workload, layer, d, seed=0):
    """fp32 [d] gain of the RMSNorm applied to a layer's compressed entries."""
    return rng(seed, w.cid, layer, S_GAIN).uniform(0.5, 1.5, d).astype(np.float32)


def queries(w: Workload, layer, seed=0):
    """bf16 bit patterns [B, H, d]."""
    return to_bf16_bits(_normal(rng(seed, w.cid, layer, S_Q), (w.B, w.H, w.d)))


def index_keys(w: Workload, layer, b, N, d_idx, m, members=(), seed=0):
    """fp32 indexer keys [N, d_idx] of sequence b (shared-prefix entries equal)."""
    npre = w.shared_prefix_blocks * BLOCK // m
    return _with_prefix(w, seed, layer, S_IDXK, b, set(members), N, npre, (d_idx,))


def index_queries(w: Workload, layer, h_idx, d_idx, seed=0):
    return to_bf16_bits(_normal(rng(seed, w.cid, layer, S_IDXQ), (w.B, h_idx, d_idx)))


def index_weights(w: Workload, layer, h_idx, seed=0):
    return _normal(rng(seed, w.cid, layer, S_IDXW), (w.B, h_idx))


def redraw_keys(w: Workload, layer, b, rows, d_idx, attempt, seed=0):
    """Fresh fp32 keys for the given rows (used to clear near-ties at the top-k cut)."""
    g = rng(seed, w.cid, layer, S_REDRAW, (b << 8) + attempt)
    return _normal(g, (len(rows), d_idx))


def device_normal(shape, std, key, device="cuda", dtype=None):
    """Seeded N(0, std^2) draw made on the GPU by torch's device generator."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence(list(key)).generate_state(1, np.uint64)[0] & ((1 << 63) - 1)))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t if dtype is None else t.to(dtype)
