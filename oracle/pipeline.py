"""One decode step of one layer for one sequence, composed from the oracle's
stages in the order the pages give them ([V4-vLLM] 3.2.2: after the Q/K
projections, the indexer, the main-KV compression and the window insert run
independently, then attention).

The stages are the plainest composition: compress the whole context
(compressor), quantize every entry page (paging), insert the window pages,
quantize the indexer keys, score and select (indexer, c4a only), then attend
(attention).  Nothing is fused or reordered.
"""

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import attention, compressor, indexer, paging
from .paging import BLOCK_TOKENS


@dataclass
class LayerSpec:
    m: int  # compression ratio (4: c4a, 128: c128a, 1: uncompressed)
    d: int  # shared K=V dim
    H: int  # query heads
    window: int  # raw window tokens (0: none)
    topk: Optional[int]  # None: attend to every entry (c128a)
    kv_dtype: str  # "fp8" | "bf16" (main entries and window rows)
    idx_dtype: Optional[str] = None  # "fp8" | "fp4" | "bf16" for c4a indexer keys
    d_idx: int = 0
    h_idx: int = 16
    theta: float = 1.0e6
    scale: Optional[float] = None  # default 1/sqrt(d)
    gamma: Optional[np.ndarray] = None  # RMSNorm gain of the entries ([V4-vLLM] 3.2.1), None: no norm
    eps: float = 1e-6
    overlap: int = 0  # tokens of the previous group in each entry's window (4 for c4a's 8-token window)

    @property
    def epp(self):
        return paging.entries_per_page(self.m)

    @property
    def softmax_scale(self):
        return self.scale if self.scale is not None else 1.0 / np.sqrt(self.d)


def window_blocks(L: int, window: int):
    """Logical window blocks that overlap [L-W, L) ([vLLM-0.7.2] 2.3: only blocks
    inside the window are loaded)."""
    if window <= 0 or L <= 0:
        return []
    first = max(0, L - window) // BLOCK_TOKENS
    last = (L - 1) // BLOCK_TOKENS
    return list(range(first, last + 1))


def fill_entries(spec: LayerSpec, pool, table_row, x, z, beta):
    """Compress a whole context and quantize all of its entry pages.  Returns the
    fp64 entries (before quantization)."""
    if spec.overlap > 0:
        e = compressor.compress_overlap(x, z, beta, spec.m, spec.overlap, spec.theta, gamma=spec.gamma,
                                        eps=spec.eps)
    else:
        e = compressor.compress(x, z, beta, spec.m, spec.theta, gamma=spec.gamma, eps=spec.eps)
    paging.write_run(pool, table_row, 0, e.astype(np.float32))
    return e


def fill_window(spec: LayerSpec, pool, wtable_row, x, L: int):
    """Quantize the window pages: each mapped block holds every token of its
    256-token block that is < L, rotated at its own position."""
    for blk in window_blocks(L, spec.window):
        t0, t1 = blk * BLOCK_TOKENS, min(L, (blk + 1) * BLOCK_TOKENS)
        rows = compressor.window_rows(x[t0:t1], t0, spec.theta)
        paging.write_run(pool, wtable_row, t0, rows.astype(np.float32))


def fill_index_keys(pool, table_row, keys32):
    paging.write_run(pool, table_row, 0, np.asarray(keys32, np.float32))


def select(spec: LayerSpec, L: int, idx_pool, table_row, q_idx, w_idx):
    """Indices of the entries attended to: top-k by indexer score for c4a, all of
    them otherwise.  Returns (sel, scores-or-None)."""
    N = int(compressor.n_entries(L, spec.m))
    if spec.topk is None:
        return np.arange(N, dtype=np.int64), None
    keys = paging.decode_rows(idx_pool, table_row, np.arange(N))
    s = indexer.scores(q_idx, w_idx, keys)
    return indexer.topk(s, spec.topk), s


def attend(spec: LayerSpec, L: int, q, kv_pool, table_row, win_pool, wtable_row, sel):
    """Gather the decoded rows (selected entries, then window tokens) and attend."""
    rows = paging.decode_rows(kv_pool, table_row, sel)
    if spec.window > 0:
        wpos = attention.window_positions(L, spec.window)
        rows = np.concatenate([rows, paging.decode_rows(win_pool, wtable_row, wpos)], axis=0)
    return attention.attend(q, rows, L, spec.softmax_scale, spec.theta)
