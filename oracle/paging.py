"""Paged storage of compressed entries and window tokens (quantize + block-table reads).

[V4-vLLM] 3.1.1: every layer uses one logical block of 256 raw tokens, so a c4a
block holds 256/4 = 64 entries, a c128a block 256/128 = 2 entries and a window
block 256 tokens.  [V4-vLLM] 3.1.3: page size = block size x compress ratio x
bytes per entry element, with fp8 at 1 byte and fp4 at half a byte.
[vLLM-0.7.2] 2.1: a per-sequence table maps logical blocks to physical pages,
and pages may be shared between sequences.  [V4-vLLM] 2.1/2.2: main KV in fp8,
indexer keys in fp8 or fp4.

Readings adopted:
* epp (entries per page) = 256/m; entry e of a sequence lives in physical page
  table[e // epp], slot e % epp; the window pool uses m = 1 (256 tokens a page);
* fp8 pages carry one fp32 scale per physical page, s = fl32(amax/448) over the
  page's valid elements (s = 1 when amax = 0); codes are E4M3(fl32(x/s));
* fp4 keys carry one E4M3 scale per 32 consecutive elements of a key,
  sc = E4M3(fl32(amax32/6)); codes are E2M1(fl32(x/sc)), all zero when sc
  decodes to 0; element 2c sits in the low nibble of byte c;
* bf16 pages hold RNE-rounded values and no scale;
* slots past the valid count of a page are unspecified (written as zero here).
"""

import numpy as np

from . import codecs

BLOCK_TOKENS = 256


def entries_per_page(m: int) -> int:
    assert BLOCK_TOKENS % m == 0
    return BLOCK_TOKENS // m


def page_bytes(m: int, d: int, bytes_per_elem: float) -> float:
    """[V4-vLLM] 3.1.3 page size: block size x compress ratio x bytes per entry."""
    return BLOCK_TOKENS * (1.0 / m) * d * bytes_per_elem


class Pool:
    """A pool of physical pages for one KV kind of one layer."""

    def __init__(self, dtype: str, num_pages: int, epp: int, d: int):
        assert dtype in ("bf16", "fp8", "fp4")
        self.dtype, self.num_pages, self.epp, self.d = dtype, num_pages, epp, d
        if dtype == "fp8":
            self.codes = np.zeros((num_pages, epp, d), np.uint8)
            self.scales = np.ones((num_pages,), np.float32)
        elif dtype == "fp4":
            assert d % 32 == 0
            self.codes = np.zeros((num_pages, epp, d // 2), np.uint8)
            self.scales = np.zeros((num_pages, epp, d // 32), np.uint8)
        else:
            self.codes = np.zeros((num_pages, epp, d), np.uint16)
            self.scales = None


def quantize_page(rows32, dtype: str, epp: int):
    """One page from its valid rows (fp32, [n <= epp, d]).  Returns (codes, scales)
    in the pool's per-page layout."""
    rows32 = np.asarray(rows32, dtype=np.float32)
    n, d = rows32.shape
    assert n <= epp
    if dtype == "fp8":
        codes = np.zeros((epp, d), np.uint8)
        amax = np.float32(np.abs(rows32).max()) if n else np.float32(0)
        s = np.float32(amax) / np.float32(codecs.E4M3_MAX) if amax > 0 else np.float32(1)
        y = (rows32 / np.float32(s)).astype(np.float32)
        codes[:n] = codecs.e4m3_encode(y)
        return codes, np.float32(s)
    if dtype == "fp4":
        codes = np.zeros((epp, d // 2), np.uint8)
        scales = np.zeros((epp, d // 32), np.uint8)
        blocks = rows32.reshape(n, d // 32, 32)
        amax = np.abs(blocks).max(axis=2).astype(np.float32)
        sc = codecs.e4m3_encode((amax / np.float32(codecs.E2M1_MAX)).astype(np.float32))
        sdec = codecs.e4m3_decode(sc).astype(np.float32)  # exact in fp32
        safe = np.where(sdec > 0, sdec, np.float32(1)).astype(np.float32)
        y = (blocks / safe[:, :, None]).astype(np.float32)
        nib = codecs.e2m1_encode(y).astype(np.uint8)
        nib = np.where(sdec[:, :, None] > 0, nib, 0).reshape(n, d)
        codes[:n] = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        scales[:n] = sc
        return codes, scales
    codes = np.zeros((epp, d), np.uint16)
    codes[:n] = codecs.bf16_encode(rows32)
    return codes, None


def write_run(pool: Pool, table_row, e0: int, rows32):
    """Quantize entries e0 .. e0+len(rows)-1 of one sequence (e0 a multiple of
    epp) into the physical pages its block-table row names."""
    epp = pool.epp
    assert e0 % epp == 0
    rows32 = np.asarray(rows32, dtype=np.float32)
    n = rows32.shape[0]
    for p0 in range(0, n, epp):
        lb = (e0 + p0) // epp
        phys = int(table_row[lb])
        assert phys >= 0, "writing through an unmapped block"
        codes, scales = quantize_page(rows32[p0 : p0 + epp], pool.dtype, epp)
        pool.codes[phys] = codes
        if pool.dtype == "fp8":
            pool.scales[phys] = scales
        elif pool.dtype == "fp4":
            pool.scales[phys] = scales


def decode_rows(pool: Pool, table_row, idx) -> np.ndarray:
    """Decoded fp64 rows for entry indices ``idx`` of one sequence, read through
    its block-table row."""
    idx = np.asarray(idx, dtype=np.int64)
    phys = np.asarray(table_row, dtype=np.int64)[idx // pool.epp]
    assert (phys >= 0).all(), "reading through an unmapped block"
    slot = idx % pool.epp
    c = pool.codes[phys, slot]
    if pool.dtype == "fp8":
        return codecs.e4m3_decode(c) * pool.scales[phys].astype(np.float64)[:, None]
    if pool.dtype == "fp4":
        lo = c & 0xF
        hi = c >> 4
        nib = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), np.uint8)
        nib[..., 0::2], nib[..., 1::2] = lo, hi
        vals = codecs.e2m1_decode(nib)
        sc = codecs.e4m3_decode(pool.scales[phys, slot])  # [n, d/32]
        return vals * np.repeat(sc, 32, axis=-1)
    return codecs.bf16_decode(c)


def gather_bytes(pool: Pool, table_row, n_rows: int):
    """Raw bytes of rows 0..n_rows-1 of one sequence in contiguous order (codes,
    and per-row scale material), read through the block table: the paged ->
    contiguous gather whose result must be bit-identical on every layout."""
    idx = np.arange(n_rows)
    phys = np.asarray(table_row, dtype=np.int64)[idx // pool.epp]
    slot = idx % pool.epp
    codes = pool.codes[phys, slot]
    if pool.dtype == "fp8":
        return codes, pool.scales[phys]
    if pool.dtype == "fp4":
        return codes, pool.scales[phys, slot]
    return codes, None
