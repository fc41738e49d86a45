"""Python binding of libhca: decode attention over hybrid compressed KV caches
on AMD MI355X (gfx950).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of ``libhca.so``; torch supplies device memory and streams.  The
functions carry the names of the C entry points (``include/hca.h``), take torch
tensors, and raise ``HcaError`` on a non-OK status.  Importing works without a
GPU; calling a function needs the built library and raises if it is missing.

Build the library with ``python -m decode_attention_compressed_amd.build``.
"""

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("HCA_LIB") or os.path.join(_PKG, "libhca.so")  # HCA_LIB: another build of the library

BF16, FP8_E4M3, FP4_E2M1 = 0, 1, 2
DTYPES = {"bf16": BF16, "fp8": FP8_E4M3, "fp4": FP4_E2M1}
STATUS = {0: "HCA_OK", 1: "HCA_ERR_INVALID", 2: "HCA_ERR_UNSUPPORTED", 3: "HCA_ERR_WORKSPACE", 4: "HCA_ERR_HIP"}

#: every symbol the C headers declare (include/hca.h and include/hca_testing.h)
EXPORTS = (
    "hca_status_string", "hca_version", "hca_debug_status", "kv_compress", "kv_prefill_pages", "kv_compress_insert",
    "kv_compress_insert_jobs",
    "kv_quantize_page_workspace",
    "kv_quantize_page",
    "indexer_topk_workspace",
    "indexer_topk", "indexer_topk_with_updates", "paged_hybrid_decode_workspace", "paged_hybrid_decode",
    "paged_hybrid_decode_noalloc_max_bytes", "paged_hybrid_decode_noalloc", "kv_gather",
    "hca_host_e4m3_encode", "hca_host_e2m1_encode", "hca_host_bf16_encode", "hca_probe_decode", "hca_probe_e4m3_sweep", "hca_probe_mfma",
    "hca_indexer_score", "hca_attention_split",
    "hca_page_bytes", "hca_pool_plan", "hca_pool_create", "hca_pool_destroy", "hca_pool_view", "hca_pool_bucket",
    "hca_pool_alloc", "hca_pool_share", "hca_pool_release", "hca_pool_publish", "hca_pool_lookup", "hca_pool_stats",
)


class HcaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class CPagedCache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("num_pages", ctypes.c_int32),
                ("epp", ctypes.c_int32), ("dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class CKvKind(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class CInsertJob(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("x_stride_b", ctypes.c_int64), ("gate_logit", ctypes.c_void_p),
                ("z_stride_b", ctypes.c_int64), ("pos_bias", ctypes.c_void_p), ("pos0", ctypes.c_void_p),
                ("ntok", ctypes.c_void_p), ("m", ctypes.c_int32), ("overlap", ctypes.c_int32),
                ("rope_theta", ctypes.c_float),
                ("norm_gamma", ctypes.c_void_p), ("norm_eps", ctypes.c_float), ("stage", ctypes.c_void_p), ("stage_stride_b", ctypes.c_int64), ("e0", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("bt_stride", ctypes.c_int32), ("dst", CPagedCache),
                ("append", ctypes.c_int32), ("fold_state", ctypes.c_void_p), ("fold_state_stride_b", ctypes.c_int64)]


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _F32, _SZ = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded libhca.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m decode_attention_compressed_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.hca_status_string.restype = ctypes.c_char_p
        L.hca_status_string.argtypes = [ctypes.c_int]
        L.hca_version.restype = ctypes.c_char_p
        L.hca_debug_status.argtypes = [ctypes.POINTER(ctypes.c_uint32)]
        L.kv_compress.argtypes = [_P, _I64, _P, _I64, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _F32, _P, _F32, _P,
                                  _I64, _P]
        L.kv_prefill_pages.argtypes = [_P, _I64, _P, _I64, _P, _P, _P, _I32, _I32, _I32, _I32, _F32, _P, _F32, _P,
                                       _I32, CPagedCache, _P]
        L.kv_compress_insert.argtypes = [_P, _I64, _P, _I64, _P, _P, _P, _I32, _I32, _I32, _F32, _P, _F32, _P, _I64,
                                         _P, _P, _I32, CPagedCache, _I32, _P, _I64, _P]
        L.kv_compress_insert_jobs.argtypes = [ctypes.POINTER(CInsertJob), _I32, _I32, _P]
        L.kv_quantize_page_workspace.argtypes = [_I32, _I32, CPagedCache]
        L.kv_quantize_page_workspace.restype = _SZ
        L.kv_quantize_page.argtypes = [_P, _I64, _P, _P, _I32, _I32, _P, _I32, CPagedCache, _P, _SZ, _P]
        L.indexer_topk_workspace.argtypes = [_I32, _I32, _I32, _I32]
        L.indexer_topk_workspace.restype = _SZ
        L.indexer_topk.argtypes = [_P, _P, _I32, CPagedCache, _P, _I32, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _SZ, _P]
        L.indexer_topk_with_updates.argtypes = [_P, _P, _I32, CPagedCache, _P, _I32, _P, _I32, _I32, _I32, _I32, _P, _P,
                                                _P, _SZ, ctypes.POINTER(CInsertJob), _I32, _P]
        L.paged_hybrid_decode_workspace.argtypes = [_I32, _I32, _I32, _I32, _I32, _I32, _I32]
        L.paged_hybrid_decode_workspace.restype = _SZ
        L.paged_hybrid_decode.argtypes = [_P, _I32, CPagedCache, _P, _I32, CPagedCache, _P, _I32, _P, _I32, _I32,
                                          _I32, _I32, _P, _P, _I32, _F32, _F32, _P, _P, _P, _P, _P, _SZ, _P]
        L.paged_hybrid_decode_noalloc_max_bytes.argtypes = []
        L.paged_hybrid_decode_noalloc_max_bytes.restype = _SZ
        L.paged_hybrid_decode_noalloc.argtypes = [_P, _I32, CPagedCache, _P, _I32, CPagedCache, _P, _I32, _P, _I32,
                                                  _I32, _I32, _I32, _P, _P, _I32, _F32, _F32, _P, _P, _P, _P, _P]
        L.kv_gather.argtypes = [CPagedCache, _P, _I32, _P, _I32, _I32, _P, _P, _P]
        L.hca_host_e4m3_encode.argtypes = [_P, _P, _I64]
        L.hca_host_e2m1_encode.argtypes = [_P, _P, _I64]
        L.hca_host_bf16_encode.argtypes = [_P, _P, _I64]
        L.hca_probe_decode.argtypes = [_P, _P, _I32, _I32, _P]
        L.hca_probe_e4m3_sweep.argtypes = [ctypes.c_uint32, ctypes.c_uint32, _P, _P]
        L.hca_probe_mfma.argtypes = [_P, _P, _P, _I32, _P]
        L.hca_indexer_score.argtypes = [_P, _P, _I32, CPagedCache, _P, _I32, _P, _I32, _I32, _I32, _I32, _P, _SZ, _P]
        L.hca_attention_split.argtypes = [_P, _I32, CPagedCache, _P, _I32, CPagedCache, _P, _I32, _P, _I32, _I32, _I32,
                                          _I32, _P, _P, _I32, _F32, _F32, _P, _SZ, _P]
        L.hca_page_bytes.argtypes = [CKvKind, _P, _P]
        L.hca_pool_plan.argtypes = [_P, _I32, _P, _P]
        L.hca_pool_create.argtypes = [_P, _I32, _P, _P, _P]
        L.hca_pool_destroy.argtypes = [_P]
        L.hca_pool_destroy.restype = None
        L.hca_pool_view.argtypes = [_P, _I32, _P, ctypes.POINTER(CPagedCache)]
        L.hca_pool_bucket.argtypes = [_P, _I32]
        L.hca_pool_alloc.argtypes = [_P, _I32, _I32, _P]
        L.hca_pool_share.argtypes = [_P, _I32, _P, _I32]
        L.hca_pool_release.argtypes = [_P, _I32, _P, _I32]
        L.hca_pool_publish.argtypes = [_P, _I32, _I32, ctypes.c_uint64]
        L.hca_pool_lookup.argtypes = [_P, _I32, ctypes.c_uint64, _P]
        L.hca_pool_stats.argtypes = [_P, _I32, _P, _P, _P, _P, _P]
        for name in EXPORTS:
            if name not in ("hca_status_string", "hca_version", "indexer_topk_workspace",
                            "paged_hybrid_decode_workspace", "kv_quantize_page_workspace", "hca_pool_destroy",
                            "paged_hybrid_decode_noalloc_max_bytes"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != 0:
        raise HcaError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


@dataclass
class PagedCache:
    """One pool of physical pages (a torch tensor of codes, and scales)."""

    codes: torch.Tensor
    scales: Optional[torch.Tensor]
    epp: int
    dim: int
    dtype: str

    @property
    def num_pages(self) -> int:
        return self.codes.shape[0]

    @staticmethod
    def empty(num_pages: int, epp: int, dim: int, dtype: str, device="cuda") -> "PagedCache":
        if dtype == "fp8":
            codes = torch.zeros((num_pages, epp, dim), dtype=torch.uint8, device=device)
            scales = torch.ones((num_pages,), dtype=torch.float32, device=device)
        elif dtype == "fp4":
            codes = torch.zeros((num_pages, epp, dim // 2), dtype=torch.uint8, device=device)
            scales = torch.zeros((num_pages, epp, dim // 32), dtype=torch.uint8, device=device)
        else:
            codes = torch.zeros((num_pages, epp, dim), dtype=torch.int16, device=device)
            scales = None
        return PagedCache(codes, scales, epp, dim, dtype)

    def c(self) -> CPagedCache:
        return CPagedCache(self.codes.data_ptr(), 0 if self.scales is None else self.scales.data_ptr(),
                           self.num_pages, self.epp, self.dim, DTYPES[self.dtype])


def _null_cache() -> CPagedCache:
    return CPagedCache(0, 0, 0, 0, 0, 0)


def version() -> str:
    return lib().hca_version().decode()


def debug_status():
    """The debug build's index checks (hca_debug_status): waits for the device and returns (status, bits), where
    bits has 1 for a page id outside its pool, 2 for a block-table slot past the table, 4 for a selected entry
    outside its sequence and 8 for a row outside its page; the release build returns (HCA_ERR_UNSUPPORTED, 0)."""
    bits = ctypes.c_uint32(0)
    st = lib().hca_debug_status(ctypes.byref(bits))
    return int(st), int(bits.value)


def kv_compress(x, gate_logit, pos_bias, pos0, ntok, m: int, rope_theta: float, out, max_ntok: int, stream=None,
                norm_gamma=None, norm_eps: float = 1e-6, overlap: int = 0):
    """x: bf16 [B, T, d] (or int16 bit patterns); gate_logit f32 [B, T]; pos_bias f32 [m + overlap];
    pos0, ntok int32 [B]; out f32 [B, ceil(T/m), d]; norm_gamma f32 [d] or None.  With an
    overlap, x and gate_logit are views whose rows -overlap .. -1 hold the tokens before pos0."""
    B, T, d = x.shape
    _check(lib().kv_compress(_ptr(x), x.stride(0), _ptr(gate_logit), gate_logit.stride(0), _ptr(pos_bias),
                             _ptr(pos0), _ptr(ntok), B, max_ntok, d, m, overlap, rope_theta, _ptr(norm_gamma),
                             norm_eps, _ptr(out), out.stride(0), _stream(stream)), "kv_compress")


def kv_prefill_pages(x, gate_logit, pos_bias, pos0, ntok, m: int, rope_theta: float, max_ntok: int, block_table,
                     dst: "PagedCache", stream=None, norm_gamma=None, norm_eps: float = 1e-6, overlap: int = 0):
    """The fused prefill of one pool: kv_compress + kv_quantize_page in one launch, no fp32 entries.
    x: bf16 [B, T, d] (or int16 bit patterns); gate_logit f32 [B, T]; pos0 (multiples of 256), ntok int32 [B];
    block_table int32 [B, nb]; with an overlap, rows -overlap .. -1 of x and gate_logit hold the tokens before pos0."""
    B = x.shape[0]
    _check(lib().kv_prefill_pages(_ptr(x), x.stride(0), _ptr(gate_logit), gate_logit.stride(0), _ptr(pos_bias),
                                  _ptr(pos0), _ptr(ntok), B, max_ntok, m, overlap, rope_theta, _ptr(norm_gamma),
                                  norm_eps, _ptr(block_table), block_table.stride(0), dst.c(), _stream(stream)),
           "kv_prefill_pages")


def kv_compress_insert(x, gate_logit, pos_bias, pos0, ntok, m: int, rope_theta: float, stage, e0, block_table,
                       dst: PagedCache, append: bool = False, stream=None, norm_gamma=None, norm_eps: float = 1e-6,
                       overlap: int = 0, fold_state=None):
    """Decode-step update of one pool in one launch: x bf16 [B, m, d] (the open
    group's tokens); gate_logit f32 [B, m]; pos_bias f32 [m]; pos0, ntok, e0
    int32 [B]; stage f32 [B, epp, d] (the open page's staging); block_table
    int32 [B, nb]; norm_gamma f32 [d] or None; with an overlap, x and gate_logit
    point at row `overlap` of rings of overlap + m rows; fold_state f32 [B, S] or None, the update
    state (S >= 4: the open page's closed-rows amax; + 2 * (4 + d) running fold states for m > 16)."""
    B = x.shape[0]
    _check(lib().kv_compress_insert(_ptr(x), x.stride(0), _ptr(gate_logit), gate_logit.stride(0), _ptr(pos_bias),
                                    _ptr(pos0), _ptr(ntok), B, m, overlap, rope_theta, _ptr(norm_gamma), norm_eps,
                                    _ptr(stage), stage.stride(0), _ptr(e0), _ptr(block_table),
                                    block_table.stride(0), dst.c(), 1 if append else 0, _ptr(fold_state),
                                    0 if fold_state is None else fold_state.stride(0), _stream(stream)),
           "kv_compress_insert")


def insert_job(stage, pos0, e0, block_table, dst: PagedCache, m: int, x=None, gate_logit=None, pos_bias=None,
               ntok=None, rope_theta: float = 0.0, append: bool = False, norm_gamma=None,
               norm_eps: float = 1e-6, overlap: int = 0, fold_state=None) -> "CInsertJob":
    """One job of kv_compress_insert_jobs (x None: the open row is already in stage).
    The job holds references to the tensors it names, so they stay alive as
    long as the job does."""
    job = CInsertJob(_ptr(x), 0 if x is None else x.stride(0), _ptr(gate_logit),
                      0 if gate_logit is None else gate_logit.stride(0), _ptr(pos_bias), _ptr(pos0), _ptr(ntok), m,
                      overlap, rope_theta, _ptr(norm_gamma), norm_eps, _ptr(stage), stage.stride(0), _ptr(e0),
                      _ptr(block_table), block_table.stride(0), dst.c(), 1 if append else 0, _ptr(fold_state),
                      0 if fold_state is None else fold_state.stride(0))
    job._keep = (stage, pos0, e0, block_table, dst, x, gate_logit, pos_bias, ntok, norm_gamma, fold_state)
    return job


def kv_compress_insert_jobs(jobs, B: int, stream=None):
    """Several kv_compress_insert calls over the same B sequences in one launch."""
    arr = (CInsertJob * max(len(jobs), 1))(*jobs)
    _check(lib().kv_compress_insert_jobs(arr, len(jobs), B, _stream(stream)), "kv_compress_insert_jobs")


def kv_quantize_page_workspace(B: int, max_ne: int, dst: PagedCache) -> int:
    return int(lib().kv_quantize_page_workspace(B, max_ne, dst.c()))


def kv_quantize_page(src, e0, ne, max_ne: int, block_table, dst: PagedCache, ws=None, stream=None):
    """src f32 [B, rows, dim]; e0, ne int32 [B]; block_table int32 [B, nb];
    ws: None or a uint8 tensor of kv_quantize_page_workspace(...) bytes (fp8 pages split over blocks)."""
    B = src.shape[0]
    wp, wn = (None, 0) if ws is None else (_ptr(ws), ws.numel() * ws.element_size())
    _check(lib().kv_quantize_page(_ptr(src), src.stride(0), _ptr(e0), _ptr(ne), B, max_ne, _ptr(block_table),
                                  block_table.stride(0), dst.c(), wp, wn, _stream(stream)), "kv_quantize_page")


def indexer_topk_workspace(B: int, max_seq_len: int, m: int, k: int) -> int:
    return int(lib().indexer_topk_workspace(B, max_seq_len, m, k))


def indexer_topk(q_idx, head_w, idx_keys: PagedCache, block_table, seq_lens, max_seq_len: int, m: int, k: int,
                 out_idx, out_n, ws, stream=None):
    """q_idx bf16 [B, HI, dI]; head_w f32 [B, HI]; out_idx int32 [B, k]; out_n int32 [B];
    ws: uint8 workspace, zero-filled before its first use (left zeroed by every call)."""
    B, HI, _ = q_idx.shape
    _check(lib().indexer_topk(_ptr(q_idx), _ptr(head_w), HI, idx_keys.c(), _ptr(block_table),
                              block_table.stride(0), _ptr(seq_lens), B, max_seq_len, m, k, _ptr(out_idx),
                              _ptr(out_n), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "indexer_topk")


def indexer_topk_with_updates(q_idx, head_w, idx_keys: PagedCache, block_table, seq_lens, max_seq_len: int, m: int,
                              k: int, out_idx, out_n, ws, jobs, stream=None):
    """indexer_topk with update jobs (insert_job(...) descriptors, none writing idx_keys) run beside its score pass;
    the same results as kv_compress_insert_jobs(jobs, B) then indexer_topk(...)."""
    B, HI, _ = q_idx.shape
    arr = (CInsertJob * max(len(jobs), 1))(*jobs)
    _check(lib().indexer_topk_with_updates(_ptr(q_idx), _ptr(head_w), HI, idx_keys.c(), _ptr(block_table),
                                           block_table.stride(0), _ptr(seq_lens), B, max_seq_len, m, k, _ptr(out_idx),
                                           _ptr(out_n), _ptr(ws), ws.numel() * ws.element_size(), arr, len(jobs),
                                           _stream(stream)), "indexer_topk_with_updates")


def indexer_score(q_idx, head_w, idx_keys: PagedCache, block_table, seq_lens, max_seq_len: int, m: int, k: int, ws,
                  stream=None):
    """Measurement hook: the scoring kernel of indexer_topk alone (ws reserved for it)."""
    B, HI, _ = q_idx.shape
    _check(lib().hca_indexer_score(_ptr(q_idx), _ptr(head_w), HI, idx_keys.c(), _ptr(block_table),
                                   block_table.stride(0), _ptr(seq_lens), B, max_seq_len, m, k, _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)), "hca_indexer_score")


def attention_split(q, kv: PagedCache, block_table, win: Optional[PagedCache], win_block_table, seq_lens,
                    max_seq_len: int, m: int, window: int, sel_idx, sel_n, softmax_scale: float, rope_theta: float, ws,
                    stream=None):
    """Measurement hook: the split kernel of paged_hybrid_decode alone (partials into ws, no output)."""
    B, H, d = q.shape
    k = 0 if sel_idx is None else sel_idx.shape[1]
    wc = win.c() if (win is not None and window > 0) else _null_cache()
    wbt = win_block_table if window > 0 else None
    _check(lib().hca_attention_split(_ptr(q), H, kv.c(), _ptr(block_table), block_table.stride(0), wc, _ptr(wbt),
                                     0 if wbt is None else wbt.stride(0), _ptr(seq_lens), B, max_seq_len, m, window,
                                     _ptr(sel_idx), _ptr(sel_n), k, softmax_scale, rope_theta, _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)), "hca_attention_split")


def paged_hybrid_decode_workspace(B: int, H: int, d: int, max_seq_len: int, m: int, window: int, k: int) -> int:
    """k = 0 when the call will attend to all entries (sel_idx None)."""
    return int(lib().paged_hybrid_decode_workspace(B, H, d, max_seq_len, m, window, k))


def paged_hybrid_decode(q, kv: PagedCache, block_table, win: Optional[PagedCache], win_block_table, seq_lens,
                        max_seq_len: int, m: int, window: int, sel_idx, sel_n, softmax_scale: float,
                        rope_theta: float, out, lse, ws, stream=None, out_fp8=None, out_scale=None):
    """q bf16 [B, H, d]; sel_idx int32 [B, k] or None (all entries); out f32 [B, H, d] or None;
    lse f32 [B, H] or None; out_fp8 uint8 [B, H, d] with out_scale f32 [B, H], or None."""
    B, H, d = q.shape
    k = 0 if sel_idx is None else sel_idx.shape[1]
    wc = win.c() if (win is not None and window > 0) else _null_cache()
    wbt = win_block_table if window > 0 else None
    _check(lib().paged_hybrid_decode(_ptr(q), H, kv.c(), _ptr(block_table), block_table.stride(0), wc, _ptr(wbt),
                                     0 if wbt is None else wbt.stride(0), _ptr(seq_lens), B, max_seq_len, m, window,
                                     _ptr(sel_idx), _ptr(sel_n), k, softmax_scale, rope_theta, _ptr(out), _ptr(lse),
                                     _ptr(out_fp8), _ptr(out_scale), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)), "paged_hybrid_decode")


def paged_hybrid_decode_noalloc_max_bytes() -> int:
    return int(lib().paged_hybrid_decode_noalloc_max_bytes())


def paged_hybrid_decode_noalloc(q, kv: PagedCache, block_table, win: Optional[PagedCache], win_block_table, seq_lens,
                                max_seq_len: int, m: int, window: int, sel_idx, sel_n, softmax_scale: float,
                                rope_theta: float, out, lse, stream=None, out_fp8=None, out_scale=None):
    """paged_hybrid_decode with the library's static per-GPU scratch instead of a workspace
    (allocates nothing; calls that overlap in time on one GPU race)."""
    B, H, d = q.shape
    k = 0 if sel_idx is None else sel_idx.shape[1]
    wc = win.c() if (win is not None and window > 0) else _null_cache()
    wbt = win_block_table if window > 0 else None
    _check(lib().paged_hybrid_decode_noalloc(_ptr(q), H, kv.c(), _ptr(block_table), block_table.stride(0), wc,
                                             _ptr(wbt), 0 if wbt is None else wbt.stride(0), _ptr(seq_lens), B,
                                             max_seq_len, m, window, _ptr(sel_idx), _ptr(sel_n), k, softmax_scale,
                                             rope_theta, _ptr(out), _ptr(lse), _ptr(out_fp8), _ptr(out_scale),
                                             _stream(stream)), "paged_hybrid_decode_noalloc")


def kv_gather(src: PagedCache, block_table, n_rows, max_rows: int, dst_codes, dst_scales, stream=None):
    B = n_rows.shape[0]
    _check(lib().kv_gather(src.c(), _ptr(block_table), block_table.stride(0), _ptr(n_rows), B, max_rows,
                           _ptr(dst_codes), _ptr(dst_scales), _stream(stream)), "kv_gather")


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled, 256-byte aligned workspace of at least nbytes."""
    return torch.zeros((max(1, nbytes),), dtype=torch.uint8, device=device)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


# ----------------------------------------------------------------- page-pool packing


def page_bytes(m: int, dim: int, dtype: str):
    """(code bytes, scale bytes) of one page of a KV kind."""
    c, sc = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().hca_page_bytes(CKvKind(m, dim, DTYPES[dtype]), ctypes.byref(c), ctypes.byref(sc)), "hca_page_bytes")
    return c.value, sc.value


class PagePool:
    """Size buckets of fixed-size pages for several KV kinds in one device arena.

    kinds: [(m, dim, dtype)]; capacity: pages per bucket (bucket_of(kind) maps
    a kind to its bucket).  `arena_bytes` is what the caller allocates;
    `view(kind, arena)` is the PagedCache of a kind inside it."""

    def __init__(self, kinds, capacity):
        self.kinds = list(kinds)
        arr = (CKvKind * len(self.kinds))(*[CKvKind(m, d, DTYPES[t]) for m, d, t in self.kinds])
        self._karr = arr
        kb = (ctypes.c_int32 * len(self.kinds))()
        nb = ctypes.c_int32(0)
        _check(lib().hca_pool_plan(arr, len(self.kinds), kb, ctypes.byref(nb)), "hca_pool_plan")
        self.kind_bucket = list(kb)
        self.n_buckets = nb.value
        cap = list(capacity) if hasattr(capacity, "__len__") else [int(capacity)] * self.n_buckets
        carr = (ctypes.c_int32 * max(1, self.n_buckets))(*cap)
        ab = ctypes.c_size_t(0)
        h = ctypes.c_void_p(0)
        _check(lib().hca_pool_create(arr, len(self.kinds), carr, ctypes.byref(ab), ctypes.byref(h)), "hca_pool_create")
        self._h = h
        self.arena_bytes = ab.value

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            try:
                _lib.hca_pool_destroy(h)
            except Exception:  # interpreter shutdown
                pass
            self._h = None

    def bucket_of(self, kind: int) -> int:
        return self.kind_bucket[kind]

    def view(self, kind: int, arena) -> "PagedCache":
        c = CPagedCache()
        _check(lib().hca_pool_view(self._h, kind, _ptr(arena), ctypes.byref(c)), "hca_pool_view")
        import torch

        m, d, t = self.kinds[kind]
        epp = 256 // m
        cb, sb = page_bytes(m, d, t)
        base = arena.data_ptr()
        n = c.num_pages
        off_c = c.codes - base
        codes = arena[off_c: off_c + n * cb]
        if t == "bf16":
            codes = codes.view(torch.int16).view(n, epp, d)
            scales = None
        elif t == "fp8":
            codes = codes.view(n, epp, d)
            off_s = c.scales - base
            scales = arena[off_s: off_s + n * sb].view(torch.float32)
        else:
            codes = codes.view(n, epp, d // 2)
            off_s = c.scales - base
            scales = arena[off_s: off_s + n * sb].view(n, epp, d // 32)
        return PagedCache(codes, scales, epp, d, t)

    def alloc(self, bucket: int, n: int):
        out = (ctypes.c_int32 * max(1, n))()
        _check(lib().hca_pool_alloc(self._h, bucket, n, out), "hca_pool_alloc")
        return list(out)[:n]

    def share(self, bucket: int, pages):
        arr = (ctypes.c_int32 * max(1, len(pages)))(*pages)
        _check(lib().hca_pool_share(self._h, bucket, arr, len(pages)), "hca_pool_share")

    def release(self, bucket: int, pages):
        arr = (ctypes.c_int32 * max(1, len(pages)))(*pages)
        _check(lib().hca_pool_release(self._h, bucket, arr, len(pages)), "hca_pool_release")

    def publish(self, bucket: int, page: int, key: int):
        _check(lib().hca_pool_publish(self._h, bucket, page, key), "hca_pool_publish")

    def lookup(self, bucket: int, key: int) -> int:
        p = ctypes.c_int32(-1)
        _check(lib().hca_pool_lookup(self._h, bucket, key, ctypes.byref(p)), "hca_pool_lookup")
        return p.value

    def stats(self, bucket: int):
        """(free, cached, held) pages and the codes and scales offsets in the arena."""
        v = [ctypes.c_int64(0) for _ in range(3)] + [ctypes.c_size_t(0) for _ in range(2)]
        _check(lib().hca_pool_stats(self._h, bucket, *[ctypes.byref(x) for x in v]), "hca_pool_stats")
        return tuple(x.value for x in v)
