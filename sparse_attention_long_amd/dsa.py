"""Python binding of the DSA C ABI (include/dsa.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Tensor arguments
may be torch tensors on the GPU (their data pointers are passed) or plain
integer device addresses.  `stream` defaults to torch's current stream.
A non-zero status raises DSAError with the library's own message.  There is
no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)

# Every symbol include/dsa.h declares.
EXPORTS = (
    "dsa_indexer_scores", "dsa_topk", "dsa_attn_workspace_size", "dsa_sparse_mla_attn",
    "dsa_forward_workspace_size", "dsa_forward", "dsa_quantize_e4m3", "dsa_cache_append",
    "dsa_indexer_scores_paged", "dsa_topk_paged", "dsa_sparse_mla_attn_paged", "dsa_forward_paged",
    "dsa_gather_stats", "dsa_indexer_kl", "dsa_forward_kl", "dsa_selection_mask", "dsa_mha_decompress",
    "dsa_masked_mha_attn", "dsa_masked_mha_workspace_size", "dsa_masked_mha_forward", "dsa_status_string",
    "dsa_last_error", "dsa_version", "dsa_topk_workspace_size", "dsa_topk_ws", "dsa_forward_plan_of",
    "dsa_validate", "dsa_sparse_mla_attn_noalloc",
)

# dsa_validate's counters, in order.
VALIDATE_COUNTS = ("bad_q_scale", "nonfinite_w", "bad_k_scale", "idx_out_of_range", "idx_rows_not_canonical",
                   "seq_lens_out_of_range", "page_entries_out_of_range", "reserved")


class DSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q", "n_kv", "q_pos0", "idx_heads", "idx_dim", "heads", "dim_qk", "dim_v", "topk")]

    @classmethod
    def of(cls, wl=None, **kw):
        """Dims from a workload object (anything with these attribute names) and/or keywords."""
        vals = {n: getattr(wl, n) for n, _ in cls._fields_} if wl is not None else {}
        vals.update(kw)
        return cls(**vals)


class PagedKV(ctypes.Structure):
    """dsa_paged_kv: device pointers (ints) to seq_lens [B] and page_table
    [B, max_pages] (0 for dense caches), and the page geometry."""
    _fields_ = [("seq_lens", ctypes.c_void_p), ("page_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int32)]

    @classmethod
    def of(cls, seq_lens, page_table=None, page_size: int = 0, max_pages: int = 0, num_pages: int = 0):
        return cls(_ptr(seq_lens), _ptr(page_table), page_size, max_pages, num_pages)


class ForwardPlan(ctypes.Structure):
    """dsa_forward_plan: how dsa_forward splits its work for given dims."""
    _fields_ = [("chunk_rows", ctypes.c_int64), ("topk_parts", ctypes.c_int32), ("attn_splits", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t)]


_lib = None
_P = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        D = ctypes.POINTER(Dims)
        L.dsa_indexer_scores.argtypes = [D, _P, _P, _P, _P, _P, _P, ctypes.c_int64, _P]
        L.dsa_topk.argtypes = [D, _P, ctypes.c_int64, _P, _P]
        L.dsa_attn_workspace_size.argtypes = [D]
        L.dsa_attn_workspace_size.restype = ctypes.c_size_t
        L.dsa_sparse_mla_attn.argtypes = [D, _P, _P, _P, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]
        L.dsa_forward_workspace_size.argtypes = [D]
        L.dsa_forward_workspace_size.restype = ctypes.c_size_t
        L.dsa_forward.argtypes = [D, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.dsa_quantize_e4m3.argtypes = [_P, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, _P, _P, _P]
        L.dsa_cache_append.argtypes = [D, _P, ctypes.c_int, _P, _P, _P, _P, _P]
        K = ctypes.POINTER(PagedKV)
        L.dsa_indexer_scores_paged.argtypes = [D, K, _P, _P, _P, _P, _P, _P, ctypes.c_int64, _P]
        L.dsa_topk_paged.argtypes = [D, K, _P, ctypes.c_int64, _P, _P]
        L.dsa_sparse_mla_attn_paged.argtypes = [D, K, _P, _P, _P, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]
        L.dsa_forward_paged.argtypes = [D, K, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P,
                                        ctypes.c_size_t, _P]
        L.dsa_gather_stats.argtypes = [D, ctypes.c_int32, _P, _P, _P]
        L.dsa_indexer_kl.argtypes = [D, K, _P, _P, _P, _P, _P, ctypes.c_int64, ctypes.c_float, _P, _P]
        L.dsa_forward_kl.argtypes = [D, K, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P,
                                     ctypes.c_size_t, _P]
        I32 = ctypes.c_int32
        L.dsa_selection_mask.argtypes = [D, _P, _P, _P]
        L.dsa_mha_decompress.argtypes = [D, I32, I32, _P, _P, _P, I32, _P, _P, _P]
        L.dsa_masked_mha_attn.argtypes = [D, I32, I32, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P]
        L.dsa_masked_mha_workspace_size.argtypes = [D, I32, I32]
        L.dsa_masked_mha_workspace_size.restype = ctypes.c_size_t
        L.dsa_masked_mha_forward.argtypes = [D, I32, I32, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P,
                                             _P, _P, _P, ctypes.c_size_t, _P]
        L.dsa_topk_workspace_size.argtypes = [D]
        L.dsa_topk_workspace_size.restype = ctypes.c_size_t
        L.dsa_topk_ws.argtypes = [D, _P, ctypes.c_int64, _P, _P, ctypes.c_size_t, _P]
        L.dsa_forward_plan_of.argtypes = [D, ctypes.POINTER(ForwardPlan)]
        L.dsa_validate.argtypes = [D, K, _P, _P, _P, _P, _P, _P]
        L.dsa_sparse_mla_attn_noalloc.argtypes = [D, _P, _P, _P, ctypes.c_float, _P, _P, _P]
        L.dsa_status_string.argtypes = [ctypes.c_int]
        L.dsa_status_string.restype = ctypes.c_char_p
        L.dsa_last_error.restype = ctypes.c_char_p
        for f in ("dsa_indexer_scores", "dsa_topk", "dsa_sparse_mla_attn", "dsa_forward", "dsa_quantize_e4m3",
                  "dsa_cache_append", "dsa_indexer_scores_paged", "dsa_topk_paged", "dsa_sparse_mla_attn_paged",
                  "dsa_forward_paged", "dsa_gather_stats", "dsa_indexer_kl", "dsa_forward_kl", "dsa_selection_mask",
                  "dsa_mha_decompress", "dsa_masked_mha_attn", "dsa_masked_mha_forward", "dsa_version",
                  "dsa_topk_ws", "dsa_forward_plan_of", "dsa_validate", "dsa_sparse_mla_attn_noalloc"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int):
    if status != OK:
        L = lib()
        raise DSAError(status, f"{L.dsa_status_string(status).decode()}: {L.dsa_last_error().decode()}")


def dsa_version() -> int:
    return lib().dsa_version()


def dsa_indexer_scores(dims: Dims, q_idx, q_scale, w_idx, k_idx, k_scale, scores, ld: int, stream=None):
    _check(lib().dsa_indexer_scores(ctypes.byref(dims), _ptr(q_idx), _ptr(q_scale), _ptr(w_idx), _ptr(k_idx),
                                    _ptr(k_scale), _ptr(scores), int(ld), _stream(stream)))


def dsa_topk(dims: Dims, scores, ld: int, idx, stream=None):
    _check(lib().dsa_topk(ctypes.byref(dims), _ptr(scores), int(ld), _ptr(idx), _stream(stream)))


def dsa_topk_workspace_size(dims: Dims) -> int:
    return int(lib().dsa_topk_workspace_size(ctypes.byref(dims)))


def dsa_topk_ws(dims: Dims, scores, ld: int, idx, ws=None, ws_bytes: int = 0, stream=None):
    _check(lib().dsa_topk_ws(ctypes.byref(dims), _ptr(scores), int(ld), _ptr(idx), _ptr(ws), int(ws_bytes),
                             _stream(stream)))


def dsa_forward_plan_of(dims: Dims) -> ForwardPlan:
    plan = ForwardPlan()
    _check(lib().dsa_forward_plan_of(ctypes.byref(dims), ctypes.byref(plan)))
    return plan


def dsa_validate(dims: Dims, layout, q_scale, w_idx, k_scale, idx, counts, stream=None):
    """layout: a PagedKV, or None for dense caches; any input may be None to
    skip its check.  counts: device int32 [8] (see VALIDATE_COUNTS)."""
    _check(lib().dsa_validate(ctypes.byref(dims), ctypes.byref(layout) if layout is not None else None,
                              _ptr(q_scale), _ptr(w_idx), _ptr(k_scale), _ptr(idx), _ptr(counts), _stream(stream)))


def dsa_attn_workspace_size(dims: Dims) -> int:
    return int(lib().dsa_attn_workspace_size(ctypes.byref(dims)))


def dsa_sparse_mla_attn(dims: Dims, q, kv, idx, sm_scale: float, out, lse=None, ws=None, ws_bytes: int = 0,
                        stream=None):
    _check(lib().dsa_sparse_mla_attn(ctypes.byref(dims), _ptr(q), _ptr(kv), _ptr(idx), float(sm_scale), _ptr(out),
                                     _ptr(lse), _ptr(ws), int(ws_bytes), _stream(stream)))


def dsa_sparse_mla_attn_noalloc(dims: Dims, q, kv, idx, sm_scale: float, out, lse=None, stream=None):
    _check(lib().dsa_sparse_mla_attn_noalloc(ctypes.byref(dims), _ptr(q), _ptr(kv), _ptr(idx), float(sm_scale),
                                             _ptr(out), _ptr(lse), _stream(stream)))


def dsa_forward_workspace_size(dims: Dims) -> int:
    return int(lib().dsa_forward_workspace_size(ctypes.byref(dims)))


def dsa_forward(dims: Dims, q_idx, q_scale, w_idx, k_idx, k_scale, q, kv, sm_scale: float, out, lse=None,
                idx_out=None, ws=None, ws_bytes: int = 0, stream=None):
    _check(lib().dsa_forward(ctypes.byref(dims), _ptr(q_idx), _ptr(q_scale), _ptr(w_idx), _ptr(k_idx),
                             _ptr(k_scale), _ptr(q), _ptr(kv), float(sm_scale), _ptr(out), _ptr(lse),
                             _ptr(idx_out), _ptr(ws), int(ws_bytes), _stream(stream)))


def _dtype_code(x, dtype):
    if dtype is not None:
        return int(dtype)
    name = str(getattr(x, "dtype", ""))
    if "float32" in name:
        return 0
    if "bfloat16" in name or "int16" in name:
        return 1
    raise ValueError("pass dtype=0 (f32) or dtype=1 (bf16) for raw pointers")


def dsa_quantize_e4m3(x, n_tokens: int, token_len: int, codes, scales, dtype=None, stream=None):
    """x: f32 or bf16 (bits in an int16 / bfloat16 tensor); codes uint8; scales f32."""
    _check(lib().dsa_quantize_e4m3(_ptr(x), _dtype_code(x, dtype), int(n_tokens), int(token_len), _ptr(codes),
                                   _ptr(scales), _stream(stream)))


def dsa_cache_append(dims: Dims, k_new, k_idx, k_scale, kv_new=None, kv=None, k_dtype=None, stream=None):
    _check(lib().dsa_cache_append(ctypes.byref(dims), _ptr(k_new), _dtype_code(k_new, k_dtype), _ptr(kv_new),
                                  _ptr(k_idx), _ptr(k_scale), _ptr(kv), _stream(stream)))


def dsa_indexer_scores_paged(dims: Dims, layout: PagedKV, q_idx, q_scale, w_idx, k_idx, k_scale, scores, ld: int,
                             stream=None):
    _check(lib().dsa_indexer_scores_paged(ctypes.byref(dims), ctypes.byref(layout), _ptr(q_idx), _ptr(q_scale),
                                          _ptr(w_idx), _ptr(k_idx), _ptr(k_scale), _ptr(scores), int(ld),
                                          _stream(stream)))


def dsa_topk_paged(dims: Dims, layout: PagedKV, scores, ld: int, idx, stream=None):
    _check(lib().dsa_topk_paged(ctypes.byref(dims), ctypes.byref(layout), _ptr(scores), int(ld), _ptr(idx),
                                _stream(stream)))


def dsa_sparse_mla_attn_paged(dims: Dims, layout: PagedKV, q, kv, idx, sm_scale: float, out, lse=None, ws=None,
                              ws_bytes: int = 0, stream=None):
    _check(lib().dsa_sparse_mla_attn_paged(ctypes.byref(dims), ctypes.byref(layout), _ptr(q), _ptr(kv), _ptr(idx),
                                           float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws), int(ws_bytes),
                                           _stream(stream)))


def dsa_forward_paged(dims: Dims, layout: PagedKV, q_idx, q_scale, w_idx, k_idx, k_scale, q, kv, sm_scale: float,
                      out, lse=None, idx_out=None, ws=None, ws_bytes: int = 0, stream=None):
    _check(lib().dsa_forward_paged(ctypes.byref(dims), ctypes.byref(layout), _ptr(q_idx), _ptr(q_scale),
                                   _ptr(w_idx), _ptr(k_idx), _ptr(k_scale), _ptr(q), _ptr(kv), float(sm_scale),
                                   _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(ws), int(ws_bytes), _stream(stream)))


def dsa_gather_stats(dims: Dims, page_size: int, idx, stats, stream=None):
    _check(lib().dsa_gather_stats(ctypes.byref(dims), int(page_size), _ptr(idx), _ptr(stats), _stream(stream)))


def dsa_indexer_kl(dims: Dims, layout, q, kv, idx, lse, scores, ld: int, sm_scale: float, kl, stream=None):
    """layout: a PagedKV, or None for dense caches."""
    _check(lib().dsa_indexer_kl(ctypes.byref(dims), ctypes.byref(layout) if layout is not None else None, _ptr(q),
                                _ptr(kv), _ptr(idx), _ptr(lse), _ptr(scores), int(ld), float(sm_scale), _ptr(kl),
                                _stream(stream)))


def dsa_forward_kl(dims: Dims, layout, q_idx, q_scale, w_idx, k_idx, k_scale, q, kv, sm_scale: float, out, lse,
                   idx_out, kl, ws=None, ws_bytes: int = 0, stream=None):
    """layout: a PagedKV, or None for dense caches."""
    _check(lib().dsa_forward_kl(ctypes.byref(dims), ctypes.byref(layout) if layout is not None else None,
                                _ptr(q_idx), _ptr(q_scale), _ptr(w_idx), _ptr(k_idx), _ptr(k_scale), _ptr(q),
                                _ptr(kv), float(sm_scale), _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(kl), _ptr(ws),
                                int(ws_bytes), _stream(stream)))


def dsa_selection_mask(dims: Dims, idx, mask, stream=None):
    _check(lib().dsa_selection_mask(ctypes.byref(dims), _ptr(idx), _ptr(mask), _stream(stream)))


def dsa_mha_decompress(dims: Dims, dim_nope: int, dim_vh: int, kv, w_uk, w_uv, n_rows: int, k_mha, v_mha,
                       stream=None):
    _check(lib().dsa_mha_decompress(ctypes.byref(dims), int(dim_nope), int(dim_vh), _ptr(kv), _ptr(w_uk), _ptr(w_uv),
                                    int(n_rows), _ptr(k_mha), _ptr(v_mha), _stream(stream)))


def dsa_masked_mha_attn(dims: Dims, dim_nope: int, dim_vh: int, q_mha, kv, k_mha, v_mha, mask, sm_scale: float, out,
                        lse=None, stream=None):
    _check(lib().dsa_masked_mha_attn(ctypes.byref(dims), int(dim_nope), int(dim_vh), _ptr(q_mha), _ptr(kv),
                                     _ptr(k_mha), _ptr(v_mha), _ptr(mask), float(sm_scale), _ptr(out), _ptr(lse),
                                     _stream(stream)))


def dsa_masked_mha_workspace_size(dims: Dims, dim_nope: int, dim_vh: int) -> int:
    return int(lib().dsa_masked_mha_workspace_size(ctypes.byref(dims), int(dim_nope), int(dim_vh)))


def dsa_masked_mha_forward(dims: Dims, dim_nope: int, dim_vh: int, q_idx, q_scale, w_idx, k_idx, k_scale, q_mha, kv,
                           w_uk, w_uv, sm_scale: float, out, lse=None, idx_out=None, ws=None, ws_bytes: int = 0,
                           stream=None):
    _check(lib().dsa_masked_mha_forward(ctypes.byref(dims), int(dim_nope), int(dim_vh), _ptr(q_idx), _ptr(q_scale),
                                        _ptr(w_idx), _ptr(k_idx), _ptr(k_scale), _ptr(q_mha), _ptr(kv), _ptr(w_uk),
                                        _ptr(w_uv), float(sm_scale), _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(ws),
                                        int(ws_bytes), _stream(stream)))
