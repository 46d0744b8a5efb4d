"""Python binding of libqas (query-aware sparse attention over a paged KV
cache, HIP for gfx950).

Argument marshalling only: every function below forwards torch tensors'
device pointers and the current HIP stream to the C entry point of the same
name declared in include/qas.h.  All computation runs in the library's HIP
kernels; there is no fallback path, and importing this package fails loudly
if libqas.so has not been built (``python -m query_aware_sparse_amd.build``).
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# QAS_LIB_PATH selects another build of the same library (same ABI)
LIB_PATH = os.environ.get("QAS_LIB_PATH") or os.path.join(_HERE, "libqas.so")

QAS_OK = 0
QAS_F32, QAS_F16, QAS_BF16, QAS_FP8_E4M3 = 0, 1, 2, 3
QAS_OP_SPARSE_DECODE, QAS_OP_DECODE_LAYER = 1, 2

_TORCH_DTYPE = {torch.float32: QAS_F32, torch.float16: QAS_F16,
                torch.bfloat16: QAS_BF16, torch.float8_e4m3fn: QAS_FP8_E4M3}


class QasError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"qas status {status}: {detail}")
        self.status = status


class qas_cache(ctypes.Structure):
    _fields_ = [("page_size", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("num_pool_pages", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("summary", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("summary_fp8", ctypes.c_void_p),
                ("summary_fp8_scale", ctypes.c_void_p)]


class qas_batch(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("total_pages", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("seq_lens", ctypes.c_void_p), ("page_indptr", ctypes.c_void_p),
                ("page_indices", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGNATURES = {
    "qas_append": (_I, [_P, _P, _P, _I, _I, _P, _P, _P]),
    "qas_append_fp8": (_I, [_P, _P, _P, _I, _I, _P, _P, _I, _P]),
    "qas_rollback": (_I, [_P, _P, _P]),
    "qas_score_pages": (_I, [_P, _P, _P, _I, _I, _P, _P]),
    "qas_topk_pages": (_I, [_P, _P, _I, _I, _I, _P, _P, _P]),
    "qas_selection_capacity": (_I, [_I, _I, _I, _I]),
    "qas_select_pages": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _P]),
    "qas_sparse_decode": (_I, [_P, _P, _P, _I, _I, _P, _I, _I, ctypes.c_float,
                               _P, _P, _P, ctypes.c_size_t, _P]),
    "qas_decode_layer": (_I, [_P, _P, _P, _I, _I, _I, ctypes.c_float, _P, _P, _P,
                              _P, _P, _P, ctypes.c_size_t, _P]),
    "qas_decode_layer_mixed": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, ctypes.c_float, _P, _P,
                                    _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "qas_decode_layer_noalloc": (_I, [_P, _P, _P, _I, _I, _I, ctypes.c_float, _P, _P, _P,
                                      _P, _P, _P]),
    "qas_workspace_bytes": (ctypes.c_size_t, [_I, _P, _P, _I, _I]),
    "qas_decode_positions": (_I, [_P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P, _P, _P, _P,
                                  ctypes.c_size_t, _P]),
    "qas_positions_workspace_bytes": (ctypes.c_size_t, [_P, _P, _I, _I, _I]),
    "qas_exact_top_r": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "qas_exact_top_r_workspace_bytes": (ctypes.c_size_t, [_P, _P, _I, _I]),
    "qas_chunk_groups": (_I, [_I, _I, _I]),
    "qas_regroup_queries": (_I, [_P, _P, _I, _P, _I, _I, _I, _I, _I, _P, _P]),
    "qas_union_pages": (_I, [_P, _P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "qas_chunk_attention": (_I, [_P, _P, _P, _I, _P, _P, _I, _I, _P, _I, _I, _P,
                                 ctypes.c_float, _P, _P, _P]),
    "qas_status_string": (ctypes.c_char_p, [_I]),
    "qas_last_error": (ctypes.c_char_p, []),
    "qas_version": (ctypes.c_char_p, []),
}


_lib = None


def _load():
    """Load libqas.so on first use (so the build step can import this package
    before the library exists); raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -m query_aware_sparse_amd.build` "
                "(there is no non-HIP fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def __getattr__(name):
    if name == "lib":
        return _load()
    raise AttributeError(name)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status):
    if status != QAS_OK:
        raise QasError(status, _load().qas_last_error().decode())


def dtype_code(t):
    return _TORCH_DTYPE[t.dtype]


def make_cache(k_pool, v_pool, summary, k_scale=None, v_scale=None, summary_fp8=None,
               summary_fp8_scale=None):
    """qas_cache over caller-owned tensors: pools [pages][H_kv][S][d],
    summary [pages][H_kv][2][d], optional e4m3 summary copy (uint8 codes
    [pages][H_kv][2][d] and float scales [pages][H_kv]).  The tensors must
    outlive every call."""
    pages, H_kv, S, d = k_pool.shape
    c = qas_cache(S, d, H_kv, pages, dtype_code(k_pool), 0, k_pool.data_ptr(),
                  v_pool.data_ptr(), 0 if summary is None else summary.data_ptr(),
                  0 if k_scale is None else k_scale.data_ptr(),
                  0 if v_scale is None else v_scale.data_ptr(),
                  0 if summary_fp8 is None else summary_fp8.data_ptr(),
                  0 if summary_fp8_scale is None else summary_fp8_scale.data_ptr())
    c._keep = (k_pool, v_pool, summary, k_scale, v_scale, summary_fp8, summary_fp8_scale)
    return c


def make_batch(seq_lens, page_indptr, page_indices, total_pages, max_pages):
    """qas_batch over int32 device tensors; total/max pages are host ints."""
    b = qas_batch(seq_lens.numel(), int(total_pages), int(max_pages), 0,
                  seq_lens.data_ptr(), page_indptr.data_ptr(),
                  0 if page_indices is None else page_indices.data_ptr())
    b._keep = (seq_lens, page_indptr, page_indices)
    return b


def qas_append(cache, batch, new_indptr, total_new, max_new, k_new, v_new, stream=None):
    _check(_load().qas_append(ctypes.byref(cache), ctypes.byref(batch), _ptr(new_indptr),
                          int(total_new), int(max_new), _ptr(k_new), _ptr(v_new),
                          _stream(stream)))


def qas_append_fp8(cache, batch, new_indptr, total_new, max_new, k_new, v_new, stream=None):
    """Quantise new K/V rows (f32/f16/bf16 tensors [total_new][H_kv][128])
    into an FP8 E4M3 chunk cache with its per-head scales (see qas.h)."""
    if k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must share a dtype")
    _check(_load().qas_append_fp8(ctypes.byref(cache), ctypes.byref(batch), _ptr(new_indptr),
                              int(total_new), int(max_new), _ptr(k_new), _ptr(v_new),
                              dtype_code(k_new), _stream(stream)))


def qas_rollback(cache, batch, stream=None):
    """Rebuild the tail-page summaries after the cache is cut back to
    batch's seq_lens (see qas.h)."""
    _check(_load().qas_rollback(ctypes.byref(cache), ctypes.byref(batch), _stream(stream)))


def qas_score_pages(cache, batch, q, scores, stream=None):
    _check(_load().qas_score_pages(ctypes.byref(cache), ctypes.byref(batch), _ptr(q),
                               dtype_code(q), q.shape[1], _ptr(scores), _stream(stream)))


def qas_topk_pages(scores, batch, num_kv_heads, page_size, k, sel, sel_count=None,
                   stream=None):
    _check(_load().qas_topk_pages(_ptr(scores), ctypes.byref(batch), int(num_kv_heads),
                              int(page_size), int(k), _ptr(sel), _ptr(sel_count),
                              _stream(stream)))


def qas_selection_capacity(k, page_size, sink_tokens, local_tokens):
    return int(_load().qas_selection_capacity(int(k), int(page_size), int(sink_tokens),
                                              int(local_tokens)))


def qas_select_pages(scores, batch, num_kv_heads, page_size, k, sink_tokens, local_tokens, sel,
                     sel_count=None, stream=None):
    """sel: int32 [B][H_kv][stride], stride >= qas_selection_capacity(...)."""
    _check(_load().qas_select_pages(_ptr(scores), ctypes.byref(batch), int(num_kv_heads),
                                    int(page_size), int(k), int(sink_tokens), int(local_tokens),
                                    _ptr(sel), sel.shape[-1], _ptr(sel_count), _stream(stream)))


def qas_workspace_bytes(op, cache, batch, num_q_heads, k):
    return int(_load().qas_workspace_bytes(int(op), ctypes.byref(cache), ctypes.byref(batch),
                                       int(num_q_heads), int(k)))


def make_workspace(op, cache, batch, num_q_heads, k, device="cuda"):
    """A zero-filled device workspace of qas_workspace_bytes() for `op`."""
    n = qas_workspace_bytes(op, cache, batch, num_q_heads, k)
    return torch.zeros(max(n, 1), dtype=torch.uint8, device=device)


def qas_sparse_decode(cache, batch, q, sel, sel_len, sm_scale, out, lse, workspace,
                      stream=None):
    _check(_load().qas_sparse_decode(ctypes.byref(cache), ctypes.byref(batch), _ptr(q),
                                 dtype_code(q), q.shape[1], _ptr(sel), sel.shape[-1],
                                 int(sel_len), float(sm_scale), _ptr(out), _ptr(lse),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream)))


def qas_decode_layer(cache, batch, q, k, sm_scale, out, lse, workspace, k_new=None,
                     v_new=None, sel_out=None, stream=None):
    _check(_load().qas_decode_layer(ctypes.byref(cache), ctypes.byref(batch), _ptr(q),
                                dtype_code(q), q.shape[1], int(k), float(sm_scale),
                                _ptr(k_new), _ptr(v_new), _ptr(sel_out), _ptr(out),
                                _ptr(lse), _ptr(workspace),
                                workspace.numel() * workspace.element_size(),
                                _stream(stream)))


def qas_decode_layer_noalloc(cache, batch, q, k, sm_scale, out, lse, k_new=None, v_new=None,
                             sel_out=None, stream=None):
    """qas_decode_layer with the library's per-GPU static scratch instead of a
    caller workspace (no device allocation; overlapping calls on one GPU race)."""
    _check(_load().qas_decode_layer_noalloc(ctypes.byref(cache), ctypes.byref(batch), _ptr(q),
                                            dtype_code(q), q.shape[1], int(k), float(sm_scale),
                                            _ptr(k_new), _ptr(v_new), _ptr(sel_out), _ptr(out),
                                            _ptr(lse), _stream(stream)))


def qas_decode_layer_mixed(cache, batch, q, k, sink_tokens, local_tokens, sm_scale, out, lse,
                           workspace, k_new=None, v_new=None, sel_out=None, stream=None):
    _check(_load().qas_decode_layer_mixed(ctypes.byref(cache), ctypes.byref(batch), _ptr(q),
                                          dtype_code(q), q.shape[1], int(k), int(sink_tokens),
                                          int(local_tokens), float(sm_scale), _ptr(k_new),
                                          _ptr(v_new), _ptr(sel_out), _ptr(out), _ptr(lse),
                                          _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(stream)))


def qas_positions_workspace_bytes(cache, batch, num_q_heads, gamma, k):
    return int(_load().qas_positions_workspace_bytes(ctypes.byref(cache), ctypes.byref(batch),
                                                     int(num_q_heads), int(gamma), int(k)))


def qas_decode_positions(cache, batch, q, k, sm_scale, out, lse, workspace, sel_out=None,
                         stream=None):
    """q: [B][gamma][H_q][d] draft-position queries (the drafts already
    appended); out like q; lse [B][gamma][H_q] or None; sel_out
    [B][gamma][H_kv][k] or None."""
    _check(_load().qas_decode_positions(ctypes.byref(cache), ctypes.byref(batch), _ptr(q),
                                        dtype_code(q), q.shape[2], q.shape[1], int(k),
                                        float(sm_scale), _ptr(sel_out), _ptr(out), _ptr(lse),
                                        _ptr(workspace),
                                        workspace.numel() * workspace.element_size(),
                                        _stream(stream)))


def qas_exact_top_r_workspace_bytes(cache, batch, num_q_heads, R):
    return int(_load().qas_exact_top_r_workspace_bytes(ctypes.byref(cache), ctypes.byref(batch),
                                                       int(num_q_heads), int(R)))


def qas_exact_top_r(cache, batch, q, R, top_tokens, top_logits, workspace, pages_read=None,
                    stream=None):
    """Exact token top-R per (request, query head) by branch-and-bound over
    the page bounds; q [B][H_q][d], outputs [B][H_q][R], workspace of
    qas_exact_top_r_workspace_bytes (see qas.h)."""
    _check(_load().qas_exact_top_r(ctypes.byref(cache), ctypes.byref(batch), _ptr(q),
                                   dtype_code(q), q.shape[1], int(R), _ptr(top_tokens),
                                   _ptr(top_logits), _ptr(pages_read), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(),
                                   _stream(stream)))


def qas_chunk_groups(num_queries, batch, group):
    return int(_load().qas_chunk_groups(int(num_queries), int(batch), int(group)))


def qas_regroup_queries(batch, q_indptr, sets, page_size, window, group, ids, stream=None):
    """sets: int32 [N][H_kv][kq]; ids: int32 [H_kv][N] (execution order out)."""
    N, H_kv, kq = sets.shape
    _check(_load().qas_regroup_queries(ctypes.byref(batch), _ptr(q_indptr), N, _ptr(sets), H_kv,
                                       kq, int(page_size), int(window), int(group), _ptr(ids),
                                       _stream(stream)))


def qas_union_pages(batch, q_indptr, sets, group, page_size, union_pages, union_count,
                    membership, ids=None, stream=None):
    """sets: int32 [N][H_kv][kq]; outputs sized by qas_chunk_groups(); ids:
    optional execution order [H_kv][N] from qas_regroup_queries."""
    N, H_kv, kq = sets.shape
    _check(_load().qas_union_pages(ctypes.byref(batch), _ptr(q_indptr), N, _ptr(sets), H_kv, kq,
                               int(group), int(page_size), _ptr(ids), _ptr(union_pages),
                               _ptr(union_count), _ptr(membership), _stream(stream)))


def qas_chunk_attention(cache, batch, q_indptr, q_pos, q, sets, group, sm_scale, out, lse=None,
                        ids=None, stream=None):
    """q: bf16 [N][H_q][d]; sets: int32 [N][H_kv][kq]; out like q; ids:
    optional execution order [H_kv][N] from qas_regroup_queries."""
    N, H_q, _ = q.shape
    _check(_load().qas_chunk_attention(ctypes.byref(cache), ctypes.byref(batch), _ptr(q_indptr), N,
                                   _ptr(q_pos), _ptr(q), dtype_code(q), H_q, _ptr(sets),
                                   sets.shape[-1], int(group), _ptr(ids), float(sm_scale),
                                   _ptr(out), _ptr(lse), _stream(stream)))


def version():
    return _load().qas_version().decode()


__all__ = ["qas_append", "qas_append_fp8", "qas_rollback", "qas_score_pages", "qas_topk_pages", "qas_selection_capacity",
           "qas_select_pages", "qas_sparse_decode", "qas_decode_layer", "qas_decode_layer_mixed", "qas_decode_layer_noalloc",
           "qas_decode_positions",
           "qas_positions_workspace_bytes", "qas_exact_top_r", "qas_exact_top_r_workspace_bytes",
           "qas_workspace_bytes", "make_workspace", "qas_chunk_groups", "qas_regroup_queries", "qas_union_pages",
           "qas_chunk_attention", "make_cache", "make_batch",
           "qas_cache", "qas_batch", "QasError", "version", "lib", "LIB_PATH"]
