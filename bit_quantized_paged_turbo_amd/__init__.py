"""Python binding of libxq.so, the TurboQuant paged KV cache for MI355X.

Argument marshalling only: every step of the path runs in the HIP kernels behind the
C ABI (include/xq.h). Tensors are passed by device pointer; torch is used by callers for
device memory and streams. There is no CPU fallback: if libxq.so has not been built,
every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libxq.so")

KV_BF16, KV_TURBO8, KV_TURBO4, KV_TURBO3, KV_TURBO2, KV_FP8 = 0, 8, 4, 3, 2, 16
OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4

# Every symbol include/xq.h declares.
EXPORTS = ("xq_block_bytes", "xq_page_stride_bytes", "xq_pool_bytes", "xq_decode_num_splits",
           "xq_decode_workspace_bytes", "xq_prefill_workspace_bytes", "xq_status_string", "xq_last_error",
           "xq_quantize_append", "xq_paged_decode_attention", "xq_paged_prefill_attention",
           "xq_decode_plan", "xq_paged_decode_attention_planned", "xq_append_decode_attention",
           "xq_hbm_read_probe", "xq_paged_decode_attention_noalloc", "xq_decode_plan_entries",
           "xq_decode_plan_balanced", "xq_decode_workspace_bytes_balanced", "xq_decode_attention_balanced")


class XqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class CacheLayout(ctypes.Structure):
    """xq_cache_layout: geometry shared by the K and V pools."""
    _fields_ = [("kv_dtype", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int64)]

    def __init__(self, kv_dtype: int, num_kv_heads: int, page_size: int, num_pages: int,
                 head_dim: int = 128):
        super().__init__(kv_dtype, head_dim, num_kv_heads, page_size, num_pages)


_lib = None


def load() -> ctypes.CDLL:
    """Load libxq.so (built by bit_quantized_paged_turbo_amd.build); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m bit_quantized_paged_turbo_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    LP = ctypes.POINTER(CacheLayout)
    sig = {
        "xq_block_bytes": (I64, [LP]),
        "xq_page_stride_bytes": (I64, [LP]),
        "xq_pool_bytes": (I64, [LP]),
        "xq_decode_num_splits": (I32, [LP, I32, I32, I32, I32]),
        "xq_decode_workspace_bytes": (I64, [LP, I32, I32, I32, I32]),
        "xq_prefill_workspace_bytes": (I64, [LP, I32, I32, I32, I32]),
        "xq_status_string": (ctypes.c_char_p, [I32]),
        "xq_last_error": (ctypes.c_char_p, []),
        "xq_quantize_append": (I32, [LP, P, P, I32, P, P, P, I32, P, P, P]),
        "xq_paged_decode_attention": (I32, [LP, P, I32, I32, P, P, P, I32, P, I32, F32, I32,
                                            P, I64, P, P]),
        "xq_paged_prefill_attention": (I32, [LP, P, I32, I32, P, P, P, I32, I32, F32, I32,
                                             P, I64, P, P]),
        "xq_decode_plan": (I32, [LP, I32, I32, I32, I32, P, P]),
        "xq_decode_plan_entries": (I32, [LP, I32, I32, I32, I32]),
        "xq_append_decode_attention": (I32, [LP, P, P, P, I32, I32, P, P, P, I32, P, I32, F32, I32,
                                             P, I64, P, P, I32, P]),
        "xq_paged_decode_attention_planned": (I32, [LP, P, I32, I32, P, P, P, I32, P, I32, F32, I32,
                                                    P, I64, P, P, I32, P]),
        "xq_hbm_read_probe": (I32, [P, I64, I64, I32, I64, P, P, P]),
        "xq_paged_decode_attention_noalloc": (I32, [LP, P, I32, I32, P, P, P, I32, P, I32, F32, I32, P, P]),
        "xq_decode_plan_balanced": (I32, [LP, I32, I32, I32, P, P, P]),
        "xq_decode_workspace_bytes_balanced": (I64, [LP, I32, I32, I32]),
        "xq_decode_attention_balanced": (I32, [LP, P, I32, I32, P, P, P, I32, P, I32, F32, I32, P, P,
                                               P, P, P, P, I32, P, P, P, I64, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _entries(plan) -> int:
    """Entries of a device plan (a tensor) for the planned calls; 0 without one."""
    return 0 if plan is None else int(plan.numel())


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != OK:
        lib = load()
        raise XqError(status, lib.xq_last_error().decode() or lib.xq_status_string(status).decode())


def xq_block_bytes(layout: CacheLayout) -> int:
    return load().xq_block_bytes(ctypes.byref(layout))


def xq_page_stride_bytes(layout: CacheLayout) -> int:
    return load().xq_page_stride_bytes(ctypes.byref(layout))


def xq_pool_bytes(layout: CacheLayout) -> int:
    return load().xq_pool_bytes(ctypes.byref(layout))


def xq_decode_num_splits(layout, batch, num_q_heads, max_context_len, num_splits_hint=0) -> int:
    return load().xq_decode_num_splits(ctypes.byref(layout), batch, num_q_heads,
                                       max_context_len, num_splits_hint)


def xq_decode_workspace_bytes(layout, batch, num_q_heads, max_context_len, num_splits_hint=0) -> int:
    return load().xq_decode_workspace_bytes(ctypes.byref(layout), batch, num_q_heads,
                                            max_context_len, num_splits_hint)


def xq_prefill_workspace_bytes(layout, n_query, num_q_heads, start_pos, num_splits_hint=0) -> int:
    return load().xq_prefill_workspace_bytes(ctypes.byref(layout), n_query, num_q_heads,
                                             start_pos, num_splits_hint)


def xq_quantize_append(layout: CacheLayout, k_new, v_new, n_tokens: int, token_seq, token_pos,
                       block_tables, max_pages_per_seq: int, k_pool, v_pool, stream=None):
    """See xq_quantize_append in include/xq.h. Tensors are passed by data_ptr()."""
    _check(load().xq_quantize_append(ctypes.byref(layout), _ptr(k_new), _ptr(v_new), n_tokens,
                                     _ptr(token_seq), _ptr(token_pos), _ptr(block_tables),
                                     max_pages_per_seq, _ptr(k_pool), _ptr(v_pool),
                                     _stream(stream)))


def xq_paged_decode_attention(layout: CacheLayout, q, batch: int, num_q_heads: int, k_pool,
                              v_pool, block_tables, max_pages_per_seq: int, context_lens,
                              max_context_len: int, softmax_scale: float, num_splits_hint: int,
                              workspace, workspace_bytes: int, out, stream=None):
    """See xq_paged_decode_attention in include/xq.h. Tensors are passed by data_ptr()."""
    _check(load().xq_paged_decode_attention(
        ctypes.byref(layout), _ptr(q), batch, num_q_heads, _ptr(k_pool), _ptr(v_pool),
        _ptr(block_tables), max_pages_per_seq, _ptr(context_lens), max_context_len,
        float(softmax_scale), num_splits_hint, _ptr(workspace), int(workspace_bytes), _ptr(out),
        _stream(stream)))


def xq_paged_prefill_attention(layout: CacheLayout, q, n_query: int, num_q_heads: int, k_pool,
                               v_pool, block_table, max_pages: int, start_pos: int,
                               softmax_scale: float, num_splits_hint: int, workspace,
                               workspace_bytes: int, out, stream=None):
    """See xq_paged_prefill_attention in include/xq.h. Tensors are passed by data_ptr()."""
    _check(load().xq_paged_prefill_attention(
        ctypes.byref(layout), _ptr(q), n_query, num_q_heads, _ptr(k_pool), _ptr(v_pool),
        _ptr(block_table), max_pages, start_pos, float(softmax_scale), num_splits_hint,
        _ptr(workspace), int(workspace_bytes), _ptr(out), _stream(stream)))


def xq_decode_plan_entries(layout: CacheLayout, batch: int, num_q_heads: int, max_context_len: int,
                           num_splits_hint: int = 0) -> int:
    return load().xq_decode_plan_entries(ctypes.byref(layout), batch, num_q_heads, max_context_len,
                                         num_splits_hint)


def xq_decode_plan(layout: CacheLayout, batch: int, num_q_heads: int, max_context_len: int,
                   num_splits_hint: int, context_lens) -> "list[int]":
    """See xq_decode_plan in include/xq.h. context_lens: host sequence of ints; returns the plan
    (xq_decode_plan_entries entries)."""
    n = xq_decode_plan_entries(layout, batch, num_q_heads, max_context_len, num_splits_hint)
    if n < 0:
        raise XqError(EINVAL, "invalid layout, batch, head count, context length or split hint")
    lens = (ctypes.c_int32 * max(1, batch))(*[int(x) for x in context_lens])
    order = (ctypes.c_int32 * max(1, n))()
    _check(load().xq_decode_plan(ctypes.byref(layout), batch, num_q_heads, max_context_len,
                                 num_splits_hint, ctypes.cast(lens, ctypes.c_void_p),
                                 ctypes.cast(order, ctypes.c_void_p)))
    return list(order)[:n]


def xq_paged_decode_attention_planned(layout: CacheLayout, q, batch: int, num_q_heads: int, k_pool,
                                      v_pool, block_tables, max_pages_per_seq: int, context_lens,
                                      max_context_len: int, softmax_scale: float, num_splits_hint: int,
                                      workspace, workspace_bytes: int, out, seq_order, stream=None):
    """See xq_paged_decode_attention_planned in include/xq.h. Tensors are passed by data_ptr()."""
    _check(load().xq_paged_decode_attention_planned(
        ctypes.byref(layout), _ptr(q), batch, num_q_heads, _ptr(k_pool), _ptr(v_pool),
        _ptr(block_tables), max_pages_per_seq, _ptr(context_lens), max_context_len,
        float(softmax_scale), num_splits_hint, _ptr(workspace), int(workspace_bytes), _ptr(out),
        _ptr(seq_order), _entries(seq_order), _stream(stream)))


def xq_append_decode_attention(layout: CacheLayout, k_new, v_new, q, batch: int, num_q_heads: int,
                               k_pool, v_pool, block_tables, max_pages_per_seq: int, context_lens,
                               max_context_len: int, softmax_scale: float, num_splits_hint: int,
                               workspace, workspace_bytes: int, out, seq_order=None, stream=None):
    """See xq_append_decode_attention in include/xq.h. Tensors are passed by data_ptr()."""
    _check(load().xq_append_decode_attention(
        ctypes.byref(layout), _ptr(k_new), _ptr(v_new), _ptr(q), batch, num_q_heads, _ptr(k_pool),
        _ptr(v_pool), _ptr(block_tables), max_pages_per_seq, _ptr(context_lens), max_context_len,
        float(softmax_scale), num_splits_hint, _ptr(workspace), int(workspace_bytes), _ptr(out),
        _ptr(seq_order), _entries(seq_order), _stream(stream)))


def xq_decode_plan_balanced(layout: CacheLayout, batch: int, num_q_heads: int, max_context_len: int,
                            context_lens):
    """See xq_decode_plan_balanced in include/xq.h. context_lens: host sequence of ints. Returns
    (nsplits, seq_tps list [batch], units list of 2 * batch * nsplits * num_kv_heads ints)."""
    lib = load()
    lens = (ctypes.c_int32 * max(1, batch))(*[int(x) for x in context_lens])
    tps = (ctypes.c_int32 * max(1, batch))()
    ns = lib.xq_decode_plan_balanced(ctypes.byref(layout), batch, num_q_heads, max_context_len,
                                     ctypes.cast(lens, ctypes.c_void_p), ctypes.cast(tps, ctypes.c_void_p), None)
    if ns < 1:
        raise XqError(EINVAL, lib.xq_last_error().decode())
    n = 2 * batch * ns * layout.num_kv_heads
    units = (ctypes.c_int32 * max(1, n))()
    ns2 = lib.xq_decode_plan_balanced(ctypes.byref(layout), batch, num_q_heads, max_context_len,
                                      ctypes.cast(lens, ctypes.c_void_p), ctypes.cast(tps, ctypes.c_void_p),
                                      ctypes.cast(units, ctypes.c_void_p))
    assert ns2 == ns
    return ns, list(tps)[:batch], list(units)[:n]


def xq_decode_workspace_bytes_balanced(layout: CacheLayout, batch: int, num_q_heads: int, nsplits: int) -> int:
    return load().xq_decode_workspace_bytes_balanced(ctypes.byref(layout), batch, num_q_heads, nsplits)


def xq_decode_attention_balanced(layout: CacheLayout, q, batch: int, num_q_heads: int, k_pool, v_pool,
                                 block_tables, max_pages_per_seq: int, context_lens, max_context_len: int,
                                 softmax_scale: float, nsplits: int, units, seq_tps, k_new, v_new,
                                 workspace, workspace_bytes: int, out, stream=None, chunk_k=None, chunk_v=None,
                                 chunk_tokens: int = 0, chunk_seq=None, chunk_pos=None):
    """See xq_decode_attention_balanced in include/xq.h. Tensors are passed by data_ptr()."""
    _check(load().xq_decode_attention_balanced(
        ctypes.byref(layout), _ptr(q), batch, num_q_heads, _ptr(k_pool), _ptr(v_pool), _ptr(block_tables),
        max_pages_per_seq, _ptr(context_lens), max_context_len, float(softmax_scale), nsplits, _ptr(units),
        _ptr(seq_tps), _ptr(k_new), _ptr(v_new), _ptr(chunk_k), _ptr(chunk_v), int(chunk_tokens),
        _ptr(chunk_seq), _ptr(chunk_pos), _ptr(workspace), int(workspace_bytes), _ptr(out), _stream(stream)))


def xq_hbm_read_probe(buf, buf_bytes: int, n_blocks: int, block_bytes: int, block_stride: int,
                      block_order, sink, stream=None):
    """See xq_hbm_read_probe in include/xq.h (a streaming-read reference for the roofline)."""
    _check(load().xq_hbm_read_probe(_ptr(buf), int(buf_bytes), int(n_blocks), int(block_bytes),
                                    int(block_stride), _ptr(block_order), _ptr(sink), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20


def xq_paged_decode_attention_noalloc(layout: CacheLayout, q, batch: int, num_q_heads: int, k_pool,
                                      v_pool, block_tables, max_pages_per_seq: int, context_lens,
                                      max_context_len: int, softmax_scale: float, num_splits_hint: int,
                                      out, stream=None):
    """See xq_paged_decode_attention_noalloc in include/xq.h (no workspace: the library's scratch)."""
    _check(load().xq_paged_decode_attention_noalloc(
        ctypes.byref(layout), _ptr(q), batch, num_q_heads, _ptr(k_pool), _ptr(v_pool),
        _ptr(block_tables), max_pages_per_seq, _ptr(context_lens), max_context_len,
        float(softmax_scale), num_splits_hint, _ptr(out), _stream(stream)))
