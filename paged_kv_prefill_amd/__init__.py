"""Chunked prefill attention over a paged KV cache on MI355X (gfx950).

A thin ctypes binding over ``libpaged_prefill.so`` (C ABI in
``include/paged_prefill.h``).  It only marshals arguments: torch tensors give
device pointers, shapes and the current HIP stream; every step of the
computation runs in the library's HIP kernels.  There is no CPU fallback:
if the library is missing or fails to load, importing the entry points
raises.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpaged_prefill.so")

PPA_F16 = 0
PPA_BF16 = 1


class PagedPrefillError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {strerror(code)} (code {code})")


class Plan(ctypes.Structure):
    _fields_ = [
        ("n_splits", ctypes.c_int32),
        ("split_tokens", ctypes.c_int32),
        ("m_tile", ctypes.c_int32),
        ("kv_tile", ctypes.c_int32),
        ("tiles_m", ctypes.c_int32),
        ("grid", ctypes.c_int32),
        ("merge_grid", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_ if name != "reserved"}


_lib = None

_VP = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64

_SIGNATURES = {
    "paged_prefill_attention": (_I32, [_VP, _VP, _VP, _VP, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _I32, _VP]),
    "contiguous_prefill_attention": (_I32, [_VP, _VP, _VP, _I64, _I32, _I32, _I32, _I32, _I32, _VP, _I32, _VP]),
    "paged_prefill_attention_pieces": (_I32, [_VP, _VP, _VP, _VP, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _I32, _VP]),
    "paged_prefill_attention_pieces_noalloc": (_I32, [_VP, _VP, _VP, _VP, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                                      _VP, _I32, _VP]),
    "contiguous_prefill_attention_pieces": (_I32, [_VP, _VP, _VP, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _VP, _I32, _VP]),
    "paged_prefill_plan": (_I32, [_I64, _I32, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(Plan)]),
    "paged_prefill_split_rule": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "paged_prefill_piece_rows": (_I32, [_I64, _I32, _I64]),
    "paged_prefill_check_block_table": (_I32, [_VP, _I64, _I64]),
    "paged_prefill_release_workspaces": (_I32, []),
    "paged_prefill_workspace_bytes": (_I64, [_VP]),
    "paged_prefill_strerror": (ctypes.c_char_p, [_I32]),
    "paged_prefill_version": (_I32, []),
    "paged_kv_append": (_I32, [_VP, _VP, _VP, _VP, _VP, _I64, _I32, _I32, _I32, _I32, _I32, _VP]),
    "paged_prefill_attention_varlen": (_I32, [_VP, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32, _I32, _I64, _I32,
                                              _I32, _I32, _I32, _I32, _VP, _I32, _VP]),
    "paged_prefill_plan_varlen": (_I32, [_I32, _I32, _I32, _I64, _I32, _I32, _I32, _I32, _I32, ctypes.POINTER(Plan)]),
    "paged_prefill_attention_q8": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                          _VP, _I32, _VP]),
    "paged_kv_append_q8": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _I32, _I32, _I32, _I32, _I32, _VP]),
    "paged_prefill_attention_varlen_q8": (_I32, [_VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _VP, _I32, _I32, _I32,
                                                 _I64, _I32, _I32, _I32, _I32, _I32, _VP, _I32, _VP]),
}


def lib():
    """The loaded library (raises if it is not built).

    torch is imported first: its wheel carries its own HIP runtime
    (torch/lib/libamdhip64.so, soname libamdhip64.so.7).  Loaded after the
    library, whose dependency resolves to the system runtime, torch's copy
    would be a second HIP runtime in the process, and the streams and device
    memory torch hands the library would belong to the other one (launches on
    them fail).  Loaded before it, the library's dependency resolves to
    torch's runtime by soname: one runtime."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def strerror(code):
    return lib().paged_prefill_strerror(int(code)).decode()


def _check(code, where):
    if code != 0:
        raise PagedPrefillError(code, where)


def _dtype_code(t):
    import torch
    if t.dtype == torch.float16:
        return PPA_F16
    if t.dtype == torch.bfloat16:
        return PPA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need_cuda(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _check_kinds(q, kv, out, int32=(), int64=()):
    """Element types and output shape the C ABI cannot see: K/V and out in
    q's type, out shaped like q, index arrays int32 / int64."""
    import torch
    _dtype_code(q)
    for t in kv:
        if t.dtype != q.dtype:
            raise TypeError(f"K/V dtype {t.dtype} differs from q's {q.dtype}")
    if out is not None and (out.dtype != q.dtype or tuple(out.shape) != tuple(q.shape)):
        raise ValueError("out must have q's dtype and shape")
    for t in int32:
        if t.dtype != torch.int32:
            raise TypeError("block tables and row offsets are int32")
    for t in int64:
        if t.dtype != torch.int64:
            raise TypeError("history lengths are int64")


def _check_table(block_table, history_len, rows, page_size):
    """The block table must name a page for every position 0 .. H+R-1: the
    kernels read ceil((H + R) / page_size) entries and cannot see its length."""
    need = -(-(int(history_len) + int(rows)) // int(page_size))
    if int(history_len) < 0 or int(rows) < 0:
        return
    if block_table.numel() < need:
        raise ValueError(f"block_table has {block_table.numel()} entries; history_len + rows = "
                         f"{int(history_len) + int(rows)} tokens need {need} pages of {int(page_size)}")


def paged_prefill_attention(q, k_pages, v_pages, block_table, history_len, n_splits=0, out=None,
                            piece_rows=0, stream=None):
    """out[R][Hq][d] = causal attention of q[R][Hq][d] (rows at positions
    history_len .. history_len+R-1) over the paged cache k_pages/v_pages
    [pool][page_size][Hkv][d] addressed by block_table (int32).  piece_rows
    > 0 runs the chunk in pieces of that many rows."""
    _check_kinds(q, (k_pages, v_pages), out, int32=(block_table,))
    rows, n_q_heads, head_dim = q.shape
    _, page_size, n_kv_heads, kd = k_pages.shape
    _check_table(block_table, history_len, rows, page_size)
    _need_cuda(q, k_pages, v_pages, block_table, out)
    if kd != head_dim or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("k_pages/v_pages shape mismatch")
    if out is None:
        out = q.new_empty(q.shape)
    common = (int(history_len), int(rows))
    tail = (int(n_q_heads), int(n_kv_heads), int(head_dim), int(page_size), int(n_splits), _ptr(out),
            _dtype_code(q), _stream_handle(stream, q.device))
    if piece_rows:
        rc = lib().paged_prefill_attention_pieces(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                                  *common, int(piece_rows), *tail)
        _check(rc, "paged_prefill_attention_pieces")
    else:
        rc = lib().paged_prefill_attention(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                                           *common, *tail)
        _check(rc, "paged_prefill_attention")
    return out


def contiguous_prefill_attention(q, k, v, history_len, n_splits=0, out=None, piece_rows=0, stream=None):
    """The same over contiguous k/v [>= H+R][Hkv][d]."""
    _check_kinds(q, (k, v), out)
    _need_cuda(q, k, v, out)
    rows, n_q_heads, head_dim = q.shape
    n_kv_heads = k.shape[1]
    if k.dim() != 3 or k.shape[2] != head_dim or tuple(v.shape) != tuple(k.shape) \
            or k.shape[0] < int(history_len) + rows:
        raise ValueError("k and v must be [>= history_len + rows][Hkv][d] with q's d")
    if out is None:
        out = q.new_empty(q.shape)
    args = (int(history_len), int(rows))
    tail = (int(n_q_heads), int(n_kv_heads), int(head_dim), int(n_splits), _ptr(out), _dtype_code(q),
            _stream_handle(stream, q.device))
    if piece_rows:
        rc = lib().contiguous_prefill_attention_pieces(_ptr(q), _ptr(k), _ptr(v), *args, int(piece_rows), *tail)
        _check(rc, "contiguous_prefill_attention_pieces")
    else:
        rc = lib().contiguous_prefill_attention(_ptr(q), _ptr(k), _ptr(v), *args, *tail)
        _check(rc, "contiguous_prefill_attention")
    return out


def paged_prefill_attention_varlen(q, k_pages, v_pages, block_tables, cu_rows, history_lens, max_rows,
                                   max_context, n_splits=0, out=None, stream=None):
    """Several sequences in one launch.  q, out [total_rows][Hq][d] hold the
    sequences' rows back to back; sequence s owns rows cu_rows[s] ..
    cu_rows[s+1]-1 (cu_rows: int32 [n+1] on the GPU), has history
    history_lens[s] (int64 [n] on the GPU) and block table block_tables[s]
    (int32 [n][stride] on the GPU) into the shared k_pages/v_pages pool.
    max_rows and max_context (host ints) bound every sequence's rows and
    history + rows."""
    import torch
    _check_kinds(q, (k_pages, v_pages), out, int32=(block_tables, cu_rows), int64=(history_lens,))
    _need_cuda(q, k_pages, v_pages, block_tables, cu_rows, history_lens, out)
    if block_tables.dim() != 2 or block_tables.dtype != torch.int32 or cu_rows.dtype != torch.int32 \
            or history_lens.dtype != torch.int64:
        raise ValueError("block_tables int32 [n][stride], cu_rows int32 [n+1], history_lens int64 [n]")
    n_seqs = history_lens.shape[0]
    if block_tables.shape[0] != n_seqs or cu_rows.shape[0] != n_seqs + 1:
        raise ValueError("block_tables, cu_rows and history_lens disagree on the sequence count")
    total_rows, n_q_heads, head_dim = q.shape
    _, page_size, n_kv_heads, kd = k_pages.shape
    if kd != head_dim or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("k_pages/v_pages shape mismatch")
    if out is None:
        out = q.new_empty(q.shape)
    rc = lib().paged_prefill_attention_varlen(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_tables), int(block_tables.shape[1]), _ptr(cu_rows),
        _ptr(history_lens), int(n_seqs), int(total_rows), int(max_rows), int(max_context), int(n_q_heads),
        int(n_kv_heads), int(head_dim), int(page_size), int(n_splits), _ptr(out), _dtype_code(q),
        _stream_handle(stream, q.device))
    _check(rc, "paged_prefill_attention_varlen")
    return out


def paged_prefill_plan_varlen(n_seqs, total_rows, max_rows, max_context, n_q_heads, n_kv_heads, head_dim,
                              page_size=16, n_splits=0):
    plan = Plan()
    rc = lib().paged_prefill_plan_varlen(int(n_seqs), int(total_rows), int(max_rows), int(max_context),
                                         int(n_q_heads), int(n_kv_heads), int(head_dim), int(page_size),
                                         int(n_splits), ctypes.byref(plan))
    _check(rc, "paged_prefill_plan_varlen")
    return plan.as_dict()


def paged_prefill_attention_q8(q, k_quant, k_scale, v_quant, v_scale, block_table, history_len, n_splits=0,
                               out=None, piece_rows=0, stream=None):
    """Attention over 8-bit pages: k_quant/v_quant int8 [pool][page_size][Hkv][d],
    k_scale/v_scale fp16 [pool][page_size][Hkv][d/32] (value = scale * quant per
    block of 32 along d).  q and out fp16 or bf16 [R][Hq][d]."""
    import torch
    _check_kinds(q, (), out, int32=(block_table,))
    rows, n_q_heads, head_dim = q.shape
    _, page_size, n_kv_heads, kd = k_quant.shape
    _check_table(block_table, history_len, rows, page_size)
    _need_cuda(q, k_quant, k_scale, v_quant, v_scale, block_table, out)
    if kd != head_dim or tuple(v_quant.shape) != tuple(k_quant.shape) or k_quant.dtype != torch.int8 \
            or v_quant.dtype != torch.int8 or tuple(k_scale.shape) != (k_quant.shape[0], page_size, n_kv_heads, kd // 32) \
            or tuple(v_scale.shape) != tuple(k_scale.shape) or k_scale.element_size() != 2 or v_scale.element_size() != 2:
        raise ValueError("int8 quants [pool][ps][Hkv][d] and 16-bit scales [pool][ps][Hkv][d/32] expected")
    if out is None:
        out = q.new_empty(q.shape)
    rc = lib().paged_prefill_attention_q8(
        _ptr(q), _ptr(k_quant), _ptr(k_scale), _ptr(v_quant), _ptr(v_scale), _ptr(block_table), int(history_len),
        int(rows), int(piece_rows), int(n_q_heads), int(n_kv_heads), int(head_dim), int(page_size), int(n_splits),
        _ptr(out), _dtype_code(q), _stream_handle(stream, q.device))
    _check(rc, "paged_prefill_attention_q8")
    return out


def paged_prefill_attention_varlen_q8(q, k_quant, k_scale, v_quant, v_scale, block_tables, cu_rows, history_lens,
                                      max_rows, max_context, n_splits=0, out=None, stream=None):
    """paged_prefill_attention_varlen over 8-bit pages (the quants and scales
    of paged_prefill_attention_q8)."""
    import torch
    _check_kinds(q, (), out, int32=(block_tables, cu_rows), int64=(history_lens,))
    _need_cuda(q, k_quant, k_scale, v_quant, v_scale, block_tables, cu_rows, history_lens, out)
    if block_tables.dim() != 2 or block_tables.dtype != torch.int32 or cu_rows.dtype != torch.int32 \
            or history_lens.dtype != torch.int64:
        raise ValueError("block_tables int32 [n][stride], cu_rows int32 [n+1], history_lens int64 [n]")
    n_seqs = history_lens.shape[0]
    if block_tables.shape[0] != n_seqs or cu_rows.shape[0] != n_seqs + 1:
        raise ValueError("block_tables, cu_rows and history_lens disagree on the sequence count")
    total_rows, n_q_heads, head_dim = q.shape
    _, page_size, n_kv_heads, kd = k_quant.shape
    if kd != head_dim or tuple(v_quant.shape) != tuple(k_quant.shape) or k_quant.dtype != torch.int8 \
            or v_quant.dtype != torch.int8 or tuple(k_scale.shape) != (k_quant.shape[0], page_size, n_kv_heads, kd // 32) \
            or tuple(v_scale.shape) != tuple(k_scale.shape) or k_scale.element_size() != 2 or v_scale.element_size() != 2:
        raise ValueError("int8 quants [pool][ps][Hkv][d] and 16-bit scales [pool][ps][Hkv][d/32] expected")
    if out is None:
        out = q.new_empty(q.shape)
    rc = lib().paged_prefill_attention_varlen_q8(
        _ptr(q), _ptr(k_quant), _ptr(k_scale), _ptr(v_quant), _ptr(v_scale), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(cu_rows), _ptr(history_lens), int(n_seqs), int(total_rows), int(max_rows),
        int(max_context), int(n_q_heads), int(n_kv_heads), int(head_dim), int(page_size), int(n_splits), _ptr(out),
        _dtype_code(q), _stream_handle(stream, q.device))
    _check(rc, "paged_prefill_attention_varlen_q8")
    return out


def paged_kv_append_q8(k_new, v_new, k_quant, k_scale, v_quant, v_scale, block_table, history_len, stream=None):
    """Quantize k_new/v_new [R][Hkv][d] (fp16 or bf16) into their slots of the
    8-bit pools, in place."""
    import torch
    _check_kinds(k_new, (v_new,), None, int32=(block_table,))
    rows, n_kv_heads, head_dim = k_new.shape
    _, page_size, pkv, pd = k_quant.shape
    _check_table(block_table, history_len, rows, page_size)
    _need_cuda(k_new, v_new, k_quant, k_scale, v_quant, v_scale, block_table)
    if (pkv, pd) != (n_kv_heads, head_dim) or tuple(v_new.shape) != tuple(k_new.shape) \
            or k_quant.dtype != torch.int8 or v_quant.dtype != torch.int8 or tuple(v_quant.shape) != tuple(k_quant.shape) \
            or tuple(k_scale.shape) != (k_quant.shape[0], page_size, n_kv_heads, head_dim // 32) \
            or tuple(v_scale.shape) != tuple(k_scale.shape):
        raise ValueError("k_new/v_new/quant/scale shapes do not match")
    rc = lib().paged_kv_append_q8(_ptr(k_new), _ptr(v_new), _ptr(k_quant), _ptr(k_scale), _ptr(v_quant),
                                  _ptr(v_scale), _ptr(block_table), int(history_len), int(rows), int(n_kv_heads),
                                  int(head_dim), int(page_size), _dtype_code(k_new),
                                  _stream_handle(stream, k_new.device))
    _check(rc, "paged_kv_append_q8")
    return k_quant, k_scale, v_quant, v_scale


def paged_kv_append(k_new, v_new, k_pages, v_pages, block_table, history_len, stream=None):
    """Write k_new/v_new [R][Hkv][d] (tokens at positions history_len ..
    history_len+R-1) into their slots of k_pages/v_pages
    [pool][page_size][Hkv][d] through block_table (int32), in place."""
    _check_kinds(k_new, (v_new, k_pages, v_pages), None, int32=(block_table,))
    rows, n_kv_heads, head_dim = k_new.shape
    _, page_size, pkv, pd = k_pages.shape
    _check_table(block_table, history_len, rows, page_size)
    _need_cuda(k_new, v_new, k_pages, v_pages, block_table)
    if (pkv, pd) != (n_kv_heads, head_dim) or tuple(v_pages.shape) != tuple(k_pages.shape) \
            or tuple(v_new.shape) != tuple(k_new.shape) or k_new.dtype != k_pages.dtype:
        raise ValueError("k_new/v_new/k_pages/v_pages shapes or dtypes do not match")
    rc = lib().paged_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_pages), _ptr(v_pages), _ptr(block_table),
                               int(history_len), int(rows), int(n_kv_heads), int(head_dim), int(page_size),
                               _dtype_code(k_new), _stream_handle(stream, k_new.device))
    _check(rc, "paged_kv_append")
    return k_pages, v_pages


def paged_prefill_plan(history_len, chunk_rows, n_q_heads, n_kv_heads, head_dim, page_size=16, n_splits=0):
    plan = Plan()
    rc = lib().paged_prefill_plan(int(history_len), int(chunk_rows), int(n_q_heads), int(n_kv_heads),
                                  int(head_dim), int(page_size), int(n_splits), ctypes.byref(plan))
    _check(rc, "paged_prefill_plan")
    return plan.as_dict()


def paged_prefill_split_rule(gpu_cores, kv_heads, tiles, per_core=32, floor_tg=32, slot_cap=256, max_splits=32):
    rc = lib().paged_prefill_split_rule(gpu_cores, kv_heads, tiles, per_core, floor_tg, slot_cap, max_splits)
    if rc < 0:
        raise PagedPrefillError(rc, "paged_prefill_split_rule")
    return rc


def paged_prefill_piece_rows(history_len, chunk_rows=2048, budget=0):
    return lib().paged_prefill_piece_rows(int(history_len), int(chunk_rows), int(budget))


def paged_prefill_check_block_table(block_table_host, n_pool_pages):
    import numpy as np
    arr = np.ascontiguousarray(block_table_host, dtype=np.int32)
    rc = lib().paged_prefill_check_block_table(arr.ctypes.data_as(ctypes.c_void_p), int(arr.size),
                                               int(n_pool_pages))
    return rc


def paged_prefill_release_workspaces():
    _check(lib().paged_prefill_release_workspaces(), "paged_prefill_release_workspaces")


def paged_prefill_workspace_bytes(stream=None, device=None):
    """Bytes of the split workspace the library holds for `stream` (the
    current stream by default)."""
    import torch
    dev = device if device is not None else torch.cuda.current_device()
    rc = lib().paged_prefill_workspace_bytes(_stream_handle(stream, dev))
    if rc < 0:
        raise PagedPrefillError(rc, "paged_prefill_workspace_bytes")
    return int(rc)


def paged_prefill_attention_noalloc(q, k_pages, v_pages, block_table, history_len, n_splits=0, out=None,
                                    piece_rows=0, stream=None):
    """paged_prefill_attention (pieces form) with the split workspace in the
    library's fixed device array: no device allocation by the library (out
    must be given to avoid torch's).  Overlapping calls on one GPU race on
    that array."""
    _check_kinds(q, (k_pages, v_pages), out, int32=(block_table,))
    rows, n_q_heads, head_dim = q.shape
    _, page_size, n_kv_heads, kd = k_pages.shape
    _check_table(block_table, history_len, rows, page_size)
    _need_cuda(q, k_pages, v_pages, block_table, out)
    if kd != head_dim or tuple(v_pages.shape) != tuple(k_pages.shape):
        raise ValueError("k_pages/v_pages shape mismatch")
    if out is None:
        out = q.new_empty(q.shape)
    rc = lib().paged_prefill_attention_pieces_noalloc(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), int(history_len), int(rows), int(piece_rows),
        int(n_q_heads), int(n_kv_heads), int(head_dim), int(page_size), int(n_splits), _ptr(out), _dtype_code(q),
        _stream_handle(stream, q.device))
    _check(rc, "paged_prefill_attention_pieces_noalloc")
    return out
