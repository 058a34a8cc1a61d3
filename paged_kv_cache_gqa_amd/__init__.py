"""Python binding of libpagedattn.so (include/pagedattn.h): argument
marshalling only.  Every step of the attention path runs in the HIP kernels;
torch tensors are used for device memory and streams.

The library must have been built (``python paged_kv_cache_gqa_amd/build.py``);
importing this module without it raises ImportError -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

PA_OK, PA_ERR_NULL_ARG, PA_ERR_BAD_SHAPE, PA_ERR_UNSUPPORTED = 0, 1, 2, 3
PA_ERR_WORKSPACE_TOO_SMALL, PA_ERR_HIP = 4, 5
PA_KV_BF16, PA_KV_FP8_E4M3, PA_KV_MXFP4 = 0, 1, 2
TIMING_APPEND, TIMING_PREFILL, TIMING_DECODE, TIMING_MERGE, TIMING_STEP = 0, 1, 2, 3, 4
TIMING_KINDS = 5

# Every symbol the header declares.
EXPORTS = ("kv_append", "paged_attn_forward", "pa_workspace_size", "pa_last_error",
           "pa_debug_gather", "pa_timing_enable", "pa_timing_read", "pa_debug_plan",
           "pa_debug_plan_groups", "pa_peak_mfma", "pa_peak_read", "pa_device_shape",
           "pa_debug_xcc_ids", "paged_attn_forward_noalloc", "paged_attn_forward_cascade",
           "paged_attn_step", "pa_debug_step_flags", "pa_debug_overlap_cus")
NOALLOC_SCRATCH_BYTES = 128 << 20  # PA_NOALLOC_SCRATCH_BYTES


class pa_kv_cache(C.Structure):
    _fields_ = [("k_cache", C.c_void_p), ("v_cache", C.c_void_p),
                ("k_scale", C.c_void_p), ("v_scale", C.c_void_p),
                ("num_blocks", C.c_int32), ("num_kv_heads", C.c_int32),
                ("block_size", C.c_int32), ("head_dim", C.c_int32),
                ("dtype", C.c_int)]


class PagedAttnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"pagedattn status {status}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with python paged_kv_cache_gqa_amd/build.py")
    L = C.CDLL(LIB_PATH)
    P, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
    pc = C.POINTER(pa_kv_cache)
    L.kv_append.argtypes = [pc, P, P, P, i32, P]
    L.paged_attn_forward.argtypes = [P, pc, P, i32, P, P, i32, i32, C.c_float, P, P, P, sz, P]
    L.pa_workspace_size.argtypes = [P, P, i32, i32, pc]
    L.pa_workspace_size.restype = sz
    L.pa_last_error.argtypes = []
    L.pa_last_error.restype = C.c_char_p
    L.pa_debug_gather.argtypes = [pc, P, i32, P, P, P]
    L.pa_timing_enable.argtypes = [C.c_int]
    L.pa_timing_read.argtypes = [C.c_int, C.POINTER(C.c_double), C.POINTER(i64)]
    L.pa_debug_plan.argtypes = [P, P, i32, i32, pc, P, i32, P]
    L.pa_debug_plan_groups.argtypes = [P, P, i32, i32, pc, P, i32, P]
    L.pa_peak_mfma.argtypes = [P, i32, P]
    L.pa_peak_read.argtypes = [P, sz, P, P]
    L.pa_device_shape.argtypes = [C.POINTER(i32), C.POINTER(i32)]
    L.pa_debug_xcc_ids.argtypes = [P, i32, P]
    L.paged_attn_forward_noalloc.argtypes = [P, pc, P, i32, P, P, i32, i32, C.c_float, P, P, P]
    L.paged_attn_forward_cascade.argtypes = [P, pc, P, i32, P, P, i32, i32, C.c_float, P, P, P, P, i32, P,
                                             C.POINTER(sz), P]
    L.paged_attn_step.argtypes = [pc, P, P, P, P, P, i32, P, P, i32, i32, C.c_float, P, P, P, C.POINTER(sz), P]
    L.pa_debug_step_flags.argtypes = [P, pc, P, P, i32, i32, C.POINTER(C.c_uint32), P]
    L.pa_debug_overlap_cus.argtypes = [i32]
    for f in ("kv_append", "paged_attn_forward", "paged_attn_forward_noalloc", "paged_attn_forward_cascade",
              "paged_attn_step", "pa_debug_step_flags", "pa_debug_gather", "pa_timing_enable",
              "pa_timing_read", "pa_debug_plan", "pa_debug_plan_groups", "pa_peak_mfma",
              "pa_peak_read", "pa_device_shape", "pa_debug_xcc_ids", "pa_debug_overlap_cus"):
        getattr(L, f).restype = C.c_int
    return L


lib = _load()


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _check(status):
    if status != PA_OK:
        raise PagedAttnError(status, lib.pa_last_error().decode())


# ---------------------------------------------------------------------------
# Argument validation.  The library trusts device *contents* (block ids,
# slots) and sees only raw pointers, so a tensor of the wrong dtype, device,
# layout or shape would be reinterpreted silently and could make the GPU read
# out of bounds.  Every tensor argument is checked here before the call;
# shapes and dtypes first, the device last (so the checks can be exercised
# without a GPU).  These are checks only: no value is computed or converted.

def _bad(msg):
    raise PagedAttnError(PA_ERR_BAD_SHAPE, msg)


def _tensor(t, name, dtypes, shape=None):
    import torch
    if not isinstance(t, torch.Tensor):
        _bad(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        _bad(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(a) != int(w)
                                        for a, w in zip(t.shape, shape)):
            want = "[" + ", ".join("*" if w is None else str(w) for w in shape) + "]"
            _bad(f"{name} has shape {list(t.shape)}, expected {want}")
    if not t.is_contiguous():
        _bad(f"{name} must be contiguous")
    return (t, name)


def _on_device(checked, device=None):
    """Second pass over the (tensor, name) pairs _tensor accepted: each must
    live on the GPU (the cache's device when that is known)."""
    for t, name in checked:
        if not t.is_cuda:
            _bad(f"{name} must be a GPU tensor (got device {t.device})")
        if device is not None and t.device != device:
            _bad(f"{name} is on {t.device}, the cache on {device}")


def _bf16():
    import torch
    return (torch.bfloat16,)


def _code_dtypes():
    import torch
    return (torch.uint8, torch.float8_e4m3fn)


def make_cache(k_cache, v_cache, k_scale=None, v_scale=None) -> pa_kv_cache:
    """Describe caches [num_blocks, num_kv_heads, block_size, head_dim]: bf16;
    E4M3 codes (uint8 / float8_e4m3fn) with fp32 [num_blocks, num_kv_heads]
    scales; or MXFP4, codes uint8 [num_blocks, num_kv_heads, block_size,
    head_dim / 2] with E8M0 scale bytes (uint8 / float8_e8m0fnu)
    [num_blocks, num_kv_heads, head_dim / 32, block_size].  The scales' dtype
    tells E4M3 from MXFP4.  The tensors must outlive every call that uses the
    returned descriptor."""
    import torch
    if not isinstance(k_cache, torch.Tensor) or k_cache.dim() != 4:
        _bad("k_cache must be a 4-D tensor [num_blocks, num_kv_heads, block_size, head_dim]")
    nb, hkv, bs, last = (int(x) for x in k_cache.shape)
    coded = k_cache.dtype in _code_dtypes()
    e8m0 = (torch.uint8,) + ((torch.float8_e8m0fnu,) if hasattr(torch, "float8_e8m0fnu") else ())
    fp4 = coded and isinstance(k_scale, torch.Tensor) and k_scale.dtype in e8m0
    d = 2 * last if fp4 else last
    dtypes = _code_dtypes() if coded else _bf16()
    ok = [_tensor(k_cache, "k_cache", dtypes),
          _tensor(v_cache, "v_cache", (k_cache.dtype,), (nb, hkv, bs, last))]
    if coded:
        if k_scale is None or v_scale is None:
            raise PagedAttnError(PA_ERR_NULL_ARG, "an E4M3 or MXFP4 cache needs k_scale and v_scale")
        if fp4:
            if d % 32:
                _bad(f"MXFP4 head_dim {d} is not a multiple of 32")
            ok += [_tensor(k_scale, "k_scale", e8m0, (nb, hkv, d // 32, bs)),
                   _tensor(v_scale, "v_scale", (k_scale.dtype,), (nb, hkv, d // 32, bs))]
        else:
            ok += [_tensor(k_scale, "k_scale", (torch.float32,), (nb, hkv)),
                   _tensor(v_scale, "v_scale", (torch.float32,), (nb, hkv))]
    elif k_scale is not None or v_scale is not None:
        _bad("a bf16 cache takes no scales")
    _on_device(ok, k_cache.device)
    c = pa_kv_cache(k_cache.data_ptr(), v_cache.data_ptr(),
                    None if k_scale is None else k_scale.data_ptr(),
                    None if v_scale is None else v_scale.data_ptr(),
                    nb, hkv, bs, d, PA_KV_MXFP4 if fp4 else PA_KV_FP8_E4M3 if coded else PA_KV_BF16)
    c.device = k_cache.device
    return c


def _host_i32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def kv_append(cache: pa_kv_cache, k_new, v_new, slot_mapping, stream=None):
    """Scatter new K/V rows [T, Hkv, d] (bf16) into the slots slot_mapping [T] (int64)."""
    import torch
    dev = getattr(cache, "device", None)
    ok = [_tensor(slot_mapping, "slot_mapping", (torch.int64,), (None,))]
    T = int(slot_mapping.shape[0])
    shape = (T, cache.num_kv_heads, cache.head_dim)
    ok += [_tensor(k_new, "k_new", _bf16(), shape), _tensor(v_new, "v_new", _bf16(), shape)]
    _on_device(ok, dev)
    _check(lib.kv_append(C.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), T,
                         _stream_ptr(stream)))


def pa_workspace_size(hist_lens, incr_lens, num_q_heads, cache: pa_kv_cache) -> int:
    h, n = _host_i32(hist_lens), _host_i32(incr_lens)
    if h.shape != n.shape or h.ndim != 1:
        _bad("hist_lens and incr_lens must be 1-D of equal length")
    r = lib.pa_workspace_size(h.ctypes.data_as(C.c_void_p), n.ctypes.data_as(C.c_void_p),
                              len(h), num_q_heads, C.byref(cache))
    if r == 0:
        raise PagedAttnError(PA_ERR_BAD_SHAPE, lib.pa_last_error().decode())
    return int(r)


def paged_attn_forward(q, cache: pa_kv_cache, block_tables, hist_lens, incr_lens, scale, out,
                       workspace, lse_out=None, stream=None):
    """Attention of q [total_q, Hq, d] over the paged cache; writes out (and lse_out)."""
    import torch
    h, n = _host_i32(hist_lens), _host_i32(incr_lens)
    if h.shape != n.shape or h.ndim != 1:
        _bad("hist_lens and incr_lens must be 1-D of equal length")
    dev = getattr(cache, "device", None)
    total_q = int(n.astype(np.int64).sum())
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        _bad("q must be a 3-D tensor [total_q, num_q_heads, head_dim]")
    hq = int(q.shape[1])
    ok = [_tensor(q, "q", _bf16(), (total_q, hq, cache.head_dim)),
          _tensor(out, "out", _bf16(), (total_q, hq, cache.head_dim))]
    if lse_out is not None:
        ok.append(_tensor(lse_out, "lse_out", (torch.float32,), (total_q, hq)))
    ok.append(_tensor(block_tables, "block_tables", (torch.int32,), (None, None)))
    if int(block_tables.shape[0]) < len(h):
        _bad(f"block_tables has {int(block_tables.shape[0])} rows for {len(h)} sequences")
    if not isinstance(workspace, torch.Tensor):
        _bad("workspace must be a torch.Tensor")
    ok.append(_tensor(workspace, "workspace", (workspace.dtype,)))
    _on_device(ok, dev)
    _check(lib.paged_attn_forward(
        _ptr(q), C.byref(cache), _ptr(block_tables), int(block_tables.shape[1]),
        h.ctypes.data_as(C.c_void_p), n.ctypes.data_as(C.c_void_p), len(h), hq,
        float(scale), _ptr(out), _ptr(lse_out), _ptr(workspace),
        int(workspace.numel() * workspace.element_size()), _stream_ptr(stream)))


def _groups(group_of, group_len, num_seqs):
    go = _host_i32(group_of)
    gl = _host_i32(group_len)
    if go.shape != (num_seqs,) or gl.ndim != 1:
        _bad("group_of must have one entry per sequence and group_len be 1-D")
    return go, gl


def cascade_workspace_size(hist_lens, incr_lens, num_q_heads, cache: pa_kv_cache, block_tables,
                           group_of, group_len, scale) -> int:
    """Workspace bytes paged_attn_forward_cascade needs for this step."""
    h, n = _host_i32(hist_lens), _host_i32(incr_lens)
    go, gl = _groups(group_of, group_len, len(h))
    need = C.c_size_t(0)
    _check(lib.paged_attn_forward_cascade(
        None, C.byref(cache), None, int(block_tables.shape[1]), h.ctypes.data_as(C.c_void_p),
        n.ctypes.data_as(C.c_void_p), len(h), int(num_q_heads), float(scale), None, None,
        go.ctypes.data_as(C.c_void_p), gl.ctypes.data_as(C.c_void_p), len(gl), None, C.byref(need), None))
    return int(need.value)


def step_workspace_size(hist_lens, incr_lens, num_q_heads, cache: pa_kv_cache, block_tables, scale) -> int:
    """Workspace bytes paged_attn_step needs for this step."""
    h, n = _host_i32(hist_lens), _host_i32(incr_lens)
    need = C.c_size_t(0)
    _check(lib.paged_attn_step(C.byref(cache), None, None, None, None, None, int(block_tables.shape[1]),
                               h.ctypes.data_as(C.c_void_p), n.ctypes.data_as(C.c_void_p), len(h),
                               int(num_q_heads), float(scale), None, None, None, C.byref(need), None))
    return int(need.value)


def paged_attn_step(cache: pa_kv_cache, k_new, v_new, slot_mapping, q, block_tables, hist_lens, incr_lens,
                    scale, out, workspace, lse_out=None, stream=None):
    """kv_append of the step's new tokens and paged_attn_forward in one launch."""
    import torch
    h, n = _host_i32(hist_lens), _host_i32(incr_lens)
    if h.shape != n.shape or h.ndim != 1:
        _bad("hist_lens and incr_lens must be 1-D of equal length")
    dev = getattr(cache, "device", None)
    total_q = int(n.astype(np.int64).sum())
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        _bad("q must be a 3-D tensor [total_q, num_q_heads, head_dim]")
    hq = int(q.shape[1])
    kv_shape = (total_q, cache.num_kv_heads, cache.head_dim)
    ok = [_tensor(q, "q", _bf16(), (total_q, hq, cache.head_dim)),
          _tensor(out, "out", _bf16(), (total_q, hq, cache.head_dim)),
          _tensor(k_new, "k_new", _bf16(), kv_shape), _tensor(v_new, "v_new", _bf16(), kv_shape),
          _tensor(slot_mapping, "slot_mapping", (torch.int64,), (total_q,))]
    if lse_out is not None:
        ok.append(_tensor(lse_out, "lse_out", (torch.float32,), (total_q, hq)))
    ok.append(_tensor(block_tables, "block_tables", (torch.int32,), (None, None)))
    if int(block_tables.shape[0]) < len(h):
        _bad(f"block_tables has {int(block_tables.shape[0])} rows for {len(h)} sequences")
    if not isinstance(workspace, torch.Tensor):
        _bad("workspace must be a torch.Tensor")
    ok.append(_tensor(workspace, "workspace", (workspace.dtype,)))
    _on_device(ok, dev)
    cap = C.c_size_t(int(workspace.numel() * workspace.element_size()))
    _check(lib.paged_attn_step(
        C.byref(cache), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(q), _ptr(block_tables),
        int(block_tables.shape[1]), h.ctypes.data_as(C.c_void_p), n.ctypes.data_as(C.c_void_p), len(h), hq,
        float(scale), _ptr(out), _ptr(lse_out), _ptr(workspace), C.byref(cap), _stream_ptr(stream)))


def pa_debug_step_flags(workspace, cache: pa_kv_cache, hist_lens, incr_lens, num_q_heads, stream=None) -> int:
    """Flag word of the last paged_attn_step on `workspace` (bit 0: a bounded wait gave up)."""
    h, n = _host_i32(hist_lens), _host_i32(incr_lens)
    f = C.c_uint32(0)
    _check(lib.pa_debug_step_flags(_ptr(workspace), C.byref(cache), h.ctypes.data_as(C.c_void_p),
                                   n.ctypes.data_as(C.c_void_p), len(h), int(num_q_heads), C.byref(f),
                                   _stream_ptr(stream)))
    return int(f.value)


def paged_attn_forward_cascade(q, cache: pa_kv_cache, block_tables, hist_lens, incr_lens, scale, out,
                               workspace, group_of, group_len, lse_out=None, stream=None):
    """paged_attn_forward with declared shared-prefix groups (group_of [num_seqs],
    -1 = none; group_len [num_groups], tokens, multiples of the block size)."""
    import torch
    h, n = _host_i32(hist_lens), _host_i32(incr_lens)
    if h.shape != n.shape or h.ndim != 1:
        _bad("hist_lens and incr_lens must be 1-D of equal length")
    go, gl = _groups(group_of, group_len, len(h))
    dev = getattr(cache, "device", None)
    total_q = int(n.astype(np.int64).sum())
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        _bad("q must be a 3-D tensor [total_q, num_q_heads, head_dim]")
    hq = int(q.shape[1])
    ok = [_tensor(q, "q", _bf16(), (total_q, hq, cache.head_dim)),
          _tensor(out, "out", _bf16(), (total_q, hq, cache.head_dim))]
    if lse_out is not None:
        ok.append(_tensor(lse_out, "lse_out", (torch.float32,), (total_q, hq)))
    ok.append(_tensor(block_tables, "block_tables", (torch.int32,), (None, None)))
    if int(block_tables.shape[0]) < len(h):
        _bad(f"block_tables has {int(block_tables.shape[0])} rows for {len(h)} sequences")
    if not isinstance(workspace, torch.Tensor):
        _bad("workspace must be a torch.Tensor")
    ok.append(_tensor(workspace, "workspace", (workspace.dtype,)))
    _on_device(ok, dev)
    cap = C.c_size_t(int(workspace.numel() * workspace.element_size()))
    _check(lib.paged_attn_forward_cascade(
        _ptr(q), C.byref(cache), _ptr(block_tables), int(block_tables.shape[1]),
        h.ctypes.data_as(C.c_void_p), n.ctypes.data_as(C.c_void_p), len(h), hq, float(scale),
        _ptr(out), _ptr(lse_out), go.ctypes.data_as(C.c_void_p), gl.ctypes.data_as(C.c_void_p), len(gl),
        _ptr(workspace), C.byref(cap), _stream_ptr(stream)))


def paged_attn_forward_noalloc(q, cache: pa_kv_cache, block_tables, hist_lens, incr_lens, scale,
                               out, lse_out=None, stream=None):
    """paged_attn_forward without a workspace: the library's static scratch
    (for callers that cannot allocate)."""
    import torch
    h, n = _host_i32(hist_lens), _host_i32(incr_lens)
    if h.shape != n.shape or h.ndim != 1:
        _bad("hist_lens and incr_lens must be 1-D of equal length")
    dev = getattr(cache, "device", None)
    total_q = int(n.astype(np.int64).sum())
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        _bad("q must be a 3-D tensor [total_q, num_q_heads, head_dim]")
    hq = int(q.shape[1])
    ok = [_tensor(q, "q", _bf16(), (total_q, hq, cache.head_dim)),
          _tensor(out, "out", _bf16(), (total_q, hq, cache.head_dim))]
    if lse_out is not None:
        ok.append(_tensor(lse_out, "lse_out", (torch.float32,), (total_q, hq)))
    ok.append(_tensor(block_tables, "block_tables", (torch.int32,), (None, None)))
    if int(block_tables.shape[0]) < len(h):
        _bad(f"block_tables has {int(block_tables.shape[0])} rows for {len(h)} sequences")
    _on_device(ok, dev)
    _check(lib.paged_attn_forward_noalloc(
        _ptr(q), C.byref(cache), _ptr(block_tables), int(block_tables.shape[1]),
        h.ctypes.data_as(C.c_void_p), n.ctypes.data_as(C.c_void_p), len(h), hq,
        float(scale), _ptr(out), _ptr(lse_out), _stream_ptr(stream)))


def pa_debug_gather(cache: pa_kv_cache, block_table_row, ctx, k_out, v_out, stream=None):
    """Raw gather of one sequence's first ctx tokens through a table row (test hook)."""
    import torch
    dev = getattr(cache, "device", None)
    ok = [_tensor(block_table_row, "block_table_row", (torch.int32,), (None,))]
    if int(block_table_row.shape[0]) * cache.block_size < int(ctx):
        _bad(f"block_table_row covers {int(block_table_row.shape[0]) * cache.block_size} tokens, ctx {ctx}")
    # (MXFP4: the values, bf16)
    dt = _code_dtypes() if cache.dtype == PA_KV_FP8_E4M3 else _bf16()
    shape = (int(ctx), cache.num_kv_heads, cache.head_dim)
    ok += [_tensor(k_out, "k_out", dt, shape), _tensor(v_out, "v_out", dt, shape)]
    _on_device(ok, dev)
    _check(lib.pa_debug_gather(C.byref(cache), _ptr(block_table_row), int(ctx), _ptr(k_out),
                               _ptr(v_out), _stream_ptr(stream)))


def pa_last_error() -> str:
    return lib.pa_last_error().decode()


PEAK_MFMA_THREADS = 256 * 512      # out entries of pa_peak_mfma
PEAK_MFMA_FLOPS_PER_ITER = 1 << 28  # 256 groups x 8 waves x 8 MFMAs x 16,384 flops
PEAK_READ_THREADS = 256 * 256      # out entries of pa_peak_read


def pa_peak_mfma(out, iters, stream=None):
    """Enqueue the MFMA-loop measurement kernel (out: float32 [PEAK_MFMA_THREADS])."""
    _check(lib.pa_peak_mfma(_ptr(out), int(iters), _stream_ptr(stream)))


def pa_peak_read(buf, out, stream=None):
    """Enqueue a streaming read of the device buffer buf (out: int32 [PEAK_READ_THREADS])."""
    _check(lib.pa_peak_read(_ptr(buf), int(buf.numel() * buf.element_size()), _ptr(out),
                            _stream_ptr(stream)))


def pa_debug_overlap_cus(n):
    """CUs that stream decode items beside the prefill in later plans: n < 0
    the planner's choice (default), n >= 0 forced (0: no co-scheduling)."""
    _check(lib.pa_debug_overlap_cus(int(n)))


def pa_device_shape():
    """(compute units, XCDs) the planner cuts plans for on the current device."""
    cus, xcds = C.c_int32(), C.c_int32()
    _check(lib.pa_device_shape(C.byref(cus), C.byref(xcds)))
    return cus.value, xcds.value


def pa_debug_xcc_ids(out, stream=None):
    """Enqueue out.numel() work-groups, each writing the XCD it ran on (out: int32, GPU)."""
    import torch
    _on_device([_tensor(out, "out", (torch.int32,), (None,))])
    _check(lib.pa_debug_xcc_ids(_ptr(out), int(out.numel()), _stream_ptr(stream)))


def pa_timing_enable(on: bool):
    _check(lib.pa_timing_enable(1 if on else 0))


def pa_timing_read(kind: int):
    ms, cnt = C.c_double(), C.c_int64()
    _check(lib.pa_timing_read(kind, C.byref(ms), C.byref(cnt)))
    return ms.value, cnt.value


def pa_debug_plan(hist_lens, incr_lens, num_q_heads, cache: pa_kv_cache):
    """The planner's work list for these lengths: (items int32 [n, 8], counts[4])."""
    h, n = _host_i32(hist_lens), _host_i32(incr_lens)
    counts = np.zeros(4, dtype=np.int32)
    args = [h.ctypes.data_as(C.c_void_p), n.ctypes.data_as(C.c_void_p), len(h), num_q_heads,
            C.byref(cache)]
    st = lib.pa_debug_plan(*args, None, 0, counts.ctypes.data_as(C.c_void_p))
    if st not in (PA_OK, PA_ERR_WORKSPACE_TOO_SMALL):
        _check(st)
    cap = int(counts[0] + counts[1])
    items = np.zeros((max(cap, 1), 8), dtype=np.int32)
    _check(lib.pa_debug_plan(*args, items.ctypes.data_as(C.c_void_p), cap,
                             counts.ctypes.data_as(C.c_void_p)))
    return items[:cap], counts


def pa_debug_plan_groups(hist_lens, incr_lens, num_q_heads, cache: pa_kv_cache):
    """Per-work-group item offsets of the persistent prefill launch (int32 [n + 1]);
    empty when the plan has no such launch."""
    h, n = _host_i32(hist_lens), _host_i32(incr_lens)
    ng = C.c_int32(0)
    args = [h.ctypes.data_as(C.c_void_p), n.ctypes.data_as(C.c_void_p), len(h), num_q_heads,
            C.byref(cache)]
    st = lib.pa_debug_plan_groups(*args, None, 0, C.byref(ng))
    if st not in (PA_OK, PA_ERR_WORKSPACE_TOO_SMALL):
        _check(st)
    if ng.value == 0:
        return np.zeros(0, dtype=np.int32)
    first = np.zeros(ng.value + 1, dtype=np.int32)
    _check(lib.pa_debug_plan_groups(*args, first.ctypes.data_as(C.c_void_p), len(first), C.byref(ng)))
    return first
