"""fp64 CPU oracle for paged-KV GQA attention and kv_append (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``paged_kv_cache_gqa_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double, OpenMP across
independent outputs only); this module only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

KV_BF16 = 0
KV_E4M3 = 1
KV_MXFP4 = 2


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, no fast-math)."""
    stale = (not os.path.exists(_LIB_PATH)
             or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC))
    if force or stale:
        cmd = ["gcc", "-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
               "-shared", "-std=c11", "-Wall", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        i32, i64 = C.c_int32, C.c_int64
        L.orc_cdiv.argtypes = [i64, i64]
        L.orc_cdiv.restype = i64
        L.orc_num_blocks.argtypes = [i64, i32]
        L.orc_num_blocks.restype = i64
        L.orc_bf16_to_double.argtypes = [C.c_uint16]
        L.orc_bf16_to_double.restype = C.c_double
        L.orc_e4m3_to_double.argtypes = [C.c_uint8]
        L.orc_e4m3_to_double.restype = C.c_double
        L.orc_e4m3_from_float.argtypes = [C.c_float]
        L.orc_e4m3_from_float.restype = C.c_uint8
        L.orc_div_f32.argtypes = [C.c_float, C.c_float]
        L.orc_div_f32.restype = C.c_float
        L.orc_e2m1_to_double.argtypes = [C.c_uint8]
        L.orc_e2m1_to_double.restype = C.c_double
        L.orc_e8m0_to_double.argtypes = [C.c_uint8]
        L.orc_e8m0_to_double.restype = C.c_double
        L.orc_e2m1_from_double.argtypes = [C.c_double]
        L.orc_e2m1_from_double.restype = C.c_uint8
        L.orc_mxfp4_scale_byte.argtypes = [C.c_double]
        L.orc_mxfp4_scale_byte.restype = C.c_uint8
        L.orc_mxfp4_encode_group.argtypes = [P, i32, P, P]
        L.orc_mxfp4_encode_group.restype = None
        L.orc_mxfp4_quantize_pool.argtypes = [P, P, P, i64, i32, i32, i32]
        L.orc_mxfp4_quantize_pool.restype = None
        L.orc_gather_values.argtypes = [P, P, i32, i32, i32, i32, i32, P, i64, P]
        L.orc_gather_values.restype = C.c_int
        L.orc_kv_append.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, P, P, P, i64]
        L.orc_kv_append.restype = C.c_int
        L.orc_e4m3_quantize_pool.argtypes = [P, P, P, i64, i32, i32, i32]
        L.orc_e4m3_quantize_pool.restype = None
        L.orc_gather.argtypes = [P, i32, i32, i32, i32, i32, P, i64, P]
        L.orc_gather.restype = C.c_int
        L.orc_attention.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, P, i32, P, P, i32,
                                    i32, C.c_float, P, i64, P, P]
        L.orc_attention.restype = C.c_int
        L.orc_attention_partial.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, P, i32, i64,
                                            i64, i64, C.c_float, P, P, P]
        L.orc_attention_partial.restype = C.c_int
        L.orc_merge.argtypes = [P, P, i32, i32, P, P]
        L.orc_merge.restype = None
        L.orc_num_threads.argtypes = []
        L.orc_num_threads.restype = C.c_int
        L.orc_set_num_threads.argtypes = [C.c_int]
        L.orc_set_num_threads.restype = C.c_int
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _elem(dtype: int):
    return np.uint16 if dtype == KV_BF16 else np.uint8


def _head_dim(cache, dtype: int) -> int:
    """head_dim of a cache array [nb, hkv, bs, last] (MXFP4 packs two per byte)."""
    return cache.shape[3] * 2 if dtype == KV_MXFP4 else cache.shape[3]


def _scales(s, dtype: int):
    if s is None:
        return None
    return np.ascontiguousarray(s, dtype=np.uint8 if dtype == KV_MXFP4 else np.float32)


def cdiv(a: int, b: int) -> int:
    return int(lib().orc_cdiv(a, b))


def num_blocks(ctx: int, block_size: int) -> int:
    return int(lib().orc_num_blocks(ctx, block_size))


def bf16_to_f64(bits: int) -> float:
    return float(lib().orc_bf16_to_double(int(bits)))


def e4m3_to_f64(code: int) -> float:
    return float(lib().orc_e4m3_to_double(int(code)))


def e4m3_from_f32(x: float) -> int:
    return int(lib().orc_e4m3_from_float(float(np.float32(x))))


def div_f32(x: float, s: float) -> float:
    return float(lib().orc_div_f32(float(np.float32(x)), float(np.float32(s))))


def e2m1_to_f64(code: int) -> float:
    return float(lib().orc_e2m1_to_double(int(code)))


def e8m0_to_f64(byte: int) -> float:
    return float(lib().orc_e8m0_to_double(int(byte)))


def e2m1_from_f64(v: float) -> int:
    return int(lib().orc_e2m1_from_double(float(v)))


def mxfp4_scale_byte(amax: float) -> int:
    return int(lib().orc_mxfp4_scale_byte(float(amax)))


def mxfp4_encode_group(x_bits):
    """(codes uint8 [n], scale byte) of one group of bf16 values."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    codes = np.empty(x.shape[0], dtype=np.uint8)
    sb = np.empty(1, dtype=np.uint8)
    lib().orc_mxfp4_encode_group(_p(x), x.shape[0], _p(codes), _p(sb))
    return codes, int(sb[0])


def mxfp4_quantize_pool(src_bits):
    """MXFP4-encode a bf16 pool [nb, hkv, bs, d]: (codes [nb, hkv, bs, d/2],
    scales [nb, hkv, d/32, bs])."""
    src = np.ascontiguousarray(src_bits, dtype=np.uint16)
    nb, hkv, bs, d = src.shape
    codes = np.empty((nb, hkv, bs, d // 2), dtype=np.uint8)
    scales = np.empty((nb, hkv, d // 32, bs), dtype=np.uint8)
    lib().orc_mxfp4_quantize_pool(_p(src), _p(codes), _p(scales), nb, hkv, bs, d)
    return codes, scales


def gather_values(cache, scale, dtype, bt_row, ctx):
    """Element values of one sequence's cache in fp64: [ctx, hkv, head_dim]."""
    nb, hkv, bs, _ = cache.shape
    d = _head_dim(cache, dtype)
    bt = np.ascontiguousarray(bt_row, dtype=np.int32)
    out = np.empty((ctx, hkv, d), dtype=np.float64)
    rc = lib().orc_gather_values(_p(cache), _p(_scales(scale, dtype)), dtype, nb, hkv, bs, d, _p(bt), ctx,
                                 _p(out))
    if rc:
        raise ValueError("oracle gather_values: block id out of range")
    return out


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> int:
    """Threads for the following calls; returns the previous count."""
    return int(lib().orc_set_num_threads(int(n)))


def kv_append(k_cache, v_cache, k_scale, v_scale, dtype, k_new, v_new, slot_mapping):
    """Apply the scatter in place on host cache arrays [nb, hkv, bs, d]."""
    nb, hkv, bs, _ = k_cache.shape
    d = _head_dim(k_cache, dtype)
    assert k_cache.dtype == _elem(dtype) and v_cache.dtype == _elem(dtype)
    k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
    v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    if dtype == KV_MXFP4:  # the scales are written: they must be the caller's arrays
        assert k_scale.dtype == np.uint8 and k_scale.flags["C_CONTIGUOUS"]
        assert v_scale.dtype == np.uint8 and v_scale.flags["C_CONTIGUOUS"]
        ks, vs = k_scale, v_scale
    else:
        ks, vs = _scales(k_scale, dtype), _scales(v_scale, dtype)
    rc = lib().orc_kv_append(_p(k_cache), _p(v_cache), _p(ks), _p(vs), nb, hkv, bs, d, dtype,
                             _p(k_new), _p(v_new), _p(slots), slots.shape[0])
    if rc:
        raise ValueError("oracle kv_append: slot out of range")


def quantize_pool(src_bits, scale):
    """E4M3-encode a bf16 pool [nb, hkv, bs, d] with per-(block, head) scales."""
    src = np.ascontiguousarray(src_bits, dtype=np.uint16)
    sc = np.ascontiguousarray(scale, dtype=np.float32)
    nb, hkv, bs, d = src.shape
    assert sc.shape == (nb, hkv)
    out = np.empty(src.shape, dtype=np.uint8)
    lib().orc_e4m3_quantize_pool(_p(src), _p(sc), _p(out), nb, hkv, bs, d)
    return out


def gather(cache, bt_row, ctx):
    """Raw per-sequence gather: out[p, kvh, :] = cache[bt_row[p // bs], kvh, p % bs, :]."""
    nb, hkv, bs, d = cache.shape
    bt = np.ascontiguousarray(bt_row, dtype=np.int32)
    out = np.empty((ctx, hkv, d), dtype=cache.dtype)
    rc = lib().orc_gather(_p(cache), nb, hkv, bs, d, cache.dtype.itemsize, _p(bt), ctx, _p(out))
    if rc:
        raise ValueError("oracle gather: block id out of range")
    return out


def attention(q_bits, k_cache, v_cache, k_scale, v_scale, dtype, block_tables, hist, incr,
              num_q_heads, scale, rows=None):
    """Full-definition paged attention.  Returns (out f64 [n, hq, d], lse f64 [n, hq])."""
    nb, hkv, bs, _ = k_cache.shape
    d = _head_dim(k_cache, dtype)
    q = np.ascontiguousarray(q_bits, dtype=np.uint16)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    h = np.ascontiguousarray(hist, dtype=np.int32)
    n_ = np.ascontiguousarray(incr, dtype=np.int32)
    num_seqs = h.shape[0]
    total_q = int(n_.astype(np.int64).sum())
    assert q.shape == (total_q, num_q_heads, d)
    r = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = total_q if r is None else r.shape[0]
    out = np.empty((nrows, num_q_heads, d), dtype=np.float64)
    lse = np.empty((nrows, num_q_heads), dtype=np.float64)
    ks, vs = _scales(k_scale, dtype), _scales(v_scale, dtype)
    rc = lib().orc_attention(_p(q), _p(k_cache), _p(v_cache), _p(ks), _p(vs), dtype, nb, hkv, bs,
                             d, _p(bt), bt.shape[1], _p(h), _p(n_), num_seqs, num_q_heads,
                             float(np.float32(scale)), _p(r), nrows, _p(out), _p(lse))
    if rc:
        raise ValueError("oracle attention: bad lengths or block ids")
    return out, lse


def attention_partial(q_row_bits, k_cache, v_cache, k_scale, v_scale, dtype, bt_row, kvh, pos,
                      k_lo, k_hi, scale, want_probs=False):
    """Partial attention of one (row, head) over keys [k_lo, k_hi) ∩ [0, pos]."""
    nb, hkv, bs, _ = k_cache.shape
    d = _head_dim(k_cache, dtype)
    q = np.ascontiguousarray(q_row_bits, dtype=np.uint16)
    bt = np.ascontiguousarray(bt_row, dtype=np.int32)
    o = np.empty(d, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    n = max(0, min(k_hi, pos + 1) - k_lo)
    probs = np.empty(max(n, 1), dtype=np.float64) if want_probs else None
    ks, vs = _scales(k_scale, dtype), _scales(v_scale, dtype)
    lib().orc_attention_partial(_p(q), _p(k_cache), _p(v_cache), _p(ks), _p(vs), dtype, nb, hkv,
                                bs, d, _p(bt), kvh, pos, k_lo, k_hi, float(np.float32(scale)),
                                _p(o), _p(lse), _p(probs))
    if want_probs:
        return o, float(lse[0]), probs[:n]
    return o, float(lse[0])


def merge(o_parts, lse_parts):
    """LSE-weighted merge of partial outputs [n, d] with lse [n]."""
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lse_parts = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n, d = o_parts.shape
    o = np.empty(d, dtype=np.float64)
    lse = np.empty(1, dtype=np.float64)
    lib().orc_merge(_p(o_parts), _p(lse_parts), n, d, _p(o), _p(lse))
    return o, float(lse[0])
