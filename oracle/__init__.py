"""CPU oracle for paged KV attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product path (the HIP
library and its Python binding) never touches it, and this package never
imports the product package.

The arithmetic lives in ``oracle.c`` (fp64, explicit page gather, two-pass
softmax), built with gcc into ``liboracle.so`` next to it; ``brute.py`` is an
independent pure-Python implementation for tiny shapes.  This module only
marshals numpy arrays into the C functions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DT_CODE = {"f32": 0, "bf16": 1, "fp8": 2}

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (-O2 -fopenmp) into liboracle.so."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        i32, i64, f32, f64, vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                  ctypes.c_double, ctypes.c_void_p)
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_value.restype = f64
        L.oracle_fp8_value.argtypes = [ctypes.c_uint8]
        L.oracle_fp8_value.restype = f64
        L.oracle_fp8_encode.argtypes = [f32]
        L.oracle_fp8_encode.restype = ctypes.c_uint8
        L.oracle_fp8_encode_array.argtypes = [i64, vp, vp]
        L.oracle_fp8_quantize.argtypes = [i64, vp, f32, vp]
        L.oracle_metadata.argtypes = [i32, vp, vp, vp, i64, i32, i32, i32, vp, vp, i64, vp, vp,
                                      vp, i64]
        L.oracle_metadata.restype = ctypes.c_int
        L.oracle_save_kv.argtypes = [i64, i32, i32, i32, i32, i32, vp, vp, vp, f32, f32, vp, vp]
        L.oracle_save_kv.restype = ctypes.c_int
        L.oracle_attention.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, i64, i32, i32, vp,
                                       i32, vp, vp, f64, f64, f64, i64, vp, vp, vp, i32]
        L.oracle_attention.restype = ctypes.c_int
        L.oracle_pool_bytes.argtypes = [i64, i64, i64, i64]
        L.oracle_pool_bytes.restype = i64
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _raw(x: np.ndarray, dtype: str) -> np.ndarray:
    """View an array of values in a cache dtype as its raw storage."""
    want = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}[dtype]
    x = np.ascontiguousarray(x)
    assert x.dtype == want, (x.dtype, dtype)
    return x


# ----------------------------------------------------------------- values

def bf16_value(bits) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    f = lib().oracle_bf16_value
    return np.array([f(int(b)) for b in bits.ravel()], dtype=np.float64).reshape(bits.shape)


def fp8_value(codes) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    f = lib().oracle_fp8_value
    return np.array([f(int(c)) for c in codes.ravel()], dtype=np.float64).reshape(codes.shape)


def fp8_encode(y) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, dtype=np.uint8)
    lib().oracle_fp8_encode_array(y.size, _ptr(y), _ptr(out))
    return out


def fp8_quantize(bf16_bits: np.ndarray, scale: float) -> np.ndarray:
    x = np.ascontiguousarray(bf16_bits, dtype=np.uint16)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_fp8_quantize(x.size, _ptr(x), float(scale), _ptr(out))
    return out


def pool_bytes(tokens: int, heads: int, head_dim: int, elem_bytes: int) -> int:
    return int(lib().oracle_pool_bytes(tokens, heads, head_dim, elem_bytes))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


# --------------------------------------------------------------- metadata

def metadata(seq_lens, extend_lens, page_table, page_size: int, num_pages: int) -> dict:
    """Index buffers of one batch; extend_lens None means decode."""
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    ext = None if extend_lens is None else np.ascontiguousarray(extend_lens, dtype=np.int32)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    B = seq_lens.shape[0]
    P = int(page_size)
    pages = int(sum((int(L) + P - 1) // P for L in seq_lens))
    N = B if ext is None else int(ext.sum())
    out = dict(kv_indptr=np.zeros(B + 1, np.int32), kv_indices=np.zeros(max(pages, 1), np.int32),
               kv_last_page_len=np.zeros(B, np.int32), qo_indptr=np.zeros(B + 1, np.int32),
               out_cache_loc=np.zeros(max(N, 1), np.int32))
    rc = lib().oracle_metadata(B, _ptr(seq_lens), _ptr(ext), _ptr(pt), pt.shape[1], pt.shape[1], P,
                               int(num_pages), _ptr(out["kv_indptr"]), _ptr(out["kv_indices"]),
                               out["kv_indices"].size, _ptr(out["kv_last_page_len"]),
                               _ptr(out["qo_indptr"]), _ptr(out["out_cache_loc"]),
                               out["out_cache_loc"].size)
    if rc != 0:
        raise ValueError("oracle_metadata rejected the batch")
    out["kv_indices"] = out["kv_indices"][:pages]
    out["out_cache_loc"] = out["out_cache_loc"][:N]
    return out


# ---------------------------------------------------------------- save_kv

def save_kv(slots, k_new, v_new, src_dtype: str, kv_dtype: str, k_pool, v_pool,
            k_scale: float = 1.0, v_scale: float = 1.0) -> None:
    """Scatter new rows (K [N, Hkv, Dk], V [N, Hkv, Dv]) into the pools in place."""
    slots = np.ascontiguousarray(slots, dtype=np.int32)
    k_new, v_new = _raw(k_new, src_dtype), _raw(v_new, src_dtype)
    assert k_pool.flags["C_CONTIGUOUS"] and v_pool.flags["C_CONTIGUOUS"]
    N, Hkv, Dk = k_new.shape
    Dv = v_new.shape[2]
    assert k_pool.shape[1:] == (Hkv, Dk) and v_pool.shape[1:] == (Hkv, Dv)
    rc = lib().oracle_save_kv(N, Hkv, Dk, Dv, DT_CODE[src_dtype], DT_CODE[kv_dtype], _ptr(slots),
                              _ptr(k_new), _ptr(v_new), float(k_scale), float(v_scale),
                              _ptr(k_pool), _ptr(v_pool))
    if rc != 0:
        raise ValueError("oracle_save_kv: unsupported dtype pair")


# -------------------------------------------------------------- attention

def attention(seq_lens, extend_lens, page_table, page_size: int, num_pages: int, q, q_dtype: str,
              k_pool, v_pool, kv_dtype: str, scale: float, k_scale: float = 1.0,
              v_scale: float = 1.0, sel=None, threads: int = 0):
    """fp64 attention.  q: [N, Hq, Dk] raw storage; pools: K [slots, Hkv, Dk],
    V [slots, Hkv, Dv] raw (the value width may differ from the key width).

    Returns (out, lse): out [N, Hq, Dv] and lse [N, Hq] float64, or, with
    ``sel`` (flat indices token*Hq + head), out [len(sel), Dv], lse [len(sel)].
    """
    seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    ext = None if extend_lens is None else np.ascontiguousarray(extend_lens, dtype=np.int32)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    q = _raw(q, q_dtype)
    k_pool, v_pool = _raw(k_pool, kv_dtype), _raw(v_pool, kv_dtype)
    N, Hq, Dk = q.shape
    Hkv = k_pool.shape[1]
    Dv = v_pool.shape[2]
    assert k_pool.shape[2] == Dk and v_pool.shape[1] == Hkv
    if sel is None:
        n_sel, sel_arr = N * Hq, None
    else:
        sel_arr = np.ascontiguousarray(sel, dtype=np.int64)
        n_sel = sel_arr.size
    out = np.empty((n_sel, Dv), dtype=np.float64)
    lse = np.empty((n_sel,), dtype=np.float64)
    rc = lib().oracle_attention(seq_lens.shape[0], Hq, Hkv, Dk, Dv, int(page_size), _ptr(seq_lens),
                                _ptr(ext), _ptr(pt), pt.shape[1], int(num_pages),
                                DT_CODE[q_dtype], _ptr(q), DT_CODE[kv_dtype], _ptr(k_pool),
                                _ptr(v_pool), float(scale), float(k_scale), float(v_scale), n_sel,
                                _ptr(sel_arr), _ptr(out), _ptr(lse), int(threads))
    if rc != 0:
        raise ValueError("oracle_attention rejected the input")
    if sel is None:
        return out.reshape(N, Hq, Dv), lse.reshape(N, Hq)
    return out, lse
