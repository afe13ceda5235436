"""CPU oracle for the NVFP4 paged-KV append and causal paged prefill.

TEST INFRASTRUCTURE ONLY: tests/, the smoke check in __graft_entry__ and the
benchmark's cpu_baseline leg may import this package; the product path
(nvfp4_paged_kv_amd) never does.  The arithmetic lives in plain C
(nvfp4_oracle.c, built with gcc into liboracle.so); this module only
marshals numpy arrays through ctypes.  It shares no code with the HIP path.

Every function here is pinned by tests/test_oracle_*.py against values that
do not come from the oracle itself (library conversions, closed forms,
brute force, invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Error bits reported by the oracle (same meaning as the library's device flag).
BAD_K_SCALE = 1
BAD_V_SCALE = 2
SLOT_OOB = 4
PAGE_OOB = 8


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (no fused multiply-add, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
             "-shared", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.oracle_e2m1_encode_mag.restype = ctypes.c_int
        L.oracle_e2m1_encode_mag.argtypes = [ctypes.c_float]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_int]
        L.oracle_e4m3_encode.restype = ctypes.c_int
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e2m1_encode_array.argtypes = [P, ctypes.c_int64, P]
        L.oracle_e4m3_encode_array.argtypes = [P, ctypes.c_int64, P]
        L.oracle_scale_ok.restype = ctypes.c_int
        L.oracle_scale_ok.argtypes = [ctypes.c_float]
        L.oracle_quantize_block.argtypes = [P, ctypes.c_float, P, P]
        L.oracle_append.restype = ctypes.c_uint32
        L.oracle_append.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_float, ctypes.c_float,
                                    P, P, P, P, ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, ctypes.c_int]
        L.oracle_dequant_rows.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int,
                                          ctypes.c_double, P]
        L.oracle_prefill.restype = ctypes.c_uint32
        L.oracle_prefill.argtypes = [P, P, P, P, P, ctypes.c_int, P, P, P, P, ctypes.c_int64,
                                     ctypes.c_int, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_double, P, ctypes.c_int,
                                     P, ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _threads() -> int:
    # at most 16 worker threads
    return max(1, min(os.cpu_count() or 1, 16))


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(int(code))


def e2m1_encode(y: np.ndarray) -> np.ndarray:
    """Signed 4-bit codes (sign of y in bit 3) of fp32 values y."""
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint8)
    lib().oracle_e2m1_encode_array(_ptr(y), y.size, _ptr(out))
    return out


def e4m3_encode(s: np.ndarray) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty(s.shape, np.uint8)
    lib().oracle_e4m3_encode_array(_ptr(s), s.size, _ptr(out))
    return out


def scale_ok(g: float) -> bool:
    return bool(lib().oracle_scale_ok(float(g)))


def quantize_block(x_bf16_bits: np.ndarray, g: float):
    """16 bf16 values (as uint16 bit patterns) -> (8 packed bytes, scale byte)."""
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16).reshape(16)
    packed = np.zeros(8, np.uint8)
    sf = np.zeros(1, np.uint8)
    lib().oracle_quantize_block(_ptr(x), ctypes.c_float(g), _ptr(packed), _ptr(sf))
    return packed, int(sf[0])


def append(k_bits, v_bits, slot_mapping, k_scale, v_scale, k_cache, v_cache, k_sf, v_sf,
           page_size, nthreads=None) -> int:
    """Quantize k/v ([T, H_kv, D] bf16 bit patterns, uint16) and write them into
    the numpy caches in place.  Returns the error bits."""
    T, H, D = k_bits.shape
    assert v_bits.shape == k_bits.shape and k_bits.dtype == np.uint16
    assert slot_mapping.dtype == np.int64 and slot_mapping.shape == (T,)
    P = k_cache.shape[0]
    assert k_cache.shape == (P, page_size, H, D // 2) and k_sf.shape == (P, page_size, H, D // 16)
    for a in (k_cache, v_cache, k_sf, v_sf):
        assert a.dtype == np.uint8 and a.flags["C_CONTIGUOUS"]
    return int(lib().oracle_append(
        _ptr(np.ascontiguousarray(k_bits)), _ptr(np.ascontiguousarray(v_bits)),
        _ptr(np.ascontiguousarray(slot_mapping)), T, ctypes.c_float(k_scale),
        ctypes.c_float(v_scale), _ptr(k_cache), _ptr(v_cache), _ptr(k_sf), _ptr(v_sf), P,
        page_size, H, D, nthreads or _threads()))


def dequant_rows(cache, sf, rows, head_dim, g) -> np.ndarray:
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.empty((rows.size, head_dim), np.float64)
    lib().oracle_dequant_rows(_ptr(np.ascontiguousarray(cache)), _ptr(np.ascontiguousarray(sf)),
                              _ptr(rows), rows.size, head_dim, float(g), _ptr(out))
    return out


def prefill(q_bits, qo_indptr, kv_indptr, page_table, kv_lens, k_cache, v_cache, k_sf, v_sf,
            k_scale, v_scale, num_q_heads, sm_scale, requests=None, out=None, nthreads=None):
    """fp64 causal paged prefill.  q_bits: [total_q, H_q, D] uint16 (bf16 bits).
    Returns (out [total_q, H_q, D] float64, error bits)."""
    total_q, Hq, D = q_bits.shape
    assert Hq == num_q_heads
    P, ps, Hk, _ = k_cache.shape
    B = kv_lens.shape[0]
    qo = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    kvp = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    kvl = np.ascontiguousarray(kv_lens, dtype=np.int32)
    if out is None:
        out = np.full((total_q, Hq, D), np.nan, np.float64)
    reqs = None if requests is None else np.ascontiguousarray(requests, dtype=np.int32)
    err = lib().oracle_prefill(
        _ptr(np.ascontiguousarray(q_bits)), _ptr(qo), _ptr(kvp), _ptr(pt), _ptr(kvl), B,
        _ptr(k_cache), _ptr(v_cache), _ptr(k_sf), _ptr(v_sf), P, ps, ctypes.c_float(k_scale),
        ctypes.c_float(v_scale), Hq, Hk, D, float(sm_scale),
        None if reqs is None else _ptr(reqs), 0 if reqs is None else reqs.size, _ptr(out),
        nthreads or _threads())
    return out, int(err)
