"""CPU oracle for paged-KV-cache decode attention (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The GPU
library never imports it and shares no code with it; see ``pkv_oracle.c`` for
the definitions, their sources on the pages, and the conventions fixed where
the pages are silent.

Arrays are numpy.  Element types are named explicitly because numpy has no
bfloat16 or fp8 type: ``"f32"`` (float32 array), ``"bf16"`` (uint16 array of
bfloat16 bit patterns), ``"fp8"`` (uint8 array of OCP E4M3 codes).

Pool layouts (see ``pkv_oracle.c``): the K pool is
``[num_blocks, H_kv, D // X, block_size, X]`` with ``X = 16 // element size``
(16-byte chunks of consecutive dimensions, chunk-major), the V pool is
``[num_blocks, H_kv, D, block_size]`` (dimension-major).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": 0, "bf16": 1, "fp8": 2}
_NP = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}
_ELT = {"f32": 4, "bf16": 2, "fp8": 1}


def k_pool_shape(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str, block_size: int = 16):
    x = 16 // _ELT[dtype]
    return (num_blocks, num_kv_heads, head_dim // x, block_size, x)


def v_pool_shape(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str = "", block_size: int = 16):
    return (num_blocks, num_kv_heads, head_dim, block_size)

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED = 0, 1, 2


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: oracle status {status}")
        self.status = status


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, IEEE arithmetic, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
               "-fno-fast-math", "-fPIC", "-shared", "-pthread",
               "-o", _LIB_PATH, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return _LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        p, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        lib.oracle_kv_write.argtypes = [p, p, ctypes.c_int, p, p, ctypes.c_int, p, i32,
                                        i32, i32, i32, i32, f32, f32]
        lib.oracle_kv_write.restype = ctypes.c_int
        lib.oracle_paged_attention.argtypes = [p, p, ctypes.c_int, p, p, ctypes.c_int, p, i32,
                                               p, i32, i32, i32, i32, i32, i32,
                                               f32, f32, f32, i32, i32]
        lib.oracle_paged_attention.restype = ctypes.c_int
        lib.oracle_paged_attention_varlen.argtypes = [p, p, ctypes.c_int, p, p, p, ctypes.c_int, p, i32,
                                                      p, i32, i32, i32, i32, i32, i32, f32, f32, f32, i32]
        lib.oracle_paged_attention_varlen.restype = ctypes.c_int
        lib.oracle_fp8_e4m3_decode_n.argtypes = [p, p, i64]
        lib.oracle_fp8_e4m3_quantise_n.argtypes = [p, p, i64, f32]
        lib.oracle_bf16_to_double_n.argtypes = [p, p, i64]
        lib.oracle_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _check(a: np.ndarray, dtype: str, name: str) -> np.ndarray:
    if a.dtype != _NP[dtype]:
        raise TypeError(f"{name}: expected numpy {_NP[dtype].__name__} for {dtype}, got {a.dtype}")
    if not a.flags.c_contiguous:
        raise ValueError(f"{name} must be C-contiguous")
    return a


def num_threads(requested: int = 0) -> int:
    """Threads the attention oracle actually uses for ``requested`` (0 = all cores)."""
    return _load().oracle_num_threads(int(requested))


def fp8_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3 codes (uint8) -> float64 values (NaN for 0x7F / 0xFF)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(codes.shape, dtype=np.float64)
    _load().oracle_fp8_e4m3_decode_n(_ptr(codes), _ptr(out), codes.size)
    return out


def fp8_quantise(x: np.ndarray, scale: float = 1.0) -> np.ndarray:
    """float32 values -> OCP E4M3 codes of fp32(x / scale), saturating, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().oracle_fp8_e4m3_quantise_n(_ptr(x), _ptr(out), x.size, ctypes.c_float(scale))
    return out


def bf16_to_double(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_bf16_to_double_n(_ptr(bits), _ptr(out), bits.size)
    return out


def kv_write(k_new, v_new, in_dtype, k_cache, v_cache, cache_dtype, slot_mapping,
             block_size=16, k_scale=1.0, v_scale=1.0):
    """Write tokens into the pools in place (see ``oracle_kv_write``).

    k_new, v_new: [T, H_kv, D]; caches: ``k_pool_shape`` / ``v_pool_shape``; slot_mapping: [T] int32.
    """
    _check(k_new, in_dtype, "k_new"); _check(v_new, in_dtype, "v_new")
    _check(k_cache, cache_dtype, "k_cache"); _check(v_cache, cache_dtype, "v_cache")
    slot_mapping = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    T, H, D = k_new.shape
    NB = k_cache.shape[0]
    if v_new.shape != k_new.shape or slot_mapping.shape != (T,):
        raise ValueError("shape mismatch")
    if k_cache.shape != k_pool_shape(NB, H, D, cache_dtype, block_size) or \
            v_cache.shape != v_pool_shape(NB, H, D, cache_dtype, block_size):
        raise ValueError("pool shape mismatch")
    st = _load().oracle_kv_write(_ptr(k_new), _ptr(v_new), DTYPES[in_dtype],
                                 _ptr(k_cache), _ptr(v_cache), DTYPES[cache_dtype],
                                 _ptr(slot_mapping), T, H, D, block_size, NB,
                                 ctypes.c_float(k_scale), ctypes.c_float(v_scale))
    if st != OK:
        raise OracleError(st, "oracle_kv_write")


def paged_attention(q, q_dtype, k_cache, v_cache, cache_dtype, block_table, context_lens,
                    scale, k_scale=1.0, v_scale=1.0, block_size=16, partition_size=0,
                    threads=0) -> np.ndarray:
    """float64 [B, H_q, D] attention output (see ``oracle_paged_attention``)."""
    _check(q, q_dtype, "q")
    _check(k_cache, cache_dtype, "k_cache"); _check(v_cache, cache_dtype, "v_cache")
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    B, Hq, D = q.shape
    NB, Hkv = k_cache.shape[0], k_cache.shape[1]
    if k_cache.shape != k_pool_shape(NB, Hkv, D, cache_dtype, block_size) or \
            v_cache.shape != v_pool_shape(NB, Hkv, D, cache_dtype, block_size):
        raise ValueError("cache shape mismatch")
    if block_table.ndim != 2 or block_table.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("table shape mismatch")
    MB = block_table.shape[1]
    out = np.zeros((B, Hq, D), dtype=np.float64)
    st = _load().oracle_paged_attention(_ptr(out), _ptr(q), DTYPES[q_dtype],
                                        _ptr(k_cache), _ptr(v_cache), DTYPES[cache_dtype],
                                        _ptr(block_table), MB, _ptr(context_lens),
                                        B, Hq, Hkv, D, block_size, NB,
                                        ctypes.c_float(scale), ctypes.c_float(k_scale),
                                        ctypes.c_float(v_scale), int(partition_size), int(threads))
    if st != OK:
        raise OracleError(st, "oracle_paged_attention")
    return out


def paged_attention_varlen(q, q_dtype, cu_seqlens_q, k_cache, v_cache, cache_dtype, block_table, context_lens,
                           scale, k_scale=1.0, v_scale=1.0, block_size=16, threads=0) -> np.ndarray:
    """float64 [T, H_q, D]: every new query token attends causally to its sequence's context
    (see ``oracle_paged_attention_varlen``)."""
    _check(q, q_dtype, "q")
    _check(k_cache, cache_dtype, "k_cache"); _check(v_cache, cache_dtype, "v_cache")
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    context_lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    T, Hq, D = q.shape
    B = context_lens.shape[0]
    NB, Hkv = k_cache.shape[0], k_cache.shape[1]
    if cu.shape != (B + 1,) or int(cu[-1]) != T:
        raise ValueError("cu_seqlens_q must be [B + 1] and end at the number of query rows")
    if k_cache.shape != k_pool_shape(NB, Hkv, D, cache_dtype, block_size) or \
            v_cache.shape != v_pool_shape(NB, Hkv, D, cache_dtype, block_size):
        raise ValueError("cache shape mismatch")
    if block_table.ndim != 2 or block_table.shape[0] != B:
        raise ValueError("table shape mismatch")
    MB = block_table.shape[1]
    out = np.zeros((T, Hq, D), dtype=np.float64)
    st = _load().oracle_paged_attention_varlen(_ptr(out), _ptr(q), DTYPES[q_dtype], _ptr(cu),
                                               _ptr(k_cache), _ptr(v_cache), DTYPES[cache_dtype],
                                               _ptr(block_table), MB, _ptr(context_lens),
                                               B, Hq, Hkv, D, block_size, NB,
                                               ctypes.c_float(scale), ctypes.c_float(k_scale),
                                               ctypes.c_float(v_scale), int(threads))
    if st != OK:
        raise OracleError(st, "oracle_paged_attention_varlen")
    return out
