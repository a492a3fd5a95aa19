"""ctypes wrapper around the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check in
``__graft_entry__`` and by the CPU-baseline leg of ``bench.py``.  The product
package never imports it.  The oracle shares no code with the HIP library.

Arrays are numpy arrays holding raw bit patterns: bf16 as ``uint16``, e4m3fn
as ``uint8``, scales as ``float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

GROUP = 128
E4M3_MAX = 448.0
SCALE_FLOOR = np.float32(1e-12)


def build() -> str:
    """Compile ``oracle.c`` with gcc (no fast-math, no FP contraction)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-std=c11", "-fPIC", "-shared", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.oracle_bf16_decode.restype = ctypes.c_double
        L.oracle_bf16_decode.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_encode.restype = ctypes.c_uint16
        L.oracle_bf16_encode.argtypes = [ctypes.c_double]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_dual_rmsnorm_group_quant.restype = None
        L.oracle_dual_rmsnorm_group_quant.argtypes = [
            p, i64, p, i64, p, p, ctypes.c_float, i64, i64, i64,
            ctypes.c_int, ctypes.c_int, p, p, p, p, p]
        L.oracle_block_scaled_fp8_gemm.restype = None
        L.oracle_block_scaled_fp8_gemm.argtypes = [
            p, p, ctypes.c_int, p, p, p, i64, i64, i64]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_group_quant.restype = None
        L.oracle_e8m0_decode.restype = ctypes.c_double
        L.oracle_e8m0_decode.argtypes = [ctypes.c_uint8]
        L.oracle_dual_rmsnorm_group_quant_e8m0.restype = None
        L.oracle_dual_rmsnorm_group_quant_e8m0.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_float, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_tile_weight.restype = None
        L.oracle_tile_weight.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        L.oracle_untile_weight.restype = None
        L.oracle_untile_weight.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]
        L.oracle_group_quant.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_rmsnorm_group_quant.restype = None
        L.oracle_rmsnorm_group_quant.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float,
                                                 ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def e8m0_decode(e: int) -> float:
    """Value of an e8m0 scale byte: 2^(e - 127) (255: NaN)."""
    return lib().oracle_e8m0_decode(int(e))


def e8m0_decode_array(e: np.ndarray) -> np.ndarray:
    table = np.array([e8m0_decode(i) for i in range(256)], dtype=np.float64)
    return table[np.asarray(e, dtype=np.uint8)]


def dual_rmsnorm_group_quant_e8m0(q, kv, gamma_q, gamma_kv, eps, transpose_scale, want_ratio=False):
    """The dual RMSNorm + per-1x128 group quant with e8m0 (power-of-two)
    scales.  Returns a dict with ``q`` (uint8 codes [M, Nq]), ``scale``
    (uint8 e8m0 bytes, M*Nq/128 in the requested layout), ``kv`` (uint16
    bf16 [M, Nkv]) and, when asked, ``ratio`` (y * 2^-e, float64)."""
    q, qs = _row_view(q, np.uint16)
    kv, ks = _row_view(kv, np.uint16)
    M, Nq = q.shape
    Nkv = kv.shape[1]
    assert kv.shape[0] == M and Nq % GROUP == 0
    gamma_q = np.ascontiguousarray(gamma_q, dtype=np.uint16)
    gamma_kv = np.ascontiguousarray(gamma_kv, dtype=np.uint16)
    out_q = np.zeros((M, Nq), np.uint8)
    out_s = np.zeros(M * (Nq // GROUP), np.uint8)
    out_kv = np.zeros((M, Nkv), np.uint16)
    ratio = np.zeros((M, Nq), np.float64) if want_ratio else None
    lib().oracle_dual_rmsnorm_group_quant_e8m0(
        _ptr(q), qs, _ptr(kv), ks, _ptr(gamma_q), _ptr(gamma_kv), ctypes.c_float(eps), M, Nq, Nkv,
        int(bool(transpose_scale)), _ptr(out_q), _ptr(out_s), _ptr(out_kv), _ptr(ratio))
    res = {"q": out_q, "scale": out_s, "kv": out_kv}
    if want_ratio:
        res["ratio"] = ratio
    return res


def tile_weight(w: np.ndarray) -> np.ndarray:
    """The tiled byte order of an [N, K] uint8 weight (flat, N*K bytes)."""
    w = np.ascontiguousarray(w, dtype=np.uint8)
    N, K = w.shape
    assert N % 16 == 0 and K % GROUP == 0
    out = np.zeros(N * K, np.uint8)
    lib().oracle_tile_weight(_ptr(w), N, K, _ptr(out))
    return out


def untile_weight(tiled: np.ndarray, N: int, K: int) -> np.ndarray:
    """Inverse of tile_weight: flat tiled bytes -> [N, K] row-major."""
    tiled = np.ascontiguousarray(tiled, dtype=np.uint8).reshape(-1)
    assert tiled.size == N * K and N % 16 == 0 and K % GROUP == 0
    out = np.zeros((N, K), np.uint8)
    lib().oracle_untile_weight(_ptr(tiled), N, K, _ptr(out))
    return out


def _ptr(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


# -- scalar codecs ----------------------------------------------------------

def bf16_decode(bits: int) -> float:
    return lib().oracle_bf16_decode(int(bits))


def bf16_encode(v: float) -> int:
    return lib().oracle_bf16_encode(float(v))


def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(int(code))


def e4m3_encode(v: float) -> int:
    return lib().oracle_e4m3_encode(float(v))


def e4m3_decode_array(codes: np.ndarray) -> np.ndarray:
    table = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def bf16_decode_array(bits: np.ndarray) -> np.ndarray:
    table = np.array([bf16_decode(b) for b in range(65536)], dtype=np.float64)
    return table[np.asarray(bits, dtype=np.uint16)]


def num_threads() -> int:
    return lib().oracle_num_threads()


# -- the method --------------------------------------------------------------

def _row_view(x: np.ndarray, dtype) -> tuple[np.ndarray, int]:
    """Return (base array, row stride in elements) for a 2-D view whose inner
    stride is one element."""
    assert x.dtype == dtype and x.ndim == 2
    item = x.dtype.itemsize
    assert x.strides[1] == item, "inner stride must be one element"
    return x, x.strides[0] // item


def dual_rmsnorm_group_quant(q: np.ndarray, kv: np.ndarray,
                             gamma_q: np.ndarray, gamma_kv: np.ndarray,
                             eps: float, transpose_scale: bool,
                             sequential: bool = False, want_ratio: bool = False):
    """Run the oracle on 2-D bf16 views ``q`` [M, Nq] and ``kv`` [M, Nkv]
    (row strides arbitrary, unit inner stride).

    Returns a dict with ``q`` (uint8 [M, Nq]), ``scale`` (float32, M*G values
    in the requested layout), ``kv`` (uint16 [M, Nkv]) and, when asked,
    ``ratio`` / ``y`` (float64 [M, Nq])."""
    q, qs = _row_view(q, np.uint16)
    kv, ks = _row_view(kv, np.uint16)
    M, Nq = q.shape
    M2, Nkv = kv.shape
    assert M == M2 and Nq % GROUP == 0
    gamma_q = np.ascontiguousarray(gamma_q, dtype=np.uint16)
    gamma_kv = np.ascontiguousarray(gamma_kv, dtype=np.uint16)
    assert gamma_q.shape == (Nq,) and gamma_kv.shape == (Nkv,)
    out_q = np.zeros((M, Nq), np.uint8)
    out_s = np.zeros(M * (Nq // GROUP), np.float32)
    out_kv = np.zeros((M, Nkv), np.uint16)
    ratio = np.zeros((M, Nq), np.float64) if want_ratio else None
    y = np.zeros((M, Nq), np.float64) if want_ratio else None
    lib().oracle_dual_rmsnorm_group_quant(
        _ptr(q), qs, _ptr(kv), ks, _ptr(gamma_q), _ptr(gamma_kv),
        ctypes.c_float(eps), M, Nq, Nkv, int(bool(transpose_scale)),
        int(bool(sequential)), _ptr(out_q), _ptr(out_s), _ptr(out_kv),
        _ptr(ratio), _ptr(y))
    res = {"q": out_q, "scale": out_s, "kv": out_kv}
    if want_ratio:
        res["ratio"] = ratio
        res["y"] = y
    return res


def group_quant(x: np.ndarray, transpose_scale: bool, want_ratio: bool = False):
    """Per-1x128 dynamic FP8 quant of a 2-D bf16 view ``x`` [M, N] (no
    normalisation).  Returns a dict with ``q`` (uint8 [M, N]), ``scale``
    (float32, M*N/128 values in the requested layout) and, when asked,
    ``ratio`` (float64 x / s)."""
    x, xs = _row_view(x, np.uint16)
    M, N = x.shape
    assert N % GROUP == 0
    out_q = np.zeros((M, N), np.uint8)
    out_s = np.zeros(M * (N // GROUP), np.float32)
    ratio = np.zeros((M, N), np.float64) if want_ratio else None
    lib().oracle_group_quant(_ptr(x), xs, M, N, int(bool(transpose_scale)), _ptr(out_q), _ptr(out_s), _ptr(ratio))
    res = {"q": out_q, "scale": out_s}
    if want_ratio:
        res["ratio"] = ratio
    return res


def rmsnorm_group_quant(x: np.ndarray, gamma: np.ndarray, eps: float, transpose_scale: bool,
                        want_ratio: bool = False):
    """Single-input RMSNorm + per-1x128 FP8 group quant of a 2-D bf16 view
    ``x`` [M, N] with bf16 ``gamma`` [N].  Same outputs as group_quant."""
    x, xs = _row_view(x, np.uint16)
    M, N = x.shape
    assert N % GROUP == 0
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    assert gamma.shape == (N,)
    out_q = np.zeros((M, N), np.uint8)
    out_s = np.zeros(M * (N // GROUP), np.float32)
    ratio = np.zeros((M, N), np.float64) if want_ratio else None
    lib().oracle_rmsnorm_group_quant(_ptr(x), xs, _ptr(gamma), ctypes.c_float(eps), M, N,
                                     int(bool(transpose_scale)), _ptr(out_q), _ptr(out_s), _ptr(ratio))
    res = {"q": out_q, "scale": out_s}
    if want_ratio:
        res["ratio"] = ratio
    return res


def block_scaled_fp8_gemm(a: np.ndarray, a_scale: np.ndarray, a_scale_transposed: bool,
                          w: np.ndarray, w_scale: np.ndarray) -> np.ndarray:
    """fp64 reference of the block-scaled GEMM: ``a`` uint8 [M, K], ``a_scale``
    float32 with M*K/128 values, ``w`` uint8 [N, K], ``w_scale`` float32
    [N/128, K/128].  Returns float64 [M, N]."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.uint8)
    a_scale = np.ascontiguousarray(a_scale, dtype=np.float32).reshape(-1)
    w_scale = np.ascontiguousarray(w_scale, dtype=np.float32).reshape(-1)
    M, K = a.shape
    N, K2 = w.shape
    assert K == K2 and K % GROUP == 0 and N % GROUP == 0
    assert a_scale.size == M * (K // GROUP)
    assert w_scale.size == (N // GROUP) * (K // GROUP)
    out = np.zeros((M, N), np.float64)
    lib().oracle_block_scaled_fp8_gemm(_ptr(a), _ptr(a_scale), int(bool(a_scale_transposed)),
                                       _ptr(w), _ptr(w_scale), _ptr(out), M, N, K)
    return out
