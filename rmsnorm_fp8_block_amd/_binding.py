"""Thin ctypes binding of ``libmi_normquant.so`` (the C ABI of
``include/mi_normquant.h``).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  torch supplies device memory and the current
stream.  If the library is not built the first call raises; there is no
CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmi_normquant.so")
GROUP = 128

MI_OK, MI_ERR_NULL, MI_ERR_SHAPE, MI_ERR_STRIDE, MI_ERR_ALIGN, MI_ERR_HIP, MI_ERR_ALIAS, MI_ERR_LAYOUT = range(8)
MI_WEIGHT_ROW_MAJOR, MI_WEIGHT_TILED = 0, 1
MI_CAP_AS_ROW_MAJOR, MI_CAP_AS_COL_MAJOR, MI_CAP_WEIGHT_TILED, MI_CAP_SCALE_E8M0 = 1, 2, 4, 8

EXPORTED = (
    "mi_fused_dual_rmsnorm_group_quant",
    "mi_fused_dual_rmsnorm_group_quant_e8m0",
    "mi_rmsnorm_group_quant",
    "mi_group_quant_1x128",
    "mi_block_scaled_fp8_gemm",
    "mi_block_scaled_fp8_gemm_ex",
    "mi_block_scaled_fp8_gemm_e8m0",
    "mi_block_scaled_fp8_gemm_pair",
    "mi_block_scaled_fp8_gemm_pair_ex",
    "mi_block_scaled_fp8_gemm_pair_e8m0",
    "mi_fused_normquant_gemm_pair",
    "mi_fused_normquant_gemm_pair_e8m0",
    "mi_fused_normquant_gemm_pair_launches",
    "mi_gemm_capabilities",
    "mi_preferred_weight_layout",
    "mi_relayout_weight",
    "mi_negotiate_scale_layout",
    "mi_status_string",
    "mi_init",
)


class MiError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {text}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m rmsnorm_fp8_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.mi_fused_dual_rmsnorm_group_quant.restype = c_int
        L.mi_fused_dual_rmsnorm_group_quant.argtypes = [
            p, i64, p, i64, p, p, ctypes.c_float, i64, i64, i64, c_int, p, p, p, p]
        L.mi_rmsnorm_group_quant.restype = c_int
        L.mi_rmsnorm_group_quant.argtypes = [p, i64, p, ctypes.c_float, i64, i64, c_int, p, p, p]
        L.mi_group_quant_1x128.restype = c_int
        L.mi_group_quant_1x128.argtypes = [p, i64, i64, i64, c_int, p, p, p]
        L.mi_fused_dual_rmsnorm_group_quant_e8m0.restype = c_int
        L.mi_fused_dual_rmsnorm_group_quant_e8m0.argtypes = [
            p, i64, p, i64, p, p, ctypes.c_float, i64, i64, i64, c_int, p, p, p, p]
        L.mi_block_scaled_fp8_gemm_e8m0.restype = c_int
        L.mi_block_scaled_fp8_gemm_e8m0.argtypes = [p, p, c_int, p, c_int, p, p, i64, i64, i64, p]
        L.mi_block_scaled_fp8_gemm_pair_e8m0.restype = c_int
        L.mi_block_scaled_fp8_gemm_pair_e8m0.argtypes = [p, p, c_int, c_int, p, p, p, i64, p, p, p, i64, i64, i64, p]
        L.mi_block_scaled_fp8_gemm.restype = c_int
        L.mi_block_scaled_fp8_gemm.argtypes = [p, p, c_int, p, p, p, i64, i64, i64, p]
        L.mi_block_scaled_fp8_gemm_pair.restype = c_int
        L.mi_block_scaled_fp8_gemm_pair.argtypes = [p, p, c_int, p, p, p, i64, p, p, p, i64, i64, i64, p]
        L.mi_block_scaled_fp8_gemm_ex.restype = c_int
        L.mi_block_scaled_fp8_gemm_ex.argtypes = [p, p, c_int, p, c_int, p, p, i64, i64, i64, p]
        L.mi_block_scaled_fp8_gemm_pair_ex.restype = c_int
        L.mi_block_scaled_fp8_gemm_pair_ex.argtypes = [p, p, c_int, c_int, p, p, p, i64, p, p, p, i64, i64, i64, p]
        L.mi_fused_normquant_gemm_pair.restype = c_int
        L.mi_fused_normquant_gemm_pair.argtypes = [
            p, i64, p, i64, p, p, ctypes.c_float, i64, i64, i64, c_int, p, p, p,
            c_int, p, p, p, i64, p, p, p, i64, p]
        L.mi_fused_normquant_gemm_pair_e8m0.restype = c_int
        L.mi_fused_normquant_gemm_pair_e8m0.argtypes = L.mi_fused_normquant_gemm_pair.argtypes
        L.mi_fused_normquant_gemm_pair_launches.restype = c_int
        L.mi_fused_normquant_gemm_pair_launches.argtypes = [i64, i64, i64, i64, i64]
        L.mi_gemm_capabilities.restype = ctypes.c_uint
        L.mi_gemm_capabilities.argtypes = []
        L.mi_preferred_weight_layout.restype = c_int
        L.mi_preferred_weight_layout.argtypes = [i64, i64]
        L.mi_relayout_weight.restype = c_int
        L.mi_relayout_weight.argtypes = [p, c_int, p, c_int, i64, i64, p]
        L.mi_negotiate_scale_layout.restype = c_int
        L.mi_negotiate_scale_layout.argtypes = [ctypes.POINTER(c_int), c_int]
        L.mi_init.restype = c_int
        L.mi_init.argtypes = []
        L.mi_status_string.restype = ctypes.c_char_p
        L.mi_status_string.argtypes = [c_int]
        _lib = L
    return _lib


def mi_init() -> None:
    """Prepare the current device (see mi_init in include/mi_normquant.h):
    call it before capturing calls of this library into a HIP graph."""
    _check("mi_init", lib().mi_init())


def mi_status_string(status: int) -> str:
    return lib().mi_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != MI_OK:
        raise MiError(fn, status, mi_status_string(status))


def _stream(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


E8M0_DTYPES = (torch.uint8, getattr(torch, "float8_e8m0fnu", torch.uint8))


def _u8(t: torch.Tensor) -> torch.Tensor:
    """An e8m0 scale tensor as uint8 bytes (float8_e8m0fnu is viewed)."""
    return t if t.dtype == torch.uint8 else t.view(torch.uint8)


def _rows(t: torch.Tensor, name: str, dtype: torch.dtype) -> int:
    """Row stride (elements) of a 2-D tensor with unit inner stride (checked
    for every row count: the kernels read each row as contiguous elements)."""
    if not isinstance(t, torch.Tensor) or t.dim() != 2 or t.dtype != dtype:
        raise ValueError(f"{name}: expected a 2-D {dtype} tensor, got "
                         f"{tuple(t.shape) if isinstance(t, torch.Tensor) else type(t)} "
                         f"{getattr(t, 'dtype', '')}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name}: inner stride must be 1, got {t.stride()}")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _vector(t, name: str, dtype: torch.dtype, n: int) -> None:
    """A contiguous 1-D-able tensor of exactly n elements of the given dtype
    (the RMSNorm weights)."""
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_contiguous() or t.numel() != n:
        raise ValueError(f"{name}: expected a contiguous {dtype} tensor of {n} elements, got "
                         f"{tuple(getattr(t, 'shape', ()))} {getattr(t, 'dtype', type(t))}")


def _output(t, name: str, dtypes, n: int) -> None:
    """A contiguous output buffer of at least n elements of one of dtypes."""
    if not isinstance(t, torch.Tensor) or t.dtype not in dtypes:
        raise ValueError(f"{name}: expected a tensor of {' / '.join(map(str, dtypes))}, got "
                         f"{getattr(t, 'dtype', type(t))}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: output must be contiguous, got strides {t.stride()}")
    if t.numel() < n:
        raise ValueError(f"{name}: output buffer too small ({t.numel()} < {n} elements)")


def _same_gpu(ref: torch.Tensor, ref_name: str, **tensors) -> None:
    """Every tensor on the GPU that ``ref`` is on: the library dereferences
    each pointer on that device (a host pointer there is a memory fault)."""
    if not ref.is_cuda:
        raise ValueError(f"{ref_name}: expected a GPU tensor, got one on {ref.device}")
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name}: on {t.device}, expected {ref.device} (the device of {ref_name})")


Q_DTYPES = (torch.uint8,) + ((torch.float8_e4m3fn,) if hasattr(torch, "float8_e4m3fn") else ())


def _dual_args(q, kv, gamma_q, gamma_kv, out_q, out_scale, out_kv, e8m0: bool, alloc: bool,
               devices: bool = True):
    """Checks of the dual norm-quant's operands, shared by the eager and
    prepared calls and the one-call step.  With ``alloc`` missing outputs
    are allocated on q's device.  Returns (q row stride, kv row stride, M,
    Nq, Nkv, out_q, out_scale (uint8 view for e8m0), out_kv)."""
    qs = _rows(q, "q", torch.bfloat16)
    ks = _rows(kv, "kv", torch.bfloat16)
    M, Nq = q.shape
    Nkv = kv.shape[1]
    if kv.shape[0] != M:
        raise ValueError(f"q and kv must have the same number of rows ({M} vs {kv.shape[0]})")
    if Nq % GROUP:
        raise ValueError(f"q width {Nq} is not a multiple of {GROUP}")
    _vector(gamma_q, "gamma_q", torch.bfloat16, Nq)
    _vector(gamma_kv, "gamma_kv", torch.bfloat16, Nkv)
    G = Nq // GROUP
    sdt = E8M0_DTYPES if e8m0 else (torch.float32,)
    if alloc:
        dev = q.device
        out_q = torch.empty((M, Nq), dtype=torch.uint8, device=dev) if out_q is None else out_q
        out_scale = torch.empty(M * G, dtype=sdt[0], device=dev) if out_scale is None else out_scale
        out_kv = torch.empty((M, Nkv), dtype=torch.bfloat16, device=dev) if out_kv is None else out_kv
    _output(out_q, "out_q", Q_DTYPES, M * Nq)
    _output(out_scale, "out_scale", sdt, M * G)
    _output(out_kv, "out_kv", (torch.bfloat16,), M * Nkv)
    if devices:
        _same_gpu(q, "q", kv=kv, gamma_q=gamma_q, gamma_kv=gamma_kv, out_q=out_q, out_scale=out_scale,
                  out_kv=out_kv)
    return qs, ks, M, Nq, Nkv, out_q, (_u8(out_scale) if e8m0 else out_scale), out_kv


def mi_fused_dual_rmsnorm_group_quant(q: torch.Tensor, kv: torch.Tensor,
                                      gamma_q: torch.Tensor, gamma_kv: torch.Tensor,
                                      eps: float, transpose_scale: bool,
                                      out_q: torch.Tensor | None = None,
                                      out_scale: torch.Tensor | None = None,
                                      out_kv: torch.Tensor | None = None):
    """Fused dual RMSNorm + per-1x128 FP8 group quant on the current stream.

    ``q`` [M, Nq] and ``kv`` [M, Nkv] are bf16 device tensors with unit inner
    stride (split views of one fused buffer are fine).  Returns
    ``(q_fp8, scale, kv_out)``: ``q_fp8`` uint8 e4m3fn codes [M, Nq],
    ``scale`` fp32 with logical shape [M, Nq/128] whose strides give the
    layout ((G, 1) row-major, or (1, M) when ``transpose_scale``), and
    ``kv_out`` bf16 [M, Nkv], contiguous."""
    qs, ks, M, Nq, Nkv, out_q, out_scale, out_kv = _dual_args(
        q, kv, gamma_q, gamma_kv, out_q, out_scale, out_kv, e8m0=False, alloc=True)
    G = Nq // GROUP
    status = lib().mi_fused_dual_rmsnorm_group_quant(
        _ptr(q), qs, _ptr(kv), ks, _ptr(gamma_q), _ptr(gamma_kv), ctypes.c_float(eps),
        M, Nq, Nkv, int(bool(transpose_scale)), _ptr(out_q), _ptr(out_scale), _ptr(out_kv),
        _stream(q))
    _check("mi_fused_dual_rmsnorm_group_quant", status)
    return out_q, _scale_view(out_scale, M, G, transpose_scale), out_kv


def mi_fused_dual_rmsnorm_group_quant_e8m0(q: torch.Tensor, kv: torch.Tensor,
                                           gamma_q: torch.Tensor, gamma_kv: torch.Tensor,
                                           eps: float, transpose_scale: bool,
                                           out_q: torch.Tensor | None = None,
                                           out_scale: torch.Tensor | None = None,
                                           out_kv: torch.Tensor | None = None):
    """As :func:`mi_fused_dual_rmsnorm_group_quant` with e8m0 (power-of-two)
    scales: ``scale`` is a uint8 tensor of exponent bytes with logical shape
    [M, Nq/128] and the requested layout."""
    qs, ks, M, Nq, Nkv, out_q, out_scale, out_kv = _dual_args(
        q, kv, gamma_q, gamma_kv, out_q, out_scale, out_kv, e8m0=True, alloc=True)
    G = Nq // GROUP
    status = lib().mi_fused_dual_rmsnorm_group_quant_e8m0(
        _ptr(q), qs, _ptr(kv), ks, _ptr(gamma_q), _ptr(gamma_kv), ctypes.c_float(eps),
        M, Nq, Nkv, int(bool(transpose_scale)), _ptr(out_q), _ptr(out_scale), _ptr(out_kv), _stream(q))
    _check("mi_fused_dual_rmsnorm_group_quant_e8m0", status)
    return out_q, _scale_view(out_scale, M, G, transpose_scale), out_kv


def _single_args(x, gamma, out_q, out_scale, normalize: bool, alloc: bool):
    """Checks of the single-input quantisations' operands (eager and
    prepared).  Returns (row stride, M, N, out_q, out_scale)."""
    xs = _rows(x, "x", torch.bfloat16)
    M, N = x.shape
    if N % GROUP:
        raise ValueError(f"x width {N} is not a multiple of {GROUP}")
    if normalize:
        _vector(gamma, "gamma", torch.bfloat16, N)
    G = N // GROUP
    if alloc:
        out_q = torch.empty((M, N), dtype=torch.uint8, device=x.device) if out_q is None else out_q
        out_scale = torch.empty(M * G, dtype=torch.float32, device=x.device) if out_scale is None else out_scale
    _output(out_q, "out_q", Q_DTYPES, M * N)
    _output(out_scale, "out_scale", (torch.float32,), M * G)
    _same_gpu(x, "x", gamma=gamma if normalize else None, out_q=out_q, out_scale=out_scale)
    return xs, M, N, out_q, out_scale


def _scale_view(out_scale: torch.Tensor, M: int, G: int, transpose_scale: bool) -> torch.Tensor:
    flat = out_scale.reshape(-1)[:M * G]
    return flat.as_strided((M, G), (1, M)) if transpose_scale else flat.view(M, G)


def mi_rmsnorm_group_quant(x: torch.Tensor, gamma: torch.Tensor, eps: float, transpose_scale: bool,
                           out_q: torch.Tensor | None = None, out_scale: torch.Tensor | None = None):
    """Single-input RMSNorm + per-1x128 FP8 group quant on the current
    stream.  ``x`` [M, N] bf16 with unit inner stride; returns ``(x_fp8,
    scale)`` laid out as in :func:`mi_fused_dual_rmsnorm_group_quant`."""
    xs, M, N, out_q, out_scale = _single_args(x, gamma, out_q, out_scale, normalize=True, alloc=True)
    status = lib().mi_rmsnorm_group_quant(_ptr(x), xs, _ptr(gamma), ctypes.c_float(eps), M, N,
                                          int(bool(transpose_scale)), _ptr(out_q), _ptr(out_scale), _stream(x))
    _check("mi_rmsnorm_group_quant", status)
    return out_q, _scale_view(out_scale, M, N // GROUP, transpose_scale)


def mi_group_quant_1x128(x: torch.Tensor, transpose_scale: bool,
                         out_q: torch.Tensor | None = None, out_scale: torch.Tensor | None = None):
    """Per-1x128 dynamic FP8 quant of a bf16 activation (no normalisation)
    on the current stream; returns ``(x_fp8, scale)``."""
    xs, M, N, out_q, out_scale = _single_args(x, None, out_q, out_scale, normalize=False, alloc=True)
    status = lib().mi_group_quant_1x128(_ptr(x), xs, M, N, int(bool(transpose_scale)), _ptr(out_q),
                                        _ptr(out_scale), _stream(x))
    _check("mi_group_quant_1x128", status)
    return out_q, _scale_view(out_scale, M, N // GROUP, transpose_scale)


def scale_is_transposed(a_scale: torch.Tensor) -> bool:
    """Layout of a [M, K/128] scale tensor, read from its strides: False for
    row-major (strides (K/128, 1)), True for column-major ((1, M)).  With one
    row or one column both layouts hold the same bytes (False).  Any other
    strides raise."""
    M, KB = a_scale.shape
    row = (KB == 1 or a_scale.stride(1) == 1) and (M == 1 or a_scale.stride(0) == KB)
    col = (M == 1 or a_scale.stride(0) == 1) and (KB == 1 or a_scale.stride(1) == M)
    if row:
        return False
    if col:
        return True
    raise ValueError(f"a_scale strides {a_scale.stride()} are neither row- nor column-major")


class TiledWeight:
    """An [N, K] e4m3fn weight in the MI_WEIGHT_TILED byte order (see
    include/mi_normquant.h): ``data`` is a flat uint8 device tensor of N*K
    bytes.  Only :func:`relayout_weight` makes one, so a weight cannot be
    relaid out twice through this binding (the relayout is a permutation,
    not an involution)."""

    def __init__(self, data: torch.Tensor, N: int, K: int):
        self.data, self.N, self.K = data, int(N), int(K)

    @property
    def shape(self):
        return (self.N, self.K)

    @property
    def device(self):
        return self.data.device


def weight_already_tiled(w) -> bool:
    return isinstance(w, TiledWeight)


def mi_gemm_capabilities() -> int:
    return int(lib().mi_gemm_capabilities())


def mi_preferred_weight_layout(N: int, K: int) -> int:
    return int(lib().mi_preferred_weight_layout(N, K))


def relayout_weight(w: torch.Tensor) -> TiledWeight:
    """Row-major uint8 [N, K] weight -> a new TiledWeight (on w's stream)."""
    if isinstance(w, TiledWeight):
        raise TypeError("weight is already tiled: relaying it out again would permute it twice")
    if w.dtype != torch.uint8 or w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w: expected a contiguous 2-D uint8 tensor")
    _same_gpu(w, "w")
    N, K = w.shape
    dst = torch.empty(N * K, dtype=torch.uint8, device=w.device)
    status = lib().mi_relayout_weight(_ptr(w), MI_WEIGHT_ROW_MAJOR, _ptr(dst), MI_WEIGHT_TILED, N, K, _stream(w))
    _check("mi_relayout_weight", status)
    return TiledWeight(dst, N, K)


def untile_weight(tw: TiledWeight) -> torch.Tensor:
    """TiledWeight -> a new row-major uint8 [N, K] tensor."""
    if not isinstance(tw, TiledWeight):
        raise TypeError("expected a TiledWeight")
    _same_gpu(tw.data, "tw.data")
    dst = torch.empty((tw.N, tw.K), dtype=torch.uint8, device=tw.device)
    status = lib().mi_relayout_weight(_ptr(tw.data), MI_WEIGHT_TILED, _ptr(dst), MI_WEIGHT_ROW_MAJOR, tw.N, tw.K,
                                      _stream(dst))
    _check("mi_relayout_weight", status)
    return dst


def _weight_arg(w):
    """(data tensor, layout, N, K) of a row-major tensor or a TiledWeight."""
    if isinstance(w, TiledWeight):
        return w.data, MI_WEIGHT_TILED, w.N, w.K
    if w.dtype != torch.uint8 or w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w: expected a contiguous 2-D uint8 tensor or a TiledWeight")
    return w, MI_WEIGHT_ROW_MAJOR, w.shape[0], w.shape[1]


def _check_gemm_operands(a, a_scale, w, w_scale):
    """Returns (M, N, K, weight data tensor, weight layout).  Scales are
    fp32, or e8m0 exponent bytes (uint8 / float8_e8m0fnu) for both."""
    e8m0 = a_scale.dtype in E8M0_DTYPES
    sdt = "e8m0 (uint8)" if e8m0 else torch.float32
    for name, t, ok in (("a", a, a.dtype == torch.uint8), ("w_scale", w_scale, (w_scale.dtype in E8M0_DTYPES) == e8m0
                                                              and (e8m0 or w_scale.dtype == torch.float32)),
                        ("a_scale", a_scale, e8m0 or a_scale.dtype == torch.float32)):
        if not ok or t.dim() != 2:
            raise ValueError(f"{name}: expected a 2-D tensor of {'uint8' if name == 'a' else sdt}")
    if not (a.is_contiguous() and w_scale.is_contiguous()):
        raise ValueError("a and w_scale must be contiguous")
    wd, wl, N, Kw = _weight_arg(w)
    M, K = a.shape
    if Kw != K or tuple(a_scale.shape) != (M, K // GROUP) or tuple(w_scale.shape) != (N // GROUP, K // GROUP):
        raise ValueError("shape mismatch between a, a_scale, w, w_scale")
    scale_is_transposed(a_scale)  # raises unless row- or column-major
    return M, N, K, wd, wl


def _gemm_out(out, M, N, device, name="out"):
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=device)
    if not isinstance(out, torch.Tensor) or out.dtype != torch.bfloat16 or not out.is_contiguous() or \
            tuple(out.shape) != (M, N):
        raise ValueError(f"{name} must be a contiguous bf16 [{M}, {N}] tensor")
    return out


def mi_block_scaled_fp8_gemm(a: torch.Tensor, a_scale: torch.Tensor, w, w_scale: torch.Tensor,
                             out: torch.Tensor | None = None,
                             a_scale_transposed: bool | None = None):
    """Block-scaled FP8 GEMM on the current stream: ``a`` uint8 [M, K],
    ``a_scale`` fp32 [M, K/128] (row- or column-major, read from its strides
    unless ``a_scale_transposed`` is given and agrees), ``w`` uint8 [N, K]
    (row-major) or a :class:`TiledWeight`, ``w_scale`` fp32 [N/128, K/128].
    Returns bf16 [M, N]."""
    M, N, K, wd, wl = _check_gemm_operands(a, a_scale, w, w_scale)
    layout = scale_is_transposed(a_scale)
    if a_scale_transposed is not None and M > 1 and bool(a_scale_transposed) != layout:
        raise ValueError("a_scale_transposed disagrees with the strides of a_scale")
    out = _gemm_out(out, M, N, a.device)
    _same_gpu(a, "a", a_scale=a_scale, w=wd, w_scale=w_scale, out=out)
    fn = "mi_block_scaled_fp8_gemm_e8m0" if a_scale.dtype in E8M0_DTYPES else "mi_block_scaled_fp8_gemm_ex"
    status = getattr(lib(), fn)(
        _ptr(a), _ptr(a_scale), int(layout), _ptr(wd), wl, _ptr(w_scale), _ptr(out), M, N, K, _stream(a))
    _check(fn, status)
    return out


def mi_block_scaled_fp8_gemm_pair(a: torch.Tensor, a_scale: torch.Tensor, w1, w1_scale: torch.Tensor,
                                  w2, w2_scale: torch.Tensor,
                                  out1: torch.Tensor | None = None,
                                  out2: torch.Tensor | None = None):
    """Both consumers of one pre-quantised pair on the current stream:
    returns (bf16 [M, N1], bf16 [M, N2]), each equal to
    mi_block_scaled_fp8_gemm(a, a_scale, w_i, w_i_scale).  Both weights in
    the same layout."""
    M, N1, K, wd1, wl1 = _check_gemm_operands(a, a_scale, w1, w1_scale)
    _, N2, _, wd2, wl2 = _check_gemm_operands(a, a_scale, w2, w2_scale)
    if wl1 != wl2:
        raise ValueError("both weights of a pair must have the same layout")
    out1 = _gemm_out(out1, M, N1, a.device, "out1")
    out2 = _gemm_out(out2, M, N2, a.device, "out2")
    _same_gpu(a, "a", a_scale=a_scale, w1=wd1, w1_scale=w1_scale, w2=wd2, w2_scale=w2_scale, out1=out1, out2=out2)
    fn = "mi_block_scaled_fp8_gemm_pair_e8m0" if a_scale.dtype in E8M0_DTYPES else "mi_block_scaled_fp8_gemm_pair_ex"
    status = getattr(lib(), fn)(
        _ptr(a), _ptr(a_scale), int(scale_is_transposed(a_scale)), wl1, _ptr(wd1), _ptr(w1_scale), _ptr(out1), N1,
        _ptr(wd2), _ptr(w2_scale), _ptr(out2), N2, M, K, _stream(a))
    _check(fn, status)
    return out1, out2


def _step_operands(q, kv, gamma_q, gamma_kv, w1, w1_scale, w2, w2_scale, out_q, out_scale, out_kv, alloc):
    """Checks of the one-call step (the dual norm-quant's, then both
    weights'); returns the norm-quant's marshalled operands and outputs, the
    scale type and (weight data, layout, N, scale) of both weights."""
    e8m0 = isinstance(w1_scale, torch.Tensor) and w1_scale.dtype in E8M0_DTYPES
    if out_scale is not None and isinstance(out_scale, torch.Tensor) and (out_scale.dtype in E8M0_DTYPES) != e8m0:
        raise ValueError("out_scale must have the weight scales' type")
    qs, ks, M, Nq, Nkv, out_q, out_scale, out_kv = _dual_args(
        q, kv, gamma_q, gamma_kv, out_q, out_scale, out_kv, e8m0=e8m0, alloc=alloc, devices=False)
    ws = []
    for name, w, w_scale in (("w1", w1, w1_scale), ("w2", w2, w2_scale)):
        wd, wl, N, K = _weight_arg(w)
        if K != Nq:
            raise ValueError(f"{name}: K must equal the q width {Nq}")
        ok_dtype = isinstance(w_scale, torch.Tensor) and (
            (w_scale.dtype in E8M0_DTYPES) if e8m0 else w_scale.dtype == torch.float32)
        if not ok_dtype or not w_scale.is_contiguous() or tuple(w_scale.shape) != (N // GROUP, K // GROUP):
            raise ValueError(f"{name}: scale must be contiguous {'e8m0' if e8m0 else 'fp32'} [N/128, K/128]"
                             " (both weights' scales of one type)")
        ws.append((wd, wl, N, w_scale if not e8m0 else _u8(w_scale)))
    if ws[0][1] != ws[1][1]:
        raise ValueError("both weights of a pair must have the same layout")
    _same_gpu(q, "q", kv=kv, gamma_q=gamma_q, gamma_kv=gamma_kv, out_q=out_q, out_scale=out_scale, out_kv=out_kv,
              w1=ws[0][0], w1_scale=ws[0][3], w2=ws[1][0], w2_scale=ws[1][3])
    return (qs, ks, M, Nq, Nkv, out_q, out_scale, out_kv), e8m0, ws


def mi_fused_normquant_gemm_pair(q: torch.Tensor, kv: torch.Tensor, gamma_q: torch.Tensor,
                                 gamma_kv: torch.Tensor, eps: float, transpose_scale: bool,
                                 w1, w1_scale: torch.Tensor, w2, w2_scale: torch.Tensor,
                                 out_q=None, out_scale=None, out_kv=None, out1=None, out2=None):
    """The decode step on the current stream: the fused dual norm-quant of
    (q, kv) and both block-scaled FP8 GEMMs of its output, in one launch
    where the shape allows.  Returns ``(q_fp8, scale, kv_out, out1, out2)``,
    bit-identical to mi_fused_dual_rmsnorm_group_quant followed by
    mi_block_scaled_fp8_gemm_pair.  With e8m0 weight scales (uint8 /
    float8_e8m0fnu) the step is the e8m0 one
    (mi_fused_dual_rmsnorm_group_quant_e8m0, then the e8m0 pair) and
    ``scale`` holds exponent bytes."""
    (qs, ks, M, Nq, Nkv, out_q, out_scale, out_kv), e8m0, ((wd1, wl, N1, ws1), (wd2, _, N2, ws2)) = \
        _step_operands(q, kv, gamma_q, gamma_kv, w1, w1_scale, w2, w2_scale, out_q, out_scale, out_kv, alloc=True)
    G = Nq // GROUP
    out1 = _gemm_out(out1, M, N1, q.device, "out1")
    out2 = _gemm_out(out2, M, N2, q.device, "out2")
    _same_gpu(q, "q", out1=out1, out2=out2)
    fn = "mi_fused_normquant_gemm_pair_e8m0" if e8m0 else "mi_fused_normquant_gemm_pair"
    status = getattr(lib(), fn)(
        _ptr(q), qs, _ptr(kv), ks, _ptr(gamma_q), _ptr(gamma_kv), ctypes.c_float(eps), M, Nq, Nkv,
        int(bool(transpose_scale)), _ptr(out_q), _ptr(out_scale), _ptr(out_kv),
        wl, _ptr(wd1), _ptr(ws1), _ptr(out1), N1, _ptr(wd2), _ptr(ws2), _ptr(out2), N2, _stream(q))
    _check(fn, status)
    return out_q, _scale_view(out_scale, M, G, transpose_scale), out_kv, out1, out2


def mi_fused_normquant_gemm_pair_launches(M: int, Nq: int, Nkv: int, N1: int, N2: int) -> int:
    """Kernel launches mi_fused_normquant_gemm_pair makes for these sizes (1
    for one launch, else 2 or 3: the norm-quant's plus the pair's; 0 for
    M == 0; -1 for sizes it rejects), aligned operands assumed."""
    return int(lib().mi_fused_normquant_gemm_pair_launches(M, Nq, Nkv, N1, N2))


def mi_negotiate_scale_layout(consumer_wants_transposed) -> bool | None:
    """True / False when every consumer wants column-major / row-major
    scales, None when they disagree (do not share one quantised pair)."""
    vals = [int(bool(v)) for v in consumer_wants_transposed]
    arr = (ctypes.c_int * max(len(vals), 1))(*vals)
    r = lib().mi_negotiate_scale_layout(arr, len(vals))
    return None if r < 0 else bool(r)


class PreparedCall:
    """One entry point with its arguments marshalled once: calling it
    enqueues the launch on torch's current stream of the tensors' device
    (so it can be captured into a HIP graph) and raises on a non-zero
    status.  The tensors must stay alive as long as the call is used."""

    def __init__(self, name: str, args: tuple, keep: tuple, device):
        self.name = name
        self._fn = getattr(lib(), name)
        self._args = args
        self._keep = keep
        self._device = device

    def __call__(self) -> None:
        st = self._fn(*self._args, ctypes.c_void_p(torch.cuda.current_stream(self._device).cuda_stream))
        if st != MI_OK:
            raise MiError(self.name, st, mi_status_string(st))


def prepare_fused_dual_rmsnorm_group_quant(q, kv, gamma_q, gamma_kv, eps, transpose_scale,
                                           out_q, out_scale, out_kv) -> PreparedCall:
    """Marshal the arguments of mi_fused_dual_rmsnorm_group_quant once (same
    checks as :func:`mi_fused_dual_rmsnorm_group_quant`; outputs required)."""
    qs, ks, M, Nq, Nkv, out_q, out_scale, out_kv = _dual_args(
        q, kv, gamma_q, gamma_kv, out_q, out_scale, out_kv, e8m0=False, alloc=False)
    args = (_ptr(q), qs, _ptr(kv), ks, _ptr(gamma_q), _ptr(gamma_kv), ctypes.c_float(eps),
            M, Nq, Nkv, int(bool(transpose_scale)), _ptr(out_q), _ptr(out_scale), _ptr(out_kv))
    return PreparedCall("mi_fused_dual_rmsnorm_group_quant", args,
                        (q, kv, gamma_q, gamma_kv, out_q, out_scale, out_kv), q.device)


def prepare_rmsnorm_group_quant(x, gamma, eps, transpose_scale, out_q, out_scale) -> PreparedCall:
    """Marshal the arguments of mi_rmsnorm_group_quant once (outputs required)."""
    xs, M, N, out_q, out_scale = _single_args(x, gamma, out_q, out_scale, normalize=True, alloc=False)
    args = (_ptr(x), xs, _ptr(gamma), ctypes.c_float(eps), M, N, int(bool(transpose_scale)), _ptr(out_q),
            _ptr(out_scale))
    return PreparedCall("mi_rmsnorm_group_quant", args, (x, gamma, out_q, out_scale), x.device)


def prepare_group_quant_1x128(x, transpose_scale, out_q, out_scale) -> PreparedCall:
    """Marshal the arguments of mi_group_quant_1x128 once (outputs required)."""
    xs, M, N, out_q, out_scale = _single_args(x, None, out_q, out_scale, normalize=False, alloc=False)
    args = (_ptr(x), xs, M, N, int(bool(transpose_scale)), _ptr(out_q), _ptr(out_scale))
    return PreparedCall("mi_group_quant_1x128", args, (x, out_q, out_scale), x.device)


def prepare_fused_dual_rmsnorm_group_quant_e8m0(q, kv, gamma_q, gamma_kv, eps, transpose_scale,
                                                out_q, out_scale, out_kv) -> PreparedCall:
    """Marshal the arguments of mi_fused_dual_rmsnorm_group_quant_e8m0 once."""
    qs, ks, M, Nq, Nkv, out_q, out_scale, out_kv = _dual_args(
        q, kv, gamma_q, gamma_kv, out_q, out_scale, out_kv, e8m0=True, alloc=False)
    args = (_ptr(q), qs, _ptr(kv), ks, _ptr(gamma_q), _ptr(gamma_kv), ctypes.c_float(eps),
            M, Nq, Nkv, int(bool(transpose_scale)), _ptr(out_q), _ptr(out_scale), _ptr(out_kv))
    return PreparedCall("mi_fused_dual_rmsnorm_group_quant_e8m0", args,
                        (q, kv, gamma_q, gamma_kv, out_q, out_scale, out_kv), q.device)


def prepare_block_scaled_fp8_gemm(a, a_scale, w, w_scale, out) -> PreparedCall:
    """Marshal the arguments of mi_block_scaled_fp8_gemm_ex (or its e8m0
    form) once; the As layout is read from the strides of ``a_scale`` ([M,
    K/128]), the weight layout from the type of ``w``."""
    M, N, K, wd, wl = _check_gemm_operands(a, a_scale, w, w_scale)
    if out is None:
        raise ValueError("out is required")
    out = _gemm_out(out, M, N, a.device)
    _same_gpu(a, "a", a_scale=a_scale, w=wd, w_scale=w_scale, out=out)
    args = (_ptr(a), _ptr(a_scale), int(scale_is_transposed(a_scale)), _ptr(wd), wl, _ptr(w_scale),
            _ptr(out), M, N, K)
    fn = "mi_block_scaled_fp8_gemm_e8m0" if a_scale.dtype in E8M0_DTYPES else "mi_block_scaled_fp8_gemm_ex"
    return PreparedCall(fn, args, (a, a_scale, wd, w_scale, out), a.device)


def prepare_block_scaled_fp8_gemm_pair(a, a_scale, w1, w1_scale, out1, w2, w2_scale, out2) -> PreparedCall:
    """Marshal the arguments of mi_block_scaled_fp8_gemm_pair_ex (or its
    e8m0 form) once."""
    M, N1, K, wd1, wl1 = _check_gemm_operands(a, a_scale, w1, w1_scale)
    _, N2, _, wd2, wl2 = _check_gemm_operands(a, a_scale, w2, w2_scale)
    if wl1 != wl2:
        raise ValueError("both weights of a pair must have the same layout")
    if out1 is None or out2 is None:
        raise ValueError("out1 and out2 are required")
    out1 = _gemm_out(out1, M, N1, a.device, "out1")
    out2 = _gemm_out(out2, M, N2, a.device, "out2")
    _same_gpu(a, "a", a_scale=a_scale, w1=wd1, w1_scale=w1_scale, w2=wd2, w2_scale=w2_scale, out1=out1, out2=out2)
    args = (_ptr(a), _ptr(a_scale), int(scale_is_transposed(a_scale)), wl1, _ptr(wd1), _ptr(w1_scale), _ptr(out1),
            N1, _ptr(wd2), _ptr(w2_scale), _ptr(out2), N2, M, K)
    fn = "mi_block_scaled_fp8_gemm_pair_e8m0" if a_scale.dtype in E8M0_DTYPES else "mi_block_scaled_fp8_gemm_pair_ex"
    return PreparedCall(fn, args, (a, a_scale, wd1, w1_scale, out1, wd2, w2_scale, out2), a.device)


def prepare_fused_normquant_gemm_pair(q, kv, gamma_q, gamma_kv, eps, transpose_scale, w1, w1_scale, w2, w2_scale,
                                      out_q, out_scale, out_kv, out1, out2) -> PreparedCall:
    """Marshal the arguments of mi_fused_normquant_gemm_pair (or its e8m0
    form, chosen by the weight scales' type) once (outputs required; the
    same checks as :func:`mi_fused_normquant_gemm_pair`)."""
    if out_q is None or out_scale is None or out_kv is None or out1 is None or out2 is None:
        raise ValueError("all five outputs are required")
    (qs, ks, M, Nq, Nkv, out_q, out_scale, out_kv), e8m0, ((wd1, wl, N1, ws1), (wd2, _, N2, ws2)) = \
        _step_operands(q, kv, gamma_q, gamma_kv, w1, w1_scale, w2, w2_scale, out_q, out_scale, out_kv, alloc=False)
    out1 = _gemm_out(out1, M, N1, q.device, "out1")
    out2 = _gemm_out(out2, M, N2, q.device, "out2")
    _same_gpu(q, "q", out1=out1, out2=out2)
    args = (_ptr(q), qs, _ptr(kv), ks, _ptr(gamma_q), _ptr(gamma_kv), ctypes.c_float(eps), M, Nq, Nkv,
            int(bool(transpose_scale)), _ptr(out_q), _ptr(out_scale), _ptr(out_kv),
            wl, _ptr(wd1), _ptr(ws1), _ptr(out1), N1, _ptr(wd2), _ptr(ws2), _ptr(out2), N2)
    fn = "mi_fused_normquant_gemm_pair_e8m0" if e8m0 else "mi_fused_normquant_gemm_pair"
    return PreparedCall(fn, args,
                        (q, kv, gamma_q, gamma_kv, wd1, ws1, wd2, ws2, out_q, out_scale, out_kv, out1, out2),
                        q.device)
