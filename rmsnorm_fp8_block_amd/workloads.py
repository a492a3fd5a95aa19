"""Seeded synthetic inputs shaped like the MLA decode and prefill workloads.

This module holds none of the method's arithmetic.  It draws numbers with
numpy's PCG64 generator and stores them in the input formats the operation
takes: bf16 bit patterns (rounded by torch's CPU ``float32 -> bfloat16``
cast) and, for the GEMM weights, fp8 e4m3fn codes with fp32 128x128 block
scales (torch's CPU ``float8_e4m3fn`` cast).  The same bytes are handed to the
HIP library and to the CPU oracle.

Shapes follow DeepSeek-V4's MLA latents as the pages describe them
(vLLM PR #53540, "Purpose": a q-lora latent and a kv latent split from one
fused projection): Nq = 1536, Nkv = 512, one row per token, a 128-element
quantisation group.  Values: N(0, 1) activations, gammas 1 + N(0, 0.1),
eps = 1e-6.  The end-to-end benchmarks and the accuracy eval the pages run
(SA InferenceX 8k1k, GSM8K) are not available here; these inputs stand in for
the activations of those runs.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

NQ = 1536            # q-lora rank
NKV = 512            # kv latent width
WIDTH = NQ + NKV     # width of the fused projection buffer
GROUP = 128          # quantisation group (1 x 128)
EPS = 1e-6
GAMMA_SEED = 100

W_A_SHAPE = (24576, 1536)   # attention wq_b
W_B_SHAPE = (8192, 1536)    # indexer wq_b
W_A_SEED = 11
W_B_SEED = 12


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def gammas(nq: int = NQ, nkv: int = NKV, seed: int = GAMMA_SEED):
    r = rng(seed)
    gq = np.float32(1.0) + np.float32(0.1) * r.standard_normal(nq, dtype=np.float32)
    gk = np.float32(1.0) + np.float32(0.1) * r.standard_normal(nkv, dtype=np.float32)
    return f32_to_bf16_bits(gq), f32_to_bf16_bits(gk)


@dataclass
class NormQuantCase:
    """One input of the fused norm-quant.  ``q`` and ``kv`` are 2-D uint16
    views (unit inner stride; the row stride may exceed the width when they
    are split views of one fused buffer ``buffer``)."""
    name: str
    q: np.ndarray
    kv: np.ndarray
    gamma_q: np.ndarray
    gamma_kv: np.ndarray
    eps: float = EPS
    layouts: tuple = (0,)
    buffer: np.ndarray | None = None
    notes: dict = field(default_factory=dict)

    @property
    def M(self) -> int:
        return self.q.shape[0]


def _normal_bf16(shape, seed: int) -> np.ndarray:
    return f32_to_bf16_bits(rng(seed).standard_normal(shape, dtype=np.float32))


def split_views(buf: np.ndarray, nq: int = NQ):
    """q = columns [0, nq), kv = the rest, as views sharing ``buf``'s rows."""
    return buf[:, :nq], buf[:, nq:]


def decode_single(seed: int = 1) -> NormQuantCase:
    """Single-token decode: separate contiguous q [1,1536] and kv [1,512]."""
    r = rng(seed)
    q = f32_to_bf16_bits(r.standard_normal((1, NQ), dtype=np.float32))
    kv = f32_to_bf16_bits(r.standard_normal((1, NKV), dtype=np.float32))
    gq, gk = gammas()
    return NormQuantCase("decode_M1", q, kv, gq, gk, layouts=(0, 1))


def strided_batch(M: int = 64, seed: int = 2) -> NormQuantCase:
    """Decode batch: q and kv are strided split views of one [M, 2048] buffer."""
    buf = _normal_bf16((M, WIDTH), seed)
    q, kv = split_views(buf)
    gq, gk = gammas()
    return NormQuantCase(f"strided_M{M}", q, kv, gq, gk, layouts=(0,), buffer=buf)


def outlier_stress(M: int = 256, seed: int = 3, frac: float = 0.01,
                   mult: float = 50.0) -> NormQuantCase:
    """N(0,1) with a Bernoulli(frac) subset of elements multiplied by ``mult``
    (in fp32, before the bf16 rounding) and, in every row m, the q group
    (m mod G) set to zero."""
    r = rng(seed)
    G = NQ // GROUP
    q32 = r.standard_normal((M, NQ), dtype=np.float32)
    kv32 = r.standard_normal((M, NKV), dtype=np.float32)
    q32[r.random((M, NQ)) < frac] *= np.float32(mult)
    kv32[r.random((M, NKV)) < frac] *= np.float32(mult)
    for m in range(M):
        g = m % G
        q32[m, g * GROUP:(g + 1) * GROUP] = 0.0
    gq, gk = gammas()
    return NormQuantCase(f"outliers_M{M}", f32_to_bf16_bits(q32), f32_to_bf16_bits(kv32),
                         gq, gk, layouts=(1,), notes={"zero_group": "m % 12"})


def prefill(M: int = 8192, seed: int = 4) -> NormQuantCase:
    """Prefill: strided split views of an [M, 2048] buffer, both scale layouts."""
    buf = _normal_bf16((M, WIDTH), seed)
    q, kv = split_views(buf)
    gq, gk = gammas()
    return NormQuantCase(f"prefill_M{M}", q, kv, gq, gk, layouts=(0, 1), buffer=buf)


def producer_activations(M: int, seed: int = 5, rows: int = 256) -> NormQuantCase:
    """The first M rows of one seeded [256, 2048] fused buffer (split views)."""
    assert 1 <= M <= rows
    buf = _normal_bf16((rows, WIDTH), seed)[:M]
    q, kv = split_views(buf)
    gq, gk = gammas()
    return NormQuantCase(f"producer_M{M}", q, kv, gq, gk, layouts=(0, 1), buffer=buf)


def single_input(M: int, N: int = NQ, seed: int = 6, pad: int = 0, frac: float = 0.01,
                 mult: float = 50.0):
    """Input of the single-input quantisations: a [M, N] bf16 view of a
    [M, N + pad] buffer (pad > 0: a strided view, like a column slice of a
    wider projection output), N(0,1) with a Bernoulli(frac) subset scaled by
    ``mult`` and, in every row m, the group (m mod G) set to zero; plus a
    seeded bf16 gamma [N] near 1.  Returns (x, gamma)."""
    r = rng(seed)
    G = N // GROUP
    x32 = r.standard_normal((M, N + pad), dtype=np.float32)
    x32[r.random((M, N + pad)) < frac] *= np.float32(mult)
    for m in range(M):
        g = m % G
        x32[m, g * GROUP:(g + 1) * GROUP] = 0.0
    gamma = f32_to_bf16_bits((1.0 + 0.1 * r.standard_normal(N)).astype(np.float32))
    return f32_to_bf16_bits(x32)[:, :N], gamma


@dataclass
class BlockFp8Weight:
    """A weight [N, K] as e4m3fn codes plus fp32 scales [N/128, K/128]
    (dequantised value = dec(code) * scale of its 128x128 block)."""
    codes: np.ndarray   # uint8 [N, K]
    scale: np.ndarray   # float32 [N/128, K/128]

    @property
    def shape(self):
        return self.codes.shape


def block_fp8_weight(N: int, K: int, seed: int, std: float = 0.02) -> BlockFp8Weight:
    """Checkpoint-style fp8 weight: W ~ N(0, std) in fp32, one fp32 scale per
    128x128 block (block amax / 448, floored at 1e-12), codes = torch's
    float8_e4m3fn cast of W / scale (clamped to +-448 first)."""
    assert N % GROUP == 0 and K % GROUP == 0
    w = torch.from_numpy(rng(seed).standard_normal((N, K), dtype=np.float32)) * std
    blocks = w.view(N // GROUP, GROUP, K // GROUP, GROUP)
    amax = blocks.abs().amax(dim=(1, 3))
    scale = torch.clamp(amax / 448.0, min=1e-12).to(torch.float32)
    codes = (blocks / scale[:, None, :, None]).clamp(-448.0, 448.0)
    codes = codes.reshape(N, K).to(torch.float8_e4m3fn).view(torch.uint8)
    return BlockFp8Weight(codes.numpy().copy(), scale.numpy().copy())


@dataclass
class BlockFp8WeightE8m0:
    """A weight [N, K] as e4m3fn codes plus e8m0 block scales [N/128, K/128]
    (exponent bytes; dequantised value = dec(code) * 2^(byte - 127))."""
    codes: np.ndarray   # uint8 [N, K]
    scale: np.ndarray   # uint8 [N/128, K/128]

    @property
    def shape(self):
        return self.codes.shape


def block_fp8_weight_e8m0(N: int, K: int, seed: int, std: float = 0.02) -> BlockFp8WeightE8m0:
    """Checkpoint-style fp8 weight with power-of-two block scales: the same
    N(0, std) draw as block_fp8_weight, each 128x128 block scaled by 2^e, the
    smallest power of two not below block amax / 448 (floored at 1e-12),
    codes = torch's float8_e4m3fn cast of W * 2^-e (exact power-of-two
    scaling, |.| <= 448)."""
    assert N % GROUP == 0 and K % GROUP == 0
    w = torch.from_numpy(rng(seed).standard_normal((N, K), dtype=np.float32)) * std
    blocks = w.view(N // GROUP, GROUP, K // GROUP, GROUP).double()
    t = torch.clamp(blocks.abs().amax(dim=(1, 3)) / 448.0, min=float(np.float32(1e-12)))
    m, ex = torch.frexp(t)                      # t = m * 2^ex, m in [0.5, 1)
    e = torch.where(m == 0.5, ex - 1, ex)
    codes = torch.ldexp(blocks, -e[:, None, :, None].double()).clamp(-448.0, 448.0).float()
    codes = codes.reshape(N, K).to(torch.float8_e4m3fn).view(torch.uint8)
    return BlockFp8WeightE8m0(codes.numpy().copy(), (e + 127).to(torch.uint8).numpy().copy())
