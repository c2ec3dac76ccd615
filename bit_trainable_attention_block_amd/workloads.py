"""Seeded synthetic workloads for the SageBwd attention path.

This module is the only code shared by the GPU path's tests/benchmark and the
CPU oracle. It holds the five shape configurations and the seeded input
recipe, nothing of the attention method's arithmetic.

Input recipe (all tensors are laid out [B, H, N, D], row-major):

* ``numpy.random.Generator(PCG64(seed))`` with
  ``seed = 1000 * config + 10 * variant + tensor`` where tensor is
  Q=0, K=1, V=2, dO=3, K-offset=4 and variant is the sigma index of the sigma
  sweep (0 elsewhere).
* Draw float32 N(0, 1) and multiply by sigma where the workload states one.
* Where the workload uses QK-norm (SageBwd paper, preliminaries on QK-norm:
  per-token RMS normalisation of Q and K with a unit gain), each token vector
  x becomes x / sqrt(mean_c x^2 + 1e-6), computed in float64 and rounded once
  to float32.  K then receives a per-(b, h, channel) offset drawn from
  N(0, offset_sigma^2), shared by every token, to exercise K-smoothing.
* The result is rounded once (round-to-nearest-even) to the I/O dtype
  (fp16 or bf16).  Consumers get both the raw 16-bit patterns (what the GPU
  reads) and the exact values of those patterns as float32 arrays (what the
  oracle reads), so both sides see identical numbers.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np

FP16 = 0
BF16 = 1

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3, "koff": 4, "qoff": 5}


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload shape plus the method's switches."""

    name: str
    index: int            # 1-based workload number used in the seed
    B: int
    H: int
    N: int
    D: int
    dtype: int            # FP16 or BF16
    bq: int               # query block (rows per Q / dO quantisation block)
    bkv: int              # key/value block (rows per K / V quantisation block)
    causal: bool
    k_smooth: bool = True
    q_smooth: bool = False
    sigma: float = 1.0    # sigma of Q and K draws
    variant: int = 0      # sigma index (sigma sweep) or 0
    qk_norm: bool = False
    k_offset_sigma: float = 0.0
    q_offset_sigma: float = 0.0  # per-(b,h,channel) offset of Q, shared by all tokens
    dp_int8: bool = False # ablation: dP from INT8 codes (the method keeps it 16-bit)
    p_static: bool = False  # ablation: static forward P scale 1/127 (the method: per token)
    qk_norm_fused: bool = False  # QK-norm applied by sage_quantize (not by the generator)
    fp8: bool = False            # variant: E4M3 codes in place of INT8

    @property
    def sm_scale(self) -> float:
        return float(1.0 / np.sqrt(self.D))

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    @property
    def elements(self) -> int:
        return self.B * self.H * self.N * self.D

    def attention_ops(self) -> Tuple[float, float]:
        """(fwd, bwd) attention operation counts in the FlashAttention
        convention: fwd 4*B*H*N^2*D, bwd 10*B*H*N^2*D, halved when causal."""
        base = float(self.B * self.H) * self.N * self.N * self.D
        f = 0.5 if self.causal else 1.0
        return 4.0 * base * f, 10.0 * base * f


SIGMAS = (1.0, 3.0, 5.0, 8.0, 10.0)

# The five workloads.  Tiny (1) is the oracle-sized case; (2) d=64 both
# causal settings; (3) d=128 N=8K causal QK-normed (the headline workload);
# (4) the sigma sweep; (5) long context with optional Q-smoothing.
C1 = Config("tiny", 1, 1, 1, 128, 64, FP16, 64, 64, causal=False)
C2 = Config("d64_n2k", 2, 4, 16, 2048, 64, BF16, 128, 64, causal=False)
C2_CAUSAL = C2.replace(name="d64_n2k_causal", causal=True)
C3 = Config("d128_n8k_causal_qknorm", 3, 2, 16, 8192, 128, BF16, 128, 64, causal=True,
            qk_norm=True, k_offset_sigma=2.0)
C4 = tuple(Config(f"sigma{int(s)}_d128_n4k", 4, 1, 32, 4096, 128, BF16, 128, 64, causal=False,
                  sigma=s, variant=vi) for vi, s in enumerate(SIGMAS))
C5 = Config("long_n32k_causal_qknorm", 5, 1, 8, 32768, 128, BF16, 128, 64, causal=True,
            qk_norm=True, k_offset_sigma=1.0)
C5_QSMOOTH = C5.replace(name="long_n32k_causal_qknorm_qsmooth", q_smooth=True)
# the d=128 N=8K workload with the INT8-dP ablation (not the method)
C3_DPINT8 = C3.replace(name="d128_n8k_causal_qknorm_dpint8", dp_int8=True)
# ... and with the static forward P scale (not the method)
C3_PSTATIC = C3.replace(name="d128_n8k_causal_qknorm_pstatic", p_static=True)
# ... and with raw inputs, QK-norm applied by sage_quantize instead of the generator
C3_QKNORM_FUSED = C3.replace(name="d128_n8k_causal_qknorm_fused", qk_norm=False, qk_norm_fused=True)
# E4M3 variant of the same workload (not the method)
C3_FP8 = C3.replace(name="d128_n8k_causal_qknorm_fp8", fp8=True)

ALL = {c.name: c for c in (C1, C2, C3, C5)}


def _rng(cfg: Config, tensor: str) -> np.random.Generator:
    seed = 1000 * cfg.index + 10 * cfg.variant + TENSOR_IDS[tensor]
    return np.random.Generator(np.random.PCG64(seed))


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bits_to_float32(bits: np.ndarray, dtype: int) -> np.ndarray:
    """Exact float32 values of fp16 / bf16 bit patterns."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32)
    return bits.view(np.float16).astype(np.float32)


def to_io_bits(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == BF16:
        return round_to_bf16_bits(x)
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def _qk_norm(x: np.ndarray) -> np.ndarray:
    x64 = x.astype(np.float64)
    rms = np.sqrt(np.mean(x64 * x64, axis=-1, keepdims=True) + 1e-6)
    return (x64 / rms).astype(np.float32)


def generate(cfg: Config, heads: Optional[Tuple[int, int]] = None) -> Dict[str, Dict[str, np.ndarray]]:
    """Return {"q"|"k"|"v"|"do": {"bits": uint16[B,H,N,D], "f32": float32[B,H,N,D]}}.

    ``heads`` = (b, h) restricts the output to one head ([1,1,N,D]) while
    drawing exactly the same numbers as the full tensor would hold there.
    """
    shape = (cfg.B, cfg.H, cfg.N, cfg.D)
    out = {}
    for name in ("q", "k", "v", "do"):
        x = _rng(cfg, name).standard_normal(shape, dtype=np.float32)
        if name in ("q", "k") and cfg.sigma != 1.0:
            x = (x * np.float32(cfg.sigma)).astype(np.float32)
        if name in ("q", "k") and cfg.qk_norm:
            x = _qk_norm(x)
        if name == "k" and cfg.k_offset_sigma:
            off = _rng(cfg, "koff").standard_normal((cfg.B, cfg.H, 1, cfg.D), dtype=np.float32)
            x = (x + off * np.float32(cfg.k_offset_sigma)).astype(np.float32)
        if name == "q" and cfg.q_offset_sigma:
            off = _rng(cfg, "qoff").standard_normal((cfg.B, cfg.H, 1, cfg.D), dtype=np.float32)
            x = (x + off * np.float32(cfg.q_offset_sigma)).astype(np.float32)
        if heads is not None:
            b, h = heads
            x = x[b:b + 1, h:h + 1]
        bits = to_io_bits(x, cfg.dtype)
        out[name] = {"bits": np.ascontiguousarray(bits), "f32": bits_to_float32(bits, cfg.dtype)}
    return out
