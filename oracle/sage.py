"""SageBwd INT8 attention, step by step, on the CPU.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): the tests, the smoke check
and the benchmark's CPU-baseline leg may call this; the GPU library never does.

What is computed, and where the pages define it
-----------------------------------------------
* SageBwd paper summary (paper.rainbus.top, "method step details"): the
  forward steps (1)-(5) and backward steps (1)-(7) that this module follows
  in order; K-smoothing on and Q-smoothing off by default.
* SageBwd paper summary, prerequisites "INT8 quantisation": scale
  delta_X = max|X| / 127 and codes round(X / delta_X); per-block granularity
  aligned with the FlashAttention tiles.
* SageAttention3 write-up, Eq. 1 (online softmax: running max m and running
  sum l, initialised to -inf and 0, rescaled by exp(m_old - m_new)), Eq. 7
  (INT8 per-block quantisation), Eq. 8 (INT8 logits and the per-token P scale
  s_P = exp(rowmax(S_ij) - m_ij) / 127) and Eq. 9 with its INT8 backward
  updates (dV, dP kept in 16-bit, dS = P o (dP - D), dQ, dK).
* SageBwd paper summary, prerequisites "K-smoothing and Q-smoothing", and
  paperlayer section 6: K is centred by its token mean at kernel entry with no
  backward change; Q is centred per query block, the low-rank term
  mu_Qi K^T is added to the logits in high precision and dK gains the bias
  (dS^T 1) mu_Q^T.

Numeric model (the readings taken where the pages leave a choice open)
----------------------------------------------------------------------
* Everything is float64 except where a value is stored by the method or
  decides an integer code; there the kernel's precision, IEEE float32 with
  round-to-nearest-even, is used:
    - mu_K = f32(sum_n K[n] / N) (sum in float64); K_sm = f32(K - mu_K);
      the same per query block for mu_Q and Q_sm;
    - a block's scale s = f32(max|X| / 127) (correctly rounded float32
      division), codes = clamp(rint(f32(X / s)), -127, 127), rint being
      round-half-to-even; a block whose max is 0 gets s = 0 and zero codes;
    - the forward P codes: s_P = f32(f32(exp(rm - m_new)) / 127) and
      codes = clamp(rint(f32(f32(P~) / s_P)), 0, 127); a row with no visible
      key in the tile gets s_P = 0 and zero codes;
    - the backward P and dS codes: one scale per (query block, key block)
      tile, computed as above from f32(P) and f32(dS);
    - stored outputs: O rounded to the I/O dtype, L and delta to float32.
* The logits carry the 1/sqrt(D) softmax scale (S = Q K^T / sqrt(d), as the
  prerequisites state); by the chain rule dQ and dK are multiplied by it.
* The running sum l adds the unquantised P~ (Eq. 1); the quantised codes only
  feed the P V product.
* L is the logsumexp of the logits the method forms, i.e. with K-smoothing
  of Q (K - mu_K)^T * scale; it differs from the unsmoothed logsumexp by
  -scale * q . mu_K per row, while O is unchanged.  The backward recomputes
  P = exp(S - L) from the same smoothed logits.
* Causal masking is top-left aligned (key n visible to query r iff n <= r);
  tiles whose keys all lie after the block's last query are skipped.
* delta = rowsum(dO o O) uses the stored (rounded) O.
* dP = dO V^T uses the 16-bit input values exactly, summed in float64.
* QK-norm fused into the preprocessing (Shape.qk_norm, for training use; the
  SageBwd paper summary trains with QK-norm, prerequisites "QK-norm"): rows
  of Q and K are scaled by r = f32(1/sqrt(mean(x^2) + 1e-6)) (mean exact in
  float64) and rounded to float32 before smoothing and quantisation; the
  gradients w.r.t. the inputs are r * (dX_n - X_n * mean(dX_n o X_n)).
* Ablation switch Shape.p_static (not the method; the SageAttention3 write-up
  names the static per-block scale 1/127 beside Eq. 8 as less accurate):
  the forward's P codes use s_P = 1/127 and P^ = P~ / s_P, P~ taken against
  the running maximum.
* Ablation switch Shape.dp_int8 (not the method; the SageAttention3 write-up,
  Table 1c, compares dO V^T in INT8 against FP16): dP = (dO^_i V^_j^T) *
  s_dO,i * s_V,j from the same per-block codes the other products use.

* Variant switch Shape.fp8 (not the method, which is INT8; the
  SageAttention3 write-up compares INT8 and FP8 SageBwd gradients in its
  INT8-versus-FP8 training table): every quantised operand takes E4M3 codes
  (OCP 8-bit float: 4 exponent bits with bias 7, 3 mantissa bits, no
  infinities, largest finite 448) in place of INT8.  The scales use 448 in
  place of 127 (s = f32(max|X| / 448); forward s_P = f32(f32(exp(rm - m)) /
  448)) and a code is the float32 quotient rounded to the nearest E4M3 value,
  ties to even.  The products are sums of the decoded codes, as for INT8.

Quantisation-off mode (quant=False): every quantise/dequantise pair becomes
the identity (codes = values, scales = 1), nothing is rounded, and the result
must equal full-precision attention (oracle.fpa) to float64 rounding.

Tensors are per head, [N, D], as float arrays holding the exact input values.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, Optional

import numpy as np

F32 = np.float32
F64 = np.float64


def r32(x):
    """Round to IEEE float32 (round-to-nearest-even) and return as float64."""
    return np.asarray(x, dtype=F64).astype(F32).astype(F64)


def round_io(x, dtype: int):
    """Round float64 values to the I/O dtype (0 = fp16, 1 = bf16) with
    round-to-nearest-even, directly from float64 (no intermediate float32)."""
    x = np.asarray(x, dtype=F64)
    sig_bits, min_q, max_finite = (8, -133, 3.3895313892515355e38) if dtype == 1 else (11, -24, 65504.0)
    out = np.zeros_like(x)
    nz = x != 0
    _, e = np.frexp(x[nz])                       # x = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e - sig_bits, min_q).astype(F64)
    step = np.exp2(q)
    out[nz] = np.rint(x[nz] / step) * step       # exact scaling by powers of two
    big = np.abs(out) > max_finite
    out[big] = np.sign(out[big]) * np.inf
    return out


@dataclasses.dataclass
class Shape:
    """The switches of one call: quantisation blocks and method options."""

    N: int
    D: int
    bq: int
    bkv: int
    causal: bool = False
    k_smooth: bool = True
    q_smooth: bool = False
    dtype: int = 1
    sm_scale: Optional[float] = None
    # Ablation, not the method: dP = dO V^T from the per-block INT8 codes of
    # dO (bq-row blocks) and V (bkv-row blocks) instead of the 16-bit values
    # (SageAttention3 write-up, Table 1c compares the two).
    dp_int8: bool = False
    # Ablation, not the method: the forward's P codes with the static scale
    # s_P = 1/127 against the running maximum, P^ = P~ / s_P (the alternative
    # the SageAttention3 write-up names beside Eq. 8 and finds less accurate)
    p_static: bool = False
    # QK-norm fused into the preprocessing (training use): per-token RMS
    # normalisation of Q and K with unit gain before smoothing and
    # quantisation; the gradients then pass back through it
    qk_norm: bool = False
    # Variant, not the method: E4M3 codes with 448 in place of INT8 and 127
    # (the SageAttention3 write-up's INT8-versus-FP8 training comparison)
    fp8: bool = False

    def __post_init__(self):
        if self.fp8 and (self.dp_int8 or self.p_static):
            raise ValueError("the E4M3 variant takes neither the INT8 dP ablation nor the static P scale")

    @property
    def qmax(self) -> int:
        """Largest code magnitude: 127 (INT8) or 448 (E4M3)."""
        return 448 if self.fp8 else 127

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.D)) if self.sm_scale is None else float(self.sm_scale)

    @property
    def Tm(self) -> int:
        return self.N // self.bq

    @property
    def Tn(self) -> int:
        return self.N // self.bkv

    @staticmethod
    def of(cfg) -> "Shape":
        """Build from a workload description (anything with the same fields)."""
        return Shape(N=cfg.N, D=cfg.D, bq=cfg.bq, bkv=cfg.bkv, causal=bool(cfg.causal),
                     k_smooth=bool(cfg.k_smooth), q_smooth=bool(cfg.q_smooth), dtype=int(cfg.dtype),
                     dp_int8=bool(getattr(cfg, "dp_int8", False)), p_static=bool(getattr(cfg, "p_static", False)),
                     qk_norm=bool(getattr(cfg, "qk_norm_fused", False)), fp8=bool(getattr(cfg, "fp8", False)))


# ---------------------------------------------------------------------------
# Per-block INT8 quantisation (prerequisites "INT8 quantisation"; SA3 Eq. 7)
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0


def e4m3_round(x):
    """Nearest E4M3 value of each element (OCP 8-bit float: sign, 4 exponent
    bits with bias 7, 3 mantissa bits; subnormals below 2^-6 in steps of 2^-9;
    no infinities, largest finite 448), ties to even; magnitudes beyond 448
    saturate to 448.  Returns float64."""
    x = np.asarray(x, dtype=F64)
    out = np.zeros_like(x)
    nz = x != 0
    _, e = np.frexp(x[nz])                   # |x| = m 2^e, 0.5 <= m < 1: leading bit 2^(e-1)
    step = np.exp2(np.maximum(e - 1, -6) - 3)  # value spacing in x's binade (subnormal: 2^-9)
    out[nz] = np.rint(x[nz] / step) * step   # exact scaling by a power of two, half-even
    return np.clip(out, -E4M3_MAX, E4M3_MAX)


def e4m3_bits(v):
    """The byte encoding of E4M3 values (sign bit 7, exponent bits 6-3, mantissa
    bits 2-0); v must hold representable values (e.g. from e4m3_round)."""
    v = np.asarray(v, dtype=F64)
    a = np.abs(v)
    sign = np.signbit(v).astype(np.uint8) << 7
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    normal = a >= 2.0 ** -6
    ex = np.where(normal, e - 1 + 7, 0)
    man = np.where(normal, a / np.exp2(e - 1.0) * 8 - 8, a / 2.0 ** -9)
    return (sign | (ex.astype(np.uint8) << 3) | man.astype(np.uint8)).astype(np.uint8)


def round_codes(x, fp8: bool, lo: float):
    """Codes from scaled float32 quotients: INT8 rint clamped to [lo, 127]
    (half-even), or E4M3 rounding (whose range ends at 448)."""
    if fp8:
        return np.maximum(e4m3_round(x), lo)
    return np.clip(np.rint(x), lo, 127)


def quantize_block(X, quant=True, fp8=False):
    """delta = max|X| / 127, codes = round(X / delta) (E4M3: 448 and the
    nearest E4M3 value).

    X holds float32-representable values.  Returns (codes as float64 values,
    scale).  Quantisation off: (X, 1.0)."""
    X = np.asarray(X, dtype=F64)
    if not quant:
        return X.copy(), 1.0
    qmax = 448 if fp8 else 127
    x32 = X.astype(F32)
    a = np.max(np.abs(x32)) if x32.size else F32(0)
    if a == 0:
        return np.zeros_like(X), 0.0
    s = F32(a) / F32(qmax)                                   # float32 / float32: correctly rounded
    codes = round_codes((x32 / s).astype(F64), fp8, -qmax)   # float32 division, then the code rounding
    return codes.astype(F64), float(s)


@dataclasses.dataclass
class Quantized:
    """Result of the preprocessing step for one head."""

    Qc: np.ndarray      # [N, D] codes of Q_sm (integer-valued float64; values when quant off)
    sQ: np.ndarray      # [Tm]
    Kc: np.ndarray      # [N, D]
    sK: np.ndarray      # [Tn]
    Vc: np.ndarray      # [N, D]
    sV: np.ndarray      # [Tn]
    mu_k: np.ndarray    # [D]  (zeros when K-smoothing is off)
    mu_q: np.ndarray    # [Tm, D] (zeros when Q-smoothing is off)
    K_sm: np.ndarray    # [N, D] smoothed, unquantised K (for the Q-smoothing bias)
    rq: Optional[np.ndarray] = None   # [N] inverse RMS of each Q row (QK-norm), else None
    rk: Optional[np.ndarray] = None   # [N] the same for K


QK_NORM_EPS = 1e-6


def rms_norm(X, quant=True):
    """QK-norm (SageBwd paper summary, prerequisites "QK-norm"; unit gain):
    per row r = 1 / sqrt(mean(x^2) + eps) and X_n = X * r.  The mean is exact
    in float64; with quantisation on, r is rounded once to float32 and X_n
    rounded to float32 (the values the codes are taken from)."""
    X = np.asarray(X, dtype=F64)
    ms = np.sum(X * X, axis=1) / X.shape[1]
    r = 1.0 / np.sqrt(ms + QK_NORM_EPS)
    if quant:
        r = r32(r)
        return r32(X * r[:, None]), r
    return X * r[:, None], r


def rms_norm_backward(X, r, dXn, quant=True):
    """Gradient through X_n = X * r(X) for rows X, given dL/dX_n:
    dL/dX = r * (dX_n - X_n * mean(dX_n o X_n)) (the derivative of
    (mean(x^2) + eps)^(-1/2) is -r^3 x / D)."""
    X, dXn = np.asarray(X, dtype=F64), np.asarray(dXn, dtype=F64)
    Xn = X * r[:, None]
    if quant:
        Xn = r32(Xn)
    c = np.sum(dXn * Xn, axis=1) / X.shape[1]
    return r[:, None] * (dXn - Xn * c[:, None])


def quantize(Q, K, V, sh: Shape, quant=True) -> Quantized:
    """Forward steps (1)-(2): smoothing, then per-block quantisation of
    Q (bq-row blocks), K and V (bkv-row blocks); with QK-norm the rows of Q
    and K are normalised first."""
    Q, K, V = (np.asarray(a, dtype=F64) for a in (Q, K, V))
    N, D = Q.shape
    rnd = r32 if quant else (lambda x: np.asarray(x, dtype=F64))
    rq = rk = None
    if sh.qk_norm:
        Q, rq = rms_norm(Q, quant)
        K, rk = rms_norm(K, quant)

    # K-smoothing: subtract the mean over all N tokens of the head.
    if sh.k_smooth:
        mu_k = rnd(np.sum(K, axis=0) / N)
        K_sm = rnd(K - mu_k[None, :])
    else:
        mu_k = np.zeros(D)
        K_sm = K.copy()

    # Q-smoothing: subtract the mean of each bq-row query block.
    mu_q = np.zeros((sh.Tm, D))
    Q_sm = Q.copy()
    if sh.q_smooth:
        for i in range(sh.Tm):
            rows = slice(i * sh.bq, (i + 1) * sh.bq)
            mu_q[i] = rnd(np.sum(Q[rows], axis=0) / sh.bq)
            Q_sm[rows] = rnd(Q[rows] - mu_q[i][None, :])

    Qc = np.zeros((N, D)); sQ = np.zeros(sh.Tm)
    Kc = np.zeros((N, D)); sK = np.zeros(sh.Tn)
    Vc = np.zeros((N, D)); sV = np.zeros(sh.Tn)
    for i in range(sh.Tm):
        rows = slice(i * sh.bq, (i + 1) * sh.bq)
        Qc[rows], sQ[i] = quantize_block(Q_sm[rows], quant, sh.fp8)
    for j in range(sh.Tn):
        rows = slice(j * sh.bkv, (j + 1) * sh.bkv)
        Kc[rows], sK[j] = quantize_block(K_sm[rows], quant, sh.fp8)
        Vc[rows], sV[j] = quantize_block(V[rows], quant, sh.fp8)
    return Quantized(Qc, sQ, Kc, sK, Vc, sV, mu_k, mu_q, K_sm, rq, rk)


# ---------------------------------------------------------------------------
# Tiles and logits (forward step (3); SA3 Eq. 8)
# ---------------------------------------------------------------------------

def tile_visible(i: int, j: int, sh: Shape) -> bool:
    """False when every key of block j lies after the last query of block i."""
    return (not sh.causal) or (j * sh.bkv <= (i + 1) * sh.bq - 1)


def tile_mask(i: int, j: int, sh: Shape) -> np.ndarray:
    """[bq, bkv] True where query (i*bq + r) sees key (j*bkv + n)."""
    q = i * sh.bq + np.arange(sh.bq)[:, None]
    k = j * sh.bkv + np.arange(sh.bkv)[None, :]
    return np.ones((sh.bq, sh.bkv), bool) if not sh.causal else (k <= q)


def qsmooth_bias(qz: Quantized, i: int, j: int, sh: Shape) -> np.ndarray:
    """scale * mu_Qi K_sm,j^T, the low-rank logit term Q-smoothing moves out of
    the INT8 product, kept in float64 ([bkv] row vector shared by the block)."""
    keys = slice(j * sh.bkv, (j + 1) * sh.bkv)
    return sh.scale * (qz.K_sm[keys] @ qz.mu_q[i])


def logits(qz: Quantized, i: int, j: int, sh: Shape) -> np.ndarray:
    """S_ij = M(Q^_i, K^_j) * s_Q * s_K * scale (+ Q-smoothing bias), masked
    entries set to -inf."""
    rows = slice(i * sh.bq, (i + 1) * sh.bq)
    keys = slice(j * sh.bkv, (j + 1) * sh.bkv)
    A = qz.Qc[rows] @ qz.Kc[keys].T                       # exact integer sums
    S = A * (qz.sQ[i] * qz.sK[j] * sh.scale)
    if sh.q_smooth:
        S = S + qsmooth_bias(qz, i, j, sh)[None, :]
    return np.where(tile_mask(i, j, sh), S, -np.inf)


def _exp_shift(S, m):
    """exp(S - m) row-wise with exp(-inf - anything) = 0 (no NaN for m = -inf)."""
    with np.errstate(invalid="ignore"):
        E = np.exp(S - m[:, None])
    return np.where(np.isneginf(S), 0.0, E)


def per_token_p_quant(P_tilde, rm, m_new, quant=True, fp8=False):
    """Forward step (4), SA3 Eq. 8: s_P = exp(rowmax(S_ij) - m_ij) / 127,
    P^_ij = P~_ij / s_P, rounded to integers in [0, 127] (E4M3: 448 and the
    nearest E4M3 value)."""
    if not quant:
        return np.ones(P_tilde.shape[0]), P_tilde.copy()
    qmax = 448 if fp8 else 127
    with np.errstate(invalid="ignore"):
        ex = np.where(np.isneginf(rm), 0.0, np.exp(rm - m_new))
    sP = (np.asarray(ex).astype(F32) / F32(qmax)).astype(F32)   # float32 division
    codes = np.zeros_like(P_tilde)
    live = sP > 0
    p32 = P_tilde[live].astype(F32)
    codes[live] = round_codes((p32 / sP[live][:, None]).astype(F64), fp8, 0)
    return sP.astype(F64), codes


def static_p_quant(P_tilde, rm, quant=True):
    """The static alternative to Eq. 8: s_P = 1/127 for every row with a
    visible key, P^ = P~ / s_P rounded to integers in [0, 127] (P~ is taken
    against the running maximum, so it lies in [0, 1]).  INT8 only."""
    if not quant:
        return np.ones(P_tilde.shape[0]), P_tilde.copy()
    sP = np.where(np.isneginf(rm), F32(0), F32(1) / F32(127)).astype(F32)
    codes = np.zeros_like(P_tilde)
    live = sP > 0
    p32 = P_tilde[live].astype(F32)
    codes[live] = np.clip(np.rint(p32 / sP[live][:, None]), 0, 127)
    return sP.astype(F64), codes


# ---------------------------------------------------------------------------
# Forward (forward steps (3)-(5); SA3 Eq. 1 and Eq. 8)
# ---------------------------------------------------------------------------

def forward(qz: Quantized, sh: Shape, quant=True, q_blocks: Optional[Iterable[int]] = None):
    """Online-softmax INT8 forward.  Returns (O [N, D], L [N]); rows of query
    blocks not in ``q_blocks`` are left as NaN.  O is rounded to the I/O dtype
    and L (natural-log logsumexp) to float32 when quant is on."""
    N, D = qz.Qc.shape
    O = np.full((N, D), np.nan)
    L = np.full(N, np.nan)
    blocks = range(sh.Tm) if q_blocks is None else q_blocks
    for i in blocks:
        rows = slice(i * sh.bq, (i + 1) * sh.bq)
        m = np.full(sh.bq, -np.inf)
        l = np.zeros(sh.bq)
        acc = np.zeros((sh.bq, D))
        for j in range(sh.Tn):
            if not tile_visible(i, j, sh):
                continue
            keys = slice(j * sh.bkv, (j + 1) * sh.bkv)
            S = logits(qz, i, j, sh)
            rm = S.max(axis=1)
            m_new = np.maximum(m, rm)
            P_tilde = _exp_shift(S, m_new)
            if sh.p_static:
                sP, P_hat = static_p_quant(P_tilde, rm, quant)
            else:
                sP, P_hat = per_token_p_quant(P_tilde, rm, m_new, quant, sh.fp8)
            with np.errstate(invalid="ignore"):
                alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
            l = alpha * l + P_tilde.sum(axis=1)
            acc = alpha[:, None] * acc + (P_hat @ qz.Vc[keys]) * (sP[:, None] * qz.sV[j])
            m = m_new
        O[rows] = acc / l[:, None]
        L[rows] = m + np.log(l)
    if quant:
        done = ~np.isnan(L)
        O[done] = round_io(O[done], sh.dtype)
        L[done] = r32(L[done])
    return O, L


def forward_two_pass(qz: Quantized, sh: Shape, quant=True):
    """The same forward written without the streaming recurrence: the running
    max after tile j is the prefix maximum of the tile row maxima, and every
    tile is rescaled straight to the final row maximum.  Used only to check the
    online recurrence (Eq. 1) of :func:`forward`."""
    N, D = qz.Qc.shape
    O = np.zeros((N, D)); L = np.zeros(N)
    for i in range(sh.Tm):
        rows = slice(i * sh.bq, (i + 1) * sh.bq)
        tiles = [j for j in range(sh.Tn) if tile_visible(i, j, sh)]
        S_all = [logits(qz, i, j, sh) for j in tiles]
        rms = np.stack([S.max(axis=1) for S in S_all])            # [tiles, bq]
        prefix = np.maximum.accumulate(rms, axis=0)
        M = prefix[-1]
        num = np.zeros((sh.bq, D)); den = np.zeros(sh.bq)
        for t, j in enumerate(tiles):
            keys = slice(j * sh.bkv, (j + 1) * sh.bkv)
            P_tilde = _exp_shift(S_all[t], prefix[t])
            sP, P_hat = per_token_p_quant(P_tilde, rms[t], prefix[t], quant, sh.fp8)
            to_final = np.exp(prefix[t] - M)
            num += to_final[:, None] * ((P_hat @ qz.Vc[keys]) * (sP[:, None] * qz.sV[j]))
            den += to_final * P_tilde.sum(axis=1)
        O[rows] = num / den[:, None]
        L[rows] = M + np.log(den)
    if quant:
        O = round_io(O, sh.dtype)
        L = r32(L)
    return O, L


# ---------------------------------------------------------------------------
# Backward pre-pass (backward step (1))
# ---------------------------------------------------------------------------

def backward_pre(O, dO, sh: Shape, quant=True):
    """D_i = rowsum(dO o O) over the stored O, and the per-block (bq rows)
    INT8 quantisation of dO.  Returns (delta [N], dOc [N, D], sdO [Tm])."""
    O, dO = np.asarray(O, dtype=F64), np.asarray(dO, dtype=F64)
    delta = np.sum(dO * O, axis=1)
    if quant:
        delta = r32(delta)
    dOc = np.zeros_like(dO); sdO = np.zeros(sh.Tm)
    for i in range(sh.Tm):
        rows = slice(i * sh.bq, (i + 1) * sh.bq)
        dOc[rows], sdO[i] = quantize_block(dO[rows], quant, sh.fp8)
    return delta, dOc, sdO


# ---------------------------------------------------------------------------
# Backward (backward steps (2)-(7); SA3 Eq. 9 INT8 updates)
# ---------------------------------------------------------------------------

def backward_tile(qz: Quantized, V, dO, dOc, sdO, L, delta, i: int, j: int, sh: Shape, quant=True):
    """All contributions of tile (i, j).  Returns a dict with the tile's
    dV_j, dK_j, dKbias_j, dQ_i terms and the intermediates P, dP, dS."""
    rows = slice(i * sh.bq, (i + 1) * sh.bq)
    keys = slice(j * sh.bkv, (j + 1) * sh.bkv)
    # (2) recompute S_ij and P_ij = exp(S_ij - L_i)
    S = logits(qz, i, j, sh)
    P = _exp_shift(S, L[rows])
    # (3) dV_j += M(P^_ij^T, dO^_i) * s_P * s_dO, P quantised per tile
    P_hat, sPb = quantize_block(P, quant, sh.fp8)
    dV = (P_hat.T @ dOc[rows]) * (sPb * sdO[i])
    # (4) dP_ij = dO_i V_j^T from the 16-bit values, no quantisation; the
    # ablation takes it from the INT8 codes of dO_i and V_j with their scales
    if sh.dp_int8:
        dP = (dOc[rows] @ qz.Vc[keys].T) * (sdO[i] * qz.sV[j])
    else:
        dP = dO[rows] @ V[keys].T
    # (5) dS_ij = P_ij o (dP_ij - D_i), then per-tile INT8 quantisation
    dS = P * (dP - delta[rows][:, None])
    dS_hat, sdS = quantize_block(dS, quant, sh.fp8)
    # (6) dQ_i += M(dS^_ij, K^_j) * s_dS * s_K
    dQ = (dS_hat @ qz.Kc[keys]) * (sdS * qz.sK[j])
    # (7) dK_j += M(dS^_ij^T, Q^_i) * s_dS * s_Q
    dK = (dS_hat.T @ qz.Qc[rows]) * (sdS * qz.sQ[i])
    # Q-smoothing bias gradient: (dS^T 1) mu_Qi^T from the unquantised dS
    dKb = np.outer(dS.sum(axis=0), qz.mu_q[i]) if sh.q_smooth else np.zeros_like(dK)
    return {"dV": dV, "dK": dK, "dKb": dKb, "dQ": dQ, "P": P, "dP": dP, "dS": dS,
            "sPb": sPb, "sdS": sdS, "P_hat": P_hat, "dS_hat": dS_hat}


def backward(qz: Quantized, V, dO, dOc, sdO, L, delta, sh: Shape, quant=True,
             kv_blocks: Optional[Iterable[int]] = None, q_blocks: Optional[Iterable[int]] = None):
    """KV blocks outer, query blocks inner (paperlayer A.1).  Returns (dQ, dK,
    dV) as float64 [N, D]: dK/dV rows only for ``kv_blocks`` and dQ rows only
    for ``q_blocks`` (NaN elsewhere; None = all).  dQ and dK carry the softmax
    scale; dK includes the Q-smoothing bias term."""
    V, dO = np.asarray(V, dtype=F64), np.asarray(dO, dtype=F64)
    N, D = V.shape
    kv_sel = set(range(sh.Tn) if kv_blocks is None else kv_blocks)
    q_sel = set(range(sh.Tm) if q_blocks is None else q_blocks)
    dQ = np.full((N, D), np.nan); dK = np.full((N, D), np.nan); dV = np.full((N, D), np.nan)
    for i in q_sel:
        dQ[i * sh.bq:(i + 1) * sh.bq] = 0.0
    for j in kv_sel:
        dK[j * sh.bkv:(j + 1) * sh.bkv] = 0.0
        dV[j * sh.bkv:(j + 1) * sh.bkv] = 0.0
    for j in range(sh.Tn):
        for i in range(sh.Tm):
            if not tile_visible(i, j, sh) or (j not in kv_sel and i not in q_sel):
                continue
            t = backward_tile(qz, V, dO, dOc, sdO, L, delta, i, j, sh, quant)
            if j in kv_sel:
                keys = slice(j * sh.bkv, (j + 1) * sh.bkv)
                dV[keys] += t["dV"]
                dK[keys] += t["dK"] + t["dKb"]
            if i in q_sel:
                dQ[i * sh.bq:(i + 1) * sh.bq] += t["dQ"]
    return dQ * sh.scale, dK * sh.scale, dV


# ---------------------------------------------------------------------------
# Whole pass over all heads
# ---------------------------------------------------------------------------

def run_head(Q, K, V, dO, sh: Shape, quant=True) -> Dict[str, np.ndarray]:
    """quantise -> forward -> backward pre-pass -> backward for one head."""
    qz = quantize(Q, K, V, sh, quant)
    O, L = forward(qz, sh, quant)
    delta, dOc, sdO = backward_pre(O, dO, sh, quant)
    dQ, dK, dV = backward(qz, V, dO, dOc, sdO, L, delta, sh, quant)
    out = {"qz": qz, "O": O, "L": L, "delta": delta, "dOc": dOc, "sdO": sdO, "dQ": dQ, "dK": dK, "dV": dV}
    if sh.qk_norm:
        # dQ, dK above are w.r.t. the normalised rows; these are w.r.t. the inputs
        out["dQ_in"] = rms_norm_backward(Q, qz.rq, dQ, quant)
        out["dK_in"] = rms_norm_backward(K, qz.rk, dK, quant)
    return out

