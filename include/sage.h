/*
 * sage.h — C ABI of libsage.so: SageBwd INT8 attention (forward and backward)
 * on AMD Instinct MI355X (gfx950).
 *
 * The method: "SageBwd: A Trainable Low-bit Attention" (arXiv 2603.02170) and
 * the SageBwd part of "SageAttention3" (arXiv 2505.11594).  Six of the seven
 * attention products run on INT8 matrix cores with one float32 scale per
 * block; dP = dO V^T stays in 16-bit floating point.
 *
 * Calls, in the order a training step makes them:
 *   sage_quantize  smoothing + per-block INT8 quantisation of Q, K, V
 *   sage_fwd       INT8 forward with online softmax -> O and logsumexp L
 *   sage_bwd_pre   delta = rowsum(dO o O) and INT8 quantisation of dO
 *   sage_bwd       recompute S and P, dP in 16-bit, dS, INT8 dV, dQ, dK
 *
 * Conventions shared by every call
 *   - Every pointer is a device pointer unless stated otherwise.  The caller
 *     allocates and owns every buffer, including the workspace; the library
 *     allocates nothing and keeps no pointer after a call returns.
 *   - Calls are asynchronous on the given HIP stream (NULL = the default
 *     stream) and never synchronise the host.  Buffers must stay valid until
 *     the stream's work is done.  Calls on one stream run in order; calls on
 *     different streams that share buffers must be ordered by the caller.
 *   - All 16-bit tensors (Q, K, V, O, dO) are contiguous [B, H, N, D],
 *     row-major, in the dtype the shape names.  Every base pointer must be
 *     16-byte aligned.
 *   - Return value 0 (SAGE_OK) on success, a negative SAGE_E* code otherwise.
 *     Arguments are checked on the host before anything is launched; on an
 *     argument error nothing is launched and no buffer is touched.  An empty
 *     problem (B, H or N equal to 0) launches nothing and returns SAGE_OK.
 *   - No exception, abort or exit crosses this interface.
 *
 * Quantised-tensor layouts (element (row, col) of a [N, D] head; a "group"
 * is 32 or 64 consecutive rows; each layout is [B, H, N/group, ...]):
 *   R32   row tiles:  byte (row, col) at group row/32, offset
 *         ((col/16) * 32 + row%32) * 16 + col%16.
 *   C64P  column tiles, 64-row groups, permuted: offset (g * D + col) * 16 + e,
 *         with in-group row r = 16*(e/4) + 4*g + e%4  (g in [0,4)).
 * These orders are the operand orders of the gfx950 INT8 matrix instruction
 * the kernels use, so tiles move into LDS as plain copies; the other operand
 * orders are read out of the same tiles with the LDS transpose read.
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t* sage_stream_t;

enum {
    SAGE_OK = 0,
    SAGE_EINVAL = -1,       /* NULL pointer, negative size, misaligned pointer */
    SAGE_EUNSUPPORTED = -2, /* D, block sizes, dtype or N outside what is built */
    SAGE_EHIP = -3,         /* a HIP launch failed; see sage_last_hip_error() */
    SAGE_ESCRATCH = -4      /* sage_quantize_noalloc: the problem needs more than
                               SAGE_NOALLOC_SCRATCH_BYTES of scratch */
};

enum { SAGE_FP16 = 0, SAGE_BF16 = 1 };

/* Problem description shared by all calls. */
typedef struct sage_shape {
    int32_t B, H, N, D; /* batch, heads, sequence length, head dim (64 or 128) */
    int32_t bq;         /* rows per Q / dO quantisation block: 64 or 128 */
    int32_t bkv;        /* rows per K / V quantisation block: 64 */
    int32_t dtype;      /* SAGE_FP16 or SAGE_BF16, for Q, K, V, O, dO */
    int32_t causal;     /* 1 = key n visible to query r iff n <= r */
    int32_t k_smooth;   /* 1 = subtract the per-head token mean of K */
    int32_t q_smooth;   /* 1 = subtract the mean of each Q block */
    float sm_scale;     /* softmax scale; 0 selects 1/sqrt(D) */
    int32_t dp_int8;    /* 0 = the method: dP = dO V^T from the 16-bit values.
                           1 = ablation (SageAttention3 write-up, Table 1c
                           compares it with FP16): dP from the per-block INT8
                           codes of dO and V, dP = f32(dO^ V^^T) * f32(s_dO * s_V).
                           Then sage_quantize also stores V's codes as row
                           tiles in `vr`, sage_bwd_pre dO's in `dor`, and
                           sage_bwd reads them; the three calls must agree
                           on it. */
    int32_t p_static;   /* 0 = the method: the forward's P codes per token,
                           s_P = exp(rowmax(S_ij) - m_ij) / 127 (Eq. 8).
                           1 = ablation (the SageAttention3 write-up names it
                           beside Eq. 8 as less accurate): the static scale
                           s_P = 1/127 against the running maximum. */
    int32_t qk_norm;    /* 1 = QK-norm fused into sage_quantize (training use;
                           the SageBwd method summary trains with QK-norm,
                           prerequisites "QK-norm"): each row x of Q and K is
                           replaced by f32(x * r), r = f32(1/sqrt(mean(x^2)
                           + 1e-6)) (mean exact in float64, IEEE double sqrt
                           and division), before smoothing and quantisation;
                           r goes to rq / rk.  sage_bwd's dQ, dK are then
                           w.r.t. the normalised rows; sage_qk_norm_bwd turns
                           them into gradients w.r.t. the inputs. */
    int32_t fp8;        /* 0 = the method: INT8 codes, s = max|X| / 127.
                           1 = E4M3 variant (the SageAttention3 write-up's
                           INT8-versus-FP8 training comparison): every code
                           tensor (q, k, vt, dot and the dS workspace)
                           holds E4M3 bytes (OCP: sign, 4 exponent bits with
                           bias 7, 3 mantissa bits, largest finite 448), the
                           scales use 448 in place of 127 (block s =
                           f32(max|X| / 448), code = the nearest E4M3 value of
                           f32(x / s), ties to even; forward P against 448),
                           and the products accumulate in float32.  Not with
                           dp_int8 or p_static (SAGE_EUNSUPPORTED).  All four
                           calls must agree on it. */
} sage_shape;
/* Supported: D in {64, 128}; bq in {64, 128}; bkv = 64; N a multiple of bq
 * and of bkv (the pages define T_m = N / B_q blocks; a ragged block is
 * reported as SAGE_EUNSUPPORTED, not padded). */

/* Output of sage_quantize, input of sage_fwd / sage_bwd.  Sizes in bytes
 * for one head, T_m = N/bq, T_n = N/bkv. */
typedef struct sage_qtensors {
    int8_t* q;        /* R32,  N*D:   codes of Q (of Q - mu_Q with q_smooth) */
    float* sq;        /* T_m floats:  Q block scales */
    int8_t* k;        /* R32,  N*D:   codes of K - mu_K (K if !k_smooth) */
    float* sk;        /* T_n floats:  K block scales */
    int8_t* vt;       /* C64P, N*D:   codes of V, column tiles */
    float* sv;        /* T_n floats:  V block scales */
    int8_t* vr;       /* R32,  N*D:   dp_int8 only: V's codes again, as row
                         tiles (the ablation's dP operand); else NULL */
    float* mu_k;      /* D floats:    K token mean (written if k_smooth) */
    float* mu_q;      /* T_m*D floats: Q block means (q_smooth; else NULL) */
    float* qk_bias;   /* T_m*N floats: sm_scale * mu_Qi . (K_n - mu_K)
                         (q_smooth; else NULL).  Causal: written only for
                         query blocks i >= 128 floor(n / 128) / bq, the ones
                         the attention kernels read; the rest is left as is */
    float* rq;        /* N floats: QK-norm factor r of each Q row (qk_norm;
                         else NULL) */
    float* rk;        /* N floats: the same for K (qk_norm; else NULL) */
} sage_qtensors;

/* Output of sage_bwd_pre. */
typedef struct sage_dotensors {
    float* delta;     /* N floats per head: rowsum(dO o O) */
    int8_t* dot;      /* C64P, N*D: codes of dO, bq-row blocks */
    float* sdo;       /* T_m floats: dO block scales */
    int8_t* dor;      /* R32, N*D: dp_int8 only: dO's codes again, as row
                         tiles (the ablation's dP operand); else NULL */
} sage_dotensors;

/* Bytes of workspace sage_quantize needs: the float64 column sums of K of
 * every bkv-row block, B*H*(N/bkv)*D*8 bytes (used with k_smooth only). */
size_t sage_quantize_workspace_bytes(const sage_shape* shape);

/*
 * sage_quantize — forward steps (1)-(2) of the SageBwd method summary
 * (paper.rainbus.top, "method step details"): K-smoothing (prerequisites,
 * "K-smoothing and Q-smoothing"), optional Q-smoothing, and per-block INT8
 * quantisation with scale max|X|/127 (prerequisites "INT8 quantisation";
 * SageAttention3 write-up Eq. 7).
 *   mu_K = f32(sum_n K[n] / N), the sum exact in float64; K_sm = f32(K - mu_K)
 *   mu_Q,i likewise over the bq rows of block i; Q_sm = f32(Q - mu_Q,i)
 *   per block: s = f32(max|X| / 127); code = clamp(rint(f32(x / s)), +-127),
 *   half-to-even; a block of zeros gets s = 0 and zero codes.
 * Codes and scales are bit-identical to that definition.
 * Q, K, V: [B,H,N,D] 16-bit inputs.  out: q, sq, k, sk, vt and sv must be
 * set; mu_k with k_smooth; mu_q and qk_bias with q_smooth; rq and rk with
 * qk_norm; vr with dp_int8 (each may be NULL otherwise).
 * workspace: sage_quantize_workspace_bytes() bytes, 8-byte aligned, any
 * content (every byte read is written first by the same call); may be NULL
 * when k_smooth is 0.  mu_K is summed in a fixed order (each 64-row block's
 * column sums, then the blocks in order, in float64), so repeated calls give
 * identical bits.
 */
int sage_quantize(const sage_shape* shape, const void* Q, const void* K, const void* V,
                  const sage_qtensors* out, void* workspace, sage_stream_t stream);

/* Largest workspace sage_quantize_noalloc can stand in for (8 MiB). */
#define SAGE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/*
 * sage_quantize_noalloc — for callers that cannot allocate device memory
 * (code being captured into a HIP graph, tight serving loops, harnesses that
 * forbid hipMalloc): sage_quantize with its workspace taken from a fixed
 * array of SAGE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends.  Same arguments, layouts, results (bit for bit)
 * and errors as sage_quantize, without `workspace`; the call allocates
 * nothing.  Problems whose sage_quantize_workspace_bytes() exceed the array
 * return SAGE_ESCRATCH before anything is launched (with k_smooth 0 there is
 * no limit).  The first call on a device looks up the array's device address
 * (a HIP failure there returns SAGE_EHIP).  Every call on one GPU shares that
 * GPU's array: calls that may overlap on one GPU (several streams, several
 * host threads) race on it and must be ordered by the caller.
 */
int sage_quantize_noalloc(const sage_shape* shape, const void* Q, const void* K, const void* V,
                          const sage_qtensors* out, sage_stream_t stream);

/*
 * sage_fwd — forward steps (3)-(5): for each query block, the INT8 logits
 * S_ij = M(Q^_i, K^_j) s_Q s_K * sm_scale (+ the Q-smoothing bias), online
 * softmax (SageAttention3 Eq. 1), per-token P codes with
 * s_P = exp(rowmax(S_ij) - m_ij) / 127 and the INT8 product M(P^_ij, V^_j)
 * (Eq. 8).  The running sum l adds the unquantised probabilities.
 * O: [B,H,N,D] in the shape's dtype (round-to-nearest-even from float32).
 * L: [B,H,N] float32, natural-log logsumexp of the (smoothed) logits.
 */
int sage_fwd(const sage_shape* shape, const sage_qtensors* qk, void* O, float* L,
             sage_stream_t stream);

/*
 * sage_bwd_pre — backward step (1): D_i = rowsum(dO o O) over the stored O
 * (summed exactly in float64, rounded once to float32), and per-block (bq
 * rows) INT8 quantisation of dO exactly as in sage_quantize.  out: delta, dot
 * and sdo must be set; dor with dp_int8 (may be NULL otherwise).
 */
int sage_bwd_pre(const sage_shape* shape, const void* O, const void* dO,
                 const sage_dotensors* out, sage_stream_t stream);

/* Bytes of workspace sage_bwd needs: the INT8 dS codes of every (visible)
 * bq x bkv tile plus one float32 scale per tile, handed from the key-outer
 * backward kernel to the query-outer dQ kernel (about N^2/2 bytes per head
 * when causal, N^2 otherwise). */
size_t sage_bwd_workspace_bytes(const sage_shape* shape);

/*
 * sage_bwd — backward steps (2)-(7) (SageAttention3 write-up Eq. 9 INT8
 * updates), key blocks outer and query blocks inner: recompute S and
 * P = exp(S - L); quantise P per (bq x bkv) tile; dV += M(P^T, dO^) s_P s_dO;
 * dP = dO V^T from the 16-bit values with float32 accumulation;
 * dS = P o (dP - D); quantise dS per tile; dK += M(dS^T, Q^) s_dS s_Q
 * (+ (dS^T 1) mu_Q^T with q_smooth); then, in a second query-outer pass over
 * the stored dS codes, dQ += M(dS^, K^) s_dS s_K.  dQ and dK include
 * sm_scale.  qk is sage_quantize's output, dos sage_bwd_pre's, L sage_fwd's.
 * V, dO: the [B,H,N,D] 16-bit tensors given to sage_quantize and
 * sage_bwd_pre (dP is formed from their values).  dQ, dK, dV: [B,H,N,D]
 * float32 outputs, each written exactly once (no atomics, no clearing).
 * workspace: sage_bwd_workspace_bytes() bytes, 16-byte aligned, any content.
 */
int sage_bwd(const sage_shape* shape, const sage_qtensors* qk, const sage_dotensors* dos, const void* V,
             const void* dO, const float* L, void* workspace, float* dQ, float* dK, float* dV,
             sage_stream_t stream);

/*
 * sage_qk_norm_bwd — the gradient through QK-norm (shape->qk_norm = 1), in
 * place: for each row of Q (K likewise), with r from sage_quantize (`qk`
 * rq / rk) and x_n = f32(x * r) as the forward formed it,
 *   dX = r * (dX_n - x_n * mean(dX_n o x_n))       (mean in float64),
 * turning sage_bwd's dQ and dK (w.r.t. the normalised rows) into gradients
 * w.r.t. the inputs Q and K ([B,H,N,D] 16-bit, the same tensors
 * sage_quantize was given).  dQ, dK: [B,H,N,D] float32, read and written.
 * Errors: SAGE_EINVAL without qk_norm in the shape or for a missing or
 * misaligned pointer (rq, rk included); nothing launched then.
 */
int sage_qk_norm_bwd(const sage_shape* shape, const void* Q, const void* K, const sage_qtensors* qk, float* dQ,
                     float* dK, sage_stream_t stream);

/*
 * sage_cast_grads — the 16-bit form of the gradients: each float32 element
 * of dQ, dK and dV rounded to the shape's I/O dtype (bf16 or fp16) to
 * nearest, ties to even; infinities and NaNs stay infinities and (quiet)
 * NaNs, fp16 overflow gives infinity.  The pages fix no gradient dtype
 * (their training runs in BF16, SageBwd method summary, training setup);
 * sage_bwd's outputs stay float32, and this is the optional cast of them.
 * dQ, dK, dV: [B,H,N,D] float32 inputs (sage_bwd's, or sage_qk_norm_bwd's
 * in-place results); dQ16, dK16, dV16: [B,H,N,D] 16-bit outputs, written
 * once.  Each input/output pair may be left out (both NULL; all three left
 * out, or an empty shape, is a no-op); all pointers given must be 16-byte
 * aligned.  Errors: SAGE_EINVAL for a pair with one NULL or a misaligned
 * pointer; nothing launched then.
 */
int sage_cast_grads(const sage_shape* shape, const float* dQ, const float* dK, const float* dV, void* dQ16,
                    void* dK16, void* dV16, sage_stream_t stream);

/* Text for a status code (static storage). */
const char* sage_status_str(int status);
/* HIP error code of the most recent SAGE_EHIP in this thread (0 if none). */
int sage_last_hip_error(void);
/* Library version string. */
const char* sage_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SAGE_H */
