/*
 * attn.h — C ABI of the gfx950 (MI355X) exact attention library, libattn.so.
 *
 * The operation is the fused, tiled attention forward pass
 *     O = softmax(scale * Q K^T [+ causal mask]) V
 * together with the per-row log-sum-exp of the scaled scores; also its
 * grouped-query form, its gradients, and the unfused three-kernel forward
 * kept as the comparison path.
 *
 * Sources (cited by page title and section):
 *   [naive-attn]  cishoon.github.io, "flashattention" post, section 1.1.2:
 *                 the attention formula, the 1/sqrt(d) scaling (item 2) and
 *                 the row-wise safe softmax (item 3); sections 2-3: the
 *                 unfused three-kernel method (attn_fwd_unfused).
 *   [v2-naive]    "Flash Attention（二）v2版本朴素实现 cuda core":
 *                 section 1.1 (Q-tile outer loop, K/V-tile inner loop),
 *                 1.2 (row max m and row sum l kept on chip), 1.3 (deferred
 *                 1/l normalisation), 1.4 and 3.4 (causal: tiles above the
 *                 diagonal skipped, the diagonal tile masked element-wise,
 *                 row i sees keys j <= i), 3.2 (out-of-range keys zero-filled
 *                 and masked), 3.5 (rows past N are not written).
 *   [FA2-principles] "Flash Attention v2 的核心优化原理与工程实现", section 4:
 *                 per-row statistics are written next to O (here folded into
 *                 one log-sum-exp per row); References item 5: Flash
 *                 Attention combined with grouped-query attention (GQA).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. lse is always fp32. */
typedef enum { ATTN_F32 = 0, ATTN_F16 = 1, ATTN_BF16 = 2 } attn_dtype_t;

/* Return codes. */
enum {
    ATTN_OK = 0,
    ATTN_EINVAL = -1,       /* bad argument (null pointer, size, H_kv, dtype, scale, causal) */
    ATTN_EUNSUPPORTED = -2, /* head dimension other than 64 or 128 */
    ATTN_EALIGN = -3,       /* a base pointer misaligned (see each function) */
    ATTN_EHIP = -4,         /* the HIP launch failed */
    ATTN_ETOOBIG = -5       /* attn_bwd_noalloc: B*H*N > ATTN_BWD_NOALLOC_MAX_ROWS */
};

/* Rows (B*H*N) the static row-statistic array of attn_bwd_noalloc holds:
 * 4 Mi floats, 16 MiB of device memory per GPU the library runs on. */
#define ATTN_BWD_NOALLOC_MAX_ROWS (4 * 1024 * 1024)

/*
 * attn_fwd — exact attention forward on the GPU.
 *
 * For every (b, h) slice and query row i < N:
 *   o[b,h,i,:] = sum_j p_ij v[b,h,j,:],  p_ij = exp(s_ij - lse_i),
 *   s_ij = scale * q[b,h,i,:] . k[b,h,j,:],
 *   lse[b,h,i] = ln sum_j exp(s_ij)   (natural log of the scaled scores),
 * with j ranging over all keys, or over j <= i when causal = 1.
 *
 * q, k, v   DEVICE pointers, [B,H,N,d] contiguous, element type `dtype`,
 *           each 16-byte aligned. Read only.
 * o         DEVICE pointer, [B,H,N,d] contiguous, `dtype`, 16-byte aligned;
 *           written (rounded to nearest even from fp32 for f16/bf16).
 * lse       DEVICE pointer, [B,H,N] fp32, 4-byte aligned; written.
 * B, H, N   batch, heads, sequence length (queries = keys), all >= 1.
 * d         head dimension: 64 or 128.
 * causal    0 or 1 (1: row i attends to keys j <= i, diagonal included).
 * scale     finite, > 0; multiplied into q.k (the usual value is 1/sqrt(d)).
 * dtype     ATTN_F32, ATTN_F16 or ATTN_BF16. Products are accumulated in
 *           fp32 for every dtype; f16/bf16 probabilities are rounded to the
 *           input type before the P.V product.
 * stream    hipStream_t to launch on (NULL = the null stream).
 *
 * Asynchronous: returns once the kernel is enqueued; no host synchronisation
 * and no device allocation. The caller owns every buffer; outputs must not
 * alias inputs. Arguments are validated before any HIP call: on an error
 * code nothing has been launched. Inputs must be finite (NaN/Inf inputs give
 * unspecified outputs). Calls on the same stream are ordered as usual;
 * concurrent calls writing the same o/lse race.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
             int dtype, void* stream);

/*
 * attn_fwd_gqa — the same forward pass with grouped-query attention
 * ([FA2-principles], References item 5): k and v carry H_kv heads, and query
 * head h reads key/value head h / (H / H_kv), so groups of H / H_kv
 * consecutive query heads share one K/V head:
 *   s_ij = scale * q[b,h,i,:] . k[b,h/G,j,:],  o[b,h,i,:] = sum_j p_ij v[b,h/G,j,:],
 * G = H / H_kv. H_kv = H is attn_fwd itself; H_kv = 1 is multi-query attention.
 *
 * q, o      [B,H,N,d] as in attn_fwd; lse [B,H,N].
 * k, v      DEVICE pointers, [B,H_kv,N,d] contiguous, `dtype`, 16-byte aligned.
 * H_kv      >= 1 and dividing H; otherwise ATTN_EINVAL.
 * Everything else (types, alignment, errors, asynchrony, ownership) is as
 * for attn_fwd.
 */
int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d, int causal,
                 float scale, int dtype, void* stream);

/*
 * attn_bwd — gradients of the forward pass (of attn_fwd_gqa; H_kv = H for
 * attn_fwd) for an incoming gradient dout of o. The pages name the backward
 * pass that consumes the saved row statistics ([FA2-principles], comparison
 * section); its formulas are the chain rule of the forward definition:
 *   p_ij  = exp(s_ij - lse_i),  s_ij = scale * q[b,h,i,:] . k[b,h/G,j,:]
 *   D_i   = sum_c dout[b,h,i,c] * o[b,h,i,c]
 *   ds_ij = p_ij * (dout[b,h,i,:] . v[b,h/G,j,:] - D_i)
 *   dq[b,h,i,:]   = scale * sum_j ds_ij k[b,h/G,j,:]
 *   dk[b,h_kv,j,:] = scale * sum over h with h/G = h_kv, and i, of ds_ij q[b,h,i,:]
 *   dv[b,h_kv,j,:] = sum over the same h, i of p_ij dout[b,h,i,:]
 * with j over the visible keys of row i (all, or j <= i when causal = 1).
 *
 * q, o, dout   DEVICE pointers, [B,H,N,d] contiguous, `dtype`, 16-byte aligned:
 *              the forward inputs, its output o and the incoming gradient.
 * k, v         DEVICE pointers, [B,H_kv,N,d] contiguous, `dtype`, 16-byte aligned.
 * lse          DEVICE pointer, [B,H,N] fp32: the forward's log-sum-exp.
 * dq           DEVICE pointer, [B,H,N,d] `dtype`, 16-byte aligned; written. For
 *              f16/bf16 with grouped-query heads (H_kv < H) its memory may
 *              first hold fp32 partial sums of dk and dv (before dq itself
 *              is written), so that the call allocates nothing.
 * dk, dv       DEVICE pointers, [B,H_kv,N,d] `dtype`, 16-byte aligned; written
 *              (not accumulated into).
 * delta        DEVICE pointer, [B,H,N] fp32, 4-byte aligned; written with D_i
 *              (fp32 dot product of the stored o and dout rows). It holds the
 *              row statistic the gradient kernels share, so that the call
 *              allocates nothing; its contents are valid after the call.
 * B, H, H_kv, N, d, causal, scale
 *              as for attn_fwd_gqa.
 * dtype        ATTN_F32, ATTN_F16 or ATTN_BF16. Products are accumulated in
 *              fp32; for f16/bf16, p and ds are rounded to `dtype` as the
 *              operands of the dv, dk and dq products and outputs are rounded
 *              once (nearest even) from fp32; fp32 rounds nothing below fp32.
 *              p comes from the hardware exp2, which has no subnormal
 *              results: every p below 2^-126 is taken as 0 (all dtypes).
 * stream       hipStream_t (NULL = the null stream).
 *
 * Asynchronous: three kernels (four when the f16/bf16 dk/dv work of
 * grouped-query heads is cut into partial sums) are enqueued on `stream`
 * and the call returns;
 * no host synchronisation, no device allocation, no atomics (results do not
 * depend on scheduling). Validation precedes any HIP call. Outputs must not
 * alias inputs or each other.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, float* delta,
             int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d, int causal,
             float scale, int dtype, void* stream);

/*
 * attn_bwd_noalloc — attn_bwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation, kernels and results, without the
 * `delta` argument. The row statistic D_i (B*H*N floats) is kept in a
 * static device array of ATTN_BWD_NOALLOC_MAX_ROWS floats that each GPU
 * holds from the library's load until the process ends; the call performs
 * no hipMalloc, hipFree or other allocation.
 *
 * Arguments as for attn_bwd, without delta.
 * Errors: as attn_bwd (validation before any HIP call), plus ATTN_ETOOBIG
 * when B*H*N > ATTN_BWD_NOALLOC_MAX_ROWS; ATTN_EHIP also if the static
 * array's device address cannot be obtained.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (D is written in full before it is read, so nothing needs
 * clearing). Calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race on the array: serialise them.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                     int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d, int causal,
                     float scale, int dtype, void* stream);

/*
 * attn_fwd_unfused — the same forward pass (multi-head, H_kv = H) computed
 * the unfused way, one kernel per step with the N x N matrices in memory:
 * S = scale Q K^T (fp32), a row softmax into P (rounded to `dtype`) and lse,
 * then O = P V. This is the materialised three-kernel method of [naive-attn]
 * sections 2-3, kept as the baseline that shows what fusion gains; under
 * causal = 1 the full S is computed and the softmax gives the keys j > i
 * probability 0.
 *
 * q, k, v, o, lse, B, H, N, d, causal, scale, stream: as for attn_fwd.
 * dtype        ATTN_F32, ATTN_F16 or ATTN_BF16.
 * workspace    DEVICE pointer, 256-byte aligned, of workspace_bytes >=
 *              attn_unfused_workspace_bytes(B, H, N, dtype) bytes, owned by the
 *              caller; overwritten (S and P, rows padded to a multiple of 64
 *              columns). Too small or NULL: ATTN_EINVAL.
 * Asynchronous on `stream`, allocates nothing; validation precedes any HIP
 * call.
 */
int attn_fwd_unfused(const void* q, const void* k, const void* v, void* o, float* lse,
                     void* workspace, int64_t workspace_bytes, int64_t B, int64_t H, int64_t N,
                     int64_t d, int causal, float scale, int dtype, void* stream);

/* attn_unfused_workspace_bytes — bytes of workspace attn_fwd_unfused needs
 * for `dtype`: B*H*N*ld*(4 + p) with ld = N rounded up to 64 and p the bytes
 * of one probability (4 for ATTN_F32, 2 for ATTN_F16 / ATTN_BF16); -1 for
 * sizes out of range or an unknown dtype. */
int64_t attn_unfused_workspace_bytes(int64_t B, int64_t H, int64_t N, int dtype);

/* attn_strerror — static description of a return code (never NULL). */
const char* attn_strerror(int code);

/*
 * attn_debug_set_fwd_variant — debugging and testing only: force the
 * variant that attn_fwd / attn_fwd_gqa choose per call for fp16 and bf16
 * inputs, for every later call from any thread of the process (a call
 * already being launched on another thread may or may not see it).
 *
 *   query_blocks  0: automatic; 1: one 32-row query block per wave (256-row
 *                 work items); 2: two blocks per wave (512-row items), which
 *                 only the d = 64 kernels have: at d = 128 2 acts as 0.
 *   order         0: automatic; 1: tile-major work order (longest query
 *                 tiles first, consecutive items on different slices);
 *                 2: XCD-major (each of the 8 XCDs takes its K/V slices one
 *                 after another), applied only when B*H_kv is a multiple of
 *                 8, elsewhere 2 acts as 0.
 *
 * Every variant computes each output row with the same arithmetic in the
 * same order, so outputs are bit-identical across variants; only the work
 * decomposition and the speed change. Returns ATTN_OK, or ATTN_EINVAL (and
 * changes nothing) for a value outside the ranges above. Makes no HIP call.
 */
int attn_debug_set_fwd_variant(int query_blocks, int order);

/*
 * attn_debug_set_fwd_first_pass — debugging and testing only: at d = 64,
 * fp16 and bf16, force whether attn_fwd / attn_fwd_gqa run the first pass
 * without the per-tile overflow test (handing a work item to the exact pass
 * when some row's l exceeds the rescale threshold), for every later call
 * from any thread of the process, like attn_debug_set_fwd_variant.
 *
 *   mode  0: automatic (bf16 always; fp16 up to N = 32768 keys);
 *         1: the exact pass only; 2: the first pass at any N.
 *
 * A work item's first-pass result is kept only when every row's l shows
 * that no probability exceeded the threshold, in which case the exact pass,
 * which moves a row's exponent base only past that threshold, gives the
 * same bits: outputs are bit-identical across modes. Returns ATTN_OK, or
 * ATTN_EINVAL (and changes nothing) for a mode outside 0..2. Makes no HIP
 * call.
 */
int attn_debug_set_fwd_first_pass(int mode);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
