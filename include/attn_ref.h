/*
 * attn_ref.h — C ABI of the CPU fp64 oracle for exact attention forward.
 *
 * TEST INFRASTRUCTURE. The oracle lives in oracle/ as its own shared library
 * (liboracle_attn.so). Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load it; the GPU library never calls or links it, and the
 * two share no source, header, table or helper.
 *
 * Sources (cited by page title and section):
 *   [naive-attn]  cishoon.github.io, "flashattention" post, section 1.1.2
 *                 (attention formula, 1/sqrt(d) scaling, safe softmax,
 *                 o_i = sum_j alpha_ij v_j) and section 2 (the three
 *                 materialised steps S, softmax, P.V).
 *   [v2-naive]    "Flash Attention（二）v2版本朴素实现 cuda core",
 *                 section 3.3 (scale multiplied into S), section 3.4
 *                 (row i sees keys j <= i under the causal mask).
 *   [FA2-principles] "Flash Attention v2 的核心优化原理与工程实现",
 *                 section 4 (the kernel writes per-row statistics next to O).
 */
#ifndef ATTN_REF_H
#define ATTN_REF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input element types. Same numeric values as the GPU library's dtype codes
 * so the Python side can pass one integer to either; declared separately on
 * purpose (the oracle shares no header with the GPU path). */
enum { ATTN_REF_F32 = 0, ATTN_REF_F16 = 1, ATTN_REF_BF16 = 2 };

/* Return codes. */
enum { ATTN_REF_OK = 0, ATTN_REF_EINVAL = -1, ATTN_REF_ENOMEM = -5 };

/*
 * attn_fwd_ref — full oracle.
 *
 * For every (b, h) slice and every query row i it computes, in fp64:
 *   s_ij  = scale * sum_c q_ic k_jc           for visible keys j
 *   m_i   = max_j s_ij,  e_ij = exp(s_ij - m_i),  l_i = sum_j e_ij
 *   p_ij  = e_ij / l_i,   o_ic = sum_j p_ij v_jc,  lse_i = m_i + ln(l_i)
 * Visible keys: all j < N, or j <= i when causal != 0 ([v2-naive] 3.4).
 *
 * q, k, v   HOST pointers, [B,H,N,d] contiguous, element type `dtype`
 *           (raw IEEE binary32, binary16 or bfloat16 bits). Read only.
 * o_ref     HOST, [B,H,N,d] doubles, written.
 * lse_ref   HOST, [B,H,N] doubles (natural-log log-sum-exp of the scaled
 *           scores), written. May be NULL.
 * scale     multiplied into the dot product after widening to double; must
 *           be finite. (0 is allowed: it gives uniform weights.)
 * num_threads  worker threads; <= 0 means all online cores.
 * Ownership: the caller owns every buffer. Synchronous.
 * Errors: ATTN_REF_EINVAL for null inputs, B/H/N/d <= 0, unknown dtype,
 * causal not 0/1, non-finite scale; ATTN_REF_ENOMEM if scratch allocation
 * fails. Nothing is written on error.
 */
int attn_fwd_ref(const void* q, const void* k, const void* v,
                 double* o_ref, double* lse_ref,
                 int64_t B, int64_t H, int64_t N, int64_t d,
                 int causal, float scale, int dtype, int num_threads);

/*
 * attn_fwd_ref_rows — the same computation for a chosen set of query rows
 * only, so that full-size workloads can be checked on sampled outputs.
 *
 * rows      HOST, n_rows flat row ids r = (b*H + h)*N + i, each in
 *           [0, B*H*N). Any order; duplicates allowed.
 * o_rows    HOST, [n_rows, d] doubles: output row for rows[t] at t*d.
 * lse_rows  HOST, [n_rows] doubles, may be NULL.
 * Other arguments and errors as attn_fwd_ref; an out-of-range row id is
 * ATTN_REF_EINVAL.
 */
int attn_fwd_ref_rows(const void* q, const void* k, const void* v,
                      int64_t B, int64_t H, int64_t N, int64_t d,
                      int causal, float scale, int dtype,
                      const int64_t* rows, int64_t n_rows,
                      double* o_rows, double* lse_rows, int num_threads);

/*
 * attn_fwd_ref_gqa / attn_fwd_ref_rows_gqa — the same with grouped-query
 * attention ([FA2-principles], References item 5: GQA combined with Flash
 * Attention). q and the outputs have H heads, k and v have H_kv heads,
 * [B,H_kv,N,d] contiguous; query head h reads K/V head h / (H / H_kv).
 * H_kv must divide H (H_kv = H: multi-head, H_kv = 1: multi-query);
 * otherwise ATTN_REF_EINVAL. Row ids r = (b*H + h)*N + i as above.
 * attn_fwd_ref and attn_fwd_ref_rows are these with H_kv = H.
 */
int attn_fwd_ref_gqa(const void* q, const void* k, const void* v,
                     double* o_ref, double* lse_ref,
                     int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                     int causal, float scale, int dtype, int num_threads);
int attn_fwd_ref_rows_gqa(const void* q, const void* k, const void* v,
                          int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                          int causal, float scale, int dtype,
                          const int64_t* rows, int64_t n_rows,
                          double* o_rows, double* lse_rows, int num_threads);

/*
 * attn_bwd_ref — gradients of the forward definition above for an incoming
 * dO, in fp64, by the chain rule (the pages name the backward pass without
 * stating it: "Flash Attention v2 的核心优化原理与工程实现", comparison
 * section; the forward definition is [naive-attn] section 1.1.2):
 *   p_ij = softmax_j(scale q_i . k_j over the visible keys), o_i = sum_j p_ij v_j,
 *   D_i = dO_i . o_i, ds_ij = p_ij (dO_i . v_j - D_i),
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
 *   dv_j = sum_i p_ij dO_i,
 * the sums over i running over every query head that reads K/V head j's head
 * (grouped-query attention as in attn_fwd_ref_gqa).
 *
 * q, dout      host, [B,H,N,d] in `dtype`; k, v host, [B,H_kv,N,d].
 * dq           host double [B,H,N,d]; dk, dv host double [B,H_kv,N,d].
 * eq, ek, ev, zq, zk, zv
 *              optional (all NULL or all non-NULL), shaped like dq, dk, dv,
 *              dq, dk, dv: error scales. With A_i = sum_c |dO_ic o_ic|,
 *              w_ij = |ds_ij| + p_ij A_i, g_i = sum_c |dO_ic|, z_ij = 1 + p_ij g_i:
 *              eq_ic = scale sum_j w_ij |k_jc|, ek_jc = scale sum_i w_ij |q_ic|,
 *              ev_jc = sum_i p_ij |dO_ic|, zq_ic = scale sum_j z_ij |k_jc|,
 *              zk_jc = scale sum_i z_ij |q_ic|, zv_jc = sum_i |dO_ic|. To first
 *              order, rounding p, ds and o to a type whose rounding error is
 *              at most u |x| + s/2 (s: its subnormal spacing) moves each
 *              gradient element by at most u e + (s/2) z.
 * Other arguments and return codes as for attn_fwd_ref_gqa. Synchronous;
 * parallel over query rows within each K/V slice.
 */
int attn_bwd_ref(const void* q, const void* k, const void* v, const void* dout,
                 double* dq, double* dk, double* dv,
                 double* eq, double* ek, double* ev,
                 double* zq, double* zk, double* zv,
                 int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                 int causal, float scale, int dtype, int num_threads);

/* attn_ref_decode — widen n elements of `dtype` to double, exactly, from the
 * format definitions (sign, exponent, mantissa). Exposed so the decoder can
 * be checked against every 16-bit pattern. Returns ATTN_REF_OK or EINVAL. */
int attn_ref_decode(const void* src, double* dst, int64_t n, int dtype);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_REF_H */
