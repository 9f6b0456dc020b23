// bwd_mfma16.hip — attention backward (dQ, dK, dV) for bf16 / fp16 inputs on
// gfx950.
//
// What is computed: the gradient of the forward pass
//     S = scale Q K^T [+ causal mask],  P = softmax(S),  O = P V
// for an incoming dO, from the saved row statistic lse (the forward writes it
// for this purpose: "Flash Attention v2 的核心优化原理与工程实现", section 4
// stores the row statistics next to O, and its comparison section names the
// backward pass that consumes them). By the chain rule:
//     P_ij  = exp(S_ij - lse_i)              (recomputed, never stored)
//     D_i   = sum_c dO_ic O_ic  (= sum_j P_ij dP_ij)
//     dV_j  = sum_i P_ij dO_i
//     dP_ij = dO_i . V_j
//     dS_ij = P_ij (dP_ij - D_i)
//     dQ_i  = scale sum_j dS_ij K_j
//     dK_j  = scale sum_i dS_ij Q_i
// Grouped-query attention: dK and dV of a K/V head sum over the query heads
// that share it.
//
// gfx950 design:
//   * Three kernels on the caller's stream, no atomics, results independent
//     of scheduling: (1) D per row into the caller's fp32 `delta` buffer;
//     (2) dK, dV: a workgroup owns 128 keys of one K/V head (32 per wave, its
//     K and V fragments held in VGPRs) and streams every query tile that can
//     see them, of every query head in the group, through LDS (for
//     grouped-query heads at d = 64, three groups of waves taking turns);
//     (3) dQ: a
//     workgroup owns 128 query rows (32 per wave, Q and dO held in VGPRs) and
//     streams the K/V tiles. dQ is thus recomputed from S rather than summed
//     across the dK/dV workgroups: one more product instead of a
//     cross-workgroup reduction.
//   * Every product is a v_mfma_f32_32x32x16_{bf16,f16} with fp32
//     accumulation. In the dK/dV kernel the 32x32 accumulator gives lane l
//     the key column l%32, so P and dS leave it already in the B-operand
//     layout of dV^T += dO^T P and dK^T += Q^T dS (contraction over queries);
//     in the dQ kernel lane l owns query l%32, as in the forward kernel, and
//     dS^T is the B operand of dQ^T += K^T dS^T. The A operands of those
//     products (dO^T, Q^T, K^T) come from row-major LDS tiles through
//     ds_read_b64_tr_b16.
//   * D enters as the initial accumulator of dP (stored negated), so
//     dP - D costs no vector instruction; lse enters the exponent as
//     lse * log2(e), staged once per query tile.
//   * Tiles read both by rows and transposed use one XOR swizzle that keeps
//     both access patterns free of LDS bank conflicts.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_internal.h"
#include "bwd_chunks.h"
#include "mfma_common.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.44269504088896341f;
constexpr int kBwdThreads = 256;   // 4 waves
constexpr int kBwdWaves = kBwdThreads / 64;
constexpr int kKeyBlock = kBwdWaves * 32;     // keys per dK/dV workgroup
constexpr int kQStage = 64;                   // query rows per LDS stage (dK/dV kernel)
static_assert(kKeyBlock == bwdplan::kKeyBlock && kQStage == bwdplan::kQStage,
              "the dK/dV item plan uses the kernel's tile sizes");
constexpr int kQueryBlock = kBwdWaves * 32;   // query rows per dQ workgroup
constexpr int kKStage = 64;                   // keys per LDS stage (dQ kernel)
constexpr int kComputeUnits = 256;
constexpr int kGqaGroups = bwdplan::kGroupedWaveGroups;   // wave groups of a grouped-query d = 64 item
// 16-bit value to fp32.
template <bool IS_BF16>
__device__ __forceinline__ float lo16(uint32_t w) {
    if constexpr (IS_BF16) return __builtin_bit_cast(float, w << 16);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <bool IS_BF16>
__device__ __forceinline__ float hi16(uint32_t w) {
    if constexpr (IS_BF16) return __builtin_bit_cast(float, w & 0xffff0000u);
    else return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// ---------------------------------------------------------------------------
// (1) D_i = dO_i . O_i, fp32, one row per D/8 consecutive lanes.
template <bool IS_BF16, int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_delta_kernel(BwdParams p) {
    constexpr int LPR = D / 8;                  // lanes per row, 8 elements each
    constexpr int RPB = kBwdThreads / LPR;      // rows per workgroup
    const int64_t rows = (int64_t)p.BH * p.N;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int c = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const u32x4 o = *(const u32x4*)((const uint16_t*)p.o + row * D + 8 * c);
        const u32x4 g = *(const u32x4*)((const uint16_t*)p.dout + row * D + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc = fmaf(lo16<IS_BF16>(o[e]), lo16<IS_BF16>(g[e]), acc);
            acc = fmaf(hi16<IS_BF16>(o[e]), hi16<IS_BF16>(g[e]), acc);
        }
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (c == 0 && row < rows) p.delta[row] = acc;
}

// ---------------------------------------------------------------------------
// (2) dK, dV. Work item: (key tile of 128, b*H_kv + h_kv), or, when p.chunk > 0,
// a chunk of p.chunk consecutive steps of such a key tile (bwd_chunks.h);
// causal items are ordered key tile 0 first: it is seen by the most query
// rows. The item's query steps (query tiles of the query heads of the group
// that can see the keys, head-major) are dealt round-robin to GROUPS groups
// of 4 waves, each with
// its own LDS stage buffers and its own partial dK, dV for the same 128
// keys; the partials are summed through LDS at the end. Groups shorten the
// sequential length of an item at no extra traffic; three are used for
// grouped-query heads at d = 64, where an item spans G heads and the items
// are G times fewer (three waves per SIMD: the most the kernel's ~166
// VGPRs allow). (With one query head per item, 4-wave workgroups, three
// per CU, keep more independent work in flight; at d = 128 the registers
// do not hold a second group's waves.)
template <bool IS_BF16, int D, bool CAUSAL, int GROUPS>
__global__ __launch_bounds__(kBwdThreads * GROUPS, GROUPS == 3 ? 3 : 2) void bwd_dkdv_kernel(BwdParams p) {
    using Op = Op16<IS_BF16>;
    using T = BTile<kQStage, D>;
    using Cp = BCopy<kQStage, D, kBwdWaves>;
    constexpr int NKD = D / 16;   // contraction steps over d
    constexpr int NDB = D / 32;   // 32-row blocks of dK^T / dV^T

    // Per parity, one tile per group: Q, dO, lse * log2(e) and -D. After the
    // loop the Q and dO space holds group 1's partial sums.
    static_assert(GROUPS == 1 || 4 * GROUPS * T::kBytes >= 2 * NDB * 16 * kBwdThreads * 4,
                  "reduction space");
    // One LDS block, the four row-statistic arrays first: their addresses
    // then fit the 16-bit offset field of an LDS instruction, so one lane
    // address serves all four (at d = 128 the tiles take 64 KB, and placed
    // after them the arrays cost three more address registers, spilled).
    constexpr int kStat = GROUPS * kQStage * 4;       // bytes of one array
    static_assert((4 * kStat) % 1024 == 0, "tiles stay 1024-byte aligned");
    __shared__ __attribute__((aligned(1024))) char smem[4 * kStat + 4 * GROUPS * T::kBytes];
    LDS_AS char* const lds = (LDS_AS char*)smem;
    LDS_AS float* const l_lds0 = (LDS_AS float*)(lds);                 // lse * log2(e)
    LDS_AS float* const l_lds1 = (LDS_AS float*)(lds + kStat);
    LDS_AS float* const d_lds0 = (LDS_AS float*)(lds + 2 * kStat);     // -D
    LDS_AS float* const d_lds1 = (LDS_AS float*)(lds + 3 * kStat);
    LDS_AS char* const q_lds0 = lds + 4 * kStat;
    LDS_AS char* const q_lds1 = q_lds0 + GROUPS * T::kBytes;
    LDS_AS char* const o_lds0 = q_lds1 + GROUPS * T::kBytes;          // dO
    LDS_AS char* const o_lds1 = o_lds0 + GROUPS * T::kBytes;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = GROUPS == 1 ? 0 : wave >> 2;   // step group
    const int wk = wave & 3;                     // key block of this wave
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int N = (int)p.N;
    LDS_AS char* const qL[2] = {q_lds0 + grp * T::kBytes, q_lds1 + grp * T::kBytes};
    LDS_AS char* const oL[2] = {o_lds0 + grp * T::kBytes, o_lds1 + grp * T::kBytes};
    LDS_AS float* const lL[2] = {l_lds0 + grp * kQStage, l_lds1 + grp * kQStage};
    LDS_AS float* const dL[2] = {d_lds0 + grp * kQStage, d_lds1 + grp * kQStage};

    // Item w: key tile kt of K/V slice kv_bh, its steps s0 .. s0 + n_steps - 1.
    const int w = blockIdx.x;
    const int n_qt = (N + kQStage - 1) / kQStage;
    int kt, kv_bh, s0, n_steps;
    int64_t part_row = 0;
    bool partial = false;   // write partial sums (a cut key tile) instead of dK, dV
    if (p.chunk > 0) {
        const bwdplan::Item it = bwdplan::locate(w, N, p.G, p.BH_kv, CAUSAL, p.chunk);
        if (!it.valid) return;   // (the grid holds exactly the plan's items)
        kt = it.kt;
        kv_bh = it.slice;
        s0 = it.s0;
        n_steps = it.s1 - it.s0;
        part_row = it.part_row;
        partial = it.partial;
    } else {
        kt = w / p.BH_kv;
        kv_bh = w - kt * p.BH_kv;
        s0 = 0;
        n_steps = bwdplan::kv_steps(p.G, n_qt, kt, CAUSAL);
    }
    const int k0 = kt * kKeyBlock;
    const int kw = k0 + 32 * wk;                 // first key of this wave
    const int key = kw + l32;                    // this lane's key
    const size_t kv_base = (size_t)kv_bh * (size_t)N * D;
    // The K/V head's query heads: b*H + h_kv*G + 0 .. G-1.
    const int bh0 = kv_bh * p.G;

    // K and V fragments (B operands of S = Q K^T and dP = dO V^T): lane l
    // holds row key, elements 16kd + 8g .. +7. Keys past N read as zero.
    u32x4 kf[NKD], vf[NKD];
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
        kf[kd] = u32x4{0u, 0u, 0u, 0u};
        vf[kd] = u32x4{0u, 0u, 0u, 0u};
    }
    if (key < N) {
        const uint16_t* kr = (const uint16_t*)p.k + kv_base + (size_t)key * D + 8 * g;
        const uint16_t* vr = (const uint16_t*)p.v + kv_base + (size_t)key * D + 8 * g;
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) {
            kf[kd] = *(const u32x4*)(kr + 16 * kd);
            vf[kd] = *(const u32x4*)(vr + 16 * kd);
        }
    }
    // vmcnt(0): the fragments are in. Without this wait the compiler places
    // its waits for them at their first use inside the query loop, where
    // every step then also waits for the next stage's copies in flight
    // (they count in the same counter): vmcnt(0) in the middle of each
    // 32-query block.
    __builtin_amdgcn_s_waitcnt(0x0f70);

    int roff[NKD];   // row reads: row l32 (+32 qb), logical chunk 2kd + g
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) roff[kd] = T::row_off(l32, 2 * kd + g);
    int troff[NDB][2];
    tr_offsets<kQStage, D>(lane, troff);
    int coff[Cp::kPerWave];
    Cp::offsets(wk, lane, coff);

    const int t0 = CAUSAL ? k0 / kQStage : 0;    // first query tile that sees these keys
    const int n_t = n_qt - t0;
    const int n_iter = (n_steps + GROUPS - 1) / GROUPS;   // steps GROUPS*i + grp
    const float c2 = p.scale_log2;

    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            dk[db][i] = 0.f;
            dv[db][i] = 0.f;
        }

    // Item step s is step s0 + s of the key tile: query head bh0 + (s0 + s) / n_t,
    // query tile t0 + (s0 + s) % n_t.
    auto stage_issue = [&](int s, LDS_AS char* qbuf, LDS_AS char* obuf, float& nl, float& nd)
        __attribute__((always_inline)) {
        const int hh = (s0 + s) / n_t;
        const int t = t0 + (s0 + s - hh * n_t);
        const size_t base = (size_t)(bh0 + hh) * (size_t)N;
        Cp::copy((const uint16_t*)p.q + base * D, t * kQStage, N, qbuf, wk, coff);
        Cp::copy((const uint16_t*)p.dout + base * D, t * kQStage, N, obuf, wk, coff);
        if (wk == 0) {
            const int row = t * kQStage + lane;
            // Rows past N: P = exp2(-inf) = 0, so they contribute nothing.
            nl = row < N ? p.lse[base + row] * kLog2e : INFINITY;
            nd = row < N ? -p.delta[base + row] : 0.f;
        }
    };
    auto stage_publish = [&](LDS_AS float* lbuf, LDS_AS float* dbuf, float nl, float nd) __attribute__((always_inline)) {
        if (wk == 0) {
            lbuf[lane] = nl;
            dbuf[lane] = nd;
        }
    };

    // One 32-query block (rows 32 qb .. +31 of the stage tile at query qs).
    auto block = [&](const LDS_AS char* qbuf, const LDS_AS char* obuf, const LDS_AS float* lbuf,
                     const LDS_AS float* dbuf, int qb, int qs) __attribute__((always_inline)) {
        const LDS_AS char* qrow = qbuf + 32 * qb * T::kRowBytes;
        const LDS_AS char* orow = obuf + 32 * qb * T::kRowBytes;
        // S[query][key] = Q K^T
        f32x16 sacc;
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) {
            const u32x4 a = *(const LDS_AS u32x4*)(qrow + roff[kd]);
            sacc = Op::mfma(a, kf[kd], kd == 0 ? f32x16{} : sacc);
        }
        // Entry i of the accumulator is query 8(i/4) + 4g + i%4 of the block.
        float pf[16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const f32x4 lv = *(const LDS_AS f32x4*)(lbuf + 32 * qb + 8 * r + 4 * g);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                pf[4 * r + k] = __builtin_amdgcn_exp2f(fmaf(sacc[4 * r + k], c2, -lv[k]));
        }
        if (CAUSAL && kw + 31 > qs) {   // the block crosses the diagonal
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (key > qs + 8 * (i >> 2) + 4 * g + (i & 3)) pf[i] = 0.f;
        }
        u32x4 pb[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int e = 0; e < 4; ++e) pb[kb2][e] = Op::pack2(pf[8 * kb2 + 2 * e], pf[8 * kb2 + 2 * e + 1]);
        // dV^T[d][key] += dO^T P
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                const LDS_AS char* rb = orow + 16 * kb2 * T::kRowBytes;
                dv[db] = Op::mfma(tr_read(rb + troff[db][0], rb + troff[db][1]), pb[kb2], dv[db]);
            }
        // E = dO V^T - D  (the accumulator starts at -D)
        f32x16 eacc;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const f32x4 dvv = *(const LDS_AS f32x4*)(dbuf + 32 * qb + 8 * r + 4 * g);
#pragma unroll
            for (int k = 0; k < 4; ++k) eacc[4 * r + k] = dvv[k];
        }
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) {
            const u32x4 a = *(const LDS_AS u32x4*)(orow + roff[kd]);
            eacc = Op::mfma(a, vf[kd], eacc);
        }
        // dS = P E; dK^T[d][key] += Q^T dS
        u32x4 sb[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 8 * kb2 + 2 * e;
                sb[kb2][e] = Op::pack2(pf[i] * eacc[i], pf[i + 1] * eacc[i + 1]);
            }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2) {
                const LDS_AS char* rb = qrow + 16 * kb2 * T::kRowBytes;
                dk[db] = Op::mfma(tr_read(rb + troff[db][0], rb + troff[db][1]), sb[kb2], dk[db]);
            }
    };

    // Iteration i: this group's step s = GROUPS*i + grp (every group runs
    // n_iter iterations, one barrier each; a group past its last step waits).
    auto step = [&](int i, auto par_tag) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_tag)::value;
        const int s = GROUPS * i + grp;
        float nl = 0.f, nd = 0.f;
        if (s + GROUPS < n_steps) stage_issue(s + GROUPS, qL[1 - PAR], oL[1 - PAR], nl, nd);
        ATTN_PROBE(i);
        if (GROUPS == 1 || s < n_steps) {   // one group: s < n_steps always
            const int hh = (s0 + s) / n_t;
            const int t = t0 + (s0 + s - hh * n_t);
#pragma unroll
            for (int qb = 0; qb < kQStage / 32; ++qb) {
                const int qs = t * kQStage + 32 * qb;
                // Skip blocks past N, and (causal) blocks whose queries all
                // precede this wave's keys.
                if (qs < N && (!CAUSAL || qs + 31 >= kw)) block(qL[PAR], oL[PAR], lL[PAR], dL[PAR], qb, qs);
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): the next stage's copies and loads
        if (s + GROUPS < n_steps) stage_publish(lL[1 - PAR], dL[1 - PAR], nl, nd);
        ATTN_PROBE(i + 1);
        __syncthreads();
    };

    {
        float nl = 0.f, nd = 0.f;
        if (grp < n_steps) stage_issue(grp, qL[0], oL[0], nl, nd);
        __builtin_amdgcn_s_waitcnt(0x0f70);
        if (grp < n_steps) stage_publish(lL[0], dL[0], nl, nd);
        __syncthreads();
    }
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int i = 0;
    for (; i + 1 < n_iter; i += 2) {
        step(i, P0{});
        step(i + 1, P1{});
    }
    if (i < n_iter) step(i, P0{});

    if constexpr (GROUPS > 1) {
        // Groups 1 .. GROUPS-1 in turn hand their partial sums to group 0
        // through the Q and dO tiles (no copy is in flight and every wave is
        // past its last read): element j of the thread's 2*NDB*16 sums at
        // float j*256 + 64 wk + lane, spread over the four tile arrays.
        constexpr int kQuarter = GROUPS * T::kBytes / 4;   // floats per array
        LDS_AS float* const red4[4] = {(LDS_AS float*)q_lds0, (LDS_AS float*)q_lds1,
                                       (LDS_AS float*)o_lds0, (LDS_AS float*)o_lds1};
        auto red = [&](int idx) -> LDS_AS float& { return red4[idx / kQuarter][idx % kQuarter]; };
        const int slot = wk * 64 + lane;
        for (int src = 1; src < GROUPS; ++src) {
            if (grp == src) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        red(((2 * db + 0) * 16 + r) * kBwdThreads + slot) = dk[db][r];
                        red(((2 * db + 1) * 16 + r) * kBwdThreads + slot) = dv[db][r];
                    }
            }
            __syncthreads();
            if (grp == 0) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        dk[db][r] += red(((2 * db + 0) * 16 + r) * kBwdThreads + slot);
                        dv[db][r] += red(((2 * db + 1) * 16 + r) * kBwdThreads + slot);
                    }
            }
            // Group 0 has read one hand-over before the next is written.
            if (src + 1 < GROUPS) __syncthreads();
        }
        if (grp != 0) return;
    }

    // dK = scale dK^T^T, dV = dV^T^T: lane l writes key `key`, entries
    // d = 32 db + 8 i4 + 4g .. +3. A chunk of a cut key tile writes fp32
    // partial sums (not yet scaled) into dq's memory instead, in the layout
    // of bwd_chunks.h; bwd_kv_reduce_kernel adds them up before dq is written.
    if (partial) {
        if (key < N) {
            const int rows = bwdplan::tile_rows(N, kt);
            float* blk = (float*)p.dq + ((size_t)part_row * p.BH_kv + (size_t)kv_bh * rows) * (2 * D);
            float* pk = blk + (size_t)(key - k0) * D;
            float* pv = blk + (size_t)(rows + key - k0) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int dd = 32 * db + 8 * i4 + 4 * g;
                    *(f32x4*)(pk + dd) = f32x4{dk[db][4 * i4], dk[db][4 * i4 + 1],
                                               dk[db][4 * i4 + 2], dk[db][4 * i4 + 3]};
                    *(f32x4*)(pv + dd) = f32x4{dv[db][4 * i4], dv[db][4 * i4 + 1],
                                               dv[db][4 * i4 + 2], dv[db][4 * i4 + 3]};
                }
        }
        return;
    }
    if (key < N) {
        uint16_t* dkr = (uint16_t*)p.dk + kv_base + (size_t)key * D;
        uint16_t* dvr = (uint16_t*)p.dv + kv_base + (size_t)key * D;
        const float sc = p.scale;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int dd = 32 * db + 8 * i4 + 4 * g;
                const u32x2 kv = {Op::pack2(dk[db][4 * i4] * sc, dk[db][4 * i4 + 1] * sc),
                                  Op::pack2(dk[db][4 * i4 + 2] * sc, dk[db][4 * i4 + 3] * sc)};
                const u32x2 vv = {Op::pack2(dv[db][4 * i4], dv[db][4 * i4 + 1]),
                                  Op::pack2(dv[db][4 * i4 + 2], dv[db][4 * i4 + 3])};
                *(u32x2*)(dkr + dd) = kv;
                *(u32x2*)(dvr + dd) = vv;
            }
    }
}

// ---------------------------------------------------------------------------
// (2b) Chunked dK/dV: dK = scale * the sum of a cut key tile's partial dK^T,
// dV = the sum of its partial dV^T, added in chunk order (deterministic).
// Workgroup: RW rows of key tile kt of K/V slice `slice`, 4 columns a thread.
template <bool IS_BF16, int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_kv_reduce_kernel(BwdParams p, bool causal) {
    using Op = Op16<IS_BF16>;
    constexpr int TPR = D / 4;                 // threads per row
    constexpr int RW = kBwdThreads / TPR;      // rows per workgroup
    constexpr int WPT = kKeyBlock / RW;        // workgroups per key tile
    const int N = (int)p.N;
    const int w = blockIdx.x;
    const int kt = w / (WPT * p.BH_kv);
    const int rem = w - kt * (WPT * p.BH_kv);
    const int rb = rem / p.BH_kv;
    const int slice = rem - rb * p.BH_kv;
    const int rows = bwdplan::tile_rows(N, kt);
    const int r = rb * RW + (int)threadIdx.x / TPR;
    const int j = 4 * ((int)threadIdx.x % TPR);
    if (r >= rows) return;
    const int n_qt = bwdplan::n_query_stages(N);
    const int nc = bwdplan::n_chunks(bwdplan::kv_steps(p.G, n_qt, kt, causal), p.chunk);
    if (nc < 2) return;   // a key tile of one chunk wrote dK, dV itself
    const int first = bwdplan::first_chunk(kt, N, p.G, causal, p.chunk);
    const float* part = (const float*)p.dq;
    f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < nc; ++c) {
        const size_t blk = ((size_t)((int64_t)first * kKeyBlock + (int64_t)c * rows) * p.BH_kv +
                            (size_t)slice * rows) * (2 * D);
        const f32x4 a = *(const f32x4*)(part + blk + (size_t)r * D + j);
        const f32x4 b = *(const f32x4*)(part + blk + (size_t)(rows + r) * D + j);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            sk[x] += a[x];
            sv[x] += b[x];
        }
    }
    const float sc = p.scale;
    const size_t o = ((size_t)slice * N + (size_t)kt * kKeyBlock + r) * D + j;
    *(u32x2*)((uint16_t*)p.dk + o) = u32x2{Op::pack2(sk[0] * sc, sk[1] * sc), Op::pack2(sk[2] * sc, sk[3] * sc)};
    *(u32x2*)((uint16_t*)p.dv + o) = u32x2{Op::pack2(sv[0], sv[1]), Op::pack2(sv[2], sv[3])};
}

// ---------------------------------------------------------------------------
// (3) dQ. Work item: (query tile of 128, b*H + h), longest first when causal.
template <bool IS_BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(BwdParams p) {
    using Op = Op16<IS_BF16>;
    using T = BTile<kKStage, D>;
    using Cp = BCopy<kKStage, D, kBwdWaves>;
    constexpr int NKD = D / 16;
    constexpr int NDB = D / 32;

    __shared__ __attribute__((aligned(1024))) char k_lds0[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char k_lds1[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds0[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds1[T::kBytes];
    LDS_AS char* const kL[2] = {(LDS_AS char*)k_lds0, (LDS_AS char*)k_lds1};
    LDS_AS char* const vL[2] = {(LDS_AS char*)v_lds0, (LDS_AS char*)v_lds1};

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int N = (int)p.N;

    const int n_qt = (N + kQueryBlock - 1) / kQueryBlock;
    const int w = blockIdx.x;
    const int tile = CAUSAL ? n_qt - 1 - w / p.BH : w / p.BH;
    const int r = w - (w / p.BH) * p.BH;
    // Query slice and its K/V slice (h_kv = h / G); the query heads of one
    // K/V head take the items kv, kv + BH_kv, ... (one XCD when BH_kv % 8 == 0).
    const int kv_bh = r % p.BH_kv;
    const int bh = kv_bh * p.G + r / p.BH_kv;
    const int q0 = tile * kQueryBlock;
    const int qw = q0 + 32 * wave;
    const int qi = qw + l32;
    const int qc = min(qi, N - 1);
    const size_t q_base = (size_t)bh * (size_t)N;
    const size_t kv_base = (size_t)kv_bh * (size_t)N * D;
    const uint16_t* Kg = (const uint16_t*)p.k + kv_base;
    const uint16_t* Vg = (const uint16_t*)p.v + kv_base;

    // Q and dO fragments (B operands of S^T = K Q^T and dP^T = V dO^T).
    u32x4 qf[NKD], of[NKD];
    {
        const uint16_t* qr = (const uint16_t*)p.q + (q_base + qc) * D + 8 * g;
        const uint16_t* orr = (const uint16_t*)p.dout + (q_base + qc) * D + 8 * g;
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd) {
            qf[kd] = *(const u32x4*)(qr + 16 * kd);
            of[kd] = *(const u32x4*)(orr + 16 * kd);
        }
    }
    const float lq = p.lse[q_base + qc] * kLog2e;
    const float neg_d = -p.delta[q_base + qc];
    const float c2 = p.scale_log2;

    int roff[NKD];
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) roff[kd] = T::row_off(l32, 2 * kd + g);
    int troff[NDB][2];
    tr_offsets<kKStage, D>(lane, troff);
    int coff[Cp::kPerWave];
    Cp::offsets(wave, lane, coff);

    const int n_tiles = ((CAUSAL ? min(q0 + kQueryBlock, N) : N) + kKStage - 1) / kKStage;
    const int n_live = CAUSAL ? min(n_tiles, (qw + 31) / kKStage + 1)
                              : __builtin_amdgcn_readfirstlane(n_tiles);
    int j_mask = N / kKStage;   // first tile crossing N or this wave's diagonal
    if (CAUSAL) j_mask = min(j_mask, (qw + 1) / kKStage);

    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;

    auto tile_compute = [&](int j, const LDS_AS char* kbuf, const LDS_AS char* vbuf) __attribute__((always_inline)) {
        // S^T[key][query] = K Q^T, two 32-key blocks
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) {
                const u32x4 a = *(const LDS_AS u32x4*)(kbuf + 32 * kb * T::kRowBytes + roff[kd]);
                s[kb] = Op::mfma(a, qf[kd], kd == 0 ? f32x16{} : s[kb]);
            }
        // Entry i of block kb is key 64j + 32kb + 8(i/4) + 4g + i%4.
        if (j >= j_mask) {
            const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - j * kKStage - 4 * g;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    s[kb][i] = (32 * kb + 8 * (i >> 2) + (i & 3) > lim) ? -INFINITY : s[kb][i];
        }
        // E^T = V dO^T - D
        f32x16 e[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) {
                const u32x4 a = *(const LDS_AS u32x4*)(vbuf + 32 * kb * T::kRowBytes + roff[kd]);
                f32x16 c;
                if (kd == 0) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) c[i] = neg_d;
                } else {
                    c = e[kb];
                }
                e[kb] = Op::mfma(a, of[kd], c);
            }
        // dS^T = P^T E^T, packed as the B operand of dQ^T += K^T dS^T
        u32x4 sb[4];
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                const int i = 8 * (kb2 & 1) + 2 * x;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb2 >> 1][i], c2, -lq));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb2 >> 1][i + 1], c2, -lq));
                sb[kb2][x] = Op::pack2(p0 * e[kb2 >> 1][i], p1 * e[kb2 >> 1][i + 1]);
            }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int kb2 = 0; kb2 < 4; ++kb2) {
                const LDS_AS char* rb = kbuf + 16 * kb2 * T::kRowBytes;
                dq[db] = Op::mfma(tr_read(rb + troff[db][0], rb + troff[db][1]), sb[kb2], dq[db]);
            }
    };

    auto step = [&](int j, auto par_tag) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_tag)::value;
        if (j + 1 < n_tiles) {
            Cp::copy(Kg, (j + 1) * kKStage, N, kL[1 - PAR], wave, coff);
            Cp::copy(Vg, (j + 1) * kKStage, N, vL[1 - PAR], wave, coff);
        }
        ATTN_PROBE(j);
        if (j < n_live) tile_compute(j, kL[PAR], vL[PAR]);
        __builtin_amdgcn_s_waitcnt(0x0f70);
        ATTN_PROBE(j + 1);
        __syncthreads();
    };

    Cp::copy(Kg, 0, N, kL[0], wave, coff);
    Cp::copy(Vg, 0, N, vL[0], wave, coff);
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    int j = 0;
    for (; j + 1 < n_tiles; j += 2) {
        step(j, P0{});
        step(j + 1, P1{});
    }
    if (j < n_tiles) step(j, P0{});

    if (qi < N) {
        uint16_t* dqr = (uint16_t*)p.dq + (q_base + qi) * D;
        const float sc = p.scale;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int dd = 32 * db + 8 * i4 + 4 * g;
                const u32x2 wv = {Op::pack2(dq[db][4 * i4] * sc, dq[db][4 * i4 + 1] * sc),
                                  Op::pack2(dq[db][4 * i4 + 2] * sc, dq[db][4 * i4 + 3] * sc)};
                *(u32x2*)(dqr + dd) = wv;
            }
    }
}

template <bool IS_BF16, int D, bool CAUSAL>
hipError_t launch(const BwdParams& p, hipStream_t s) {
    constexpr int RPB = kBwdThreads / (D / 8);
    const int64_t rows = (int64_t)p.BH * p.N;
    hipLaunchKernelGGL((bwd_delta_kernel<IS_BF16, D>), dim3((unsigned)((rows + RPB - 1) / RPB)),
                       dim3(kBwdThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // Grouped-query heads make few, long dK/dV items (key tiles of unequal
    // length under a causal mask): cut them into chunks of equal length, no
    // more items than the device holds at once, when their partial sums fit
    // dq's memory (bwd_chunks.h); dq is written last.
    BwdParams q = p;
    // the kernel launched below
    const int groups = bwdplan::dkdv_groups(D, CAUSAL, q.G, q.N, q.BH_kv, kComputeUnits);
    q.chunk = bwdplan::choose_chunk(q.N, q.G, q.BH_kv, CAUSAL,
                                    bwdplan::dkdv_resident(D, groups, kComputeUnits));
    const int64_t items = q.chunk > 0 ? bwdplan::plan_items(q.N, q.G, q.BH_kv, CAUSAL, q.chunk)
                                      : (int64_t)bwdplan::n_key_tiles(q.N) * q.BH_kv;
    const dim3 grid_kv((unsigned)items);
    bool two_groups = false;
    if constexpr (D == 64) {
        if (groups == kGqaGroups) {
            hipLaunchKernelGGL((bwd_dkdv_kernel<IS_BF16, D, CAUSAL, kGqaGroups>), grid_kv,
                               dim3(kGqaGroups * kBwdThreads), 0, s, q);
            two_groups = true;
        }
    }
    if (!two_groups)
        hipLaunchKernelGGL((bwd_dkdv_kernel<IS_BF16, D, CAUSAL, 1>), grid_kv, dim3(kBwdThreads), 0,
                           s, q);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (q.chunk > 0) {
        constexpr int WPT = kKeyBlock / (kBwdThreads / (D / 4));
        const int64_t n_red = (int64_t)bwdplan::n_key_tiles(q.N) * WPT * q.BH_kv;
        hipLaunchKernelGGL((bwd_kv_reduce_kernel<IS_BF16, D>), dim3((unsigned)n_red),
                           dim3(kBwdThreads), 0, s, q, CAUSAL);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int n_qt = (int)((p.N + kQueryBlock - 1) / kQueryBlock);
    hipLaunchKernelGGL((bwd_dq_kernel<IS_BF16, D, CAUSAL>), dim3((unsigned)(n_qt * q.BH)),
                       dim3(kBwdThreads), 0, s, q);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd16(const BwdParams& p, bool is_bf16, int d, bool causal, hipStream_t s) {
    if (is_bf16) {
        if (d == 64) return causal ? launch<true, 64, true>(p, s) : launch<true, 64, false>(p, s);
        return causal ? launch<true, 128, true>(p, s) : launch<true, 128, false>(p, s);
    }
    if (d == 64) return causal ? launch<false, 64, true>(p, s) : launch<false, 64, false>(p, s);
    return causal ? launch<false, 128, true>(p, s) : launch<false, 128, false>(p, s);
}

}  // namespace attn
