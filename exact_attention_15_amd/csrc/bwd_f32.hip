// bwd_f32.hip — attention backward (dQ, dK, dV) for fp32 inputs on gfx950.
//
// The same gradients as the 16-bit backward (the chain rule of the forward:
// D_i = dO_i . O_i, P = exp(S - lse), dV = P^T dO, dS = P (dO V^T - D),
// dQ = scale dS K, dK = scale dS^T Q), with every product on
// v_mfma_f32_32x32x2_f32: exact fp32 products, fp32 accumulation, nothing
// rounded below fp32. Structure as in the 16-bit kernels: a row-statistic
// kernel writes D into the caller's `delta`; a dK/dV kernel owns a tile of
// keys (32 per wave, K rows in VGPRs, the tile's V rows in LDS) and streams
// 32-row Q / dO stages; a dQ kernel owns a tile of query rows (32 per wave,
// Q and dO rows in VGPRs) and streams 32-key K / V stages. At d = 64 four
// wave groups share an item's stages (see FLayout). Tiles go HBM -> LDS by
// direct copies (16 bytes per lane).
//
// fp32 32x32x2 products take one value per lane: lane l supplies A[l%32][k]
// and B[k][l%32] with k = l/32. A contraction over d is split by lane half
// (half g takes d in [g D/2, (g+1) D/2)), so each lane reads D/2 contiguous
// floats of its row. A contraction over the 32 rows of an accumulator uses
// entry kk of lane half g, row 8(kk/4) + 4g + kk%4, as the B operand as it
// is, and the matching row's element (32 db + l%32) of the other factor as A.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_internal.h"
#include "mfma_common.h"

namespace attn {
namespace {

constexpr float kLog2eF = 1.44269504088896341f;
constexpr int kFThreads = 256;      // the row-statistic kernel's workgroup
constexpr int kFQStage = 32;        // query rows per LDS stage (dK/dV)
constexpr int kFKStage = 32;        // keys per LDS stage (dQ)

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ROWS x D fp32 tile in LDS, row-major, 16-byte chunk c of row r stored at
// chunk c ^ (r & 15): 16 lanes reading rows 0-15 at one logical chunk hit
// 16 different 16-byte bank groups.
template <int ROWS, int D>
struct FTile {
    static constexpr int kRowBytes = D * 4;
    static constexpr int kChunks = D / 4;
    static constexpr int kBytes = ROWS * kRowBytes;
    static __device__ __forceinline__ int chunk_off(int r, int c) {
        return r * kRowBytes + ((c ^ (r & 15)) << 4);
    }
    static __device__ __forceinline__ int elem_off(int r, int col) {
        return chunk_off(r, col >> 2) + (col & 3) * 4;
    }
};

// Direct HBM -> LDS copy of a ROWS x D fp32 tile by NW waves; rows past N
// are outside the buffer range and arrive as zeros.
template <int ROWS, int D, int NW>
struct FCopy {
    using T = FTile<ROWS, D>;
    static constexpr int kPerWave = T::kBytes / 1024 / NW;
    static_assert(kPerWave >= 1 && T::kBytes % (1024 * NW) == 0, "tile / copy waves mismatch");
    static __device__ __forceinline__ void offsets(int cw, int lane, int* off) {
#pragma unroll
        for (int u = 0; u < kPerWave; ++u) {
            const int s = (cw * kPerWave + u) * 64 + lane;
            const int r = s / T::kChunks;
            off[u] = r * T::kRowBytes + (((s % T::kChunks) ^ (r & 15)) << 4);
        }
    }
    static __device__ __forceinline__ void copy(const float* g_slice, int row0, int N,
                                                LDS_AS char* buf, int cw, const int* off) {
        const int rows = min(max(N - row0, 0), ROWS);
        const i32x4 rsrc = buffer_rsrc(g_slice + (size_t)row0 * D, rows * T::kRowBytes);
        const uint32_t lds0 = (uint32_t)(uintptr_t)buf;
#pragma unroll
        for (int u = 0; u < kPerWave; ++u)
            dma16(rsrc, lds0 + (cw * kPerWave + u) * 64 * 16, off[u]);
    }
};

// (1) D_i = dO_i . O_i, D/4 lanes per row.
template <int D>
__global__ __launch_bounds__(kFThreads) void bwd_delta_f32_kernel(BwdParams p) {
    constexpr int LPR = D / 4;
    constexpr int RPB = kFThreads / LPR;
    const int64_t rows = (int64_t)p.BH * p.N;
    const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
    const int c = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const f32x4 o = *(const f32x4*)((const float*)p.o + row * D + 4 * c);
        const f32x4 g = *(const f32x4*)((const float*)p.dout + row * D + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf(o[e], g[e], acc);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (c == 0 && row < rows) p.delta[row] = acc;
}

// Work items of the two gradient kernels. At d = 64 an item is 64 keys
// (dK/dV) or 64 query rows (dQ), two waves of 32, and four groups of such
// waves take the item's streamed stages in turn (stage s to group s mod 4),
// each with its own LDS buffers; at the end groups 1-3 hand their partial
// dK, dV or dQ to group 0 through LDS, which adds them in group order (the
// sums are plain sums: P comes from the final lse). Under a causal mask an
// item is the pair of tiles t, T-1-t of one slice, processed one after the
// other, so that every item holds the same work. At d = 128 one group of
// four waves (128 keys or rows) and one workgroup per CU, so that a wave may
// use the AGPR half of the register file (Q, dO and dQ^T alone take 192
// registers in the dQ kernel).
template <int D>
struct FLayout {
    static constexpr int kGroups = D == 64 ? 4 : 1;
    static constexpr int kWaves = D == 64 ? 2 : 4;   // waves per group
    static constexpr int kGroupThreads = 64 * kWaves;
    static constexpr int kThreads = kGroups * kGroupThreads;
    static constexpr int kBlock = 32 * kWaves;       // keys or query rows per item tile
    static constexpr bool kPaired = kGroups > 1;
};

// Tiles of one slice, and the work items of one slice (pairs when paired).
template <int D, bool CAUSAL>
__host__ __device__ __forceinline__ int f_items(int n_tiles) {
    return CAUSAL && FLayout<D>::kPaired ? (n_tiles + 1) / 2 : n_tiles;
}

// (2) dK, dV: work item (key tile(s), b*H_kv + h_kv); without pairing key
// tile 0 first (it sees the most queries under a causal mask).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(FLayout<D>::kThreads, 1) void bwd_dkdv_f32_kernel(BwdParams p) {
    using L = FLayout<D>;
    constexpr int NG = L::kGroups;
    constexpr int KW = L::kWaves;
    constexpr int GT = L::kGroupThreads;
    constexpr int BK = L::kBlock;
    using TQ = FTile<kFQStage, D>;
    using TV = FTile<BK, D>;
    using CQ = FCopy<kFQStage, D, KW>;
    using CV = FCopy<BK, D, NG * KW>;
    constexpr int HALF = D / 2;
    constexpr int NDB = D / 32;
    // Merge slots: one group's dK (or dV) partial sums take kSlotBytes; an
    // array of NG stage buffers holds kSlotsPerArray of them.
    constexpr int kSlotBytes = GT * NDB * 16 * 4;
    constexpr int kSlotsPerArray = NG * TQ::kBytes / kSlotBytes;
    static_assert(NG == 1 || 2 * kSlotsPerArray >= NG - 1, "merge space");

    // Q and dO stages (two each per group, group gg at offset gg*kBytes);
    // lse*log2(e) and -D of each stage. Separately named arrays, each buffer
    // picked by a select (an array of LDS pointers indexed at run time would
    // be placed in memory as a table).
    __shared__ __attribute__((aligned(1024))) char q_lds0[NG * TQ::kBytes];
    __shared__ __attribute__((aligned(1024))) char q_lds1[NG * TQ::kBytes];
    __shared__ __attribute__((aligned(1024))) char o_lds0[NG * TQ::kBytes];
    __shared__ __attribute__((aligned(1024))) char o_lds1[NG * TQ::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds[TV::kBytes];
    __shared__ __attribute__((aligned(16))) float l_lds[NG][2][kFQStage];
    __shared__ __attribute__((aligned(16))) float d_lds[NG][2][kFQStage];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = NG == 1 ? 0 : wave / KW;   // takes stages s with s % NG == grp
    const int wk = wave - grp * KW;            // wave within the group
    const int gtid = tid - grp * GT;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int N = (int)p.N;

    const int goff = grp * TQ::kBytes;
    auto qL = [&](int par) { return (par ? (LDS_AS char*)q_lds1 : (LDS_AS char*)q_lds0) + goff; };
    auto oL = [&](int par) { return (par ? (LDS_AS char*)o_lds1 : (LDS_AS char*)o_lds0) + goff; };
    const LDS_AS char* const vL = (const LDS_AS char*)v_lds;

    const int w = blockIdx.x;
    const int item = w / p.BH_kv;
    const int kv_bh = w - item * p.BH_kv;
    const size_t kv_base = (size_t)kv_bh * (size_t)N * D;
    const int bh0 = kv_bh * p.G;
    const float* Kg = (const float*)p.k + kv_base;
    const float* Vg = (const float*)p.v + kv_base;
    const float c2 = p.scale_log2;

    int voff[CV::kPerWave];
    CV::offsets(wave, lane, voff);
    int coff[CQ::kPerWave];
    CQ::offsets(wk, lane, coff);

    auto process = [&](int kt) __attribute__((always_inline)) {
        const int k0 = kt * BK;
        const int kw = k0 + 32 * wk;
        const int key = kw + l32;

        // The tile's BK V rows into LDS (read by rows in dP = dO V^T).
        CV::copy(Vg, k0, N, (LDS_AS char*)v_lds, wave, voff);
        // K half-row of this lane's key (B operand of S = Q K^T).
        float kf[HALF];
        {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < HALF / 4; ++c) {
                const f32x4 t = key < N ? *(const f32x4*)(Kg + (size_t)key * D + g * HALF + 4 * c) : z;
#pragma unroll
                for (int e = 0; e < 4; ++e) kf[4 * c + e] = t[e];
            }
        }

        const int n_qt = (N + kFQStage - 1) / kFQStage;
        const int t0 = CAUSAL ? k0 / kFQStage : 0;
        const int n_t = n_qt - t0;
        const int n_steps = p.G * n_t;
        const int n_iter = (n_steps + NG - 1) / NG;

        f32x16 dk[NDB], dv[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                dk[db][i] = 0.f;
                dv[db][i] = 0.f;
            }

        auto stage_issue = [&](int s, int par, float& nl, float& nd) __attribute__((always_inline)) {
            const int hh = s / n_t;
            const int t = t0 + (s - hh * n_t);
            const size_t base = (size_t)(bh0 + hh) * (size_t)N;
            CQ::copy((const float*)p.q + base * D, t * kFQStage, N, qL(par), wk, coff);
            CQ::copy((const float*)p.dout + base * D, t * kFQStage, N, oL(par), wk, coff);
            if (wk == 0 && lane < kFQStage) {
                const int row = t * kFQStage + lane;
                nl = row < N ? p.lse[base + row] * kLog2eF : INFINITY;   // rows past N: P = 0
                nd = row < N ? -p.delta[base + row] : 0.f;
            }
        };
        auto stage_publish = [&](int par, float nl, float nd) __attribute__((always_inline)) {
            if (wk == 0 && lane < kFQStage) {
                l_lds[grp][par][lane] = nl;
                d_lds[grp][par][lane] = nd;
            }
        };

        auto block = [&](int par, int qs) __attribute__((always_inline)) {
            const LDS_AS char* qb = qL(par);
            const LDS_AS char* ob = oL(par);
            // S[query][key] = Q K^T
            f32x16 s = {};
#pragma unroll
            for (int c = 0; c < HALF / 4; ++c) {
                const f32x4 a = *(const LDS_AS f32x4*)(qb + TQ::chunk_off(l32, g * (HALF / 4) + c));
#pragma unroll
                for (int e = 0; e < 4; ++e) s = mfma_f32(a[e], kf[4 * c + e], s);
            }
            // Entry i: query 8(i/4) + 4g + i%4 of the tile.
            float pf[16];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x4 lv = *(const f32x4*)(&l_lds[grp][par][8 * r + 4 * g]);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    pf[4 * r + k] = __builtin_amdgcn_exp2f(fmaf(s[4 * r + k], c2, -lv[k]));
            }
            if (CAUSAL && kw + 31 > qs) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (key > qs + 8 * (i >> 2) + 4 * g + (i & 3)) pf[i] = 0.f;
            }
            // dV^T[d][key] += dO^T P (row kk of the accumulator, both halves)
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const int qr = 8 * (kk >> 2) + 4 * g + (kk & 3);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const float a = *(const LDS_AS float*)(ob + TQ::elem_off(qr, 32 * db + l32));
                    dv[db] = mfma_f32(a, pf[kk], dv[db]);
                }
            }
            // E = dO V^T - D
            f32x16 e;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x4 dvv = *(const f32x4*)(&d_lds[grp][par][8 * r + 4 * g]);
#pragma unroll
                for (int k = 0; k < 4; ++k) e[4 * r + k] = dvv[k];
            }
#pragma unroll
            for (int c = 0; c < HALF / 4; ++c) {
                const f32x4 a = *(const LDS_AS f32x4*)(ob + TQ::chunk_off(l32, g * (HALF / 4) + c));
                const f32x4 b = *(const LDS_AS f32x4*)(vL + TV::chunk_off(32 * wk + l32, g * (HALF / 4) + c));
#pragma unroll
                for (int x = 0; x < 4; ++x) e = mfma_f32(a[x], b[x], e);
            }
            // dS = P E; dK^T[d][key] += Q^T dS
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const int qr = 8 * (kk >> 2) + 4 * g + (kk & 3);
                const float ds = pf[kk] * e[kk];
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const float a = *(const LDS_AS float*)(qb + TQ::elem_off(qr, 32 * db + l32));
                    dk[db] = mfma_f32(a, ds, dk[db]);
                }
            }
        };

        {
            float nl = 0.f, nd = 0.f;
            if (grp < n_steps) stage_issue(grp, 0, nl, nd);
            __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): V rows, K, this group's first stage
            if (grp < n_steps) stage_publish(0, nl, nd);
            __syncthreads();
        }
        for (int it = 0; it < n_iter; ++it) {
            const int par = it & 1;
            const int s = it * NG + grp;
            float nl = 0.f, nd = 0.f;
            const bool next = s + NG < n_steps;
            if (next) stage_issue(s + NG, par ^ 1, nl, nd);
            ATTN_PROBE(it);
            if (s < n_steps) {
                const int hh = s / n_t;
                const int qs = (t0 + (s - hh * n_t)) * kFQStage;
                if (qs < N && (!CAUSAL || qs + 31 >= kw)) block(par, qs);
            }
            __builtin_amdgcn_s_waitcnt(0x0f70);
            if (next) stage_publish(par ^ 1, nl, nd);
            ATTN_PROBE(it + 1);
            __syncthreads();
        }

        // Groups 1.. hand their partial sums to group 0 (every stage read is
        // done): group gg's dK in slot gg-1 of the Q stage arrays, its dV in
        // the same slot of the dO stage arrays (slot k: array k / kSlots,
        // byte offset (k % kSlots) * kSlotBytes); value k of thread t at
        // float k * GT + t of the slot.
        if constexpr (NG > 1) {
            auto slot = [&](LDS_AS char* a0, LDS_AS char* a1, int k) __attribute__((always_inline)) {
                return (LDS_AS float*)((k < kSlotsPerArray ? a0 : a1) +
                                       (k % kSlotsPerArray) * kSlotBytes);
            };
            if (grp != 0) {
                LDS_AS float* const mk = slot((LDS_AS char*)q_lds0, (LDS_AS char*)q_lds1, grp - 1);
                LDS_AS float* const mv = slot((LDS_AS char*)o_lds0, (LDS_AS char*)o_lds1, grp - 1);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        mk[(db * 16 + i) * GT + gtid] = dk[db][i];
                        mv[(db * 16 + i) * GT + gtid] = dv[db][i];
                    }
            }
            __syncthreads();
            if (grp == 0) {
#pragma unroll
                for (int gg = 1; gg < NG; ++gg) {
                    const LDS_AS float* const ok = slot((LDS_AS char*)q_lds0, (LDS_AS char*)q_lds1, gg - 1);
                    const LDS_AS float* const ov = slot((LDS_AS char*)o_lds0, (LDS_AS char*)o_lds1, gg - 1);
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            dk[db][i] += ok[(db * 16 + i) * GT + gtid];
                            dv[db][i] += ov[(db * 16 + i) * GT + gtid];
                        }
                }
            }
        }
        if (grp == 0 && key < N) {
            float* dkr = (float*)p.dk + kv_base + (size_t)key * D;
            float* dvr = (float*)p.dv + kv_base + (size_t)key * D;
            const float sc = p.scale;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int dd = 32 * db + 8 * i4 + 4 * g;
                    *(f32x4*)(dkr + dd) = f32x4{dk[db][4 * i4] * sc, dk[db][4 * i4 + 1] * sc,
                                                dk[db][4 * i4 + 2] * sc, dk[db][4 * i4 + 3] * sc};
                    *(f32x4*)(dvr + dd) = f32x4{dv[db][4 * i4], dv[db][4 * i4 + 1],
                                                dv[db][4 * i4 + 2], dv[db][4 * i4 + 3]};
                }
        }
        // The next tile of the item reuses every LDS buffer.
        __syncthreads();
    };

    // Paired: tile `item` (the longer one) and then tile n_kt-1-item, as two
    // trips of one loop (one copy of the body).
    const int n_kt = (N + BK - 1) / BK;
    const int n_rep = CAUSAL && L::kPaired && n_kt - 1 - item != item ? 2 : 1;
    for (int rp = 0; rp < n_rep; ++rp) process(rp == 0 ? item : n_kt - 1 - item);
}

// (3) dQ: work item (query tile(s), b*H + h); without pairing the longest
// tile first under a causal mask.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(FLayout<D>::kThreads, 1) void bwd_dq_f32_kernel(BwdParams p) {
    using L = FLayout<D>;
    constexpr int NG = L::kGroups;
    constexpr int QW = L::kWaves;
    constexpr int GT = L::kGroupThreads;
    constexpr int BQ = L::kBlock;
    using T = FTile<kFKStage, D>;
    using Cp = FCopy<kFKStage, D, QW>;
    constexpr int HALF = D / 2;
    constexpr int NDB = D / 32;
    constexpr int kMergeFloats = GT * NDB * 16;
    static_assert(NG == 1 || (NG - 1) * kMergeFloats * 4 <= NG * 4 * T::kBytes, "merge space");

    // Per group: K stage [2], V stage [2].
    __shared__ __attribute__((aligned(1024))) char kv_lds[NG * 4 * T::kBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = NG == 1 ? 0 : wave / QW;   // takes key stages j with j % NG == grp
    const int wq = wave - grp * QW;            // wave within the group
    const int gtid = tid - grp * GT;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;
    const int N = (int)p.N;

    LDS_AS char* const kvb = (LDS_AS char*)kv_lds + grp * 4 * T::kBytes;
    auto kL = [&](int par) { return kvb + par * T::kBytes; };
    auto vL = [&](int par) { return kvb + (2 + par) * T::kBytes; };

    const int n_qt = (N + BQ - 1) / BQ;
    const int w = blockIdx.x;
    const int item = w / p.BH;
    const int r = w - item * p.BH;
    const int kv_bh = r % p.BH_kv;
    const int bh = kv_bh * p.G + r / p.BH_kv;
    const size_t q_base = (size_t)bh * (size_t)N;
    const size_t kv_base = (size_t)kv_bh * (size_t)N * D;
    const float* Kg = (const float*)p.k + kv_base;
    const float* Vg = (const float*)p.v + kv_base;
    const float c2 = p.scale_log2;
    int coff[Cp::kPerWave];
    Cp::offsets(wq, lane, coff);

    auto process = [&](int tile) __attribute__((always_inline)) {
        const int q0 = tile * BQ;
        const int qw = q0 + 32 * wq;
        const int qi = qw + l32;
        const int qc = min(qi, N - 1);

        float qf[HALF], of[HALF];
#pragma unroll
        for (int c = 0; c < HALF / 4; ++c) {
            const f32x4 a = *(const f32x4*)((const float*)p.q + (q_base + qc) * D + g * HALF + 4 * c);
            const f32x4 b = *(const f32x4*)((const float*)p.dout + (q_base + qc) * D + g * HALF + 4 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qf[4 * c + e] = a[e];
                of[4 * c + e] = b[e];
            }
        }
        const float lq = p.lse[q_base + qc] * kLog2eF;
        const float neg_d = -p.delta[q_base + qc];

        const int n_tiles = ((CAUSAL ? min(q0 + BQ, N) : N) + kFKStage - 1) / kFKStage;
        const int n_iter = (n_tiles + NG - 1) / NG;

        f32x16 dq[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;

        if (grp < n_tiles) {
            Cp::copy(Kg, grp * kFKStage, N, kL(0), wq, coff);
            Cp::copy(Vg, grp * kFKStage, N, vL(0), wq, coff);
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);
        __syncthreads();
        for (int it = 0; it < n_iter; ++it) {
            const int par = it & 1;
            const int j = it * NG + grp;
            const int kv0 = j * kFKStage;
            if (j + NG < n_tiles) {
                Cp::copy(Kg, kv0 + NG * kFKStage, N, kL(par ^ 1), wq, coff);
                Cp::copy(Vg, kv0 + NG * kFKStage, N, vL(par ^ 1), wq, coff);
            }
            ATTN_PROBE(it);
            if (j < n_tiles && (!CAUSAL || kv0 <= qw + 31)) {
                const LDS_AS char* kb = kL(par);
                const LDS_AS char* vb = vL(par);
                // S^T[key][query] = K Q^T and E^T = V dO^T - D
                f32x16 s = {};
                f32x16 e;
#pragma unroll
                for (int i = 0; i < 16; ++i) e[i] = neg_d;
#pragma unroll
                for (int c = 0; c < HALF / 4; ++c) {
                    const f32x4 a = *(const LDS_AS f32x4*)(kb + T::chunk_off(l32, g * (HALF / 4) + c));
                    const f32x4 b = *(const LDS_AS f32x4*)(vb + T::chunk_off(l32, g * (HALF / 4) + c));
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        s = mfma_f32(a[x], qf[4 * c + x], s);
                        e = mfma_f32(b[x], of[4 * c + x], e);
                    }
                }
                // Entry i: key kv0 + 8(i/4) + 4g + i%4.
                const bool edge = (CAUSAL && kv0 + kFKStage - 1 > qw) || kv0 + kFKStage > N;
                if (edge) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int kk = kv0 + 8 * (i >> 2) + 4 * g + (i & 3);
                        if (kk >= N || (CAUSAL && kk > qi)) s[i] = -INFINITY;
                    }
                }
                float ds[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) ds[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -lq)) * e[i];
                // dQ^T[d][query] += K^T dS^T
#pragma unroll
                for (int kk = 0; kk < 16; ++kk) {
                    const int kr = 8 * (kk >> 2) + 4 * g + (kk & 3);
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const float a = *(const LDS_AS float*)(kb + T::elem_off(kr, 32 * db + l32));
                        dq[db] = mfma_f32(a, ds[kk], dq[db]);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0x0f70);
            ATTN_PROBE(it + 1);
            __syncthreads();
        }

        // Groups 1.. hand their partial dQ to group 0 (every stage read is
        // done); value k of thread t of group gg at float
        // (gg-1) * kMergeFloats + k * GT + t.
        if constexpr (NG > 1) {
            float* const mrg = (float*)kv_lds;
            if (grp != 0) {
                float* const my = mrg + (grp - 1) * kMergeFloats;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) my[(db * 16 + i) * GT + gtid] = dq[db][i];
            }
            __syncthreads();
            if (grp == 0) {
#pragma unroll
                for (int gg = 1; gg < NG; ++gg) {
                    const float* const other = mrg + (gg - 1) * kMergeFloats;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) dq[db][i] += other[(db * 16 + i) * GT + gtid];
                }
            }
        }
        if (grp == 0 && qi < N) {
            float* dqr = (float*)p.dq + (q_base + qi) * D;
            const float sc = p.scale;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int dd = 32 * db + 8 * i4 + 4 * g;
                    *(f32x4*)(dqr + dd) = f32x4{dq[db][4 * i4] * sc, dq[db][4 * i4 + 1] * sc,
                                                dq[db][4 * i4 + 2] * sc, dq[db][4 * i4 + 3] * sc};
                }
        }
        // The next tile of the item reuses every LDS buffer.
        __syncthreads();
    };

    // Causal: the longer tile n_qt-1-item first; paired, then tile `item`,
    // as a second trip of one loop (one copy of the body).
    const int first = CAUSAL ? n_qt - 1 - item : item;
    const int n_rep = CAUSAL && L::kPaired && item != first ? 2 : 1;
    for (int rp = 0; rp < n_rep; ++rp) process(rp == 0 ? first : item);
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdParams& p, hipStream_t s) {
    using L = FLayout<D>;
    constexpr int RPB = kFThreads / (D / 4);
    const int64_t rows = (int64_t)p.BH * p.N;
    hipLaunchKernelGGL((bwd_delta_f32_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)),
                       dim3(kFThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_t = (int)((p.N + L::kBlock - 1) / L::kBlock);
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL>),
                       dim3((unsigned)(f_items<D, CAUSAL>(n_t) * p.BH_kv)), dim3(L::kThreads), 0,
                       s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL>),
                       dim3((unsigned)(f_items<D, CAUSAL>(n_t) * p.BH)), dim3(L::kThreads), 0, s,
                       p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd32(const BwdParams& p, int d, bool causal, hipStream_t s) {
    if (d == 64) return causal ? launch<64, true>(p, s) : launch<64, false>(p, s);
    return causal ? launch<128, true>(p, s) : launch<128, false>(p, s);
}

}  // namespace attn
