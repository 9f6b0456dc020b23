// fwd_f32.hip — fused attention forward for fp32 inputs on gfx950.
//
// Same method as the bf16/fp16 kernel (Q-tile outer loop, K/V-tile inner
// loop, online softmax with deferred 1/l, causal tile skipping and diagonal
// masking — "Flash Attention（二）v2版本朴素实现 cuda core", sections 1.1-1.4
// and 3.2-3.5, whose kernel is itself fp32), with every product on the fp32
// matrix cores (v_mfma_f32_32x32x2_f32): gfx950 has no reduced-precision
// (xf32) fp32 MFMA, so scores and P.V are exact fp32 products accumulated in
// fp32 and P is never rounded below fp32.
//
// Layout: 8 wave64s in NG groups (NG = 4 at d = 64, 2 at d = 128) of 8/NG
// waves x 32 query rows; K/V tiles of 32 keys. The groups own the same
// query tile (64 rows at d = 64, 128 at d = 128) and take K/V tiles in turn
// (tile j goes to group j mod NG, each group with its own LDS buffers), so
// the sequential length of a work item is 1/NG of its tiles; at the end
// groups 1.. hand their running (m, l, O) to group 0, which merges them by
// the online-softmax rule (the rescale of "Flash Attention（二）v2版本朴素实现
// cuda core", section 1.3, applied across the partial results).
// Under a causal mask a work item is the pair of query tiles t and T-1-t of
// one slice (T tiles per slice), processed one after the other: every item
// then holds the same number of key tiles, so a grid of about one item per
// compute unit finishes together instead of waiting for its longest item.
// One lane owns one query, as in the 16-bit kernel:
//   S^T[key][query] = K . Q^T : the contraction over d is split so that lane
//       half g takes d in [g*D/2, (g+1)*D/2): each lane reads D/2 contiguous
//       floats of a K row (16-byte LDS reads) and keeps D/2 floats of Q.
//   O^T[d][query] += V^T . P^T : contraction step kk uses accumulator row kk
//       of S^T as the B operand as is; the A operand is the matching key's V
//       row, read straight from row-major LDS (lanes 0-31 read 32 consecutive
//       floats of one key row).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLn2 = 0.693147180559945309f;
constexpr int kBlockN = 32;
constexpr int kThreads = 512;   // 8 waves

template <int D>
struct Smem32 {
    static constexpr int kGroups = D == 64 ? 4 : 2;        // K/V-tile groups
    static constexpr int kGroupThreads = kThreads / kGroups;
    static constexpr int kBlockM = kGroupThreads / 2;      // query rows: 32 per wave
    static constexpr int kRowBytes = D * 4;
    static constexpr int kTileBytes = kBlockN * D * 4;
    static constexpr int kGroupBytes = 4 * kTileBytes;   // K[2] + V[2] of one group
    static constexpr int kBytes = kGroups * kGroupBytes;
    // merge: (O, m, l) of groups 1 .. kGroups-1
    static constexpr int kMergeFloats = (D / 2 + 2) * kGroupThreads;
    static_assert((kGroups - 1) * kMergeFloats * 4 <= kBytes, "merge space");
};

// K rows: 16-byte chunk c of row r stored at chunk c ^ (r mod 8).
template <int D>
__device__ __forceinline__ int k_off32(int r, int c) {
    return r * Smem32<D>::kRowBytes + ((c ^ (r & 7)) << 4);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd32_kernel(FwdParams p) {
    using S = Smem32<D>;
    constexpr int NG = S::kGroups;
    constexpr int GT = S::kGroupThreads;
    constexpr int BM = S::kBlockM;
    constexpr int CH = D / 4;                          // 16-byte chunks per row
    constexpr int ITEMS = kBlockN * CH / GT;           // chunks per thread per tensor
    constexpr int HALF = D / 2;
    static_assert(ITEMS >= 1 && kBlockN * CH % GT == 0, "tile / thread mismatch");

    __shared__ __attribute__((aligned(16))) char smem_all[S::kBytes];

    const int grp = threadIdx.x / GT;   // takes K/V tiles j with j % NG == grp
    const int tid = threadIdx.x % GT;   // thread within the group
    char* const smem = smem_all + grp * S::kGroupBytes;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // Work item: one query tile (no mask) or the pair T-1-t, t (causal);
    // consecutive ids -> different slices.
    const int w = blockIdx.x;
    const int pair = w / p.BH;
    const SliceIds ids = slice_of(p, w - pair * p.BH);
    const int bh = ids.bh;
    const int N = (int)p.N;
    const size_t base = (size_t)bh * (size_t)N * D;
    const size_t kv_base = (size_t)ids.kv_bh * (size_t)N * D;

    const float* __restrict__ Qg = (const float*)p.q + base;
    const float* __restrict__ Kg = (const float*)p.k + kv_base;
    const float* __restrict__ Vg = (const float*)p.v + kv_base;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    auto process_tile = [&](int tile) __attribute__((always_inline)) {
        const int q0 = tile * BM;
        const int qi = q0 + wave * 32 + l32;

        // Q half-row of this lane: q[qi][g*D/2 .. g*D/2 + D/2 - 1].
        float qf[HALF];
#pragma unroll
        for (int c = 0; c < HALF / 4; ++c) {
            const f32x4 t = qi < N ? *(const f32x4*)(Qg + (size_t)qi * D + g * HALF + 4 * c) : zero4;
            qf[4 * c + 0] = t[0];
            qf[4 * c + 1] = t[1];
            qf[4 * c + 2] = t[2];
            qf[4 * c + 3] = t[3];
        }

        const int kv_end = CAUSAL ? min(q0 + BM, N) : N;
        const int n_tiles = (kv_end + kBlockN - 1) / kBlockN;

        f32x4 kreg[ITEMS], vreg[ITEMS];
        auto load_tile = [&](int kv0) {
#pragma unroll
            for (int it = 0; it < ITEMS; ++it) {
                const int item = tid + GT * it;
                const int r = item / CH, c = item % CH;
                const int key = kv0 + r;
                kreg[it] = key < N ? *(const f32x4*)(Kg + (size_t)key * D + 4 * c) : zero4;
                vreg[it] = key < N ? *(const f32x4*)(Vg + (size_t)key * D + 4 * c) : zero4;
            }
        };
        auto store_tile = [&](int buf) {
            char* ks = smem + buf * S::kTileBytes;
            char* vs = smem + (2 + buf) * S::kTileBytes;
#pragma unroll
            for (int it = 0; it < ITEMS; ++it) {
                const int item = tid + GT * it;
                const int r = item / CH, c = item % CH;
                *(f32x4*)(ks + k_off32<D>(r, c)) = kreg[it];
                *(f32x4*)(vs + r * S::kRowBytes + 16 * c) = vreg[it];
            }
        };

        const float c2 = p.scale_log2;
        float m_run = -INFINITY;
        float l_run = 0.f;
        f32x16 o[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] = 0.f;

        // Iteration it: this group's tile j = NG it + grp. Every group runs
        // n_iter iterations with one barrier each.
        const int n_iter = (n_tiles + NG - 1) / NG;
        if (grp < n_tiles) {
            load_tile(grp * kBlockN);
            store_tile(0);
        }
        __syncthreads();

        for (int it = 0; it < n_iter; ++it) {
            const int cur = it & 1;
            const int j = NG * it + grp;
            const int kv0 = j * kBlockN;
            const bool next = j + NG < n_tiles;
            if (next) load_tile(kv0 + NG * kBlockN);
            ATTN_PROBE(it);

            const bool wave_live = j < n_tiles && (!CAUSAL || kv0 <= q0 + wave * 32 + 31);
            if (wave_live) {
                const char* ks = smem + cur * S::kTileBytes;
                const float* vs = (const float*)(smem + (2 + cur) * S::kTileBytes);

                f32x16 s;
#pragma unroll
                for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
                for (int c = 0; c < HALF / 4; ++c) {
                    const f32x4 a = *(const f32x4*)(ks + k_off32<D>(l32, g * (HALF / 4) + c));
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[4 * c + e], s, 0, 0, 0);
                }

                const bool diag = CAUSAL && (kv0 + kBlockN - 1 > q0);
                const bool tail = kv0 + kBlockN > N;
                if (diag || tail) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kv0 + 8 * (i >> 2) + 4 * g + (i & 3);
                        const bool dead = key >= N || (CAUSAL && key > qi);
                        if (dead) s[i] = -INFINITY;
                    }
                }

                float mx = s[0];
#pragma unroll
                for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float m_new = fmaxf(m_run, mx * c2);
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);

                float lsum = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c2, -m_use));
                    lsum += s[i];
                }
                l_run = alpha * l_run + lsum;
                m_run = m_new;

#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[db][i] *= alpha;

                // Step kk: lane half g contributes key 8(kk/4) + 4g + kk%4, whose
                // probability is accumulator entry kk of this lane.
#pragma unroll
                for (int kk = 0; kk < 16; ++kk) {
                    const int key = 8 * (kk >> 2) + 4 * g + (kk & 3);
#pragma unroll
                    for (int db = 0; db < D / 32; ++db) {
                        const float a = vs[key * D + 32 * db + l32];
                        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kk], o[db], 0, 0, 0);
                    }
                }
            }

            ATTN_PROBE(it + 1);
            if (next) store_tile(cur ^ 1);
            __syncthreads();
        }

        // Merge: the (m, l, O) of groups 1 .. NG-1 through LDS (every tile read
        // is done); value k of thread t of group gg at float
        // (gg-1) * kMergeFloats + k * GT + t. Group 0 folds them in one by one.
        float* const mrg = (float*)smem_all;
        if (grp != 0) {
            float* const my = mrg + (grp - 1) * S::kMergeFloats;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) my[(db * 16 + i) * GT + tid] = o[db][i];
            my[(D / 2) * GT + tid] = m_run;
            my[(D / 2 + 1) * GT + tid] = l_run;
        }
        __syncthreads();
        if (grp == 0) {
#pragma unroll
            for (int gg = 1; gg < NG; ++gg) {
                const float* const other = mrg + (gg - 1) * S::kMergeFloats;
                const float m1 = other[(D / 2) * GT + tid];
                const float l1 = other[(D / 2 + 1) * GT + tid];
                const float m = fmaxf(m_run, m1);
                const float m_use = m == -INFINITY ? 0.f : m;
                const float a0 = __builtin_amdgcn_exp2f(m_run - m_use);
                const float a1 = __builtin_amdgcn_exp2f(m1 - m_use);
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        o[db][i] = o[db][i] * a0 + other[(db * 16 + i) * GT + tid] * a1;
                l_run = l_run * a0 + l1 * a1;
                m_run = m;
            }

            const float l_tot = l_run + __shfl_xor(l_run, 32);
            const float inv = 1.f / l_tot;
            if (qi < N) {
                float* Og = (float*)p.o + base + (size_t)qi * D;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) {
                        const int dd = 32 * db + 8 * i4 + 4 * g;
                        const f32x4 wv = {o[db][4 * i4] * inv, o[db][4 * i4 + 1] * inv,
                                          o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv};
                        *(f32x4*)(Og + dd) = wv;
                    }
                if (g == 0) p.lse[(size_t)bh * N + qi] = (m_run + log2f(l_tot)) * kLn2;
            }
        }   // group 0
        // The next tile of the item reuses the LDS that the merge read.
        __syncthreads();
    };

    if (CAUSAL) {
        const int ta = p.n_qtiles - 1 - pair;   // the longer tile first
        process_tile(ta);
        if (pair != ta) process_tile(pair);
    } else {
        process_tile(pair);
    }
}

template <int D, bool CAUSAL>
hipError_t launch(FwdParams p, hipStream_t s) {
    constexpr int BM = Smem32<D>::kBlockM;
    p.n_qtiles = (int)((p.N + BM - 1) / BM);
    // causal: pairs (T-1-t, t), the middle tile alone when T is odd
    const int items = CAUSAL ? (p.n_qtiles + 1) / 2 : p.n_qtiles;
    const dim3 grid((unsigned)(items * p.BH));
    hipLaunchKernelGGL((fwd32_kernel<D, CAUSAL>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd32(const FwdParams& p, int d, bool causal, hipStream_t s) {
    if (d == 64) return causal ? launch<64, true>(p, s) : launch<64, false>(p, s);
    return causal ? launch<128, true>(p, s) : launch<128, false>(p, s);
}

}  // namespace attn
