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
// one slice (T tiles per slice): every item then holds the same number of
// key tiles, so a grid of about one item per compute unit finishes together
// instead of waiting for its longest item. At d = 64 the pair runs in one
// pass over the longer tile's keys (the shorter tile's keys are a prefix of
// them): both tiles' Q and O stay in registers, every K fragment and V row
// read from LDS feeds both tiles' MFMAs while the shorter one is live, and
// the item has one prologue and one loop (+6 % at B1 H32 N1024 against the
// two tiles one after the other). At d = 128 the registers hold one tile,
// and the two run one after the other.
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

#include <type_traits>

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

    // Query tiles of the work item: at most two (the causal pair at d = 64,
    // see run_item); block b's rows start at q0[b], this lane's row is qi[b].
    constexpr int NQ_MAX = (D == 64 && CAUSAL) ? 2 : 1;
    float qf[NQ_MAX][HALF];   // Q half-row of this lane: q[qi][g*D/2 .. +D/2-1]
    float m_run[NQ_MAX], l_run[NQ_MAX];
    f32x16 o[NQ_MAX][D / 32];
    int q0[NQ_MAX], qi[NQ_MAX];

    auto start_block = [&](int b, int tile) __attribute__((always_inline)) {
        q0[b] = tile * BM;
        qi[b] = q0[b] + wave * 32 + l32;
#pragma unroll
        for (int c = 0; c < HALF / 4; ++c) {
            const f32x4 t = qi[b] < N ? *(const f32x4*)(Qg + (size_t)qi[b] * D + g * HALF + 4 * c) : zero4;
            qf[b][4 * c + 0] = t[0];
            qf[b][4 * c + 1] = t[1];
            qf[b][4 * c + 2] = t[2];
            qf[b][4 * c + 3] = t[3];
        }
        m_run[b] = -INFINITY;
        l_run[b] = 0.f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[b][db][i] = 0.f;
    };

    f32x4 kreg[ITEMS], vreg[ITEMS];
    auto load_tile = [&](int kv0) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int item = tid + GT * it;
            const int r = item / CH, c = item % CH;
            const int key = kv0 + r;
            kreg[it] = key < N ? *(const f32x4*)(Kg + (size_t)key * D + 4 * c) : zero4;
            vreg[it] = key < N ? *(const f32x4*)(Vg + (size_t)key * D + 4 * c) : zero4;
        }
    };
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
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

    // One 32-key tile for query blocks 0 .. NQ-1 (every block live for this
    // wave): each K fragment and each V row read from LDS feeds NQ MFMAs.
    auto tile_step = [&](auto nq_tag, int kv0, const char* ks, const float* vs) __attribute__((always_inline)) {
        constexpr int NQ = decltype(nq_tag)::value;
        f32x16 sc[NQ];
#pragma unroll
        for (int b = 0; b < NQ; ++b)
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[b][i] = 0.f;
#pragma unroll
        for (int c = 0; c < HALF / 4; ++c) {
            const f32x4 a = *(const f32x4*)(ks + k_off32<D>(l32, g * (HALF / 4) + c));
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int b = 0; b < NQ; ++b)
                    sc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[b][4 * c + e], sc[b], 0, 0, 0);
        }

#pragma unroll
        for (int b = 0; b < NQ; ++b) {
            const bool diag = CAUSAL && (kv0 + kBlockN - 1 > q0[b]);
            const bool tail = kv0 + kBlockN > N;
            if (diag || tail) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kv0 + 8 * (i >> 2) + 4 * g + (i & 3);
                    const bool dead = key >= N || (CAUSAL && key > qi[b]);
                    if (dead) sc[b][i] = -INFINITY;
                }
            }

            float mx = sc[b][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[b][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run[b], mx * c2);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run[b] - m_use);

            float lsum = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                sc[b][i] = __builtin_amdgcn_exp2f(fmaf(sc[b][i], c2, -m_use));
                lsum += sc[b][i];
            }
            l_run[b] = alpha * l_run[b] + lsum;
            m_run[b] = m_new;

#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[b][db][i] *= alpha;
        }

        // Step kk: lane half g contributes key 8(kk/4) + 4g + kk%4, whose
        // probability is accumulator entry kk of this lane.
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const int key = 8 * (kk >> 2) + 4 * g + (kk & 3);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const float a = vs[key * D + 32 * db + l32];
#pragma unroll
                for (int b = 0; b < NQ; ++b)
                    o[b][db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sc[b][kk], o[b][db], 0, 0, 0);
            }
        }
    };

    // Merge of block b: the (m, l, O) of groups 1 .. NG-1 through LDS (every
    // tile read is done); value k of thread t of group gg at float
    // (gg-1) * kMergeFloats + k * GT + t. Group 0 folds them in one by one
    // and writes O and lse.
    auto merge_store = [&](int b) __attribute__((always_inline)) {
        float* const mrg = (float*)smem_all;
        if (grp != 0) {
            float* const my = mrg + (grp - 1) * S::kMergeFloats;
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) my[(db * 16 + i) * GT + tid] = o[b][db][i];
            my[(D / 2) * GT + tid] = m_run[b];
            my[(D / 2 + 1) * GT + tid] = l_run[b];
        }
        __syncthreads();
        if (grp == 0) {
            float m_b = m_run[b], l_b = l_run[b];
#pragma unroll
            for (int gg = 1; gg < NG; ++gg) {
                const float* const other = mrg + (gg - 1) * S::kMergeFloats;
                const float m1 = other[(D / 2) * GT + tid];
                const float l1 = other[(D / 2 + 1) * GT + tid];
                const float m = fmaxf(m_b, m1);
                const float m_use = m == -INFINITY ? 0.f : m;
                const float a0 = __builtin_amdgcn_exp2f(m_b - m_use);
                const float a1 = __builtin_amdgcn_exp2f(m1 - m_use);
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        o[b][db][i] = o[b][db][i] * a0 + other[(db * 16 + i) * GT + tid] * a1;
                l_b = l_b * a0 + l1 * a1;
                m_b = m;
            }

            const float l_tot = l_b + __shfl_xor(l_b, 32);
            const float inv = 1.f / l_tot;
            if (qi[b] < N) {
                float* Og = (float*)p.o + base + (size_t)qi[b] * D;
#pragma unroll
                for (int db = 0; db < D / 32; ++db)
#pragma unroll
                    for (int i4 = 0; i4 < 4; ++i4) {
                        const int dd = 32 * db + 8 * i4 + 4 * g;
                        const f32x4 wv = {o[b][db][4 * i4] * inv, o[b][db][4 * i4 + 1] * inv,
                                          o[b][db][4 * i4 + 2] * inv, o[b][db][4 * i4 + 3] * inv};
                        *(f32x4*)(Og + dd) = wv;
                    }
                if (g == 0) p.lse[(size_t)bh * N + qi[b]] = (m_b + log2f(l_tot)) * kLn2;
            }
        }   // group 0
        // The LDS the merge read is reused next.
        __syncthreads();
    };

    // One work item: query tile ta, and with `two` also tile tb < ta of the
    // same slice in the same pass over ta's keys (tb's keys are a prefix of
    // them), so the pair shares every K/V tile, one prologue and one loop.
    auto run_item = [&](int ta, int tb, bool two) __attribute__((always_inline)) {
        start_block(0, ta);
        if constexpr (NQ_MAX == 2) {
            if (two) start_block(1, tb);
        }
        const int kv_end = CAUSAL ? min(q0[0] + BM, N) : N;
        const int n_tiles = (kv_end + kBlockN - 1) / kBlockN;
        int n_tiles_b = 0;
        if constexpr (NQ_MAX == 2) {
            if (two) n_tiles_b = (min(q0[1] + BM, N) + kBlockN - 1) / kBlockN;
        }

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

            // Block 0 (the longer tile) is live for every key tile that block
            // 1 sees, since its rows all follow block 1's.
            const bool live_a = j < n_tiles && (!CAUSAL || kv0 <= q0[0] + wave * 32 + 31);
            bool live_b = false;
            if constexpr (NQ_MAX == 2) live_b = j < n_tiles_b && kv0 <= q0[1] + wave * 32 + 31;
            if (live_a) {
                const char* ks = smem + cur * S::kTileBytes;
                const float* vs = (const float*)(smem + (2 + cur) * S::kTileBytes);
                if constexpr (NQ_MAX == 2) {
                    if (live_b) tile_step(std::integral_constant<int, 2>{}, kv0, ks, vs);
                    else tile_step(std::integral_constant<int, 1>{}, kv0, ks, vs);
                } else {
                    tile_step(std::integral_constant<int, 1>{}, kv0, ks, vs);
                }
            }

            ATTN_PROBE(it + 1);
            if (next) store_tile(cur ^ 1);
            __syncthreads();
        }

        merge_store(0);
        if constexpr (NQ_MAX == 2) {
            if (two) merge_store(1);
        }
    };

    if (CAUSAL) {
        const int ta = p.n_qtiles - 1 - pair;   // the longer tile first
        if constexpr (NQ_MAX == 2) {
            run_item(ta, pair, pair != ta);
        } else {
            run_item(ta, 0, false);
            if (pair != ta) run_item(pair, 0, false);
        }
    } else {
        run_item(pair, 0, false);
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
