// fwd_mfma16.hip — fused attention forward for bf16 / fp16 inputs on gfx950.
//
// Method (cited by page title and section):
//   [v2-naive] "Flash Attention（二）v2版本朴素实现 cuda core":
//     1.1  one workgroup owns a tile of query rows (outer loop) and streams
//          every K/V tile past it (inner loop);
//     1.2  the Q tile, the row max m and the row sum l stay on chip for the
//          whole inner loop; O is written to HBM once;
//     1.3  the accumulator is kept unnormalised and rescaled by
//          exp(m_old - m_new); one reciprocal of l per row at the end;
//     1.4 / 3.4  causal: K/V tiles wholly above the diagonal are never
//          visited; only tiles crossing it are masked element by element;
//     3.2  K/V tiles are double-buffered (the next tile's loads are in
//          flight while the current one is used); keys past N are
//          zero-filled and masked to -inf;
//     3.3  P is computed once per tile and reused for every output column.
//   [G7] "Flash Attention CUDA Kernel 优化: 从 56 到 986 TFLOPS on B300 —
//          G7: 回归 1CTA", lesson 6: exp is taken as exp2 with log2(e)
//          folded into the score scale.
//   [naive-attn] cishoon.github.io "flashattention", 3.5: shared-memory
//          bank conflicts are avoided by changing the layout (here an XOR
//          swizzle of 16-byte chunks instead of padding).
//
// gfx950 design (not the pages'):
//   * 256 threads = 4 wave64s; each wave owns 32 query rows; the workgroup
//     owns 128 rows. K/V tiles hold 64 keys.
//   * Both products use v_mfma_f32_32x32x16_{bf16,f16} with fp32
//     accumulation, in transposed form so that one lane owns one query:
//        S^T[key][query] = K . Q^T     (A = K rows from LDS, B = Q in VGPRs)
//        O^T[d][query]  += V^T . P^T   (A = V^T from LDS, B = P in VGPRs)
//     The 32x32 accumulator gives lane l the column l%32 (its query) and 16
//     rows (keys, or head-dim entries), so the row max / row sum of the
//     softmax are in-lane reductions plus one exchange with lane l^32, and
//     the per-row rescale of O is a per-lane scalar multiply.
//   * P leaves the S^T accumulator already in the B-operand shape of the
//     P.V product: the order of keys inside a contraction is free, so V^T is
//     stored in LDS with its keys permuted to match (see vt_pos()).
//   * Work items (b*H+h, query tile) are dispatched longest-first for causal
//     inputs, and consecutive workgroup ids map to different (b,h) slices so
//     that, with the round-robin placement of workgroups over the 8 XCDs,
//     every workgroup of one slice runs on the same XCD and shares its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"

namespace attn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLn2 = 0.693147180559945309f;

template <bool IS_BF16> struct Op16;

template <> struct Op16<true> {
    static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // Round two floats to bf16 (nearest even) and pack: x in the low half.
    static __device__ __forceinline__ uint32_t pack2(float x, float y) {
        bf16x2 v;
        v[0] = (__bf16)x;
        v[1] = (__bf16)y;
        return __builtin_bit_cast(uint32_t, v);
    }
    // acc + (both packed values): sums exactly what the P.V product consumes.
    static __device__ __forceinline__ float sum2(uint32_t pk, float acc) {
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), one, acc, false);
    }
};

template <> struct Op16<false> {
    static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float x, float y) {
        f16x2 v;
        v[0] = (_Float16)x;
        v[1] = (_Float16)y;
        return __builtin_bit_cast(uint32_t, v);
    }
    static __device__ __forceinline__ float sum2(uint32_t pk, float acc) {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), one, acc, false);
    }
};

constexpr int kBlockN = 64;   // keys per K/V tile
constexpr int kThreads = 256;

// Position of key `k` (0..63 inside a tile) in a V^T row. Bits 2 and 3 of the
// key index are swapped, so that the 8 keys one lane contributes to one
// 32x32x16 P.V step (keys 16a + 8b + 4g + e for b in {0,1}, e in 0..3, where
// g = lane/32) sit in 8 consecutive positions: one 16-byte LDS read.
__device__ __forceinline__ int vt_pos(int k) {
    return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <int D>
struct Smem {
    static constexpr int kRowBytes = D * 2;             // one K row
    static constexpr int kTileBytes = kBlockN * D * 2;  // one K tile == one V^T tile
    static constexpr int kVtRowBytes = kBlockN * 2;     // one V^T row (64 keys)
    static constexpr int kBytes = 4 * kTileBytes;       // K[2] + V^T[2]
};

// Byte offset of 16-byte chunk c of K row r: chunk index XOR (r mod 8), so the
// 8 lanes that read the same logical chunk of 8 consecutive rows hit 8
// different bank groups.
template <int D>
__device__ __forceinline__ int k_off(int r, int c) {
    return r * Smem<D>::kRowBytes + ((c ^ (r & 7)) << 4);
}

// Byte offset of 16-byte chunk pc of V^T row dd (same swizzle).
__device__ __forceinline__ int vt_off(int dd, int pc) {
    return dd * (kBlockN * 2) + ((pc ^ (dd & 7)) << 4);
}

template <bool IS_BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fwd16_kernel(FwdParams p) {
    using Op = Op16<IS_BF16>;
    using S = Smem<D>;
    constexpr int KCH = D / 8;                             // 16-byte chunks per row
    constexpr int K_ITEMS = kBlockN * KCH / kThreads;      // K chunks per thread
    constexpr int V_ITEMS = (kBlockN / 2) * KCH / kThreads;  // (key pair, chunk) per thread
    static_assert(K_ITEMS >= 1 && V_ITEMS >= 1, "tile / thread mismatch");

    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // Work item: longest query tiles first; consecutive ids -> different slices.
    const int w = blockIdx.x;
    const int tile = p.n_qtiles - 1 - w / p.BH;
    const int bh = w - (w / p.BH) * p.BH;
    const int N = (int)p.N;
    const int q0 = tile * kBlockM;
    const int qi = q0 + wave * 32 + l32;   // this lane's query row
    const size_t base = (size_t)bh * (size_t)N * D;

    const uint16_t* __restrict__ Qg = (const uint16_t*)p.q + base;
    const uint16_t* __restrict__ Kg = (const uint16_t*)p.k + base;
    const uint16_t* __restrict__ Vg = (const uint16_t*)p.v + base;

    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    // Q fragments (B operand of S^T = K Q^T): lane holds q[qi][16kd + 8g .. +7].
    u32x4 qf[D / 16];
#pragma unroll
    for (int kd = 0; kd < D / 16; ++kd)
        qf[kd] = qi < N ? *(const u32x4*)(Qg + (size_t)qi * D + 16 * kd + 8 * g) : zero4;

    const int kv_end = CAUSAL ? min(q0 + kBlockM, N) : N;
    const int n_tiles = (kv_end + kBlockN - 1) / kBlockN;

    // Register staging of the next K/V tile.
    u32x4 kreg[K_ITEMS];
    u32x4 vreg[V_ITEMS][2];

    auto load_tile = [&](int kv0) {
#pragma unroll
        for (int it = 0; it < K_ITEMS; ++it) {
            const int item = tid + kThreads * it;
            const int r = item / KCH, c = item % KCH;
            const int key = kv0 + r;
            kreg[it] = key < N ? *(const u32x4*)(Kg + (size_t)key * D + 8 * c) : zero4;
        }
#pragma unroll
        for (int it = 0; it < V_ITEMS; ++it) {
            const int item = tid + kThreads * it;
            const int c = item / (kBlockN / 2), pp = item % (kBlockN / 2);
            const int key = kv0 + 2 * pp;
            vreg[it][0] = key < N ? *(const u32x4*)(Vg + (size_t)key * D + 8 * c) : zero4;
            vreg[it][1] = key + 1 < N ? *(const u32x4*)(Vg + (size_t)(key + 1) * D + 8 * c) : zero4;
        }
    };

    auto store_tile = [&](int buf) {
        char* ks = smem + buf * S::kTileBytes;
        char* vt = smem + (2 + buf) * S::kTileBytes;
#pragma unroll
        for (int it = 0; it < K_ITEMS; ++it) {
            const int item = tid + kThreads * it;
            const int r = item / KCH, c = item % KCH;
            *(u32x4*)(ks + k_off<D>(r, c)) = kreg[it];
        }
#pragma unroll
        for (int it = 0; it < V_ITEMS; ++it) {
            const int item = tid + kThreads * it;
            const int c = item / (kBlockN / 2), pp = item % (kBlockN / 2);
            const int pos = vt_pos(2 * pp);          // keys 2pp, 2pp+1 stay adjacent
            const int pc = pos >> 3, pw = (pos & 7) * 2;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int dd = 8 * c + jj;
                const uint32_t x = vreg[it][0][jj >> 1], y = vreg[it][1][jj >> 1];
                const uint32_t word = (jj & 1) ? ((x >> 16) | (y & 0xffff0000u))
                                               : ((x & 0xffffu) | (y << 16));
                *(uint32_t*)(vt + vt_off(dd, pc) + pw) = word;
            }
        }
    };

    const float c2 = p.scale_log2;
    float m_run = -INFINITY;   // running row max of the scaled (log2) scores
    float l_run = 0.f;         // this lane's half of the running row sum
    f32x16 o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int j = 0; j < n_tiles; ++j) {
        const int cur = j & 1;
        const int kv0 = j * kBlockN;
        if (j + 1 < n_tiles) load_tile(kv0 + kBlockN);

        // Causal: a tile that starts past this wave's last row contributes
        // nothing to it (wave-uniform branch).
        const bool wave_live = !CAUSAL || kv0 <= q0 + wave * 32 + 31;
        if (wave_live) {
            const char* ks = smem + cur * S::kTileBytes;
            const char* vt = smem + (2 + cur) * S::kTileBytes;

            // S^T = K Q^T for 2 blocks of 32 keys.
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
                const int r = 32 * kb + l32;
#pragma unroll
                for (int kd = 0; kd < D / 16; ++kd) {
                    const u32x4 a = *(const u32x4*)(ks + k_off<D>(r, 2 * kd + g));
                    s[kb] = Op::mfma(a, qf[kd], s[kb]);
                }
            }

            // Element masks only on tiles that cross the diagonal or N.
            const bool diag = CAUSAL && (kv0 + kBlockN - 1 > q0);
            const bool tail = kv0 + kBlockN > N;
            if (diag || tail) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kv0 + 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
                        const bool dead = key >= N || (CAUSAL && key > qi);
                        if (dead) s[kb][i] = -INFINITY;
                    }
            }

            // Online softmax in the log2 domain.
            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float m_new = fmaxf(m_run, mx * c2);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);

            uint32_t pk[2][8];
            float lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; i += 2) {
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][i], c2, -m_use));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][i + 1], c2, -m_use));
                    pk[kb][i >> 1] = Op::pack2(p0, p1);
                    lsum = Op::sum2(pk[kb][i >> 1], lsum);
                }
            l_run = alpha * l_run + lsum;
            m_run = m_new;

#pragma unroll
            for (int db = 0; db < D / 32; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;

            // O^T += V^T P^T, four steps of 16 keys per 32 head-dim rows.
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
                const int rr = 32 * db + l32;
#pragma unroll
                for (int kb2 = 0; kb2 < 4; ++kb2) {
                    const u32x4 a = *(const u32x4*)(vt + vt_off(rr, 2 * kb2 + g));
                    const int h = 4 * (kb2 & 1);
                    const u32x4 b = {pk[kb2 >> 1][h], pk[kb2 >> 1][h + 1],
                                     pk[kb2 >> 1][h + 2], pk[kb2 >> 1][h + 3]};
                    o[db] = Op::mfma(a, b, o[db]);
                }
            }
        }

        if (j + 1 < n_tiles) store_tile(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: O = O~ / l, rounded once to the output type; lse in fp32.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    if (qi < N) {
        uint16_t* Og = (uint16_t*)p.o + base + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int dd = 32 * db + 8 * i4 + 4 * g;
                const u32x2 wv = {Op::pack2(o[db][4 * i4] * inv, o[db][4 * i4 + 1] * inv),
                                  Op::pack2(o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv)};
                *(u32x2*)(Og + dd) = wv;
            }
        if (g == 0) p.lse[(size_t)bh * N + qi] = (m_run + log2f(l_tot)) * kLn2;
    }
}

template <bool IS_BF16, int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, hipStream_t s) {
    const dim3 grid((unsigned)(p.n_qtiles * p.BH));
    hipLaunchKernelGGL((fwd16_kernel<IS_BF16, D, CAUSAL>), grid, dim3(kThreads),
                       Smem<D>::kBytes, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd16(const FwdParams& p, bool is_bf16, int d, bool causal, hipStream_t s) {
    if (is_bf16) {
        if (d == 64) return causal ? launch<true, 64, true>(p, s) : launch<true, 64, false>(p, s);
        return causal ? launch<true, 128, true>(p, s) : launch<true, 128, false>(p, s);
    }
    if (d == 64) return causal ? launch<false, 64, true>(p, s) : launch<false, 64, false>(p, s);
    return causal ? launch<false, 128, true>(p, s) : launch<false, 128, false>(p, s);
}

}  // namespace attn
