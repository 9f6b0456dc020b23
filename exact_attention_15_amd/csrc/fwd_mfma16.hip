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
//     3.2  K/V tiles are double-buffered (the next tiles' loads are in
//          flight while the current ones are used); keys past N are masked
//          to -inf and never meet a non-finite V value;
//     3.3  P is computed once per tile and reused for every output column.
//   [G7] "Flash Attention CUDA Kernel 优化: 从 56 到 986 TFLOPS on B300 —
//          G7: 回归 1CTA": exp is taken as exp2 with log2(e) folded into the
//          score scale (lesson 6); QK^T and P.V of different tiles are issued
//          so that they interleave with the softmax (V45, V50); the rescale
//          of the accumulator is made conditional (carried over from G6).
//   [naive-attn] cishoon.github.io "flashattention", 3.5: shared-memory bank
//          conflicts are removed by the layout (here XOR swizzles of 16-byte
//          chunks instead of padding).
//
// gfx950 design (not the pages'):
//   * 256 threads = 4 wave64s; each wave owns 32 query rows; the workgroup
//     owns 128 rows. K/V tiles hold 64 keys.
//   * Both products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32
//     accumulation, in transposed form so that one lane owns one query:
//        S^T[key][query] = K . Q^T     (A = K rows from LDS, B = Q in VGPRs)
//        O^T[d][query]  += V^T . P^T   (A = V^T from LDS, B = P in VGPRs)
//     The 32x32 accumulator gives lane l the column l%32 (its query) and 16
//     rows (keys, or head-dim entries), so the softmax row max / row sum are
//     in-lane reductions plus one v_permlane32_swap, and the rescale of O is
//     a per-lane scalar multiply.
//   * P leaves the S^T accumulator already in the B-operand layout of the
//     P.V product (the order of keys inside a contraction is free); the
//     matching V^T operand is read from row-major V in LDS with
//     ds_read_b64_tr_b16, two reads per MFMA.
//   * K and V tiles go from HBM straight into LDS (global_load_lds_dwordx4,
//     16 bytes per lane, no VGPR staging); the XOR swizzle is applied by
//     choosing which global chunk each lane fetches.
//   * Software pipeline inside each wave: iteration j issues the MFMAs of
//     S(j+1) = K(j+1) Q^T and of O += P(j-1) V(j-1), neither of which depends
//     on the softmax of tile j that runs on the VALU in the same iteration,
//     so matrix and vector work overlap without relying on other waves.
//   * Lazy rescale: the exponent base m only moves when a tile's row max
//     exceeds it by more than 2^8 in probability; otherwise P <= 256 is used
//     as is. The final O / l is unchanged by the choice of base, and a
//     bf16/fp16 P keeps its relative precision at that magnitude.
//   * Work items (b*H+h, query tile) are dispatched longest-first for causal
//     inputs; consecutive workgroup ids map to different (b,h) slices so,
//     with the round-robin placement of workgroups over the 8 XCDs, all
//     workgroups of one slice share one XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
typedef __attribute__((ext_vector_type(4))) short i16x4;

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kRescaleThreshold = 8.0f;   // log2 units: P may reach 2^8
constexpr int kBlockN = 64;                 // keys per K/V tile
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

#ifndef ATTN_L_MFMA
#define ATTN_L_MFMA 0
#endif

#ifndef ATTN_MFMA_PREFETCH
#define ATTN_MFMA_PREFETCH 0
#endif

#ifndef ATTN_PP_MODE
#define ATTN_PP_MODE 0
#endif

#ifndef ATTN_PINGPONG
#define ATTN_PINGPONG 1
#endif

#ifndef ATTN_WAVES_PER_SIMD
#define ATTN_WAVES_PER_SIMD 1
#endif

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
    // acc + both packed values: sums exactly what the P.V product consumes.
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

// LDS layout of one K or V tile: 64 rows of D 16-bit values, row-major, with
// 16-byte chunk c of row r stored at chunk c ^ swz(r).
//  * K is read 16 bytes per lane, one row per lane, 16 lanes per LDS cycle:
//    rows r..r+15 at one logical chunk must land in 16 different 16-byte bank
//    groups (64 banks x 4 bytes).
//  * V is read with ds_read_b64_tr_b16: 32 lanes read 4 consecutive rows x
//    64 contiguous bytes; rows 2 apart (D = 64) or adjacent rows (D = 128)
//    would otherwise share banks.
template <int D, int WAVES = kWaves>
struct Tile {
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;             // 16-byte chunks per row
    static constexpr int kBytes = kBlockN * kRowBytes;
    static constexpr int kLoadsPerWave = kBytes / 1024 / WAVES;    // 1 KiB per wave load
    static __device__ __forceinline__ int swz_k(int r) { return D == 64 ? (r >> 1) & 7 : r & 15; }
    static __device__ __forceinline__ int swz_v(int r) { return D == 64 ? ((r >> 1) & 1) << 2 : (r & 3) << 2; }
};

// Per-lane byte offsets, inside a tile, of the 16-byte global chunks this
// lane copies: load u of wave `wave` fills LDS chunk slots
// s = (wave*U + u)*64 + lane, i.e. row s / kChunks, physical chunk
// s % kChunks, holding the global chunk (physical ^ swz(row)).
template <int D, bool IS_V, int WAVES = kWaves>
__device__ __forceinline__ void tile_src_offsets(int wave, int lane, int* off) {
    using T = Tile<D, WAVES>;
#pragma unroll
    for (int u = 0; u < T::kLoadsPerWave; ++u) {
        const int s = (wave * T::kLoadsPerWave + u) * 64 + lane;
        const int r = s / T::kChunks;
        const int pc = s % T::kChunks;
        const int lc = pc ^ (IS_V ? T::swz_v(r) : T::swz_k(r));
        off[u] = r * T::kRowBytes + lc * 16;
    }
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// One 16-byte-per-lane HBM -> LDS copy (buffer_load_dwordx4 ... lds): lane l
// writes LDS bytes [lds_addr + 16 l, +16). Issued from inline assembly so
// that the compiler does not guard later LDS reads of *other* buffers with a
// wait for the copy; every wait for these copies is explicit (vmcnt(0)
// before the barrier that publishes a tile). The compiler's own vmcnt
// accounting stays safe: extra outstanding loads only make its waits longer.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_addr, int voffset) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voffset), "s"(rsrc)
                 : "memory", "m0");
}

// Issue this wave's share of the direct HBM -> LDS copy of one K or V tile
// (keys kv0 .. kv0+63). The buffer descriptor covers rows kv0 .. N-1 only,
// so chunks of rows past N are out of range and arrive as zeros (the
// zero-fill of the pages' asynchronous copy); their scores are masked.
template <int D, int WAVES = kWaves>
__device__ __forceinline__ void load_tile(const uint16_t* g_slice, int kv0, int N, LDS_AS char* buf,
                                          int wave, const int* off) {
    using T = Tile<D, WAVES>;
    const int rows = max(N - kv0, 0);
    const uint64_t addr = (uint64_t)(g_slice + (size_t)kv0 * D);
    i32x4 rsrc;
    rsrc[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    rsrc[1] = __builtin_amdgcn_readfirstlane((int)((addr >> 32) & 0xffff));   // stride 0
    rsrc[2] = __builtin_amdgcn_readfirstlane(rows * T::kRowBytes);            // bytes in range
    rsrc[3] = 0x00020000;                                                     // 32-bit data format
    const uint32_t lds0 = (uint32_t)(uintptr_t)buf;
#pragma unroll
    for (int u = 0; u < T::kLoadsPerWave; ++u) {
        const int slot0 = (wave * T::kLoadsPerWave + u) * 64;
        dma16(rsrc, lds0 + slot0 * 16, off[u]);
    }
}

__device__ __forceinline__ float wave_half_max(float x) {
    // v_permlane32_swap(x, x): lanes < 32 get (x[l], x[l+32]), lanes >= 32 get
    // (x[l-32], x[l]); the max of the pair is the max over lanes l and l^32.
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)r[0]),
                                         __builtin_bit_cast(float, (uint32_t)r[1]));
}

__device__ __forceinline__ float wave_half_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

template <bool IS_BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, ATTN_WAVES_PER_SIMD) void fwd16_kernel(FwdParams p) {
    using Op = Op16<IS_BF16>;
    using T = Tile<D>;
    constexpr int NKD = D / 16;   // QK^T contraction steps
    constexpr int NDB = D / 32;   // 32-row blocks of O^T

    // Four distinct LDS objects, so that the compiler can tell the HBM->LDS
    // copies into one buffer from the reads of another and need not wait for
    // the copies before those reads.
    __shared__ __attribute__((aligned(1024))) char k_lds0[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char k_lds1[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds0[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds1[T::kBytes];
    LDS_AS char* const kbuf[2] = {(LDS_AS char*)k_lds0, (LDS_AS char*)k_lds1};
    LDS_AS char* const vbuf[2] = {(LDS_AS char*)v_lds0, (LDS_AS char*)v_lds1};

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // Work item: longest query tiles first; consecutive ids -> different slices.
    const int w = blockIdx.x;
    const int tile = p.n_qtiles - 1 - w / p.BH;
    const int bh = w - (w / p.BH) * p.BH;
    const int N = (int)p.N;
    const int q0 = tile * kBlockM;
    const int qw = q0 + wave * 32;          // first query row of this wave
    const int qi = qw + l32;                // this lane's query row
    const size_t base = (size_t)bh * (size_t)N * D;

    const uint16_t* __restrict__ Qg = (const uint16_t*)p.q + base;
    const uint16_t* __restrict__ Kg = (const uint16_t*)p.k + base;
    const uint16_t* __restrict__ Vg = (const uint16_t*)p.v + base;

    const int n_tiles = ((CAUSAL ? min(q0 + kBlockM, N) : N) + kBlockN - 1) / kBlockN;
    // First tile that needs element masks for this wave: the first one that
    // crosses its diagonal (causal) or N. Tiles before it are fully visible.
    // Tile j crosses N when 64(j+1) > N, and crosses this wave's diagonal
    // when 64j + 63 > qw.
    int j_mask = N / kBlockN;
    if (CAUSAL) j_mask = min(j_mask, (qw + 1) / kBlockN);
    j_mask = min(j_mask, n_tiles);

    // Prologue loads: K(0), K(1).
    int koff_src[T::kLoadsPerWave], voff_src[T::kLoadsPerWave];
    tile_src_offsets<D, false>(wave, lane, koff_src);
    tile_src_offsets<D, true>(wave, lane, voff_src);
    load_tile<D>(Kg, 0, N, kbuf[0], wave, koff_src);
    load_tile<D>(Kg, kBlockN, N, kbuf[1], wave, koff_src);

    // Q fragments (B operand of S^T = K Q^T): lane holds q[qi][16kd + 8g .. +7].
    u32x4 qf[NKD];
    {
        const int qrow = min(qi, N - 1);
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd)
            qf[kd] = *(const u32x4*)(Qg + (size_t)qrow * D + 16 * kd + 8 * g);
    }

    // Per-lane LDS offsets of the K reads (row l32 of a 32-key block, logical
    // chunk 2kd+g) and of the V transposed reads (see pv()).
    int koff[NKD];
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd)
        koff[kd] = l32 * T::kRowBytes + (((2 * kd + g) ^ T::swz_k(l32)) << 4);
    // ds_read_b64_tr_b16: in each group of 16 lanes, output lane j receives
    // element j%4 of the 8-byte reads of source lanes j/4 + 4k (k = 0..3).
    // Source lane (G = lane/16, i = lane%16) therefore reads row 4g + i/4
    // (+16kb2 + 8h) at columns 32db + 16(G%2) + 4(i%4): output lane l gets
    // V[16kb2 + 8h + 4g + k][32db + l%32] for k = 0..3, the A operand of the
    // P.V step with the key order of the S^T accumulator.
    const int G = lane >> 4, i16 = lane & 15;
    const int vrow = 4 * g + (i16 >> 2);
    int voff[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + 16 * (G & 1) + 4 * (i16 & 3);   // element column
        const int chunk = col >> 3, half = (col >> 2) & 1;
        voff[db] = vrow * T::kRowBytes + ((chunk ^ T::swz_v(vrow)) << 4) + half * 8;
    }

    const float c2 = p.scale_log2;
    float m_used = -INFINITY;   // exponent base (log2 domain) of P and O
    float l_run = 0.f;          // this lane's half of the row sum
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;

    // ---- building blocks ------------------------------------------------
    auto qk = [&](const LDS_AS char* kb_base, f32x16* s_out) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) {
                const u32x4 a = *(const LDS_AS u32x4*)(kb_base + koff[kd] + kb * 32 * T::kRowBytes);
                s_out[kb] = Op::mfma(a, qf[kd], kd == 0 ? f32x16{} : s_out[kb]);
            }
        }
    };

    auto pv = [&](const LDS_AS char* vb_base, const u32x4* p_in) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int kb2 = 0; kb2 < 4; ++kb2) {
                const LDS_AS char* a0 = vb_base + voff[db] + (16 * kb2) * T::kRowBytes;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)a0);
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(a0 + 8 * T::kRowBytes));
                const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
                const u32x4 a = {lo2[0], lo2[1], hi2[0], hi2[1]};
                o[db] = Op::mfma(a, p_in[kb2], o[db]);
            }
        }
    };

    // Masks on tile j (keys kv0..kv0+63): the key index inside the tile of
    // accumulator entry (kb, i) is 32kb + 8(i/4) + 4g + i%4; it is dead past
    // `lim`. A tile past this wave's rows is thereby fully dead (P = 0).
    auto apply_mask = [&](f32x16* s, int kv0) __attribute__((always_inline)) {
        const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - kv0 - 4 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                s[kb][i] = (32 * kb + 8 * (i >> 2) + (i & 3) > lim) ? -INFINITY : s[kb][i];
    };

    // Online softmax of one S^T tile: P packed for the P.V product, l updated,
    // and alpha (the factor O must be multiplied by) when the base moved.
    auto softmax = [&](const f32x16* s, u32x4* p_out, float& alpha) __attribute__((always_inline)) -> bool {
        // v_maximum3_f32: two entries per instruction (inputs are finite or
        // -inf, so its NaN propagation never matters).
        float mx = __builtin_elementwise_maximum(s[0][0], s[0][1]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = (kb == 0 ? 2 : 0); i < 16; i += 2)
                mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s[kb][i], s[kb][i + 1]));
        mx = wave_half_max(mx) * c2;
        const bool need = mx > m_used + kRescaleThreshold;
        const float m_new = need ? mx : m_used;
        alpha = need ? __builtin_amdgcn_exp2f(m_used - m_new) : 1.f;
        m_used = m_new;
        const float m_sub = m_new == -INFINITY ? 0.f : m_new;
        float lsum = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // entries 8(kb2%2) + 2e, +1 of S block kb2/2
                const int i = 8 * (kb2 & 1) + 2 * e;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb2 >> 1][i], c2, -m_sub));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb2 >> 1][i + 1], c2, -m_sub));
                p_out[kb2][e] = Op::pack2(p0, p1);
                lsum = Op::sum2(p_out[kb2][e], lsum);
            }
        }
        l_run = alpha * l_run + lsum;
        return __builtin_amdgcn_ballot_w64(need) != 0;
    };

    auto rescale_o = [&](float alpha) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
    };

    // ---- pipeline --------------------------------------------------------
    // Iteration j (parity PAR = j & 1):
    //   wait for this lane's copies; barrier;
    //   issue copies K(j+2) -> kbuf[PAR], V(j) -> vbuf[PAR];
    //   MFMA: S(j+1) = K(j+1) Q^T from kbuf[1-PAR]; O += P(j-1) V(j-1) from vbuf[1-PAR];
    //   VALU: softmax of S(j) -> P(j);  then O *= alpha(j) if the base moved.
    // Copies past the last tile read clamped rows into buffers nobody reads.
    f32x16 sa[2], sb[2];
    u32x4 pa[4], pb[4];

    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this lane's prologue copies
    __syncthreads();
    qk(kbuf[0], sa);

    // Steady state: no masks, every product needed; one basic block, so the
    // scheduler can interleave the MFMAs with the softmax.
    auto body_main = [&](int j, auto par_tag, f32x16* s_cur, f32x16* s_next, const u32x4* p_prev,
                         u32x4* p_cur) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_tag)::value;
        __builtin_amdgcn_s_waitcnt(0x0f70);
        __syncthreads();
        load_tile<D>(Kg, (j + 2) * kBlockN, N, kbuf[PAR], wave, koff_src);
        load_tile<D>(Vg, j * kBlockN, N, vbuf[PAR], wave, voff_src);
        qk(kbuf[1 - PAR], s_next);
        pv(vbuf[1 - PAR], p_prev);
        float alpha;
        const bool rescale = softmax(s_cur, p_cur, alpha);
        if (rescale) rescale_o(alpha);
    };
    // First, diagonal, tail and dead tiles: the general form.
    auto body_edge = [&](int j, auto par_tag, f32x16* s_cur, f32x16* s_next, const u32x4* p_prev,
                         u32x4* p_cur) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_tag)::value;
        __builtin_amdgcn_s_waitcnt(0x0f70);
        __syncthreads();
        load_tile<D>(Kg, (j + 2) * kBlockN, N, kbuf[PAR], wave, koff_src);
        load_tile<D>(Vg, j * kBlockN, N, vbuf[PAR], wave, voff_src);
        if (j + 1 < n_tiles) qk(kbuf[1 - PAR], s_next);
        if (j >= 1) pv(vbuf[1 - PAR], p_prev);
        if (j >= j_mask) apply_mask(s_cur, j * kBlockN);
        float alpha;
        const bool rescale = softmax(s_cur, p_cur, alpha);
        if (rescale) rescale_o(alpha);
    };

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    // j = 0 is always an edge iteration (no P.V yet).
    body_edge(0, P0{}, sa, sb, pb, pa);
    int j = 1;
    // Main iterations need j + 1 < n_tiles and j < j_mask; pairs keep the
    // register roles static (odd j: S in sb, P into pb).
    const int j_main_end = min(j_mask, n_tiles - 1);
    for (; j + 1 < j_main_end; j += 2) {
        body_main(j, P1{}, sb, sa, pa, pb);
        body_main(j + 1, P0{}, sa, sb, pb, pa);
    }
    for (; j < n_tiles; j += 2) {
        if (j < j_main_end) body_main(j, P1{}, sb, sa, pa, pb);
        else body_edge(j, P1{}, sb, sa, pa, pb);
        if (j + 1 < n_tiles) body_edge(j + 1, P0{}, sa, sb, pb, pa);
    }
    // Last P.V: P(n_tiles-1) with V(n_tiles-1), copied by the last iteration.
    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    {
        const int last = n_tiles - 1;
        if (last & 1) pv(vbuf[1], pb);
        else pv(vbuf[0], pa);
    }

    // Epilogue: O = O~ / l, rounded once to the output type; lse in fp32.
    const float l_tot = wave_half_sum(l_run);
    const float inv = 1.f / l_tot;
    if (qi < N) {
        uint16_t* Og = (uint16_t*)p.o + base + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int dd = 32 * db + 8 * i4 + 4 * g;
                const u32x2 wv = {Op::pack2(o[db][4 * i4] * inv, o[db][4 * i4 + 1] * inv),
                                  Op::pack2(o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv)};
                *(u32x2*)(Og + dd) = wv;
            }
        if (g == 0) p.lse[(size_t)bh * N + qi] = (m_used + log2f(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------------------
// Ping-pong variant (the default): 512 threads = 8 wave64s, 32 query rows
// each (256 rows per workgroup). Waves w and w+4 share one SIMD; waves 0-3
// (group A) and 4-7 (group B) run the same per-tile sequence
//    MFMA step j : S(j) = K(j) Q^T  and  O += P(j-1) V(j-1)
//    VALU step j : softmax of S(j) -> P(j), rescale of O when needed
// with a workgroup barrier after every step, group B one step behind
// group A. Between two barriers one wave of each SIMD feeds the matrix core
// while the other keeps the vector ALU busy. Group A copies K(j+1) and V(j)
// HBM -> LDS at the start of its MFMA step j, into the buffers of K(j-1) and
// V(j-2), and waits for them before the barrier that ends its VALU step j.
constexpr int kPPThreads = 512;
constexpr int kPPWaves = kPPThreads / 64;
constexpr int kPPBlockM = kPPWaves * 32;

template <bool IS_BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(kPPThreads, 1) void fwd16_pp_kernel(FwdParams p) {
    using Op = Op16<IS_BF16>;
    using T = Tile<D, kPPWaves>;
    constexpr int NKD = D / 16;
    constexpr int NDB = D / 32;

    __shared__ __attribute__((aligned(1024))) char k_lds0[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char k_lds1[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds0[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds1[T::kBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;              // 0: leads, 1: one phase behind
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    const int w = blockIdx.x;
    const int tile = p.n_qtiles - 1 - w / p.BH;
    const int bh = w - (w / p.BH) * p.BH;
    const int N = (int)p.N;
    const int q0 = tile * kPPBlockM;
    const int qw = q0 + wave * 32;
    const int qi = qw + l32;
    const size_t base = (size_t)bh * (size_t)N * D;

    const uint16_t* __restrict__ Qg = (const uint16_t*)p.q + base;
    const uint16_t* __restrict__ Kg = (const uint16_t*)p.k + base;
    const uint16_t* __restrict__ Vg = (const uint16_t*)p.v + base;

    const int n_tiles = ((CAUSAL ? min(q0 + kPPBlockM, N) : N) + kBlockN - 1) / kBlockN;
    const int n_live = CAUSAL ? min(n_tiles, (qw + 31) / kBlockN + 1) : n_tiles;
    int j_mask = N / kBlockN;
    if (CAUSAL) j_mask = min(j_mask, (qw + 1) / kBlockN);

    // Copies are issued by the four waves of group A only.
    int koff_src[Tile<D, 4>::kLoadsPerWave], voff_src[Tile<D, 4>::kLoadsPerWave];
    tile_src_offsets<D, false, 4>(wave & 3, lane, koff_src);
    tile_src_offsets<D, true, 4>(wave & 3, lane, voff_src);
    if (grp == 0) load_tile<D, 4>(Kg, 0, N, (LDS_AS char*)k_lds0, wave, koff_src);

    u32x4 qf[NKD];
    {
        const int qrow = min(qi, N - 1);
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd)
            qf[kd] = *(const u32x4*)(Qg + (size_t)qrow * D + 16 * kd + 8 * g);
    }

    int koff[NKD];
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd)
        koff[kd] = l32 * T::kRowBytes + (((2 * kd + g) ^ T::swz_k(l32)) << 4);
    const int G = lane >> 4, i16 = lane & 15;
    const int vrow = 4 * g + (i16 >> 2);
    int voff[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + 16 * (G & 1) + 4 * (i16 & 3);
        const int chunk = col >> 3, half = (col >> 2) & 1;
        voff[db] = vrow * T::kRowBytes + ((chunk ^ T::swz_v(vrow)) << 4) + half * 8;
    }

    const float c2 = p.scale_log2;
    float m_used = -INFINITY;
    float l_run = 0.f;
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    f32x16 s[2];
    u32x4 pk[4];
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2) pk[kb2] = u32x4{0u, 0u, 0u, 0u};
#if ATTN_L_MFMA
    f32x16 lacc = {};
    const uint32_t one2 = IS_BF16 ? 0x3f803f80u : 0x3c003c00u;   // two 1.0 in bf16 / fp16
    const u32x4 kOnes = {one2, one2, one2, one2};
#endif

    __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();

    // MFMA step of tile jj: S(jj) = K(jj) Q^T, and O += P(jj-1) V(jj-1) when
    // HAS_PV. K(jj) sits in k_lds[jj&1], V(jj-1) in v_lds[(jj-1)&1]: KPAR = jj&1.
    auto mfma_step = [&](int jj, auto kpar_tag, auto has_pv_tag) __attribute__((always_inline)) {
        constexpr int KPAR = decltype(kpar_tag)::value;
        constexpr bool HAS_PV = decltype(has_pv_tag)::value;
        const LDS_AS char* kb_base = (const LDS_AS char*)(KPAR ? k_lds1 : k_lds0);
        const LDS_AS char* vb_base = (const LDS_AS char*)(KPAR ? v_lds0 : v_lds1);
#if ATTN_MFMA_PREFETCH
        // LDS operand reads are issued ahead of the MFMAs that use them, so
        // their latency overlaps: all K fragments and the first VPRE blocks
        // of V^T fragments up front, the rest behind the S(jj) MFMAs.
        constexpr int VPRE = NDB < 2 ? NDB : 2;
        auto read_v = [&](int db, int kb2) __attribute__((always_inline)) -> u32x4 {
            const LDS_AS char* a0 = vb_base + voff[db] + (16 * kb2) * T::kRowBytes;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)a0);
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(a0 + 8 * T::kRowBytes));
            return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        u32x4 kf[2][NKD];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd)
                kf[kb][kd] = *(const LDS_AS u32x4*)(kb_base + koff[kd] + kb * 32 * T::kRowBytes);
        // P of a tile past this wave's rows is all zero, so its P.V is skipped.
        const bool do_pv = HAS_PV && jj - 1 < n_live;
        u32x4 vf[NDB][4];
        if (do_pv) {
#pragma unroll
            for (int db = 0; db < VPRE; ++db)
#pragma unroll
                for (int kb2 = 0; kb2 < 4; ++kb2) vf[db][kb2] = read_v(db, kb2);
        }
        __builtin_amdgcn_sched_barrier(0);
        // S is computed for every tile, also ones this wave does not need
        // (their S is never read): a conditional S would cost register copies.
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                s[kb] = Op::mfma(kf[kb][kd], qf[kd], kd == 0 ? f32x16{} : s[kb]);
        if (do_pv) {
#pragma unroll
            for (int db = VPRE; db < NDB; ++db)
#pragma unroll
                for (int kb2 = 0; kb2 < 4; ++kb2) vf[db][kb2] = read_v(db, kb2);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int kb2 = 0; kb2 < 4; ++kb2) o[db] = Op::mfma(vf[db][kb2], pk[kb2], o[db]);
#if ATTN_L_MFMA
            // Row sums of P on the matrix core: an all-ones A operand makes
            // every row of the 32x32 result the column sums of P^T.
#pragma unroll
            for (int kb2 = 0; kb2 < 4; ++kb2) lacc = Op::mfma(kOnes, pk[kb2], lacc);
#endif
        }
#else
        // S is computed for every tile, also ones this wave does not need
        // (their S is never read): a conditional S would cost register copies.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd) {
                const u32x4 a = *(const LDS_AS u32x4*)(kb_base + koff[kd] + kb * 32 * T::kRowBytes);
                s[kb] = Op::mfma(a, qf[kd], kd == 0 ? f32x16{} : s[kb]);
            }
        // P of a tile past this wave's rows is all zero, so its P.V is skipped.
        if (HAS_PV && jj - 1 < n_live) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int kb2 = 0; kb2 < 4; ++kb2) {
                    const LDS_AS char* a0 = vb_base + voff[db] + (16 * kb2) * T::kRowBytes;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)a0);
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(a0 + 8 * T::kRowBytes));
                    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    o[db] = Op::mfma(a, pk[kb2], o[db]);
                }
#if ATTN_L_MFMA
            // Row sums of P on the matrix core: an all-ones A operand makes
            // every row of the 32x32 result the column sums of P^T.
#pragma unroll
            for (int kb2 = 0; kb2 < 4; ++kb2) lacc = Op::mfma(kOnes, pk[kb2], lacc);
#endif
        }
#endif
    };

    // VALU step of tile jj: online softmax of S(jj) into P, rescale of O.
    auto valu_step = [&](int jj) __attribute__((always_inline)) {
        if (jj >= n_live) return;
        const int kv0 = jj * kBlockN;
        if (jj >= j_mask) {
            const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - kv0 - 4 * g;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    s[kb][i] = (32 * kb + 8 * (i >> 2) + (i & 3) > lim) ? -INFINITY : s[kb][i];
        }
        float mx = __builtin_elementwise_maximum(s[0][0], s[0][1]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = (kb == 0 ? 2 : 0); i < 16; i += 2)
                mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s[kb][i], s[kb][i + 1]));
        mx = wave_half_max(mx) * c2;
        const bool need = mx > m_used + kRescaleThreshold;
        const float m_new = need ? mx : m_used;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_used - m_new) : 1.f;
        m_used = m_new;
        const float m_sub = m_new == -INFINITY ? 0.f : m_new;
        float lpart[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 8 * (kb2 & 1) + 2 * e;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb2 >> 1][i], c2, -m_sub));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb2 >> 1][i + 1], c2, -m_sub));
                pk[kb2][e] = Op::pack2(p0, p1);
#if !ATTN_L_MFMA
                // fp32 adds: v_dot2 would run on the matrix pipe and stall
                // behind the other wave's MFMAs.
                lpart[e] += p0 + p1;
#endif
            }
#if ATTN_L_MFMA
        (void)lpart;
#else
        l_run = alpha * l_run + ((lpart[0] + lpart[1]) + (lpart[2] + lpart[3]));
#endif
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
#if ATTN_L_MFMA
#pragma unroll
            for (int i = 0; i < 16; ++i) lacc[i] *= alpha;
#endif
        }
    };

    // Workgroup barrier without a memory fence: the LDS reads of a phase are
    // consumed by its MFMAs before the wave gets here, and the copies are
    // waited for explicitly, so a fence would only expose HBM latency.
    auto barrier = [&]() __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // Group A issues all copies, at the start of its MFMA step of tile j:
    // K(j+1) -> k_lds[(j+1)&1], V(j) -> v_lds[j&1].
    auto copies = [&](int j, auto par_tag) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_tag)::value;   // j & 1
        if (grp == 0) {
            if (j + 1 < n_tiles)
                load_tile<D, 4>(Kg, (j + 1) * kBlockN, N, (LDS_AS char*)(PAR ? k_lds0 : k_lds1), wave, koff_src);
            load_tile<D, 4>(Vg, j * kBlockN, N, (LDS_AS char*)(PAR ? v_lds1 : v_lds0), wave, voff_src);
        }
    };
#if ATTN_PP_MODE == 0
    // One tile: MFMA phase, barrier, VALU phase, barrier (group A first waits
    // for its copies, which the next phase reads).
    auto tile_steps = [&](int j, auto par_tag, auto has_pv_tag) __attribute__((always_inline)) {
        copies(j, par_tag);
        mfma_step(j, par_tag, has_pv_tag);
        barrier();
        valu_step(j);
        if (grp == 0) __builtin_amdgcn_s_waitcnt(0x0f70);
        barrier();
    };
#else
    // One barrier per tile. Mode 1: every wave runs MFMA(j) then VALU(j).
    // Mode 2: group B runs VALU(j-1) then MFMA(j), so inside each barrier
    // interval the two waves of a SIMD use the two units in opposite order.
    auto tile_steps = [&](int j, auto par_tag, auto has_pv_tag) __attribute__((always_inline)) {
        copies(j, par_tag);
        if (ATTN_PP_MODE == 2 && grp == 1) {
            if (j >= 1) valu_step(j - 1);
            mfma_step(j, par_tag, has_pv_tag);
        } else {
            mfma_step(j, par_tag, has_pv_tag);
            valu_step(j);
        }
        if (grp == 0) __builtin_amdgcn_s_waitcnt(0x0f70);
        barrier();
    };
#endif

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using NoPV = std::integral_constant<bool, false>;
    using WithPV = std::integral_constant<bool, true>;

#if ATTN_PP_MODE == 0
    // Group B runs one phase behind group A.
    if (grp == 1) barrier();
#endif
    tile_steps(0, P0{}, NoPV{});
    int j = 1;
    for (; j + 1 < n_tiles; j += 2) {
        tile_steps(j, P1{}, WithPV{});
        tile_steps(j + 1, P0{}, WithPV{});
    }
    if (j < n_tiles) {
        tile_steps(j, P1{}, WithPV{});
        ++j;
    }
#if ATTN_PP_MODE == 2
    if (grp == 1) valu_step(n_tiles - 1);
#endif
    // Final P.V of tile n_tiles-1 (the S computed alongside is unused).
    if (n_tiles & 1) mfma_step(n_tiles, P1{}, WithPV{});
    else mfma_step(n_tiles, P0{}, WithPV{});
#if ATTN_PP_MODE == 0
    if (grp == 0) barrier();
#endif

#if ATTN_L_MFMA
    const float l_tot = lacc[0];
#else
    const float l_tot = wave_half_sum(l_run);
#endif
    const float inv = 1.f / l_tot;
    if (qi < N) {
        uint16_t* Og = (uint16_t*)p.o + base + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int dd = 32 * db + 8 * i4 + 4 * g;
                const u32x2 wv = {Op::pack2(o[db][4 * i4] * inv, o[db][4 * i4 + 1] * inv),
                                  Op::pack2(o[db][4 * i4 + 2] * inv, o[db][4 * i4 + 3] * inv)};
                *(u32x2*)(Og + dd) = wv;
            }
        if (g == 0) p.lse[(size_t)bh * N + qi] = (m_used + log2f(l_tot)) * kLn2;
    }
}

template <bool IS_BF16, int D, bool CAUSAL>
hipError_t launch(FwdParams p, hipStream_t s) {
#if ATTN_PINGPONG
    p.n_qtiles = (int)((p.N + kPPBlockM - 1) / kPPBlockM);
    const dim3 grid((unsigned)(p.n_qtiles * p.BH));
    hipLaunchKernelGGL((fwd16_pp_kernel<IS_BF16, D, CAUSAL>), grid, dim3(kPPThreads), 0, s, p);
#else
    p.n_qtiles = (int)((p.N + kBlockM - 1) / kBlockM);
    const dim3 grid((unsigned)(p.n_qtiles * p.BH));
    hipLaunchKernelGGL((fwd16_kernel<IS_BF16, D, CAUSAL>), grid, dim3(kThreads), 0, s, p);
#endif
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
