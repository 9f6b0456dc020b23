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
//     3.2  K/V tiles are double-buffered (the next tiles' copies are in
//          flight while the current ones are used); rows past N are
//          zero-filled and their keys masked to -inf;
//     3.3  P is computed once per tile and reused for every output column.
//   [G7] "Flash Attention CUDA Kernel 优化: 从 56 到 986 TFLOPS on B300 —
//          G7: 回归 1CTA": exp is taken as exp2 with log2(e) folded into the
//          score scale (lesson 6); QK^T and P.V are issued so that they
//          interleave with the softmax (V45, V50); the rescale of the
//          accumulator is conditional (carried over from G6).
//   [naive-attn] cishoon.github.io "flashattention", 3.5: shared-memory bank
//          conflicts are removed through the layout (XOR swizzles of 16-byte
//          chunks here, instead of padding).
//
// gfx950 design (not the pages'):
//   * 512 threads = 8 wave64s; each wave owns QB blocks of 32 query rows,
//     QB = 1 or 2 (2 only at d = 64, where the registers hold two blocks).
//     The launcher takes QB = 2 for long runs (twice the reuse of every K/V
//     fragment), under a causal mask only from 8192 keys on, and QB = 1 for
//     shorter causal runs (half as many diagonal tiles per work item) or
//     when QB = 2 would leave compute units without a work item. K/V tiles
//     hold 64 keys.
//   * Both products run on v_mfma_f32_32x32x16_{bf16,f16} with fp32
//     accumulation, in transposed form so that one lane owns one query:
//        S^T[key][query] = K . Q^T     (A = K rows from LDS, B = Q in VGPRs)
//        O^T[d][query]  += V^T . P^T   (A = V^T from LDS, B = P in VGPRs)
//     The 32x32 accumulator gives lane l the column l%32 (its query) and 16
//     rows (keys, or head-dim entries), so the softmax row max / row sum are
//     in-lane reductions plus one v_permlane32_swap, and the rescale of O is
//     a per-lane scalar multiply. With QB = 2 every K or V^T fragment read
//     from LDS feeds two MFMAs.
//   * P leaves the S^T accumulator already in the B-operand layout of the
//     P.V product (the order of keys inside a contraction is free); the
//     matching V^T operand comes from row-major V in LDS through
//     ds_read_b64_tr_b16, two reads per MFMA.
//   * K and V tiles go from HBM straight into LDS (buffer_load_dwordx4 ...
//     lds, 16 bytes per lane, no VGPR staging); the XOR swizzle is applied
//     by choosing which global chunk each lane fetches, and rows past N fall
//     outside the buffer descriptor's range and arrive as zeros.
//   * Ping-pong: waves w and w+4 share a SIMD. Waves 0-3 (group A) and 4-7
//     (group B) run the same per-tile sequence
//         MFMA step j : S(j) = K(j) Q^T  and  O += P(j-1) V(j-1)
//         VALU step j : softmax of S(j) -> P(j), rescale of O when needed
//     with a workgroup barrier after every step, group B one step behind,
//     so in every barrier interval one wave of each SIMD feeds the matrix
//     core while the other runs the softmax on the vector ALU. At d = 64
//     with one query block the MFMA step does the P.V products first: the
//     registers the S products are about to fill stage the V^T operands
//     read ahead, and the P registers then stage the K operands.
//   * Lazy rescale: the exponent base m only moves when a tile's row max
//     exceeds it by more than the threshold T in probability (T = 2^15 for
//     fp16, below its 65504 maximum; 2^64 for bf16, whose P has fp32's
//     exponent range); otherwise P <= T is used as is. The final
//     O / l does not depend on the base, and a 16-bit P keeps its relative
//     precision at any magnitude its type represents.
//   * The softmax step does not take the row maximum first: it
//     exponentiates against the current base, then tests whether any packed
//     P exceeds T (or overflowed) with 3-input packed 16-bit maxima, eight
//     per tile and query block instead of ~25 instructions for the fp32
//     maximum, its lane exchange and the comparison. Only if some row fails
//     does the wave take the maximum and redo the tile against the moved
//     base; the P it keeps is the same either way. At d = 64 the vector ALU
//     is the busier unit, so this is +4-5 % at the causal workloads and
//     +5 % with two query blocks; at d = 128 it is +0-1 %.
//   * At d = 64 the kernel goes one step further: a first pass takes no
//     overflow test at all (each row keeps the base tile 0 gave it), and
//     the test moves to the end of the work item, on the row sums: every P
//     of a row is at most its l, so a row with l <= T never had a P above
//     T, and its bits are those the per-tile test would give. If some row
//     fails (its score maximum rose by more than ~64 (bf16) or ~15 (fp16)
//     log2 units after tile 0, or many keys came close to T), the
//     workgroup computes the item again with the per-tile test, in a
//     function of its own so that the rare path takes nothing from the main
//     path's registers. Which rows share a workgroup thus
//     never changes a row's bits. On gfx950 a full-rate vector instruction
//     (the maxima, the compare) hardly overlaps another wave's MFMAs, while
//     exp2 and the 16-bit packs do: +3 % at the causal workloads, +4 % with
//     two query blocks.
//   * The softmax row sum l runs on the matrix core as well: a 16x16x32
//     MFMA with a constant 0/1 A operand sums the P operand of the P.V step
//     over its keys (four per tile and query block), which takes ~60 fp32
//     adds per tile off the vector ALU, the busier unit at d = 64. l is
//     then the sum of the same rounded P values that weight V.
//   * Work items (b*H+h, query tile), fwd_order.h: under a causal mask the
//     longest query tiles of every slice first (tile-major), consecutive
//     workgroup ids on different slices, so that with the round-robin
//     placement of workgroups over the 8 XCDs all workgroups of one slice
//     share one XCD's L2; without a mask (all items equally long) each XCD
//     takes its K/V slices one after another (XCD-major), so that a slice's
//     K and V pass through that L2 once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_internal.h"
#include "fwd_order.h"
#include "mfma_common.h"

namespace attn {
namespace {

constexpr float kLn2 = 0.693147180559945309f;
// Largest P the lazy rescale lets through (log2 units): 2^15 for fp16, below
// its 65504 maximum; 2^64 for bf16, whose P has fp32's exponent range and the
// same relative precision at any magnitude (O then stays finite for |V| up
// to ~2^60). Both keep O and l, which accumulate in fp32, far from overflow.
template <bool IS_BF16>
constexpr float rescale_threshold() { return IS_BF16 ? 64.0f : 15.0f; }
constexpr int kBlockN = 64;                 // keys per K/V tile
constexpr int kThreads = 512;               // 8 waves
constexpr int kWaves = kThreads / 64;
constexpr int kCopyWaves = 4;               // group A issues the HBM -> LDS copies

constexpr int kComputeUnits = 256;         // MI355X

// Query rows per work item with QB 32-row blocks per wave.
template <int QB>
constexpr int block_m() { return kWaves * 32 * QB; }

// LDS layout of one K or V tile: 64 rows of D 16-bit values, row-major, with
// 16-byte chunk c of row r stored at chunk c ^ swz(r).
//  * K is read 16 bytes per lane, one row per lane, 16 lanes per LDS cycle:
//    rows r..r+15 at one logical chunk must land in 16 different 16-byte bank
//    groups (64 banks x 4 bytes).
//  * V is read with ds_read_b64_tr_b16: 32 lanes read 4 consecutive rows x
//    64 contiguous bytes; rows 2 apart (D = 64) or adjacent rows (D = 128)
//    would otherwise share banks.
template <int D>
struct Tile {
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;             // 16-byte chunks per row
    static constexpr int kBytes = kBlockN * kRowBytes;
    static constexpr int kCopiesPerWave = kBytes / 1024 / kCopyWaves;   // 1 KiB per wave copy
    static __device__ __forceinline__ int swz_k(int r) { return D == 64 ? (r >> 1) & 7 : r & 15; }
    static __device__ __forceinline__ int swz_v(int r) { return D == 64 ? ((r >> 1) & 1) << 2 : (r & 3) << 2; }
};

// Per-lane byte offsets, inside a tile, of the 16-byte global chunks this
// lane copies: copy u of copy-wave cw fills LDS chunk slots
// s = (cw*U + u)*64 + lane, i.e. row s / kChunks, physical chunk
// s % kChunks, holding the global chunk (physical ^ swz(row)).
template <int D, bool IS_V>
__device__ __forceinline__ void tile_src_offsets(int cw, int lane, int* off) {
    using T = Tile<D>;
#pragma unroll
    for (int u = 0; u < T::kCopiesPerWave; ++u) {
        const int s = (cw * T::kCopiesPerWave + u) * 64 + lane;
        const int r = s / T::kChunks;
        const int pc = s % T::kChunks;
        const int lc = pc ^ (IS_V ? T::swz_v(r) : T::swz_k(r));
        off[u] = r * T::kRowBytes + lc * 16;
    }
}

// This copy-wave's share of the HBM -> LDS copy of one K or V tile (keys
// kv0 .. kv0+63). The buffer descriptor covers rows kv0 .. min(N, kv0+64)-1, so
// chunks of rows past N are out of range and arrive as zeros (the zero-fill
// of the pages' asynchronous copy); their scores are masked.
template <int D>
__device__ __forceinline__ void copy_tile(const uint16_t* g_slice, int kv0, int N, LDS_AS char* buf,
                                          int cw, const int* off) {
    using T = Tile<D>;
    const int rows = min(max(N - kv0, 0), kBlockN);   // one tile: the range cannot overflow
    const i32x4 rsrc = buffer_rsrc(g_slice + (size_t)kv0 * D, rows * T::kRowBytes);
    const uint32_t lds0 = (uint32_t)(uintptr_t)buf;
#pragma unroll
    for (int u = 0; u < T::kCopiesPerWave; ++u) {
        const int slot0 = (cw * T::kCopiesPerWave + u) * 64;
        dma16(rsrc, lds0 + slot0 * 16, off[u]);
    }
}

// v_permlane32_swap(x, x): lanes < 32 get (x[l], x[l+32]), lanes >= 32 get
// (x[l-32], x[l]); combining the pair reduces over lanes l and l^32.
__device__ __forceinline__ float half_swap_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)r[0]),
                                         __builtin_bit_cast(float, (uint32_t)r[1]));
}

// max(m, a, b) as one v_maximum3_f32 (IEEE maximum; the operands here are
// finite or -inf). Written as assembly so that a running maximum stays a
// chain of 3-input maxima: the compiler would rebuild it as a tree that
// spends three instructions on every four new values.
__device__ __forceinline__ float max3(float m, float a, float b) {
    float r;
    asm("v_maximum3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
    return r;
}

// Elementwise maximum of three pairs of 16-bit values read as fp16, one
// v_pk_maximum3_f16 (IEEE maximum: a NaN operand gives NaN).
__device__ __forceinline__ uint32_t pk_max3_f16(uint32_t a, uint32_t b, uint32_t c) {
    uint32_t r;
    asm("v_pk_maximum3_f16 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// v_permlane16_swap(x, y): the odd 16-lane rows of x trade places with the
// even rows of y. Returns (new x, new y).
__device__ __forceinline__ float permlane16_swap_x(float x, float y) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, y), false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]);
}

__device__ __forceinline__ float permlane16_swap_y(float x, float y) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, y), false, false);
    return __builtin_bit_cast(float, (uint32_t)r[1]);
}

// One pass of a workgroup over its work item. OPT (d = 64 only): no overflow
// test per tile; returns false, without writing anything, when some row of
// the item needs the exact pass (decided by the whole workgroup).
template <bool IS_BF16, int D, bool CAUSAL, int QB, bool OPT>
__device__ __forceinline__ bool fwd16_pass(const FwdParams& p, int tid, int bid) {
    static_assert(!OPT || D == 64, "the pass without the overflow test is d = 64 only");
    static_assert(QB == 1 || (QB == 2 && D == 64), "two query blocks per wave only at d = 64");
    using Op = Op16<IS_BF16>;
    using T = Tile<D>;
    constexpr int BM = block_m<QB>();
    constexpr int NKD = D / 16;   // QK^T contraction steps
    constexpr int NDB = D / 32;   // 32-row blocks of O^T

    // Four distinct LDS objects, so every buffer is named statically.
    __shared__ __attribute__((aligned(1024))) char k_lds0[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char k_lds1[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds0[T::kBytes];
    __shared__ __attribute__((aligned(1024))) char v_lds1[T::kBytes];

    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave >> 2;              // 0: leads, 1: one step behind
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int g = lane >> 5;

    // Work item, longest query tiles first (fwd_order.h).
    const fwdorder::Item it = fwdorder::item(p.xcd_order != 0, bid, p.n_qtiles, p.BH,
                                             p.BH_kv, p.H_kv, p.G);
    const int tile = it.tile;
    const SliceIds ids = {it.bh, it.kv_bh};
    const int bh = ids.bh;
    const int N = (int)p.N;
    const int q0 = tile * BM;
    const int qw = q0 + wave * 32 * QB;     // first query row of this wave
    const size_t base = (size_t)bh * (size_t)N * D;
    const size_t kv_base = (size_t)ids.kv_bh * (size_t)N * D;

    const uint16_t* __restrict__ Qg = (const uint16_t*)p.q + base;
    const uint16_t* __restrict__ Kg = (const uint16_t*)p.k + kv_base;
    const uint16_t* __restrict__ Vg = (const uint16_t*)p.v + kv_base;

    const int n_tiles = ((CAUSAL ? min(q0 + BM, N) : N) + kBlockN - 1) / kBlockN;
    // Tiles this wave needs at all: causal tiles starting past its last row
    // are dead for every one of its rows. (Without a mask it is n_tiles; the
    // readfirstlane hides that from the compiler, whose loop versioning on it
    // otherwise runs out of registers.)
    const int n_live = CAUSAL ? min(n_tiles, (qw + 32 * QB - 1) / kBlockN + 1)
                              : __builtin_amdgcn_readfirstlane(n_tiles);
    // First tile needing element masks: it crosses N (64(j+1) > N) or this
    // wave's diagonal (64j + 63 > qw).
    int j_mask = N / kBlockN;
    if (CAUSAL) j_mask = min(j_mask, (qw + 1) / kBlockN);

    // Group A copies; offsets of this lane's chunks inside a K / V tile.
    int koff_src[T::kCopiesPerWave], voff_src[T::kCopiesPerWave];
    tile_src_offsets<D, false>(wave & 3, lane, koff_src);
    tile_src_offsets<D, true>(wave & 3, lane, voff_src);
    if (grp == 0) copy_tile<D>(Kg, 0, N, (LDS_AS char*)k_lds0, wave, koff_src);

    // Q fragments (B operand of S^T = K Q^T): lane holds q[row][16kd + 8g .. +7].
    u32x4 qf[QB][NKD];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = min(qw + 32 * qb + l32, N - 1);
#pragma unroll
        for (int kd = 0; kd < NKD; ++kd)
            qf[qb][kd] = *(const u32x4*)(Qg + (size_t)qrow * D + 16 * kd + 8 * g);
    }

    // Per-lane LDS offsets of the K reads (row l32 of a 32-key block, logical
    // chunk 2kd+g) and of the V transposed reads.
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

    // Row-sum MFMA (16x16x32): B = the P operand of the P.V step, read as
    // B[k][c] with k-block l/16 of lane l = (query half, key half):
    //   k-blocks 0, 2 hold query c, k-blocks 1, 3 query c + 16 (c = l % 16).
    // A lane l holds A[l % 16][8(l/16) .. +7]; ones where row & 7 equals the
    // k-block's query half, so D rows 0 and 8 are the sums of queries c and
    // rows 1 and 9 those of queries c + 16; every other row is zero. D gives
    // lane l rows 4(l/16) .. +3 of column l % 16: entries 0 and 1 of lanes
    // 0-15 and 32-47 carry the sums.
    const uint32_t one_w = ((lane & 7) == ((lane >> 4) & 1) && (lane & 6) == 0) ? Op16<IS_BF16>::kOnePair : 0u;
    const u32x4 ones = {one_w, one_w, one_w, one_w};

    const float c2 = p.scale_log2;
    float m_used[QB];   // exponent base (log2 domain)
    f32x4 lacc[QB];     // row sums, in the D layout above
    f32x16 o[QB][NDB];
    f32x16 s[QB][2];
    u32x4 pk[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_used[qb] = -INFINITY;
        lacc[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[qb][db][i] = 0.f;
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2) pk[qb][kb2] = u32x4{0u, 0u, 0u, 0u};
    }

    // Rescale decisions of the current tile (the row maxima are only taken
    // when a tile's packed P fails the overflow test in the VALU step).
    float m_old[QB];
    bool need[QB];
    // Scores past the causal diagonal or past N become -inf.
    auto mask_tile = [&](int jj) __attribute__((always_inline)) {
        if (jj >= j_mask) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                // key index inside the tile of accumulator entry (kb, i) is
                // 32kb + 8(i/4) + 4g + i%4; it is dead past `lim`.
                const int qi = qw + 32 * qb + l32;
                const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - jj * kBlockN - 4 * g;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        s[qb][kb][i] = (32 * kb + 8 * (i >> 2) + (i & 3) > lim) ? -INFINITY : s[qb][kb][i];
            }
        }
    };
    // The row maximum of the (masked) tile and the lazy choice of the
    // exponent base.
    auto row_max_need = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            // Two chains of 3-input maxima, two entries per instruction.
            float mxa = s[qb][0][0], mxb = s[qb][1][0];
#pragma unroll
            for (int i = 1; i < 15; i += 2) {
                mxa = max3(mxa, s[qb][0][i], s[qb][0][i + 1]);
                mxb = max3(mxb, s[qb][1][i], s[qb][1][i + 1]);
            }
            float mx = max3(mxa, mxb, max3(s[qb][0][15], s[qb][1][15], s[qb][1][15]));
            mx = half_swap_max(mx) * c2;
            m_old[qb] = m_used[qb];
            need[qb] = mx > m_old[qb] + rescale_threshold<IS_BF16>();
            m_used[qb] = need[qb] ? mx : m_old[qb];
        }
    };

    // Set by any wave whose rows need the exact pass.
    __shared__ int redo_flag;
    if (OPT && tid == 0) redo_flag = 0;
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): this lane's copy of K(0)
    __syncthreads();

    // MFMA step of tile jj: S(jj) = K(jj) Q^T when HAS_S, and O += P(jj-1)
    // V(jj-1) when HAS_PV. K(jj) sits in k_lds[jj&1], V(jj-1) in
    // v_lds[(jj-1)&1]: KPAR = jj&1.
    auto mfma_step = [&](int jj, auto kpar_tag, auto has_pv_tag, auto has_s_tag) __attribute__((always_inline)) {
        constexpr int KPAR = decltype(kpar_tag)::value;
        constexpr bool HAS_PV = decltype(has_pv_tag)::value;
        constexpr bool HAS_S = decltype(has_s_tag)::value;
        const LDS_AS char* kb_base = (const LDS_AS char*)(KPAR ? k_lds1 : k_lds0);
        const LDS_AS char* vb_base = (const LDS_AS char*)(KPAR ? v_lds0 : v_lds1);
        if constexpr (D == 64 && QB == 1) {
            // P.V of the previous tile first, then S. At ~128 registers the
            // wave has no spare ones to read operands ahead, but the S
            // accumulators are dead until the S products (their last values
            // became P in the softmax step) and P is dead after the P.V
            // products: the V^T fragments are read ahead into the former,
            // the K fragments into the latter, four fragments ahead each,
            // so the MFMAs do not wait for LDS one by one (measured: +3 % at
            // the causal headline; at d = 128 the S-first order below is
            // kept, it measured 0.5 % faster there).
            if (HAS_PV && jj - 1 < n_live) {
                constexpr int NF = 4 * NDB;   // V^T fragments
                constexpr int PF = 4;         // read ahead
                u32x4 vf[NF];
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    const LDS_AS char* a0 = vb_base + voff[f % NDB] + (16 * (f / NDB)) * T::kRowBytes;
                    vf[f] = tr_read(a0, a0 + 8 * T::kRowBytes);
                }
                // The row-sum MFMAs (no LDS operand) cover the first reads.
#pragma unroll
                for (int kb2 = 0; kb2 < 4; ++kb2) lacc[0] = Op::mfma16(ones, pk[0][kb2], lacc[0]);
                // d blocks innermost: consecutive MFMAs share their P operand.
#pragma unroll
                for (int f = 0; f < NF; ++f) o[0][f % NDB] = Op::mfma(vf[f], pk[0][f / NDB], o[0][f % NDB]);
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 2);
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 2);
#pragma unroll
                for (int f = PF; f < NF; ++f) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, PF, 2);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (HAS_S) {
#pragma unroll
            for (int kd = 0; kd < NKD; ++kd)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const u32x4 a = *(const LDS_AS u32x4*)(kb_base + koff[kd] + kb * 32 * T::kRowBytes);
                    s[0][kb] = Op::mfma(a, qf[0][kd], kd == 0 ? f32x16{} : s[0][kb]);
                }
            constexpr int kSReads = 2 * NKD, KF = 4;
            __builtin_amdgcn_sched_group_barrier(0x100, KF, 3);
#pragma unroll
            for (int r = KF; r < kSReads; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 3);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 3);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, KF, 3);
            __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            // The two key blocks' products alternate, so that consecutive MFMAs
            // share their Q operand (each accumulator still sums over d in
            // order): fewer operand bits toggle, and under the power limit that
            // is clock (+0.5 % at d = 128 and at fp16 N = 16k).
            if constexpr (HAS_S) {
    #pragma unroll
            for (int kd = 0; kd < NKD; ++kd)
    #pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const u32x4 a = *(const LDS_AS u32x4*)(kb_base + koff[kd] + kb * 32 * T::kRowBytes);
    #pragma unroll
                    for (int qb = 0; qb < QB; ++qb)
                        s[qb][kb] = Op::mfma(a, qf[qb][kd], kd == 0 ? f32x16{} : s[qb][kb]);
                }
            }
            // Order: three K fragment reads ahead, then one more read per QB
            // MFMAs, so that LDS latency hides behind the matrix core.
            if constexpr (HAS_S) {
            constexpr int kSReads = 2 * NKD;
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 1);
    #pragma unroll
            for (int r = 3; r < kSReads; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x008, QB, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 3 * QB, 1);
            }
            // Keeps the P.V operand reads from being hoisted over the S products
            // (more live registers than the wave has).
            __builtin_amdgcn_sched_barrier(0);
            // No P.V for a tile past this wave's rows (no P was made for it).
            if (HAS_PV && jj - 1 < n_live) {
    #pragma unroll
                for (int kb2 = 0; kb2 < 4; ++kb2)
    #pragma unroll
                    for (int qb = 0; qb < QB; ++qb) lacc[qb] = Op::mfma16(ones, pk[qb][kb2], lacc[qb]);
                // d blocks innermost: consecutive MFMAs share their P operand.
    #pragma unroll
                for (int kb2 = 0; kb2 < 4; ++kb2)
    #pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        const LDS_AS char* a0 = vb_base + voff[db] + (16 * kb2) * T::kRowBytes;
                        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)a0);
                        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(a0 + 8 * T::kRowBytes));
                        const u32x4 a = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    #pragma unroll
                        for (int qb = 0; qb < QB; ++qb) o[qb][db] = Op::mfma(a, pk[qb][kb2], o[qb][db]);
                    }
                // Order: two V^T fragments (four reads) ahead, the row-sum MFMAs
                // (no LDS operand) while they arrive, then one fragment per QB
                // MFMAs.
                constexpr int kVFrags = 4 * NDB;
                __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);
                __builtin_amdgcn_sched_group_barrier(0x008, 4 * QB, 2);
    #pragma unroll
                for (int f = 2; f < kVFrags; ++f) {
                    __builtin_amdgcn_sched_group_barrier(0x008, QB, 2);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * QB, 2);
            }
        }
    };

    // VALU step of tile jj: online softmax of S(jj) into P for every query
    // block, and the rescale of O where the exponent base moved. In the
    // common case (no P above the threshold) it is one straight stretch of
    // fma, exp2, pack and packed maxima (no maxima in a first pass, opt);
    // the row maxima and the rescale branches only run on tile 0 and where
    // a base moves.
    auto valu_step = [&](int jj, bool opt) __attribute__((always_inline)) {
        // (Tiles past this wave's rows go to dead_steps and do not get here;
        // the check is kept for the register allocation it leads to: without
        // it the two-block kernel takes two more VGPRs.)
        if (jj >= n_live) return;
        mask_tile(jj);
        if (jj > 0) {
            // Past tile 0 every row's base is finite (each row sees key 0
            // there): P against it, keeping S for the rare case below, and
            // the lane's largest packed P. P >= 0, and non-negative 16-bit
            // floats order as their bit patterns do, so bf16 values read as
            // fp16 keep their order up to ~2^121; beyond that they read as
            // inf or NaN, which the test below also catches (as it catches
            // an overflowed P, inf or NaN).
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float m_sub = m_used[qb];
#pragma unroll
                for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 8 * (kb2 & 1) + 2 * e;
                        const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb2 >> 1][i], c2, -m_sub));
                        const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb2 >> 1][i + 1], c2, -m_sub));
                        pk[qb][kb2][e] = Op::pack2(p0, p1);
                    }
            }
            if (opt) {
                // First pass: no overflow test (l is checked at the end).
                // The empty asm keeps P inside this step: with nothing here
                // reading it, the compiler would sink its computation past
                // the barrier into the next MFMA step, next to the products
                // that use it.
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    need[qb] = false;
#pragma unroll
                    for (int kb2 = 0; kb2 < 4; ++kb2) asm volatile("" : "+v"(pk[qb][kb2]));
                }
                return;
            }
            uint32_t c = 0u;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                uint32_t cq = pk_max3_f16(pk[qb][0][0], pk[qb][0][1], pk[qb][0][2]);
                cq = pk_max3_f16(cq, pk[qb][0][3], pk[qb][1][0]);
                cq = pk_max3_f16(cq, pk[qb][1][1], pk[qb][1][2]);
                cq = pk_max3_f16(cq, pk[qb][1][3], pk[qb][2][0]);
                cq = pk_max3_f16(cq, pk[qb][2][1], pk[qb][2][2]);
                cq = pk_max3_f16(cq, pk[qb][2][3], pk[qb][3][0]);
                cq = pk_max3_f16(cq, pk[qb][3][1], pk[qb][3][2]);
                cq = pk_max3_f16(cq, pk[qb][3][3], pk[qb][3][3]);
                c = qb == 0 ? cq : pk_max3_f16(c, cq, cq);
            }
            // The threshold as a packed value read as fp16: bf16 2^64 (0x5f80)
            // reads 480, fp16 2^15 is 32768.
            const _Float16 lim = IS_BF16 ? (_Float16)480.0f : (_Float16)32768.0f;
            const _Float16 lo = __builtin_bit_cast(_Float16, (uint16_t)(c & 0xffffu));
            const _Float16 hi = __builtin_bit_cast(_Float16, (uint16_t)(c >> 16));
            const bool over = !(lo <= lim) || !(hi <= lim);
            if (__builtin_amdgcn_ballot_w64(over) == 0) {
                // No P above the threshold: every base stays.
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) need[qb] = false;
                return;
            }
        }
        // Tile 0, or some P above the threshold: the exact rule, on S.
        row_max_need();
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            // The base is -inf only while every score so far is masked, which
            // takes a masked tile; it is then replaced by 0 so that the -inf
            // scores give 0 instead of NaN.
            const float m_sub = (jj >= j_mask && m_used[qb] == -INFINITY) ? 0.f : m_used[qb];
#pragma unroll
            for (int kb2 = 0; kb2 < 4; ++kb2)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // entries 8(kb2%2) + 2e, +1 of S block kb2/2
                    const int i = 8 * (kb2 & 1) + 2 * e;
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb2 >> 1][i], c2, -m_sub));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb2 >> 1][i + 1], c2, -m_sub));
                    pk[qb][kb2][e] = Op::pack2(p0, p1);
                }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            if (__builtin_amdgcn_ballot_w64(need[qb]) != 0) {
                // Rare: the base moved for some row of the block.
                const float alpha = need[qb] ? __builtin_amdgcn_exp2f(m_old[qb] - m_used[qb]) : 1.f;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) o[qb][db][i] *= alpha;
                // Row-sum entries 0 / 1 belong to queries l%16 / l%16 + 16.
                lacc[qb][0] *= alpha;
                lacc[qb][1] *= permlane16_swap_y(alpha, alpha);
            }
        }
    };

    // Workgroup barrier without a memory fence: the LDS reads of a step are
    // consumed by its MFMAs before the wave gets here, and the copies are
    // waited for explicitly, so a fence would only expose HBM latency. The
    // scheduling barriers keep every instruction of a step inside its
    // interval, so MFMA and softmax work of one wave never share one.
    auto barrier = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };
    // Group A issues all copies, at the start of its MFMA step of tile j:
    // K(j+1) -> k_lds[(j+1)&1], V(j) -> v_lds[j&1].
    auto copies = [&](int j, auto par_tag) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_tag)::value;   // j & 1
        if (grp == 0) {
            if (j + 1 < n_tiles)
                copy_tile<D>(Kg, (j + 1) * kBlockN, N, (LDS_AS char*)(PAR ? k_lds0 : k_lds1), wave, koff_src);
            copy_tile<D>(Vg, j * kBlockN, N, (LDS_AS char*)(PAR ? v_lds1 : v_lds0), wave, voff_src);
        }
    };
    // One tile: MFMA step, barrier, VALU step, barrier (group A first waits
    // for its copies, which the next step reads).
    auto tile_steps = [&](int j, auto par_tag, auto has_pv_tag, bool opt) __attribute__((always_inline)) {
        copies(j, par_tag);
        ATTN_PROBE(j);
        mfma_step(j, par_tag, has_pv_tag, std::true_type{});
        ATTN_PROBE(j + 1);
        barrier();
        valu_step(j, opt);
        if (grp == 0) __builtin_amdgcn_s_waitcnt(0x0f70);
        ATTN_PROBE(j + 2);
        barrier();
    };

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using NoPV = std::integral_constant<bool, false>;
    using WithPV = std::integral_constant<bool, true>;

    // Under a causal mask the tiles n_live .. n_tiles-1 are dead for this
    // wave: it only takes part in their copies and barriers (every wave of
    // the workgroup passes the same 2 n_tiles + 1 barriers), and the first
    // of them still holds the P.V products of tile n_live-1. Leaving out
    // their S products (which a branch inside the MFMA step could only do
    // with register copies and spills) is +1.2-1.4 % on the causal
    // workloads.
    auto dead_steps = [&](int j, auto par_tag, auto first_tag) __attribute__((always_inline)) {
        copies(j, par_tag);
        ATTN_PROBE(j);
        if constexpr (decltype(first_tag)::value) mfma_step(j, par_tag, std::true_type{}, std::false_type{});
        ATTN_PROBE(j + 1);
        barrier();
        if (grp == 0) __builtin_amdgcn_s_waitcnt(0x0f70);
        ATTN_PROBE(j + 2);
        barrier();
    };

    constexpr bool opt = OPT;
    // Group B runs one step behind group A.
    if (grp == 1) barrier();
    tile_steps(0, P0{}, NoPV{}, opt);
    int j = 1;
    // (Without a mask n_live is n_tiles.)
    const int n_loop = CAUSAL ? n_live : n_tiles;
    for (; j + 1 < n_loop; j += 2) {
        tile_steps(j, P1{}, WithPV{}, opt);
        tile_steps(j + 1, P0{}, WithPV{}, opt);
    }
    if (j < n_loop) tile_steps(j, P1{}, WithPV{}, opt);
    if constexpr (CAUSAL) {
        j = n_live;
        if (j < n_tiles) {
            if (j & 1) dead_steps(j, P1{}, std::true_type{});
            else dead_steps(j, P0{}, std::true_type{});
            for (++j; j < n_tiles; ++j) {
                if (j & 1) dead_steps(j, P1{}, std::false_type{});
                else dead_steps(j, P0{}, std::false_type{});
            }
        }
    }
    // Final P.V of tile n_tiles-1 when it is live for this wave (no S).
    if (n_tiles & 1) mfma_step(n_tiles, P1{}, WithPV{}, std::false_type{});
    else mfma_step(n_tiles, P0{}, WithPV{}, std::false_type{});
    if (grp == 0) barrier();

    if constexpr (OPT) {
        // Without the per-tile test every row kept the base tile 0 gave it.
        // A P above the threshold T would make its row's l (at least every P
        // of the row) exceed it, so a row with l <= T saw no such P, and its
        // bits are those of the exact pass, which only moves a base where
        // some P exceeds T. If any row of the item fails (score maxima that
        // rise by more than log2 T after tile 0, an overflow, or, for fp16,
        // many keys close to T), the workgroup hands the item to the exact
        // pass.
        bool bad = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            bad = bad || !(permlane16_swap_x(lacc[qb][0], lacc[qb][1]) <= (IS_BF16 ? 0x1p64f : 0x1p15f));
        if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) redo_flag = 1;
        __syncthreads();
        // (Read as a wave-uniform value, so that the branch is uniform too
        // and nothing of this pass stays live into the exact one.)
        if (__builtin_amdgcn_readfirstlane(redo_flag) != 0) return false;
    }

    // Epilogue: O = O~ / l, rounded once to the output type; lse in fp32.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qi = qw + 32 * qb + l32;
        // Entry 1 of lanes 0-15 / 32-47 moves to lanes 16-31 / 48-63.
        const float l_tot = permlane16_swap_x(lacc[qb][0], lacc[qb][1]);
        const float inv = 1.f / l_tot;
        if (qi < N) {
            uint16_t* Og = (uint16_t*)p.o + base + (size_t)qi * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int dd = 32 * db + 8 * i4 + 4 * g;
                    const u32x2 wv = {Op::pack2(o[qb][db][4 * i4] * inv, o[qb][db][4 * i4 + 1] * inv),
                                      Op::pack2(o[qb][db][4 * i4 + 2] * inv, o[qb][db][4 * i4 + 3] * inv)};
                    *(u32x2*)(Og + dd) = wv;
                }
            if (g == 0) p.lse[(size_t)bh * N + qi] = (m_used[qb] + log2f(l_tot)) * kLn2;
        }
    }
    return true;
}

// The exact pass for a bf16 work item whose first pass failed its check: a
// function of its own, so that its registers are allocated apart from the
// kernel's main path, which it follows only in that rare case.
// (Arguments reach a function in vector registers: the parameters and the
// workgroup index are made wave-uniform again; the thread index is passed
// in, so that the kernel need not keep the hardware's work-item ids for the
// call.)
template <bool IS_BF16, int D, bool CAUSAL, int QB>
__device__ __attribute__((noinline)) void fwd16_exact_item(FwdParams pv, int tid, int bid) {
    static_assert(sizeof(FwdParams) % 4 == 0, "FwdParams is read as 32-bit words");
    uint32_t w[sizeof(FwdParams) / 4];
    __builtin_memcpy(w, &pv, sizeof(FwdParams));
#pragma unroll
    for (int i = 0; i < (int)(sizeof(FwdParams) / 4); ++i) w[i] = __builtin_amdgcn_readfirstlane(w[i]);
    FwdParams p;
    __builtin_memcpy(&p, w, sizeof(FwdParams));
    (void)fwd16_pass<IS_BF16, D, CAUSAL, QB, false>(p, tid, __builtin_amdgcn_readfirstlane(bid));
}

// d = 64 with one query block: four waves per SIMD (two workgroups per
// compute unit), i.e. at most 128 VGPRs; the others take two waves per SIMD.
// FIRST: the pass without the per-tile overflow test first (d = 64 only).
template <bool IS_BF16, int D, bool CAUSAL, int QB, bool FIRST>
__global__ __launch_bounds__(kThreads, (D == 64 && QB == 1) ? 4 : 1) void fwd16_kernel(FwdParams p) {
    static_assert(!FIRST || D == 64, "the first pass is d = 64 only");
    const int tid = threadIdx.x, bid = blockIdx.x;
    if constexpr (FIRST) {
        if (!fwd16_pass<IS_BF16, D, CAUSAL, QB, true>(p, tid, bid)) {
            fwd16_exact_item<IS_BF16, D, CAUSAL, QB>(p, tid, bid);
            // The wave ends here: no path leads from the call back into the
            // first pass's epilogue (whose values would then have to live
            // across the call).
            __builtin_amdgcn_endpgm();
        }
    } else {
        (void)fwd16_pass<IS_BF16, D, CAUSAL, QB, false>(p, tid, bid);
    }
}

// Sequence length up to which fp16 takes the first pass: its check, l <= 2^15,
// holds on every row whose later scores stay at or below its first tile's
// maximum as long as N <= 2^15 (each P <= 1, so l <= N), flat rows
// included, and on i.i.d. rows far beyond (l ~ 5600 at N = 16384); past
// 2^15 keys flat rows would fail it and pay for both passes. Measured
// against the exact pass alone (B1 H8 d64): N = 24576 +5.7 %, 32768 +3.8 %,
// 32768 causal +6.4 %, 32768 flat +8.5 %. bf16 (2^64) always takes it.
constexpr int64_t kFp16FirstPassMaxN = 32768;

template <bool IS_BF16, int D, bool CAUSAL, int QB>
hipError_t launch_qb(FwdParams p, int force_first, hipStream_t s) {
    p.n_qtiles = (int)((p.N + block_m<QB>() - 1) / block_m<QB>());
    // XCD-major order only without a causal mask, where every item is as
    // long as every other: measured at B1 H32 N8192 d128 it cuts the L2
    // misses from 3.0x the Q, K, V bytes to 1.0x at the same speed. Under a
    // causal mask it would put all query tiles of a few slices into one
    // round (long and short items sharing compute units): 22 % slower at
    // B4 H16 N4096 d64, so those grids stay tile-major.
    p.xcd_order = (!CAUSAL && fwdorder::xcd_major_applies(p.BH_kv)) ? 1 : 0;
    if (p.force_order == 1) p.xcd_order = 0;
    if (p.force_order == 2 && fwdorder::xcd_major_applies(p.BH_kv)) p.xcd_order = 1;
    const dim3 grid((unsigned)(p.n_qtiles * p.BH));
    // d = 64: first the pass without the per-tile overflow test (+3 % at
    // the causal workloads, +4 % with two query blocks); at d = 128 (+0.8 %
    // alone, and the call into the exact pass costs more than that there)
    // the exact pass only.
    if constexpr (D == 64) {
        const bool first = force_first == 0 ? (IS_BF16 || p.N <= kFp16FirstPassMaxN) : force_first == 2;
        if (first) {
            hipLaunchKernelGGL((fwd16_kernel<IS_BF16, D, CAUSAL, QB, true>), grid, dim3(kThreads), 0, s, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((fwd16_kernel<IS_BF16, D, CAUSAL, QB, false>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

// Two query blocks per wave only at d = 64, when their work items still
// cover every compute unit, and under a causal mask only from 8192 keys on
// (measured: +2.5 to +6 % on long non-causal runs; causal, bf16, against
// one block: N = 2048 -5.4 %, 4096 -0.7 %, 8192 +3.0 %, 16384 +4.5 %: the
// 512-row items' diagonal tiles, whose dead waves no second workgroup on
// the compute unit fills, weigh less in longer items; on short sequences
// one block is up to 50 % faster through the doubled item count).
constexpr int64_t kCausalTwoBlockMinN = 8192;

template <bool IS_BF16, int D, bool CAUSAL>
hipError_t launch(const FwdParams& p, int force_first, hipStream_t s) {
    if constexpr (D == 64) {
        const int64_t items2 = (p.N + block_m<2>() - 1) / block_m<2>() * p.BH;
        const bool automatic = items2 >= kComputeUnits && (!CAUSAL || p.N >= kCausalTwoBlockMinN);
        const bool two = p.force_qb == 0 ? automatic : p.force_qb == 2;
        if (two) return launch_qb<IS_BF16, D, CAUSAL, 2>(p, force_first, s);
    }
    return launch_qb<IS_BF16, D, CAUSAL, 1>(p, force_first, s);
}
}  // namespace

hipError_t launch_fwd16(const FwdParams& p, bool is_bf16, int d, bool causal, int force_first,
                        hipStream_t s) {
    const int f = force_first;
    if (is_bf16) {
        if (d == 64) return causal ? launch<true, 64, true>(p, f, s) : launch<true, 64, false>(p, f, s);
        return causal ? launch<true, 128, true>(p, f, s) : launch<true, 128, false>(p, f, s);
    }
    if (d == 64) return causal ? launch<false, 64, true>(p, f, s) : launch<false, 64, false>(p, f, s);
    return causal ? launch<false, 128, true>(p, f, s) : launch<false, 128, false>(p, f, s);
}

}  // namespace attn
