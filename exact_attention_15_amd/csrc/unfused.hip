// unfused.hip — the unfused three-step attention forward on gfx950, kept as
// the comparison that shows what fusion gains.
//
// Method: the materialised algorithm of the cishoon.github.io
// "flashattention" post, sections 2-3 (one kernel per step, the N x N score
// and probability matrices in global memory):
//   (1) S = scale Q K^T           -> fp32 [B*H, N, ld] in the workspace
//   (2) row softmax of S           -> P in the input type [B*H, N, ld], lse
//       (causal: keys j > i get probability 0, as in the fused path)
//   (3) O = P V                    -> O in the input type
// ld = N rounded up to 64, so that every row starts 16-byte aligned; P is
// zero in the padding columns.
//
// gfx950 design for bf16 / fp16: both products on
// v_mfma_f32_32x32x16_{bf16,f16} with fp32 accumulation. (1): a wave
// computes a 32x32 block of S straight from the Q and K rows in global
// memory (both operands are rows with the contraction index contiguous).
// (2): one wave per row, three passes over the row (max, sum, write).
// (3): O^T = V^T P^T per 32 query rows: P rows are the B operand as they lie
// in memory, V^T comes from 64-row V tiles in LDS through
// ds_read_b64_tr_b16 (natural row order).
// fp32: the same steps on v_mfma_f32_32x32x2f32, one pair of contraction
// indices per instruction: in (1) lane half g takes the head-dimension
// columns [g D/2, (g+1) D/2) of its Q and K rows, in (3) the keys
// [16g, 16g+16) of each 32-key step, with V tiles in LDS read one element
// per lane. P stays fp32.
// The full N x N matrices are computed even when causal, as the
// materialised method does.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "mfma_common.h"

namespace attn {
namespace {

constexpr int kUThreads = 256;   // 4 waves
constexpr float kULog2e = 1.44269504088896341f;
constexpr float kULn2 = 0.693147180559945309f;

// Writes a 32x32 accumulator block of scale Q K^T: entry r is row
// i0 + 8(r/4) + 4g + r%4, column j (one column per lane).
__device__ __forceinline__ void store_scores(const UnfusedParams& p, int bh, int i0, int j, int g,
                                             const f32x16& acc) {
    const int N = (int)p.N;
    if (j >= N) return;
    float* srow = p.s + (size_t)bh * N * p.ld + j;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int i = i0 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (i < N) srow[(size_t)i * p.ld] = acc[r] * p.scale;
    }
}

// (1) one 64x64 block of S per workgroup, a 32x32 block per wave.
template <bool IS_BF16, int D>
__global__ __launch_bounds__(kUThreads) void scores_kernel(UnfusedParams p) {
    using Op = Op16<IS_BF16>;
    constexpr int NKD = D / 16;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int N = (int)p.N;
    const int nt = (N + 63) / 64;
    const int w = blockIdx.x;
    const int bh = w / (nt * nt);
    const int rem = w - bh * nt * nt;
    const int i0 = (rem / nt) * 64 + 32 * (wave >> 1);
    const int j0 = (rem % nt) * 64 + 32 * (wave & 1);
    const size_t slice = (size_t)bh * N * D;
    const uint16_t* qr = (const uint16_t*)p.q + slice + (size_t)min(i0 + l32, N - 1) * D + 8 * g;
    const uint16_t* kr = (const uint16_t*)p.k + slice + (size_t)min(j0 + l32, N - 1) * D + 8 * g;
    f32x16 acc;
#pragma unroll
    for (int kd = 0; kd < NKD; ++kd) {
        const u32x4 a = *(const u32x4*)(qr + 16 * kd);
        const u32x4 b = *(const u32x4*)(kr + 16 * kd);
        acc = Op::mfma(a, b, kd == 0 ? f32x16{} : acc);
    }
    store_scores(p, bh, i0, j0 + l32, g, acc);
}

// fp32 (1): lane half g contracts the columns [g D/2, (g+1) D/2).
template <int D>
__global__ __launch_bounds__(kUThreads) void scores_f32_kernel(UnfusedParams p) {
    constexpr int HALF = D / 2;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int N = (int)p.N;
    const int nt = (N + 63) / 64;
    const int w = blockIdx.x;
    const int bh = w / (nt * nt);
    const int rem = w - bh * nt * nt;
    const int i0 = (rem / nt) * 64 + 32 * (wave >> 1);
    const int j0 = (rem % nt) * 64 + 32 * (wave & 1);
    const size_t slice = (size_t)bh * N * D;
    const float* qr = (const float*)p.q + slice + (size_t)min(i0 + l32, N - 1) * D + HALF * g;
    const float* kr = (const float*)p.k + slice + (size_t)min(j0 + l32, N - 1) * D + HALF * g;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int c = 0; c < HALF / 4; ++c) {
        const f32x4 a = *(const f32x4*)(qr + 4 * c);
        const f32x4 b = *(const f32x4*)(kr + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], acc, 0, 0, 0);
    }
    store_scores(p, bh, i0, j0 + l32, g, acc);
}

// (2) softmax of one row per wave: P = exp(s - m) / l over the visible keys,
// 0 elsewhere (masked keys and the padding columns); lse = m + ln l.
// PT: 0 fp16, 1 bf16, 2 fp32 probabilities.
template <int PT>
__global__ __launch_bounds__(kUThreads) void softmax_kernel(UnfusedParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kUThreads / 64) + (threadIdx.x >> 6);
    const int N = (int)p.N;
    if (row >= (int64_t)p.BH * N) return;
    const int i = (int)(row % N);
    const int n_vis = p.causal ? i + 1 : N;
    const float* srow = p.s + (size_t)row * p.ld;
    float m = -INFINITY;
    for (int j = lane; j < n_vis; j += 64) m = fmaxf(m, srow[j]);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) m = fmaxf(m, __shfl_xor(m, x));
    float l = 0.f;
    for (int j = lane; j < n_vis; j += 64) l += exp2f((srow[j] - m) * kULog2e);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) l += __shfl_xor(l, x);
    const float inv = 1.f / l;
    // Pairs of columns: ld is even, so every pair is one aligned store.
    for (int j = 2 * lane; j < p.ld; j += 128) {
        const float p0 = j < n_vis ? exp2f((srow[j] - m) * kULog2e) * inv : 0.f;
        const float p1 = j + 1 < n_vis ? exp2f((srow[j + 1] - m) * kULog2e) * inv : 0.f;
        if constexpr (PT == 2) {
            *(float2*)((float*)p.pm + (size_t)row * p.ld + j) = make_float2(p0, p1);
        } else {
            *(uint32_t*)((uint16_t*)p.pm + (size_t)row * p.ld + j) = Op16<PT == 1>::pack2(p0, p1);
        }
    }
    if (lane == 0) p.lse[row] = m + log2f(l) * kULn2;
}

// (3) O^T = V^T P^T for 32 query rows per wave, 64-key V tiles through LDS.
template <bool IS_BF16, int D>
__global__ __launch_bounds__(kUThreads) void pv_kernel(UnfusedParams p) {
    using Op = Op16<IS_BF16>;
    using T = BTile<64, D>;
    using Cp = BCopy<64, D, kUThreads / 64>;
    constexpr int NDB = D / 32;
    __shared__ __attribute__((aligned(1024))) char v_lds[T::kBytes];
    LDS_AS char* const vL = (LDS_AS char*)v_lds;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int N = (int)p.N;
    const int nq = (N + 127) / 128;
    const int bh = blockIdx.x / nq;
    const int qi = (blockIdx.x - bh * nq) * 128 + 32 * wave + l32;
    const uint16_t* Vg = (const uint16_t*)p.v + (size_t)bh * N * D;
    // B operand: lane l holds P[query l%32][key 8g .. 8g+7] of each 16-key chunk.
    const uint16_t* prow = (const uint16_t*)p.pm + ((size_t)bh * N + min(qi, N - 1)) * p.ld + 8 * g;
    int troff[NDB][2];
    tr_offsets<64, D, false>(lane, troff);
    int coff[Cp::kPerWave];
    Cp::offsets(wave, lane, coff);

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

    const int n_tiles = (N + 63) / 64;
    for (int t = 0; t < n_tiles; ++t) {
        Cp::copy(Vg, t * 64, N, vL, wave, coff);
        u32x4 pb[4];
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2) pb[kb2] = *(const u32x4*)(prow + t * 64 + 16 * kb2);
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): the tile copy and P
        ATTN_PROBE(t + 1);
        __syncthreads();
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int kb2 = 0; kb2 < 4; ++kb2) {
                const LDS_AS char* rb = vL + 16 * kb2 * T::kRowBytes;
                o[db] = Op::mfma(tr_read(rb + troff[db][0], rb + troff[db][1]), pb[kb2], o[db]);
            }
        ATTN_PROBE(t);
        __syncthreads();   // every wave has read the tile before the next copy
    }
    if (qi < N) {
        uint16_t* orow = (uint16_t*)p.o + ((size_t)bh * N + qi) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int dd = 32 * db + 8 * i4 + 4 * g;
                const u32x2 wv = {Op::pack2(o[db][4 * i4], o[db][4 * i4 + 1]),
                                  Op::pack2(o[db][4 * i4 + 2], o[db][4 * i4 + 3])};
                *(u32x2*)(orow + dd) = wv;
            }
    }
}

// fp32 (3): O^T = V^T P^T for 32 query rows per wave. Per 32-key step, lane
// half g takes keys [16g, 16g+16): B = P[query l32][key] from the lane's own
// P row, A = V[key][32 db + l32] from the 64-row V tile in LDS (row-major,
// unpadded; the two lane halves read different rows of one column block).
template <int D>
__global__ __launch_bounds__(kUThreads) void pv_f32_kernel(UnfusedParams p) {
    constexpr int NDB = D / 32;
    constexpr int kTileBytes = 64 * D * 4;
    constexpr int kPerWave = kTileBytes / 1024 / (kUThreads / 64);   // 16-byte chunks per lane
    __shared__ __attribute__((aligned(1024))) float v_lds[64 * D];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(LDS_AS char*)v_lds;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l32 = lane & 31, g = lane >> 5;
    const int N = (int)p.N;
    const int nq = (N + 127) / 128;
    const int bh = blockIdx.x / nq;
    const int qi = (blockIdx.x - bh * nq) * 128 + 32 * wave + l32;
    const float* Vg = (const float*)p.v + (size_t)bh * N * D;
    const float* prow = (const float*)p.pm + ((size_t)bh * N + min(qi, N - 1)) * p.ld + 16 * g;

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = 0.f;

    const int n_tiles = (N + 63) / 64;
    for (int t = 0; t < n_tiles; ++t) {
        // V rows t*64 .. : the buffer range ends at row N, later rows read 0.
        const i32x4 rsrc = buffer_rsrc(Vg + (size_t)t * 64 * D, min(N - t * 64, 64) * D * 4);
#pragma unroll
        for (int u = 0; u < kPerWave; ++u) {
            const int c = wave * kPerWave + u;
            dma16(rsrc, lds0 + c * 1024, (c * 64 + lane) * 16);
        }
        f32x4 pb[8];   // pb[4h + i]: keys 32h + 16g + 4i .. +3 of the tile
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) pb[4 * h + i] = *(const f32x4*)(prow + t * 64 + 32 * h + 4 * i);
        __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): the tile copy and P
        ATTN_PROBE(t + 1);
        __syncthreads();
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int tt = 0; tt < 16; ++tt) {
                const float* vr = v_lds + (32 * h + 16 * g + tt) * D + l32;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[32 * db], pb[4 * h + (tt >> 2)][tt & 3],
                                                                 o[db], 0, 0, 0);
            }
        ATTN_PROBE(t);
        __syncthreads();   // every wave has read the tile before the next copy
    }
    if (qi < N) {
        float* orow = (float*)p.o + ((size_t)bh * N + qi) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const f32x4 wv = {o[db][4 * i4], o[db][4 * i4 + 1], o[db][4 * i4 + 2], o[db][4 * i4 + 3]};
                *(f32x4*)(orow + 32 * db + 8 * i4 + 4 * g) = wv;
            }
    }
}

template <bool IS_BF16, int D>
hipError_t launch(const UnfusedParams& p, hipStream_t s) {
    const int64_t nt = (p.N + 63) / 64;
    hipLaunchKernelGGL((scores_kernel<IS_BF16, D>), dim3((unsigned)(p.BH * nt * nt)),
                       dim3(kUThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)p.BH * p.N;
    hipLaunchKernelGGL((softmax_kernel<IS_BF16 ? 1 : 0>), dim3((unsigned)((rows + 3) / 4)),
                       dim3(kUThreads), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nq = (p.N + 127) / 128;
    hipLaunchKernelGGL((pv_kernel<IS_BF16, D>), dim3((unsigned)(p.BH * nq)), dim3(kUThreads), 0,
                       s, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const UnfusedParams& p, hipStream_t s) {
    const int64_t nt = (p.N + 63) / 64;
    hipLaunchKernelGGL((scores_f32_kernel<D>), dim3((unsigned)(p.BH * nt * nt)), dim3(kUThreads),
                       0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)p.BH * p.N;
    hipLaunchKernelGGL((softmax_kernel<2>), dim3((unsigned)((rows + 3) / 4)), dim3(kUThreads), 0,
                       s, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nq = (p.N + 127) / 128;
    hipLaunchKernelGGL((pv_f32_kernel<D>), dim3((unsigned)(p.BH * nq)), dim3(kUThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_unfused16(const UnfusedParams& p, bool is_bf16, int d, hipStream_t s) {
    if (is_bf16) return d == 64 ? launch<true, 64>(p, s) : launch<true, 128>(p, s);
    return d == 64 ? launch<false, 64>(p, s) : launch<false, 128>(p, s);
}

hipError_t launch_unfused32(const UnfusedParams& p, int d, hipStream_t s) {
    return d == 64 ? launch_f32<64>(p, s) : launch_f32<128>(p, s);
}

}  // namespace attn
