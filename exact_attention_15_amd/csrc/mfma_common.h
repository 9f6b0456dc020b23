// mfma_common.h — pieces shared by the gfx950 bf16/fp16 attention kernels:
// vector types, the 16-bit MFMA wrappers, the direct HBM -> LDS copy, and
// the LDS tiles read both by rows and through ds_read_b64_tr_b16.
// Internal to libattn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

template <bool IS_BF16> struct Op16;

template <> struct Op16<true> {
    static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static constexpr uint32_t kOnePair = 0x3f803f80u;   // two bf16 1.0
    // Round two floats to bf16 (nearest even) and pack: x in the low half.
    static __device__ __forceinline__ uint32_t pack2(float x, float y) {
        bf16x2 v;
        v[0] = (__bf16)x;
        v[1] = (__bf16)y;
        return __builtin_bit_cast(uint32_t, v);
    }
};

template <> struct Op16<false> {
    static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static constexpr uint32_t kOnePair = 0x3c003c00u;   // two f16 1.0
    static __device__ __forceinline__ uint32_t pack2(float x, float y) {
        f16x2 v;
        v[0] = (_Float16)x;
        v[1] = (_Float16)y;
        return __builtin_bit_cast(uint32_t, v);
    }
};

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

// Buffer resource (V#) for raw buffer loads of `bytes` bytes from `base`:
// accesses at offsets >= bytes are out of range and return zeros.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int bytes) {
    const uint64_t addr = (uint64_t)base;
    i32x4 rsrc;
    rsrc[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
    rsrc[1] = __builtin_amdgcn_readfirstlane((int)((addr >> 32) & 0xffff));   // stride 0
    rsrc[2] = __builtin_amdgcn_readfirstlane(bytes);                          // bytes in range
    rsrc[3] = 0x00020000;                                                     // 32-bit data format
    return rsrc;
}

// A ROWS x D tile of 16-bit values in LDS, row-major, 16-byte chunk c of
// row r stored at chunk c ^ swz(r). The tile is read two ways:
//  * by rows: 16 bytes per lane, lanes 0-15 at rows 0-15 and one logical
//    chunk; needs rows 0-15 in 16 different 16-byte bank groups;
//  * by ds_read_b64_tr_b16: 32 lanes read 4 consecutive rows (4m .. 4m+3)
//    x 64 bytes (an aligned block of 4 chunks); needs the 4 rows' blocks in
//    4 different places.
// d = 64 (two rows per 256-byte bank row): swz takes bits 1-3 of r so that
// rows of one parity get 8 different values, with rows r and r+2 differing
// in bit 2 (the 64-byte half). d = 128: swz swaps the two low bit pairs of
// r, a permutation of 0-15 whose bits 2-3 differ across 4 aligned rows.
template <int ROWS, int D>
struct BTile {
    static constexpr int kRowBytes = D * 2;
    static constexpr int kChunks = D / 8;
    static constexpr int kBytes = ROWS * kRowBytes;
    static __device__ __forceinline__ int swz(int r) {
        return D == 64 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3))
                       : (((r & 3) << 2) | ((r >> 2) & 3));
    }
    // Row read: row r, logical chunk c.
    static __device__ __forceinline__ int row_off(int r, int c) {
        return r * kRowBytes + ((c ^ swz(r)) << 4);
    }
};

// HBM -> LDS copy of one ROWS x D tile by NW waves (16 bytes per lane per
// copy). Copy u of wave cw fills LDS chunk slots s = (cw*U + u)*64 + lane,
// i.e. row s / kChunks, physical chunk s % kChunks, with the global chunk
// (physical ^ swz(row)). Rows past N are outside the buffer range: zeros.
template <int ROWS, int D, int NW>
struct BCopy {
    using T = BTile<ROWS, D>;
    static constexpr int kPerWave = T::kBytes / 1024 / NW;
    static_assert(kPerWave >= 1 && T::kBytes % (1024 * NW) == 0, "tile / copy waves mismatch");
    static __device__ __forceinline__ void offsets(int cw, int lane, int* off) {
#pragma unroll
        for (int u = 0; u < kPerWave; ++u) {
            const int s = (cw * kPerWave + u) * 64 + lane;
            const int r = s / T::kChunks;
            const int pc = s % T::kChunks;
            off[u] = r * T::kRowBytes + ((pc ^ T::swz(r)) << 4);
        }
    }
    static __device__ __forceinline__ void copy(const uint16_t* g_slice, int row0, int N,
                                                LDS_AS char* buf, int cw, const int* off) {
        const int rows = min(max(N - row0, 0), ROWS);
        const i32x4 rsrc = buffer_rsrc(g_slice + (size_t)row0 * D, rows * T::kRowBytes);
        const uint32_t lds0 = (uint32_t)(uintptr_t)buf;
#pragma unroll
        for (int u = 0; u < kPerWave; ++u)
            dma16(rsrc, lds0 + (cw * kPerWave + u) * 64 * 16, off[u]);
    }
};

// Offsets of the ds_read_b64_tr_b16 reads that build a 32x32x16 A operand
// X^T[d][row] from a row-major tile X: in each group of 16 lanes, output
// lane j receives element j%4 of the 8-byte reads of source lanes j/4 + 4k.
// Source lane (G = lane/16, i = lane%16) reads row R(g, h) + i/4 (+16 kb2)
// at columns 32 db + 16 (G%2) + 4 (i%4), so output lane l holds
// X[16 kb2 + R(g, h) + k][32 db + l%32], k = 0..3, for the first (h = 0)
// and second (h = 1) read, i.e. operand element 4h + k of lane group g.
//   ACC_ORDER: R = 8h + 4g, the row order of a 32x32 accumulator's entries
//              (for operands paired with P or dS taken from an accumulator);
//   otherwise: R = 8g + 4h, natural order (operand element e of lane group
//              g is row 8g + e, as a B operand loaded from memory has it).
// The swizzle depends on row bits 2-3, hence one offset per h.
template <int ROWS, int D, bool ACC_ORDER = true>
__device__ __forceinline__ void tr_offsets(int lane, int (*off)[2]) {
    using T = BTile<ROWS, D>;
    const int g = lane >> 5, G = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = (ACC_ORDER ? 8 * h + 4 * g : 8 * g + 4 * h) + (i16 >> 2);
            const int col = 32 * db + 16 * (G & 1) + 4 * (i16 & 3);
            off[db][h] = row * T::kRowBytes + (((col >> 3) ^ T::swz(row)) << 4) + ((col >> 2) & 1) * 8;
        }
}

__device__ __forceinline__ u32x4 tr_read(const LDS_AS char* p0, const LDS_AS char* p1) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)p0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)p1);
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace
}  // namespace attn
