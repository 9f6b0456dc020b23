// mfma_common.h — pieces shared by the gfx950 bf16/fp16 attention kernels
// (forward and backward): vector types, the 16-bit MFMA wrappers and the
// direct HBM -> LDS copy. Internal to libattn.so.
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

}  // namespace
}  // namespace attn
