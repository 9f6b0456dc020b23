// attn_internal.h — parameters shared by the host entry point and the
// kernel launchers inside libattn.so (not part of the public C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int64_t N;          // sequence length (queries = keys)
    int BH;             // B * H query slices
    int BH_kv;          // B * H_kv key/value slices
    int H_kv;           // key/value heads; H_kv divides H
    int G;              // H / H_kv query heads per key/value head
    int n_qtiles;       // ceil(N / query-tile rows)
    int xcd_order;      // 1: XCD-major work order (fwd_order.h), 0: tile-major
    int force_qb;       // 0 automatic, 1 or 2 query blocks (attn_debug_set_fwd_variant)
    int force_order;    // 0 automatic, 1 tile-major, 2 XCD-major
    float scale_log2;   // scale * log2(e): scores enter exp2 directly
};

// Slice indices of work item r in [0, BH): the (b, h) query slice and the
// (b, h_kv) key/value slice it reads, h_kv = h / G (grouped-query attention:
// G consecutive query heads share one K/V head). The G query heads of one K/V
// head take the work items kv, kv + BH_kv, kv + 2 BH_kv, ...: the same
// position modulo 8, so the same XCD and L2, whenever BH_kv is a multiple
// of 8. With G = 1 both indices are r.
struct SliceIds {
    int bh;
    int kv_bh;
};

__device__ __forceinline__ SliceIds slice_of(const FwdParams& p, int r) {
    const int kv_bh = r % p.BH_kv;
    const int g = r / p.BH_kv;
    const int b = kv_bh / p.H_kv;
    const int h = (kv_bh - b * p.H_kv) * p.G + g;
    return {b * p.H_kv * p.G + h, kv_bh};
}

// Backward pass (gradients of the forward above).
struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    float* delta;       // D_i = dO_i . O_i, written by the first kernel
    void* dq;
    void* dk;
    void* dv;
    int64_t N;
    int BH;             // B * H query slices
    int BH_kv;          // B * H_kv key/value slices
    int H_kv;
    int G;              // H / H_kv
    int chunk;          // steps per dK/dV item when > 0 (partial dK, dV in dq's memory), else whole key tiles
    float scale;        // multiplied into dQ and dK
    float scale_log2;   // scale * log2(e)
};

// Unfused three-step forward (the materialised comparison path).
struct UnfusedParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    float* s;           // [B*H, N, ld] fp32 scores (workspace)
    void* pm;           // [B*H, N, ld] probabilities in the input type (workspace)
    int64_t N;
    int64_t ld;         // row stride of s and pm: N rounded up to 64
    int BH;
    int causal;
    float scale;
};

// Timing probe, compiled in only by the race-check build (ATTN_DELAY_PROBE):
// at each marked point a third of the (wave, step, workgroup) combinations
// sleep ~512 cycles, so the waves of a workgroup reach their barriers and
// buffer reuses in orders the normal build does not produce. Nothing else
// changes; results must stay bit-identical unless a buffer is overwritten
// while another wave still reads it.
#ifdef ATTN_DELAY_PROBE
#define ATTN_PROBE(step)                                                                      \
    do {                                                                                      \
        const int probe_w_ = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);           \
        if ((probe_w_ * 5 + (int)(step) * 3 + (int)blockIdx.x) % 3 == 0) __builtin_amdgcn_s_sleep(8); \
    } while (0)
#else
#define ATTN_PROBE(step) \
    do {                 \
    } while (0)
#endif

// The fewest query rows any forward workgroup takes (fp32, d = 64); bounds
// the one-dimensional grids.
constexpr int kMinBlockM = 64;

// Launchers return the hipError_t of the launch.
// force_first: 0 automatic, 1 exact pass only, 2 first pass at any N
// (attn_debug_set_fwd_first_pass). It stays out of FwdParams: the d = 64
// kernels hand FwdParams by value to their out-of-line exact pass, and one
// more word there made that call take the work-item ids and the dispatch
// pointer along: 6.7 % slower at B4 H16 N4096 d64 causal bf16 and 1.0 %
// at B1 H8 N16384 d64 fp16 (same machine, both builds alternating).
hipError_t launch_fwd16(const FwdParams& p, bool is_bf16, int d, bool causal, int force_first,
                        hipStream_t s);
hipError_t launch_fwd32(const FwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_bwd16(const BwdParams& p, bool is_bf16, int d, bool causal, hipStream_t s);
hipError_t launch_bwd32(const BwdParams& p, int d, bool causal, hipStream_t s);
hipError_t launch_unfused16(const UnfusedParams& p, bool is_bf16, int d, hipStream_t s);
hipError_t launch_unfused32(const UnfusedParams& p, int d, hipStream_t s);

}  // namespace attn
