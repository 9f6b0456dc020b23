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
    int BH;             // B * H slices
    int n_qtiles;       // ceil(N / query-tile rows)
    float scale_log2;   // scale * log2(e): scores enter exp2 directly
};

// Query rows per workgroup for every kernel here.
constexpr int kBlockM = 128;

// Launchers return the hipError_t of the launch.
hipError_t launch_fwd16(const FwdParams& p, bool is_bf16, int d, bool causal, hipStream_t s);
hipError_t launch_fwd32(const FwdParams& p, int d, bool causal, hipStream_t s);

}  // namespace attn
