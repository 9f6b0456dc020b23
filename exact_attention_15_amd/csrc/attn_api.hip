// attn_api.hip — the C ABI of libattn.so: argument validation, dispatch on
// (dtype, head dim, causal) and launch on the caller's stream.
//
// Validation happens before any HIP call, so an error code means nothing was
// enqueued. The library allocates nothing; its one piece of state is the
// per-device address of attn_bwd_noalloc's static row-statistic array.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/attn.h"
#include "attn_internal.h"

namespace {

int validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
             int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d, int causal, float scale,
             int dtype) {
    if (!q || !k || !v || !o || !lse) return ATTN_EINVAL;
    if (B < 1 || H < 1 || N < 1) return ATTN_EINVAL;
    if (H_kv < 1 || H % H_kv != 0) return ATTN_EINVAL;
    if (causal != 0 && causal != 1) return ATTN_EINVAL;
    if (!isfinite(scale) || !(scale > 0.f)) return ATTN_EINVAL;
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_EINVAL;
    // Positions are 32-bit inside the kernels; the grid is one-dimensional.
    if (N > (int64_t)INT32_MAX - attn::kMinBlockM) return ATTN_EINVAL;
    if (B > INT32_MAX / H) return ATTN_EINVAL;
    const int64_t n_qtiles = (N + attn::kMinBlockM - 1) / attn::kMinBlockM;
    if (n_qtiles * B * H > (int64_t)INT32_MAX) return ATTN_EINVAL;
    if (d != 64 && d != 128) return ATTN_EUNSUPPORTED;
    const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u;
    if (mis != 0 || ((uintptr_t)lse & 3u) != 0) return ATTN_EALIGN;
    return ATTN_OK;
}

// attn_bwd's checks other than those of `delta`.
int validate_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, const void* dq, const void* dk, const void* dv, int64_t B,
                 int64_t H, int64_t H_kv, int64_t N, int64_t d, int causal, float scale,
                 int dtype) {
    const int rc = validate(q, k, v, o, lse, B, H, H_kv, N, d, causal, scale, dtype);
    if (rc != ATTN_OK) return rc;
    if (!dout || !dq || !dk || !dv) return ATTN_EINVAL;
    // The row-statistic kernel covers 16 rows or more per workgroup.
    if (B * H * N / 16 >= (int64_t)INT32_MAX) return ATTN_EINVAL;
    const uintptr_t mis = ((uintptr_t)dout | (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15u;
    return mis != 0 ? ATTN_EALIGN : ATTN_OK;
}

// Variant overrides of attn_debug_set_fwd_variant (0: automatic).
std::atomic<int> g_force_qb{0};
std::atomic<int> g_force_order{0};
// Override of attn_debug_set_fwd_first_pass (0: automatic).
std::atomic<int> g_force_first{0};

}  // namespace

extern "C" int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                            int causal, float scale, int dtype, void* stream) {
    const int rc = validate(q, k, v, o, lse, B, H, H_kv, N, d, causal, scale, dtype);
    if (rc != ATTN_OK) return rc;

    attn::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.N = N;
    p.BH = (int)(B * H);
    p.BH_kv = (int)(B * H_kv);
    p.H_kv = (int)H_kv;
    p.G = (int)(H / H_kv);
    p.n_qtiles = 0;    // set by the launcher for its own query tile
    p.xcd_order = 0;   // chosen by the launcher
    p.force_qb = g_force_qb.load(std::memory_order_relaxed);
    p.force_order = g_force_order.load(std::memory_order_relaxed);
    // scale * log2(e), rounded once to fp32: scores go straight into exp2.
    p.scale_log2 = (float)((double)scale * 1.4426950408889634074);

    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();   // clear a stale error so the launch is judged alone
    hipError_t e;
    if (dtype == ATTN_F32)
        e = attn::launch_fwd32(p, (int)d, causal != 0, s);
    else
        e = attn::launch_fwd16(p, dtype == ATTN_BF16, (int)d, causal != 0,
                              g_force_first.load(std::memory_order_relaxed), s);
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        float* delta, int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                        int causal, float scale, int dtype, void* stream) {
    const int rc = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, N, d, causal,
                                scale, dtype);
    if (rc != ATTN_OK) return rc;
    if (!delta) return ATTN_EINVAL;
    if (((uintptr_t)delta & 3u) != 0) return ATTN_EALIGN;

    attn::BwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = dout;
    p.lse = lse;
    p.delta = delta;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.N = N;
    p.BH = (int)(B * H);
    p.BH_kv = (int)(B * H_kv);
    p.H_kv = (int)H_kv;
    p.G = (int)(H / H_kv);
    p.chunk = 0;    // chosen by the launcher
    p.scale = scale;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634074);

    (void)hipGetLastError();
    const hipError_t e =
        dtype == ATTN_F32
            ? attn::launch_bwd32(p, (int)d, causal != 0, (hipStream_t)stream)
            : attn::launch_bwd16(p, dtype == ATTN_BF16, (int)d, causal != 0, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

// ---------------------------------------------------------------------------
// Allocation-free backward: the row statistic D (B*H*N floats), which
// attn_bwd keeps in the caller's `delta`, lives in this file-scope device
// array instead. Each device holds its own copy from the library's load to
// the end of the process. In host code `scratch` names a host-side stand-in,
// not device memory: kernels get the address hipGetSymbolAddress returns for
// the current device, fetched once per device on its first call.
static __device__ __align__(256) float scratch[ATTN_BWD_NOALLOC_MAX_ROWS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, or nullptr on a HIP
// error (the error code goes to *err).
float* device_scratch(hipError_t* err) {
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (*err != hipSuccess || !ptr) {
            if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
            return nullptr;
        }
        g_scratch_ptr[dev] = (float*)ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t d,
                                int causal, float scale, int dtype, void* stream) {
    // attn_bwd's checks and the size limit of the static array, before any
    // HIP call.
    const int rc = validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, N, d, causal,
                                scale, dtype);
    if (rc != ATTN_OK) return rc;
    if (B * H > ATTN_BWD_NOALLOC_MAX_ROWS / N) return ATTN_ETOOBIG;
    hipError_t e;
    float* delta = device_scratch(&e);
    if (!delta) return ATTN_EHIP;
    return attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, H_kv, N, d, causal, scale,
                    dtype, stream);
}

extern "C" int64_t attn_unfused_workspace_bytes(int64_t B, int64_t H, int64_t N, int dtype) {
    if (B < 1 || H < 1 || N < 1 || N > (int64_t)INT32_MAX - 64) return -1;
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return -1;
    const int64_t ld = (N + 63) / 64 * 64;
    if (B > INT64_MAX / H || B * H > INT64_MAX / N || B * H * N > INT64_MAX / ld / 8) return -1;
    // fp32 scores + probabilities in the input type
    return B * H * N * ld * (dtype == ATTN_F32 ? 8 : 6);
}

extern "C" int attn_fwd_unfused(const void* q, const void* k, const void* v, void* o, float* lse,
                                void* workspace, int64_t workspace_bytes, int64_t B, int64_t H,
                                int64_t N, int64_t d, int causal, float scale, int dtype,
                                void* stream) {
    const int rc = validate(q, k, v, o, lse, B, H, H, N, d, causal, scale, dtype);
    if (rc != ATTN_OK) return rc;
    if (!workspace) return ATTN_EINVAL;
    const int64_t need = attn_unfused_workspace_bytes(B, H, N, dtype);
    if (need < 0 || workspace_bytes < need) return ATTN_EINVAL;
    const int64_t nt = (N + 63) / 64;
    if (B * H > (int64_t)INT32_MAX / nt / nt) return ATTN_EINVAL;   // one-dimensional grid
    if (((uintptr_t)workspace & 255u) != 0) return ATTN_EALIGN;

    attn::UnfusedParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.N = N;
    p.ld = nt * 64;
    p.BH = (int)(B * H);
    p.causal = causal;
    p.scale = scale;
    p.s = (float*)workspace;
    p.pm = (char*)workspace + B * H * N * p.ld * 4;
    (void)hipGetLastError();
    const hipError_t e =
        dtype == ATTN_F32
            ? attn::launch_unfused32(p, (int)d, (hipStream_t)stream)
            : attn::launch_unfused16(p, dtype == ATTN_BF16, (int)d, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : ATTN_EHIP;
}

extern "C" int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                        int dtype, void* stream) {
    return attn_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, dtype, stream);
}

extern "C" int attn_debug_set_fwd_variant(int query_blocks, int order) {
    if (query_blocks < 0 || query_blocks > 2 || order < 0 || order > 2) return ATTN_EINVAL;
    g_force_qb.store(query_blocks, std::memory_order_relaxed);
    g_force_order.store(order, std::memory_order_relaxed);
    return ATTN_OK;
}

extern "C" int attn_debug_set_fwd_first_pass(int mode) {
    if (mode < 0 || mode > 2) return ATTN_EINVAL;
    g_force_first.store(mode, std::memory_order_relaxed);
    return ATTN_OK;
}

extern "C" const char* attn_strerror(int code) {
    switch (code) {
        case ATTN_OK: return "ok";
        case ATTN_EINVAL: return "invalid argument (pointer, size, H_kv, dtype, scale or causal)";
        case ATTN_EUNSUPPORTED: return "unsupported head dimension (need 64 or 128)";
        case ATTN_EALIGN: return "a tensor pointer is misaligned (16 bytes; lse, delta 4; workspace 256)";
        case ATTN_EHIP: return "HIP kernel launch failed";
        case ATTN_ETOOBIG:
            return "B*H*N exceeds the static row-statistic array of attn_bwd_noalloc "
                   "(ATTN_BWD_NOALLOC_MAX_ROWS)";
        default: return "unknown error code";
    }
}
