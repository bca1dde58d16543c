// kda_fwd_chunked_noalloc: the chunked prefill for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  It is kda_fwd_chunked with its
// workspace taken from a fixed array that the library itself holds on every
// device it runs on, instead of a caller buffer.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "kda.h"
#include "kda_launch.h"

#define KDA_API extern "C" __attribute__((visibility("default")))

namespace {

// The scratch array: one copy per device, resident until the process ends.
// Its name is a host-side stand-in; host code uses only the per-device
// address that hipGetSymbolAddress returns (scratch_ptr below).
constexpr size_t kScratchBytes = KDA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices];
bool g_have[kMaxDevices];

// Address of `scratch` on `dev`, looked up once per device with that device
// current.
hipError_t scratch_ptr(int dev, void **out)
{
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_have[dev]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        g_ptr[dev] = p;
        g_have[dev] = true;
    }
    *out = g_ptr[dev];
    return hipSuccess;
}

}  // namespace

KDA_API kda_status kda_fwd_chunked_noalloc(const void *q, const void *k, const void *v,
                                           const float *g, const float *beta, const float *S0,
                                           const int32_t *cu_seqlens, int32_t n_seqs,
                                           int64_t n_tokens, int32_t H, int32_t d_k,
                                           int32_t d_v, kda_dtype in_dtype,
                                           kda_dtype out_dtype, void *o, float *S_T,
                                           kda_stream_t stream)
{
    // a packed batch never takes the sequence-split path; invalid sizes give
    // 0 here and are reported by kda_fwd_chunked
    const size_t need =
        cu_seqlens ? 0 : kda_fwd_workspace_bytes(n_seqs, n_tokens, H, d_k, d_v, in_dtype);
    if (need > kScratchBytes)
        return kda::set_error(KDA_ERR_INVALID_ARG,
                              "kda_fwd_chunked_noalloc: these sizes need %zu bytes of scratch, "
                              "above the %zu bytes the library holds per device; call "
                              "kda_fwd_chunked with a workspace instead",
                              need, kScratchBytes);
    if (need == 0)
        return kda_fwd_chunked(q, k, v, g, beta, S0, cu_seqlens, n_seqs, n_tokens, H, d_k, d_v,
                               in_dtype, out_dtype, o, S_T, nullptr, 0, stream);
    int dev = 0;
    hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
    void *ws = nullptr;
    if (e == hipSuccess) e = scratch_ptr(dev, &ws);
    if (e != hipSuccess)
        return kda::set_error(KDA_ERR_HIP, "kda_fwd_chunked_noalloc: scratch address: %s",
                              hipGetErrorString(e));
    return kda_fwd_chunked(q, k, v, g, beta, S0, cu_seqlens, n_seqs, n_tokens, H, d_k, d_v,
                           in_dtype, out_dtype, o, S_T, ws, need, stream);
}
