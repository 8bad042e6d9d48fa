// sgla_chunk_bwd_noalloc: the chunked backward without a caller workspace and
// without any allocation, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). Its kernels are those of sgla_chunk_bwd; the scratch they need
// (the per sequence-head partial sums of da) lives in a fixed device array of
// this file instead of a workspace argument.
//
// The array is a file-scope __device__ symbol, so every GPU the library runs
// on holds its own copy, at its own address, until the process ends. Host
// code never passes the array's name to a kernel (on the host it only stands
// in for the symbol): the device address comes from hipGetSymbolAddress, once
// per device with that device current, and is kept per device.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "sgla.h"
#include "sgla_internal.h"

namespace {

static __device__ __align__(256) char scratch[SGLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up on the
// first call made with that device current.
sgla_status current_scratch(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        char msg[160];
        std::snprintf(msg, sizeof(msg), "hipGetDevice: %s", hipGetErrorString(e));
        return sgla::api_fail(SGLA_ERR_HIP, msg);
    }
    if (dev < 0 || dev >= kMaxDevices) return sgla::api_fail(SGLA_ERR_UNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            char msg[160];
            std::snprintf(msg, sizeof(msg), "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
            return sgla::api_fail(SGLA_ERR_HIP, msg);
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return SGLA_OK;
}

}  // namespace

extern "C" sgla_status sgla_chunk_bwd_noalloc(const void* q, const void* k, const void* v, const void* dO,
                                              const float* lambda, const float* a, const float* init_state,
                                              const float* d_final_state, void* dq, void* dk, void* dv,
                                              float* da, float* d_init_state, const int32_t* cu_seqlens,
                                              int n_seq, int B, int H, int T, int d_k, int d_v, int chunk,
                                              sgla_dtype dtype, void* hip_stream)
{
    // argument errors first, before any HIP call
    sgla::ChunkProblem p;
    const sgla_status pre = sgla::check_chunk_bwd(q, k, v, dO, lambda, a, init_state, d_final_state, dq, dk, dv,
                                                  da, d_init_state, cu_seqlens, n_seq, B, H, T, d_k, d_v, chunk,
                                                  dtype, &p);
    if (pre != SGLA_OK) return pre;
    const int N = (cu_seqlens != nullptr) ? n_seq : B;
    const size_t need = sgla_chunk_bwd_workspace_bytes(N, H, d_k);
    if (need > (size_t)SGLA_NOALLOC_SCRATCH_BYTES) {
        char msg[200];
        std::snprintf(msg, sizeof(msg),
                      "sgla_chunk_bwd_noalloc: %d sequences x %d heads x d_k %d need %zu bytes of scratch, "
                      "more than the fixed %d",
                      N, H, d_k, need, (int)SGLA_NOALLOC_SCRATCH_BYTES);
        return sgla::api_fail(SGLA_ERR_WORKSPACE, msg);
    }
    void* ws = nullptr;
    const sgla_status st = current_scratch(&ws);
    if (st != SGLA_OK) return st;
    return sgla_chunk_bwd(q, k, v, dO, lambda, a, init_state, d_final_state, dq, dk, dv, da, d_init_state,
                          cu_seqlens, n_seq, B, H, T, d_k, d_v, chunk, dtype, ws,
                          (size_t)SGLA_NOALLOC_SCRATCH_BYTES, hip_stream);
}
