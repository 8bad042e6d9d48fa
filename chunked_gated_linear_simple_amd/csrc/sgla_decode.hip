// Single-token Simple GLA decode for gfx950.
//
// Method: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
// attention model on AWS Trainium2 with native PyTorch", section "Inference
// optimization on Trainium2" (constant per-sequence recurrent state kept in a
// pool page, read and written once per generated token), with the recurrence
// of section "i14 and the Laplace 3B architecture", paragraph "GLA mixer":
//   S <- lam S + k v^T ;  o = S^T q + sigmoid(sum_i a_i q_i k_i) v
//
// The step is a pure streaming read-modify-write of the fp32 state (d_k*d_v*4
// bytes in and out per sequence-head, 0.5 flop/byte), so the kernel is built
// for HBM bandwidth: one workgroup per (sequence, head); thread (rg, cg) owns
// four adjacent state columns (one 16-byte vector) in rows rg, rg+RG, ... (12
// row groups of 8 rows for a 96 x 192 state, 576 threads; other head widths
// run in the thread layout of the next larger width, the unused rows and
// column groups masked); all
// of its state loads are issued before any use; loads and stores are
// non-temporal (the pool is far larger than the caches and is not re-read
// within a step); the readout reduction over rows is per-thread partial sums
// then one fixed-order pass through LDS. Nothing is shared between units, so
// each sequence's result is independent of N and of its position.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgla_internal.h"

namespace sgla {
namespace {

typedef unsigned short u16;
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ld_f(const u16* p, size_t i) { return __uint_as_float((uint32_t)p[i] << 16); }
__device__ __forceinline__ float ld_f(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ void st_f(u16* p, size_t i, float x)
{
    p[i] = __builtin_bit_cast(u16, static_cast<__bf16>(x));
}
__device__ __forceinline__ void st_f(float* p, size_t i, float x) { p[i] = x; }

__device__ __forceinline__ float sigmoid_dec(float z)
{
    if (z >= 0.0f) return 1.0f / (1.0f + expf(-z));
    float e = expf(z);
    return e / (1.0f + e);
}

// A dk x dv state per unit, dk <= DK and dv <= DV (EXACT: equal); CG = DV/4
// column groups; RG row groups. Column groups at or past dv / 4 and rows at or
// past dk do nothing.
template <typename E, int DK, int DV, int RG, bool EXACT>
__global__ __launch_bounds__((DV / 4) * RG) void k_decode(const E* __restrict__ q, const E* __restrict__ k,
                                                           const E* __restrict__ v,
                                                           const float* __restrict__ lambda,
                                                           const float* __restrict__ a,
                                                           float* __restrict__ state,
                                                           const int32_t* __restrict__ slot,
                                                           E* __restrict__ o, int N, int P, int H, int dk_rt,
                                                           int dv_rt)
{
    constexpr int CG = DV / 4;
    constexpr int NT = CG * RG;
    constexpr int RPT = (DK + RG - 1) / RG;  // rows per thread
    static_assert(DV % 4 == 0, "DV");
    const int dk = EXACT ? DK : dk_rt;
    const int dv = EXACT ? DV : dv_rt;
    const int cgn = EXACT ? CG : dv / 4;       // column groups in use (dv is a multiple of 4)

    __shared__ float qs[DK], ks[DK];
    __shared__ float zsh;
    __shared__ f32x4 red[RG][CG];

    const int unit = blockIdx.x;  // n * H + h
    const int n = unit / H, h = unit - (unit / H) * H;
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    const bool col = EXACT || cg < cgn;

    int page = (slot != nullptr) ? slot[n] : n;
    const bool valid = page >= 0 && page < P;

    const size_t qk_base = (size_t)unit * dk;
    const size_t v_base = (size_t)unit * dv;
    if (!valid) {
        for (int c = tid; c < dv; c += NT) st_f(o, v_base + c, __builtin_nanf(""));
        return;
    }
    f32x4* S = reinterpret_cast<f32x4*>(state + ((size_t)page * H + h) * (size_t)dk * dv);

    // issue the state loads first (the bandwidth-critical part)
    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int d = rg + RG * m;
        if (d < dk && col) s[m] = __builtin_nontemporal_load(&S[(size_t)d * cgn + cg]);
    }

    for (int d = tid; d < dk; d += NT) {
        qs[d] = ld_f(q, qk_base + d);
        ks[d] = ld_f(k, qk_base + d);
    }
    __syncthreads();
    if (tid < 64) {
        float z = 0.0f;
        if (a != nullptr)
            for (int d = tid; d < dk; d += 64) z += a[(size_t)h * dk + d] * qs[d] * ks[d];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
        if (tid == 0) zsh = z;
    }

    const float lam = lambda[h];
    f32x4 vv = {0.f, 0.f, 0.f, 0.f};
    if (col) {
        vv.x = ld_f(v, v_base + 4 * cg + 0);
        vv.y = ld_f(v, v_base + 4 * cg + 1);
        vv.z = ld_f(v, v_base + 4 * cg + 2);
        vv.w = ld_f(v, v_base + 4 * cg + 3);
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int d = rg + RG * m;
        if (d < dk && col) {
            const float kd = ks[d], qd = qs[d];
            f32x4 x = s[m];
            x.x = lam * x.x + kd * vv.x;
            x.y = lam * x.y + kd * vv.y;
            x.z = lam * x.z + kd * vv.z;
            x.w = lam * x.w + kd * vv.w;
            __builtin_nontemporal_store(x, &S[(size_t)d * cgn + cg]);
            acc.x += x.x * qd;
            acc.y += x.y * qd;
            acc.z += x.z * qd;
            acc.w += x.w * qd;
        }
    }
    red[rg][cg] = acc;
    __syncthreads();
    if (rg == 0 && col) {
        f32x4 r = red[0][cg];
#pragma unroll
        for (int j = 1; j < RG; ++j) {
            const f32x4 t = red[j][cg];
            r.x += t.x;
            r.y += t.y;
            r.z += t.z;
            r.w += t.w;
        }
        const float gte = sigmoid_dec(zsh);
        st_f(o, v_base + 4 * cg + 0, r.x + gte * vv.x);
        st_f(o, v_base + 4 * cg + 1, r.y + gte * vv.y);
        st_f(o, v_base + 4 * cg + 2, r.z + gte * vv.z);
        st_f(o, v_base + 4 * cg + 3, r.w + gte * vv.w);
    }
}

template <typename E, int DK, int DV, int RG, bool EXACT>
hipError_t run_decode(const void* q, const void* k, const void* v, const float* lambda,
                      const float* a, float* state, const int32_t* slot, void* o, int N, int P,
                      int H, int d_k, int d_v, hipStream_t stream)
{
    const int units = N * H;
    hipLaunchKernelGGL((k_decode<E, DK, DV, RG, EXACT>), dim3(units), dim3((DV / 4) * RG), 0, stream,
                       reinterpret_cast<const E*>(q), reinterpret_cast<const E*>(k),
                       reinterpret_cast<const E*>(v), lambda, a, state, slot,
                       reinterpret_cast<E*>(o), N, P, H, d_k, d_v);
    return hipGetLastError();
}

// Other widths: the thread layout of the next larger width, eight rows a row group.
template <typename E, int DK>
hipError_t run_decode_dk(const void* q, const void* k, const void* v, const float* lambda, const float* a,
                         float* state, const int32_t* slot, void* o, int N, int P, int H, int d_k, int d_v,
                         hipStream_t stream)
{
    if (d_v <= 64)
        return run_decode<E, DK, 64, DK / 8, false>(q, k, v, lambda, a, state, slot, o, N, P, H, d_k, d_v, stream);
    if (d_v <= 128)
        return run_decode<E, DK, 128, DK / 8, false>(q, k, v, lambda, a, state, slot, o, N, P, H, d_k, d_v, stream);
    return run_decode<E, DK, 192, DK / 8, false>(q, k, v, lambda, a, state, slot, o, N, P, H, d_k, d_v, stream);
}

template <typename E>
hipError_t run_decode_any(const void* q, const void* k, const void* v, const float* lambda, const float* a,
                          float* state, const int32_t* slot, void* o, int N, int P, int H, int d_k, int d_v,
                          hipStream_t stream)
{
    if (d_k == 96 && d_v == 192)
        return run_decode<E, 96, 192, 12, true>(q, k, v, lambda, a, state, slot, o, N, P, H, d_k, d_v, stream);
    if (d_k == 16 && d_v == 32)
        return run_decode<E, 16, 32, 8, true>(q, k, v, lambda, a, state, slot, o, N, P, H, d_k, d_v, stream);
    if (d_k <= 32) return run_decode_dk<E, 32>(q, k, v, lambda, a, state, slot, o, N, P, H, d_k, d_v, stream);
    if (d_k <= 64) return run_decode_dk<E, 64>(q, k, v, lambda, a, state, slot, o, N, P, H, d_k, d_v, stream);
    return run_decode_dk<E, 96>(q, k, v, lambda, a, state, slot, o, N, P, H, d_k, d_v, stream);
}

}  // namespace

hipError_t launch_decode_step(int bf16, const void* q, const void* k, const void* v,
                              const float* lambda, const float* a, float* state,
                              const int32_t* slot, void* o, int N, int P, int H, int d_k, int d_v,
                              hipStream_t stream)
{
    // 4 <= d_k <= 96 and 4 <= d_v <= 192, multiples of 4 (checked by the caller)
    if (bf16) return run_decode_any<u16>(q, k, v, lambda, a, state, slot, o, N, P, H, d_k, d_v, stream);
    return run_decode_any<float>(q, k, v, lambda, a, state, slot, o, N, P, H, d_k, d_v, stream);
}

}  // namespace sgla
