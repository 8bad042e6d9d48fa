// Mixer epilogue for gfx950: Head RMSNorm per decay tier, concatenation of the
// heads and the SiLU(g) output gate.
//
// Method: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
// attention model on AWS Trainium2 with native PyTorch", section "i14 and the
// Laplace 3B architecture": the end of the "GLA mixer" paragraph (each head's
// output goes through a Head RMSNorm within its decay tier; the heads are
// concatenated and gated by SiLU(g_t)) and the "Decay schedule's reach"
// paragraph (the heads of a tier share one Head RMSNorm):
//
//   out[b,t,h,c] = silu(g[b,t,h,c]) * gamma[tier(h)][c] * o[b,h,t,c] / sqrt(mean_c' o[b,h,t,c']^2 + eps)
//   tier(h) = h / (H / n_tiers)
//
// o arrives in the mixer's head-major layout [B, H, T, d_v]; g and out are
// token-major [B, T, H, d_v] (heads concatenated), the layout of the gate
// stream and of the output projection's input.
//
// The operation is a stream (read o and g, write out; ~10 flops per element),
// so the kernel is built for HBM bandwidth. Sixteen lanes own one (b, h, t)
// row of d_v channels: lane j holds channels 64m + 4j .. 64m + 4j + 3 of
// chunk m, so each load or store instruction of a 16-lane group covers 64
// contiguous channels (one 128-byte line in bf16, two in fp32) of its row. A
// wave's four 16-lane groups take consecutive rows (consecutive tokens of one
// head, contiguous in o), four rows per group, and every load of those rows
// is issued before any is used; the sum of squares is reduced across the 16
// lanes with xor shuffles, in a fixed order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgla_internal.h"

namespace sgla {
namespace {

typedef unsigned short u16;
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NORM_THREADS = 256;  // four waves
constexpr int NORM_STEPS = 4;      // rows per 16-lane group

__device__ __forceinline__ float silu_g(float x)
{
    // x / (1 + e^-x); e^-x overflows to inf for very negative x, giving -0
    const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * x);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// 4 channels: 8 bytes of bf16 or 16 of fp32. The rows stream through once
// (every element is read and written by one lane, once), so loads and stores
// carry the non-temporal hint.
typedef unsigned int u32v2 __attribute__((ext_vector_type(2)));
template <typename E> struct Ch4;
template <> struct Ch4<u16> {
    typedef uint2 Raw;
    static __device__ __forceinline__ Raw load(const u16* p)
    {
        const u32v2 w = __builtin_nontemporal_load(reinterpret_cast<const u32v2*>(p));
        return uint2{w[0], w[1]};
    }
    static __device__ __forceinline__ Raw zero() { return uint2{0u, 0u}; }
    static __device__ __forceinline__ void unpack(Raw r, float* x)
    {
        x[0] = __uint_as_float(r.x << 16);
        x[1] = __uint_as_float(r.x & 0xffff0000u);
        x[2] = __uint_as_float(r.y << 16);
        x[3] = __uint_as_float(r.y & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(u16* p, const float* y)
    {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 lo = {static_cast<__bf16>(y[0]), static_cast<__bf16>(y[1])};
        const bf16x2 hi = {static_cast<__bf16>(y[2]), static_cast<__bf16>(y[3])};
        const u32v2 w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        __builtin_nontemporal_store(w, reinterpret_cast<u32v2*>(p));
    }
};
template <> struct Ch4<float> {
    typedef f32x4 Raw;
    static __device__ __forceinline__ Raw load(const float* p)
    {
        return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    }
    static __device__ __forceinline__ Raw zero() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
    static __device__ __forceinline__ void unpack(Raw r, float* x)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = r[i];
    }
    static __device__ __forceinline__ void store(float* p, const float* y)
    {
        __builtin_nontemporal_store(f32x4{y[0], y[1], y[2], y[3]}, reinterpret_cast<f32x4*>(p));
    }
};

// One row = one (b, h, t): 16 lanes, lane j holding channels 64m + 4j .. +3 of
// chunk m < NC (FULL: d_v = 64 NC, so no chunk is partial). A wave holds four
// rows at a time, one per 16-lane group; lane group q of wave w owns rows
// w * 4 STEPS + 4 s + q for s < STEPS. rows = B * H * T < 2^31.
template <typename E, int NC, bool FULL, bool GAMMA>
__global__ __launch_bounds__(NORM_THREADS) void k_head_norm_gate(const E* __restrict__ o, const E* g,
                                                                 const float* __restrict__ gamma, E* out,
                                                                 int rows, int H, int T, int d_v, int per_tier,
                                                                 float inv_dv, float eps)
{
    constexpr int S = NORM_STEPS;
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, j = lane & 15;
    const int wave = blockIdx.x * (NORM_THREADS / 64) + (threadIdx.x >> 6);

    // this lane's rows: offsets into o (head-major) and g / out (token-major)
    int oo[S], go[S], tier[S];
    bool live[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int r = wave * (4 * S) + 4 * s + q;
        live[s] = r < rows;
        const int rr = live[s] ? r : rows - 1;  // a dead row reads a valid one and stores nothing
        const int bh = rr / T;
        const int t = rr - bh * T;
        const int b = bh / H;
        const int h = bh - b * H;
        tier[s] = h / per_tier;
        oo[s] = rr * d_v;
        go[s] = ((b * T + t) * H + h) * d_v;
    }
    auto in_row = [&](int m) { return FULL || 64 * m + 4 * j < d_v; };

    // every load first
    typename Ch4<E>::Raw ro[S][NC], rg[S][NC];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int m = 0; m < NC; ++m) {
            const int c = 64 * m + 4 * j;
            if (in_row(m)) {
                ro[s][m] = Ch4<E>::load(o + (size_t)oo[s] + c);
                rg[s][m] = Ch4<E>::load(g + (size_t)go[s] + c);
            } else {
                ro[s][m] = Ch4<E>::zero();
                rg[s][m] = Ch4<E>::zero();
            }
        }

#pragma unroll
    for (int s = 0; s < S; ++s) {
        float x[NC][4];
        float ss = 0.0f;
#pragma unroll
        for (int m = 0; m < NC; ++m) {
            Ch4<E>::unpack(ro[s][m], x[m]);
#pragma unroll
            for (int i = 0; i < 4; ++i) ss = fmaf(x[m][i], x[m][i], ss);
        }
        // sum over the row's 16 lanes (xor within the 16-lane group, fixed order)
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
        const float inv = __builtin_amdgcn_rsqf(fmaf(ss, inv_dv, eps));
        if (!live[s]) continue;
#pragma unroll
        for (int m = 0; m < NC; ++m) {
            if (!in_row(m)) continue;
            const int c = 64 * m + 4 * j;
            f32x4 sc = {inv, inv, inv, inv};
            if (GAMMA) {
                const f32x4 gm = *reinterpret_cast<const f32x4*>(gamma + (size_t)tier[s] * d_v + c);
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[i] = gm[i] * inv;
            }
            float gv[4], y[4];
            Ch4<E>::unpack(rg[s][m], gv);
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = silu_g(gv[i]) * (sc[i] * x[m][i]);
            Ch4<E>::store(out + (size_t)go[s] + c, y);
        }
    }
}

template <typename E, int NC, bool FULL>
hipError_t run_norm(const void* o, const void* g, const float* gamma, void* out, int B, int H, int T, int d_v,
                    int n_tiers, float eps, hipStream_t stream)
{
    const int rows = B * H * T;
    const int rows_per_block = (NORM_THREADS / 64) * 4 * NORM_STEPS;
    const int blocks = (rows + rows_per_block - 1) / rows_per_block;
    const float inv_dv = 1.0f / (float)d_v;
    if (gamma != nullptr)
        hipLaunchKernelGGL((k_head_norm_gate<E, NC, FULL, true>), dim3(blocks), dim3(NORM_THREADS), 0, stream,
                           reinterpret_cast<const E*>(o), reinterpret_cast<const E*>(g), gamma,
                           reinterpret_cast<E*>(out), rows, H, T, d_v, H / n_tiers, inv_dv, eps);
    else
        hipLaunchKernelGGL((k_head_norm_gate<E, NC, FULL, false>), dim3(blocks), dim3(NORM_THREADS), 0, stream,
                           reinterpret_cast<const E*>(o), reinterpret_cast<const E*>(g), gamma,
                           reinterpret_cast<E*>(out), rows, H, T, d_v, H / n_tiers, inv_dv, eps);
    return hipGetLastError();
}

template <typename E>
hipError_t run_norm_dv(const void* o, const void* g, const float* gamma, void* out, int B, int H, int T, int d_v,
                       int n_tiers, float eps, hipStream_t stream)
{
    switch (d_v) {
    case 64: return run_norm<E, 1, true>(o, g, gamma, out, B, H, T, d_v, n_tiers, eps, stream);
    case 128: return run_norm<E, 2, true>(o, g, gamma, out, B, H, T, d_v, n_tiers, eps, stream);
    case 192: return run_norm<E, 3, true>(o, g, gamma, out, B, H, T, d_v, n_tiers, eps, stream);
    case 256: return run_norm<E, 4, true>(o, g, gamma, out, B, H, T, d_v, n_tiers, eps, stream);
    default: break;
    }
    switch ((d_v + 63) / 64) {
    case 1: return run_norm<E, 1, false>(o, g, gamma, out, B, H, T, d_v, n_tiers, eps, stream);
    case 2: return run_norm<E, 2, false>(o, g, gamma, out, B, H, T, d_v, n_tiers, eps, stream);
    case 3: return run_norm<E, 3, false>(o, g, gamma, out, B, H, T, d_v, n_tiers, eps, stream);
    default: return run_norm<E, 4, false>(o, g, gamma, out, B, H, T, d_v, n_tiers, eps, stream);
    }
}

// ---------------------------------------------------------------------------
// Gradients of the epilogue. Per (b, h, t) row, with r = sqrt(mean o^2 + eps),
// y = o / r, s = silu(g), gm = gamma[tier(h)] (one without gamma) and
// w = dout s gm:
//   dg     = dout gm y silu'(g),   silu'(x) = sigmoid(x) (1 + x (1 - sigmoid(x)))
//   d_o    = (w - y mean_c (w y)) / r
//   dgamma[tier] = sum over the tier's rows of dout s y
// A block takes 64 consecutive tokens of one (b, h) (so one tier): lane group
// q of wave w owns tokens 16 w + 4 s + q, 16 lanes per row as in the forward.
// Its dgamma contribution is summed over its 16 lane groups in a fixed order
// into part[(b H + h) nTB + tb][d_v]; k_dgamma_sum then adds the partials of
// each tier in a fixed order, so dgamma is bitwise reproducible.
constexpr int NB_TOK = 64;  // tokens per block

__device__ __forceinline__ float sigmoid_g(float x)
{
    // 1 / (1 + e^-x); e^-x -> inf for very negative x gives 0
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
}

template <typename E, int NC, bool FULL, bool GAMMA, bool DGAMMA>
__global__ __launch_bounds__(NORM_THREADS) void k_head_norm_gate_bwd(
    const E* __restrict__ o, const E* __restrict__ g, const float* __restrict__ gamma, const E* dout,
    E* __restrict__ d_o, E* dg, float* __restrict__ part, int H, int T, int d_v, int per_tier, float inv_dv,
    float eps)
{
    constexpr int S = NORM_STEPS;
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, j = lane & 15;
    const int w = threadIdx.x >> 6;
    const int tb = blockIdx.x, bh = blockIdx.y;
    const int b = bh / H, h = bh - b * H;
    const int tier = h / per_tier;
    auto in_row = [&](int m) { return FULL || 64 * m + 4 * j < d_v; };

    int oo[S], go[S];
    bool live[S];
#pragma unroll
    for (int s = 0; s < S; ++s) {
        const int t = tb * NB_TOK + 16 * w + 4 * s + q;
        live[s] = t < T;
        const int tt = live[s] ? t : T - 1;  // a dead row reads a valid one and stores nothing
        oo[s] = (bh * T + tt) * d_v;
        go[s] = ((b * T + tt) * H + h) * d_v;
    }
    float gm[NC][4];
#pragma unroll
    for (int m = 0; m < NC; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) gm[m][i] = 1.0f;
    if (GAMMA) {
#pragma unroll
        for (int m = 0; m < NC; ++m)
            if (in_row(m)) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(gamma + (size_t)tier * d_v + 64 * m + 4 * j);
#pragma unroll
                for (int i = 0; i < 4; ++i) gm[m][i] = x[i];
            }
    }

    // every load first
    typename Ch4<E>::Raw ro[S][NC], rg[S][NC], rd[S][NC];
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
        for (int m = 0; m < NC; ++m) {
            const int c = 64 * m + 4 * j;
            if (in_row(m)) {
                ro[s][m] = Ch4<E>::load(o + (size_t)oo[s] + c);
                rg[s][m] = Ch4<E>::load(g + (size_t)go[s] + c);
                rd[s][m] = Ch4<E>::load(dout + (size_t)go[s] + c);
            } else {
                ro[s][m] = Ch4<E>::zero();
                rg[s][m] = Ch4<E>::zero();
                rd[s][m] = Ch4<E>::zero();
            }
        }

    float acc[NC][4];
#pragma unroll
    for (int m = 0; m < NC; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[m][i] = 0.0f;

#pragma unroll
    for (int s = 0; s < S; ++s) {
        float x[NC][4], gv[NC][4], dv[NC][4];
        float ss = 0.0f;
#pragma unroll
        for (int m = 0; m < NC; ++m) {
            Ch4<E>::unpack(ro[s][m], x[m]);
            Ch4<E>::unpack(rg[s][m], gv[m]);
            Ch4<E>::unpack(rd[s][m], dv[m]);
#pragma unroll
            for (int i = 0; i < 4; ++i) ss = fmaf(x[m][i], x[m][i], ss);
        }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
        const float inv = __builtin_amdgcn_rsqf(fmaf(ss, inv_dv, eps));
        // y, silu and w; the row's sum of w y
        float y[NC][4], sg[NC][4], wv[NC][4];
        float p = 0.0f;
#pragma unroll
        for (int m = 0; m < NC; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                y[m][i] = x[m][i] * inv;
                sg[m][i] = sigmoid_g(gv[m][i]);
                wv[m][i] = dv[m][i] * (gv[m][i] * sg[m][i]) * gm[m][i];
                p = fmaf(wv[m][i], y[m][i], p);
            }
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) p += __shfl_xor(p, off);
        const float pm = p * inv_dv;
        if (!live[s]) continue;
#pragma unroll
        for (int m = 0; m < NC; ++m) {
            if (!in_row(m)) continue;
            const int c = 64 * m + 4 * j;
            float a[4], bgr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = inv * fmaf(-y[m][i], pm, wv[m][i]);
                bgr[i] = dv[m][i] * gm[m][i] * y[m][i] * sg[m][i] * fmaf(gv[m][i], 1.0f - sg[m][i], 1.0f);
                if (DGAMMA) acc[m][i] = fmaf(dv[m][i] * (gv[m][i] * sg[m][i]), y[m][i], acc[m][i]);
            }
            Ch4<E>::store(d_o + (size_t)oo[s] + c, a);
            Ch4<E>::store(dg + (size_t)go[s] + c, bgr);
        }
    }

    if (DGAMMA) {
        // the block's dgamma row: 16 lane groups (4 per wave) summed in order
        __shared__ float red[16][NC * 64];
        const int grp = 4 * w + q;
#pragma unroll
        for (int m = 0; m < NC; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[grp][64 * m + 4 * j + i] = acc[m][i];
        __syncthreads();
        const int nTB = gridDim.x;
        for (int c = threadIdx.x; c < d_v; c += NORM_THREADS) {
            float t = 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) t += red[k][c];
            part[((size_t)bh * nTB + tb) * d_v + c] = t;
        }
    }
}

constexpr int SUM_BATCH = 8;

// dgamma[tier][c] = sum over b, the tier's heads and the token blocks, in
// that fixed order split 64 ways: thread (k, c) of a block of 16 channels sums
// entries k, k + 64, ...; then the 64 sums are added in order.
__global__ __launch_bounds__(1024) void k_dgamma_sum(const float* __restrict__ part, float* __restrict__ dgamma,
                                                     int B, int H, int nTB, int d_v, int per_tier)
{
    __shared__ float red[64][16];
    const int tier = blockIdx.x;
    const int cl = threadIdx.x & 15, k = threadIdx.x >> 4;
    const int c = blockIdx.y * 16 + cl;
    const int n_ent = B * per_tier * nTB;
    float t = 0.0f;
    if (c < d_v) {
        // eight loads in flight, added in the same order as one at a time
        for (int e0 = k; e0 < n_ent; e0 += 64 * SUM_BATCH) {
            float x[SUM_BATCH];
#pragma unroll
            for (int i = 0; i < SUM_BATCH; ++i) {
                const int e = e0 + 64 * i;
                x[i] = 0.0f;
                if (e < n_ent) {
                    const int bb = e / (per_tier * nTB);
                    const int rem = e - bb * per_tier * nTB;
                    const int hh = tier * per_tier + rem / nTB;
                    const int tb = rem - (rem / nTB) * nTB;
                    x[i] = part[(((size_t)bb * H + hh) * nTB + tb) * d_v + c];
                }
            }
#pragma unroll
            for (int i = 0; i < SUM_BATCH; ++i)
                if (e0 + 64 * i < n_ent) t += x[i];
        }
    }
    red[k][cl] = t;
    __syncthreads();
    if (k == 0 && c < d_v) {
        float x = 0.0f;
        for (int i = 0; i < 64; ++i) x += red[i][cl];
        dgamma[(size_t)tier * d_v + c] = x;
    }
}

template <typename E, int NC, bool FULL, bool GAMMA>
hipError_t run_norm_bwd(const void* o, const void* g, const float* gamma, const void* dout, void* d_o,
                        void* dg, float* dgamma, float* part, int B, int H, int T, int d_v, int n_tiers,
                        float eps, hipStream_t stream)
{
    const int nTB = (T + NB_TOK - 1) / NB_TOK;
    const dim3 grid(nTB, B * H);
    const float inv_dv = 1.0f / (float)d_v;
    if (dgamma != nullptr) {
        hipLaunchKernelGGL((k_head_norm_gate_bwd<E, NC, FULL, GAMMA, true>), grid, dim3(NORM_THREADS), 0, stream,
                           reinterpret_cast<const E*>(o), reinterpret_cast<const E*>(g), gamma,
                           reinterpret_cast<const E*>(dout), reinterpret_cast<E*>(d_o), reinterpret_cast<E*>(dg),
                           part, H, T, d_v, H / n_tiers, inv_dv, eps);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_dgamma_sum, dim3(n_tiers, (d_v + 15) / 16), dim3(1024), 0, stream, part, dgamma, B, H,
                           nTB, d_v, H / n_tiers);
    } else {
        hipLaunchKernelGGL((k_head_norm_gate_bwd<E, NC, FULL, GAMMA, false>), grid, dim3(NORM_THREADS), 0, stream,
                           reinterpret_cast<const E*>(o), reinterpret_cast<const E*>(g), gamma,
                           reinterpret_cast<const E*>(dout), reinterpret_cast<E*>(d_o), reinterpret_cast<E*>(dg),
                           part, H, T, d_v, H / n_tiers, inv_dv, eps);
    }
    return hipGetLastError();
}

template <typename E, int NC, bool FULL>
hipError_t run_norm_bwd_g(const void* o, const void* g, const float* gamma, const void* dout, void* d_o, void* dg,
                          float* dgamma, float* part, int B, int H, int T, int d_v, int n_tiers, float eps,
                          hipStream_t stream)
{
    if (gamma != nullptr)
        return run_norm_bwd<E, NC, FULL, true>(o, g, gamma, dout, d_o, dg, dgamma, part, B, H, T, d_v, n_tiers,
                                               eps, stream);
    return run_norm_bwd<E, NC, FULL, false>(o, g, gamma, dout, d_o, dg, dgamma, part, B, H, T, d_v, n_tiers, eps,
                                            stream);
}

template <typename E>
hipError_t run_norm_bwd_dv(const void* o, const void* g, const float* gamma, const void* dout, void* d_o,
                           void* dg, float* dgamma, float* part, int B, int H, int T, int d_v, int n_tiers,
                           float eps, hipStream_t stream)
{
#define SGLA_NB(NC, FULL) \
    return run_norm_bwd_g<E, NC, FULL>(o, g, gamma, dout, d_o, dg, dgamma, part, B, H, T, d_v, n_tiers, eps, stream)
    switch (d_v) {
    case 64: SGLA_NB(1, true);
    case 128: SGLA_NB(2, true);
    case 192: SGLA_NB(3, true);
    case 256: SGLA_NB(4, true);
    default: break;
    }
    switch ((d_v + 63) / 64) {
    case 1: SGLA_NB(1, false);
    case 2: SGLA_NB(2, false);
    case 3: SGLA_NB(3, false);
    default: SGLA_NB(4, false);
    }
#undef SGLA_NB
}

}  // namespace

size_t head_norm_gate_bwd_part_floats(int B, int H, int T, int d_v)
{
    return (size_t)B * H * ((T + NB_TOK - 1) / NB_TOK) * d_v;
}

hipError_t launch_head_norm_gate_bwd(int bf16, const void* o, const void* g, const float* gamma, const void* dout,
                                     void* d_o, void* dg, float* dgamma, float* part, int B, int H, int T, int d_v,
                                     int n_tiers, float eps, hipStream_t stream)
{
    if (bf16)
        return run_norm_bwd_dv<u16>(o, g, gamma, dout, d_o, dg, dgamma, part, B, H, T, d_v, n_tiers, eps, stream);
    return run_norm_bwd_dv<float>(o, g, gamma, dout, d_o, dg, dgamma, part, B, H, T, d_v, n_tiers, eps, stream);
}

hipError_t launch_head_norm_gate(int bf16, const void* o, const void* g, const float* gamma, void* out, int B,
                                 int H, int T, int d_v, int n_tiers, float eps, hipStream_t stream)
{
    if (bf16) return run_norm_dv<u16>(o, g, gamma, out, B, H, T, d_v, n_tiers, eps, stream);
    return run_norm_dv<float>(o, g, gamma, out, B, H, T, d_v, n_tiers, eps, stream);
}

}  // namespace sgla
