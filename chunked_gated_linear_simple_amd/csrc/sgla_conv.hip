// Convolution prologue of the mixer for gfx950: depthwise causal Conv1d of
// width 4 with SiLU, over whole sequences and as a decode step on a pool of
// per-sequence conv states.
//
// Method: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
// attention model on AWS Trainium2 with native PyTorch", section "i14 and the
// Laplace 3B architecture" (normalisation-and-convolution paragraph; the
// architecture table's Conv row): each channel c of token t is
//
//   y_t[c] = silu(b[c] + sum_{j=0..3} w[c][j] u_{t-3+j}[c]),   silu(x) = x sigmoid(x)
//
// with the three inputs before a sequence taken from its conv state (or zero),
// and section "Inference optimization on Trainium2" ("Constant serving
// state") for the state that a generated token reads and shifts.
//
// The operation is a pure stream (one read and one write of each activation,
// 4 multiply-adds and a SiLU per element), so the kernels are built for HBM
// bandwidth.
// Forward: a thread owns one 16-byte group of channels (8 bf16 or 4 fp32) and
// walks a run of 64 consecutive tokens, keeping the three previous inputs in
// registers, so every input is read once (plus a three-token halo per run).
// The run is software-pipelined in blocks of 8 rows: the next block's loads
// are issued before the current block is computed and stored, so a wave keeps
// 8-16 row loads in flight while it writes. (Issuing all of a run's loads up
// front instead makes every wave load, then store, in lock step, and is
// slower.) Consecutive threads own consecutive channel groups, so each token
// row is read and written as contiguous 1 KB wave accesses. A run that crosses
// a sequence boundary or the end of the rows takes a row-at-a-time path.
// Decode: a thread owns 4 channels of 4 sequences; its tap weights are loaded
// once for the 4, and all 4 sequences' state and input loads are issued before
// any is used.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgla_internal.h"

namespace sgla {
namespace {

typedef unsigned short u16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int CONV_RUN = 64;      // tokens per thread in the forward
constexpr int CONV_PD = 8;        // rows per pipelined block
constexpr int CONV_THREADS = 128; // forward workgroup
constexpr int DEC_SEQ = 4;        // sequences per decode thread
constexpr int DEC_THREADS = 256;  // decode workgroup

__device__ __forceinline__ float silu_f(float x)
{
    // x / (1 + e^-x); e^-x overflows to inf for very negative x, giving -0
    const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * x);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// A channel group: 8 bf16 or 4 fp32 values in 16 bytes. The forward's rows
// stream through once (a run's three-row halo was read a whole run earlier
// and is gone from the caches either way), so its loads and stores carry the
// non-temporal hint.
template <typename E> struct Grp;
template <> struct Grp<u16> {
    static constexpr int V = 8;
    static __device__ __forceinline__ void unpack(u32x4 w, float* x)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    static __device__ __forceinline__ void load(const u16* p, float* x)
    {
        unpack(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)), x);
    }
    static __device__ __forceinline__ void store(u16* p, const float* y)
    {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x2 v = {static_cast<__bf16>(y[2 * i]), static_cast<__bf16>(y[2 * i + 1])};
            w[i] = __builtin_bit_cast(uint32_t, v);
        }
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p));
    }
};
template <> struct Grp<float> {
    static constexpr int V = 4;
    static __device__ __forceinline__ void unpack(u32x4 w, float* x)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(w[i]);
    }
    static __device__ __forceinline__ void load(const float* p, float* x)
    {
        unpack(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)), x);
    }
    static __device__ __forceinline__ void store(float* p, const float* y)
    {
        const f32x4 v = {y[0], y[1], y[2], y[3]};
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
    }
};

struct Seqs {
    const int32_t* cu;  // NULL when dense
    int n_seq, T, S;    // S = total token rows
    // token range of sequence n, clamped to [0, S]
    __device__ __forceinline__ void range(int n, int& s0, int& s1) const
    {
        if (cu == nullptr) {
            s0 = n * T;
            s1 = s0 + T;
        } else {
            s0 = min(max(cu[n], 0), S);
            s1 = min(max(cu[n + 1], s0), S);
        }
    }
    // the sequence holding row t (the last n with start <= t)
    __device__ __forceinline__ int find(int t) const
    {
        if (cu == nullptr) return t / T;
        int lo = 0, hi = n_seq - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (min(max(cu[mid], 0), S) <= t) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    }
};

// fin[n] = the last three inputs of sequence n (reaching into init), for the
// channel group grp
template <typename E>
__device__ __forceinline__ void final_state(const E* __restrict__ u, const float* init, float* fin, const Seqs& sq,
                                            int D, int n, int grp)
{
    constexpr int V = Grp<E>::V;
    const int c0 = grp * V;
    int s0, s1;
    sq.range(n, s0, s1);
    const int L = s1 - s0;
    float h[3][V];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int p = L - 3 + j;
        if (p >= 0) {
            Grp<E>::load(u + (size_t)(s0 + p) * D + c0, h[j]);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i)
                h[j][i] = (init != nullptr) ? init[((size_t)n * 3 + (3 + p)) * D + c0 + i] : 0.0f;
        }
    }
    // all reads above happen before any write: fin may equal init
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int i = 0; i < V; ++i) fin[((size_t)n * 3 + j) * D + c0 + i] = h[j][i];
}

// the final states alone, after every read of init (fin may equal init)
template <typename E>
__global__ __launch_bounds__(CONV_THREADS) void k_conv_state(const E* __restrict__ u, const float* init,
                                                             float* fin, Seqs sq, int D)
{
    const int grp = blockIdx.y * CONV_THREADS + threadIdx.x;
    if (grp * Grp<E>::V >= D) return;
    final_state<E>(u, init, fin, sq, D, blockIdx.x, grp);
}

// y for rows [RUN * blockIdx.x, ...) of channel group blockIdx.y * CONV_THREADS + tid;
// blocks runs + n (when fin is given, which then overlaps no input) write
// sequence n's final state

template <typename E, int RUN, int PD>
__global__ __launch_bounds__(CONV_THREADS) void k_conv_fwd(const E* __restrict__ u, const float* __restrict__ w,
                                                           const float* __restrict__ b,
                                                           const float* __restrict__ init, E* __restrict__ y,
                                                           float* __restrict__ fin, Seqs sq, int D, int runs)
{
    static_assert(RUN % (2 * PD) == 0, "a run is an even number of blocks");
    constexpr int V = Grp<E>::V;
    const int grp = blockIdx.y * CONV_THREADS + threadIdx.x;
    if (grp * V >= D) return;
    if ((int)blockIdx.x >= runs) {
        final_state<E>(u, init, fin, sq, D, blockIdx.x - runs, grp);
        return;
    }
    const int c0 = grp * V;
    const int t0 = blockIdx.x * RUN;
    if (t0 >= sq.S) return;
    const int t1 = min(t0 + RUN, sq.S);

    float wt[V][4], bias[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const f32x4 wv = *reinterpret_cast<const f32x4*>(w + (size_t)(c0 + i) * 4);
        wt[i][0] = wv[0];
        wt[i][1] = wv[1];
        wt[i][2] = wv[2];
        wt[i][3] = wv[3];
        bias[i] = (b != nullptr) ? b[c0 + i] : 0.0f;
    }

    int n = sq.find(t0), s0, s1;
    sq.range(n, s0, s1);
    // h[j] = u_{t-3+j} for the next token t
    float h[3][V];
    auto history = [&](int t) {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int p = t - 3 + j;
            if (p >= s0) {
                Grp<E>::load(u + (size_t)p * D + c0, h[j]);
            } else if (init != nullptr) {
                const f32x4* sp = reinterpret_cast<const f32x4*>(init + ((size_t)n * 3 + (3 + p - s0)) * D + c0);
#pragma unroll
                for (int i = 0; i < V; i += 4) {
                    const f32x4 v = sp[i / 4];
                    h[j][i] = v[0];
                    h[j][i + 1] = v[1];
                    h[j][i + 2] = v[2];
                    h[j][i + 3] = v[3];
                }
            } else {
#pragma unroll
                for (int i = 0; i < V; ++i) h[j][i] = 0.0f;
            }
        }
    };
    // one token: y_t from x = u_t and the history, which then shifts
    auto token = [&](const float* x, int t) {
        float out[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            float acc = bias[i];
            acc = fmaf(wt[i][0], h[0][i], acc);
            acc = fmaf(wt[i][1], h[1][i], acc);
            acc = fmaf(wt[i][2], h[2][i], acc);
            acc = fmaf(wt[i][3], x[i], acc);
            out[i] = silu_f(acc);
            h[0][i] = h[1][i];
            h[1][i] = h[2][i];
            h[2][i] = x[i];
        }
        Grp<E>::store(y + (size_t)t * D + c0, out);
    };
    // rows before the first sequence's start belong to none (only a malformed
    // cu_seqlens has them); history(t) needs t >= s0
    const int ts = max(t0, s0);
    history(ts);

    if (t1 - t0 == RUN && t0 >= s0 && t1 <= s1) {
        // the whole run lies in one sequence: pipelined blocks of PD rows
        const u32x4* up = reinterpret_cast<const u32x4*>(u + (size_t)t0 * D + c0);
        const size_t rs = (size_t)D / V;  // one row in 16-byte units
        u32x4 bufA[PD], bufB[PD];
        auto block = [&](const u32x4* buf, int tb) {
#pragma unroll
            for (int r = 0; r < PD; ++r) {
                float x[V];
                Grp<E>::unpack(buf[r], x);
                token(x, tb + r);
            }
        };
#pragma unroll
        for (int r = 0; r < PD; ++r) bufA[r] = up[r * rs];
#pragma unroll 1
        for (int k = 0; k < RUN / PD; k += 2) {
#pragma unroll
            for (int r = 0; r < PD; ++r) bufB[r] = up[((size_t)(k + 1) * PD + r) * rs];
            block(bufA, t0 + k * PD);
            if (k + 2 < RUN / PD) {
#pragma unroll
                for (int r = 0; r < PD; ++r) bufA[r] = up[((size_t)(k + 2) * PD + r) * rs];
            }
            block(bufB, t0 + (k + 1) * PD);
        }
        return;
    }

    // general path, one row at a time
#pragma unroll 1
    for (int t = ts; t < t1; ++t) {
        if (t >= s1) {
            // next non-empty sequence: its history is its own conv state
            while (t >= s1 && n + 1 < sq.n_seq) {
                ++n;
                sq.range(n, s0, s1);
            }
            if (t >= s1) break;  // rows past the last sequence belong to none
            history(t);
        }
        float x[V];
        Grp<E>::load(u + (size_t)t * D + c0, x);
        token(x, t);
    }
}

// 4 channels of one token row: 8 bytes of bf16 or 16 of fp32
template <typename E> struct Quad;
template <> struct Quad<u16> {
    typedef uint2 Raw;
    static __device__ __forceinline__ Raw load(const u16* p) { return *reinterpret_cast<const uint2*>(p); }
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
        *reinterpret_cast<uint2*>(p) = uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    }
    static __device__ __forceinline__ void store_nan(u16* p) { *reinterpret_cast<uint2*>(p) = uint2{0x7fc07fc0u, 0x7fc07fc0u}; }
};
template <> struct Quad<float> {
    typedef f32x4 Raw;
    static __device__ __forceinline__ Raw load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    static __device__ __forceinline__ void unpack(Raw r, float* x)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = r[i];
    }
    static __device__ __forceinline__ void store(float* p, const float* y)
    {
        *reinterpret_cast<f32x4*>(p) = f32x4{y[0], y[1], y[2], y[3]};
    }
    static __device__ __forceinline__ void store_nan(float* p)
    {
        const float q = __builtin_nanf("");
        *reinterpret_cast<f32x4*>(p) = f32x4{q, q, q, q};
    }
};

// one decode step: thread = (channels 4g..4g+3, sequences SEQ*blockIdx.x + m)
template <typename E, int SEQ>
__global__ __launch_bounds__(DEC_THREADS) void k_conv_decode(const E* __restrict__ x, const float* __restrict__ w,
                                                             const float* __restrict__ b, float* __restrict__ state,
                                                             const int32_t* __restrict__ slot, E* __restrict__ y,
                                                             int N, int P, int D)
{
    const int grp = blockIdx.y * DEC_THREADS + threadIdx.x;
    if (grp * 4 >= D) return;
    const int c0 = grp * 4;
    const int n0 = blockIdx.x * SEQ;
    const size_t rs = D / 4;  // one state row in f32x4 units

    // every load of the SEQ sequences first
    int page[SEQ];
    f32x4 s[SEQ][3];
    typename Quad<E>::Raw xr[SEQ];
#pragma unroll
    for (int m = 0; m < SEQ; ++m) {
        const int n = n0 + m;
        page[m] = -1;
        if (n < N) {
            const int pg = (slot != nullptr) ? slot[n] : n;
            if (pg >= 0 && pg < P) {
                page[m] = pg;
                const f32x4* st = reinterpret_cast<const f32x4*>(state + (size_t)pg * 3 * D + c0);
                s[m][0] = st[0];
                s[m][1] = st[rs];
                s[m][2] = st[2 * rs];
                xr[m] = Quad<E>::load(x + (size_t)n * D + c0);
            }
        }
    }
    f32x4 wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[i] = *reinterpret_cast<const f32x4*>(w + (size_t)(c0 + i) * 4);
    const f32x4 bv = (b != nullptr) ? *reinterpret_cast<const f32x4*>(b + c0) : f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int m = 0; m < SEQ; ++m) {
        const int n = n0 + m;
        if (n >= N) break;
        E* yr = y + (size_t)n * D + c0;
        if (page[m] < 0) {
            Quad<E>::store_nan(yr);
            continue;
        }
        float xv[4], out[4];
        Quad<E>::unpack(xr[m], xv);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float acc = bv[i];
            acc = fmaf(wv[i][0], s[m][0][i], acc);
            acc = fmaf(wv[i][1], s[m][1][i], acc);
            acc = fmaf(wv[i][2], s[m][2][i], acc);
            acc = fmaf(wv[i][3], xv[i], acc);
            out[i] = silu_f(acc);
        }
        f32x4* st = reinterpret_cast<f32x4*>(state + (size_t)page[m] * 3 * D + c0);
        st[0] = s[m][1];
        st[rs] = s[m][2];
        st[2 * rs] = f32x4{xv[0], xv[1], xv[2], xv[3]};
        Quad<E>::store(yr, out);
    }
}

template <typename E>
hipError_t run_conv_fwd(const void* u, const float* w, const float* b, const float* init, float* fin,
                        void* y, const int32_t* cu, int n_seq, int B, int T, int D, hipStream_t stream)
{
    constexpr int V = Grp<E>::V;
    Seqs sq{cu, n_seq, T, cu != nullptr ? T : B * T};
    const int groups = D / V;
    const int gy = (groups + CONV_THREADS - 1) / CONV_THREADS;
    const int runs = (sq.S + CONV_RUN - 1) / CONV_RUN;
    // a final state that is not the initial one (the caller guarantees it then
    // overlaps no input) is written by extra blocks of the same launch
    const bool fused = fin != nullptr && fin != init;
    hipLaunchKernelGGL((k_conv_fwd<E, CONV_RUN, CONV_PD>), dim3(runs + (fused ? n_seq : 0), gy), dim3(CONV_THREADS), 0,
                       stream, reinterpret_cast<const E*>(u), w, b, init, reinterpret_cast<E*>(y),
                       fused ? fin : nullptr, sq, D, runs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (fin != nullptr && !fused) {
        const dim3 g2(n_seq, gy);
        hipLaunchKernelGGL(k_conv_state<E>, g2, dim3(CONV_THREADS), 0, stream, reinterpret_cast<const E*>(u), init,
                           fin, sq, D);
        return hipGetLastError();
    }
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Gradients. Per sequence and channel, with x_s = u_s (s >= 0) or the initial
// state's row 3 + s, pre_t = b + sum_j w_j x_{t-3+j} and y_t = silu(pre_t):
//   dpre_t = dy_t silu'(pre_t),   silu'(x) = sigmoid(x) (1 + x (1 - sigmoid(x)))
//   du_s   = w_3 dpre_s + w_2 dpre_{s+1} + w_1 dpre_{s+2} + w_0 dpre_{s+3}
//            (dpre = 0 past the sequence) + d_final[s - (L - 3)] for s >= L - 3
//   dw_j   = sum_t dpre_t x_{t-3+j},  db = sum_t dpre_t
// k_conv_bwd: a thread owns two channels and a run of BWD_RUN rows; for
// each sequence meeting the run it walks tau from max(run start, sequence
// start) to three rows past the run's end (within the sequence), computing
// dpre_tau and, three rows behind, du. dw and db of the run's rows go to
// part[run][5][D]. Extra blocks of the same launch write the initial states'
// gradient (also for empty sequences), and k_conv_wsum adds the run partials
// in a fixed order.
constexpr int BWD_RUN = 64;
constexpr int BWD_THREADS = 128;
constexpr int BWD_PF = 4;  // rows of u and dy in flight per thread

// Two channels per access for the backward (4 bytes of bf16, 8 of fp32): a
// thread's windows, weights and partial sums then fit seven waves per SIMD.
// Its stores carry the non-temporal hint; its loads keep the default policy
// (the rows around a run's ends are read again, and the prefetch past the
// last row repeats it).
template <typename E> struct Q2;
template <> struct Q2<u16> {
    static constexpr int V = 2;
    typedef uint32_t Raw;
    static __device__ __forceinline__ Raw ld(const u16* p) { return *reinterpret_cast<const uint32_t*>(p); }
    static __device__ __forceinline__ Raw zero() { return 0u; }
    static __device__ __forceinline__ void unpack(Raw r, float* x)
    {
        x[0] = __uint_as_float(r << 16);
        x[1] = __uint_as_float(r & 0xffff0000u);
    }
    static __device__ __forceinline__ void store(u16* p, const float* y)
    {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 lo = {static_cast<__bf16>(y[0]), static_cast<__bf16>(y[1])};
        __builtin_nontemporal_store(__builtin_bit_cast(uint32_t, lo), reinterpret_cast<uint32_t*>(p));
    }
};
template <> struct Q2<float> {
    static constexpr int V = 2;
    typedef uint2 Raw;
    static __device__ __forceinline__ Raw ld(const float* p) { return *reinterpret_cast<const uint2*>(p); }
    static __device__ __forceinline__ Raw zero() { return uint2{0u, 0u}; }
    static __device__ __forceinline__ void unpack(Raw r, float* x)
    {
        x[0] = __uint_as_float(r.x);
        x[1] = __uint_as_float(r.y);
    }
    static __device__ __forceinline__ void store(float* p, const float* y)
    {
        typedef unsigned int u32v2 __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(u32v2{__float_as_uint(y[0]), __float_as_uint(y[1])}, reinterpret_cast<u32v2*>(p));
    }
};

__device__ __forceinline__ float ld_elem(const u16* p, size_t i) { return __uint_as_float((uint32_t)p[i] << 16); }
__device__ __forceinline__ float ld_elem(const float* p, size_t i) { return p[i]; }

__device__ __forceinline__ float dsilu_f(float x)
{
    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * x));
    return sg * fmaf(x, 1.0f - sg, 1.0f);
}

// The initial state's gradient of sequence n: d_init[i] = sum_{j <= i} w_j
// dpre_{i-j} (rows inside the sequence) + d_final[i - L] when the final state
// reaches back into the initial state (L < 3). One thread per channel; block
// idx takes sequence idx / ceil(D / BWD_THREADS) and the channel block after.
template <typename E>
__device__ __forceinline__ void conv_bwd_init_block(const E* __restrict__ u, const E* __restrict__ dy,
                                                    const float* __restrict__ w, const float* __restrict__ b,
                                                    const float* __restrict__ init,
                                                    const float* __restrict__ dfin, float* __restrict__ dinit,
                                                    const Seqs& sq, int D, int idx)
{
    const int iblk = (D + BWD_THREADS - 1) / BWD_THREADS;
    const int n = idx / iblk;
    const int c = (idx - n * iblk) * BWD_THREADS + threadIdx.x;
    if (c >= D) return;
    int s0, s1;
    sq.range(n, s0, s1);
    const int L = s1 - s0;
    const f32x4 wv = *reinterpret_cast<const f32x4*>(w + (size_t)c * 4);
    const float bc = (b != nullptr) ? b[c] : 0.0f;
    // x_{-3..2} of this channel and dpre_{0..2}
    float x[6], p[3];
    for (int i = 0; i < 3; ++i) x[i] = (init != nullptr) ? init[((size_t)n * 3 + i) * D + c] : 0.0f;
    for (int t = 0; t < 3; ++t) {
        float xu = 0.0f, g = 0.0f;
        if (t < L) {
            xu = ld_elem(u, (size_t)(s0 + t) * D + c);
            g = ld_elem(dy, (size_t)(s0 + t) * D + c);
        }
        x[3 + t] = xu;
        const float pre = bc + wv[0] * x[t] + wv[1] * x[t + 1] + wv[2] * x[t + 2] + wv[3] * xu;
        p[t] = (t < L) ? g * dsilu_f(pre) : 0.0f;
    }
    for (int i = 0; i < 3; ++i) {
        float acc = 0.0f;
        for (int j = 0; j <= i; ++j) acc += wv[j] * p[i - j];
        if (dfin != nullptr && i - L >= 0) acc += dfin[((size_t)n * 3 + (i - L)) * D + c];
        dinit[((size_t)n * 3 + i) * D + c] = acc;
    }
}

template <typename E>
__global__ __launch_bounds__(BWD_THREADS) void k_conv_bwd(const E* __restrict__ u, const E* __restrict__ dy,
                                                          const float* __restrict__ w, const float* __restrict__ b,
                                                          const float* __restrict__ init,
                                                          const float* __restrict__ dfin, E* __restrict__ du,
                                                          float* __restrict__ part, float* __restrict__ dinit,
                                                          Seqs sq, int D, int nblk, int n_main)
{
    // blocks past the runs' ones write the initial states' gradient
    if ((int)blockIdx.x >= n_main) {
        conv_bwd_init_block<E>(u, dy, w, b, init, dfin, dinit, sq, D, (int)blockIdx.x - n_main);
        return;
    }
    typedef Q2<E> G;
    constexpr int V = G::V;
    // the channel blocks of one run are consecutive blocks, so the rows they
    // share are read from HBM at about the same time
    const int run = blockIdx.x / nblk;
    const int grp = (blockIdx.x - run * nblk) * BWD_THREADS + threadIdx.x;
    if (grp * V >= D) return;
    const int c0 = grp * V;
    const int r0 = run * BWD_RUN, r1 = min(r0 + BWD_RUN, sq.S);

    float wt[V][4], bias[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(w + (size_t)(c0 + v) * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) wt[v][j] = t[j];
        bias[v] = (b != nullptr) ? b[c0 + v] : 0.0f;
    }
    float aw[V][4], ab[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        ab[v] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) aw[v][j] = 0.0f;
    }

    for (int n = sq.find(r0); n < sq.n_seq; ++n) {
        int s0, s1;
        sq.range(n, s0, s1);
        if (s0 >= r1) break;
        if (s1 <= r0) continue;
        const int a = max(r0, s0), e = min(r1 + 3, s1 + 3);
        // x_{a-1}, x_{a-2}, x_{a-3}: rows of the sequence or its initial state
        float x1[V], x2[V], x3[V];
        auto xrow = [&](int s, float* x) {
            if (s >= s0) {
                G::unpack(G::ld(u + (size_t)s * D + c0), x);
            } else if (init != nullptr) {
                const float* p = init + ((size_t)n * 3 + (3 + s - s0)) * D + c0;
#pragma unroll
                for (int v = 0; v < V; ++v) x[v] = p[v];
            } else {
#pragma unroll
                for (int v = 0; v < V; ++v) x[v] = 0.0f;
            }
        };
        xrow(a - 1, x1);
        xrow(a - 2, x2);
        xrow(a - 3, x3);
        float p1[V], p2[V], p3[V];  // dpre_{tau-1}, dpre_{tau-2}, dpre_{tau-3}
#pragma unroll
        for (int v = 0; v < V; ++v) p1[v] = p2[v] = p3[v] = 0.0f;
        // rows are loaded BWD_PF steps ahead of their use, into a register
        // ring; past the last row the loads repeat it (a cache hit), so every
        // step issues the same loads and the waits stay counted
        const int e_in = min(e, s1);
        const int last = e_in - 1;
        typename G::Raw bu[BWD_PF], bg[BWD_PF];
#pragma unroll
        for (int i = 0; i < BWD_PF; ++i) {
            bu[i] = G::zero();
            bg[i] = G::zero();
        }
        if (a <= last) {
#pragma unroll
            for (int i = 0; i < BWD_PF; ++i) {
                const size_t r = (size_t)min(a + i, last) * D + c0;
                bu[i] = G::ld(u + r);
                bg[i] = G::ld(dy + r);
            }
        }
        for (int t0 = a; t0 < e; t0 += BWD_PF) {
#pragma unroll
            for (int i = 0; i < BWD_PF; ++i) {
                const int tau = t0 + i;
                if (tau >= e) break;
                float p0[V];
                if (tau < s1) {
                    float xu[V], g[V];
                    G::unpack(bu[i], xu);
                    G::unpack(bg[i], g);
                    {
                        const size_t r = (size_t)min(tau + BWD_PF, last) * D + c0;
                        bu[i] = G::ld(u + r);
                        bg[i] = G::ld(dy + r);
                    }
                    const bool own = tau < r1;
#pragma unroll
                    for (int v = 0; v < V; ++v) {
                        const float pre = bias[v] + wt[v][0] * x3[v] + wt[v][1] * x2[v] + wt[v][2] * x1[v] + wt[v][3] * xu[v];
                        p0[v] = g[v] * dsilu_f(pre);
                        if (own) {
                            aw[v][0] = fmaf(p0[v], x3[v], aw[v][0]);
                            aw[v][1] = fmaf(p0[v], x2[v], aw[v][1]);
                            aw[v][2] = fmaf(p0[v], x1[v], aw[v][2]);
                            aw[v][3] = fmaf(p0[v], xu[v], aw[v][3]);
                            ab[v] += p0[v];
                        }
                        x3[v] = x2[v];
                        x2[v] = x1[v];
                        x1[v] = xu[v];
                    }
                } else {
#pragma unroll
                    for (int v = 0; v < V; ++v) p0[v] = 0.0f;
                }
                // du of row tau - 3, complete now
                const int s = tau - 3;
                if (s >= a && s < min(r1, s1)) {
                    const int k = s - (s1 - 3);
                    float o[V];
#pragma unroll
                    for (int v = 0; v < V; ++v) {
                        o[v] = wt[v][3] * p3[v] + wt[v][2] * p2[v] + wt[v][1] * p1[v] + wt[v][0] * p0[v];
                        if (dfin != nullptr && k >= 0) o[v] += dfin[((size_t)n * 3 + k) * D + c0 + v];
                    }
                    G::store(du + (size_t)s * D + c0, o);
                }
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    p3[v] = p2[v];
                    p2[v] = p1[v];
                    p1[v] = p0[v];
                }
            }
        }
    }
#pragma unroll
    for (int v = 0; v < V; ++v) {
#pragma unroll
        for (int j = 0; j < 4; ++j) part[((size_t)run * 5 + j) * D + c0 + v] = aw[v][j];
        part[((size_t)run * 5 + 4) * D + c0 + v] = ab[v];
    }
}

constexpr int WSUM_BATCH = 8;

// dw[c][j] and db[c]: the run partials, split 64 ways (thread k of a block of
// 16 channels adds runs k, k + 64, ... in order) and the 64 sums added in order.
__global__ __launch_bounds__(1024) void k_conv_wsum(const float* __restrict__ part, float* __restrict__ dw,
                                                    float* __restrict__ db, int n_runs, int D)
{
    __shared__ float red[64][16];
    const int j = blockIdx.y;                  // 0..3 taps, 4 bias
    const int cl = threadIdx.x & 15, k = threadIdx.x >> 4;
    const int c = blockIdx.x * 16 + cl;
    float acc = 0.0f;
    if (c < D)
        // eight loads in flight, added in the same order as one at a time
        for (int r0 = k; r0 < n_runs; r0 += 64 * WSUM_BATCH) {
            float x[WSUM_BATCH];
#pragma unroll
            for (int i = 0; i < WSUM_BATCH; ++i) {
                const int r = r0 + 64 * i;
                x[i] = r < n_runs ? part[((size_t)r * 5 + j) * D + c] : 0.0f;
            }
#pragma unroll
            for (int i = 0; i < WSUM_BATCH; ++i)
                if (r0 + 64 * i < n_runs) acc += x[i];
        }
    red[k][cl] = acc;
    __syncthreads();
    if (k == 0 && c < D) {
        float x = 0.0f;
        for (int i = 0; i < 64; ++i) x += red[i][cl];
        if (j < 4) dw[(size_t)c * 4 + j] = x;
        else if (db != nullptr) db[c] = x;
    }
}

template <typename E>
hipError_t run_conv_bwd(const void* u, const void* dy, const float* w, const float* b, const float* init,
                        const float* dfin, void* du, float* dw, float* db, float* dinit, const int32_t* cu, int n_seq,
                        int B, int T, int D, float* part, hipStream_t stream)
{
    Seqs sq;
    sq.cu = cu;
    sq.n_seq = n_seq;
    sq.T = T;
    sq.S = (cu != nullptr) ? T : B * T;
    const int n_runs = (sq.S + BWD_RUN - 1) / BWD_RUN;
    const int groups = D / Q2<E>::V;
    const int nblk = (groups + BWD_THREADS - 1) / BWD_THREADS;
    const int n_main = n_runs * nblk;
    const int n_init = (dinit != nullptr) ? n_seq * ((D + BWD_THREADS - 1) / BWD_THREADS) : 0;
    hipLaunchKernelGGL(k_conv_bwd<E>, dim3(n_main + n_init), dim3(BWD_THREADS), 0, stream,
                       reinterpret_cast<const E*>(u), reinterpret_cast<const E*>(dy), w, b, init, dfin,
                       reinterpret_cast<E*>(du), part, dinit, sq, D, nblk, n_main);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_conv_wsum, dim3((D + 15) / 16, 5), dim3(1024), 0, stream, part, dw, db, n_runs, D);
    return hipGetLastError();
}

}  // namespace

size_t conv_bwd_part_floats(int B, int T, int D, int packed)
{
    const long S = packed ? (long)T : (long)B * T;
    return (size_t)((S + BWD_RUN - 1) / BWD_RUN) * 5 * D;
}

hipError_t launch_conv_bwd(int bf16, const void* u, const void* dy, const float* w, const float* b,
                           const float* init_state, const float* d_final_state, void* du, float* dw, float* db,
                           float* d_init_state, const int32_t* cu, int n_seq, int B, int T, int D, float* part,
                           hipStream_t stream)
{
    if (bf16)
        return run_conv_bwd<u16>(u, dy, w, b, init_state, d_final_state, du, dw, db, d_init_state, cu, n_seq, B, T,
                                 D, part, stream);
    return run_conv_bwd<float>(u, dy, w, b, init_state, d_final_state, du, dw, db, d_init_state, cu, n_seq, B, T, D,
                               part, stream);
}

hipError_t launch_conv_fwd(int bf16, const void* u, const float* w, const float* b, const float* init_state,
                           float* final_state, void* y, const int32_t* cu, int n_seq, int B, int T, int D,
                           hipStream_t stream)
{
    if (bf16) return run_conv_fwd<u16>(u, w, b, init_state, final_state, y, cu, n_seq, B, T, D, stream);
    return run_conv_fwd<float>(u, w, b, init_state, final_state, y, cu, n_seq, B, T, D, stream);
}

hipError_t launch_conv_decode(int bf16, const void* x, const float* w, const float* b, float* state,
                              const int32_t* slot, void* y, int N, int P, int D, hipStream_t stream)
{
    const dim3 grid((N + DEC_SEQ - 1) / DEC_SEQ, (D / 4 + DEC_THREADS - 1) / DEC_THREADS);
    if (bf16)
        hipLaunchKernelGGL((k_conv_decode<u16, DEC_SEQ>), grid, dim3(DEC_THREADS), 0, stream,
                           reinterpret_cast<const u16*>(x), w, b, state, slot, reinterpret_cast<u16*>(y), N, P, D);
    else
        hipLaunchKernelGGL((k_conv_decode<float, DEC_SEQ>), grid, dim3(DEC_THREADS), 0, stream,
                           reinterpret_cast<const float*>(x), w, b, state, slot, reinterpret_cast<float*>(y), N,
                           P, D);
    return hipGetLastError();
}

}  // namespace sgla
