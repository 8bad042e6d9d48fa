// Chunked Simple GLA forward for gfx950, bf16 inputs.
//
// Method: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
// attention model on AWS Trainium2 with native PyTorch", section "Challenge 1:
// Using native PyTorch on Trainium for GLA": inside a chunk the output is
// decay-masked linear attention plus the running state's contribution, and the
// state then advances by the per-head decay compounded over the chunk plus the
// chunk's decayed key/value outer products. With rows i, j of a tile of C_c
// tokens entered with state S_in:
//
//   o_i   = lam^(i+1) S_in^T q_i + sum_{j<=i} lam^(i-j) (q_i . k_j) v_j + sigmoid(z_i) v_i
//   S_out = lam^(C_c) S_in + sum_j lam^(C_c-1-j) k_j v_j^T,   z_i = sum_d a_d q_id k_id
//
// (the self-augmentation term of section "i14 and the Laplace 3B architecture",
// paragraph "GLA mixer"). Tiles are 64 tokens; the result does not depend on
// the tile length beyond rounding.
//
// Work decomposition. One workgroup per (sequence, head, 96-column value
// slice), four waves:
//   * waves 0..2 ("column owners") each own 32 value columns. A wave keeps its
//     d_k x 32 fp32 slice of the state in matrix-core accumulators for the
//     whole sequence and computes every output of its columns, so the state
//     never leaves the wave;
//   * wave 3 ("producer") streams the tiles from HBM straight into a 3-deep
//     LDS ring (global_load_lds: no registers, two tiles in flight while the
//     owners compute a third), and for the next tile computes the gate
//     sigmoid(z) and the decay-masked score tiles P^T = mask(K Q^T), with the
//     gate added on the diagonal so that P V carries the self-augmentation
//     term. The owners take P as bf16 matrix-core fragments. One barrier per
//     tile.
//
// LDS tiles are row-major (Q, K: [64][d_k], V: [64][96]) with 16-byte segments
// permuted within each row, segment c of row r stored at c ^ sw(r), so that
// both the row reads of the score operands and the transposing reads below
// touch distinct banks.
//
// Matrix-core mapping, v_mfma_f32_32x32x16_bf16. Accumulator lane l holds
// column l%32, rows 8(i/4) + 4(l/32) + i%4 in register i. An accumulator used
// as an operand of a contraction over its rows therefore carries, for the
// 16-wide step h, rows 16h + 8a + 4g + b in slot 4a + b (g = l/32); the other
// operand is read with the same row-to-slot map. Operands that contract over
// tokens (V^T, K^T) come from the row-major tiles through ds_read_b64_tr_b16:
// within a 16-lane group, lanes 4s + q address token T0 + s at columns
// c0 + 4q, and lane i receives column c0 + i of the four tokens T0..T0+3.
// Per tile and owner wave:
//   O^T  = S^T Q^T            A = state (bf16 hi + lo pair), B = Q
//   O^T += V^T P^T            A = V^T, B = P^T from the producer
//   S    = lam^C S + K^T V - K^T (c * V),   c_j = 1 - lam^(C_c-1-j)
// The output tile is O^T (lane = token), so a lane stores 4 adjacent bf16
// columns at a time. The decayed values enter the state update as the exact
// bf16 V plus a bf16-rounded correction whose size is 1 - lam^m of it: for the
// long-memory heads, whose states dominate, the correction is a few percent of
// the term and its rounding negligible.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sgla_internal.h"

namespace sgla {
namespace fwdk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int C = 64;             // tokens per tile
constexpr int NOW = 3;            // column-owner waves
constexpr int DVS = 32 * NOW;     // value columns per workgroup
constexpr int NTHREADS = 64 * (NOW + 1);
constexpr int PRODUCER = NOW;     // wave index of the producer
constexpr int NR = 3;             // LDS ring depth (tiles)

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    // round to nearest even, a in the low half
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x16_t mma(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of accumulator register i for lane group g.
__device__ __forceinline__ constexpr int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// Barrier for LDS hand-offs: waits for this wave's LDS operations only.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float sigmoid_f(float z)
{
    // 1 / (1 + e^-z) without overflow for either sign
    const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * fabsf(z));
    const float r = __builtin_amdgcn_rcpf(1.0f + e);
    return z >= 0.0f ? r : e * r;
}

// Segment permutation of a tile row: segment c of row r lives at c ^ sw(r).
__device__ __forceinline__ int sw(int r)
{
    const int x = (r >> 1) & 3;
    return ((x & 1) << 1) | (x >> 1);
}

// Byte offset of element e of row r in a swizzled tile with SEG 16-byte segments per row.
template <int SEG>
__device__ __forceinline__ int toff(int r, int e)
{
    return r * (SEG * 16) + (((e >> 3) ^ sw(r)) << 4) + ((e & 7) << 1);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at dst + 16 l (global_load_lds_dwordx4; completion is counted by vmcnt).
__device__ __forceinline__ void dma16(const uint16_t* src, char* dst)
{
    __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

__device__ __forceinline__ u32x2_t lds_u32x2(const char* base, int off)
{
    return *reinterpret_cast<const u32x2_t*>(base + off);
}

// Four tokens T0..T0+3 of column c0 + (lane % 16): the lane of a 16-lane group
// passes the address of token T0 + (lane % 16) / 4, columns c0 + 4 (lane % 4).
template <int SEG>
__device__ __forceinline__ u32x2_t tr_read(const char* tile, int T0, int c0, int lane)
{
    const int j = lane & 15;
    const int off = toff<SEG>(T0 + (j >> 2), c0 + 4 * (j & 3));
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(tile + off));
    return __builtin_bit_cast(u32x2_t, v);
}

__device__ __forceinline__ bf16x8_t frag(u32x2_t lo, u32x2_t hi)
{
    u32x4_t w = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8_t, w);
}

template <int DK>
struct Lay {
    static constexpr int NDB = DK / 32;        // 32-row blocks of the state
    static constexpr int SEGK = DK / 8;        // 16-byte segments of a q/k row
    static constexpr int SEGV = DVS / 8;       // ... of a v row
    static constexpr int SZ_Q = C * DK * 2;
    static constexpr int SZ_V = C * DVS * 2;
    static constexpr int SLOT = 2 * SZ_Q + SZ_V;  // Q, K, V of one tile
    static constexpr int OFF_P = NR * SLOT;       // 2 x [3 score tiles][2 steps][64 lanes][16 B]
    static constexpr int SZ_P = 3 * 2 * 64 * 16;
    static constexpr int OFF_CORR = OFF_P + 2 * SZ_P;  // c_j for a full and the last tile [2][C]
    static constexpr int LDS = OFF_CORR + 2 * C * 4;
    static constexpr int NLQ = SZ_Q / 1024;          // 1 KB load instructions per q (or k) tile
    static constexpr int NLV = SZ_V / 1024;
    static constexpr int NLOAD = 2 * NLQ + NLV;
    static_assert(DK % 32 == 0 && DK <= 96, "DK");
    static_assert(NLOAD <= 63, "vmcnt");
    static_assert(LDS <= 160 * 1024, "LDS");
};

struct Args {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    const float* lambda;
    const float* a;          // [H, dkr] or NULL
    const int32_t* cu;       // NULL when dense
    const float* s_init;     // [units, dkr, dvr] or NULL
    float* s_final;          // or NULL
    int H, T, n_units, nsl, dkr, dvr;
};

template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int DK>
__global__ __launch_bounds__(NTHREADS) void k_fwd(Args p)
{
    typedef Lay<DK> Ly;
    constexpr int NDB = Ly::NDB, SEGK = Ly::SEGK, SEGV = Ly::SEGV;
    __shared__ __attribute__((aligned(16))) char smem[Ly::LDS];

    // blockIdx -> (unit, slice); the slices of one unit share an XCD (blocks
    // are dealt to the eight XCDs round-robin) and so share its L2
    const int b = blockIdx.x;
    const int slice = (b >> 3) % p.nsl;
    const int unit = ((b >> 3) / p.nsl) * 8 + (b & 7);
    if (unit >= p.n_units) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;
    const int H = p.H;
    const int seq = unit / H, h = unit - seq * H;
    const int dkr = p.dkr, dvr = p.dvr;
    const int n0 = slice * DVS;

    long row0;
    int len;
    if (p.cu != nullptr) {
        int s0 = p.cu[seq], s1 = p.cu[seq + 1];
        s0 = min(max(s0, 0), p.T);
        s1 = min(max(s1, s0), p.T);
        row0 = (long)h * p.T + s0;
        len = s1 - s0;
    } else {
        row0 = ((long)seq * H + h) * p.T;
        len = p.T;
    }
    const int nch = (len + C - 1) / C;
    const int clast = len - (nch - 1) * C;  // length of the last tile
    const float lam = p.lambda[h];
    const float l2 = log2f(lam);           // -inf for lam = 0

    float* corr = reinterpret_cast<float*>(smem + Ly::OFF_CORR);
    // c_j = 1 - lam^(C_c-1-j) for a full tile and for the last tile (j < C_c)
    for (int i = tid; i < 2 * C; i += NTHREADS) {
        const int cl = (i < C) ? C : clast;
        const int j = i & (C - 1);
        const int m = cl - 1 - j;
        corr[i] = (j < cl) ? ((m == 0) ? 0.0f : 1.0f - __builtin_amdgcn_exp2f((float)m * l2)) : 0.0f;
    }

    if (wave == PRODUCER) {
        // ------------------------------------------------------------ producer
        // tile c -> ring slot c % NR, global rows row0 + 64 c + r (the last
        // tile's rows past the sequence are clamped, then zeroed in LDS)
        // per-lane element offsets of the 1 KB load blocks within a tile (rows
        // clamped to the tile length, columns to the real widths)
        int offq[Ly::NLQ], offv[Ly::NLV];
        auto offsets = [&](int cl) {
#pragma unroll
            for (int m = 0; m < Ly::NLQ; ++m) {
                const int P = 64 * m + lane;              // physical 16-byte slot
                const int r = P / SEGK;
                const int cs = (P - r * SEGK) ^ sw(r);    // logical segment
                offq[m] = min(r, cl - 1) * dkr + min(8 * cs, dkr - 8);
            }
#pragma unroll
            for (int m = 0; m < Ly::NLV; ++m) {
                const int P = 64 * m + lane;
                const int r = P / SEGV;
                const int cs = (P - r * SEGV) ^ sw(r);
                offv[m] = min(r, cl - 1) * dvr + min(n0 + 8 * cs, dvr - 8);
            }
        };
        offsets(nch > 1 ? C : clast);
        auto issue = [&](int c) {
            char* st = smem + (c % NR) * Ly::SLOT;
            if (c == nch - 1 && clast < C) offsets(clast);
            const uint16_t* qb = p.q + (row0 + (long)c * C) * dkr;
            const uint16_t* kb = p.k + (row0 + (long)c * C) * dkr;
            const uint16_t* vb = p.v + (row0 + (long)c * C) * dvr;
#pragma unroll
            for (int m = 0; m < Ly::NLQ; ++m) {
                dma16(qb + offq[m], st + 1024 * m);
                dma16(kb + offq[m], st + Ly::SZ_Q + 1024 * m);
            }
#pragma unroll
            for (int m = 0; m < Ly::NLV; ++m)
                dma16(vb + offv[m], st + 2 * Ly::SZ_Q + 1024 * m);
        };
        // rows past the tile and columns past the real widths read as zero
        auto fixup = [&](int c) {
            const int cl = min(C, len - c * C);
            if (cl == C && dkr == DK && n0 + DVS <= dvr) return;
            char* st = smem + (c % NR) * Ly::SLOT;
            const u32x4_t zero = {0u, 0u, 0u, 0u};
            for (int P = lane; P < C * SEGK; P += 64) {
                const int r = P / SEGK;
                const int cs = (P - r * SEGK) ^ sw(r);
                if (r >= cl || 8 * cs >= dkr) {
                    *reinterpret_cast<u32x4_t*>(st + 16 * P) = zero;
                    *reinterpret_cast<u32x4_t*>(st + Ly::SZ_Q + 16 * P) = zero;
                }
            }
            for (int P = lane; P < C * SEGV; P += 64) {
                const int r = P / SEGV;
                const int cs = (P - r * SEGV) ^ sw(r);
                if (r >= cl || n0 + 8 * cs >= dvr)
                    *reinterpret_cast<u32x4_t*>(st + 2 * Ly::SZ_Q + 16 * P) = zero;
            }
        };

        // decay-and-mask factors of the score tiles (constant over tiles):
        // diagonal tile: lam^(t-j) for j <= t else 0; below it: lam^(32 + t - j)
        float dmd[16], dmo[16], dsel[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int diff = l32 - acc_row(i, g);
            dmd[i] = diff < 0 ? 0.0f : (diff == 0 ? 1.0f : __builtin_amdgcn_exp2f((float)diff * l2));
            dmo[i] = __builtin_amdgcn_exp2f((float)(32 + diff) * l2);
            dsel[i] = (diff == 0) ? 1.0f : 0.0f;   // this lane's diagonal element
        }
        // diag(a) as A operands: lane (row d = 32 db + l32, group g) holds, for
        // the 16-wide step h, slots d' = 32 db + 16 h + 8 g + j; only d' = d is
        // non-zero (a_d rounded to bf16)
        bf16x8_t adiag[NDB][2];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int j = l32 - 16 * hh - 8 * g;
                const int dcol = 32 * db + l32;
                const float ad = (p.a != nullptr && dcol < dkr) ? p.a[(size_t)h * dkr + dcol] : 0.0f;
                u32x4_t w;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2)
                    w[s2] = pack2(j == 2 * s2 ? ad : 0.0f, j == 2 * s2 + 1 ? ad : 0.0f);
                adiag[db][hh] = __builtin_bit_cast(bf16x8_t, w);
            }

        // gate and masked scores of tile c (its loads have landed)
        auto scores = [&](int c) {
            const char* st = smem + (c % NR) * Ly::SLOT;
            const char* Qs = st;
            const char* Ks = st + Ly::SZ_Q;
            char* Pb = smem + Ly::OFF_P + (c & 1) * Ly::SZ_P;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                // Q rows of the strip as B operands (lane group g: d = 16 kb + 8 g + 0..7)
                bf16x8_t qf[DK / 16];
#pragma unroll
                for (int kb = 0; kb < DK / 16; ++kb)
                    qf[kb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                              Qs + toff<SEGK>(32 * s + l32, 16 * kb + 8 * g)));
                // gate argument on the matrix cores: Q'^T = diag(a) Q^T (a one-hot A
                // operand per 16-wide step), then z_t = (K Q'^T)[t][t]
                float gt;
                {
                    f32x16_t zt = {};
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        f32x16_t qa = {};
                        qa = mma(adiag[db][0], qf[2 * db], qa);
                        qa = mma(adiag[db][1], qf[2 * db + 1], qa);
                        // qa[i]: a_d q_td for d = 32 db + acc_row(i, g), column t
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            u32x4_t bw;
#pragma unroll
                            for (int s2 = 0; s2 < 4; ++s2) bw[s2] = pack2(qa[8 * hh + 2 * s2], qa[8 * hh + 2 * s2 + 1]);
                            const int e0 = 32 * db + 16 * hh + 4 * g;
                            const bf16x8_t kz = frag(lds_u32x2(Ks, toff<SEGK>(32 * s + l32, e0)),
                                                     lds_u32x2(Ks, toff<SEGK>(32 * s + l32, e0 + 8)));
                            zt = mma(kz, __builtin_bit_cast(bf16x8_t, bw), zt);
                        }
                    }
                    // the diagonal element (j = t) sits in one lane group
                    float z = 0.0f;
#pragma unroll
                    for (int i = 0; i < 16; ++i) z = fmaf(dsel[i], zt[i], z);
                    z += __shfl_xor(z, 32);
                    gt = sigmoid_f(z);
                }
#pragma unroll
                for (int jb = 0; jb <= s; ++jb) {
                    f32x16_t sc;
#pragma unroll
                    for (int i = 0; i < 16; ++i) sc[i] = (jb == s) ? dsel[i] * gt : 0.0f;
#pragma unroll
                    for (int kb = 0; kb < DK / 16; ++kb) {
                        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                                             Ks + toff<SEGK>(32 * jb + l32, 16 * kb + 8 * g)));
                        sc = mma(kf, qf[kb], sc);
                    }
                    // sc[i]: column t, key 32 jb + acc_row(i, g); the gate sits on the diagonal
                    const int tile = s + jb;  // (0,0) -> 0, (1,0) -> 1, (1,1) -> 2
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        u32x4_t pw;
#pragma unroll
                        for (int s2 = 0; s2 < 4; ++s2) {
                            const int i0 = 8 * hh + 2 * s2;
                            const float m0 = (jb == s) ? dmd[i0] : dmo[i0];
                            const float m1 = (jb == s) ? dmd[i0 + 1] : dmo[i0 + 1];
                            pw[s2] = pack2(sc[i0] * m0, sc[i0 + 1] * m1);
                        }
                        *reinterpret_cast<u32x4_t*>(Pb + ((tile * 2 + hh) * 64 + lane) * 16) = pw;
                    }
                }
            }
        };

        if (nch > 0) {
            issue(0);
            if (nch > 1) {
                issue(1);
                wait_vm<Ly::NLOAD>();
            } else {
                wait_vm<0>();
            }
            fixup(0);
            scores(0);
        }
        lds_barrier();
        for (int c = 0; c < nch; ++c) {
            if (c + 2 < nch) issue(c + 2);
            if (c + 1 < nch) {
                if (c + 2 < nch) wait_vm<Ly::NLOAD>();
                else wait_vm<0>();
                fixup(c + 1);
                scores(c + 1);
            }
            lds_barrier();
        }
        return;
    }

    // ---------------------------------------------------------------- owners
    const int nloc = 32 * wave + l32;          // this lane's value column in the slice
    const int ncol = n0 + nloc;                // ... in the head
    const size_t sbase = (size_t)unit * dkr * dvr;

    f32x16_t sacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int d = 32 * db + acc_row(i, g);
            sacc[db][i] = (p.s_init != nullptr && d < dkr && ncol < dvr)
                              ? p.s_init[sbase + (size_t)d * dvr + ncol] : 0.0f;
        }
    }
    // readout decays lam^(t+1) of this lane's token in each 32-row strip
    const float tdec0 = __builtin_amdgcn_exp2f((float)(l32 + 1) * l2);
    const float tdec1 = __builtin_amdgcn_exp2f((float)(l32 + 33) * l2);

    const float fC = __builtin_amdgcn_exp2f((float)C * l2);  // lam^C
    // one tile; FULL: all 64 tokens and all 96 columns are real (no masking,
    // so the whole tile is one branch-free scheduling region)
    auto tile = [&](int c, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const char* st = smem + (c % NR) * Ly::SLOT;
        const char* Qs = st;
        const char* Ks = st + Ly::SZ_Q;
        const char* Vs = st + 2 * Ly::SZ_Q;
        const char* Pb = smem + Ly::OFF_P + (c & 1) * Ly::SZ_P;
        const int cstart = c * C;
        const int cl = FULL ? C : min(C, len - cstart);
        const float* cf = corr + ((!FULL && c == nch - 1) ? C : 0);

        // operand reads of the tile, issued ahead of the math that uses them
        bf16x8_t kf[NDB][4], vf[4], pf[3][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            // V^T of this lane's column: tokens 16 kb + 8a + 4g + b in slot 4a + b
            vf[kb] = frag(tr_read<SEGV>(Vs, 16 * kb + 4 * g, 32 * wave + 16 * ((lane >> 4) & 1), lane),
                          tr_read<SEGV>(Vs, 16 * kb + 8 + 4 * g, 32 * wave + 16 * ((lane >> 4) & 1), lane));
        }
#pragma unroll
        for (int tl = 0; tl < 3; ++tl)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                pf[tl][hh] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(Pb + ((tl * 2 + hh) * 64 + lane) * 16));
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                // K^T: key column 32 db + l32, tokens 16 kb + 8a + 4g + b
                kf[db][kb] = frag(tr_read<SEGK>(Ks, 16 * kb + 4 * g, 32 * db + 16 * ((lane >> 4) & 1), lane),
                                  tr_read<SEGK>(Ks, 16 * kb + 8 + 4 * g, 32 * db + 16 * ((lane >> 4) & 1), lane));

        // ---- readout of the carried state, both strips: O^T = S^T Q^T, the
        // state entering as a bf16 hi + lo pair (A operand) built block by
        // block; each block is then decayed for the state advance
        const float fcl = FULL ? fC : __builtin_amdgcn_exp2f((float)cl * l2);
        f32x16_t oq[2] = {};
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                u32x4_t hw, lw;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    const float x0 = sacc[db][8 * hh + 2 * s2], x1 = sacc[db][8 * hh + 2 * s2 + 1];
                    const uint32_t hp = pack2(x0, x1);
                    hw[s2] = hp;
                    lw[s2] = pack2(x0 - bf_lo(hp), x1 - bf_hi(hp));
                }
                const bf16x8_t sh = __builtin_bit_cast(bf16x8_t, hw), sl = __builtin_bit_cast(bf16x8_t, lw);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    // Q row t, d = 32 db + 16 hh + 8a + 4g + b in slot 4a + b
                    const int t = 32 * s + l32;
                    const bf16x8_t qf = frag(lds_u32x2(Qs, toff<SEGK>(t, 32 * db + 16 * hh + 4 * g)),
                                             lds_u32x2(Qs, toff<SEGK>(t, 32 * db + 16 * hh + 8 + 4 * g)));
                    oq[s] = mma(sh, qf, oq[s]);
                    oq[s] = mma(sl, qf, oq[s]);
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[db][i] *= fcl;
        }

        // ---- intra-tile part: O^T += V^T P^T (a strip past a short last tile
        // computes on zeros; its stores are masked)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int t = 32 * s + l32;
            f32x16_t o = {};
#pragma unroll
            for (int jb = 0; jb <= s; ++jb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) o = mma(vf[2 * jb + hh], pf[s + jb][hh], o);
            // O^T: lane = token t, registers = columns 32 wave + acc_row(i, g)
            const float td = s ? tdec1 : tdec0;
            if (FULL || t < cl) {
                uint16_t* orow = p.o + (row0 + cstart + t) * dvr + n0 + 32 * wave + 4 * g;
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    if (FULL || n0 + 32 * wave + 8 * qd + 4 * g < dvr) {
                        const int i0 = 4 * qd;
                        u32x2_t w2 = {pack2(fmaf(td, oq[s][i0], o[i0]), fmaf(td, oq[s][i0 + 1], o[i0 + 1])),
                                      pack2(fmaf(td, oq[s][i0 + 2], o[i0 + 2]), fmaf(td, oq[s][i0 + 3], o[i0 + 3]))};
                        *reinterpret_cast<u32x2_t*>(orow + 8 * qd) = w2;
                    }
                }
            }
        }

        // ---- state advance: S = lam^cl S + K^T V - K^T (c V)  (S already decayed)
        bf16x8_t vc[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(cf + 16 * kb + 4 * g);
            const f32x4_t c1 = *reinterpret_cast<const f32x4_t*>(cf + 16 * kb + 8 + 4 * g);
            const u32x4_t vw = __builtin_bit_cast(u32x4_t, vf[kb]);
            u32x4_t cw;
            cw[0] = pack2(-c0[0] * bf_lo(vw[0]), -c0[1] * bf_hi(vw[0]));
            cw[1] = pack2(-c0[2] * bf_lo(vw[1]), -c0[3] * bf_hi(vw[1]));
            cw[2] = pack2(-c1[0] * bf_lo(vw[2]), -c1[1] * bf_hi(vw[2]));
            cw[3] = pack2(-c1[2] * bf_lo(vw[3]), -c1[3] * bf_hi(vw[3]));
            vc[kb] = __builtin_bit_cast(bf16x8_t, cw);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                sacc[db] = mma(kf[db][kb], vf[kb], sacc[db]);
                sacc[db] = mma(kf[db][kb], vc[kb], sacc[db]);
            }
    };

    const bool cols_full = (n0 + DVS <= dvr);
    lds_barrier();
    for (int c = 0; c < nch; ++c) {
        if (cols_full && (c < nch - 1 || clast == C)) tile(c, std::true_type{});
        else tile(c, std::false_type{});
        lds_barrier();
    }

    if (p.s_final != nullptr && ncol < dvr) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int d = 32 * db + acc_row(i, g);
                if (d < dkr) p.s_final[sbase + (size_t)d * dvr + ncol] = sacc[db][i];
            }
    }
}

template <int DK>
hipError_t run(const Args& a, hipStream_t stream)
{
    const int grid = ((a.n_units + 7) / 8) * 8 * a.nsl;
    hipLaunchKernelGGL(k_fwd<DK>, dim3(grid), dim3(NTHREADS), 0, stream, a);
    return hipGetLastError();
}

}  // namespace fwdk

// bf16 forward with d_k <= 96 (padded to 32, 64 or 96) and any d_v (96-column slices).
hipError_t launch_fwd_bf16(const ChunkProblem& p, const void* q, const void* k, const void* v,
                           const float* init_state, float* final_state, void* o,
                           hipStream_t stream)
{
    fwdk::Args a;
    a.q = reinterpret_cast<const uint16_t*>(q);
    a.k = reinterpret_cast<const uint16_t*>(k);
    a.v = reinterpret_cast<const uint16_t*>(v);
    a.o = reinterpret_cast<uint16_t*>(o);
    a.lambda = p.lambda;
    a.a = p.a;
    a.cu = p.cu;
    a.s_init = init_state;
    a.s_final = final_state;
    a.H = p.H;
    a.T = p.T;
    a.n_units = p.n_seq * p.H;
    a.nsl = (p.d_v + fwdk::DVS - 1) / fwdk::DVS;
    a.dkr = p.d_k;
    a.dvr = p.d_v;
    if (p.d_k <= 32) return fwdk::run<32>(a, stream);
    if (p.d_k <= 64) return fwdk::run<64>(a, stream);
    return fwdk::run<96>(a, stream);
}

}  // namespace sgla
