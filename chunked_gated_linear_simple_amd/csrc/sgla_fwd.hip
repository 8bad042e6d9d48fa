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
//     96 x 32 fp32 slice of the state in matrix-core accumulators for the whole
//     sequence and computes every output of its columns, so the state never
//     leaves the wave and no wave waits on another for it;
//   * wave 3 ("producer") reads the next tile from HBM into registers while
//     the owners compute the current one, then writes it to the other half of a
//     double-buffered LDS stage: Q and K row-major, K^T and V^T token-minor, and
//     the per-token gate sigmoid(z). One barrier per tile.
//
// Matrix-core mapping, v_mfma_f32_32x32x16_bf16. Accumulator lane l holds
// column l%32, rows 8(i/4) + 4(l/32) + i%4 in register i. Any accumulator read
// back as an operand of a contraction over its rows therefore carries, for the
// 16-wide step h, the rows 16h + 8a + 4g + b in slot 4a + b (g = l/32), and the
// other operand is loaded with the same row-to-slot map (two 8-byte LDS reads).
// Per tile and owner wave:
//   O^T  = S^T Q^T            A = state (bf16 hi + lo pair), B = Q
//   P^T  = mask(K Q^T)        scores, kept in registers; the gate is added to
//                             the diagonal before the mask, so P V carries it
//   O^T += V^T P^T            A = V^T, B = scores as bf16
//   S    = lam^C S + K^T V - K^T (c * V),   c_j = 1 - lam^(C_c-1-j)
// The output tile is O^T (lane = token), so a lane stores 4 adjacent bf16
// columns at a time. The decayed values enter the state update as the exact
// bf16 V plus a bf16-rounded correction whose size is 1 - lam^m of it: for the
// long-memory heads, whose states dominate, the correction is a few percent of
// the term and its rounding negligible.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgla_internal.h"

namespace sgla {
namespace fwdk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int C = 64;             // tokens per tile
constexpr int NOW = 3;            // column-owner waves
constexpr int DVS = 32 * NOW;     // value columns per workgroup
constexpr int NTHREADS = 64 * (NOW + 1);
constexpr int PRODUCER = NOW;     // wave index of the producer

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    // round to nearest even, a in the low half
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8_t frag(u32x2_t lo, u32x2_t hi)
{
    u32x4_t w = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8_t, w);
}

__device__ __forceinline__ f32x16_t mma(bf16x8_t a, bf16x8_t b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of accumulator register i for lane group g.
__device__ __forceinline__ constexpr int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// Barrier for LDS hand-offs: waits for this wave's LDS operations only, so
// outstanding global loads (the producer's prefetch) stay in flight.
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

template <int DK>
struct Lay {
    static constexpr int NDB = DK / 32;        // 32-row blocks of the state
    static constexpr int NSEG = DK / 8;        // 16-byte segments of a q/k row
    static constexpr int LDQ = DK + 4;         // Q, K row stride (elements): 8 x odd bytes
    static constexpr int LDT = C + 4;          // K^T, V^T row stride: 136 bytes
    static constexpr int SZ_Q = C * LDQ * 2;
    static constexpr int SZ_KT = DK * LDT * 2;
    static constexpr int SZ_VT = DVS * LDT * 2;
    static constexpr int OFF_Q = 0;
    static constexpr int OFF_K = OFF_Q + SZ_Q;
    static constexpr int OFF_KT = OFF_K + SZ_Q;
    static constexpr int OFF_VT = OFF_KT + SZ_KT;
    static constexpr int OFF_G = OFF_VT + SZ_VT;   // gate sigmoid(z) [C]
    static constexpr int STAGE = OFF_G + C * 4;
    static constexpr int OFF_CORR = 2 * STAGE;     // c_j for a full tile and the last tile [2][C]
    static constexpr int LDS = OFF_CORR + 2 * C * 4;
    static constexpr int NQI = NSEG / 4;           // producer q/k items per lane
    static constexpr int NVI = DVS / 8 / 4;        // producer v items per lane (3)
    static_assert(DK % 32 == 0 && DK <= 96, "DK");
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

template <int DK>
__global__ __launch_bounds__(NTHREADS) void k_fwd(Args p)
{
    typedef Lay<DK> Ly;
    constexpr int NDB = Ly::NDB, LDQ = Ly::LDQ, LDT = Ly::LDT;
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
        constexpr int NQI = Ly::NQI, NVI = Ly::NVI;
        const int tg = lane & 15, cb = lane >> 4;   // token group of 4, first segment
        float av[NQI][8];
#pragma unroll
        for (int m = 0; m < NQI; ++m)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int col = 8 * (cb + 4 * m) + e;
                av[m][e] = (p.a != nullptr && col < dkr) ? p.a[(size_t)h * dkr + col] : 0.0f;
            }
        u32x4_t rq[NQI][4], rk[NQI][4], rv[NVI][4];
        // rows 4 tg + r of tile c; clamped into the sequence only on the last tile
        auto load = [&](int c) {
            const int cs0 = c * C;
            const bool last = (c == nch - 1);
            const int cl = min(C, len - cs0);
            const uint16_t* qb = p.q + (row0 + cs0) * dkr;
            const uint16_t* kb = p.k + (row0 + cs0) * dkr;
            const uint16_t* vb = p.v + (row0 + cs0) * dvr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int rr = last ? min(4 * tg + r, cl - 1) : 4 * tg + r;
#pragma unroll
                for (int m = 0; m < NQI; ++m) {
                    const int col = min(8 * (cb + 4 * m), dkr - 8);
                    rq[m][r] = *reinterpret_cast<const u32x4_t*>(qb + rr * dkr + col);
                    rk[m][r] = *reinterpret_cast<const u32x4_t*>(kb + rr * dkr + col);
                }
#pragma unroll
                for (int m = 0; m < NVI; ++m) {
                    const int col = min(n0 + 8 * (cb + 4 * m), dvr - 8);
                    rv[m][r] = *reinterpret_cast<const u32x4_t*>(vb + rr * dvr + col);
                }
            }
        };
        // low halves of x, y -> one word (x low); high halves likewise
        auto lo2 = [](uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x05040100u); };
        auto hi2 = [](uint32_t x, uint32_t y) { return __builtin_amdgcn_perm(y, x, 0x07060302u); };
        auto put = [&](int c) {
            char* st = smem + (c & 1) * Ly::STAGE;
            uint16_t* Qs = reinterpret_cast<uint16_t*>(st + Ly::OFF_Q);
            uint16_t* Ks = reinterpret_cast<uint16_t*>(st + Ly::OFF_K);
            uint16_t* KT = reinterpret_cast<uint16_t*>(st + Ly::OFF_KT);
            uint16_t* VT = reinterpret_cast<uint16_t*>(st + Ly::OFF_VT);
            float* gate = reinterpret_cast<float*>(st + Ly::OFF_G);
            const int cl = min(C, len - c * C);
            const u32x4_t zero = {0u, 0u, 0u, 0u};
            if (cl < C || dkr < DK || n0 + DVS > dvr) {
                // rows past the tile and columns past the real widths read as zero
#pragma unroll
                for (int m = 0; m < NQI; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool okq = (4 * tg + r < cl) && (8 * (cb + 4 * m) < dkr);
                        rq[m][r] = okq ? rq[m][r] : zero;
                        rk[m][r] = okq ? rk[m][r] : zero;
                    }
#pragma unroll
                for (int m = 0; m < NVI; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool okv = (4 * tg + r < cl) && (n0 + 8 * (cb + 4 * m) < dvr);
                        rv[m][r] = okv ? rv[m][r] : zero;
                    }
            }
            float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < NQI; ++m) {
                const int col = 8 * (cb + 4 * m);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ro = (4 * tg + r) * LDQ + col;
                    *reinterpret_cast<u32x2_t*>(Qs + ro) = u32x2_t{rq[m][r][0], rq[m][r][1]};
                    *reinterpret_cast<u32x2_t*>(Qs + ro + 4) = u32x2_t{rq[m][r][2], rq[m][r][3]};
                    *reinterpret_cast<u32x2_t*>(Ks + ro) = u32x2_t{rk[m][r][0], rk[m][r][1]};
                    *reinterpret_cast<u32x2_t*>(Ks + ro + 4) = u32x2_t{rk[m][r][2], rk[m][r][3]};
                    // gate argument z = sum_d a_d q_d k_d in fp32 (the bf16 dot2 builtin is
                    // not used: this compiler feeds it element 0 of a vector for every element)
#pragma unroll
                    for (int w2 = 0; w2 < 4; ++w2) {
                        const uint32_t qw = rq[m][r][w2], kw = rk[m][r][w2];
                        z[r] = fmaf(av[m][2 * w2], bf_lo(qw) * bf_lo(kw), z[r]);
                        z[r] = fmaf(av[m][2 * w2 + 1], bf_hi(qw) * bf_hi(kw), z[r]);
                    }
                }
                // K^T: column d of four consecutive tokens in one 8-byte write
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    const uint32_t k0 = rk[m][0][w2], k1 = rk[m][1][w2], k2 = rk[m][2][w2], k3 = rk[m][3][w2];
                    *reinterpret_cast<u32x2_t*>(KT + (col + 2 * w2) * LDT + 4 * tg) = u32x2_t{lo2(k0, k1), lo2(k2, k3)};
                    *reinterpret_cast<u32x2_t*>(KT + (col + 2 * w2 + 1) * LDT + 4 * tg) = u32x2_t{hi2(k0, k1), hi2(k2, k3)};
                }
            }
#pragma unroll
            for (int m = 0; m < NVI; ++m) {
                const int col = 8 * (cb + 4 * m);
#pragma unroll
                for (int w2 = 0; w2 < 4; ++w2) {
                    const uint32_t v0 = rv[m][0][w2], v1 = rv[m][1][w2], v2 = rv[m][2][w2], v3 = rv[m][3][w2];
                    *reinterpret_cast<u32x2_t*>(VT + (col + 2 * w2) * LDT + 4 * tg) = u32x2_t{lo2(v0, v1), lo2(v2, v3)};
                    *reinterpret_cast<u32x2_t*>(VT + (col + 2 * w2 + 1) * LDT + 4 * tg) = u32x2_t{hi2(v0, v1), hi2(v2, v3)};
                }
            }
            // the four lanes sharing a token group hold the partial sums of all segments
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                z[r] += __shfl_xor(z[r], 16);
                z[r] += __shfl_xor(z[r], 32);
            }
            if (cb == 0) {
                f32x4_t gv;
#pragma unroll
                for (int r = 0; r < 4; ++r) gv[r] = sigmoid_f(z[r]);
                *reinterpret_cast<f32x4_t*>(gate + 4 * tg) = gv;
            }
        };

        if (nch > 0) {
            load(0);
            put(0);
            if (nch > 1) load(1);
        }
        lds_barrier();
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch) put(c + 1);
            if (c + 2 < nch) load(c + 2);
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

    // decay-and-mask factors of the score tiles (constant over tiles):
    // diagonal tile: lam^(t-j) for j <= t else 0; below it: lam^(32 + t - j)
    float dmd[16], dmo[16];
    bool dsel[16];  // the diagonal element of this lane's column
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int diff = l32 - acc_row(i, g);
        dmd[i] = diff < 0 ? 0.0f : (diff == 0 ? 1.0f : __builtin_amdgcn_exp2f((float)diff * l2));
        dmo[i] = __builtin_amdgcn_exp2f((float)(32 + diff) * l2);
        dsel[i] = (diff == 0);
    }
    // readout decays lam^(t+1) of this lane's token in each 32-row strip
    const float tdec0 = __builtin_amdgcn_exp2f((float)(l32 + 1) * l2);
    const float tdec1 = __builtin_amdgcn_exp2f((float)(l32 + 33) * l2);

    lds_barrier();
    for (int c = 0; c < nch; ++c) {
        const char* st = smem + (c & 1) * Ly::STAGE;
        const uint16_t* Qs = reinterpret_cast<const uint16_t*>(st + Ly::OFF_Q);
        const uint16_t* Ks = reinterpret_cast<const uint16_t*>(st + Ly::OFF_K);
        const uint16_t* KT = reinterpret_cast<const uint16_t*>(st + Ly::OFF_KT);
        const uint16_t* VT = reinterpret_cast<const uint16_t*>(st + Ly::OFF_VT);
        const float* gate = reinterpret_cast<const float*>(st + Ly::OFF_G);
        const int cstart = c * C;
        const int cl = min(C, len - cstart);
        const float* cf = corr + ((c == nch - 1) ? C : 0);

        // V^T operand fragments of this lane's column, tokens 16 kb + 8a + 4g + b
        bf16x8_t vf[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const uint16_t* vr = VT + nloc * LDT + 16 * kb + 4 * g;
            vf[kb] = frag(*reinterpret_cast<const u32x2_t*>(vr), *reinterpret_cast<const u32x2_t*>(vr + 8));
        }
        auto qfrag = [&](int t, int db, int hh) {
            const uint16_t* qr = Qs + t * LDQ + 32 * db + 16 * hh + 4 * g;
            return frag(*reinterpret_cast<const u32x2_t*>(qr), *reinterpret_cast<const u32x2_t*>(qr + 8));
        };

        // ---- readout of the carried state, both strips: O^T = S^T Q^T with the
        // state as a bf16 hi + lo pair (A operand), built once per tile
        f32x16_t oq[2] = {};
        {
            bf16x8_t sh[NDB][2], sl[NDB][2];
#pragma unroll
            for (int db = 0; db < NDB; ++db)
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
                    sh[db][hh] = __builtin_bit_cast(bf16x8_t, hw);
                    sl[db][hh] = __builtin_bit_cast(bf16x8_t, lw);
                }
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const bf16x8_t qf = qfrag(32 * s + l32, db, hh);
                        oq[s] = mma(sh[db][hh], qf, oq[s]);
                        oq[s] = mma(sl[db][hh], qf, oq[s]);
                    }
        }

        // ---- intra-tile part of the two 32-token strips (a strip past a short
        // last tile computes on zeros; its stores are masked)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int t = 32 * s + l32;
            bf16x8_t qf[NDB][2];
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) qf[db][hh] = qfrag(t, db, hh);
            f32x16_t o = {};
            const float gt = gate[t];
#pragma unroll
            for (int jb = 0; jb <= s; ++jb) {
                f32x16_t sc;
#pragma unroll
                for (int i = 0; i < 16; ++i) sc[i] = (jb == s && dsel[i]) ? gt : 0.0f;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const uint16_t* kr = Ks + (32 * jb + l32) * LDQ + 32 * db + 16 * hh + 4 * g;
                        const bf16x8_t kf = frag(*reinterpret_cast<const u32x2_t*>(kr),
                                                 *reinterpret_cast<const u32x2_t*>(kr + 8));
                        sc = mma(kf, qf[db][hh], sc);
                    }
                // sc[i]: column t, key 32 jb + acc_row(i, g); the gate sits on the diagonal
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
                    o = mma(vf[2 * jb + hh], __builtin_bit_cast(bf16x8_t, pw), o);
                }
            }
            // O^T: lane = token t, registers = columns 32 wave + acc_row(i, g)
            const float td = s ? tdec1 : tdec0;
            if (t < cl) {
                uint16_t* orow = p.o + (row0 + cstart + t) * dvr + n0 + 32 * wave + 4 * g;
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    if (n0 + 32 * wave + 8 * qd + 4 * g < dvr) {
                        const int i0 = 4 * qd;
                        u32x2_t w2 = {pack2(fmaf(td, oq[s][i0], o[i0]), fmaf(td, oq[s][i0 + 1], o[i0 + 1])),
                                      pack2(fmaf(td, oq[s][i0 + 2], o[i0 + 2]), fmaf(td, oq[s][i0 + 3], o[i0 + 3]))};
                        *reinterpret_cast<u32x2_t*>(orow + 8 * qd) = w2;
                    }
                }
            }
        }

        // ---- state advance: S = lam^cl S + K^T V - K^T (c V)
        const float fcl = (cl == C) ? __builtin_amdgcn_exp2f((float)C * l2)
                                    : __builtin_amdgcn_exp2f((float)cl * l2);
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
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[db][i] *= fcl;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const uint16_t* kr = KT + (32 * db + l32) * LDT + 16 * kb + 4 * g;
                const bf16x8_t kf = frag(*reinterpret_cast<const u32x2_t*>(kr),
                                         *reinterpret_cast<const u32x2_t*>(kr + 8));
                sacc[db] = mma(kf, vf[kb], sacc[db]);
                sacc[db] = mma(kf, vc[kb], sacc[db]);
            }
        }
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
