// Tile-scan body shared by the bf16 forward and backward kernels for gfx950.
//
// Method: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
// attention model on AWS Trainium2 with native PyTorch", section "Challenge 1:
// Using native PyTorch on Trainium for GLA": inside a chunk the output is
// decay-masked linear attention plus the running state's contribution, and the
// state then advances by the per-head decay compounded over the chunk plus the
// chunk's decayed key/value outer products. One scan over a sequence, in the
// operand names of this file (q', k', v' and the output o'), with tiles of C_c
// tokens entered with state S_in and e = 1 (forward in time) or 0 (reverse):
//
//   o'_i  = lam^(i+e) S_in^T q'_i + sum_{j<=i} lam^(i-j) (q'_i . k'_j) v'_j + g_i
//   S_out = lam^(C_c) S_in + sum_j lam^(C_c-e-j) k'_j v'_j^T
//
// The forward and the three gradient scans are instances (roles):
//   FWD: q'=q,  k'=k,  v'=v,  o'=o,  forward, S_in = init state,
//        g_i = sigmoid(z_i) v_i with z_i = sum_d a_d q_id k_id (the
//        self-augmentation of section "i14 and the Laplace 3B architecture",
//        paragraph "GLA mixer");
//   DV:  q'=k,  k'=q,  v'=dO, o'=dv, reverse, S_in = dL/dS_final, final S =
//        dL/dS_init, g_i = sigmoid(z_i) dO_i;
//   DQ:  q'=dO, k'=v,  v'=k,  o'=dq, forward, S_in = S_init^T,
//        g_i = c_i (a (.) k_i), c_i = sigmoid'(z_i) (dO_i . v_i); also the
//        per-column sums of c_i q_i (.) k_i (the gradient of a);
//   DK:  q'=v,  k'=dO, v'=q,  o'=dk, reverse, S_in = (dL/dS_final)^T,
//        g_i = c_i (a (.) q_i).
// A reverse scan runs over the sequence back to front: tile c holds tokens
// len-1-64c-r, r = 0..63, and the readout/update exponents shift by one
// because the state seen from the back already includes the token it is read
// at. The gradient roles need z, so they stage a fourth tile (x = q for DQ,
// x = k for DK) next to v'.
//
// Work decomposition. One workgroup per (sequence, head, 96-column slice of
// v'), four waves:
//   * waves 0..2 ("column owners") each own 32 columns of v'. A wave keeps its
//     d' x 32 fp32 slice of the state in matrix-core accumulators for the
//     whole sequence and computes every output of its columns;
//   * wave 3 ("producer") streams the tiles from HBM straight into an LDS
//     ring (global_load_lds: no registers; with a 3-deep ring two tiles are in
//     flight while the owners compute a third), and for the next tile
//     computes the gate and the decay-masked score tiles P^T = mask(K' Q'^T),
//     handed to the owners as bf16 matrix-core fragments. One barrier per
//     tile.
//
// LDS tiles are row-major ([64][d'] for q', k'; [64][96] for v', x) with
// 16-byte segments permuted within each row, segment c of row r stored at
// c ^ sw(r), so that both the row reads of the score operands and the
// transposing reads below touch distinct banks.
//
// Matrix-core mapping, v_mfma_f32_32x32x16_bf16. Accumulator lane l holds
// column l%32, rows 8(i/4) + 4(l/32) + i%4 in register i. An accumulator used
// as an operand of a contraction over its rows therefore carries, for the
// 16-wide step h, rows 16h + 8a + 4g + b in slot 4a + b (g = l/32); the other
// operand is read with the same row-to-slot map. Operands that contract over
// tokens (V'^T, K'^T) come from the row-major tiles through ds_read_b64_tr_b16:
// within a 16-lane group, lanes 4s + q address token T0 + s at columns
// c0 + 4q, and lane i receives column c0 + i of the four tokens T0..T0+3.
// Per tile and owner wave:
//   O^T  = S^T Q'^T           A = state (bf16 hi + lo pair), B = Q'
//   O^T += V'^T P^T           A = V'^T, B = P^T from the producer
//   S    = lam^C S + K'^T V' - K'^T (c * V'),   c_j = 1 - lam^(C_c-e-j)
// The output tile is O^T (lane = token), so a lane stores 4 adjacent bf16
// columns at a time. The decayed values enter the state update as the exact
// bf16 V' plus a bf16-rounded correction whose size is 1 - lam^m of it: for the
// long-memory heads, whose states dominate, the correction is a few percent of
// the term and its rounding negligible.
#ifndef SGLA_SCAN_HPP
#define SGLA_SCAN_HPP

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sgla {
namespace scan {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int C = 64;             // tokens per tile
constexpr int NOW = 3;            // column-owner waves
constexpr int DVS = 32 * NOW;     // v' columns per workgroup
constexpr int NTHREADS = 64 * (NOW + 1);
constexpr int PRODUCER = NOW;     // wave index of the producer

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

// lam^m for an integer m >= 0 from l2 = log2(lam); lam^0 = 1 also for lam = 0.
__device__ __forceinline__ float powl2(int m, float l2)
{
    return m == 0 ? 1.0f : __builtin_amdgcn_exp2f((float)m * l2);
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
// The address is a uniform base plus a 32-bit lane offset in bytes, so the
// load takes its base from scalar registers.
__device__ __forceinline__ void dma16(const char* base, uint32_t off, char* dst)
{
    __builtin_amdgcn_global_load_lds(base + off, (lds_void*)dst, 16, 0, 0);
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

// As tr_read, but lanes 4s + q address columns c0 + 8q: lane i receives
// column c0 + 8 (i / 4) + i % 4 of the four tokens T0..T0+3.
template <int SEG>
__device__ __forceinline__ u32x2_t tr_read8(const char* tile, int T0, int c0, int lane)
{
    const int j = lane & 15;
    const int off = toff<SEG>(T0 + (j >> 2), c0 + 8 * (j & 3));
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(tile + off));
    return __builtin_bit_cast(u32x2_t, v);
}

__device__ __forceinline__ bf16x8_t frag(u32x2_t lo, u32x2_t hi)
{
    u32x4_t w = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8_t, w);
}

template <int N>
__device__ __forceinline__ void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// One scan, fixed at compile time.
//   DK:     padded width of q'/k' rows (32, 64, 96 or 192)
//   REV:    back-to-front over the sequence (readout lam^i, update lam^(C_c-j))
//   GRAD:   gate-derivative epilogue and a staged x tile (DQ, DK); otherwise
//           sigmoid(z) on the diagonal of P (FWD, DV)
//   DA:     accumulate the per-column sums of c_i x_i (.) v'_i
//   INIT_T: the initial state arrives transposed ([v' col][k' col])
//   NR:     LDS ring depth in tiles (2 or 3)
template <int DK_, bool REV_, bool GRAD_, bool DA_, bool INIT_T_, int NR_>
struct Role {
    static constexpr int DK = DK_;
    static constexpr bool REV = REV_, GRAD = GRAD_, DA = DA_, INIT_T = INIT_T_;
    static constexpr int NR = NR_;
    static constexpr int E = REV_ ? 0 : 1;
};
template <int DK> using RFwd = Role<DK, false, false, false, false, 3>;
template <int DK> using RDv = Role<DK, true, false, false, false, 3>;
template <int DK> using RDq = Role<DK, false, true, true, true, 2>;
template <int DK> using RDk = Role<DK, true, true, false, true, 2>;

template <class R>
struct Lay {
    static constexpr int DK = R::DK;
    static constexpr int NDB = DK / 32;        // 32-row blocks of the state
    static constexpr int SEGK = DK / 8;        // 16-byte segments of a q'/k' row
    static constexpr int SEGV = DVS / 8;       // ... of a v' (or x) row
    static constexpr int SZ_Q = C * DK * 2;
    static constexpr int SZ_V = C * DVS * 2;
    static constexpr int SZ_X = R::GRAD ? SZ_V : 0;
    static constexpr int OFF_K = SZ_Q;
    static constexpr int OFF_V = 2 * SZ_Q;
    static constexpr int OFF_X = 2 * SZ_Q + SZ_V;
    static constexpr int SLOT = 2 * SZ_Q + SZ_V + SZ_X;  // one tile
    static constexpr int OFF_P = R::NR * SLOT;            // 2 x [3 score tiles][2 steps][64 lanes][16 B]
    static constexpr int SZ_P = 3 * 2 * 64 * 16;
    static constexpr int OFF_CORR = OFF_P + 2 * SZ_P;     // c_j for a full and the last tile [2][C]
    static constexpr int OFF_CG = OFF_CORR + 2 * C * 4;   // gate-derivative factors [2][C]
    static constexpr int OFF_A = OFF_CG + (R::GRAD ? 2 * C * 4 : 0);  // a at the v' columns [DVS]
    static constexpr int LDS = OFF_A + (R::GRAD ? DVS * 4 : 0);
    static constexpr int NLQ = SZ_Q / 1024;               // 1 KB load instructions per q' (or k') tile
    static constexpr int NLV = SZ_V / 1024;
    static constexpr int NLOAD = 2 * NLQ + (R::GRAD ? 2 : 1) * NLV;
    static_assert(DK % 32 == 0 && DK <= 192, "DK");
    static_assert(R::NR == 2 || (R::NR == 3 && NLOAD <= 63), "vmcnt");
    static_assert(LDS <= 160 * 1024, "LDS");
};

// Operands of one scan. Rows of q'/k' are dkr elements (also their stride),
// rows of v', x and o' are dvr elements. Token rows: dense, unit (n, h) starts
// at row (n H + h) T; packed (cu != NULL), sequence n of head h spans rows
// h T + cu[n] .. h T + cu[n+1].
struct Args {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* x;       // GRAD roles
    uint16_t* o;
    const float* lambda;
    const float* a;          // [H][width of the gate operands] or NULL
    const int32_t* cu;       // NULL when dense
    const float* s_init;     // [units][dkr][dvr] ([dvr][dkr] for INIT_T) or NULL
    float* s_final;          // [units][dkr][dvr] or NULL
    float* da_part;          // [units][dvr] (DA roles)
    int H, T, n_units, nsl, dkr, dvr;
};

template <class R>
__device__ __forceinline__ void body(const Args& p, int unit, int slice, char* smem)
{
    typedef Lay<R> Ly;
    constexpr int DK = R::DK;
    constexpr int NDB = Ly::NDB, SEGK = Ly::SEGK, SEGV = Ly::SEGV;
    constexpr int E = R::E;
    constexpr int RS = R::REV ? -1 : 1;

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
    // global row of token r of tile c
    auto grow = [&](int c, int r) -> long { return R::REV ? row0 + len - 1 - (c * C + r) : row0 + c * C + r; };
    const int nch = (len + C - 1) / C;
    const int clast = len - (nch - 1) * C;  // length of the last tile
    const float lam = p.lambda[h];
    const float l2 = log2f(lam);           // -inf for lam = 0

    float* corr = reinterpret_cast<float*>(smem + Ly::OFF_CORR);
    // c_j = 1 - lam^(C_c-e-j) for a full tile and for the last tile (j < C_c)
    for (int i = tid; i < 2 * C; i += NTHREADS) {
        const int cl = (i < C) ? C : clast;
        const int j = i & (C - 1);
        corr[i] = (j < cl) ? 1.0f - powl2(cl - E - j, l2) : 0.0f;
    }
    if constexpr (R::GRAD) {
        // a at this slice's v' columns, for the gate-derivative epilogue
        float* at = reinterpret_cast<float*>(smem + Ly::OFF_A);
        for (int i = tid; i < DVS; i += NTHREADS)
            at[i] = (p.a != nullptr && n0 + i < dvr) ? p.a[(size_t)h * dvr + n0 + i] : 0.0f;
    }

    if (wave == PRODUCER) {
        // ------------------------------------------------------------ producer
        // tile c -> ring slot c % NR; the last tile's rows past the sequence
        // are clamped, then zeroed in LDS. Per-lane byte offsets of the 1 KB
        // load blocks within a tile, relative to the tile's lowest global row
        // (rows clamped to the tile length, columns to the real widths)
        uint32_t offq[Ly::NLQ], offv[Ly::NLV];
        auto offsets = [&](int cl) {
#pragma unroll
            for (int m = 0; m < Ly::NLQ; ++m) {
                const int P = 64 * m + lane;              // physical 16-byte slot
                const int r = P / SEGK;
                const int cs = (P - r * SEGK) ^ sw(r);    // logical segment
                const int rr = R::REV ? cl - 1 - min(r, cl - 1) : min(r, cl - 1);
                offq[m] = (uint32_t)(rr * dkr + min(8 * cs, dkr - 8)) * 2u;
            }
#pragma unroll
            for (int m = 0; m < Ly::NLV; ++m) {
                const int P = 64 * m + lane;
                const int r = P / SEGV;
                const int cs = (P - r * SEGV) ^ sw(r);
                const int rr = R::REV ? cl - 1 - min(r, cl - 1) : min(r, cl - 1);
                offv[m] = (uint32_t)(rr * dvr + min(n0 + 8 * cs, dvr - 8)) * 2u;
            }
        };
        offsets(nch > 1 ? C : clast);
        auto issue = [&](int c) {
            char* st = smem + (c % R::NR) * Ly::SLOT;
            const int cl = min(C, len - c * C);
            if (c == nch - 1 && clast < C) offsets(clast);
            const long rb = R::REV ? grow(c, cl - 1) : grow(c, 0);   // lowest row of the tile
            const char* qb = reinterpret_cast<const char*>(p.q + rb * dkr);
            const char* kb = reinterpret_cast<const char*>(p.k + rb * dkr);
            const char* vb = reinterpret_cast<const char*>(p.v + rb * dvr);
#pragma unroll
            for (int m = 0; m < Ly::NLQ; ++m) {
                dma16(qb, offq[m], st + 1024 * m);
                dma16(kb, offq[m], st + Ly::OFF_K + 1024 * m);
            }
#pragma unroll
            for (int m = 0; m < Ly::NLV; ++m) dma16(vb, offv[m], st + Ly::OFF_V + 1024 * m);
            if constexpr (R::GRAD) {
                const char* xb = reinterpret_cast<const char*>(p.x + rb * dvr);
#pragma unroll
                for (int m = 0; m < Ly::NLV; ++m) dma16(xb, offv[m], st + Ly::OFF_X + 1024 * m);
            }
        };
        // rows past the tile and columns past the real widths read as zero
        auto fixup = [&](int c) {
            const int cl = min(C, len - c * C);
            if (cl == C && dkr == DK && n0 + DVS <= dvr) return;
            char* st = smem + (c % R::NR) * Ly::SLOT;
            const u32x4_t zero = {0u, 0u, 0u, 0u};
            for (int P = lane; P < C * SEGK; P += 64) {
                const int r = P / SEGK;
                const int cs = (P - r * SEGK) ^ sw(r);
                if (r >= cl || 8 * cs >= dkr) {
                    *reinterpret_cast<u32x4_t*>(st + 16 * P) = zero;
                    *reinterpret_cast<u32x4_t*>(st + Ly::OFF_K + 16 * P) = zero;
                }
            }
            for (int P = lane; P < C * SEGV; P += 64) {
                const int r = P / SEGV;
                const int cs = (P - r * SEGV) ^ sw(r);
                if (r >= cl || n0 + 8 * cs >= dvr) {
                    *reinterpret_cast<u32x4_t*>(st + Ly::OFF_V + 16 * P) = zero;
                    if constexpr (R::GRAD) *reinterpret_cast<u32x4_t*>(st + Ly::OFF_X + 16 * P) = zero;
                }
            }
        };

        // decay-and-mask factors of the score tiles (constant over tiles):
        // diagonal tile: lam^(t-j) for j <= t else 0; below it: lam^(32 + t - j)
        float dmd[16], dmo[16], dsel[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int diff = l32 - acc_row(i, g);
            dmd[i] = diff < 0 ? 0.0f : powl2(diff, l2);
            dmo[i] = powl2(32 + diff, l2);
            dsel[i] = (diff == 0) ? 1.0f : 0.0f;   // this lane's diagonal element
        }
        // The gate operands: q'/k' rows for FWD and DV, x/v' rows (the 96-wide
        // slice) for DQ and DK.
        constexpr int GW = R::GRAD ? DVS : DK;     // padded gate width
        constexpr int GDB = GW / 32;
        constexpr int GSEG = GW / 8;
        const int gwr = R::GRAD ? dvr : dkr;       // real gate width (= row width of a)
        // diag(a) as A operands: lane (row d = 32 db + l32, group g) holds, for
        // the 16-wide step h, slots d' = 32 db + 16 h + 8 g + j; only d' = d is
        // non-zero (a_d rounded to bf16)
        bf16x8_t adiag[GDB][2];
#pragma unroll
        for (int db = 0; db < GDB; ++db)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int j = l32 - 16 * hh - 8 * g;
                const int dcol = 32 * db + l32;
                const float ad = (p.a != nullptr && dcol < gwr) ? p.a[(size_t)h * gwr + dcol] : 0.0f;
                u32x4_t w;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2)
                    w[s2] = pack2(j == 2 * s2 ? ad : 0.0f, j == 2 * s2 + 1 ? ad : 0.0f);
                adiag[db][hh] = __builtin_bit_cast(bf16x8_t, w);
            }

        // gate and masked scores of tile c (its loads have landed)
        auto scores = [&](int c) {
            const char* st = smem + (c % R::NR) * Ly::SLOT;
            const char* Qs = st;
            const char* Ks = st + Ly::OFF_K;
            const char* Gb = R::GRAD ? st + Ly::OFF_X : Qs;   // gate B-operand rows
            const char* Ga = R::GRAD ? st + Ly::OFF_V : Ks;   // gate A-operand rows
            char* Pb = smem + Ly::OFF_P + (c & 1) * Ly::SZ_P;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                // Q' rows of the strip as B operands (lane group g: d = 16 kb + 8 g + 0..7)
                bf16x8_t qf[DK / 16];
#pragma unroll
                for (int kb = 0; kb < DK / 16; ++kb)
                    qf[kb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                              Qs + toff<SEGK>(32 * s + l32, 16 * kb + 8 * g)));
                // gate argument on the matrix cores: X'^T = diag(a) X^T (a one-hot A
                // operand per 16-wide step), then z_t = (Y X'^T)[t][t]
                float gt;
                {
                    f32x16_t zt = {};
#pragma unroll
                    for (int db = 0; db < GDB; ++db) {
                        f32x16_t qa = {};
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            bf16x8_t xf;
                            if constexpr (R::GRAD)
                                xf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                                      Gb + toff<GSEG>(32 * s + l32, 32 * db + 16 * hh + 8 * g)));
                            else
                                xf = qf[2 * db + hh];
                            qa = mma(adiag[db][hh], xf, qa);
                        }
                        // qa[i]: a_d x_td for d = 32 db + acc_row(i, g), column t
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh) {
                            u32x4_t bw;
#pragma unroll
                            for (int s2 = 0; s2 < 4; ++s2) bw[s2] = pack2(qa[8 * hh + 2 * s2], qa[8 * hh + 2 * s2 + 1]);
                            const int e0 = 32 * db + 16 * hh + 4 * g;
                            const bf16x8_t kz = frag(lds_u32x2(Ga, toff<GSEG>(32 * s + l32, e0)),
                                                     lds_u32x2(Ga, toff<GSEG>(32 * s + l32, e0 + 8)));
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
                    f32x16_t sc = {};
#pragma unroll
                    for (int kb = 0; kb < DK / 16; ++kb) {
                        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                                             Ks + toff<SEGK>(32 * jb + l32, 16 * kb + 8 * g)));
                        sc = mma(kf, qf[kb], sc);
                    }
                    // the gate joins on the diagonal after the product, so that
                    // the two matrix-core chains are independent
                    if (!R::GRAD && jb == s) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) sc[i] = fmaf(dsel[i], gt, sc[i]);
                    }
                    if constexpr (R::GRAD) {
                        if (jb == s) {
                            // c_t = sigmoid'(z_t) (q'_t . k'_t), the raw score's diagonal
                            float u = 0.0f;
#pragma unroll
                            for (int i = 0; i < 16; ++i) u = fmaf(dsel[i], sc[i], u);
                            u += __shfl_xor(u, 32);
                            float* cg = reinterpret_cast<float*>(smem + Ly::OFF_CG) + (c & 1) * C;
                            if (g == 0) cg[32 * s + l32] = gt * (1.0f - gt) * u;
                        }
                    }
                    // sc[i]: column t, key 32 jb + acc_row(i, g)
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
            if (R::NR >= 3 && nch > 1) {
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
            if constexpr (R::NR >= 3) {
                if (c + 2 < nch) issue(c + 2);
                if (c + 1 < nch) {
                    if (c + 2 < nch) wait_vm<Ly::NLOAD>();
                    else wait_vm<0>();
                    fixup(c + 1);
                    scores(c + 1);
                }
            } else {
                if (c + 1 < nch) {
                    issue(c + 1);
                    wait_vm<0>();
                    fixup(c + 1);
                    scores(c + 1);
                }
            }
            lds_barrier();
        }
        return;
    }

    // ---------------------------------------------------------------- owners
    const int nloc = 32 * wave + l32;          // this lane's v' column in the slice
    const int ncol = n0 + nloc;                // ... in the row
    const size_t sbase = (size_t)unit * dkr * dvr;

    f32x16_t sacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int d = 32 * db + acc_row(i, g);
            const size_t si = R::INIT_T ? sbase + (size_t)ncol * dkr + d : sbase + (size_t)d * dvr + ncol;
            sacc[db][i] = (p.s_init != nullptr && d < dkr && ncol < dvr) ? p.s_init[si] : 0.0f;
        }
    }
    // readout decays lam^(t+e) of this lane's token in each 32-row strip
    const float tdec0 = powl2(l32 + E, l2);
    const float tdec1 = powl2(l32 + 32 + E, l2);

    // per-lane column sums of the gradient of a (columns 32 wave + acc_row(i, g))
    float dpart[R::DA ? 16 : 1];
    if constexpr (R::DA) {
#pragma unroll
        for (int i = 0; i < 16; ++i) dpart[i] = 0.0f;
    }

    const float fC = __builtin_amdgcn_exp2f((float)C * l2);  // lam^C
    // one tile; FULL: all 64 tokens and all 96 columns are real (no masking,
    // so the whole tile is one branch-free scheduling region)
    auto tile = [&](int c, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const char* st = smem + (c % R::NR) * Ly::SLOT;
        const char* Qs = st;
        const char* Ks = st + Ly::OFF_K;
        const char* Vs = st + Ly::OFF_V;
        const char* Pb = smem + Ly::OFF_P + (c & 1) * Ly::SZ_P;
        const int cstart = c * C;
        const int cl = FULL ? C : min(C, len - cstart);
        const float* cf = corr + ((!FULL && c == nch - 1) ? C : 0);

        // operand reads of the tile, issued ahead of the math that uses them
        // (K'^T only up to three 32-row blocks; wider states read it block by
        // block in the update, which keeps the registers within one wave's file)
        constexpr bool KPRE = NDB <= 3;
        bf16x8_t kf[KPRE ? NDB : 1][4], vf[4], pf[3][2];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            // V'^T of this lane's column: tokens 16 kb + 8a + 4g + b in slot 4a + b
            vf[kb] = frag(tr_read<SEGV>(Vs, 16 * kb + 4 * g, 32 * wave + 16 * ((lane >> 4) & 1), lane),
                          tr_read<SEGV>(Vs, 16 * kb + 8 + 4 * g, 32 * wave + 16 * ((lane >> 4) & 1), lane));
        }
#pragma unroll
        for (int tl = 0; tl < 3; ++tl)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                pf[tl][hh] = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(Pb + ((tl * 2 + hh) * 64 + lane) * 16));
        // K'^T: key column 32 db + l32, tokens 16 kb + 8a + 4g + b
        auto kread = [&](int db, int kb) {
            return frag(tr_read<SEGK>(Ks, 16 * kb + 4 * g, 32 * db + 16 * ((lane >> 4) & 1), lane),
                        tr_read<SEGK>(Ks, 16 * kb + 8 + 4 * g, 32 * db + 16 * ((lane >> 4) & 1), lane));
        };
        if constexpr (KPRE) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) kf[db][kb] = kread(db, kb);
        }

        // ---- readout of the carried state, both strips: O^T = S^T Q'^T, the
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
                    // Q' row t, d = 32 db + 16 hh + 8a + 4g + b in slot 4a + b
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

        // ---- intra-tile part: O^T += V'^T P^T (a strip past a short last tile
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
            float val[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) val[i] = fmaf(td, oq[s][i], o[i]);
            if constexpr (R::GRAD) {
                // + c_t a (.) v'_t ; DA: column sums of c_t x_t (.) v'_t
                const float ct = reinterpret_cast<const float*>(smem + Ly::OFF_CG)[(c & 1) * C + t];
                const char* Xs = st + Ly::OFF_X;
                const float* at = reinterpret_cast<const float*>(smem + Ly::OFF_A);
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const f32x4_t acol = *reinterpret_cast<const f32x4_t*>(at + 32 * wave + 8 * qd + 4 * g);
                    const u32x2_t yw = lds_u32x2(Vs, toff<SEGV>(t, 32 * wave + 8 * qd + 4 * g));
                    const float y[4] = {bf_lo(yw[0]), bf_hi(yw[0]), bf_lo(yw[1]), bf_hi(yw[1])};
                    float xv[4];
                    if constexpr (R::DA) {
                        const u32x2_t xw = lds_u32x2(Xs, toff<SEGV>(t, 32 * wave + 8 * qd + 4 * g));
                        xv[0] = bf_lo(xw[0]);
                        xv[1] = bf_hi(xw[0]);
                        xv[2] = bf_lo(xw[1]);
                        xv[3] = bf_hi(xw[1]);
                    }
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) {
                        const float cy = ct * y[e4];
                        val[4 * qd + e4] = fmaf(cy, acol[e4], val[4 * qd + e4]);
                        if constexpr (R::DA) dpart[4 * qd + e4] = fmaf(cy, xv[e4], dpart[4 * qd + e4]);
                    }
                }
            }
            if (FULL || t < cl) {
                uint16_t* orow = p.o + grow(c, t) * dvr + n0 + 32 * wave + 4 * g;
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    if (FULL || n0 + 32 * wave + 8 * qd + 4 * g < dvr) {
                        const int i0 = 4 * qd;
                        u32x2_t w2 = {pack2(val[i0], val[i0 + 1]), pack2(val[i0 + 2], val[i0 + 3])};
                        *reinterpret_cast<u32x2_t*>(orow + 8 * qd) = w2;
                    }
                }
            }
        }

        // ---- state advance: S = lam^cl S + K'^T V' - K'^T (c V')  (S already decayed)
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
        if constexpr (KPRE) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    sacc[db] = mma(kf[db][kb], vf[kb], sacc[db]);
                    sacc[db] = mma(kf[db][kb], vc[kb], sacc[db]);
                }
        } else {
            // two blocks of K'^T in flight: block db + 1 is read while db computes
            bf16x8_t kc[2][4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) kc[0][kb] = kread(0, kb);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                if (db + 1 < NDB) {
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb) kc[(db + 1) & 1][kb] = kread(db + 1, kb);
                }
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    sacc[db] = mma(kc[db & 1][kb], vf[kb], sacc[db]);
                    sacc[db] = mma(kc[db & 1][kb], vc[kb], sacc[db]);
                }
            }
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
    if constexpr (R::DA) {
        // sum over the 32 token lanes of each lane group; lane l32 = 0 writes
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float x = dpart[i];
#pragma unroll
            for (int off = 16; off > 0; off >>= 1) x += __shfl_xor(x, off);
            dpart[i] = x;
        }
        if (l32 == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int col = n0 + 32 * wave + acc_row(i, g);
                if (col < dvr) p.da_part[(size_t)unit * dvr + col] = dpart[i];
            }
        }
    }
}


// ----------------------------------------------------------------------------
// Eight-wave body for the scans without the gate-derivative epilogue (FWD, DV).
//
// The four-wave body above keeps one wave per SIMD, and each of its waves is
// bound by the latency of its own dependency chain (state readout -> output,
// decay -> update) rather than by matrix-core, VALU or LDS throughput. Here a
// workgroup has eight waves, two per SIMD, over the same 96-column slice:
//   * waves 0..5 ("column owners") own 16 columns each, with the state slice
//     in v_mfma_f32_16x16x32_bf16 accumulators (lane l: column l%16, rows
//     4(l/16) + r of each 16-row block; A and B operands: row or column l%16,
//     contraction index 8(l/16) + slot);
//   * wave 6 ("loader") streams tiles into a 4-deep LDS ring and computes the
//     gate sigmoid(z) of the tile two ahead;
//   * wave 7 ("scorer") computes the decay-masked scores of the next tile,
//     adds the gate on the diagonal, and writes P^T in the owners' operand
//     order (a 16-token x 32-key block is one 1 KB fragment, 16 B per lane).
// A tile's data is waited for by the loader two iterations before the owners
// use it, so the gate and the scores of tile c+1 both run during iteration c.
// Per tile and owner wave:
//   O^T  = S^T Q'^T    4 token blocks x 3 steps x (hi, lo)    24 MFMA
//   O^T += V'^T P^T    6 blocks                                  6 MFMA
//   S    = lam^C S + K'^T V' - K'^T (c * V')                    24 MFMA
// The state's 16-row accumulator blocks are interleaved in groups of four rows
// (block 2m + h, row 4g + r holds state row 32m + 8g + 4h + r), which makes
// the eight contraction slots of each lane group contiguous state rows, so the
// Q' operand is one 16-byte LDS read; the K'^T operand of the update reads
// key columns in the same order.
constexpr int NOW_W = 6;                   // owner waves
constexpr int OWC = 16;                    // columns per owner
constexpr int NTHREADS_W = 64 * (NOW_W + 2);
constexpr int LOADER_W = NOW_W, SCORER_W = NOW_W + 1;
constexpr int NR_W = 4;                    // ring depth
constexpr int NPB = 6;                     // P fragments per tile: (tb, ks) = (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)

__device__ __forceinline__ f32x4_t mma16(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ constexpr int pblk(int tb, int ks) { return tb < 2 ? tb : 2 + 2 * (tb - 2) + ks; }

template <class R>
struct LayW {
    static constexpr int DK = R::DK;
    static constexpr int NDB16 = DK / 16;      // 16-row blocks of the state
    static constexpr int NKS = DK / 32;        // 32-wide contraction steps over d
    static constexpr int SEGK = DK / 8;
    static constexpr int SEGV = DVS / 8;
    static constexpr int SZ_Q = C * DK * 2;
    static constexpr int SZ_V = C * DVS * 2;
    static constexpr int OFF_K = SZ_Q;
    static constexpr int OFF_V = 2 * SZ_Q;
    static constexpr int SLOT = 2 * SZ_Q + SZ_V;
    static constexpr int OFF_P = NR_W * SLOT;               // 2 x [NPB][64 lanes][16 B]
    static constexpr int SZ_P = NPB * 64 * 16;
    static constexpr int OFF_CORR = OFF_P + 2 * SZ_P;       // [2][C]
    static constexpr int OFF_GT = OFF_CORR + 2 * C * 4;     // gate sigmoid(z) [2][C]
    static constexpr int LDS = OFF_GT + 2 * C * 4;
    static constexpr int NLQ = SZ_Q / 1024;
    static constexpr int NLV = SZ_V / 1024;
    static constexpr int NLOAD = 2 * NLQ + NLV;
    static_assert(!R::GRAD && !R::DA, "eight-wave body: FWD and DV scans only");
    static_assert(DK % 32 == 0 && DK <= 96, "DK");
    static_assert(NLOAD <= 63, "vmcnt");
    static_assert(LDS <= 160 * 1024, "LDS");
};

template <class R>
__device__ __forceinline__ void body_wide(const Args& p, int unit, int slice, char* smem)
{
    typedef LayW<R> Ly;
    constexpr int DK = R::DK;
    constexpr int SEGK = Ly::SEGK, SEGV = Ly::SEGV;
    constexpr int E = R::E;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
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
    auto grow = [&](int c, int r) -> long { return R::REV ? row0 + len - 1 - (c * C + r) : row0 + c * C + r; };
    const int nch = (len + C - 1) / C;
    const int clast = len - (nch - 1) * C;
    const float lam = p.lambda[h];
    const float l2 = log2f(lam);

    float* corr = reinterpret_cast<float*>(smem + Ly::OFF_CORR);
    for (int i = tid; i < 2 * C; i += NTHREADS_W) {
        const int cl = (i < C) ? C : clast;
        const int j = i & (C - 1);
        corr[i] = (j < cl) ? 1.0f - powl2(cl - E - j, l2) : 0.0f;
    }
    float* gtb = reinterpret_cast<float*>(smem + Ly::OFF_GT);

    if (wave == LOADER_W) {
        // ---------------------------------------------------------- loader
        const int l32 = lane & 31, g = lane >> 5;
        uint32_t offq[Ly::NLQ], offv[Ly::NLV];
        auto offsets = [&](int cl) {
#pragma unroll
            for (int m = 0; m < Ly::NLQ; ++m) {
                const int P = 64 * m + lane;
                const int r = P / SEGK;
                const int cs = (P - r * SEGK) ^ sw(r);
                const int rr = R::REV ? cl - 1 - min(r, cl - 1) : min(r, cl - 1);
                offq[m] = (uint32_t)(rr * dkr + min(8 * cs, dkr - 8)) * 2u;
            }
#pragma unroll
            for (int m = 0; m < Ly::NLV; ++m) {
                const int P = 64 * m + lane;
                const int r = P / SEGV;
                const int cs = (P - r * SEGV) ^ sw(r);
                const int rr = R::REV ? cl - 1 - min(r, cl - 1) : min(r, cl - 1);
                offv[m] = (uint32_t)(rr * dvr + min(n0 + 8 * cs, dvr - 8)) * 2u;
            }
        };
        offsets(nch > 1 ? C : clast);
        auto issue = [&](int c) {
            char* st = smem + (c % NR_W) * Ly::SLOT;
            const int cl = min(C, len - c * C);
            if (c == nch - 1 && clast < C) offsets(clast);
            const long rb = R::REV ? grow(c, cl - 1) : grow(c, 0);
            const char* qb = reinterpret_cast<const char*>(p.q + rb * dkr);
            const char* kb = reinterpret_cast<const char*>(p.k + rb * dkr);
            const char* vb = reinterpret_cast<const char*>(p.v + rb * dvr);
#pragma unroll
            for (int m = 0; m < Ly::NLQ; ++m) {
                dma16(qb, offq[m], st + 1024 * m);
                dma16(kb, offq[m], st + Ly::OFF_K + 1024 * m);
            }
#pragma unroll
            for (int m = 0; m < Ly::NLV; ++m) dma16(vb, offv[m], st + Ly::OFF_V + 1024 * m);
        };
        auto fixup = [&](int c) {
            const int cl = min(C, len - c * C);
            if (cl == C && dkr == DK && n0 + DVS <= dvr) return;
            char* st = smem + (c % NR_W) * Ly::SLOT;
            const u32x4_t zero = {0u, 0u, 0u, 0u};
            for (int P = lane; P < C * SEGK; P += 64) {
                const int r = P / SEGK;
                const int cs = (P - r * SEGK) ^ sw(r);
                if (r >= cl || 8 * cs >= dkr) {
                    *reinterpret_cast<u32x4_t*>(st + 16 * P) = zero;
                    *reinterpret_cast<u32x4_t*>(st + Ly::OFF_K + 16 * P) = zero;
                }
            }
            for (int P = lane; P < C * SEGV; P += 64) {
                const int r = P / SEGV;
                const int cs = (P - r * SEGV) ^ sw(r);
                if (r >= cl || n0 + 8 * cs >= dvr) *reinterpret_cast<u32x4_t*>(st + Ly::OFF_V + 16 * P) = zero;
            }
        };
        float dsel[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) dsel[i] = (l32 == acc_row(i, g)) ? 1.0f : 0.0f;
        constexpr int GDB = DK / 32;
        bf16x8_t adiag[GDB][2];
#pragma unroll
        for (int db = 0; db < GDB; ++db)
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
        // sigmoid(z_t) of tile c: z_t = (K (diag(a) Q^T))[t][t] on the matrix cores
        auto gate = [&](int c) {
            const char* st = smem + (c % NR_W) * Ly::SLOT;
            const char* Qs = st;
            const char* Ks = st + Ly::OFF_K;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                f32x16_t zt = {};
#pragma unroll
                for (int db = 0; db < GDB; ++db) {
                    f32x16_t qa = {};
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const bf16x8_t xf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                                            Qs + toff<SEGK>(32 * s + l32, 32 * db + 16 * hh + 8 * g)));
                        qa = mma(adiag[db][hh], xf, qa);
                    }
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
                float z = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) z = fmaf(dsel[i], zt[i], z);
                z += __shfl_xor(z, 32);
                if (g == 0) gtb[(c & 1) * C + 32 * s + l32] = sigmoid_f(z);
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
            gate(0);
            if (nch > 1) {
                if (nch > 2) {
                    issue(2);
                    wait_vm<Ly::NLOAD>();
                } else {
                    wait_vm<0>();
                }
                fixup(1);
                gate(1);
            }
        }
        lds_barrier();
        lds_barrier();
        for (int c = 0; c < nch; ++c) {
            if (c + 3 < nch) issue(c + 3);
            if (c + 2 < nch) {
                if (c + 3 < nch) wait_vm<Ly::NLOAD>();
                else wait_vm<0>();
                fixup(c + 2);
                gate(c + 2);
            }
            lds_barrier();
        }
        return;
    }

    if (wave == SCORER_W) {
        // ---------------------------------------------------------- scorer
        const int l32 = lane & 31, g = lane >> 5;
        float dmd[16], dmo[16], dsel[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int diff = l32 - acc_row(i, g);
            dmd[i] = diff < 0 ? 0.0f : powl2(diff, l2);
            dmo[i] = powl2(32 + diff, l2);
            dsel[i] = (diff == 0) ? 1.0f : 0.0f;
        }
        // scores of tile c: 32 x 32 blocks (s, jb), jb <= s, in the 32x32x16
        // accumulator layout (column t = 32 s + l32, keys 32 jb + acc_row(i, g));
        // each lane writes its masked values into the 16x16x32 B-operand
        // fragments of the owners: token block tb = t / 16, step ks = jb, lane
        // (t % 16) + 16 (i / 4), slots 4 g + i % 4
        auto scores = [&](int c) {
            const char* st = smem + (c % NR_W) * Ly::SLOT;
            const char* Qs = st;
            const char* Ks = st + Ly::OFF_K;
            char* Pb = smem + Ly::OFF_P + (c & 1) * Ly::SZ_P;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                bf16x8_t qf[DK / 16];
#pragma unroll
                for (int kb = 0; kb < DK / 16; ++kb)
                    qf[kb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                              Qs + toff<SEGK>(32 * s + l32, 16 * kb + 8 * g)));
                const float gt = gtb[(c & 1) * C + 32 * s + l32];
                const int tb = 2 * s + (l32 >> 4);
#pragma unroll
                for (int jb = 0; jb <= s; ++jb) {
                    f32x16_t sc = {};
#pragma unroll
                    for (int kb = 0; kb < DK / 16; ++kb) {
                        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                                             Ks + toff<SEGK>(32 * jb + l32, 16 * kb + 8 * g)));
                        sc = mma(kf, qf[kb], sc);
                    }
                    if (jb == s) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) sc[i] = fmaf(dsel[i], gt, sc[i]);
                    }
                    char* blk = Pb + pblk(tb, jb) * 1024;
#pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4) {
                        const int i0 = 4 * a4;
                        const float m0 = (jb == s) ? dmd[i0] : dmo[i0], m1 = (jb == s) ? dmd[i0 + 1] : dmo[i0 + 1];
                        const float m2 = (jb == s) ? dmd[i0 + 2] : dmo[i0 + 2], m3 = (jb == s) ? dmd[i0 + 3] : dmo[i0 + 3];
                        const u32x2_t w2 = {pack2(sc[i0] * m0, sc[i0 + 1] * m1), pack2(sc[i0 + 2] * m2, sc[i0 + 3] * m3)};
                        *reinterpret_cast<u32x2_t*>(blk + ((l32 & 15) + 16 * a4) * 16 + 8 * g) = w2;
                    }
                }
            }
        };
        lds_barrier();
        if (nch > 0) scores(0);
        lds_barrier();
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch) scores(c + 1);
            lds_barrier();
        }
        return;
    }

    // -------------------------------------------------------------- owners
    constexpr int NDB16 = Ly::NDB16, NKS = Ly::NKS;
    const int w = wave;
    const int l16 = lane & 15, qg = lane >> 4;
    const int ncol = n0 + OWC * w + l16;       // this lane's v' column in the row
    const size_t sbase = (size_t)unit * dkr * dvr;

    // Accumulator row 4 qg + r of 16-row block db holds state row
    // d = 32 (db / 2) + 8 qg + 4 (db % 2) + r: the two blocks of a 32-row step
    // interleave in groups of four, so that the readout's eight contraction
    // slots of lane group qg are the contiguous rows 32 ks + 8 qg + 0..7.
    auto srow = [&](int db, int r) { return 32 * (db >> 1) + 8 * qg + 4 * (db & 1) + r; };
    f32x4_t sacc[NDB16];
#pragma unroll
    for (int db = 0; db < NDB16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = srow(db, r);
            sacc[db][r] = (p.s_init != nullptr && d < dkr && ncol < dvr) ? p.s_init[sbase + (size_t)d * dvr + ncol] : 0.0f;
        }
    float tdec[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) tdec[tb] = powl2(16 * tb + l16 + E, l2);
    const float fC = __builtin_amdgcn_exp2f((float)C * l2);

    auto tile = [&](int c, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const char* st = smem + (c % NR_W) * Ly::SLOT;
        const char* Qs = st;
        const char* Ks = st + Ly::OFF_K;
        const char* Vs = st + Ly::OFF_V;
        const char* Pb = smem + Ly::OFF_P + (c & 1) * Ly::SZ_P;
        const int cstart = c * C;
        const int cl = FULL ? C : min(C, len - cstart);
        const float* cf = corr + ((!FULL && c == nch - 1) ? C : 0);
        const float fcl = FULL ? fC : __builtin_amdgcn_exp2f((float)cl * l2);

        // V'^T (A operand of P V') and V' (B operand of the update) share one
        // register layout: lane (column l16, step slice qg) holds tokens
        // 32 ks + 8 qg + 0..7
        bf16x8_t vf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            vf[ks] = frag(tr_read<SEGV>(Vs, 32 * ks + 8 * qg, OWC * w, lane),
                          tr_read<SEGV>(Vs, 32 * ks + 8 * qg + 4, OWC * w, lane));
        bf16x8_t pf[NPB];
#pragma unroll
        for (int b = 0; b < NPB; ++b)
            pf[b] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(Pb + (b * 64 + lane) * 16));

        // ---- readout: O^T = S^T Q'^T, the state as a bf16 pair: hi = the
        // truncated upper half, lo = the remainder (exact in fp32) rounded
        f32x4_t oq[4] = {};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            u32x4_t hw, lw;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) {
                const f32x4_t& blk = (s2 < 2) ? sacc[2 * ks] : sacc[2 * ks + 1];
                const float x0 = blk[2 * (s2 & 1)], x1 = blk[2 * (s2 & 1) + 1];
                const uint32_t b0 = __float_as_uint(x0), b1 = __float_as_uint(x1);
                hw[s2] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
                lw[s2] = pack2(x0 - __uint_as_float(b0 & 0xffff0000u), x1 - __uint_as_float(b1 & 0xffff0000u));
            }
            const bf16x8_t sh = __builtin_bit_cast(bf16x8_t, hw), sl = __builtin_bit_cast(bf16x8_t, lw);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                // Q' row 16 tb + l16, d = 32 ks + 8 qg + 0..7
                const bf16x8_t qf = __builtin_bit_cast(
                    bf16x8_t, *reinterpret_cast<const u32x4_t*>(Qs + toff<SEGK>(16 * tb + l16, 32 * ks + 8 * qg)));
                oq[tb] = mma16(sh, qf, oq[tb]);
                oq[tb] = mma16(sl, qf, oq[tb]);
            }
        }
#pragma unroll
        for (int db = 0; db < NDB16; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[db][r] *= fcl;

        // ---- intra-tile part and output (lane = token 16 tb + l16, columns 4 qg + r)
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            f32x4_t o = {};
            o = mma16(vf[0], pf[pblk(tb, 0)], o);
            if (tb >= 2) o = mma16(vf[1], pf[pblk(tb, 1)], o);
            const int t = 16 * tb + l16;
            if (FULL || t < cl) {
                const int col = n0 + OWC * w + 4 * qg;
                if (FULL || col < dvr) {
                    uint16_t* orow = p.o + grow(c, t) * dvr + col;
                    const u32x2_t w2 = {pack2(fmaf(tdec[tb], oq[tb][0], o[0]), fmaf(tdec[tb], oq[tb][1], o[1])),
                                        pack2(fmaf(tdec[tb], oq[tb][2], o[2]), fmaf(tdec[tb], oq[tb][3], o[3]))};
                    *reinterpret_cast<u32x2_t*>(orow) = w2;
                }
            }
        }

        // ---- state advance: S = lam^cl S + K'^T V' - K'^T (c V')
        bf16x8_t vc[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(cf + 32 * ks + 8 * qg);
            const f32x4_t c1 = *reinterpret_cast<const f32x4_t*>(cf + 32 * ks + 8 * qg + 4);
            const u32x4_t vw = __builtin_bit_cast(u32x4_t, vf[ks]);
            u32x4_t cw;
            cw[0] = pack2(-c0[0] * bf_lo(vw[0]), -c0[1] * bf_hi(vw[0]));
            cw[1] = pack2(-c0[2] * bf_lo(vw[1]), -c0[3] * bf_hi(vw[1]));
            cw[2] = pack2(-c1[0] * bf_lo(vw[2]), -c1[1] * bf_hi(vw[2]));
            cw[3] = pack2(-c1[2] * bf_lo(vw[3]), -c1[3] * bf_hi(vw[3]));
            vc[ks] = __builtin_bit_cast(bf16x8_t, cw);
        }
#pragma unroll
        for (int db = 0; db < NDB16; ++db)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                // K'^T: row l16 of block db (key column srow with qg -> l16 / 4,
                // r -> l16 % 4), tokens 32 ks + 8 qg + 0..7
                const int kc0 = 32 * (db >> 1) + 4 * (db & 1);
                const bf16x8_t kf = frag(tr_read8<SEGK>(Ks, 32 * ks + 8 * qg, kc0, lane),
                                         tr_read8<SEGK>(Ks, 32 * ks + 8 * qg + 4, kc0, lane));
                sacc[db] = mma16(kf, vf[ks], sacc[db]);
                sacc[db] = mma16(kf, vc[ks], sacc[db]);
            }
    };

    const bool cols_full = (n0 + DVS <= dvr);
    lds_barrier();
    lds_barrier();
    for (int c = 0; c < nch; ++c) {
        if (cols_full && (c < nch - 1 || clast == C)) tile(c, std::true_type{});
        else tile(c, std::false_type{});
        lds_barrier();
    }

    if (p.s_final != nullptr && ncol < dvr) {
#pragma unroll
        for (int db = 0; db < NDB16; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = srow(db, r);
                if (d < dkr) p.s_final[sbase + (size_t)d * dvr + ncol] = sacc[db][r];
            }
    }
}

}  // namespace scan
}  // namespace sgla

#endif
