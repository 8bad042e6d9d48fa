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
// len-1-CT*c-r, r = 0..CT-1, and the readout/update exponents shift by one
// because the state seen from the back already includes the token it is read
// at. The gradient roles need z, so they stage a fourth tile (x = q for DQ,
// x = k for DK) next to v'.
//
// Conventions shared by all waves (the workgroup structure is described at
// body_wide below):
//   * LDS tiles are row-major ([CT][d'] for q', k'; [CT][96] for v', x) with
//     16-byte segments permuted within each row, segment c of row r stored at
//     c ^ sw<SEG>(r), so that the 16-byte row reads, the 8-byte row reads
//     and the 4-column transposing reads are free of bank conflicts (the
//     8-column transposing reads of K' take two passes per 32 lanes, the
//     least any segment permutation allows them).
//   * Operands that contract over tokens (V'^T, K'^T) come from the row-major
//     tiles through ds_read_b64_tr_b16: within a 16-lane group, lanes 4s + q
//     address token T0 + s at columns c0 + 4q (tr_read), and lane i receives
//     column c0 + i of the four tokens T0..T0+3.
//   * v_mfma_f32_32x32x16_bf16 (scores): accumulator lane l holds
//     column l%32, rows 8(i/4) + 4(l/32) + i%4 in register i; an accumulator
//     used as an operand of a contraction over its rows carries, for the
//     16-wide step h, rows 16h + 8a + 4g + b in slot 4a + b (g = l/32).
//   * The state update enters each decayed value lam^m v'_j (m = C_c-e-j) as
//     two bf16 operands A_j + B_j of two products K'^T A + K'^T B, chosen so
//     that the rounding never exceeds 2^-9 of the term itself:
//       lam^m >= 1/2:  A_j = v'_j (exact), B_j = bf16(-(1 - lam^m) v'_j)
//                      (|B_j| <= |term|; a few percent of it for the
//                      long-memory heads, whose states dominate);
//       lam^m <  1/2:  A_j = 0,           B_j = bf16(lam^m v'_j)
//                      (a plain correction would be nearly -v'_j here, and
//                      its rounding, 2^-9 |v'_j|, would not decay with the
//                      term: the short-memory heads' states would carry it).
//     The readout takes the state as a bf16 hi + lo pair.
#ifndef SGLA_SCAN_HPP
#define SGLA_SCAN_HPP

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sgla {
namespace scan {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

constexpr int DVS = 96;           // v' columns per workgroup

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    // round to nearest even, a in the low half
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

// x sigmoid(x); e^-x overflows to inf for very negative x, giving -0
__device__ __forceinline__ float silu_f(float x)
{
    const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * x);
    return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// For each of four words holding a bf16 pair (low half first):
// S_e = x_0 y_0 + x_1 y_1 and D_e = x_0 y_0 - x_1 y_1 (exact products, one fp32
// sum). One block of VOP3 dot products with the negate modifier on the second
// pair; a dot product's result needs three wait states before a VALU reads
// it, which the trailing s_nop provides (the compiler cannot see inside the
// block), and the outputs are early-clobber because the inputs are read after
// the first write.
__device__ __forceinline__ void dot2_sd4(const u32x4_t& x, const u32x4_t& y, float (&S)[4], float (&D)[4])
{
    asm("v_dot2_f32_bf16 %0, %8, %12, 0\n\t"
        "v_dot2_f32_bf16 %1, %8, %12, 0 neg_hi:[0,1,0]\n\t"
        "v_dot2_f32_bf16 %2, %9, %13, 0\n\t"
        "v_dot2_f32_bf16 %3, %9, %13, 0 neg_hi:[0,1,0]\n\t"
        "v_dot2_f32_bf16 %4, %10, %14, 0\n\t"
        "v_dot2_f32_bf16 %5, %10, %14, 0 neg_hi:[0,1,0]\n\t"
        "v_dot2_f32_bf16 %6, %11, %15, 0\n\t"
        "v_dot2_f32_bf16 %7, %11, %15, 0 neg_hi:[0,1,0]\n\t"
        "s_nop 2"
        : "=&v"(S[0]), "=&v"(D[0]), "=&v"(S[1]), "=&v"(D[1]), "=&v"(S[2]), "=&v"(D[2]), "=&v"(S[3]), "=&v"(D[3])
        : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]));
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

// Segment permutation of a tile row with SEG 16-byte segments: segment c of
// row r lives at c ^ sw<SEG>(r). gfx950's LDS has 64 four-byte banks and
// serves a 16-byte-per-lane access 16 lanes at a time (8-byte: 32 lanes), so
// 16 consecutive rows at one logical segment must land on 16 distinct 16-byte
// bank groups. Rows of 4 or 12 segments repeat their bank offset every 4 rows,
// so the mask cycles with r / 4; rows of 8 or 24 segments repeat it every
// 2 rows, so the mask (up to 7, which keeps c ^ mask inside the row because
// SEG is a multiple of 8) cycles with r / 2.
template <int SEG>
__device__ __forceinline__ int sw(int r)
{
    static_assert(SEG % 4 == 0, "SEG");
    if constexpr (SEG % 8 == 0) return (r >> 1) & 7;
    else return (r >> 2) & 3;
}

// Byte offset of element e of row r in a swizzled tile with SEG 16-byte segments per row.
template <int SEG>
__device__ __forceinline__ int toff(int r, int e)
{
    return r * (SEG * 16) + (((e >> 3) ^ sw<SEG>(r)) << 4) + ((e & 7) << 1);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at dst + 16 l (global_load_lds_dwordx4; completion is counted by vmcnt).
// The address is a uniform base plus a 32-bit lane offset in bytes, so the
// load takes its base from scalar registers. POL is the load's cache policy:
// 0, or POL_NT (the non-temporal hint) for data no later access of the launch
// wants from the caches.
constexpr int POL_NT = 2;
template <int POL = 0>
__device__ __forceinline__ void dma16(const char* base, uint32_t off, char* dst)
{
    __builtin_amdgcn_global_load_lds(base + off, (lds_void*)dst, 16, 0, POL);
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
    // Segments (dense sequences only; nseg <= 1: whole sequences). Sequence n
    // is cut into nseg segments of seg_len tokens (the last one shorter); a
    // launch runs segments seg_first .. seg_first + seg_count - 1 of every
    // sequence, unit = ((n seg_count) + i) H + h. The segment where the scan
    // enters the sequence (0, or the last for a reverse scan) starts from
    // s_init, the one where it leaves writes s_final; the others start from
    // s_in_seg and write s_out_seg, both [n][nseg][H][state] (NULL: zero / not
    // written). With seg_in_all set the entering segment reads s_in_seg too,
    // so that a launch whose last segment writes s_final never reads s_init.
    int nseg, seg_len, seg_first, seg_count, seg_in_all;
    const float* s_in_seg;
    float* s_out_seg;
    // Mixer epilogue applied to the output tile before the store (NG roles):
    // out[row][h][c] = silu(g[row][h][c]) gamma[h / per_tier][c] o[c] / rms,
    // token-major rows (b T + t dense, cu[n] + t packed); o is then optional.
    // The slices of one unit exchange their per-token sums of o^2 through
    // xch, [groups][nsl][NG_XR][CT] words of (tag << 32 | bits of the sum).
    // A launch runs units unit_base + group.
    const uint16_t* ng_g;
    const float* ng_gamma;   // [n_tiers][dvr] or NULL (one)
    uint16_t* ng_out;
    unsigned long long* xch;
    int* xerr;               // set to 1 when an exchange wait gives up
    int* xtick;              // [8] tickets taken per XCD index (blockIdx % 8)
    int* xdone;              // workgroups finished
    int per_tier, unit_base;
    float inv_dv, eps;
};

// Exchange slots per slice of a group (a ring over its tiles), the most
// workgroups of one fused grid, and the exchange buffer's header: int 0 is
// the error flag, ints NG_XTICK .. NG_XTICK+7 the tickets per XCD index and
// int NG_XDONE the count of finished workgroups.
constexpr int NG_XR = 4;
constexpr int NG_MAX_WG = 1024;
constexpr int NG_XHEAD = 256;
constexpr int NG_XTICK = 16, NG_XDONE = 32;
// Upper bound of the polls of one exchange wait (each after a short sleep)
// before the wait gives up: the tile's output is NaN, and the workgroup's
// later waits give up at once.
constexpr int NG_SPIN_MAX = 1 << 20;

// ----------------------------------------------------------------------------
// Eight-wave body.
//
// With one wave per SIMD each wave is bound by the latency of its own
// dependency chain (state readout -> output, decay -> update) rather than by
// matrix-core, VALU or LDS throughput, so a workgroup has eight waves, two per
// SIMD, over one 96-column slice of v':
//   * waves 0..5 ("column owners") own 16 columns each, with the state slice
//     in v_mfma_f32_16x16x32_bf16 accumulators (lane l: column l%16, rows
//     4(l/16) + r of each 16-row block; A and B operands: row or column l%16,
//     contraction index 8(l/16) + slot);
//   * wave 6 ("loader") streams tiles into a 4-deep LDS ring and computes the
//     gate sigmoid(z) of the next tile, in fp32 (lane = token), while the
//     loads of the tile three ahead fly;
//   * wave 7 ("scorer") computes the decay-masked scores of the next tile and
//     writes P^T in the owners' operand order (a 16-token x 32-key block is one
//     1 KB fragment, 16 B per lane). P leaves out the diagonal: the scorer
//     passes the raw diagonal q'_t . k'_t to the owners in fp32. FWD and DV add
//     (q'_t . k'_t + sigmoid(z_t)) v'_t in their epilogue; DQ and DK add
//     (q'_t . k'_t) v'_t and apply c_t = sigmoid'(z_t) (q'_t . k'_t). (A bf16
//     diagonal costs 2^-9 of the term that dominates a short-memory head's
//     output.)
// A tile's data is waited for by the loader two iterations before the owners
// use it, so the gate and the scores of tile c+1 both run during iteration c.
// The NG role (the epilogue applied before the store) differs: its ring is
// three deep, the fourth slot's LDS holding three tiles of the gate stream g;
// the loader forms the gate of tile c+1 on the VALU, in fp32, right after the
// tile arrives, and the scorer waits for it.
// Tiles are 64 tokens for the 96-wide contractions (FWD, DV) and 32 tokens
// for the 192-wide ones (DQ, DK), so that four tiles fit the LDS ring. Per
// 64 tokens and owner wave: state readout 4 x (d'/32) x (hi, lo), P V' 6, and
// state update 2 x 2 x (d'/16) MFMAs.
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

// Roles of the eight-wave body: as Role, plus the tile length CT.
// OUT = false keeps only the state scan: no q' tile, gate, scores, readout
// or output, for passes whose only product is the state a run leaves.
// NG = true (forward only) applies the mixer epilogue to each output tile
// before its store.
template <int DK_, bool REV_, bool GRAD_, bool DA_, bool INIT_T_, int CT_, bool OUT_ = true, bool NG_ = false>
struct WRole {
    static constexpr int DK = DK_, CT = CT_;
    static constexpr bool REV = REV_, GRAD = GRAD_, DA = DA_, INIT_T = INIT_T_, OUT = OUT_, NG = NG_;
    static constexpr int E = REV_ ? 0 : 1;
};
template <int DK, int CT = 64> using WFwd = WRole<DK, false, false, false, false, CT>;
template <int DK, int CT = 64> using WFwdNg = WRole<DK, false, false, false, false, CT, true, true>;
template <int DK, int CT = 64> using WDv = WRole<DK, true, false, false, false, CT>;
template <int DK> using WFwdState = WRole<DK, false, false, false, false, 64, false>;
template <int DK> using WDvState = WRole<DK, true, false, false, false, 64, false>;
template <int DK> using WDq = WRole<DK, false, true, true, true, 32>;
template <int DK> using WDk = WRole<DK, true, true, false, true, 32>;

__device__ __forceinline__ f32x4_t mma16(bf16x8_t a, bf16x8_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// P fragment of token block tb (16 tokens) and key step ks (32 keys, ks <= tb / 2)
__device__ __forceinline__ constexpr int pblk(int tb, int ks) { return tb < 2 ? tb : 2 + 2 * (tb - 2) + ks; }

template <class R>
struct LayW {
    static constexpr int DK = R::DK, CT = R::CT;
    static constexpr int NTB = CT / 16;        // 16-token blocks of a tile
    static constexpr int NKT = CT / 32;        // 32-token steps (also score strips)
    static constexpr int NPB = CT == 64 ? 6 : 2;
    static constexpr int NDB16 = DK / 16;      // 16-row blocks of the state
    static constexpr int NKS = DK / 32;        // 32-wide contraction steps over d'
    static constexpr int SEGK = DK / 8;
    static constexpr int SEGV = DVS / 8;
    static constexpr int SZ_Q = CT * DK * 2;
    static constexpr int SZ_V = CT * DVS * 2;
    static constexpr int SZ_X = R::GRAD ? SZ_V : 0;
    static constexpr int OFF_K = SZ_Q;
    static constexpr int OFF_V = 2 * SZ_Q;
    static constexpr int OFF_X = 2 * SZ_Q + SZ_V;
    static constexpr int SLOT = 2 * SZ_Q + SZ_V + SZ_X;
    // ring depth: the NG role gives a slot to the gate values (OFF_G)
    static constexpr int NR = R::NG ? 3 : NR_W;
    // P: 2 x [NPB][64 lanes][16 B], the tiles c and c+1 (NG: one tile's
    // hi and lo halves)
    static constexpr int OFF_P = NR * SLOT;
    static constexpr int SZ_P = NPB * 64 * 16;
    static constexpr int OFF_CORR = OFF_P + 2 * SZ_P;       // update coefficients of B [2][CT]
    static constexpr int OFF_KEEP = OFF_CORR + 2 * CT * 4;  // masks of A, one word per token pair [2][CT/2]
    static constexpr int OFF_GT = OFF_KEEP + CT * 4;        // gate sigmoid(z) [2][CT]
    // The raw diagonal of the scores in fp32 [2][CT]: it stays out of the
    // bf16 P, and the owners add it (with the gate for FWD and DV) times v'_t.
    static constexpr bool DIAG32 = R::OUT && !R::NG;
    static constexpr int OFF_DG = OFF_GT + 2 * CT * 4;
    static constexpr int OFF_A = OFF_DG + (DIAG32 ? 2 * CT * 4 : 0);  // a at the v' columns [DVS]
    static constexpr int OFF_SS = OFF_A + (R::GRAD ? DVS * 4 : 0);     // NG: owners' sums of o^2 [NOW_W][CT]
    static constexpr int OFF_INV = OFF_SS + (R::NG ? NOW_W * CT * 4 : 0);  // NG: 1 / rms per token [CT]
    // NG: sums ready, 1 / rms ready, tile and gate ready, and the
    // workgroup's ticket (set by k_fwd_ng before the body runs)
    static constexpr int OFF_CNT = OFF_INV + (R::NG ? CT * 4 : 0);
    static constexpr int OFF_G = OFF_CNT + (R::NG ? 16 : 0);            // NG: 3 x [CT][96] gate values g
    // the gate's channel weights as pairs (a_2j + a_2j+1, a_2j - a_2j+1) / 2,
    // fp32, over the q'/k' channels [DK] (FWD, DV, NG) or the slice's x/v'
    // channels [DVS] (DQ, DK)
    static constexpr int OFF_AB = OFF_G + (R::NG ? 3 * SZ_V : 0);
    static constexpr int LDS = OFF_AB + (R::OUT ? (R::GRAD ? DVS : DK) * 4 : 0);
    static constexpr int NLQ = SZ_Q / 1024;
    static constexpr int NLV = SZ_V / 1024;
    static constexpr int NLOAD = (R::OUT ? 2 : 1) * NLQ + (R::GRAD ? 2 : 1) * NLV;
    static_assert(R::OUT || !R::GRAD, "state-only roles carry no gradient tiles");
    static_assert(!R::NG || (R::OUT && !R::GRAD && !R::REV), "the epilogue belongs to the forward");
    static_assert(CT == 32 || CT == 64, "CT");
    static_assert(DK % 32 == 0 && DK <= (R::GRAD ? 192 : 96), "DK");
    static_assert(SZ_Q % 1024 == 0 && SZ_V % 1024 == 0, "load blocks");
    static_assert(NLOAD <= 63, "vmcnt");
    static_assert(!R::NG || NLOAD + 2 * NLV <= 63, "vmcnt");
    static_assert(LDS <= 160 * 1024, "LDS");
};

// Packed sequences are taken longest first, so that the long ones do not
// start behind a queue of short ones and finish last: position pos (in block
// order) runs the sequence of rank pos by length, descending, ties by index.
// The ranks are a permutation, so every sequence is still run exactly once.
// Every thread of the workgroup calls this before the waves take their roles
// (smem is free then); above LPT_MAX sequences the packed order is kept.
constexpr int LPT_MAX = 256;
__device__ __forceinline__ int longest_first(const Args& p, int pos, char* smem)
{
    const int ns = p.n_units / p.H;
    if (ns <= 1 || ns > LPT_MAX) return pos;
    int* lens = reinterpret_cast<int*>(smem);
    int* pick = lens + LPT_MAX;
    const int tid = threadIdx.x;
    for (int i = tid; i < ns; i += NTHREADS_W) {
        const int s0 = min(max(p.cu[i], 0), p.T);
        const int s1 = min(max(p.cu[i + 1], s0), p.T);
        lens[i] = s1 - s0;
    }
    __syncthreads();
    for (int i = tid; i < ns; i += NTHREADS_W) {
        const int li = lens[i];
        int r = 0;
        for (int j = 0; j < ns; ++j) {
            const int lj = lens[j];
            r += (lj > li || (lj == li && j < i)) ? 1 : 0;
        }
        if (r == pos) *pick = i;
    }
    __syncthreads();
    const int seq = *pick;
    __syncthreads();
    return seq;
}

// Returns the number of tiles of the unit. NG roles: grp is the unit's group
// (the workgroups of its slices) and tseq0 the number of tiles the group has
// run before this unit, which numbers the exchange's tags.
template <class R>
__device__ __forceinline__ int body_wide(const Args& p, int unit, int slice, char* smem, int grp = 0,
                                         int tseq0 = 0)
{
    typedef LayW<R> Ly;
    constexpr int DK = R::DK, CT = R::CT;
    constexpr int SEGK = Ly::SEGK, SEGV = Ly::SEGV;
    constexpr int NTB = Ly::NTB, NKT = Ly::NKT, NPB = Ly::NPB;
    constexpr int E = R::E;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int H = p.H;
    int seq = unit / H;
    const int h = unit - seq * H;
    // (the state-only roles serve dense segments only: no reordering there)
    if constexpr (R::OUT) {
        if (p.cu != nullptr) seq = longest_first(p, seq, smem);
    }
    int g = 0;                     // segment
    if (p.nseg > 1) {
        g = p.seg_first + seq % p.seg_count;
        seq /= p.seg_count;
    }
    const int dkr = p.dkr, dvr = p.dvr;
    const int n0 = slice * DVS;

    long row0;
    long trow0;                    // token-major row of the run's first token (NG)
    int len;
    if (p.cu != nullptr) {
        int s0 = p.cu[seq], s1 = p.cu[seq + 1];
        s0 = min(max(s0, 0), p.T);
        s1 = min(max(s1, s0), p.T);
        row0 = (long)h * p.T + s0;
        trow0 = s0;
        len = s1 - s0;
    } else {
        row0 = ((long)seq * H + h) * p.T;
        trow0 = (long)seq * p.T;
        len = p.T;
        if (p.nseg > 1) {
            row0 += (long)g * p.seg_len;
            len = min(p.seg_len, p.T - g * p.seg_len);
        }
    }
    auto grow = [&](int c, int r) -> long { return R::REV ? row0 + len - 1 - (c * CT + r) : row0 + c * CT + r; };
    const int nch = (len + CT - 1) / CT;
    const int clast = len - (nch - 1) * CT;
    const float lam = p.lambda[h];
    const float l2 = log2f(lam);

    // The update's operand pair per token (row 0: full tiles, row 1: the last
    // tile of clast tokens): B_j = corr[j] v'_j and A_j = v'_j masked by the
    // 16-bit half of keep[j / 2] (all ones when v'_j enters exactly).
    float* corr = reinterpret_cast<float*>(smem + Ly::OFF_CORR);
    uint32_t* keep = reinterpret_cast<uint32_t*>(smem + Ly::OFF_KEEP);
    for (int i = tid; i < 2 * CT; i += NTHREADS_W) {
        const int cl = (i < CT) ? CT : clast;
        const int j = i & (CT - 1);
        const float d = powl2(cl - E - j, l2);
        // NG: the decay itself (the update takes lam^m v'_j as a hi + lo pair)
        corr[i] = (j >= cl) ? 0.0f : (R::NG ? d : (d >= 0.5f ? -(1.0f - d) : d));
    }
    for (int i = tid; i < CT; i += NTHREADS_W) {
        const int cl = (i < CT / 2) ? CT : clast;
        const int j0 = 2 * (i & (CT / 2 - 1));
        const bool k0 = j0 < cl && powl2(cl - E - j0, l2) >= 0.5f;
        const bool k1 = j0 + 1 < cl && powl2(cl - E - j0 - 1, l2) >= 0.5f;
        keep[i] = (k0 ? 0x0000ffffu : 0u) | (k1 ? 0xffff0000u : 0u);
    }
    if constexpr (R::GRAD) {
        float* at = reinterpret_cast<float*>(smem + Ly::OFF_A);
        for (int i = tid; i < DVS; i += NTHREADS_W)
            at[i] = (p.a != nullptr && n0 + i < dvr) ? p.a[(size_t)h * dvr + n0 + i] : 0.0f;
    }
    if constexpr (R::OUT) {
        constexpr int NAB = R::GRAD ? DVS : DK;
        auto aval = [&](int i) -> float {
            if (p.a == nullptr) return 0.0f;
            if constexpr (R::GRAD) return n0 + i < dvr ? p.a[(size_t)h * dvr + n0 + i] : 0.0f;
            else return i < dkr ? p.a[(size_t)h * dkr + i] : 0.0f;
        };
        float* ab = reinterpret_cast<float*>(smem + Ly::OFF_AB);
        for (int i = tid; i < NAB; i += NTHREADS_W) {
            const float a0 = aval(i & ~1), a1 = aval(i | 1);
            ab[i] = 0.5f * ((i & 1) ? a0 - a1 : a0 + a1);
        }
    }
    float* gtb = reinterpret_cast<float*>(smem + Ly::OFF_GT);
    float* dgb = reinterpret_cast<float*>(smem + Ly::OFF_DG);
    // sigmoid(z_t) of tile c, z_t = sum_i a_i x_{t,i} y_{t,i}, in fp32 with a in
    // fp32 (bf16 operands for a and a (.) x would cost 2^-9 of each term,
    // coherently over the channels, which shows in the gate terms of the
    // gradients once |a| grows past ~1), by the loader's wave with lane =
    // token: the q'/k' rows for FWD, DV and NG, the x/v' rows (the 96-wide
    // slice) for DQ and DK. A channel pair (i, i+1) costs two bf16 dot
    // products, S = x_i y_i + x_{i+1} y_{i+1} and D = x_i y_i - x_{i+1} y_{i+1}
    // (exact products, one fp32 sum), and two fma:
    // a_i x_i y_i + a_{i+1} x_{i+1} y_{i+1} = alpha S + beta D with alpha, beta
    // = (a_i +- a_{i+1}) / 2 from the pair table. All row reads are issued
    // first, and four partial sums break the chain.
    constexpr int GSEG = R::GRAD ? SEGV : SEGK;
    auto gate_valu = [&](int c) {
        const char* st = smem + (c % Ly::NR) * Ly::SLOT;
        const char* Xs = R::GRAD ? st + Ly::OFF_X : st;
        const char* Ys = R::GRAD ? st + Ly::OFF_V : st + Ly::OFF_K;
        const float* ab = reinterpret_cast<const float*>(smem + Ly::OFF_AB);
        if (lane < CT) {
            u32x4_t xw[GSEG], yw[GSEG];
#pragma unroll
            for (int sg = 0; sg < GSEG; ++sg) {
                xw[sg] = *reinterpret_cast<const u32x4_t*>(Xs + toff<GSEG>(lane, 8 * sg));
                yw[sg] = *reinterpret_cast<const u32x4_t*>(Ys + toff<GSEG>(lane, 8 * sg));
            }
            float zp[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int sg = 0; sg < GSEG; ++sg) {
                const f32x4_t w0 = *reinterpret_cast<const f32x4_t*>(ab + 8 * sg);
                const f32x4_t w1 = *reinterpret_cast<const f32x4_t*>(ab + 8 * sg + 4);
                float S[4], D[4];
                dot2_sd4(xw[sg], yw[sg], S, D);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float al = (e < 2) ? w0[2 * e] : w1[2 * e - 4];
                    const float be = (e < 2) ? w0[2 * e + 1] : w1[2 * e - 3];
                    zp[e] = fmaf(al, S[e], zp[e]);
                    zp[e] = fmaf(be, D[e], zp[e]);
                }
            }
            // NG: token order (its scorer adds the gate); the others: token t at
            // (t % 16) NTB + t / 16, read by the owners in one access
            const int gi = R::NG ? lane : (lane & 15) * NTB + (lane >> 4);
            gtb[(c & 1) * CT + gi] = sigmoid_f((zp[0] + zp[1]) + (zp[2] + zp[3]));
        }
    };

    if (wave == LOADER_W) {
        // ---------------------------------------------------------- loader
        uint32_t offq[Ly::NLQ], offv[Ly::NLV];
        auto offsets = [&](int cl) {
#pragma unroll
            for (int m = 0; m < Ly::NLQ; ++m) {
                const int P = 64 * m + lane;
                const int r = P / SEGK;
                const int cs = (P - r * SEGK) ^ sw<SEGK>(r);
                const int rr = R::REV ? cl - 1 - min(r, cl - 1) : min(r, cl - 1);
                offq[m] = (uint32_t)(rr * dkr + min(8 * cs, dkr - 8)) * 2u;
            }
#pragma unroll
            for (int m = 0; m < Ly::NLV; ++m) {
                const int P = 64 * m + lane;
                const int r = P / SEGV;
                const int cs = (P - r * SEGV) ^ sw<SEGV>(r);
                const int rr = R::REV ? cl - 1 - min(r, cl - 1) : min(r, cl - 1);
                offv[m] = (uint32_t)(rr * dvr + min(n0 + 8 * cs, dvr - 8)) * 2u;
            }
        };
        offsets(nch > 1 ? CT : clast);
        auto issue = [&](int c) {
            char* st = smem + (c % Ly::NR) * Ly::SLOT;
            const int cl = min(CT, len - c * CT);
            if (c == nch - 1 && clast < CT) offsets(clast);
            const long rb = R::REV ? grow(c, cl - 1) : grow(c, 0);
            const char* qb = R::OUT ? reinterpret_cast<const char*>(p.q + rb * dkr) : nullptr;
            const char* kb = reinterpret_cast<const char*>(p.k + rb * dkr);
            const char* vb = reinterpret_cast<const char*>(p.v + rb * dvr);
            // The forward scans read every tile once, so their tiles stream
            // past the caches with the non-temporal hint, except the forward's
            // q' and k': its value slices read those too, at slightly different
            // times, and with the hint the second reader misses in L2. The
            // backward's roles read the same tiles at different times and keep
            // the default policy throughout.
            constexpr int POL = (!R::GRAD && !R::REV) ? POL_NT : 0;
            constexpr int POLQK = (R::OUT && !R::NG) ? 0 : POL;
#pragma unroll
            for (int m = 0; m < Ly::NLQ; ++m) {
                if constexpr (R::OUT) dma16<POLQK>(qb, offq[m], st + 1024 * m);
                dma16<POLQK>(kb, offq[m], st + Ly::OFF_K + 1024 * m);
            }
#pragma unroll
            for (int m = 0; m < Ly::NLV; ++m) dma16<POL>(vb, offv[m], st + Ly::OFF_V + 1024 * m);
            if constexpr (R::GRAD) {
                const char* xb = reinterpret_cast<const char*>(p.x + rb * dvr);
#pragma unroll
                for (int m = 0; m < Ly::NLV; ++m) dma16(xb, offv[m], st + Ly::OFF_X + 1024 * m);
            }
        };
        auto fixup = [&](int c) {
            const int cl = min(CT, len - c * CT);
            if (cl == CT && dkr == DK && n0 + DVS <= dvr) return;
            char* st = smem + (c % Ly::NR) * Ly::SLOT;
            const u32x4_t zero = {0u, 0u, 0u, 0u};
            for (int P = lane; P < CT * SEGK; P += 64) {
                const int r = P / SEGK;
                const int cs = (P - r * SEGK) ^ sw<SEGK>(r);
                if (r >= cl || 8 * cs >= dkr) {
                    *reinterpret_cast<u32x4_t*>(st + 16 * P) = zero;
                    *reinterpret_cast<u32x4_t*>(st + Ly::OFF_K + 16 * P) = zero;
                }
            }
            for (int P = lane; P < CT * SEGV; P += 64) {
                const int r = P / SEGV;
                const int cs = (P - r * SEGV) ^ sw<SEGV>(r);
                if (r >= cl || n0 + 8 * cs >= dvr) {
                    *reinterpret_cast<u32x4_t*>(st + Ly::OFF_V + 16 * P) = zero;
                    if constexpr (R::GRAD) *reinterpret_cast<u32x4_t*>(st + Ly::OFF_X + 16 * P) = zero;
                }
            }
        };
        if constexpr (R::NG) {
            // Three-deep ring. In iteration c the loader issues tile c+2,
            // waits for tile c+1 and forms its gate sigmoid(z) (cnt[2] = c+2
            // tells the scorer), issues the gate values g of tile c+1, then
            // waits for g of tile c, which the owners read in iteration c+1.
            constexpr int NLG = Ly::NLV;
            uint32_t offg[NLG];
            auto offsets_g = [&](int cl) {
#pragma unroll
                for (int m = 0; m < NLG; ++m) {
                    const int P = 64 * m + lane;
                    const int r = P / SEGV;
                    const int cs = (P - r * SEGV) ^ sw<SEGV>(r);
                    offg[m] = (uint32_t)(min(r, cl - 1) * H * dvr + min(n0 + 8 * cs, dvr - 8)) * 2u;
                }
            };
            offsets_g(nch > 1 ? CT : clast);
            auto issue_g = [&](int c) {
                if (c == nch - 1 && clast < CT) offsets_g(clast);
                const char* gb = reinterpret_cast<const char*>(p.ng_g + ((size_t)(trow0 + c * CT) * H + h) * dvr);
                char* dst = smem + Ly::OFF_G + (c % 3) * Ly::SZ_V;
#pragma unroll
                for (int m = 0; m < NLG; ++m) dma16<POL_NT>(gb, offg[m], dst + 1024 * m);
            };
            int* cnt = reinterpret_cast<int*>(smem + Ly::OFF_CNT);
            if (nch > 0) {
                issue(0);
                if (nch > 1) issue(1);
                issue_g(0);
                if (nch > 1) wait_vm<Ly::NLOAD + NLG>();
                else wait_vm<NLG>();
                fixup(0);
                gate_valu(0);
            }
            lds_barrier();
            lds_barrier();
            for (int c = 0; c < nch; ++c) {
                const bool n1 = c + 1 < nch, n2 = c + 2 < nch;
                if (n2) issue(c + 2);
                if (n1) {
                    // tile c+1: younger are g of tile c and tile c+2
                    if (n2) wait_vm<NLG + Ly::NLOAD>();
                    else wait_vm<NLG>();
                    fixup(c + 1);
                    gate_valu(c + 1);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    if (lane == 0)
                        __hip_atomic_store(cnt + 2, c + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    issue_g(c + 1);
                }
                // g of tile c: younger are tile c+2 and g of tile c+1
                if (n2) wait_vm<NLG + Ly::NLOAD>();
                else if (n1) wait_vm<NLG>();
                else wait_vm<0>();
                lds_barrier();
            }
            if (nch > 0) lds_barrier();     // the owners finish the last tile
            return nch;
        }
        if (nch > 0) {
            issue(0);
            if (nch > 1) {
                issue(1);
                wait_vm<Ly::NLOAD>();
            } else {
                wait_vm<0>();
            }
            fixup(0);
            if constexpr (R::OUT) gate_valu(0);
            if (nch > 1) {
                if (nch > 2) {
                    issue(2);
                    wait_vm<Ly::NLOAD>();
                } else {
                    wait_vm<0>();
                }
                fixup(1);
            }
        }
        lds_barrier();
        lds_barrier();
        // Iteration c: issue tile c+3, form the gate of tile c+1 (the owners'
        // tile of the next iteration; it arrived an iteration ago) while the
        // loads fly, then wait for tile c+2.
        for (int c = 0; c < nch; ++c) {
            if (c + 3 < nch) issue(c + 3);
            if constexpr (R::OUT) {
                if (c + 1 < nch) gate_valu(c + 1);
            }
            if (c + 2 < nch) {
                if (c + 3 < nch) wait_vm<Ly::NLOAD>();
                else wait_vm<0>();
                fixup(c + 2);
            }
            lds_barrier();
        }
        return nch;
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
            const char* st = smem + (c % Ly::NR) * Ly::SLOT;
            const char* Qs = st;
            const char* Ks = st + Ly::OFF_K;
            char* Pb = smem + Ly::OFF_P + (c & 1) * Ly::SZ_P;
#pragma unroll
            for (int s = 0; s < NKT; ++s) {
                bf16x8_t qf[DK / 16];
#pragma unroll
                for (int kb = 0; kb < DK / 16; ++kb)
                    qf[kb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                              Qs + toff<SEGK>(32 * s + l32, 16 * kb + 8 * g)));
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
                        // the raw diagonal q'_t . k'_t, which P leaves out: the owners
                        // add it in fp32 (with the gate for FWD and DV), and DQ and DK
                        // form c_t = sigmoid'(z_t) (q'_t . k'_t) from it
                        float u = 0.0f;
#pragma unroll
                        for (int i = 0; i < 16; ++i) u = fmaf(dsel[i], sc[i], u);
                        u += __shfl_xor(u, 32);
                        if (g == 0) {
                            // token t at (t % 16) NTB + t / 16: an owner lane reads its
                            // tokens' values in one access
                            const int t = 32 * s + l32;
                            dgb[(c & 1) * CT + (t & 15) * NTB + (t >> 4)] = u;
                        }
                    }
                    char* blk = Pb + pblk(tb, jb) * 1024;
#pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4) {
                        const int i0 = 4 * a4;
                        // the diagonal block's mask without the diagonal (there dmd is 1)
                        const float m0 = (jb == s) ? dmd[i0] - dsel[i0] : dmo[i0];
                        const float m1 = (jb == s) ? dmd[i0 + 1] - dsel[i0 + 1] : dmo[i0 + 1];
                        const float m2 = (jb == s) ? dmd[i0 + 2] - dsel[i0 + 2] : dmo[i0 + 2];
                        const float m3 = (jb == s) ? dmd[i0 + 3] - dsel[i0 + 3] : dmo[i0 + 3];
                        const u32x2_t w2 = {pack2(sc[i0] * m0, sc[i0 + 1] * m1), pack2(sc[i0 + 2] * m2, sc[i0 + 3] * m3)};
                        *reinterpret_cast<u32x2_t*>(blk + ((l32 & 15) + 16 * a4) * 16 + 8 * g) = w2;
                    }
                }
            }
        };
        // NG: the scores of tile c as a bf16 hi + lo pair in the one P buffer.
        // They are formed in fp32 first (masked; the gate enters the
        // diagonal afterwards); ready() returns once the owners no longer
        // read the buffer (they have finished tile c-1's output).
        auto scores_ng = [&](int c, auto ready) {
            const char* st = smem + (c % Ly::NR) * Ly::SLOT;
            const char* Qs = st;
            const char* Ks = st + Ly::OFF_K;
            char* Ph = smem + Ly::OFF_P;
            char* Pl = Ph + Ly::SZ_P;
            f32x16_t acc[NKT * (NKT + 1) / 2];
#pragma unroll
            for (int s = 0; s < NKT; ++s) {
                bf16x8_t qf[DK / 16];
#pragma unroll
                for (int kb = 0; kb < DK / 16; ++kb)
                    qf[kb] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                              Qs + toff<SEGK>(32 * s + l32, 16 * kb + 8 * g)));
#pragma unroll
                for (int jb = 0; jb <= s; ++jb) {
                    f32x16_t sc = {};
#pragma unroll
                    for (int kb = 0; kb < DK / 16; ++kb) {
                        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                                             Ks + toff<SEGK>(32 * jb + l32, 16 * kb + 8 * g)));
                        sc = mma(kf, qf[kb], sc);
                    }
#pragma unroll
                    for (int i = 0; i < 16; ++i) sc[i] *= (jb == s) ? dmd[i] : dmo[i];
                    acc[s * (s + 1) / 2 + jb] = sc;
                }
            }
            ready();
            // the gate on the diagonal (where the mask is 1)
#pragma unroll
            for (int s = 0; s < NKT; ++s) {
                const float gt = gtb[(c & 1) * CT + 32 * s + l32];
                f32x16_t& sc = acc[s * (s + 1) / 2 + s];
#pragma unroll
                for (int i = 0; i < 16; ++i) sc[i] = fmaf(dsel[i], gt, sc[i]);
            }
#pragma unroll
            for (int s = 0; s < NKT; ++s) {
                const int tb = 2 * s + (l32 >> 4);
#pragma unroll
                for (int jb = 0; jb <= s; ++jb) {
                    const f32x16_t& sc = acc[s * (s + 1) / 2 + jb];
#pragma unroll
                    for (int a4 = 0; a4 < 4; ++a4) {
                        const int i0 = 4 * a4;
                        const u32x2_t hw = {pack2(sc[i0], sc[i0 + 1]), pack2(sc[i0 + 2], sc[i0 + 3])};
                        const u32x2_t lw = {pack2(sc[i0] - bf_lo(hw[0]), sc[i0 + 1] - bf_hi(hw[0])),
                                            pack2(sc[i0 + 2] - bf_lo(hw[1]), sc[i0 + 3] - bf_hi(hw[1]))};
                        const int off = pblk(tb, jb) * 1024 + ((l32 & 15) + 16 * a4) * 16 + 8 * g;
                        *reinterpret_cast<u32x2_t*>(Ph + off) = hw;
                        *reinterpret_cast<u32x2_t*>(Pl + off) = lw;
                    }
                }
            }
        };
        lds_barrier();
        if constexpr (R::NG) {
            if (nch > 0) scores_ng(0, [] {});
        } else {
            if (R::OUT && nch > 0) scores(0);
        }
        lds_barrier();
        if constexpr (R::NG) {
            // The epilogue's statistic. In iteration c the scorer forms 1 / rms
            // of tile c-1 from its own sum and the other slice's, published an
            // iteration earlier (combine), then adds the six owners' sums of
            // o^2 of tile c and publishes them (publish); the owners store
            // tile c-1 once its 1 / rms is in LDS. Lane t handles token t.
            // The loader's gate is in gtb once cnt[2] says so.
            const float* ssb = reinterpret_cast<const float*>(smem + Ly::OFF_SS);
            float* invb = reinterpret_cast<float*>(smem + Ly::OFF_INV);
            int* cnt = reinterpret_cast<int*>(smem + Ly::OFF_CNT);
            unsigned long long* xg = p.xch + (size_t)grp * p.nsl * NG_XR * CT;
            float mine[2] = {0.0f, 0.0f};
            bool gave_up = false;
            auto publish = [&](int c) {
                const int ts = tseq0 + c;
                while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < NOW_W * (ts + 1))
                    __builtin_amdgcn_s_sleep(1);
                float part = 0.0f;
                if (lane < CT) {
#pragma unroll
                    for (int w2 = 0; w2 < NOW_W; ++w2) part += ssb[w2 * CT + lane];
                }
                mine[c & 1] = part;
                if (p.nsl > 1 && lane < CT) {
                    const unsigned long long word =
                        ((unsigned long long)(unsigned)(ts + 1) << 32) | __float_as_uint(part);
                    __hip_atomic_store(xg + ((size_t)slice * NG_XR + (ts & (NG_XR - 1))) * CT + lane, word,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            };
            auto combine = [&](int c) {
                const int ts = tseq0 + c;
                const unsigned want = (unsigned)(ts + 1);
                float tot = 0.0f;
                bool bad = gave_up;
                for (int s2 = 0; s2 < p.nsl; ++s2) {
                    if (s2 == slice) {
                        tot += mine[c & 1];
                        continue;
                    }
                    unsigned long long* slot = xg + ((size_t)s2 * NG_XR + (ts & (NG_XR - 1))) * CT + lane;
                    unsigned long long wv = (unsigned long long)want << 32;
                    for (int tries = 0; !bad; ++tries) {
                        if (lane < CT) wv = __hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (__all((unsigned)(wv >> 32) == want)) break;
                        if (tries >= NG_SPIN_MAX) {
                            bad = true;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                    }
                    if (!bad && lane < CT) {
                        // consumed: clear the word unless the next tag is already there
                        unsigned long long expect = wv;
                        __hip_atomic_compare_exchange_strong(slot, &expect, 0ull, __ATOMIC_RELAXED,
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                    tot += __uint_as_float((unsigned)wv);
                }
                gave_up = bad;
                if (bad && lane == 0) __hip_atomic_store(p.xerr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (lane < CT)
                    invb[lane] = bad ? __builtin_nanf("") : __builtin_amdgcn_rsqf(fmaf(tot, p.inv_dv, p.eps));
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (lane == 0) __hip_atomic_store(cnt + 1, ts + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            };
            for (int c = 0; c < nch; ++c) {
                // publish waits for the owners' sums of tile c, after which
                // they no longer read the P buffer
                // 1 / rms of tile c-1 first (the other slice published its
                // sums an iteration ago), so the owners never wait for it
                if (c > 0) combine(c - 1);
                if (c + 1 < nch) {
                    while (__hip_atomic_load(cnt + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < c + 2)
                        __builtin_amdgcn_s_sleep(1);
                    scores_ng(c + 1, [&] { publish(c); });
                } else {
                    publish(c);
                }
                lds_barrier();
            }
            if (nch > 0) {
                combine(nch - 1);
                lds_barrier();
            }
            return nch;
        }
        for (int c = 0; c < nch; ++c) {
            if (R::OUT && c + 1 < nch) scores(c + 1);
            lds_barrier();
        }
        return nch;
    }

    // -------------------------------------------------------------- owners
    constexpr int NDB16 = Ly::NDB16, NKS = Ly::NKS;
    const int w = wave;
    const int l16 = lane & 15, qg = lane >> 4;
    const int ncol = n0 + OWC * w + l16;       // this lane's v' column in the row
    // the state entering and leaving this unit's run of tokens
    const size_t ssz = (size_t)dkr * dvr;
    const size_t shead = ((size_t)seq * H + h) * ssz;
    const size_t sseg = (((size_t)seq * max(p.nseg, 1) + g) * H + h) * ssz;
    // a scan in time order enters the sequence at segment 0 and leaves it at
    // the last one; a reverse scan enters at the last and leaves at segment 0
    const bool last_seg = p.nseg <= 1 || g == p.nseg - 1;
    const bool enters_seq = R::REV ? last_seg : g == 0;
    const bool leaves_seq = R::REV ? g == 0 : last_seg;
    const float* s_in = (enters_seq && !p.seg_in_all) ? (p.s_init != nullptr ? p.s_init + shead : nullptr)
                                                      : (p.s_in_seg != nullptr ? p.s_in_seg + sseg : nullptr);
    float* s_out = leaves_seq ? (p.s_final != nullptr ? p.s_final + shead : nullptr)
                              : (p.s_out_seg != nullptr ? p.s_out_seg + sseg : nullptr);

    // Accumulator row 4 qg + r of 16-row block db holds state row srow(db, r)
    auto srow = [&](int db, int r) { return 32 * (db >> 1) + 8 * qg + 4 * (db & 1) + r; };
    f32x4_t sacc[NDB16];
#pragma unroll
    for (int db = 0; db < NDB16; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d = srow(db, r);
            const size_t si = R::INIT_T ? (size_t)ncol * dkr + d : (size_t)d * dvr + ncol;
            sacc[db][r] = (s_in != nullptr && d < dkr && ncol < dvr) ? s_in[si] : 0.0f;
        }
    float tdec[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) tdec[tb] = powl2(16 * tb + l16 + E, l2);
    const float fC = __builtin_amdgcn_exp2f((float)CT * l2);
    f32x4_t dpart = {0.f, 0.f, 0.f, 0.f};      // DA: column sums of c_t x_t (.) v'_t

    // NG: the output tile is stored one iteration late, once 1 / rms of its
    // tokens is known; prv holds it (fp32).
    const int ccol = n0 + OWC * w + 4 * qg;    // this lane's first output column
    f32x4_t gam = {1.f, 1.f, 1.f, 1.f};
    f32x4_t prv[NTB];
    if constexpr (R::NG) {
        if (p.ng_gamma != nullptr) {
            const float* gr = p.ng_gamma + (size_t)(h / p.per_tier) * dvr;
#pragma unroll
            for (int r = 0; r < 4; ++r) gam[r] = (ccol < dvr) ? gr[ccol + r] : 0.0f;
        }
    }
    // FULL: tile c has CT tokens and the slice d_v columns, so no store is
    // masked. (Guarded stores each sit in a branch, and at every join the
    // compiler waits for all outstanding memory operations.)
    auto ng_at = [&](int c, int t) -> size_t { return ((size_t)(trow0 + c * CT + t) * H + h) * dvr + ccol; };
    auto finish = [&](int c, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int* cnt = reinterpret_cast<const int*>(smem + Ly::OFF_CNT);
        const float* invb = reinterpret_cast<const float*>(smem + Ly::OFF_INV);
        while (__hip_atomic_load(cnt + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < tseq0 + c + 1)
            __builtin_amdgcn_s_sleep(1);
        const int cl = FULL ? CT : min(CT, len - c * CT);
        const char* gt_ = smem + Ly::OFF_G + (c % 3) * Ly::SZ_V;
        u32x2_t w2[NTB];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            const float inv = invb[16 * tb + l16];
            const u32x2_t gw = lds_u32x2(gt_, toff<SEGV>(16 * tb + l16, OWC * w + 4 * qg));
            const float gv[4] = {bf_lo(gw[0]), bf_hi(gw[0]), bf_lo(gw[1]), bf_hi(gw[1])};
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = silu_f(gv[r]) * (gam[r] * (prv[tb][r] * inv));
            w2[tb] = u32x2_t{pack2(y[0], y[1]), pack2(y[2], y[3])};
        }
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            const int t = 16 * tb + l16;
            if (FULL || (t < cl && ccol < dvr)) *reinterpret_cast<u32x2_t*>(p.ng_out + ng_at(c, t)) = w2[tb];
        }
    };

    auto tile = [&](int c, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        f32x4_t cur[NTB];
        const char* st = smem + (c % Ly::NR) * Ly::SLOT;
        const char* Qs = st;
        const char* Ks = st + Ly::OFF_K;
        const char* Vs = st + Ly::OFF_V;
        const char* Pb = smem + Ly::OFF_P + (R::NG ? 0 : (c & 1) * Ly::SZ_P);
        const int cstart = c * CT;
        const int cl = FULL ? CT : min(CT, len - cstart);
        const bool last_row = !FULL && c == nch - 1;
        const float* cf = corr + (last_row ? CT : 0);
        const uint32_t* kw = keep + (last_row ? CT / 2 : 0);
        const float fcl = FULL ? fC : __builtin_amdgcn_exp2f((float)cl * l2);

        // V'^T (A operand of P V') and V' (B operand of the update) share one
        // register layout: lane (column l16, step slice qg) holds tokens
        // 32 ks + 8 qg + 0..7
        bf16x8_t vf[NKT];
#pragma unroll
        for (int ks = 0; ks < NKT; ++ks)
            vf[ks] = frag(tr_read<SEGV>(Vs, 32 * ks + 8 * qg, OWC * w, lane),
                          tr_read<SEGV>(Vs, 32 * ks + 8 * qg + 4, OWC * w, lane));
        if constexpr (R::OUT) {
            bf16x8_t pf[NPB], pfl[R::NG ? NPB : 1];
#pragma unroll
            for (int b = 0; b < NPB; ++b)
                pf[b] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(Pb + (b * 64 + lane) * 16));
            if constexpr (R::NG) {
#pragma unroll
                for (int b = 0; b < NPB; ++b)
                    pfl[b] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                              Pb + Ly::SZ_P + (b * 64 + lane) * 16));
            }

            // the fp32 raw diagonal and the gate of this lane's tokens 16 tb + l16,
            // one access each
            float dgv[Ly::DIAG32 ? NTB : 1], gtv[Ly::DIAG32 ? NTB : 1];
            if constexpr (Ly::DIAG32) {
                const float* dgl = dgb + (c & 1) * CT + l16 * NTB;
                const float* gtl = gtb + (c & 1) * CT + l16 * NTB;
                if constexpr (NTB == 4) {
                    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(dgl);
                    const f32x4_t y = *reinterpret_cast<const f32x4_t*>(gtl);
#pragma unroll
                    for (int tb = 0; tb < NTB; ++tb) {
                        dgv[tb] = x[tb];
                        gtv[tb] = y[tb];
                    }
                } else {
#pragma unroll
                    for (int tb = 0; tb < NTB; ++tb) {
                        dgv[tb] = dgl[tb];
                        gtv[tb] = gtl[tb];
                    }
                }
            }

            // ---- readout: O^T = S^T Q'^T, the state as a bf16 pair: hi = the
            // truncated upper half, lo = the remainder (exact in fp32) rounded
            f32x4_t oq[NTB] = {};
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
                for (int tb = 0; tb < NTB; ++tb) {
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
            f32x4_t acol = {0.f, 0.f, 0.f, 0.f};
            if constexpr (R::GRAD) acol = *reinterpret_cast<const f32x4_t*>(smem + Ly::OFF_A + 4 * (OWC * w + 4 * qg));
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                f32x4_t o = {};
#pragma unroll
                for (int ks = 0; ks <= (tb >> 1); ++ks) {
                    o = mma16(vf[ks], pf[pblk(tb, ks)], o);
                    if constexpr (R::NG) o = mma16(vf[ks], pfl[pblk(tb, ks)], o);
                }
                const int t = 16 * tb + l16;
                float val[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) val[r] = fmaf(tdec[tb], oq[tb][r], o[r]);
                float y[4] = {0.f, 0.f, 0.f, 0.f};
                if constexpr (Ly::DIAG32) {
                    // + the diagonal term in fp32: the raw diagonal (plus the gate
                    // for FWD and DV) times v'_t
                    const u32x2_t yw = lds_u32x2(Vs, toff<SEGV>(t, OWC * w + 4 * qg));
                    y[0] = bf_lo(yw[0]);
                    y[1] = bf_hi(yw[0]);
                    y[2] = bf_lo(yw[1]);
                    y[3] = bf_hi(yw[1]);
                    const float dgt = R::GRAD ? dgv[tb] : dgv[tb] + gtv[tb];
#pragma unroll
                    for (int r = 0; r < 4; ++r) val[r] = fmaf(dgt, y[r], val[r]);
                }
                if constexpr (R::GRAD) {
                    // + c_t a (.) v'_t with c_t = sigmoid'(z_t) (q'_t . k'_t); DA:
                    // column sums of c_t x_t (.) v'_t
                    const float ct = gtv[tb] * (1.0f - gtv[tb]) * dgv[tb];
                    float xv[4] = {0.f, 0.f, 0.f, 0.f};
                    if constexpr (R::DA) {
                        const u32x2_t xw = lds_u32x2(st + Ly::OFF_X, toff<SEGV>(t, OWC * w + 4 * qg));
                        xv[0] = bf_lo(xw[0]);
                        xv[1] = bf_hi(xw[0]);
                        xv[2] = bf_lo(xw[1]);
                        xv[3] = bf_hi(xw[1]);
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float cy = ct * y[r];
                        val[r] = fmaf(cy, acol[r], val[r]);
                        if constexpr (R::DA) dpart[r] = fmaf(cy, xv[r], dpart[r]);
                    }
                }
                if (!R::NG || p.o != nullptr) {
                    if (FULL || t < cl) {
                        const int col = n0 + OWC * w + 4 * qg;
                        if (FULL || col < dvr) {
                            uint16_t* orow = p.o + grow(c, t) * dvr + col;
                            const u32x2_t w2 = {pack2(val[0], val[1]), pack2(val[2], val[3])};
                            *reinterpret_cast<u32x2_t*>(orow) = w2;
                        }
                    }
                }
                if constexpr (R::NG) {
                    // this owner's sum of o^2 over its 16 columns, per token
                    float x = val[0] * val[0];
#pragma unroll
                    for (int r = 1; r < 4; ++r) x = fmaf(val[r], val[r], x);
                    x += __shfl_xor(x, 16);
                    x += __shfl_xor(x, 32);
                    if (qg == 0) reinterpret_cast<float*>(smem + Ly::OFF_SS)[w * CT + t] = x;
                    cur[tb] = f32x4_t{val[0], val[1], val[2], val[3]};
                }
            }
            if constexpr (R::NG) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (lane == 0)
                    __hip_atomic_fetch_add(reinterpret_cast<int*>(smem + Ly::OFF_CNT), 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        } else {
#pragma unroll
            for (int db = 0; db < NDB16; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) sacc[db][r] *= fcl;
        }

        // ---- state advance: S = lam^cl S + K'^T A + K'^T B (the operand
        // pair of the decayed values, see the top of this file)
        bf16x8_t va[NKT], vc[NKT];
#pragma unroll
        for (int ks = 0; ks < NKT; ++ks) {
            const f32x4_t c0 = *reinterpret_cast<const f32x4_t*>(cf + 32 * ks + 8 * qg);
            const f32x4_t c1 = *reinterpret_cast<const f32x4_t*>(cf + 32 * ks + 8 * qg + 4);
            const u32x4_t vw = __builtin_bit_cast(u32x4_t, vf[ks]);
            if constexpr (R::NG) {
                // lam^m v'_j as a bf16 hi + lo pair
                const float x[8] = {c0[0] * bf_lo(vw[0]), c0[1] * bf_hi(vw[0]), c0[2] * bf_lo(vw[1]),
                                    c0[3] * bf_hi(vw[1]), c1[0] * bf_lo(vw[2]), c1[1] * bf_hi(vw[2]),
                                    c1[2] * bf_lo(vw[3]), c1[3] * bf_hi(vw[3])};
                u32x4_t hw, lw;
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) {
                    hw[s2] = pack2(x[2 * s2], x[2 * s2 + 1]);
                    lw[s2] = pack2(x[2 * s2] - bf_lo(hw[s2]), x[2 * s2 + 1] - bf_hi(hw[s2]));
                }
                va[ks] = __builtin_bit_cast(bf16x8_t, hw);
                vc[ks] = __builtin_bit_cast(bf16x8_t, lw);
            } else {
                const u32x4_t km = *reinterpret_cast<const u32x4_t*>(kw + 16 * ks + 4 * qg);
                u32x4_t cw;
                cw[0] = pack2(c0[0] * bf_lo(vw[0]), c0[1] * bf_hi(vw[0]));
                cw[1] = pack2(c0[2] * bf_lo(vw[1]), c0[3] * bf_hi(vw[1]));
                cw[2] = pack2(c1[0] * bf_lo(vw[2]), c1[1] * bf_hi(vw[2]));
                cw[3] = pack2(c1[2] * bf_lo(vw[3]), c1[3] * bf_hi(vw[3]));
                vc[ks] = __builtin_bit_cast(bf16x8_t, cw);
                va[ks] = __builtin_bit_cast(bf16x8_t, vw & km);
            }
        }
#pragma unroll
        for (int db = 0; db < NDB16; ++db)
#pragma unroll
            for (int ks = 0; ks < NKT; ++ks) {
                // K'^T: row l16 of block db (key column srow with qg -> l16 / 4,
                // r -> l16 % 4), tokens 32 ks + 8 qg + 0..7
                const int kc0 = 32 * (db >> 1) + 4 * (db & 1);
                const bf16x8_t kf = frag(tr_read8<SEGK>(Ks, 32 * ks + 8 * qg, kc0, lane),
                                         tr_read8<SEGK>(Ks, 32 * ks + 8 * qg + 4, kc0, lane));
                sacc[db] = mma16(kf, va[ks], sacc[db]);
                sacc[db] = mma16(kf, vc[ks], sacc[db]);
            }
        if constexpr (R::NG) {
            // tile c-1 is full when tile c is
            if (c > 0) finish(c - 1, full_tag);
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) prv[tb] = cur[tb];
        }
    };

    const bool cols_full = (n0 + DVS <= dvr);
    lds_barrier();
    lds_barrier();
    for (int c = 0; c < nch; ++c) {
        if (cols_full && (c < nch - 1 || clast == CT)) tile(c, std::true_type{});
        else tile(c, std::false_type{});
        lds_barrier();
    }
    if constexpr (R::NG) {
        if (nch > 0) {
            finish(nch - 1, std::false_type{});
            lds_barrier();
        }
    }

    // (the gradient scans of q and k end without a state output)
    if (!R::GRAD && s_out != nullptr && ncol < dvr) {
#pragma unroll
        for (int db = 0; db < NDB16; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = srow(db, r);
                if (d < dkr) s_out[(size_t)d * dvr + ncol] = sacc[db][r];
            }
    }
    if constexpr (R::DA) {
        // sum over the 16 token lanes of each lane group; lane l16 = 0 writes
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float x = dpart[r];
#pragma unroll
            for (int off = 8; off > 0; off >>= 1) x += __shfl_xor(x, off);
            dpart[r] = x;
        }
        if (l16 == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int col = n0 + OWC * w + 4 * qg + r;
                if (col < dvr) p.da_part[(size_t)unit * dvr + col] = dpart[r];
            }
        }
    }
    return nch;
}

// ----------------------------------------------------------------------------
// Segment scan of the states: a run of L tokens maps the state S entering it
// to lam^L S + S_loc, with S_loc the state it leaves from a zero start. With
// loc[n][g] the state leaving segment g (segment 0 from the true initial
// state, the others from zero), the state entering segment g >= 1 is
//   in[n][1] = loc[n][0],  in[n][g] = lam^L in[n][g-1] + loc[n][g-1],
// and with copy_init in[n][0] = the initial state itself.
// One thread per four state elements of one (sequence, head), in order over g.
static __global__ void k_seg_scan(const float* __restrict__ loc, float* __restrict__ in,
                           const float* __restrict__ lambda, int n_seq, int nseg, int H,
                           int ssz4, int seg_len, int copy_init, const float* __restrict__ init)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int nh = blockIdx.y;                 // n H + h
    if (i >= ssz4) return;
    const int n = nh / H, h = nh - n * H;
    const float fL = __builtin_amdgcn_exp2f((float)seg_len * log2f(lambda[h]));
    typedef float f4 __attribute__((ext_vector_type(4)));
    auto at = [&](int g) -> size_t { return (((size_t)n * nseg + g) * H + h) * (size_t)ssz4 + i; };
    if (copy_init) {
        // in[n][0] = the initial state [n][H][state] (zero when NULL)
        const f4 z = {0.f, 0.f, 0.f, 0.f};
        reinterpret_cast<f4*>(in)[at(0)] =
            init != nullptr ? reinterpret_cast<const f4*>(init)[((size_t)n * H + h) * (size_t)ssz4 + i] : z;
    }
    f4 s = reinterpret_cast<const f4*>(loc)[at(0)];
    reinterpret_cast<f4*>(in)[at(1)] = s;
    for (int g = 2; g < nseg; ++g) {
        const f4 l = reinterpret_cast<const f4*>(loc)[at(g - 1)];
        s = fL * s + l;
        reinterpret_cast<f4*>(in)[at(g)] = s;
    }
}

// Reverse scan of the state gradients over segments: with loc[n][g] the
// gradient state leaving segment g at its front (segment nseg-1 from
// d_final_state, the others from zero), the one entering segment g from the
// back is in[n][nseg-2] = loc[n][nseg-1], in[n][g] = lam^L in[n][g+1] + loc[n][g+1].
static __global__ void k_seg_rscan(const float* __restrict__ loc, float* __restrict__ in,
                            const float* __restrict__ lambda, int nseg, int H, int ssz4, int seg_len)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int nh = blockIdx.y;
    if (i >= ssz4) return;
    const int n = nh / H, h = nh - n * H;
    const float fL = __builtin_amdgcn_exp2f((float)seg_len * log2f(lambda[h]));
    typedef float f4 __attribute__((ext_vector_type(4)));
    auto at = [&](int g) -> size_t { return (((size_t)n * nseg + g) * H + h) * (size_t)ssz4 + i; };
    f4 s = reinterpret_cast<const f4*>(loc)[at(nseg - 1)];
    reinterpret_cast<f4*>(in)[at(nseg - 2)] = s;
    for (int g = nseg - 3; g >= 0; --g) {
        const f4 l = reinterpret_cast<const f4*>(loc)[at(g + 1)];
        s = fL * s + l;
        reinterpret_cast<f4*>(in)[at(g)] = s;
    }
}

}  // namespace scan
}  // namespace sgla

#endif
