// Chunked Simple GLA kernels for gfx950, fp32 tensors (forward and backward),
// and the dispatch of bf16 calls to the tile-scan kernels of sgla_fwd.hip and
// sgla_bwd.hip.
//
// Method: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
// attention model on AWS Trainium2 with native PyTorch", section "Challenge 1:
// Using native PyTorch on Trainium for GLA" (the chunked intra-chunk output
// and chunk state update). For a chunk of C_c tokens (rows i, j) entered with
// state S_in, and decay lam of the head:
//
//   o_i   = lam^(i+1) S_in^T q_i + sum_{j<=i} lam^(i-j) (q_i . k_j) v_j + aug_i
//   S_out = lam^(C_c) S_in + sum_j lam^(C_c-1-j) k_j v_j^T
//
// One "role" body below evaluates this recurrence for generic operands
// (q', k', v') and a generic per-token epilogue, optionally in reversed token
// order. The forward is the role (q, k, v). The backward is three independent
// roles that run concurrently in one launch:
//   dq: forward order,  q'=dO, k'=v, v'=k, state S^T, + sigmoid'(z)(dO.v)(a*k)
//   dk: reversed order, q'=v, k'=dO, v'=q, state G^T, + sigmoid'(z)(dO.v)(a*q)
//   dv: reversed order, q'=k, k'=q, v'=dO, state G,   + sigmoid(z) dO
// (G_t = dL/dS_t = sum_{i>=t} lam^(i-t) q_i dO_i^T + lam^(T-1-t) dS_final: in
// reversed order the carried-in dS_final enters the first token undecayed.)
//
// Work decomposition: one workgroup of 4 waves per (sequence, head, value
// slice); the state slice stays in MFMA accumulators for the whole scan over
// chunks. Per chunk the operands are staged in LDS:
//   Qs, Ks   [C][DK]   natural (rows = tokens)      -- scores, Q'S, (q'.k')
//   KTs      [DK][C]   k' transposed, unscaled      -- state update
//   VTs      [DVS][C]  v' slice transposed          -- P.V', state update, epilogue
//   STh      [DVS][DK] state^T                       -- Q'S
//   ksc      [C]       lam^(C_c-1-j), the key decays of the state update
// Waves 0..C/32-1 each own 32 query rows: they compute Q'S, the decay-masked
// score tiles K' Q'^T (kept in registers and fed straight back as the A
// operand of P.V'), the epilogue, and store. The state tiles are spread over
// the waves by a compile-time balance of the per-chunk matrix-core work.
//
// Precision: every operand and product is fp32 (v_mfma_f32_32x32x2_f32); the
// only roundings are those of fp32 arithmetic.
//
// MFMA: v_mfma_f32_32x32x2_f32 (one contraction step of 2 per instruction).
// For a 32x32 result, lane l holds column l%32 and rows 8*(i/4)+4*(l/32)+i%4
// in accumulator i. Operand lanes hold row (A) / column (B) l%32; lane group
// l/32 selects the slice of the contraction index. The pairing of contraction
// slots between A and B is lane-group- and slot-wise, so any assignment of
// contraction indices to (group, slot) works if A and B use the same one.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgla_internal.h"

namespace sgla {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int NTHREADS = 256;
constexpr int NWAVES = 4;

__device__ __forceinline__ float to_f(float x) { return x; }

template <typename E> __device__ __forceinline__ E from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }

// 2^x on the transcendental unit (v_exp_f32). Results below the smallest
// normal fp32 flush to zero; decays that small contribute nothing here.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// lam^m for an integer m >= 0 with lam^0 = 1 exactly (also for lam = 0).
__device__ __forceinline__ float decay_pow(int m, float log2lam)
{
    return (m == 0) ? 1.0f : fast_exp2((float)m * log2lam);
}

__device__ __forceinline__ float sigmoidf_(float z)
{
    if (z >= 0.0f) return 1.0f / (1.0f + expf(-z));
    float e = expf(z);
    return e / (1.0f + e);
}

// Element e of a 16-byte register vector holding E values, widened to fp32.
// (Bit operations on native vectors keep these registers out of memory.)
template <typename E> __device__ __forceinline__ float vget(const u32x4_t& v, int e);
template <> __device__ __forceinline__ float vget<float>(const u32x4_t& v, int e)
{
    return __uint_as_float(v[e]);
}

template <typename E> struct Mfma;
template <> struct Mfma<float> {
    static constexpr int KSTEP = 2;
    static constexpr int NE = 1;
    typedef float op_t;
    static __device__ __forceinline__ op_t load(const float* p) { return *p; }
    static __device__ __forceinline__ f32x16_t mma(op_t a, op_t b, f32x16_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// Workgroup barrier for LDS hand-offs. It waits only for this wave's LDS (and
// scalar) operations, not for its global loads: __syncthreads() would also
// drain vmcnt and so stall on the next chunk's prefetch it is meant to overlap.
// Every cross-wave exchange in these kernels goes through LDS.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Row (within a 32x32 tile) held by accumulator i of lane group g.
__device__ __forceinline__ int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

enum { AUG_FWD = 0, AUG_GRAD = 1 };

// Static assignment of state d-blocks (32 state rows x all value tiles of the
// slice) to waves: greedy on the per-chunk matrix-core instruction count,
// query-strip work first. Owning whole d-blocks lets one converted key
// operand of the state update feed every value tile of that block.
struct Owners {
    int count[NWAVES];
    int list[NWAVES][32];
    int max_count;
};

constexpr Owners balance(int nstrip, int strip_base, int per_block, int tile_cost, int ntiles)
{
    Owners o{};
    long load[NWAVES] = {0, 0, 0, 0};
    for (int w = 0; w < NWAVES; ++w) load[w] = (w < nstrip) ? strip_base + (w + 1) * per_block : 0;
    for (int t = 0; t < ntiles; ++t) {
        int best = 0;
        for (int w = 1; w < NWAVES; ++w)
            if (load[w] < load[best]) best = w;
        o.list[best][o.count[best]++] = t;
        load[best] += tile_cost;
    }
    o.max_count = 0;
    for (int w = 0; w < NWAVES; ++w)
        if (o.count[w] > o.max_count) o.max_count = o.count[w];
    return o;
}

// Compile-time description of one role.
//   DK:  padded width of q'/k' rows (= state rows), multiple of 32
//   DVS: padded width of the value slice a workgroup owns, multiple of 32
//   C:   chunk length (multiple of 32, <= 128)
template <typename E_, int DK_, int DVS_, int C_, int AUG_, bool REV_>
struct Role {
    typedef E_ E;
    typedef Mfma<E> M;
    static constexpr int DK = DK_, DVS = DVS_, C = C_, AUG = AUG_;
    static constexpr bool REV = REV_;
    static constexpr int PE = 16 / (int)sizeof(E);  // 16-byte row padding
    static constexpr int LDQ = DK + PE;             // Qs, Ks, STh row stride
    static constexpr int LDT = C + PE;              // KTs, VTs, XTs row stride
    static constexpr int NSTRIP = C / 32;
    static constexpr int NNT = DVS / 32;
    static constexpr int NDB = DK / 32;
    static constexpr int NTILES = NDB * NNT;
    static constexpr Owners OWN =
        balance(NSTRIP, (DK / M::KSTEP) * NNT, DK / M::KSTEP + NNT * (32 / M::KSTEP),
                NNT * (C / M::KSTEP), NDB);
    static constexpr int NDBW = OWN.max_count;  // d-blocks per wave (at most)
    static constexpr size_t SZ_ROWS = (size_t)C * LDQ * sizeof(E);
    static constexpr size_t SZ_ST = (size_t)DVS * LDQ * sizeof(E);
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t OFF_K = OFF_Q + SZ_ROWS;
    static constexpr size_t OFF_KT = OFF_K + SZ_ROWS;
    static constexpr size_t OFF_VT = OFF_KT + (size_t)DK * LDT * sizeof(E);
    static constexpr size_t OFF_STH = OFF_VT + (size_t)DVS * LDT * sizeof(E);
    static constexpr size_t OFF_XT = OFF_STH + SZ_ST;
    static constexpr size_t OFF_COEF = OFF_XT + (AUG == AUG_GRAD ? (size_t)DVS * LDT * sizeof(E) : 0);
    static constexpr size_t OFF_KSC = OFF_COEF + (size_t)C * sizeof(float);
    static constexpr int AWN = DK > 128 ? DK : 128;  // staged width of a
    static constexpr size_t OFF_A = OFF_KSC + (size_t)C * sizeof(float);
    static constexpr size_t OFF_DA = OFF_A + (size_t)AWN * sizeof(float);
    static constexpr size_t LDS = OFF_DA + (AUG == AUG_GRAD ? (size_t)NSTRIP * DVS * sizeof(float) : 0);
    static_assert(DK % 32 == 0 && DVS % 32 == 0 && C % 32 == 0 && C <= 128, "tile shape");
    static_assert(LDS <= 160 * 1024, "LDS budget");
    static_assert(NDB <= 32, "owner table");
};

// State d-block handled by a wave's kk-th accumulator group (or -1).
template <class R>
__device__ __forceinline__ int dblock_of(int wave, int kk)
{
    constexpr Owners o = R::OWN;
    switch (wave) {
    case 0: return kk < o.count[0] ? o.list[0][kk] : -1;
    case 1: return kk < o.count[1] ? o.list[1][kk] : -1;
    case 2: return kk < o.count[2] ? o.list[2][kk] : -1;
    default: return kk < o.count[3] ? o.list[3][kk] : -1;
    }
}

struct Common {
    const float* lambda;
    const float* a;      // [H, d_k] or NULL
    const int32_t* cu;   // NULL when dense
    int H, T, n_units;
};

struct RoleArgs {
    const void* qp;  // q' rows of width dkr
    const void* kp;  // k' rows of width dkr
    const void* vp;  // v' rows of width dvr
    const void* xp;  // AUG_GRAD: second operand of the gate, rows of width dvr
    void* op;        // output rows of width dvr
    const float* s_init;  // [units, ...] or NULL
    float* s_final;       // [units, ...] or NULL
    float* da_part;       // AUG_GRAD: [units, dvr] partial da, or NULL
    int dkr, dvr;         // real widths (<= DK, <= DVS * slices)
    int state_t;          // state stored [dvr][dkr] instead of [dkr][dvr]
    int final_times_lam;  // final state scaled by lam (non-empty sequences)
    int init_undecayed;   // the initial state enters the first token undecayed
};

template <class R>
__device__ __forceinline__ void role_body(const Common& cm, const RoleArgs& ra, int unit,
                                          int slice, char* smem)
{
    typedef typename R::E E;
    typedef typename R::M M;
    constexpr int C = R::C, DK = R::DK, DVS = R::DVS, LDQ = R::LDQ, LDT = R::LDT;
    constexpr int NSTRIP = R::NSTRIP, NNT = R::NNT, NDBW = R::NDBW;
    constexpr int KSTEP = M::KSTEP, NE = M::NE;
    constexpr int V16 = 16 / (int)sizeof(E);  // elements per 16-byte segment

    E* Qs = reinterpret_cast<E*>(smem + R::OFF_Q);
    E* Ks = reinterpret_cast<E*>(smem + R::OFF_K);
    E* KTs = reinterpret_cast<E*>(smem + R::OFF_KT);
    E* VTs = reinterpret_cast<E*>(smem + R::OFF_VT);
    E* STh = reinterpret_cast<E*>(smem + R::OFF_STH);
    E* XTs = reinterpret_cast<E*>(smem + R::OFF_XT);
    float* coef = reinterpret_cast<float*>(smem + R::OFF_COEF);
    float* ksc = reinterpret_cast<float*>(smem + R::OFF_KSC);
    float* dared = reinterpret_cast<float*>(smem + R::OFF_DA);
    float* a_lds = reinterpret_cast<float*>(smem + R::OFF_A);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, g = lane >> 5;

    const int H = cm.H;
    const int seq = unit / H, h = unit - seq * H;
    long row0;
    int len;
    if (cm.cu != nullptr) {
        int s0 = cm.cu[seq], s1 = cm.cu[seq + 1];
        s0 = min(max(s0, 0), cm.T);
        s1 = min(max(s1, s0), cm.T);
        row0 = (long)h * cm.T + s0;
        len = s1 - s0;
    } else {
        row0 = ((long)seq * H + h) * cm.T;
        len = cm.T;
    }
    const float lam = cm.lambda[h];
    const float l2 = log2f(lam);  // -inf for lam = 0
    const int n0 = slice * DVS;
    const int dkr = ra.dkr, dvr = ra.dvr;
    const size_t sbase = (size_t)unit * dkr * dvr;

    const E* gq = reinterpret_cast<const E*>(ra.qp);
    const E* gk = reinterpret_cast<const E*>(ra.kp);
    const E* gv = reinterpret_cast<const E*>(ra.vp);
    const E* gx = reinterpret_cast<const E*>(ra.xp);
    E* go = reinterpret_cast<E*>(ra.op);

    // ---- state slice in accumulators: d-block dbs[kk], value tile nb in
    // sacc[kk * NNT + nb]
    int dbs[NDBW];
    f32x16_t sacc[NDBW * NNT];
#pragma unroll
    for (int kk = 0; kk < NDBW; ++kk) {
        const int db = dblock_of<R>(wave, kk);
        dbs[kk] = db;
#pragma unroll
        for (int nb = 0; nb < NNT; ++nb) {
            f32x16_t& acc = sacc[kk * NNT + nb];
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
            if (db >= 0 && ra.s_init != nullptr) {
                const int nn = n0 + 32 * nb + l32;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int d = 32 * db + acc_row(i, g);
                    if (d < dkr && nn < dvr)
                        acc[i] = ra.state_t ? ra.s_init[sbase + (size_t)nn * dkr + d]
                                            : ra.s_init[sbase + (size_t)d * dvr + nn];
                }
            }
        }
    }

    float da_acc[NNT];
#pragma unroll
    for (int nt = 0; nt < NNT; ++nt) da_acc[nt] = 0.0f;

    // a (aug_balance) of this head, staged once; indexed by d (forward-type
    // roles) or by the value column (gradient roles), zero past the width
    {
        const int aw = (R::AUG == AUG_FWD) ? dkr : dvr;
        for (int i = tid; i < R::AWN; i += NTHREADS)
            a_lds[i] = (cm.a != nullptr && i < aw) ? cm.a[(size_t)h * aw + i] : 0.0f;
    }

    // ---- operand staging, software-pipelined: chunk ci+1 is read from HBM
    // into registers while chunk ci is computed out of LDS.
    constexpr bool GRAD = (R::AUG == AUG_GRAD);
    constexpr int SEGQ = DK / V16, SEGV = DVS / V16, RP = C / 2;
    constexpr int NBQ = (RP * SEGQ + NTHREADS - 1) / NTHREADS;
    constexpr int NBV = (RP * SEGV + NTHREADS - 1) / NTHREADS;
    static_assert(RP % 16 == 0 && SEGQ % 4 == 0 && SEGV % 4 == 0, "staging map");
    u32x4_t pq[NBQ][2], pk[NBQ][2], pv[NBV][2], px[GRAD ? NBV : 1][2];

    // Staging block b -> (row pair rp, 16-byte column segment cg). Sixteen
    // consecutive lanes take sixteen row pairs of one segment, so their
    // transposed LDS writes fall in distinct banks; four such lane groups take
    // four adjacent segments, i.e. 64 contiguous bytes of every row they read.
    auto block_rc = [](int b, int nseg, int& rp, int& cg) {
        const int rest = b >> 6;
        rp = (rest % (RP / 16)) * 16 + (b & 15);
        cg = (rest / (RP / 16)) * 4 + ((b >> 4) & 3);
        (void)nseg;
    };
    const int nchunks = (len + C - 1) / C;
    // The loads are unconditional, from clamped in-bounds addresses: a load
    // under a lane mask followed by a merge with zero would have to wait for
    // the data right away. Rows past the chunk and columns past the real
    // width are zeroed later, when store_chunk consumes the registers.
    auto load_chunk = [&](int cj) {
        const int cc = R::REV ? (nchunks - 1 - cj) : cj;
        const int cs = cc * C, cl = min(C, len - cs);
#pragma unroll
        for (int m = 0; m < NBQ; ++m) {
            const int b = tid + NTHREADS * m;
            int rp, cg;
            block_rc(b, SEGQ, rp, cg);
            const int col = min(cg * V16, dkr - V16);
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int r = min(2 * rp + rr, cl - 1);
                const int tok = R::REV ? (cs + cl - 1 - r) : (cs + r);
                const size_t off = (size_t)(row0 + tok) * dkr + col;
                pq[m][rr] = *reinterpret_cast<const u32x4_t*>(gq + off);
                pk[m][rr] = *reinterpret_cast<const u32x4_t*>(gk + off);
            }
        }
#pragma unroll
        for (int m = 0; m < NBV; ++m) {
            const int b = tid + NTHREADS * m;
            int rp, cg;
            block_rc(b, SEGV, rp, cg);
            const int gcol = min(n0 + cg * V16, dvr - V16);
#pragma unroll
            for (int rr = 0; rr < 2; ++rr) {
                const int r = min(2 * rp + rr, cl - 1);
                const int tok = R::REV ? (cs + cl - 1 - r) : (cs + r);
                const size_t off = (size_t)(row0 + tok) * dvr + gcol;
                pv[m][rr] = *reinterpret_cast<const u32x4_t*>(gv + off);
                if (GRAD) px[m][rr] = *reinterpret_cast<const u32x4_t*>(gx + off);
            }
        }
    };
    // element e of two rows, packed for a single transposed LDS write
    auto put_pair = [](E* dst, const u32x4_t& r0, const u32x4_t& r1, int e) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        u32x2_t pr = {r0[e], r1[e]};
        *reinterpret_cast<u32x2_t*>(dst) = pr;
    
    };
    const u32x4_t zero4 = {0u, 0u, 0u, 0u};
    auto store_chunk = [&](int cl) {
#pragma unroll
        for (int m = 0; m < NBQ; ++m) {
            const int b = tid + NTHREADS * m;
            if (b < RP * SEGQ) {
                int rp, cg;
                block_rc(b, SEGQ, rp, cg);
                const int col = cg * V16;
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const bool ok = (2 * rp + rr < cl) && (col < dkr);
                    pq[m][rr] = ok ? pq[m][rr] : zero4;
                    pk[m][rr] = ok ? pk[m][rr] : zero4;
                }
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    *reinterpret_cast<u32x4_t*>(Qs + (2 * rp + rr) * LDQ + col) = pq[m][rr];
                    *reinterpret_cast<u32x4_t*>(Ks + (2 * rp + rr) * LDQ + col) = pk[m][rr];
                }
#pragma unroll
                for (int e = 0; e < V16; ++e) put_pair(KTs + (col + e) * LDT + 2 * rp, pk[m][0], pk[m][1], e);
            }
        }
#pragma unroll
        for (int m = 0; m < NBV; ++m) {
            const int b = tid + NTHREADS * m;
            if (b < RP * SEGV) {
                int rp, cg;
                block_rc(b, SEGV, rp, cg);
                const int col = cg * V16;
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const bool ok = (2 * rp + rr < cl) && (n0 + col < dvr);
                    pv[m][rr] = ok ? pv[m][rr] : zero4;
                    if (GRAD) px[m][rr] = ok ? px[m][rr] : zero4;
                }
#pragma unroll
                for (int e = 0; e < V16; ++e) {
                    put_pair(VTs + (col + e) * LDT + 2 * rp, pv[m][0], pv[m][1], e);
                    if (GRAD) put_pair(XTs + (col + e) * LDT + 2 * rp, px[m][0], px[m][1], e);
                }
            }
        }
    };

    if (nchunks > 0) load_chunk(0);
    for (int ci = 0; ci < nchunks; ++ci) {
        const int c = R::REV ? (nchunks - 1 - ci) : ci;
        const int cstart = c * C;
        const int clen = min(C, len - cstart);
        const bool shift = ra.init_undecayed && ci == 0;

        lds_barrier();  // previous chunk's LDS readers are done

        // state before this chunk -> STh, transposed; the four
        // consecutive state rows of an accumulator group go out as one write
#pragma unroll
        for (int kt = 0; kt < NDBW * NNT; ++kt) {
            const int db = dbs[kt / NNT], nb = kt % NNT;
            if (db >= 0) {
                const f32x16_t& acc = sacc[kt];
                const int nl = 32 * nb + l32;
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int off = nl * LDQ + 32 * db + 8 * qd + 4 * g;
                    f32x4_t hv;
#pragma unroll
                    for (int e = 0; e < 4; ++e) hv[e] = acc[4 * qd + e];
                    *reinterpret_cast<f32x4_t*>(STh + off) = hv;
                
                }
            }
        }
        // key decays of the state update (not shifted: only the carried-in
        // state enters the first reversed token undecayed)
        for (int r = tid; r < C; r += NTHREADS) ksc[r] = (r < clen) ? decay_pow(clen - 1 - r, l2) : 0.0f;
        store_chunk(clen);
        if (ci + 1 < nchunks) load_chunk(ci + 1);  // in flight during this chunk's math
        lds_barrier();

        // per-token epilogue coefficient (two threads per token, 16-byte reads)
        if (tid < 2 * C) {
            const int r = tid >> 1, half = tid & 1;
            constexpr int HV = DK / V16 / 2;  // 16-byte vectors per half row
            float z = 0.0f, u = 0.0f;
#pragma unroll
            for (int vi = 0; vi < HV; ++vi) {
                const int col = (half * HV + vi) * V16;
                const u32x4_t qv = *reinterpret_cast<const u32x4_t*>(Qs + r * LDQ + col);
                const u32x4_t kv = *reinterpret_cast<const u32x4_t*>(Ks + r * LDQ + col);
#pragma unroll
                for (int e = 0; e < V16; ++e) {
                    const float p = vget<E>(qv, e) * vget<E>(kv, e);
                    if (GRAD) u += p;
                    else z += a_lds[col + e] * p;
                }
            }
            if (GRAD && cm.a != nullptr && r < clen) {
                // z = sum_n a_n v'_n x_n over the full width, read from memory:
                // this workgroup stages only a slice of v' and x
                const int tok = R::REV ? (cstart + clen - 1 - r) : (cstart + r);
                const E* vr = gv + (size_t)(row0 + tok) * dvr;
                const E* xr = gx + (size_t)(row0 + tok) * dvr;
                for (int col = half * V16; col < dvr; col += 2 * V16) {
                    const u32x4_t vv = *reinterpret_cast<const u32x4_t*>(vr + col);
                    const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xr + col);
#pragma unroll
                    for (int e = 0; e < V16; ++e) z += a_lds[col + e] * vget<E>(vv, e) * vget<E>(xv, e);
                }
            }
            z += __shfl_xor(z, 1);
            u += __shfl_xor(u, 1);
            if (half == 0) {
                const float s = sigmoidf_(z);
                coef[r] = GRAD ? s * (1.0f - s) * u : s;
            }
        }
        lds_barrier();

        // ---- query strips
        if (wave < NSTRIP && 32 * wave < clen) {
            const int t0 = 32 * wave;
            f32x16_t oacc[NNT];
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[nt][i] = 0.0f;

            // inter-chunk: Q' (S_hi + S_lo)
#pragma unroll 2
            for (int kb = 0; kb < DK / KSTEP; ++kb) {
                const typename M::op_t av = M::load(Qs + (t0 + l32) * LDQ + kb * KSTEP + g * NE);
#pragma unroll
                for (int nt = 0; nt < NNT; ++nt) {
                    const int boff = (32 * nt + l32) * LDQ + kb * KSTEP + g * NE;
                    oacc[nt] = M::mma(av, M::load(STh + boff), oacc[nt]);
                }
            }
            // rows scale by lam^(t+1), or lam^t where the carried state enters
            // the first token undecayed (first chunk of a reverse scan)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float f = decay_pow(t0 + acc_row(i, g) + (shift ? 0 : 1), l2);
#pragma unroll
                for (int nt = 0; nt < NNT; ++nt) oacc[nt][i] *= f;
            }

            // intra-chunk: decay-masked scores, then P V'
            for (int jb = 0; jb <= wave; ++jb) {
                f32x16_t sc;
#pragma unroll
                for (int i = 0; i < 16; ++i) sc[i] = 0.0f;
#pragma unroll 2
                for (int kb = 0; kb < DK / KSTEP; ++kb) {
                    const typename M::op_t av = M::load(Ks + (32 * jb + l32) * LDQ + kb * KSTEP + g * NE);
                    const typename M::op_t bv = M::load(Qs + (t0 + l32) * LDQ + kb * KSTEP + g * NE);
                    sc = M::mma(av, bv, sc);
                }
                // sc[i] = k'_j . q'_t with j = 32 jb + acc_row(i, g), t = t0 + l32
                const int t = t0 + l32;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int diff = t - (32 * jb + acc_row(i, g));
                    const float f = (diff == 0) ? 1.0f : fast_exp2((float)diff * l2);
                    sc[i] = (diff < 0) ? 0.0f : sc[i] * f;
                }
#pragma unroll
                for (int s = 0; s < 16; ++s) {
#pragma unroll
                    for (int nt = 0; nt < NNT; ++nt) {
                        const float bv = to_f(VTs[(32 * nt + l32) * LDT + 32 * jb + acc_row(s, g)]);
                        oacc[nt] = M::mma(sc[s], bv, oacc[nt]);
                    }
                }
            
            }

            // epilogue: + coef_t * w_n * v'_t[n]  (w = 1, or a for the gradient
            // roles); accumulator group qd holds 4 consecutive rows t
            E* obase = go + (size_t)(row0 + (R::REV ? cstart + clen - 1 : cstart)) * dvr + n0;
            const int ostep = R::REV ? -dvr : dvr;
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) {
                const int nl = 32 * nt + l32;
                const float wn = (R::AUG == AUG_GRAD) ? a_lds[n0 + nl] : 1.0f;
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int t = t0 + 8 * qd + 4 * g;
                    const f32x4_t cf = *reinterpret_cast<const f32x4_t*>(coef + t);
                    float vt[4], xt[4];
                    const f32x4_t v4 = *reinterpret_cast<const f32x4_t*>(VTs + nl * LDT + t);
                    f32x4_t x4 = {0.f, 0.f, 0.f, 0.f};
                    if (R::AUG == AUG_GRAD) x4 = *reinterpret_cast<const f32x4_t*>(XTs + nl * LDT + t);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        vt[e] = v4[e];
                        xt[e] = x4[e];
                    }
                
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        oacc[nt][4 * qd + e] += cf[e] * wn * vt[e];
                        if (R::AUG == AUG_GRAD) da_acc[nt] += cf[e] * vt[e] * xt[e];
                    }
                }
                if (n0 + nl < dvr) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int t = t0 + acc_row(i, g);
                        if (t < clen) obase[t * ostep + nl] = from_f<E>(oacc[nt][i]);
                    }
                }
            }
        }

        // ---- state advance: S = lam^(C_c) S + (lam^m k')^T V', decayed keys as hi + lo
        const float fc = decay_pow(clen - (shift ? 1 : 0), l2);
#pragma unroll
        for (int kk = 0; kk < NDBW; ++kk) {
            const int db = dbs[kk];
            if (db >= 0) {
#pragma unroll
                for (int nb = 0; nb < NNT; ++nb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) sacc[kk * NNT + nb][i] *= fc;
#pragma unroll 2
                for (int kb = 0; kb < C / KSTEP; ++kb) {
                    const int j0 = kb * KSTEP + g * NE;
                    const E* kr = KTs + (32 * db + l32) * LDT + j0;
                    const float av = to_f(*kr) * ksc[j0];
#pragma unroll
                    for (int nb = 0; nb < NNT; ++nb) {
                        const typename M::op_t bv = M::load(VTs + (32 * nb + l32) * LDT + j0);
                        sacc[kk * NNT + nb] = M::mma(av, bv, sacc[kk * NNT + nb]);
                    }
                
                }
            }
        }
    }

    // ---- final state
    if (ra.s_final != nullptr) {
        const float fs = (ra.final_times_lam && len > 0) ? lam : 1.0f;
#pragma unroll
        for (int kt = 0; kt < NDBW * NNT; ++kt) {
            const int db = dbs[kt / NNT], nb = kt % NNT;
            if (db >= 0) {
                const int nn = n0 + 32 * nb + l32;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int d = 32 * db + acc_row(i, g);
                    if (d < dkr && nn < dvr) {
                        const float val = sacc[kt][i] * fs;
                        if (ra.state_t) ra.s_final[sbase + (size_t)nn * dkr + d] = val;
                        else ra.s_final[sbase + (size_t)d * dvr + nn] = val;
                    }
                }
            }
        }
    }

    // ---- partial da of this (sequence, head, slice): fixed-order reduction
    if (R::AUG == AUG_GRAD && ra.da_part != nullptr) {
        lds_barrier();
        if (wave < NSTRIP) {
#pragma unroll
            for (int nt = 0; nt < NNT; ++nt) {
                const float s = da_acc[nt] + __shfl_xor(da_acc[nt], 32);
                if (g == 0) dared[wave * DVS + 32 * nt + l32] = s;
            }
        }
        lds_barrier();
        for (int nl = tid; nl < DVS; nl += NTHREADS) {
            float s = 0.0f;
            for (int w = 0; w < NSTRIP; ++w) s += dared[w * DVS + nl];
            if (n0 + nl < dvr) ra.da_part[(size_t)unit * dvr + n0 + nl] = s;
        }
    }
}

// blockIdx -> (unit, slice): consecutive slices of one unit land on the same
// XCD (blocks are dealt to the 8 XCDs round-robin), so their shared q'/k'
// reads hit the same L2.
__device__ __forceinline__ bool map_block(int nsl, int n_units, int& unit, int& slice)
{
    const int b = blockIdx.x;
    const int xcd = b & 7, loc = b >> 3;
    slice = loc % nsl;
    unit = (loc / nsl) * 8 + xcd;
    return unit < n_units;
}

template <class R>
__global__ __launch_bounds__(NTHREADS) void k_chunk_fwd(Common cm, RoleArgs ra, int nsl)
{
    __shared__ __attribute__((aligned(16))) char smem[R::LDS];
    int unit, slice;
    if (!map_block(nsl, cm.n_units, unit, slice)) return;
    role_body<R>(cm, ra, unit, slice, smem);
}

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// One launch runs the three backward scans: slices [0, nslq) are dq,
// [nslq, 2 nslq) dk, and the rest dv.
template <class RQ, class RK, class RV>
__global__ __launch_bounds__(NTHREADS) void k_chunk_bwd(Common cm, RoleArgs aq, RoleArgs ak,
                                                        RoleArgs av, int nslq, int nslv)
{
    __shared__ __attribute__((aligned(16))) char smem[cmax(RQ::LDS, cmax(RK::LDS, RV::LDS))];
    int unit, vs;
    if (!map_block(2 * nslq + nslv, cm.n_units, unit, vs)) return;
    if (vs < nslq) role_body<RQ>(cm, aq, unit, vs, smem);
    else if (vs < 2 * nslq) role_body<RK>(cm, ak, unit, vs - nslq, smem);
    else role_body<RV>(cm, av, unit, vs - 2 * nslq, smem);
}

// da[h][d] = sum over sequences n (in order) of da_part[n*H + h][d]
__global__ void k_da_reduce(const float* da_part, float* da, int n_seq, int H, int dkr)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= H * dkr) return;
    const int h = i / dkr, d = i - (i / dkr) * dkr;
    float s = 0.0f;
    for (int n = 0; n < n_seq; ++n) s += da_part[((size_t)n * H + h) * dkr + d];
    da[i] = s;
}

int round8(int x) { return (x + 7) / 8 * 8; }

template <class R>
hipError_t run_fwd(const ChunkProblem& p, const RoleArgs& ra, int nsl, hipStream_t stream)
{
    Common cm{p.lambda, p.a, p.cu, p.H, p.T, p.n_seq * p.H};
    const int grid = round8(cm.n_units) * nsl;
    hipLaunchKernelGGL(k_chunk_fwd<R>, dim3(grid), dim3(NTHREADS), 0, stream, cm, ra, nsl);
    return hipGetLastError();
}

template <class RQ, class RK, class RV>
hipError_t run_bwd(const ChunkProblem& p, const RoleArgs& aq, const RoleArgs& ak,
                   const RoleArgs& av, float* da, hipStream_t stream)
{
    static_assert(RQ::DVS == RK::DVS, "dq and dk slices");
    Common cm{p.lambda, p.a, p.cu, p.H, p.T, p.n_seq * p.H};
    const int nslq = (p.d_k + RQ::DVS - 1) / RQ::DVS;
    const int nslv = (p.d_v + RV::DVS - 1) / RV::DVS;
    const int grid = round8(cm.n_units) * (2 * nslq + nslv);
    hipLaunchKernelGGL((k_chunk_bwd<RQ, RK, RV>), dim3(grid), dim3(NTHREADS), 0, stream, cm, aq, ak,
                       av, nslq, nslv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nda = p.H * p.d_k;
    hipLaunchKernelGGL(k_da_reduce, dim3((nda + 255) / 256), dim3(256), 0, stream, aq.da_part, da,
                       p.n_seq, p.H, p.d_k);
    return hipGetLastError();
}

// Role instantiations (fp32 tensors; bf16 runs on the kernels of sgla_fwd.hip
// and sgla_bwd.hip); C is the chunk length, 32, 64 or 128 tokens
template <int C> using F32Fwd = Role<float, 32, 32, C, AUG_FWD, false>;
template <int C> using F32Dq = Role<float, 32, 32, C, AUG_GRAD, false>;
template <int C> using F32Dk = Role<float, 32, 32, C, AUG_GRAD, true>;
template <int C> using F32Dv = Role<float, 32, 32, C, AUG_FWD, true>;
// Wider fp32 heads (contraction widths up to 96 in the forward and the dv
// scan, up to 192 in the dq and dk scans, whose contraction runs over d_v):
// 32-token tiles, which keep every such role's operands within the LDS;
// widths are rounded up to the next of 32, 64, 96 (192) and padded.
template <int DK> using F32FwdW = Role<float, DK, 32, 32, AUG_FWD, false>;
template <int DV> using F32DqW = Role<float, DV, 32, 32, AUG_GRAD, false>;
template <int DV> using F32DkW = Role<float, DV, 32, 32, AUG_GRAD, true>;
template <int DK> using F32DvW = Role<float, DK, 32, 32, AUG_FWD, true>;

template <int DV>
hipError_t run_bwd_wide(const ChunkProblem& p, const RoleArgs& aq, const RoleArgs& ak, const RoleArgs& av,
                        float* da, hipStream_t stream)
{
    if (p.d_k <= 32) return run_bwd<F32DqW<DV>, F32DkW<DV>, F32DvW<32>>(p, aq, ak, av, da, stream);
    if (p.d_k <= 64) return run_bwd<F32DqW<DV>, F32DkW<DV>, F32DvW<64>>(p, aq, ak, av, da, stream);
    return run_bwd<F32DqW<DV>, F32DkW<DV>, F32DvW<96>>(p, aq, ak, av, da, stream);
}

}  // namespace

hipError_t launch_chunk_fwd(const ChunkProblem& p, const void* q, const void* k, const void* v,
                            const float* init_state, float* final_state, void* o,
                            hipStream_t stream)
{
    // bf16 shapes are limited to d_k <= 96, d_v <= 192 by the host checks
    if (p.bf16) return launch_fwd_bf16(p, q, k, v, init_state, final_state, o, stream);
    RoleArgs ra{q, k, v, nullptr, o, init_state, final_state, nullptr, p.d_k, p.d_v, 0, 0, 0};
    const int nsl = (p.d_v + 31) / 32;
    if (p.d_k > 64) return run_fwd<F32FwdW<96>>(p, ra, nsl, stream);
    if (p.d_k > 32) return run_fwd<F32FwdW<64>>(p, ra, nsl, stream);
    if (p.chunk == 32) return run_fwd<F32Fwd<32>>(p, ra, nsl, stream);
    if (p.chunk == 128) return run_fwd<F32Fwd<128>>(p, ra, nsl, stream);
    return run_fwd<F32Fwd<64>>(p, ra, nsl, stream);
}

hipError_t launch_chunk_bwd(const ChunkProblem& p, const void* q, const void* k, const void* v,
                            const void* dO, const float* init_state, const float* d_final_state,
                            void* dq, void* dk, void* dv, float* da, float* d_init_state,
                            float* da_partial, hipStream_t stream)
{
    if (p.bf16)
        return launch_bwd_bf16(p, q, k, v, dO, init_state, d_final_state, dq, dk, dv, da,
                               d_init_state, da_partial, stream);
    // dq: forward scan of S^T ([d_v][d_k]); q'=dO, k'=v, v'=k, gate operand q
    RoleArgs aq{dO, v, k, q, dq, init_state, nullptr, da_partial, p.d_v, p.d_k, 1, 0, 0};
    // dk: reverse scan of G^T ([d_v][d_k]); q'=v, k'=dO, v'=q, gate operand k
    RoleArgs ak{v, dO, q, k, dk, d_final_state, nullptr, nullptr, p.d_v, p.d_k, 1, 0, 1};
    // dv: reverse scan of G ([d_k][d_v]); q'=k, k'=q, v'=dO; final G -> d_init_state
    RoleArgs av{k, q, dO, nullptr, dv, d_final_state, d_init_state, nullptr, p.d_k, p.d_v, 0, 1, 1};
    if (p.d_v > 96) return run_bwd_wide<192>(p, aq, ak, av, da, stream);
    if (p.d_v > 64) return run_bwd_wide<96>(p, aq, ak, av, da, stream);
    if (p.d_v > 32) return run_bwd_wide<64>(p, aq, ak, av, da, stream);
    if (p.d_k > 32) return run_bwd_wide<32>(p, aq, ak, av, da, stream);
    if (p.chunk == 32) return run_bwd<F32Dq<32>, F32Dk<32>, F32Dv<32>>(p, aq, ak, av, da, stream);
    if (p.chunk == 128) return run_bwd<F32Dq<128>, F32Dk<128>, F32Dv<128>>(p, aq, ak, av, da, stream);
    return run_bwd<F32Dq<64>, F32Dk<64>, F32Dv<64>>(p, aq, ak, av, da, stream);
}

}  // namespace sgla
