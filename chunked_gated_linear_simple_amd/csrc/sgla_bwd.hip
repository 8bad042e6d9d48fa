// Chunked Simple GLA backward for gfx950, bf16 inputs: the DV, DQ and DK roles
// of the tile-scan body in sgla_scan.hpp, all in one launch.
//
// Method: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
// attention model on AWS Trainium2 with native PyTorch", section "Challenge 1:
// Using native PyTorch on Trainium for GLA" (the backward pass differentiates
// through the chunk recurrence, so the state gradient runs through the chunks
// in reverse), with the self-augmentation of section "i14 and the Laplace 3B
// architecture", paragraph "GLA mixer" (a is learned, so it has a gradient).
// For every token t of a sequence (s over the same sequence):
//   dv_s = sum_{t>=s} lam^(t-s) (q_t . k_s) dO_t + lam^(..) G k_s + sigmoid(z_s) dO_s
//   dk_s = sum_{t>=s} lam^(t-s) (dO_t . v_s) q_t + lam^(..) G v_s + c_s (a (.) q_s)
//   dq_t = sum_{s<=t} lam^(t-s) (dO_t . v_s) k_s + lam^(..) S dO_t + c_t (a (.) k_t)
//   da   = sum_t c_t q_t (.) k_t,   c_t = sigmoid'(z_t) (dO_t . v_t)
// with S the forward state and G the state gradient. DV is a reverse scan of G
// ([d_k][d_v], sliced by d_v columns), DQ a forward scan of S^T and DK a
// reverse scan of G^T ([d_v][d_k], all d_k columns in one workgroup).
//
// Workgroups per (sequence, head): DQ, DK, then one DV per 96 columns of d_v;
// all of a unit's workgroups land on one XCD. The gradient of a is summed per
// sequence-head by DQ and then over sequences in a fixed order, so the result
// is bitwise reproducible.

#include "sgla_scan.hpp"
#include "sgla_internal.h"

namespace sgla {
namespace scan {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// The three scans' operands; role = 0 (DQ), 1 (DK), 2 (DV, nsl slices).
struct BwdArgs {
    Args role[3];
};

template <int DKV, int DKG, int CTV>
__global__ __launch_bounds__(NTHREADS_W) void k_bwd(BwdArgs ba)
{
    constexpr int LDS = cmax(LayW<WDv<DKV, CTV>>::LDS, cmax(LayW<WDq<DKG>>::LDS, LayW<WDk<DKG>>::LDS));
    __shared__ __attribute__((aligned(16))) char smem[LDS];
    const int nr = ba.role[2].nsl + 2;
    const int b = blockIdx.x;
    const int r = (b >> 3) % nr;
    const int unit = ((b >> 3) / nr) * 8 + (b & 7);
    if (unit >= ba.role[2].n_units) return;
    // one role's operands, picked at run time so that only they are loaded
    const int ri = r < 2 ? r : 2;
    const Args& p = ba.role[ri];
    if (r == 0) body_wide<WDq<DKG>>(p, unit, 0, smem);
    else if (r == 1) body_wide<WDk<DKG>>(p, unit, 0, smem);
    else body_wide<WDv<DKV, CTV>>(p, unit, r - 2, smem);
}

// da[h][d] = sum over sequences n (in order) of part[n H + h][d]
__global__ void k_da_sum(const float* __restrict__ part, float* __restrict__ da, int n_seq, int H, int dk)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= H * dk) return;
    const int h = i / dk, d = i - (i / dk) * dk;
    float s = 0.0f;
    for (int n = 0; n < n_seq; ++n) s += part[((size_t)n * H + h) * dk + d];
    da[i] = s;
}

// The state passes of the segmented backward in one launch: the forward state
// scan over segments 0 .. nseg-2 (blocks [0, nf)) and the gradient state scan
// over segments 1 .. nseg-1 (the blocks after), which are independent of each
// other and write no outputs. Each role's blocks map to (unit, value slice) as
// in k_fwd.
template <int DK>
__global__ __launch_bounds__(NTHREADS_W) void k_seg_states(Args af, Args adv, int nf)
{
    constexpr int LF = LayW<WFwdState<DK>>::LDS, LD = LayW<WDvState<DK>>::LDS;
    constexpr int LDS = LF > LD ? LF : LD;
    __shared__ __attribute__((aligned(16))) char smem[LDS];
    const bool fwd = (int)blockIdx.x < nf;
    const Args& p = fwd ? af : adv;
    const int b = fwd ? (int)blockIdx.x : (int)blockIdx.x - nf;
    const int slice = (b >> 3) % p.nsl;
    const int unit = ((b >> 3) / p.nsl) * 8 + (b & 7);
    if (unit >= p.n_units) return;
    if (fwd) body_wide<WFwdState<DK>>(p, unit, slice, smem);
    else body_wide<WDvState<DK>>(p, unit, slice, smem);
}

// ctv: tile length of the dv scan (32 or 64 tokens); dq and dk always run
// 32-token tiles (their 192-wide operands fill the LDS ring at 32).
template <int DKV, int DKG>
hipError_t run_bwd(const Args& av, const Args& aq, const Args& ak, hipStream_t stream, int ctv)
{
    BwdArgs ba;
    ba.role[0] = aq;
    ba.role[1] = ak;
    ba.role[2] = av;
    const int grid = ((av.n_units + 7) / 8) * 8 * (av.nsl + 2);
    if (ctv == 32) hipLaunchKernelGGL((k_bwd<DKV, DKG, 32>), dim3(grid), dim3(NTHREADS_W), 0, stream, ba);
    else hipLaunchKernelGGL((k_bwd<DKV, DKG, 64>), dim3(grid), dim3(NTHREADS_W), 0, stream, ba);
    return hipGetLastError();
}

}  // namespace scan

static hipError_t run_bwd_any(const ChunkProblem& p, const scan::Args& av, const scan::Args& aq,
                              const scan::Args& ak, hipStream_t stream)
{
    const int ct = bf16_tile(p.chunk);
    if (p.d_k <= 32)
        return (p.d_v <= 96) ? scan::run_bwd<32, 96>(av, aq, ak, stream, ct)
                             : scan::run_bwd<32, 192>(av, aq, ak, stream, ct);
    return (p.d_v <= 96) ? scan::run_bwd<96, 96>(av, aq, ak, stream, ct)
                         : scan::run_bwd<96, 192>(av, aq, ak, stream, ct);
}

// bf16 backward of dense sequences cut into nseg >= 2 segments (see
// sgla_chunk_bwd_segmented). ws holds four [n_seq][nseg][H][d_k][d_v] arrays:
// forward states leaving / entering segments, gradient states leaving /
// entering segments; da_partial holds n_seq nseg H d_k floats. The state
// passes of step 1 write states only; step 3 writes dq, dk and dv.
hipError_t launch_bwd_bf16_segmented(const ChunkProblem& p, const void* q, const void* k, const void* v,
                                     const void* dO, const float* init_state, const float* d_final_state,
                                     void* dq, void* dk, void* dv, float* da, float* d_init_state,
                                     float* da_partial, int nseg, int seg_len, float* ws, hipStream_t stream)
{
    const size_t ssz = (size_t)p.d_k * p.d_v;
    const size_t arr = (size_t)p.n_seq * nseg * p.H * ssz;
    float* f_loc = ws;
    float* f_in = ws + arr;
    float* g_loc = ws + 2 * arr;
    float* g_in = ws + 3 * arr;

    typedef const uint16_t* cp;
    scan::Args base{};
    base.lambda = p.lambda;
    base.a = p.a;
    base.cu = nullptr;
    base.H = p.H;
    base.T = p.T;
    base.nseg = nseg;
    base.seg_len = seg_len;
    base.nsl = (p.d_v + scan::DVS - 1) / scan::DVS;
    base.dkr = p.d_k;
    base.dvr = p.d_v;

    // 1. in one launch: the forward state scan over segments 0 .. nseg-2
    // (segment 0 from init_state, the rest from zero) keeping the states they
    // leave, and the gradient state scan over segments 1 .. nseg-1 from their
    // ends (the last from d_final_state, the rest from zero) keeping the
    // states they leave at their fronts; neither writes outputs
    scan::Args af = base;
    af.q = nullptr;
    af.k = reinterpret_cast<cp>(k);
    af.v = reinterpret_cast<cp>(v);
    af.o = nullptr;
    af.s_init = init_state;
    af.s_out_seg = f_loc;
    af.seg_first = 0;
    af.seg_count = nseg - 1;
    af.n_units = p.n_seq * (nseg - 1) * p.H;
    scan::Args av = base;
    av.q = reinterpret_cast<cp>(k);
    av.k = reinterpret_cast<cp>(q);
    av.v = reinterpret_cast<cp>(dO);
    av.o = reinterpret_cast<uint16_t*>(dv);
    scan::Args a2 = av;
    a2.q = nullptr;
    a2.o = nullptr;
    a2.s_init = d_final_state;
    a2.s_out_seg = g_loc;
    a2.seg_first = 1;
    a2.seg_count = nseg - 1;
    a2.n_units = p.n_seq * (nseg - 1) * p.H;
    const int nf = ((af.n_units + 7) / 8) * 8 * af.nsl;
    const int nd = ((a2.n_units + 7) / 8) * 8 * a2.nsl;
    if (p.d_k <= 32)
        hipLaunchKernelGGL(scan::k_seg_states<32>, dim3(nf + nd), dim3(scan::NTHREADS_W), 0, stream, af, a2, nf);
    else if (p.d_k <= 64)
        hipLaunchKernelGGL(scan::k_seg_states<64>, dim3(nf + nd), dim3(scan::NTHREADS_W), 0, stream, af, a2, nf);
    else
        hipLaunchKernelGGL(scan::k_seg_states<96>, dim3(nf + nd), dim3(scan::NTHREADS_W), 0, stream, af, a2, nf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    // 2. the forward scan of the leaving states and the reverse scan of the
    // gradient states
    const int ssz4 = (int)(ssz / 4);
    hipLaunchKernelGGL(scan::k_seg_scan, dim3((ssz4 + 255) / 256, p.n_seq * p.H), dim3(256), 0, stream, f_loc,
                       f_in, p.lambda, p.n_seq, nseg, p.H, ssz4, seg_len, 0, nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scan::k_seg_rscan, dim3((ssz4 + 255) / 256, p.n_seq * p.H), dim3(256), 0, stream, g_loc,
                       g_in, p.lambda, nseg, p.H, ssz4, seg_len);
    e = hipGetLastError();
    if (e != hipSuccess) return e;

    // 3. every segment from its true states
    av.s_init = d_final_state;
    av.s_final = d_init_state;
    av.s_in_seg = g_in;
    av.s_out_seg = nullptr;
    av.seg_first = 0;
    av.seg_count = nseg;
    av.n_units = p.n_seq * nseg * p.H;
    scan::Args aq = av;
    aq.q = reinterpret_cast<cp>(dO);
    aq.k = reinterpret_cast<cp>(v);
    aq.v = reinterpret_cast<cp>(k);
    aq.x = reinterpret_cast<cp>(q);
    aq.o = reinterpret_cast<uint16_t*>(dq);
    aq.s_init = init_state;
    aq.s_final = nullptr;
    aq.s_in_seg = f_in;
    aq.da_part = da_partial;
    aq.dkr = p.d_v;
    aq.dvr = p.d_k;
    aq.nsl = 1;
    scan::Args ak = aq;
    ak.q = reinterpret_cast<cp>(v);
    ak.k = reinterpret_cast<cp>(dO);
    ak.v = reinterpret_cast<cp>(q);
    ak.x = reinterpret_cast<cp>(k);
    ak.o = reinterpret_cast<uint16_t*>(dk);
    ak.s_init = d_final_state;
    ak.s_in_seg = g_in;
    ak.da_part = nullptr;
    e = run_bwd_any(p, av, aq, ak, stream);
    if (e != hipSuccess) return e;
    const int nda = p.H * p.d_k;
    hipLaunchKernelGGL(scan::k_da_sum, dim3((nda + 255) / 256), dim3(256), 0, stream, da_partial, da,
                       p.n_seq * nseg, p.H, p.d_k);
    return hipGetLastError();
}

// bf16 backward with d_k <= 96 and d_v <= 192.
hipError_t launch_bwd_bf16(const ChunkProblem& p, const void* q, const void* k, const void* v,
                           const void* dO, const float* init_state, const float* d_final_state,
                           void* dq, void* dk, void* dv, float* da, float* d_init_state,
                           float* da_partial, hipStream_t stream)
{
    typedef const uint16_t* cp;
    scan::Args base{};
    base.lambda = p.lambda;
    base.a = p.a;
    base.cu = p.cu;
    base.H = p.H;
    base.T = p.T;
    base.n_units = p.n_seq * p.H;

    // dv: reverse scan of G; q'=k, k'=q, v'=dO; final G -> d_init_state
    scan::Args av = base;
    av.q = reinterpret_cast<cp>(k);
    av.k = reinterpret_cast<cp>(q);
    av.v = reinterpret_cast<cp>(dO);
    av.o = reinterpret_cast<uint16_t*>(dv);
    av.s_init = d_final_state;
    av.s_final = d_init_state;
    av.dkr = p.d_k;
    av.dvr = p.d_v;
    av.nsl = (p.d_v + scan::DVS - 1) / scan::DVS;
    // dq: forward scan of S^T; q'=dO, k'=v, v'=k, gate operand q
    scan::Args aq = base;
    aq.q = reinterpret_cast<cp>(dO);
    aq.k = reinterpret_cast<cp>(v);
    aq.v = reinterpret_cast<cp>(k);
    aq.x = reinterpret_cast<cp>(q);
    aq.o = reinterpret_cast<uint16_t*>(dq);
    aq.s_init = init_state;
    aq.da_part = da_partial;
    aq.dkr = p.d_v;
    aq.dvr = p.d_k;
    aq.nsl = 1;
    // dk: reverse scan of G^T; q'=v, k'=dO, v'=q, gate operand k
    scan::Args ak = aq;
    ak.q = reinterpret_cast<cp>(v);
    ak.k = reinterpret_cast<cp>(dO);
    ak.v = reinterpret_cast<cp>(q);
    ak.x = reinterpret_cast<cp>(k);
    ak.o = reinterpret_cast<uint16_t*>(dk);
    ak.s_init = d_final_state;
    ak.da_part = nullptr;

    hipError_t e = run_bwd_any(p, av, aq, ak, stream);
    if (e != hipSuccess) return e;
    const int nda = p.H * p.d_k;
    hipLaunchKernelGGL(scan::k_da_sum, dim3((nda + 255) / 256), dim3(256), 0, stream, da_partial, da,
                       p.n_seq, p.H, p.d_k);
    return hipGetLastError();
}

}  // namespace sgla
