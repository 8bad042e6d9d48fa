// Chunked Simple GLA forward for gfx950, bf16 inputs: the FWD role of the
// tile-scan body in sgla_scan.hpp (method: "Beyond the KV cache: Training and
// serving i14's Laplace 3B linear attention model on AWS Trainium2 with native
// PyTorch", section "Challenge 1: Using native PyTorch on Trainium for GLA").

#include "sgla_scan.hpp"
#include "sgla_internal.h"

namespace sgla {
namespace scan {

// One workgroup of eight waves per (sequence, head, 96-column value slice);
// the slices of one unit share an XCD (blocks are dealt to the eight XCDs
// round-robin) and so share its L2.
template <int DK>
__global__ __launch_bounds__(NTHREADS_W) void k_fwd(Args p)
{
    __shared__ __attribute__((aligned(16))) char smem[LayW<WFwd<DK>>::LDS];
    const int b = blockIdx.x;
    const int slice = (b >> 3) % p.nsl;
    const int unit = ((b >> 3) / p.nsl) * 8 + (b & 7);
    if (unit >= p.n_units) return;
    body_wide<WFwd<DK>>(p, unit, slice, smem);
}

template <int DK>
hipError_t run_fwd(const Args& a, hipStream_t stream)
{
    const int grid = ((a.n_units + 7) / 8) * 8 * a.nsl;
    hipLaunchKernelGGL(k_fwd<DK>, dim3(grid), dim3(NTHREADS_W), 0, stream, a);
    return hipGetLastError();
}

}  // namespace scan

// bf16 forward with d_k <= 96 (padded to 32, 64 or 96) and any d_v (96-column slices).
hipError_t launch_fwd_bf16(const ChunkProblem& p, const void* q, const void* k, const void* v,
                           const float* init_state, float* final_state, void* o,
                           hipStream_t stream)
{
    scan::Args a{};
    a.q = reinterpret_cast<const uint16_t*>(q);
    a.k = reinterpret_cast<const uint16_t*>(k);
    a.v = reinterpret_cast<const uint16_t*>(v);
    a.x = nullptr;
    a.o = reinterpret_cast<uint16_t*>(o);
    a.lambda = p.lambda;
    a.a = p.a;
    a.cu = p.cu;
    a.s_init = init_state;
    a.s_final = final_state;
    a.da_part = nullptr;
    a.H = p.H;
    a.T = p.T;
    a.n_units = p.n_seq * p.H;
    a.nsl = (p.d_v + scan::DVS - 1) / scan::DVS;
    a.dkr = p.d_k;
    a.dvr = p.d_v;
    if (p.d_k <= 32) return scan::run_fwd<32>(a, stream);
    if (p.d_k <= 64) return scan::run_fwd<64>(a, stream);
    return scan::run_fwd<96>(a, stream);
}

}  // namespace sgla
