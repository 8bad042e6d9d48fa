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
template <int DK, int CT>
__global__ __launch_bounds__(NTHREADS_W) void k_fwd(Args p)
{
    __shared__ __attribute__((aligned(16))) char smem[LayW<WFwd<DK, CT>>::LDS];
    const int b = blockIdx.x;
    const int slice = (b >> 3) % p.nsl;
    const int unit = ((b >> 3) / p.nsl) * 8 + (b & 7);
    if (unit >= p.n_units) return;
    body_wide<WFwd<DK, CT>>(p, unit, slice, smem);
}

// The forward with the mixer epilogue applied before the store: one group of
// nsl workgroups (the value slices) per (sequence, head) unit, units
// unit_base + group. The slices of a unit exchange the per-token sums of o^2
// while they scan, so they must run at the same time. A workgroup's group
// and slice therefore come from a ticket it takes when it starts, from the
// counter of its XCD index (blockIdx % 8): tickets nsl j .. nsl j + nsl - 1
// of counter x form group 8 j + x, so a group's slices share an XCD (and
// its L2 for q and k) as in k_fwd. The workgroups holding the tickets of a
// group have all started except, per counter, at most the group of the
// latest tickets, whose missing slices take the next tickets: every other
// group can finish and free its compute unit, so the launch needs no
// guarantee of residency (an ordinary launch, any grid size). The last
// workgroup to finish clears the counters for the next call. (A persistent
// grid looping over units keeps every unit-invariant value of all roles live
// across the loop and spills.)
template <int DK, int CT>
__global__ __launch_bounds__(NTHREADS_W) void k_fwd_ng(Args p)
{
    typedef LayW<WFwdNg<DK, CT>> Ly;
    __shared__ __attribute__((aligned(16))) char smem[Ly::LDS];
    int* cnt = reinterpret_cast<int*>(smem + Ly::OFF_CNT);
    const int x = blockIdx.x & 7;
    if (threadIdx.x < 3) cnt[threadIdx.x] = 0;
    if (threadIdx.x == 0)
        cnt[3] = __hip_atomic_fetch_add(p.xtick + x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int tk = cnt[3];
    // a counter that did not start at zero (an exchange buffer not
    // zero-filled) is caught here, before it could address past the slots
    const bool bad = tk < 0 || tk >= (int)(gridDim.x >> 3);
    if (bad && threadIdx.x == 0) __hip_atomic_store(p.xerr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int slice = tk % p.nsl;
    const int grp = (tk / p.nsl) * 8 + x;
    const int unit = p.unit_base + grp;
    if (!bad && unit < p.n_units) body_wide<WFwdNg<DK, CT>>(p, unit, slice, smem, grp, 0);
    __syncthreads();
    // (A workgroup issues this increment only after its ticket increment has
    // returned and its unit has run, so the reset below follows every ticket
    // increment in time. An acquire-release increment would say so formally,
    // but it costs an L2 writeback and invalidation at every workgroup's end.)
    if (threadIdx.x == 0 &&
        __hip_atomic_fetch_add(p.xdone, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1) {
        // every workgroup of the grid has taken its ticket and finished
        for (int i = 0; i < 8; ++i) __hip_atomic_store(p.xtick + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(p.xdone, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The state scan alone over each unit's run (no outputs), mapped as k_fwd.
template <int DK>
__global__ __launch_bounds__(NTHREADS_W) void k_fwd_state(Args p)
{
    __shared__ __attribute__((aligned(16))) char smem[LayW<WFwdState<DK>>::LDS];
    const int b = blockIdx.x;
    const int slice = (b >> 3) % p.nsl;
    const int unit = ((b >> 3) / p.nsl) * 8 + (b & 7);
    if (unit >= p.n_units) return;
    body_wide<WFwdState<DK>>(p, unit, slice, smem);
}

// ct: tile length of the output scan (32 or 64 tokens); the state-only scan
// always runs 64-token tiles.
template <int DK>
hipError_t run_fwd(const Args& a, hipStream_t stream, bool out, int ct)
{
    const int grid = ((a.n_units + 7) / 8) * 8 * a.nsl;
    if (!out) hipLaunchKernelGGL(k_fwd_state<DK>, dim3(grid), dim3(NTHREADS_W), 0, stream, a);
    else if (ct == 32) hipLaunchKernelGGL((k_fwd<DK, 32>), dim3(grid), dim3(NTHREADS_W), 0, stream, a);
    else hipLaunchKernelGGL((k_fwd<DK, 64>), dim3(grid), dim3(NTHREADS_W), 0, stream, a);
    return hipGetLastError();
}

// Launches of the fused forward: groups (a multiple of 8, the XCD mapping)
// of at most NG_MAX_WG workgroups each, as the exchange has slots for, in
// turn on the stream.
template <int DK, int CT>
static hipError_t run_fwd_ng(Args a, hipStream_t stream)
{
    const int groups = NG_MAX_WG / a.nsl / 8 * 8;
    for (int base = 0; base < a.n_units; base += groups) {
        a.unit_base = base;
        const int g = min(groups, (a.n_units - base + 7) / 8 * 8);
        hipLaunchKernelGGL((k_fwd_ng<DK, CT>), dim3(g * a.nsl), dim3(NTHREADS_W), 0, stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace scan

static scan::Args fwd_args(const ChunkProblem& p, const void* q, const void* k, const void* v,
                           const float* init_state, float* final_state, void* o)
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
    return a;
}

// Tile length of the bf16 output scans for a chunk length: 32-token tiles for
// chunk 32, else 64 (a 128-token tile does not fit the four-deep LDS ring).
int bf16_tile(int chunk) { return chunk == 32 ? 32 : 64; }

static hipError_t run_fwd_any(const scan::Args& a, int d_k, hipStream_t stream, bool out, int ct)
{
    if (d_k <= 32) return scan::run_fwd<32>(a, stream, out, ct);
    if (d_k <= 64) return scan::run_fwd<64>(a, stream, out, ct);
    return scan::run_fwd<96>(a, stream, out, ct);
}

// The states entering segments 0 .. nseg-1 of dense sequences (ws_in): the
// state scan alone over segments 0 .. nseg-2 keeping the states they leave
// (ws_loc), then the scan of those states, which also copies init_state into
// segment 0's entry.
hipError_t launch_fwd_bf16_seg_states(const ChunkProblem& p, const void* k, const void* v,
                                      const float* init_state, int nseg, int seg_len, float* ws_loc,
                                      float* ws_in, hipStream_t stream)
{
    scan::Args a = fwd_args(p, nullptr, k, v, init_state, nullptr, nullptr);
    a.nseg = nseg;
    a.seg_len = seg_len;
    a.seg_first = 0;
    a.seg_count = nseg - 1;
    a.s_in_seg = nullptr;
    a.s_out_seg = ws_loc;
    a.n_units = p.n_seq * (nseg - 1) * p.H;
    hipError_t e = run_fwd_any(a, p.d_k, stream, false, 64);
    if (e != hipSuccess) return e;
    const int ssz4 = p.d_k * p.d_v / 4;
    hipLaunchKernelGGL(scan::k_seg_scan, dim3((ssz4 + 255) / 256, p.n_seq * p.H), dim3(256), 0, stream,
                       ws_loc, ws_in, p.lambda, p.n_seq, nseg, p.H, ssz4, seg_len, 1, init_state);
    return hipGetLastError();
}

// Segment-parallel bf16 forward of dense sequences (see sgla_chunk_fwd_segmented):
// the state scan of segments 0 .. nseg-2 from zero (segment 0 from
// init_state), the scan of the states, then the forward of every segment from
// its true entering state.
hipError_t launch_fwd_bf16_segmented(const ChunkProblem& p, const void* q, const void* k,
                                     const void* v, const float* init_state, float* final_state,
                                     void* o, int nseg, int seg_len, float* ws_loc, float* ws_in,
                                     hipStream_t stream)
{
    hipError_t e = launch_fwd_bf16_seg_states(p, k, v, init_state, nseg, seg_len, ws_loc, ws_in, stream);
    if (e != hipSuccess) return e;
    scan::Args a = fwd_args(p, q, k, v, init_state, final_state, o);
    a.nseg = nseg;
    a.seg_len = seg_len;
    a.seg_first = 0;
    a.seg_count = nseg;
    a.n_units = p.n_seq * nseg * p.H;
    // segment 0 too starts from ws_in (where the scan copied init_state), so
    // final_state may alias init_state: this launch reads it nowhere
    a.seg_in_all = 1;
    a.s_in_seg = ws_in;
    a.s_out_seg = nullptr;
    return run_fwd_any(a, p.d_k, stream, true, bf16_tile(p.chunk));
}

static_assert(SGLA_FWD_NORM_GATE_EXCHANGE_BYTES ==
                  (size_t)scan::NG_XHEAD + (size_t)scan::NG_MAX_WG * scan::NG_XR * 64 * 8,
              "exchange buffer size");

// bf16 forward with the mixer epilogue fused into the store (see k_fwd_ng).
hipError_t launch_fwd_norm_gate_bf16(const ChunkProblem& p, const void* q, const void* k, const void* v,
                                     const float* init_state, float* final_state, const void* g,
                                     const float* gamma, void* out, void* o, int n_tiers, float eps,
                                     void* exchange, hipStream_t stream)
{
    scan::Args a = fwd_args(p, q, k, v, init_state, final_state, o);
    a.ng_g = reinterpret_cast<const uint16_t*>(g);
    a.ng_gamma = gamma;
    a.ng_out = reinterpret_cast<uint16_t*>(out);
    a.xerr = reinterpret_cast<int*>(exchange);
    a.xtick = a.xerr + scan::NG_XTICK;
    a.xdone = a.xerr + scan::NG_XDONE;
    a.xch = reinterpret_cast<unsigned long long*>(reinterpret_cast<char*>(exchange) + scan::NG_XHEAD);
    a.per_tier = p.H / n_tiers;
    a.inv_dv = 1.0f / (float)p.d_v;
    a.eps = eps;
    const bool t32 = bf16_tile(p.chunk) == 32;
    if (p.d_k <= 32)
        return t32 ? scan::run_fwd_ng<32, 32>(a, stream) : scan::run_fwd_ng<32, 64>(a, stream);
    if (p.d_k <= 64)
        return t32 ? scan::run_fwd_ng<64, 32>(a, stream) : scan::run_fwd_ng<64, 64>(a, stream);
    return t32 ? scan::run_fwd_ng<96, 32>(a, stream) : scan::run_fwd_ng<96, 64>(a, stream);
}

// bf16 forward with d_k <= 96 (padded to 32, 64 or 96) and any d_v (96-column slices).
hipError_t launch_fwd_bf16(const ChunkProblem& p, const void* q, const void* k, const void* v,
                           const float* init_state, float* final_state, void* o,
                           hipStream_t stream)
{
    return run_fwd_any(fwd_args(p, q, k, v, init_state, final_state, o), p.d_k, stream, true,
                       bf16_tile(p.chunk));
}

}  // namespace sgla
