// C-ABI entry points of libsgla (declared in include/sgla.h): argument
// validation on the host, then dispatch to the HIP launchers. Validation runs
// before any HIP call, so every error path can be exercised without a GPU.

#include "sgla.h"

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "sgla_internal.h"

namespace {

thread_local char g_err[512] = "";

sgla_status fail(sgla_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

sgla_status ok()
{
    g_err[0] = '\0';
    return SGLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                          \
    do {                                                                        \
        if ((p) == nullptr) return fail(SGLA_ERR_INVALID_ARG, #p " is NULL");  \
        if (!aligned16(p)) return fail(SGLA_ERR_INVALID_ARG, #p " is not 16-byte aligned"); \
    } while (0)

#define OPTIONAL_PTR(p)                                                         \
    do {                                                                        \
        if ((p) != nullptr && !aligned16(p))                                    \
            return fail(SGLA_ERR_INVALID_ARG, #p " is not 16-byte aligned");   \
    } while (0)

// Shared checks of the chunked entry points; fills the launch description.
sgla_status check_chunk(const void* q, const void* k, const void* v, const float* lambda,
                        const float* a, const int32_t* cu_seqlens, int n_seq, int B, int H,
                        int T, int d_k, int d_v, int chunk, sgla_dtype dtype,
                        sgla::ChunkProblem* out)
{
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(lambda);
    OPTIONAL_PTR(a);
    if (dtype != SGLA_F32 && dtype != SGLA_BF16)
        return fail(SGLA_ERR_INVALID_ARG, "dtype %d is not SGLA_F32 or SGLA_BF16", (int)dtype);
    if (B <= 0 || H <= 0 || T <= 0 || d_k <= 0 || d_v <= 0)
        return fail(SGLA_ERR_INVALID_ARG, "sizes must be positive (B=%d H=%d T=%d d_k=%d d_v=%d)",
                    B, H, T, d_k, d_v);
    if (cu_seqlens != nullptr) {
        if (!aligned16(cu_seqlens)) return fail(SGLA_ERR_INVALID_ARG, "cu_seqlens is not 16-byte aligned");
        if (B != 1) return fail(SGLA_ERR_INVALID_ARG, "packed input (cu_seqlens) needs B == 1, got %d", B);
        if (n_seq <= 0) return fail(SGLA_ERR_INVALID_ARG, "n_seq must be positive, got %d", n_seq);
    } else {
        n_seq = B;
    }
    // element counts must fit the kernels' 64-bit offsets and int grid sizes
    const double toks = (double)B * H * T;
    if (toks * (d_k > d_v ? d_k : d_v) > 9.0e18 || (double)n_seq * H > 2.0e8)
        return fail(SGLA_ERR_INVALID_ARG, "problem too large");
    if (dtype == SGLA_BF16) {
        if (d_k > 96 || d_v > 192 || d_k % 8 != 0 || d_v % 8 != 0)
            return fail(SGLA_ERR_UNSUPPORTED,
                        "bf16 needs d_k <= 96 and d_v <= 192, multiples of 8 (got %d, %d)", d_k, d_v);
        if (chunk != 32 && chunk != 64 && chunk != 128)
            return fail(SGLA_ERR_UNSUPPORTED, "bf16 chunk must be 32, 64 or 128, got %d", chunk);
    } else {
        if (d_k > 96 || d_v > 192 || d_k % 4 != 0 || d_v % 4 != 0)
            return fail(SGLA_ERR_UNSUPPORTED,
                        "f32 needs d_k <= 96 and d_v <= 192, multiples of 4 (got %d, %d)", d_k, d_v);
        if (chunk != 32 && chunk != 64 && chunk != 128)
            return fail(SGLA_ERR_UNSUPPORTED, "f32 chunk must be 32, 64 or 128, got %d", chunk);
    }
    out->bf16 = dtype == SGLA_BF16;
    out->B = B;
    out->H = H;
    out->T = T;
    out->n_seq = n_seq;
    out->d_k = d_k;
    out->d_v = d_v;
    out->chunk = chunk;
    out->lambda = lambda;
    out->a = a;
    out->cu = cu_seqlens;
    return SGLA_OK;
}

bool overlaps(const void* x, size_t nx, const void* y, size_t ny)
{
    if (x == nullptr || y == nullptr) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(x), b0 = reinterpret_cast<uintptr_t>(y);
    return a0 < b0 + ny && b0 < a0 + nx;
}

}  // namespace

namespace sgla {
// Sets the calling thread's error message for entry points defined in other
// source files.
sgla_status api_fail(sgla_status st, const char* msg)
{
    return fail(st, "%s", msg);
}
}  // namespace sgla

extern "C" {

int sgla_version(void) { return 100; }

const char* sgla_status_str(int status)
{
    switch (status) {
    case SGLA_OK: return "SGLA_OK";
    case SGLA_ERR_INVALID_ARG: return "SGLA_ERR_INVALID_ARG";
    case SGLA_ERR_UNSUPPORTED: return "SGLA_ERR_UNSUPPORTED";
    case SGLA_ERR_WORKSPACE: return "SGLA_ERR_WORKSPACE";
    case SGLA_ERR_HIP: return "SGLA_ERR_HIP";
    default: return "unknown sgla_status";
    }
}

const char* sgla_last_error(void) { return g_err; }

sgla_status sgla_decay_schedule(int H, double t_min, double t_max, float* lambda_out)
{
    if (lambda_out == nullptr) return fail(SGLA_ERR_INVALID_ARG, "lambda_out is NULL");
    if (H <= 0) return fail(SGLA_ERR_INVALID_ARG, "H must be positive, got %d", H);
    if (!std::isfinite(t_min) || !std::isfinite(t_max) || t_min <= 0.0 || t_max < t_min)
        return fail(SGLA_ERR_INVALID_ARG, "need 0 < t_min <= t_max (got %g, %g)", t_min, t_max);
    // half-lives geometric in the head index, endpoints included
    const double ratio = t_max / t_min;
    for (int h = 0; h < H; ++h) {
        const double e = (H == 1) ? 0.0 : (double)h / (double)(H - 1);
        const double half_life = t_min * std::pow(ratio, e);
        lambda_out[h] = (float)std::pow(2.0, -1.0 / half_life);
    }
    return ok();
}

// final_state (n_seq states) may be init_state itself (in-place carry) but may
// not overlap it otherwise, nor q, k, v or o: workgroups read one sequence's
// initial state while others write their final states.
static sgla_status check_final_state(const float* final_state, const float* init_state, const void* q,
                                     const void* k, const void* v, const void* o, int n_seq, int H,
                                     int d_k, int d_v, size_t nqk, size_t nvo)
{
    if (final_state == nullptr) return SGLA_OK;
    const size_t nst = (size_t)n_seq * H * d_k * d_v * sizeof(float);
    if (final_state != init_state && overlaps(final_state, nst, init_state, nst))
        return fail(SGLA_ERR_INVALID_ARG, "final_state must equal init_state or not overlap it");
    if (overlaps(final_state, nst, q, nqk) || overlaps(final_state, nst, k, nqk) ||
        overlaps(final_state, nst, v, nvo) || overlaps(final_state, nst, o, nvo))
        return fail(SGLA_ERR_INVALID_ARG, "final_state must not overlap q, k, v or o");
    return SGLA_OK;
}

// Every buffer a call writes must be disjoint from every buffer it reads and
// from every other one it writes (an in-place buffer is listed once, as
// written).
struct Span {
    const void* p;
    size_t n;
    const char* name;
};
static sgla_status check_disjoint(const Span* wr, int nw, const Span* rd, int nr)
{
    for (int i = 0; i < nw; ++i) {
        const sgla_status code = std::strcmp(wr[i].name, "workspace") == 0 ? SGLA_ERR_WORKSPACE
                                                                          : SGLA_ERR_INVALID_ARG;
        for (int j = 0; j < nr; ++j)
            if (overlaps(wr[i].p, wr[i].n, rd[j].p, rd[j].n))
                return fail(code, "%s must not overlap %s", wr[i].name, rd[j].name);
        for (int j = 0; j < i; ++j)
            if (overlaps(wr[i].p, wr[i].n, wr[j].p, wr[j].n))
                return fail(code, "%s must not overlap %s", wr[i].name, wr[j].name);
    }
    return SGLA_OK;
}

static sgla_status check_bwd_all(const void* q, const void* k, const void* v, const void* dO,
                                 const float* lambda, const float* a, const float* init_state,
                                 const float* d_final_state, void* dq, void* dk, void* dv, float* da,
                                 float* d_init_state, void* workspace, size_t ws_bytes, int n_seq, int B,
                                 int H, int T, int d_k, int d_v, size_t es)
{
    const size_t nqk = (size_t)B * H * T * d_k * es, nvo = (size_t)B * H * T * d_v * es;
    const size_t nst = (size_t)n_seq * H * d_k * d_v * sizeof(float);
    const size_t nda = (size_t)H * d_k * sizeof(float);
    const Span rd[8] = {{q, nqk, "q"}, {k, nqk, "k"}, {v, nvo, "v"}, {dO, nvo, "dO"},
                        {lambda, (size_t)H * sizeof(float), "lambda"}, {a, nda, "a"},
                        {init_state, nst, "init_state"}, {d_final_state, nst, "d_final_state"}};
    const Span wr[6] = {{dq, nqk, "dq"}, {dk, nqk, "dk"}, {dv, nvo, "dv"}, {da, nda, "da"},
                        {d_init_state, nst, "d_init_state"}, {workspace, ws_bytes, "workspace"}};
    return check_disjoint(wr, 6, rd, 8);
}

}  // extern "C"

namespace sgla {
// Every argument check of the chunked backward except those of its workspace
// (sizes, pointers, alignment, and the overlaps among the other buffers).
sgla_status check_chunk_bwd(const void* q, const void* k, const void* v, const void* dO, const float* lambda,
                            const float* a, const float* init_state, const float* d_final_state, void* dq,
                            void* dk, void* dv, float* da, float* d_init_state, const int32_t* cu_seqlens,
                            int n_seq, int B, int H, int T, int d_k, int d_v, int chunk, sgla_dtype dtype,
                            ChunkProblem* p)
{
    sgla_status st = check_chunk(q, k, v, lambda, a, cu_seqlens, n_seq, B, H, T, d_k, d_v, chunk, dtype, p);
    if (st != SGLA_OK) return st;
    REQUIRE_PTR(dO);
    REQUIRE_PTR(dq);
    REQUIRE_PTR(dk);
    REQUIRE_PTR(dv);
    REQUIRE_PTR(da);
    OPTIONAL_PTR(init_state);
    OPTIONAL_PTR(d_final_state);
    OPTIONAL_PTR(d_init_state);
    return check_bwd_all(q, k, v, dO, lambda, a, init_state, d_final_state, dq, dk, dv, da, d_init_state,
                         nullptr, 0, p->n_seq, B, H, T, d_k, d_v, (dtype == SGLA_BF16) ? 2 : 4);
}
}  // namespace sgla

extern "C" {

sgla_status sgla_chunk_fwd(const void* q, const void* k, const void* v, const float* lambda,
                           const float* a, const float* init_state, float* final_state, void* o,
                           const int32_t* cu_seqlens, int n_seq, int B, int H, int T, int d_k,
                           int d_v, int chunk, sgla_dtype dtype, void* hip_stream)
{
    sgla::ChunkProblem p;
    sgla_status st = check_chunk(q, k, v, lambda, a, cu_seqlens, n_seq, B, H, T, d_k, d_v, chunk,
                                 dtype, &p);
    if (st != SGLA_OK) return st;
    REQUIRE_PTR(o);
    OPTIONAL_PTR(init_state);
    OPTIONAL_PTR(final_state);
    const size_t es = (dtype == SGLA_BF16) ? 2 : 4;
    const size_t nqk = (size_t)B * H * T * d_k * es, nvo = (size_t)B * H * T * d_v * es;
    if (overlaps(o, nvo, q, nqk) || overlaps(o, nvo, k, nqk) || overlaps(o, nvo, v, nvo))
        return fail(SGLA_ERR_INVALID_ARG, "o must not alias q, k or v");
    st = check_final_state(final_state, init_state, q, k, v, o, p.n_seq, H, d_k, d_v, nqk, nvo);
    if (st != SGLA_OK) return st;
    hipError_t e = sgla::launch_chunk_fwd(p, q, k, v, init_state, final_state, o,
                                          reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SGLA_ERR_HIP, "chunk_fwd launch: %s", hipGetErrorString(e));
    return ok();
}

sgla_status sgla_chunk_fwd_norm_gate(const void* q, const void* k, const void* v, const float* lambda,
                                     const float* a, const float* init_state, float* final_state, const void* g,
                                     const float* gamma, void* out, void* o, const int32_t* cu_seqlens, int n_seq,
                                     int B, int H, int T, int d_k, int d_v, int chunk, int n_tiers, float eps,
                                     sgla_dtype dtype, void* exchange, size_t exchange_bytes, unsigned flags,
                                     void* hip_stream)
{
    sgla::ChunkProblem p;
    sgla_status st = check_chunk(q, k, v, lambda, a, cu_seqlens, n_seq, B, H, T, d_k, d_v, chunk,
                                 dtype, &p);
    if (st != SGLA_OK) return st;
    if (dtype != SGLA_BF16)
        return fail(SGLA_ERR_UNSUPPORTED, "the fused forward and epilogue is bf16 only");
    if (flags != 0u) return fail(SGLA_ERR_INVALID_ARG, "unknown flags 0x%x (none are defined)", flags);
    REQUIRE_PTR(g);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(o);
    OPTIONAL_PTR(gamma);
    OPTIONAL_PTR(init_state);
    OPTIONAL_PTR(final_state);
    if (exchange == nullptr || !aligned16(exchange))
        return fail(SGLA_ERR_WORKSPACE, "exchange must be a 16-byte aligned device buffer");
    if (exchange_bytes < SGLA_FWD_NORM_GATE_EXCHANGE_BYTES)
        return fail(SGLA_ERR_WORKSPACE, "exchange holds %zu bytes, needs %zu", exchange_bytes,
                    (size_t)SGLA_FWD_NORM_GATE_EXCHANGE_BYTES);
    if (n_tiers <= 0 || H % n_tiers != 0)
        return fail(SGLA_ERR_INVALID_ARG, "n_tiers (%d) must be positive and divide H (%d)", n_tiers, H);
    // the kernel addresses a tile's token rows (H d_v elements apart) with 32-bit offsets
    if ((long long)H * d_v > (1LL << 24))
        return fail(SGLA_ERR_UNSUPPORTED, "H * d_v must be at most 2^24 (got %lld)", (long long)H * d_v);
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return fail(SGLA_ERR_INVALID_ARG, "eps must be finite and >= 0 (got %g)", (double)eps);
    const size_t nqk = (size_t)B * H * T * d_k * 2, nvo = (size_t)B * H * T * d_v * 2;
    const size_t nst = (size_t)p.n_seq * H * d_k * d_v * sizeof(float);
    const size_t nexc = SGLA_FWD_NORM_GATE_EXCHANGE_BYTES;
    st = check_final_state(final_state, init_state, q, k, v, o, p.n_seq, H, d_k, d_v, nqk, nvo);
    if (st != SGLA_OK) return st;
    // out may be g itself (each lane reads its gate values before it writes
    // them), and final_state init_state (in-place carry): then only the
    // written buffer is listed
    const Span rd[8] = {{q, nqk, "q"}, {k, nqk, "k"}, {v, nvo, "v"}, {lambda, (size_t)H * sizeof(float), "lambda"},
                        {a, (size_t)H * d_k * sizeof(float), "a"},
                        {final_state == init_state ? nullptr : init_state, nst, "init_state"},
                        {gamma, (size_t)n_tiers * d_v * sizeof(float), "gamma"}, {out == g ? nullptr : g, nvo, "g"}};
    const Span wr[4] = {{out, nvo, "out"}, {o, nvo, "o"}, {final_state, nst, "final_state"},
                        {exchange, nexc, "workspace"}};
    st = check_disjoint(wr, 4, rd, 8);
    if (st != SGLA_OK) return st;
    hipError_t e = sgla::launch_fwd_norm_gate_bf16(p, q, k, v, init_state, final_state, g, gamma, out, o, n_tiers,
                                                   eps, exchange, reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SGLA_ERR_HIP, "chunk_fwd_norm_gate launch: %s", hipGetErrorString(e));
    return ok();
}

size_t sgla_chunk_fwd_segmented_workspace_bytes(int B, int H, int d_k, int d_v, int n_segments)
{
    if (B <= 0 || H <= 0 || d_k <= 0 || d_v <= 0 || n_segments <= 0) return 0;
    return 2 * (size_t)B * n_segments * H * d_k * d_v * sizeof(float);
}

sgla_status sgla_chunk_fwd_segmented(const void* q, const void* k, const void* v,
                                     const float* lambda, const float* a,
                                     const float* init_state, float* final_state, void* o,
                                     int B, int H, int T, int d_k, int d_v, int chunk,
                                     sgla_dtype dtype, int n_segments, void* workspace,
                                     size_t workspace_bytes, void* hip_stream)
{
    sgla::ChunkProblem p;
    sgla_status st = check_chunk(q, k, v, lambda, a, nullptr, 0, B, H, T, d_k, d_v, chunk, dtype, &p);
    if (st != SGLA_OK) return st;
    if (dtype != SGLA_BF16)
        return fail(SGLA_ERR_UNSUPPORTED, "the segmented forward needs SGLA_BF16");
    if (n_segments <= 0) return fail(SGLA_ERR_INVALID_ARG, "n_segments must be positive, got %d", n_segments);
    REQUIRE_PTR(o);
    OPTIONAL_PTR(init_state);
    OPTIONAL_PTR(final_state);
    const size_t need = sgla_chunk_fwd_segmented_workspace_bytes(B, H, d_k, d_v, n_segments);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
        return fail(SGLA_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu at %p)",
                    need, workspace_bytes, workspace);
    const size_t nqk = (size_t)B * H * T * d_k * 2, nvo = (size_t)B * H * T * d_v * 2;
    if (overlaps(o, nvo, q, nqk) || overlaps(o, nvo, k, nqk) || overlaps(o, nvo, v, nvo))
        return fail(SGLA_ERR_INVALID_ARG, "o must not alias q, k or v");
    st = check_final_state(final_state, init_state, q, k, v, o, p.n_seq, H, d_k, d_v, nqk, nvo);
    if (st != SGLA_OK) return st;
    {
        const size_t nst = (size_t)p.n_seq * H * d_k * d_v * sizeof(float);
        if (overlaps(workspace, need, q, nqk) || overlaps(workspace, need, k, nqk) ||
            overlaps(workspace, need, v, nvo) || overlaps(workspace, need, o, nvo) ||
            overlaps(workspace, need, init_state, nst) || overlaps(workspace, need, final_state, nst))
            return fail(SGLA_ERR_WORKSPACE, "workspace must not overlap any other argument");
    }
    // segments of whole 64-token tiles (the tile of the bf16 kernels)
    const int tiles = (T + 63) / 64;
    const int g = n_segments < tiles ? n_segments : tiles;
    const int seg_len = ((tiles + g - 1) / g) * 64;
    const int nseg = (T + seg_len - 1) / seg_len;
    const hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
    hipError_t e;
    if (nseg <= 1) {
        e = sgla::launch_chunk_fwd(p, q, k, v, init_state, final_state, o, stream);
    } else {
        float* ws_loc = reinterpret_cast<float*>(workspace);
        float* ws_in = ws_loc + (size_t)B * nseg * H * d_k * d_v;
        e = sgla::launch_fwd_bf16_segmented(p, q, k, v, init_state, final_state, o, nseg, seg_len,
                                            ws_loc, ws_in, stream);
    }
    if (e != hipSuccess) return fail(SGLA_ERR_HIP, "chunk_fwd_segmented launch: %s", hipGetErrorString(e));
    return ok();
}

size_t sgla_chunk_bwd_segmented_workspace_bytes(int B, int H, int d_k, int d_v, int n_segments)
{
    if (B <= 0 || H <= 0 || d_k <= 0 || d_v <= 0 || n_segments <= 0) return 0;
    const size_t units = (size_t)B * n_segments * H;
    return (4 * units * d_k * d_v + units * d_k) * sizeof(float);
}

sgla_status sgla_chunk_bwd_segmented(const void* q, const void* k, const void* v, const void* dO,
                                     const float* lambda, const float* a, const float* init_state,
                                     const float* d_final_state, void* dq, void* dk, void* dv, float* da,
                                     float* d_init_state, int B, int H, int T, int d_k, int d_v, int chunk,
                                     sgla_dtype dtype, int n_segments, void* workspace, size_t workspace_bytes,
                                     void* hip_stream)
{
    sgla::ChunkProblem p;
    sgla_status st = check_chunk(q, k, v, lambda, a, nullptr, 0, B, H, T, d_k, d_v, chunk, dtype, &p);
    if (st != SGLA_OK) return st;
    if (dtype != SGLA_BF16)
        return fail(SGLA_ERR_UNSUPPORTED, "the segmented backward needs SGLA_BF16");
    if (n_segments <= 0) return fail(SGLA_ERR_INVALID_ARG, "n_segments must be positive, got %d", n_segments);
    REQUIRE_PTR(dO);
    REQUIRE_PTR(dq);
    REQUIRE_PTR(dk);
    REQUIRE_PTR(dv);
    REQUIRE_PTR(da);
    OPTIONAL_PTR(init_state);
    OPTIONAL_PTR(d_final_state);
    OPTIONAL_PTR(d_init_state);
    const size_t need = sgla_chunk_bwd_segmented_workspace_bytes(B, H, d_k, d_v, n_segments);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
        return fail(SGLA_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu at %p)",
                    need, workspace_bytes, workspace);
    st = check_bwd_all(q, k, v, dO, lambda, a, init_state, d_final_state, dq, dk, dv, da, d_init_state,
                       workspace, need, p.n_seq, B, H, T, d_k, d_v, 2);
    if (st != SGLA_OK) return st;
    const int tiles = (T + 63) / 64;
    const int g = n_segments < tiles ? n_segments : tiles;
    const int seg_len = ((tiles + g - 1) / g) * 64;
    const int nseg = (T + seg_len - 1) / seg_len;
    const hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
    float* ws = reinterpret_cast<float*>(workspace);
    const size_t arr4 = 4 * (size_t)B * n_segments * H * d_k * d_v;
    hipError_t e;
    if (nseg <= 1) {
        e = sgla::launch_chunk_bwd(p, q, k, v, dO, init_state, d_final_state, dq, dk, dv, da, d_init_state,
                                   ws + arr4, stream);
    } else {
        // the four state arrays are sized for nseg <= n_segments segments
        const size_t arr = (size_t)B * nseg * H * d_k * d_v;
        e = sgla::launch_bwd_bf16_segmented(p, q, k, v, dO, init_state, d_final_state, dq, dk, dv, da,
                                            d_init_state, ws + 4 * arr, nseg, seg_len, ws, stream);
    }
    if (e != hipSuccess) return fail(SGLA_ERR_HIP, "chunk_bwd_segmented launch: %s", hipGetErrorString(e));
    return ok();
}

size_t sgla_chunk_bwd_workspace_bytes(int N, int H, int d_k)
{
    if (N <= 0 || H <= 0 || d_k <= 0) return 0;
    return (size_t)N * H * d_k * sizeof(float);
}

sgla_status sgla_chunk_bwd(const void* q, const void* k, const void* v, const void* dO,
                           const float* lambda, const float* a, const float* init_state,
                           const float* d_final_state, void* dq, void* dk, void* dv, float* da,
                           float* d_init_state, const int32_t* cu_seqlens, int n_seq, int B,
                           int H, int T, int d_k, int d_v, int chunk, sgla_dtype dtype,
                           void* workspace, size_t workspace_bytes, void* hip_stream)
{
    sgla::ChunkProblem p;
    sgla_status st = sgla::check_chunk_bwd(q, k, v, dO, lambda, a, init_state, d_final_state, dq, dk, dv, da,
                                           d_init_state, cu_seqlens, n_seq, B, H, T, d_k, d_v, chunk, dtype,
                                           &p);
    if (st != SGLA_OK) return st;
    const size_t need = sgla_chunk_bwd_workspace_bytes(p.n_seq, H, d_k);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
        return fail(SGLA_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu at %p)",
                    need, workspace_bytes, workspace);
    st = check_bwd_all(q, k, v, dO, lambda, a, init_state, d_final_state, dq, dk, dv, da, d_init_state,
                       workspace, need, p.n_seq, B, H, T, d_k, d_v, (dtype == SGLA_BF16) ? 2 : 4);
    if (st != SGLA_OK) return st;
    hipError_t e = sgla::launch_chunk_bwd(p, q, k, v, dO, init_state, d_final_state, dq, dk, dv,
                                          da, d_init_state, reinterpret_cast<float*>(workspace),
                                          reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SGLA_ERR_HIP, "chunk_bwd launch: %s", hipGetErrorString(e));
    return ok();
}

sgla_status sgla_decode_step(const void* q, const void* k, const void* v, const float* lambda,
                             const float* a, float* state, const int32_t* slot, void* o, int N,
                             int P, int H, int d_k, int d_v, sgla_dtype dtype, void* hip_stream)
{
    REQUIRE_PTR(q);
    REQUIRE_PTR(k);
    REQUIRE_PTR(v);
    REQUIRE_PTR(lambda);
    REQUIRE_PTR(state);
    REQUIRE_PTR(o);
    OPTIONAL_PTR(a);
    OPTIONAL_PTR(slot);
    if (dtype != SGLA_F32 && dtype != SGLA_BF16)
        return fail(SGLA_ERR_INVALID_ARG, "dtype %d is not SGLA_F32 or SGLA_BF16", (int)dtype);
    if (N <= 0 || P <= 0 || H <= 0)
        return fail(SGLA_ERR_INVALID_ARG, "N, P, H must be positive (N=%d P=%d H=%d)", N, P, H);
    if (slot == nullptr && P < N)
        return fail(SGLA_ERR_INVALID_ARG, "without slot, the pool needs P >= N (P=%d N=%d)", P, N);
    if ((double)N * H > 2.0e9) return fail(SGLA_ERR_INVALID_ARG, "N*H too large");
    if (d_k < 4 || d_k > 96 || d_k % 4 != 0 || d_v < 4 || d_v > 192 || d_v % 4 != 0)
        return fail(SGLA_ERR_UNSUPPORTED,
                    "decode needs d_k in 4..96 and d_v in 4..192, multiples of 4 (got %d, %d)", d_k, d_v);
    {
        const size_t es = (dtype == SGLA_BF16) ? 2 : 4;
        const size_t nqk = (size_t)N * H * d_k * es, nvo = (size_t)N * H * d_v * es;
        const Span rd[6] = {{q, nqk, "q"}, {k, nqk, "k"}, {v, nvo, "v"},
                            {lambda, (size_t)H * sizeof(float), "lambda"},
                            {a, (size_t)H * d_k * sizeof(float), "a"},
                            {slot, (size_t)N * sizeof(int32_t), "slot"}};
        const Span wr[2] = {{state, (size_t)P * H * d_k * d_v * sizeof(float), "state"}, {o, nvo, "o"}};
        const sgla_status st = check_disjoint(wr, 2, rd, 6);
        if (st != SGLA_OK) return st;
    }
    hipError_t e = sgla::launch_decode_step(dtype == SGLA_BF16, q, k, v, lambda, a, state, slot, o,
                                            N, P, H, d_k, d_v,
                                            reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SGLA_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
    return ok();
}

sgla_status sgla_conv_fwd(const void* u, const float* w, const float* b, const float* init_state,
                          float* final_state, void* y, const int32_t* cu_seqlens, int n_seq, int B, int T,
                          int D, sgla_dtype dtype, void* hip_stream)
{
    REQUIRE_PTR(u);
    REQUIRE_PTR(w);
    REQUIRE_PTR(y);
    OPTIONAL_PTR(b);
    OPTIONAL_PTR(init_state);
    OPTIONAL_PTR(final_state);
    if (dtype != SGLA_F32 && dtype != SGLA_BF16)
        return fail(SGLA_ERR_INVALID_ARG, "dtype %d is not SGLA_F32 or SGLA_BF16", (int)dtype);
    if (B <= 0 || T <= 0 || D <= 0)
        return fail(SGLA_ERR_INVALID_ARG, "sizes must be positive (B=%d T=%d D=%d)", B, T, D);
    if (cu_seqlens != nullptr) {
        if (B != 1) return fail(SGLA_ERR_INVALID_ARG, "packed sequences need B = 1 (got %d)", B);
        if (n_seq <= 0) return fail(SGLA_ERR_INVALID_ARG, "n_seq must be positive (got %d)", n_seq);
        if (!aligned16(cu_seqlens)) return fail(SGLA_ERR_INVALID_ARG, "cu_seqlens is not 16-byte aligned");
    } else if (n_seq != B) {
        return fail(SGLA_ERR_INVALID_ARG, "dense input needs n_seq == B (got %d, %d)", n_seq, B);
    }
    if ((double)B * T * D > 4.0e9) return fail(SGLA_ERR_INVALID_ARG, "B*T*D too large");
    const int vec = (dtype == SGLA_BF16) ? 8 : 4;
    if (D % vec != 0)
        return fail(SGLA_ERR_UNSUPPORTED, "D must be a multiple of %d for this dtype (got %d)", vec, D);
    const size_t nb = (size_t)B * T * D * (dtype == SGLA_BF16 ? 2 : 4);
    const size_t ns = (size_t)n_seq * 3 * D * sizeof(float);
    if (overlaps(y, nb, u, nb)) return fail(SGLA_ERR_INVALID_ARG, "y must not overlap u");
    if (overlaps(y, nb, init_state, ns)) return fail(SGLA_ERR_INVALID_ARG, "y must not overlap init_state");
    if (overlaps(final_state, ns, u, nb) || overlaps(final_state, ns, y, nb))
        return fail(SGLA_ERR_INVALID_ARG, "final_state must not overlap u or y");
    if (final_state != init_state && overlaps(final_state, ns, init_state, ns))
        return fail(SGLA_ERR_INVALID_ARG, "final_state must equal init_state or not overlap it");
    hipError_t e = sgla::launch_conv_fwd(dtype == SGLA_BF16, u, w, b, init_state, final_state, y, cu_seqlens,
                                         n_seq, B, T, D, reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SGLA_ERR_HIP, "conv_fwd launch: %s", hipGetErrorString(e));
    return ok();
}

size_t sgla_conv_bwd_workspace_bytes(int B, int T, int D)
{
    if (B <= 0 || T <= 0 || D <= 0) return 0;
    return sgla::conv_bwd_part_floats(B, T, D, 0) * sizeof(float);
}

sgla_status sgla_conv_bwd(const void* u, const float* w, const float* b, const float* init_state, const void* dy,
                          const float* d_final_state, void* du, float* dw, float* db, float* d_init_state,
                          const int32_t* cu_seqlens, int n_seq, int B, int T, int D, sgla_dtype dtype,
                          void* workspace, size_t workspace_bytes, void* hip_stream)
{
    REQUIRE_PTR(u);
    REQUIRE_PTR(w);
    REQUIRE_PTR(dy);
    REQUIRE_PTR(du);
    REQUIRE_PTR(dw);
    OPTIONAL_PTR(b);
    OPTIONAL_PTR(init_state);
    OPTIONAL_PTR(d_final_state);
    OPTIONAL_PTR(db);
    OPTIONAL_PTR(d_init_state);
    if (dtype != SGLA_F32 && dtype != SGLA_BF16)
        return fail(SGLA_ERR_INVALID_ARG, "dtype %d is not SGLA_F32 or SGLA_BF16", (int)dtype);
    if (B <= 0 || T <= 0 || D <= 0)
        return fail(SGLA_ERR_INVALID_ARG, "sizes must be positive (B=%d T=%d D=%d)", B, T, D);
    if (cu_seqlens != nullptr) {
        if (B != 1) return fail(SGLA_ERR_INVALID_ARG, "packed sequences need B = 1 (got %d)", B);
        if (n_seq <= 0) return fail(SGLA_ERR_INVALID_ARG, "n_seq must be positive (got %d)", n_seq);
        if (!aligned16(cu_seqlens)) return fail(SGLA_ERR_INVALID_ARG, "cu_seqlens is not 16-byte aligned");
    } else if (n_seq != B) {
        return fail(SGLA_ERR_INVALID_ARG, "dense input needs n_seq == B (got %d, %d)", n_seq, B);
    }
    if ((double)B * T * D > 4.0e9) return fail(SGLA_ERR_INVALID_ARG, "B*T*D too large");
    const int vec = (dtype == SGLA_BF16) ? 8 : 4;
    if (D % vec != 0)
        return fail(SGLA_ERR_UNSUPPORTED, "D must be a multiple of %d for this dtype (got %d)", vec, D);
    const size_t need = sgla_conv_bwd_workspace_bytes(B, T, D);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
        return fail(SGLA_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu at %p)", need,
                    workspace_bytes, workspace);
    const size_t nb = (size_t)B * T * D * (dtype == SGLA_BF16 ? 2 : 4);
    const size_t ns = (size_t)n_seq * 3 * D * sizeof(float);
    if (overlaps(du, nb, u, nb) || overlaps(du, nb, dy, nb))
        return fail(SGLA_ERR_INVALID_ARG, "du must not overlap u or dy");
    if (overlaps(d_init_state, ns, du, nb) || overlaps(d_init_state, ns, init_state, ns) ||
        overlaps(d_init_state, ns, d_final_state, ns))
        return fail(SGLA_ERR_INVALID_ARG, "d_init_state must not overlap du, init_state or d_final_state");
    {
        const Span rd[6] = {{u, nb, "u"}, {dy, nb, "dy"}, {w, (size_t)D * 4 * sizeof(float), "w"},
                            {b, (size_t)D * sizeof(float), "b"}, {init_state, ns, "init_state"},
                            {d_final_state, ns, "d_final_state"}};
        const Span wr[5] = {{du, nb, "du"}, {dw, (size_t)D * 4 * sizeof(float), "dw"},
                            {db, (size_t)D * sizeof(float), "db"}, {d_init_state, ns, "d_init_state"},
                            {workspace, need, "workspace"}};
        const sgla_status st = check_disjoint(wr, 5, rd, 6);
        if (st != SGLA_OK) return st;
    }
    hipError_t e = sgla::launch_conv_bwd(dtype == SGLA_BF16, u, dy, w, b, init_state, d_final_state, du, dw, db,
                                         d_init_state, cu_seqlens, n_seq, B, T, D,
                                         reinterpret_cast<float*>(workspace), reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SGLA_ERR_HIP, "conv_bwd launch: %s", hipGetErrorString(e));
    return ok();
}

sgla_status sgla_conv_decode_step(const void* x, const float* w, const float* b, float* state,
                                  const int32_t* slot, void* y, int N, int P, int D, sgla_dtype dtype,
                                  void* hip_stream)
{
    REQUIRE_PTR(x);
    REQUIRE_PTR(w);
    REQUIRE_PTR(state);
    REQUIRE_PTR(y);
    OPTIONAL_PTR(b);
    OPTIONAL_PTR(slot);
    if (dtype != SGLA_F32 && dtype != SGLA_BF16)
        return fail(SGLA_ERR_INVALID_ARG, "dtype %d is not SGLA_F32 or SGLA_BF16", (int)dtype);
    if (N <= 0 || P <= 0 || D <= 0)
        return fail(SGLA_ERR_INVALID_ARG, "N, P, D must be positive (N=%d P=%d D=%d)", N, P, D);
    if (slot == nullptr && P < N)
        return fail(SGLA_ERR_INVALID_ARG, "without slot, the pool needs P >= N (P=%d N=%d)", P, N);
    if ((double)P * 3 * D > 4.0e9 || (double)N * D > 4.0e9) return fail(SGLA_ERR_INVALID_ARG, "N*D or P*D too large");
    const int vec = (dtype == SGLA_BF16) ? 8 : 4;
    if (D % vec != 0)
        return fail(SGLA_ERR_UNSUPPORTED, "D must be a multiple of %d for this dtype (got %d)", vec, D);
    const size_t nx = (size_t)N * D * (dtype == SGLA_BF16 ? 2 : 4), ps = (size_t)P * 3 * D * sizeof(float);
    if (overlaps(y, nx, x, nx)) return fail(SGLA_ERR_INVALID_ARG, "y must not overlap x");
    if (overlaps(state, ps, x, nx) || overlaps(state, ps, y, nx))
        return fail(SGLA_ERR_INVALID_ARG, "state must not overlap x or y");
    hipError_t e = sgla::launch_conv_decode(dtype == SGLA_BF16, x, w, b, state, slot, y, N, P, D,
                                            reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SGLA_ERR_HIP, "conv decode launch: %s", hipGetErrorString(e));
    return ok();
}

sgla_status sgla_head_norm_gate(const void* o, const void* g, const float* gamma, void* out, int B, int H,
                                int T, int d_v, int n_tiers, float eps, sgla_dtype dtype, void* hip_stream)
{
    REQUIRE_PTR(o);
    REQUIRE_PTR(g);
    REQUIRE_PTR(out);
    OPTIONAL_PTR(gamma);
    if (dtype != SGLA_F32 && dtype != SGLA_BF16)
        return fail(SGLA_ERR_INVALID_ARG, "dtype %d is not SGLA_F32 or SGLA_BF16", (int)dtype);
    if (B <= 0 || H <= 0 || T <= 0 || d_v <= 0 || n_tiers <= 0)
        return fail(SGLA_ERR_INVALID_ARG, "sizes must be positive (B=%d H=%d T=%d d_v=%d n_tiers=%d)", B, H, T,
                    d_v, n_tiers);
    if (H % n_tiers != 0)
        return fail(SGLA_ERR_INVALID_ARG, "n_tiers (%d) must divide H (%d)", n_tiers, H);
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return fail(SGLA_ERR_INVALID_ARG, "eps must be finite and >= 0 (got %g)", (double)eps);
    if ((double)B * H * T * d_v > 2.0e9) return fail(SGLA_ERR_INVALID_ARG, "B*H*T*d_v too large");
    if (d_v % 4 != 0 || d_v > 256)
        return fail(SGLA_ERR_UNSUPPORTED, "d_v must be a multiple of 4, at most 256 (got %d)", d_v);
    const size_t nb = (size_t)B * H * T * d_v * (dtype == SGLA_BF16 ? 2 : 4);
    if (overlaps(out, nb, o, nb)) return fail(SGLA_ERR_INVALID_ARG, "out must not overlap o");
    if (out != g && overlaps(out, nb, g, nb))
        return fail(SGLA_ERR_INVALID_ARG, "out must equal g or not overlap it");
    hipError_t e = sgla::launch_head_norm_gate(dtype == SGLA_BF16, o, g, gamma, out, B, H, T, d_v, n_tiers, eps,
                                               reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SGLA_ERR_HIP, "head_norm_gate launch: %s", hipGetErrorString(e));
    return ok();
}

size_t sgla_head_norm_gate_bwd_workspace_bytes(int B, int H, int T, int d_v)
{
    if (B <= 0 || H <= 0 || T <= 0 || d_v <= 0) return 0;
    return sgla::head_norm_gate_bwd_part_floats(B, H, T, d_v) * sizeof(float);
}

sgla_status sgla_head_norm_gate_bwd(const void* o, const void* g, const float* gamma, const void* dout,
                                    void* d_o, void* dg, float* dgamma, int B, int H, int T, int d_v,
                                    int n_tiers, float eps, sgla_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* hip_stream)
{
    REQUIRE_PTR(o);
    REQUIRE_PTR(g);
    REQUIRE_PTR(dout);
    REQUIRE_PTR(d_o);
    REQUIRE_PTR(dg);
    OPTIONAL_PTR(gamma);
    OPTIONAL_PTR(dgamma);
    if (dtype != SGLA_F32 && dtype != SGLA_BF16)
        return fail(SGLA_ERR_INVALID_ARG, "dtype %d is not SGLA_F32 or SGLA_BF16", (int)dtype);
    if (B <= 0 || H <= 0 || T <= 0 || d_v <= 0 || n_tiers <= 0)
        return fail(SGLA_ERR_INVALID_ARG, "sizes must be positive (B=%d H=%d T=%d d_v=%d n_tiers=%d)", B, H, T,
                    d_v, n_tiers);
    if (H % n_tiers != 0)
        return fail(SGLA_ERR_INVALID_ARG, "n_tiers (%d) must divide H (%d)", n_tiers, H);
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return fail(SGLA_ERR_INVALID_ARG, "eps must be finite and >= 0 (got %g)", (double)eps);
    if ((double)B * H * T * d_v > 2.0e9) return fail(SGLA_ERR_INVALID_ARG, "B*H*T*d_v too large");
    if (d_v % 4 != 0 || d_v > 256)
        return fail(SGLA_ERR_UNSUPPORTED, "d_v must be a multiple of 4, at most 256 (got %d)", d_v);
    if (dgamma != nullptr) {
        const size_t need = sgla_head_norm_gate_bwd_workspace_bytes(B, H, T, d_v);
        if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace))
            return fail(SGLA_ERR_WORKSPACE, "workspace needs %zu bytes, 16-byte aligned (got %zu at %p)", need,
                        workspace_bytes, workspace);
    }
    const size_t nb = (size_t)B * H * T * d_v * (dtype == SGLA_BF16 ? 2 : 4);
    const void* ins[3] = {o, g, dout};
    for (int i = 0; i < 3; ++i) {
        if (overlaps(d_o, nb, ins[i], nb)) return fail(SGLA_ERR_INVALID_ARG, "d_o must not overlap o, g or dout");
        if (i < 2 && overlaps(dg, nb, ins[i], nb)) return fail(SGLA_ERR_INVALID_ARG, "dg must not overlap o or g");
    }
    if (dg != dout && overlaps(dg, nb, dout, nb))
        return fail(SGLA_ERR_INVALID_ARG, "dg must equal dout or not overlap it");
    if (overlaps(d_o, nb, dg, nb)) return fail(SGLA_ERR_INVALID_ARG, "d_o must not overlap dg");
    if (dgamma != nullptr) {
        // (dg may be dout itself, so the two bf16 outputs are checked above)
        const size_t ng = (size_t)n_tiers * d_v * sizeof(float);
        const Span rd[6] = {{o, nb, "o"}, {g, nb, "g"}, {dout, nb, "dout"}, {gamma, ng, "gamma"},
                            {d_o, nb, "d_o"}, {dg, nb, "dg"}};
        const Span wr[2] = {{dgamma, ng, "dgamma"},
                            {workspace, sgla_head_norm_gate_bwd_workspace_bytes(B, H, T, d_v), "workspace"}};
        const sgla_status st = check_disjoint(wr, 2, rd, 6);
        if (st != SGLA_OK) return st;
    }
    hipError_t e = sgla::launch_head_norm_gate_bwd(dtype == SGLA_BF16, o, g, gamma, dout, d_o, dg, dgamma,
                                                   reinterpret_cast<float*>(workspace), B, H, T, d_v, n_tiers,
                                                   eps, reinterpret_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(SGLA_ERR_HIP, "head_norm_gate_bwd launch: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
