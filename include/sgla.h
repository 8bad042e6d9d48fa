/*
 * libsgla: Simple Gated Linear Attention (Simple GLA) on AMD Instinct MI355X
 * (gfx950). C ABI.
 *
 * The method is the token mixer of the Laplace 3B model, as described in the
 * page "Beyond the KV cache: Training and serving i14's Laplace 3B linear
 * attention model on AWS Trainium2 with native PyTorch" (the Laplace 3B post),
 * section "i14 and the Laplace 3B architecture", paragraph "GLA mixer". Per
 * sequence and head h, with a d_k x d_v state S and a fixed decay lam_h:
 *
 *   S_t = lam_h S_{t-1} + k_t v_t^T                    (state update)
 *   o_t = S_t^T q_t + sigmoid(sum_i a_{h,i} q_{t,i} k_{t,i}) v_t
 *                                  (readout of the updated state, plus the
 *                                   self-augmentation term)
 *
 * The page's display equations are missing from its text; the readings taken
 * (readout after the update, a per (head, key channel), no scaling of q inside
 * the library, zero initial state by default) are listed with the reasons for
 * each in the design notes.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: every tensor argument is DEVICE memory owned by the caller, except
 *   where a comment says "host". The library allocates nothing and keeps no
 *   state between calls, apart from the thread-local error message.
 * Streams: GPU work is enqueued on `hip_stream` (a hipStream_t; NULL = the
 *   default stream) and the call returns without synchronizing. Outputs are
 *   valid once the stream reaches them.
 * dtype: q, k, v, o (and dO, dq, dk, dv) are all SGLA_BF16 or all SGLA_F32.
 *   States, lambda, a and da are always fp32. Arithmetic is fp32 (bf16
 *   operands into fp32-accumulating matrix cores for SGLA_BF16), with these
 *   roundings in the SGLA_BF16 chunk kernels: the state enters the readout as a
 *   bf16 hi + lo pair (about 16 significant bits); the decayed values of the
 *   state update enter as the exact bf16 value plus a bf16-rounded correction;
 *   and the intra-chunk scores below the diagonal enter the second product
 *   rounded to bf16 (sgla_chunk_fwd_norm_gate: all of them as a bf16 hi + lo
 *   pair), while the diagonal term (q_t . k_t + sigmoid(z_t)) v_t is applied
 *   in fp32. The gate argument z_t = sum_i a_i q_{t,i} k_{t,i} is formed in
 *   fp32 from a in fp32 and the exact products of the bf16 inputs, in every
 *   kernel.
 * Layouts (row-major, last index fastest):
 *   dense:  q, k [B, H, T, d_k];  v, o [B, H, T, d_v];  N = B sequences.
 *   packed: with cu_seqlens != NULL: B must be 1, T is the total token count,
 *           q, k [1, H, T, d_k], v, o [1, H, T, d_v], and sequence n holds
 *           tokens [cu_seqlens[n], cu_seqlens[n+1]) (int32, n_seq+1 entries,
 *           non-decreasing, cu_seqlens[0] = 0, cu_seqlens[n_seq] <= T).
 *   states: [N, H, d_k, d_v] fp32.   lambda: [H] fp32.   a, da: [H, d_k] fp32.
 * Alignment: every tensor pointer must be 16-byte aligned.
 * Errors: argument errors are detected on the host before anything is
 *   enqueued; the call returns a non-zero status and sgla_last_error() gives a
 *   message. A launch failure returns SGLA_ERR_HIP. Device memory contents are
 *   not inspected: NaN inputs propagate; lambda outside [0, 1] gives whatever
 *   the recurrence gives; cu_seqlens entries are clamped into [0, T] on the
 *   device (a decreasing entry yields an empty sequence) so that no access
 *   leaves the buffers.
 * Determinism: the same inputs on the same device give bitwise-identical
 *   outputs, including da (fixed-order reductions, no float atomics).
 * Supported shapes:
 *   SGLA_BF16: d_k <= 96, d_v <= 192, both multiples of 8; chunk 32, 64 or 128.
 *   SGLA_F32:  d_k <= 96, d_v <= 192, both multiples of 4; chunk 32, 64 or 128.
 *   Anything else returns SGLA_ERR_UNSUPPORTED.
 */
#ifndef SGLA_H
#define SGLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SGLA_OK = 0,
    SGLA_ERR_INVALID_ARG = 1,
    SGLA_ERR_UNSUPPORTED = 2,
    SGLA_ERR_WORKSPACE = 3,
    SGLA_ERR_HIP = 4
} sgla_status;

typedef enum { SGLA_F32 = 0, SGLA_BF16 = 1 } sgla_dtype;

/* Library version as major*10000 + minor*100 + patch. */
int sgla_version(void);

/* Static text for a status code. Never NULL. */
const char* sgla_status_str(int status);

/* Message of the last failed call on this thread ("" if none). Never NULL. */
const char* sgla_last_error(void);

/*
 * Decay schedule. Laplace 3B post, "i14 and the Laplace 3B architecture",
 * paragraphs "Decay schedule" and "Decay schedule's reach": fixed per-head
 * decays with half-lives spread geometrically from t_min (head 0) to t_max
 * (head H-1); a half-life of T tokens means lam^T = 1/2. So
 *   T_h = t_min * (t_max / t_min)^(h / (H-1))   (T_0 = t_min when H == 1)
 *   lambda_out[h] = 2^(-1 / T_h)
 * computed in fp64 and rounded to fp32. With H = 16, t_min = 1, t_max = 2048
 * this gives lambda_0 = 0.5 and lambda_15 = 0.99966 (the page: ~0.9997).
 *
 * lambda_out: HOST array of H floats, written. Runs on the host, no GPU work.
 * Errors: SGLA_ERR_INVALID_ARG if lambda_out is NULL, H <= 0, t_min <= 0 or
 * t_max < t_min (or either is not finite).
 */
sgla_status sgla_decay_schedule(int H, double t_min, double t_max, float* lambda_out);

/*
 * Chunked forward. Laplace 3B post, "Challenge 1: Using native PyTorch on
 * Trainium for GLA": the sequence is cut into chunks of `chunk` tokens; inside
 * a chunk the output is decay-masked linear attention plus the contribution of
 * the running state carried in from earlier chunks, and the state then
 * advances by the chunk's decay compounded over the chunk plus the chunk's
 * decayed key/value outer products. This is an exact rewrite of the token
 * recurrence above, so the result does not depend on `chunk` beyond rounding.
 *
 * q, k, v:     inputs (dtype, layouts above); q is used as given (no scale).
 * lambda:      [H] per-head decay.
 * a:           [H, d_k] self-augmentation scale (aug_balance), or NULL = 0.
 * init_state:  [N, H, d_k, d_v] state before the first token, or NULL = 0.
 * final_state: [N, H, d_k, d_v] state after the last token, or NULL (not
 *              written). May equal init_state (in-place carry); any other
 *              overlap with init_state, q, k, v or o is rejected
 *              (SGLA_ERR_INVALID_ARG).
 * o:           output [.., d_v] (dtype). Must not alias any input.
 * cu_seqlens:  packed-sequence offsets (see layouts) or NULL (dense).
 * n_seq:       number of sequences when cu_seqlens != NULL; ignored otherwise.
 * chunk:       chunk length C of the chunk form (32, 64 or 128). It sets the
 *              length of the tiles the kernels scan with, which changes only
 *              the rounding: SGLA_F32 tiles by C tokens, except that the
 *              forward with d_k > 32 and the backward with d_k or d_v > 32
 *              tile by 32; SGLA_BF16 tiles the
 *              forward (and the dv scan of sgla_chunk_bwd) by 32 tokens for
 *              C = 32 and by 64 for C = 64 or 128, because a 128-token tile of
 *              q, k and v does not fit the four-deep LDS ring the bf16
 *              kernels stream through (the dq and dk scans of the backward
 *              always tile by 32, and the state-only passes of the segmented
 *              calls by 64).
 */
sgla_status sgla_chunk_fwd(const void* q, const void* k, const void* v,
                           const float* lambda, const float* a,
                           const float* init_state, float* final_state, void* o,
                           const int32_t* cu_seqlens, int n_seq,
                           int B, int H, int T, int d_k, int d_v, int chunk,
                           sgla_dtype dtype, void* hip_stream);

/*
 * Size in bytes of the exchange buffer sgla_chunk_fwd_norm_gate takes.
 */
#define SGLA_FWD_NORM_GATE_EXCHANGE_BYTES ((size_t)2 * 1024 * 1024 + 256)

/*
 * Chunked forward with the mixer epilogue applied to each output tile before
 * it is stored: sgla_chunk_fwd followed by sgla_head_norm_gate in one kernel,
 * so that o need not go to memory and back. Laplace 3B post, "Challenge 1:
 * Using native PyTorch on Trainium for GLA" (the chunk form), and "i14 and
 * the Laplace 3B architecture", the end of the "GLA mixer" paragraph and
 * "Decay schedule's reach" (Head RMSNorm per decay tier, heads concatenated,
 * SiLU(g) gate):
 *   out[b,t,h,c] = silu(g[b,t,h,c]) * gamma[tier(h)][c] * o[b,h,t,c]
 *                  / sqrt(mean_c' o[b,h,t,c']^2 + eps),   tier(h) = h / (H / n_tiers)
 * with o the chunked forward's output, taken here in fp32 (sgla_chunk_fwd
 * rounds it to bf16 before the epilogue would read it).
 *
 * q, k, v, lambda, a, init_state, final_state, cu_seqlens, n_seq, B, H, T,
 * d_k, d_v, chunk: as sgla_chunk_fwd (bf16 only).
 * g:        [B, T, H, d_v] bf16 gate stream, token-major (packed: B = 1,
 *           T = total tokens).
 * gamma:    [n_tiers, d_v] fp32 scales, or NULL (one).
 * out:      [B, T, H, d_v] bf16, token-major. It may equal g (in place);
 *           otherwise it must not overlap g. It must not overlap any other
 *           argument.
 * o:        [B, H, T, d_v] bf16 (the layout of sgla_chunk_fwd), also written
 *           when not NULL (e.g. for sgla_head_norm_gate_bwd).
 * n_tiers:  divides H. eps: finite, >= 0.
 * exchange: device buffer of SGLA_FWD_NORM_GATE_EXCHANGE_BYTES that must be
 *           zero-filled before its first use. The two 96-column workgroups of
 *           a (sequence, head) with d_v > 96 pass each other their per-token
 *           sums of o^2 through it, and every workgroup takes a ticket from
 *           counters in it when it starts; consecutive tickets make up a
 *           (sequence, head), so the two partners have always both started,
 *           and ordinary launches suffice with no assumption about residency.
 *           A call that completes leaves the buffer zero-filled again. Calls
 *           that may run at the same time need distinct buffers. One launch
 *           has exchange slots for 1,024 workgroups (512 (sequence, head)
 *           units with d_v > 96, 1,024 otherwise); more units take further
 *           launches in turn on the stream. Should an exchange never arrive (other work holding the
 *           device longer than a bounded number of polls), or the buffer not
 *           have been zero-filled, the affected outputs are NaN or not
 *           written and the buffer's first int is set to 1 (zero-fill it
 *           again before the next call).
 * flags:    0 (no flags are defined).
 * Errors: as sgla_chunk_fwd; SGLA_ERR_UNSUPPORTED for SGLA_F32 (compose
 * sgla_chunk_fwd and sgla_head_norm_gate) or H * d_v above 2^24;
 * SGLA_ERR_INVALID_ARG for n_tiers
 * not dividing H, a bad eps, nonzero flags, or overlapping buffers; SGLA_ERR_WORKSPACE for a
 * NULL, misaligned or short exchange buffer; SGLA_ERR_HIP for a launch
 * failure.
 */
sgla_status sgla_chunk_fwd_norm_gate(const void* q, const void* k, const void* v,
                                     const float* lambda, const float* a,
                                     const float* init_state, float* final_state,
                                     const void* g, const float* gamma, void* out, void* o,
                                     const int32_t* cu_seqlens, int n_seq,
                                     int B, int H, int T, int d_k, int d_v, int chunk,
                                     int n_tiers, float eps, sgla_dtype dtype,
                                     void* exchange, size_t exchange_bytes, unsigned flags,
                                     void* hip_stream);

/*
 * Bytes of device workspace sgla_chunk_fwd_segmented needs: two arrays of
 * B * n_segments * H states of d_k * d_v fp32.
 */
size_t sgla_chunk_fwd_segmented_workspace_bytes(int B, int H, int d_k, int d_v, int n_segments);

/*
 * Segment-parallel chunked forward of long dense sequences, for when B * H
 * (sequence, head) pairs are too few to occupy the GPU. Same result as
 * sgla_chunk_fwd up to rounding. Laplace 3B post, "Challenge 1: Using native
 * PyTorch on Trainium for GLA": only the state update is sequential, and the
 * state after a run of L tokens is lam^L times the state before it plus the
 * run's own decayed key/value sum (the chunk state-advance equation applied
 * over the run). Each sequence is cut into segments of whole 64-token tiles,
 * ceil(T / n_segments) tokens rounded up (fewer segments when T is short):
 *   1. the state scan alone (k and v only, no outputs) over segments
 *      0 .. G-2, segment 0 from init_state and the others from zero, keeping
 *      the state each one leaves;
 *   2. a scan of those states: entering segment g, lam^L (entering g-1) plus
 *      (leaving g-1 from zero), the first being the state leaving segment 0;
 *   3. the forward over every segment from its true entering state, which
 *      writes o and final_state.
 * Three kernel launches on hip_stream: one forward's work over G times as
 * many workgroups, plus the cheaper state scan of G - 1 segments.
 *
 * q, k, v, lambda, a, init_state, final_state, o, B, H, T, d_k, d_v, chunk:
 *              as for sgla_chunk_fwd, dense layout only (no cu_seqlens);
 *              final_state may equal init_state.
 * dtype:       SGLA_BF16 only (SGLA_ERR_UNSUPPORTED otherwise).
 * n_segments:  segments per sequence requested, >= 1; 1 is sgla_chunk_fwd.
 *              The full forward launch runs G * B * H * ceil(d_v / 96)
 *              workgroups of one per CU, so G = CUs / (B * H * ceil(d_v / 96))
 *              fills the GPU once (on 256 CUs at H = 16, d_v = 192: G = 8 for
 *              B = 1, 4 for B = 2); at B * H * ceil(d_v / 96) >= CUs / 2 the
 *              single pass is as fast or faster.
 * workspace:   device buffer of at least
 *              sgla_chunk_fwd_segmented_workspace_bytes(B, H, d_k, d_v,
 *              n_segments) bytes, 16-byte aligned, owned by the caller, not
 *              overlapping any other argument (SGLA_ERR_WORKSPACE if it
 *              overlaps q, k, v, o or a state); contents on entry do not
 *              matter and are clobbered.
 * Errors: as sgla_chunk_fwd, plus SGLA_ERR_INVALID_ARG for n_segments < 1
 * and SGLA_ERR_WORKSPACE if workspace is NULL, unaligned or too small.
 */
sgla_status sgla_chunk_fwd_segmented(const void* q, const void* k, const void* v,
                                     const float* lambda, const float* a,
                                     const float* init_state, float* final_state, void* o,
                                     int B, int H, int T, int d_k, int d_v, int chunk,
                                     sgla_dtype dtype, int n_segments, void* workspace,
                                     size_t workspace_bytes, void* hip_stream);

/*
 * Bytes of device workspace sgla_chunk_bwd_segmented needs: four arrays of
 * B * n_segments * H states of d_k * d_v fp32 and B * n_segments * H * d_k
 * fp32 partial sums of da.
 */
size_t sgla_chunk_bwd_segmented_workspace_bytes(int B, int H, int d_k, int d_v, int n_segments);

/*
 * Segment-parallel chunked backward of long dense sequences: the gradients of
 * sgla_chunk_fwd (same result as sgla_chunk_bwd up to rounding, da summed in
 * a fixed order). Segments as for sgla_chunk_fwd_segmented. The dq scan needs
 * the forward state entering each segment, and the dk and dv scans (which run
 * from the back) need the state gradient G entering each segment from its
 * end. Both follow from the affine maps of the runs, as in the forward
 * ("Challenge 3: Backward-pass unrolling for a sequential recurrence": the
 * state gradient flows back through every state update). Four steps on
 * hip_stream:
 *   1. the forward state scan alone over segments 0 .. G-2 and the scan of
 *      their leaving states;
 *   2. the gradient state scan alone over segments 1 .. G-1 from their ends
 *      (the last from d_final_state, the others from zero), keeping the G
 *      each leaves at its front (steps 1 and 2 share one launch; neither
 *      writes outputs);
 *   3. the reverse scan of those: G entering segment g from its end is
 *      lam^L (G entering g+1) + (G leaving g+1 from zero);
 *   4. the full backward over every segment from its true states, which
 *      writes dq, dk, dv, the da partial sums and d_init_state, then the
 *      fixed-order sum of da.
 *
 * Arguments as for sgla_chunk_bwd, dense layout only (no cu_seqlens), plus:
 * dtype:       SGLA_BF16 only (SGLA_ERR_UNSUPPORTED otherwise).
 * n_segments:  segments per sequence requested, >= 1; 1 is sgla_chunk_bwd.
 *              Step 4 runs 4 * G * B * H workgroups at d_k <= 96, d_v <= 192
 *              (dq, dk and two dv slices), so G = CUs / (4 B H) fills the GPU
 *              once (on 256 CUs at H = 16: G = 4 for B = 1, 2 for B = 2).
 * workspace:   device buffer of at least
 *              sgla_chunk_bwd_segmented_workspace_bytes(B, H, d_k, d_v,
 *              n_segments) bytes, 16-byte aligned, owned by the caller, not
 *              overlapping any other argument; clobbered.
 * Errors: as sgla_chunk_bwd, plus SGLA_ERR_INVALID_ARG for n_segments < 1.
 */
sgla_status sgla_chunk_bwd_segmented(const void* q, const void* k, const void* v, const void* dO,
                                     const float* lambda, const float* a,
                                     const float* init_state, const float* d_final_state,
                                     void* dq, void* dk, void* dv, float* da, float* d_init_state,
                                     int B, int H, int T, int d_k, int d_v, int chunk,
                                     sgla_dtype dtype, int n_segments, void* workspace,
                                     size_t workspace_bytes, void* hip_stream);

/*
 * Bytes of device workspace sgla_chunk_bwd needs for these sizes (the per
 * sequence-head partial sums of da). N is n_seq for packed input, else B.
 */
size_t sgla_chunk_bwd_workspace_bytes(int N, int H, int d_k);

/*
 * Chunked backward: gradients of the forward above for a loss L with
 * dL/do = dO and dL/d(final_state) = d_final_state. Laplace 3B post,
 * "Challenge 3: Backward-pass unrolling for a sequential recurrence": the
 * backward differentiates through every sequential state update. Written as
 *   dq_t = S_t dO_t + sigmoid'(z_t) (dO_t . v_t) (a * k_t)
 *   G_t  = dL/dS_t = lam G_{t+1} + q_t dO_t^T      (G_{T-1} = dS_final + q dO^T)
 *   dk_t = G_t v_t + sigmoid'(z_t) (dO_t . v_t) (a * q_t)
 *   dv_t = G_t^T k_t + sigmoid(z_t) dO_t
 *   da   = sum over sequences and t of sigmoid'(z_t) (dO_t . v_t) (q_t * k_t)
 *   d_init_state = lam G_0   (= d_final_state for an empty sequence)
 * and evaluated chunk-wise, as three independent recurrences run at once
 * (a forward scan for dq and two reverse scans for dk and dv).
 *
 * q, k, v, lambda, a, init_state, cu_seqlens, n_seq, sizes, chunk, dtype:
 *              as for sgla_chunk_fwd (same values as the forward call).
 * dO:          [.., d_v] upstream gradient of o (dtype).
 * d_final_state: [N, H, d_k, d_v] or NULL = 0.
 * dq, dk, dv:  outputs (dtype), shaped like q, k, v; must not alias inputs.
 * da:          [H, d_k] fp32, overwritten with dL/da (at a = 0 when a is NULL;
 *              not zero then, since sigmoid'(0) = 1/4).
 * d_init_state: [N, H, d_k, d_v] or NULL (not written); must not overlap
 *              d_final_state or init_state (they are read while it is written).
 * workspace:   device buffer of at least sgla_chunk_bwd_workspace_bytes()
 *              bytes, 16-byte aligned, owned by the caller; its contents on
 *              entry do not matter and are clobbered.
 * Every buffer written (dq, dk, dv, da, d_init_state, workspace) must be
 * disjoint from every buffer read and from every other one written.
 * Errors: as sgla_chunk_fwd, plus SGLA_ERR_WORKSPACE if workspace is NULL,
 * too small or overlapping another argument, and SGLA_ERR_INVALID_ARG for any
 * other overlap above.
 */
sgla_status sgla_chunk_bwd(const void* q, const void* k, const void* v, const void* dO,
                           const float* lambda, const float* a,
                           const float* init_state, const float* d_final_state,
                           void* dq, void* dk, void* dv, float* da, float* d_init_state,
                           const int32_t* cu_seqlens, int n_seq,
                           int B, int H, int T, int d_k, int d_v, int chunk,
                           sgla_dtype dtype, void* workspace, size_t workspace_bytes,
                           void* hip_stream);

/*
 * Bytes of the fixed device scratch array behind sgla_chunk_bwd_noalloc.
 */
#define SGLA_NOALLOC_SCRATCH_BYTES (4 * 1024 * 1024)

/*
 * sgla_chunk_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. It computes exactly what sgla_chunk_bwd
 * computes, with the same kernels, and calls no allocating routine. The
 * scratch those kernels need (the partial sums of da, sgla_chunk_bwd_workspace_bytes
 * bytes) comes from a fixed array of SGLA_NOALLOC_SCRATCH_BYTES in device
 * memory that the library holds on every GPU it runs on until the process
 * ends; its device address is looked up on the first call made on each
 * device. Every call on a GPU reuses that GPU's array, and every call
 * overwrites all of the scratch it reads, so no state carries between calls;
 * calls that overlap in time on one GPU (on different streams, or from
 * different threads) race on the array and must not be issued.
 *
 * Arguments, layouts and errors: as sgla_chunk_bwd, without workspace and
 * workspace_bytes; argument errors are reported before any GPU call, and
 * SGLA_ERR_WORKSPACE when the da partial sums (N * H * d_k floats, N = n_seq
 * or B) exceed SGLA_NOALLOC_SCRATCH_BYTES (for H = 16, d_k = 96: N <= 682).
 */
sgla_status sgla_chunk_bwd_noalloc(const void* q, const void* k, const void* v, const void* dO,
                                   const float* lambda, const float* a,
                                   const float* init_state, const float* d_final_state,
                                   void* dq, void* dk, void* dv, float* da, float* d_init_state,
                                   const int32_t* cu_seqlens, int n_seq,
                                   int B, int H, int T, int d_k, int d_v, int chunk,
                                   sgla_dtype dtype, void* hip_stream);

/*
 * One decode step for N sequences, in place on their states. Laplace 3B post,
 * "Inference optimization on Trainium2", paragraphs "Constant serving state"
 * and "Unmodified vLLM": each sequence keeps a fixed-size recurrent state in
 * a page of a state pool, and each new token reads and writes that page:
 *   S <- lam_h S + k v^T;   o = S^T q + sigmoid(sum_i a_{h,i} q_i k_i) v
 *
 * q, k:    [N, H, d_k] (dtype).   v, o: [N, H, d_v] (dtype).
 * state:   [P, H, d_k, d_v] fp32 pool, read and written in place.
 * slot:    [N] int32 page index of each sequence, or NULL (sequence n uses
 *          page n, and then P >= N is required). Entries must be distinct;
 *          an entry outside [0, P) skips that sequence and writes NaN to its o.
 * Supported: d_k from 4 to 96 and d_v from 4 to 192, multiples of 4, either
 * dtype (every head shape the chunk entry points take).
 * The output of one sequence does not depend on N or on the other sequences.
 * state and o must be disjoint from each other and from q, k, v, lambda, a
 * and slot (SGLA_ERR_INVALID_ARG otherwise).
 */
sgla_status sgla_decode_step(const void* q, const void* k, const void* v,
                             const float* lambda, const float* a,
                             float* state, const int32_t* slot, void* o,
                             int N, int P, int H, int d_k, int d_v,
                             sgla_dtype dtype, void* hip_stream);

/*
 * Convolution prologue of the mixer (the step before the QKVG projection),
 * over whole sequences. Laplace 3B post, "i14 and the Laplace 3B
 * architecture", normalisation-and-convolution paragraph and the architecture
 * table's Conv row: every channel of every token goes through a depthwise
 * causal Conv1d of width 4 with a SiLU, a 4-gram summary of the token and its
 * three predecessors:
 *   y_t[c] = silu(b[c] + sum_{j=0..3} w[c][j] u_{t-3+j}[c]),   silu(x) = x sigmoid(x)
 * Taps are oldest first (a PyTorch depthwise Conv1d weight [D, 1, 4] with
 * three zeros of left padding). Before the first token of a sequence the three
 * previous inputs are that sequence's conv state, or zero.
 *
 * u, y:        [B, T, D] (dtype); packed (cu_seqlens != NULL): [T, D] with
 *              B = 1, sequence n holding rows [cu_seqlens[n], cu_seqlens[n+1]).
 *              y must not alias u.
 * w:           [D, 4] fp32 taps.   b: [D] fp32 bias, or NULL = none.
 * init_state:  [N, 3, D] fp32, row j = u_{-3+j} of sequence n, or NULL = zero.
 * final_state: [N, 3, D] fp32 or NULL: row j = u_{L-3+j} of sequence n (reaching
 *              into init_state when L < 3). It may equal init_state (in-place
 *              carry); otherwise it must not overlap init_state, u or y.
 *              y must not overlap init_state either.
 * n_seq:       N (= B when dense).
 * Supported: D a multiple of 8 (bf16) or 4 (fp32). All pointers 16-byte aligned.
 * Errors: SGLA_ERR_INVALID_ARG (NULL required pointer, non-positive size,
 * misaligned pointer, overlapping buffers), SGLA_ERR_UNSUPPORTED (D),
 * SGLA_ERR_HIP (launch).
 */
sgla_status sgla_conv_fwd(const void* u, const float* w, const float* b,
                          const float* init_state, float* final_state, void* y,
                          const int32_t* cu_seqlens, int n_seq, int B, int T, int D,
                          sgla_dtype dtype, void* hip_stream);

/*
 * Bytes of device workspace sgla_conv_bwd needs: five fp32 rows of D per 64
 * token rows (the per-run partial sums of the tap and bias gradients). T is
 * the total token count when packed (B = 1).
 */
size_t sgla_conv_bwd_workspace_bytes(int B, int T, int D);

/*
 * Gradients of sgla_conv_fwd for a loss L with dL/dy = dy and
 * dL/d(final_state) = d_final_state (same passages). Per sequence and
 * channel, with x_s = u_s (s >= 0) or row 3 + s of the initial state and
 * pre_t = b + sum_j w_j x_{t-3+j}:
 *   dpre_t = dy_t silu'(pre_t),     silu'(x) = sigmoid(x) (1 + x (1 - sigmoid(x)))
 *   dL/dx_s = sum_j w_j dpre_{s+3-j}  (within the sequence)
 *             + d_final_state[s - (L - 3)]  for the last three inputs
 *   du_s = dL/dx_s (s >= 0);  d_init_state[i] = dL/dx_{i-3}
 *   dw[c][j] = sum over sequences and t of dpre_t x_{t-3+j};  db[c] = sum of dpre_t
 * dw and db are summed in a fixed order (per-run partials, then a second
 * kernel), so they are bitwise reproducible.
 *
 * u, w, b, init_state, cu_seqlens, n_seq, B, T, D, dtype: as for the forward.
 * dy:            [B, T, D] (dtype), like y.
 * d_final_state: [N, 3, D] fp32 or NULL = 0.
 * du:            [B, T, D] (dtype); must not overlap u or dy.
 * dw:            [D, 4] fp32, overwritten.   db: [D] fp32 or NULL (not computed).
 * d_init_state:  [N, 3, D] fp32 or NULL (not written); must not overlap du,
 *                init_state or d_final_state.
 * workspace:     device buffer of at least sgla_conv_bwd_workspace_bytes(B,
 *                T, D) bytes, 16-byte aligned, owned by the caller, clobbered.
 * du, dw, db, d_init_state and workspace must be disjoint from every input
 * and from each other.
 * Errors: as sgla_conv_fwd, plus SGLA_ERR_WORKSPACE (workspace NULL,
 * misaligned, too small or overlapping another argument) and
 * SGLA_ERR_INVALID_ARG for any other overlap above.
 */
sgla_status sgla_conv_bwd(const void* u, const float* w, const float* b, const float* init_state,
                          const void* dy, const float* d_final_state, void* du, float* dw, float* db,
                          float* d_init_state, const int32_t* cu_seqlens, int n_seq, int B, int T,
                          int D, sgla_dtype dtype, void* workspace, size_t workspace_bytes,
                          void* hip_stream);

/*
 * One conv decode step for N sequences, in place on their conv states (the
 * per-sequence serving state of "Inference optimization on Trainium2",
 * "Constant serving state", next to the mixer state):
 *   y[c] = silu(b[c] + w[c][0] s0[c] + w[c][1] s1[c] + w[c][2] s2[c] + w[c][3] x[c]);
 *   (s0, s1, s2) <- (s1, s2, x)
 * x, y:   [N, D] (dtype).   w, b: as sgla_conv_fwd.
 * state:  [P, 3, D] fp32 pool, read and written in place.
 * slot:   [N] int32 page index, or NULL (sequence n uses page n, P >= N).
 *         Entries must be distinct; one outside [0, P) skips that sequence
 *         and writes NaN to its y.
 * y must not overlap x; the pool must overlap neither.
 * Supported and errors: as sgla_conv_fwd.
 */
sgla_status sgla_conv_decode_step(const void* x, const float* w, const float* b,
                                  float* state, const int32_t* slot, void* y,
                                  int N, int P, int D, sgla_dtype dtype, void* hip_stream);

/*
 * Mixer epilogue: Head RMSNorm per decay tier, concatenation of the heads and
 * the SiLU(g) output gate. Laplace 3B post, "i14 and the Laplace 3B
 * architecture", the end of the "GLA mixer" paragraph (the per-head outputs
 * go through a Head RMSNorm within each decay tier, are concatenated and
 * gated by SiLU(g_t)) and "Decay schedule's reach" (the heads of a tier share
 * one Head RMSNorm, i.e. its learned per-channel scale):
 *   out[b,t,h,c] = silu(g[b,t,h,c]) * gamma[tier(h)][c] * o[b,h,t,c]
 *                  / sqrt(mean_c' o[b,h,t,c']^2 + eps),   tier(h) = h / (H / n_tiers)
 * The statistic is per head (over its d_v channels); tiers are contiguous
 * groups of H / n_tiers heads, which the monotone decay schedule makes heads
 * of similar reach.
 *
 * o:       [B, H, T, d_v] (dtype), the layout sgla_chunk_fwd writes (packed
 *          sequences: B = 1, T = total tokens); a decode step's o [N, H, d_v]
 *          is B = N, T = 1.
 * g:       [B, T, H, d_v] (dtype), the gate stream, token-major.
 * gamma:   [n_tiers, d_v] fp32, or NULL (one).
 * out:     [B, T, H, d_v] (dtype), token-major (heads concatenated). It may
 *          equal g (in place); otherwise it must not overlap g. It must not
 *          overlap o.
 * n_tiers: divides H. eps: finite, >= 0 (with eps = 0 an all-zero head gives NaN).
 * Supported: d_v a multiple of 4, at most 256. All pointers 16-byte aligned.
 * Errors: SGLA_ERR_INVALID_ARG (NULL required pointer, non-positive size,
 * n_tiers not dividing H, bad eps, misaligned or overlapping buffers),
 * SGLA_ERR_UNSUPPORTED (d_v), SGLA_ERR_HIP (launch).
 */
sgla_status sgla_head_norm_gate(const void* o, const void* g, const float* gamma, void* out,
                                int B, int H, int T, int d_v, int n_tiers, float eps,
                                sgla_dtype dtype, void* hip_stream);

/*
 * Bytes of device workspace sgla_head_norm_gate_bwd needs when dgamma is
 * wanted: one fp32 row of d_v per 64 tokens of each (b, h).
 */
size_t sgla_head_norm_gate_bwd_workspace_bytes(int B, int H, int T, int d_v);

/*
 * Gradients of sgla_head_norm_gate for a loss L with dL/dout = dout (same
 * passages). With r = sqrt(mean_c o^2 + eps), y = o / r, s = silu(g),
 * gm = gamma[tier(h)][c] (one when gamma is NULL) and w = dout s gm, per
 * (b, h, t) row:
 *   dg     = dout gm y silu'(g),     silu'(x) = sigmoid(x) (1 + x (1 - sigmoid(x)))
 *   d_o    = (w - y mean_c (w y)) / r
 *   dgamma[tier][c] = sum over b, t and the tier's heads of dout s y
 * dgamma is the gradient at gamma = 1 when gamma is NULL; it is summed in a
 * fixed order (per-block partials, then a second kernel), so it is bitwise
 * reproducible.
 *
 * o, g, gamma, B, H, T, d_v, n_tiers, eps, dtype: as for the forward call.
 * dout:    [B, T, H, d_v] (dtype), token-major like out.
 * d_o:     [B, H, T, d_v] (dtype), head-major like o (the upstream gradient
 *          the chunked backward takes); must not overlap any other buffer.
 * dg:      [B, T, H, d_v] (dtype); may equal dout (in place), otherwise must
 *          not overlap it; must not overlap o or g.
 * dgamma:  [n_tiers, d_v] fp32, overwritten, or NULL (not computed).
 * workspace: device buffer of at least
 *          sgla_head_norm_gate_bwd_workspace_bytes(B, H, T, d_v) bytes,
 *          16-byte aligned, owned by the caller, clobbered; needed only when
 *          dgamma is not NULL (may be NULL otherwise).
 * dgamma and workspace must be disjoint from o, g, gamma, dout, d_o, dg and
 * each other.
 * Errors: as sgla_head_norm_gate, plus SGLA_ERR_WORKSPACE (dgamma wanted
 * and workspace NULL, misaligned, too small or overlapping another argument)
 * and SGLA_ERR_INVALID_ARG for any other overlap above.
 */
sgla_status sgla_head_norm_gate_bwd(const void* o, const void* g, const float* gamma, const void* dout,
                                    void* d_o, void* dg, float* dgamma, int B, int H, int T, int d_v,
                                    int n_tiers, float eps, sgla_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* SGLA_H */
