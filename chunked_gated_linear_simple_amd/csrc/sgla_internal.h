// Internal interface between the C-ABI host layer (sgla_api.cpp) and the HIP
// launchers (sgla_chunk.hip, sgla_decode.hip). Not installed, not part of the ABI.
#ifndef SGLA_INTERNAL_H
#define SGLA_INTERNAL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgla.h"

namespace sgla {

// Records msg as the calling thread's sgla_last_error() and returns st.
sgla_status api_fail(sgla_status st, const char* msg);

struct ChunkProblem;

// Every argument check of sgla_chunk_bwd except those of its workspace; fills
// the launch description. Enqueues nothing.
sgla_status check_chunk_bwd(const void* q, const void* k, const void* v, const void* dO, const float* lambda,
                            const float* a, const float* init_state, const float* d_final_state, void* dq,
                            void* dk, void* dv, float* da, float* d_init_state, const int32_t* cu_seqlens,
                            int n_seq, int B, int H, int T, int d_k, int d_v, int chunk, sgla_dtype dtype,
                            ChunkProblem* p);

// Everything a chunked launch needs, already validated on the host.
struct ChunkProblem {
    int bf16;          // 1: bf16 tensors, 0: fp32 tensors
    int B, H, T;       // T = tokens per sequence (dense) or total tokens (packed)
    int n_seq;         // sequences N (= B when dense)
    int d_k, d_v;
    int chunk;
    const float* lambda;
    const float* a;
    const int32_t* cu;  // NULL when dense
};

// Tile length of the bf16 output scans (forward, dv) for a chunk length.
int bf16_tile(int chunk);

hipError_t launch_chunk_fwd(const ChunkProblem& p, const void* q, const void* k, const void* v,
                            const float* init_state, float* final_state, void* o,
                            hipStream_t stream);

// bf16 forward, d_k <= 96: the FWD role of sgla_fwd.hip.
hipError_t launch_fwd_bf16(const ChunkProblem& p, const void* q, const void* k, const void* v,
                           const float* init_state, float* final_state, void* o,
                           hipStream_t stream);

// bf16 forward with the mixer epilogue applied before the store (sgla_fwd.hip);
// exchange holds SGLA_FWD_NORM_GATE_EXCHANGE_BYTES, zero-filled.
hipError_t launch_fwd_norm_gate_bf16(const ChunkProblem& p, const void* q, const void* k, const void* v,
                                     const float* init_state, float* final_state, const void* g,
                                     const float* gamma, void* out, void* o, int n_tiers, float eps,
                                     void* exchange, hipStream_t stream);

// bf16 forward of dense sequences cut into nseg >= 2 segments of seg_len
// tokens (sgla_fwd.hip); ws_loc and ws_in hold [n_seq][nseg][H][d_k][d_v] fp32.
hipError_t launch_fwd_bf16_segmented(const ChunkProblem& p, const void* q, const void* k,
                                     const void* v, const float* init_state, float* final_state,
                                     void* o, int nseg, int seg_len, float* ws_loc, float* ws_in,
                                     hipStream_t stream);

// The forward states entering segments 1 .. nseg-1 (ws_in), from the state
// scan alone over segments 0 .. nseg-2 (sgla_fwd.hip).
hipError_t launch_fwd_bf16_seg_states(const ChunkProblem& p, const void* k, const void* v,
                                      const float* init_state, int nseg, int seg_len, float* ws_loc,
                                      float* ws_in, hipStream_t stream);

// bf16 backward of dense sequences cut into nseg >= 2 segments (sgla_bwd.hip);
// ws holds 4 n_seq nseg H d_k d_v floats, da_partial n_seq nseg H d_k.
hipError_t launch_bwd_bf16_segmented(const ChunkProblem& p, const void* q, const void* k, const void* v,
                                     const void* dO, const float* init_state, const float* d_final_state,
                                     void* dq, void* dk, void* dv, float* da, float* d_init_state,
                                     float* da_partial, int nseg, int seg_len, float* ws, hipStream_t stream);

// bf16 backward, d_k <= 96, d_v <= 192: the DV/DQ/DK roles of sgla_bwd.hip.
hipError_t launch_bwd_bf16(const ChunkProblem& p, const void* q, const void* k, const void* v,
                           const void* dO, const float* init_state, const float* d_final_state,
                           void* dq, void* dk, void* dv, float* da, float* d_init_state,
                           float* da_partial, hipStream_t stream);

hipError_t launch_chunk_bwd(const ChunkProblem& p, const void* q, const void* k, const void* v,
                            const void* dO, const float* init_state, const float* d_final_state,
                            void* dq, void* dk, void* dv, float* da, float* d_init_state,
                            float* da_partial, hipStream_t stream);

hipError_t launch_decode_step(int bf16, const void* q, const void* k, const void* v,
                              const float* lambda, const float* a, float* state,
                              const int32_t* slot, void* o, int N, int P, int H, int d_k,
                              int d_v, hipStream_t stream);

// Convolution prologue (sgla_conv.hip).
hipError_t launch_conv_fwd(int bf16, const void* u, const float* w, const float* b,
                           const float* init_state, float* final_state, void* y,
                           const int32_t* cu, int n_seq, int B, int T, int D, hipStream_t stream);

hipError_t launch_conv_decode(int bf16, const void* x, const float* w, const float* b, float* state,
                              const int32_t* slot, void* y, int N, int P, int D, hipStream_t stream);

// Mixer epilogue: Head RMSNorm per decay tier + SiLU(g) gate (sgla_norm.hip).
hipError_t launch_head_norm_gate(int bf16, const void* o, const void* g, const float* gamma, void* out, int B,
                                 int H, int T, int d_v, int n_tiers, float eps, hipStream_t stream);

// Gradients of the conv prologue (sgla_conv.hip); part holds
// conv_bwd_part_floats() floats.
size_t conv_bwd_part_floats(int B, int T, int D, int packed);
hipError_t launch_conv_bwd(int bf16, const void* u, const void* dy, const float* w, const float* b,
                           const float* init_state, const float* d_final_state, void* du, float* dw, float* db,
                           float* d_init_state, const int32_t* cu, int n_seq, int B, int T, int D, float* part,
                           hipStream_t stream);

// Gradients of the mixer epilogue (sgla_norm.hip); part holds
// head_norm_gate_bwd_part_floats() floats when dgamma is wanted.
size_t head_norm_gate_bwd_part_floats(int B, int H, int T, int d_v);
hipError_t launch_head_norm_gate_bwd(int bf16, const void* o, const void* g, const float* gamma, const void* dout,
                                     void* d_o, void* dg, float* dgamma, float* part, int B, int H, int T, int d_v,
                                     int n_tiers, float eps, hipStream_t stream);

}  // namespace sgla

#endif
