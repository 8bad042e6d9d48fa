/*
 * Simple GLA oracle: a plain, slow, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this code: only the test suite, the smoke check and the
 * bench's CPU-baseline leg use it. It shares no code with the HIP library.
 *
 * Source: "Beyond the KV cache: Training and serving i14's Laplace 3B linear
 * attention model on AWS Trainium2 with native PyTorch" (AWS ML blog), section
 * "i14 and the Laplace 3B architecture", paragraphs "GLA mixer" (state update,
 * readout and self-augmentation equations), "Decay schedule" and "Decay
 * schedule's reach". The display equations are missing from the page text;
 * the formulas below are the plainest reading of the prose around them (the
 * update is a rank-1 write of the current key/value pair into a state decayed
 * by the fixed per-head rate; the readout queries the updated state; the gate
 * is a sigmoid of the query dotted with a per-channel rescaled key), written
 * out token by token:
 *
 *   S_t = lam * S_{t-1} + k_t v_t^T          (d_k x d_v state, S_{-1} = S0)
 *   z_t = sum_i a_i q_{t,i} k_{t,i}
 *   o_t = S_t^T q_t + sigmoid(z_t) v_t
 *
 * All arrays are row-major, token-major, for ONE (sequence, head) unit:
 *   q, k, dq, dk : [T][d_k]     v, o, dO, dv : [T][d_v]
 *   S0, S_final, dS_final, dS0 : [d_k][d_v]   a, da : [d_k]
 * A NULL S0 / dS_final means zero. A NULL a means a = 0 everywhere (da is
 * then the gradient at a = 0, which is not zero).
 */
#ifndef SGLA_ORACLE_H
#define SGLA_ORACLE_H

#ifdef __cplusplus
extern "C" {
#endif

/* lam[h] = 2^(-1/T_h), T_h = t_min * (t_max/t_min)^(h/(H-1)); T_0 = t_min when H == 1. */
void orc_decay_schedule(int H, double t_min, double t_max, double* lam);

/* Token-by-token forward. S_final may be NULL. */
void orc_fwd(int T, int d_k, int d_v, double lam, const double* a,
             const double* q, const double* k, const double* v,
             const double* S0, double* o, double* S_final);

/* Reverse-mode gradients of L = sum_t dO_t . o_t + sum(dS_final * S_final).
 * da is ACCUMULATED into (caller zeroes it); dS0 may be NULL. */
void orc_bwd(int T, int d_k, int d_v, double lam, const double* a,
             const double* q, const double* k, const double* v,
             const double* S0, const double* dO, const double* dS_final,
             double* dq, double* dk, double* dv, double* da, double* dS0);

/* One decode step on the state in place: S <- lam S + k v^T; o = S^T q + sigmoid(z) v. */
void orc_decode_step(int d_k, int d_v, double lam, const double* a,
                     const double* q, const double* k, const double* v,
                     double* S, double* o);

/* Convolution prologue (depthwise causal, width 4, SiLU) for ONE sequence:
 *   y_t[c] = silu(b[c] + sum_{j=0..3} w[c][j] u_{t-3+j}[c])
 * u, y : [L][D]; w : [D][4] (oldest tap first); b : [D] or NULL (zero);
 * st, st_out : [3][D] = u_{-3}, u_{-2}, u_{-1} before / u_{L-3..L-1} after
 * (NULL st means zero history; st_out may be NULL or equal st). */
void orc_conv_fwd(int L, int D, const double* w, const double* b, const double* u,
                  const double* st, double* y, double* st_out);

/* Gradients of orc_conv_fwd for ONE sequence: du [L][D] and d_st [3][D]
 * (NULL: not written) are overwritten, dw [D][4] and db [D] accumulated
 * (NULL: skipped); d_st_out [3][D] is the final state's gradient or NULL. */
void orc_conv_bwd(int L, int D, const double* w, const double* b, const double* u,
                  const double* st, const double* dy, const double* d_st_out, double* du,
                  double* d_st, double* dw, double* db);

/* One conv decode step, state [3][D] in place. */
void orc_conv_decode_step(int D, const double* w, const double* b, const double* x,
                          double* st, double* y);

/* Mixer epilogue (Head RMSNorm per decay tier, concatenation, SiLU(g) gate)
 * for ONE token:
 *   out[h][c] = silu(g[h][c]) * gamma[tier(h)][c] * o[h][c] / sqrt(mean_c' o[h][c']^2 + eps)
 * o, g, out : [H][d_v] (the token's heads, concatenated); gamma : [n_tiers][d_v]
 * or NULL (one); tier(h) = h / (H / n_tiers), H a multiple of n_tiers. */
void orc_head_norm_gate(int H, int d_v, int n_tiers, double eps, const double* o,
                        const double* g, const double* gamma, double* out);

/* Gradients of orc_head_norm_gate for ONE token given dout [H][d_v]: d_o and
 * dg [H][d_v] are overwritten, dgamma [n_tiers][d_v] is accumulated (NULL:
 * skipped). gamma NULL means one, as in the forward. */
void orc_head_norm_gate_bwd(int H, int d_v, int n_tiers, double eps, const double* o,
                            const double* g, const double* gamma, const double* dout,
                            double* d_o, double* dg, double* dgamma);

#ifdef __cplusplus
}
#endif
#endif
