/*
 * Simple GLA oracle (fp64, token by token). TEST INFRASTRUCTURE ONLY: see
 * oracle.h for who may use it and for the formulas it follows.
 *
 * Every function here is the plain definition, one token at a time, with no
 * chunking, blocking or reordering. Citations name sections of the page
 * "Beyond the KV cache: Training and serving i14's Laplace 3B linear attention
 * model on AWS Trainium2 with native PyTorch" (the Laplace 3B post).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Logistic sigmoid, evaluated so that neither branch overflows. */
static double sigmoid(double z)
{
    if (z >= 0.0) {
        return 1.0 / (1.0 + exp(-z));
    }
    double e = exp(z);
    return e / (1.0 + e);
}

/* Self-augmentation gate argument z_t = sum_i a_i q_i k_i.
 * Laplace 3B post, "GLA mixer": the gate is the query dotted with a learned
 * per-channel rescaling (aug_balance, a) of the key. */
static double aug_arg(int d_k, const double* a, const double* qt, const double* kt)
{
    double z = 0.0;
    if (a == NULL) {
        return 0.0;
    }
    for (int i = 0; i < d_k; ++i) {
        z += a[i] * qt[i] * kt[i];
    }
    return z;
}

/* Decay schedule. Laplace 3B post, "Decay schedule" and "Decay schedule's
 * reach": the per-head decays are fixed, geometric in the half-life, with
 * half-lives T_min (head 0) to T_max (last head); a half-life of T tokens
 * means lam^T = 1/2. */
void orc_decay_schedule(int H, double t_min, double t_max, double* lam)
{
    for (int h = 0; h < H; ++h) {
        double frac = (H > 1) ? (double)h / (double)(H - 1) : 0.0;
        double half_life = t_min * pow(t_max / t_min, frac);
        lam[h] = pow(2.0, -1.0 / half_life);
    }
}

/* Forward recurrence. Laplace 3B post, "GLA mixer": state update, readout,
 * then the self-augmentation term added to the head output. */
void orc_fwd(int T, int d_k, int d_v, double lam, const double* a,
             const double* q, const double* k, const double* v,
             const double* S0, double* o, double* S_final)
{
    size_t ns = (size_t)d_k * (size_t)d_v;
    double* S = (double*)calloc(ns, sizeof(double));
    if (S0 != NULL) {
        memcpy(S, S0, ns * sizeof(double));
    }
    for (int t = 0; t < T; ++t) {
        const double* qt = q + (size_t)t * d_k;
        const double* kt = k + (size_t)t * d_k;
        const double* vt = v + (size_t)t * d_v;
        double* ot = o + (size_t)t * d_v;
        /* S_t = lam S_{t-1} + k_t v_t^T */
        for (int i = 0; i < d_k; ++i) {
            for (int j = 0; j < d_v; ++j) {
                S[(size_t)i * d_v + j] = lam * S[(size_t)i * d_v + j] + kt[i] * vt[j];
            }
        }
        /* o_t = S_t^T q_t + sigmoid(z_t) v_t */
        double g = sigmoid(aug_arg(d_k, a, qt, kt));
        for (int j = 0; j < d_v; ++j) {
            double acc = 0.0;
            for (int i = 0; i < d_k; ++i) {
                acc += S[(size_t)i * d_v + j] * qt[i];
            }
            ot[j] = acc + g * vt[j];
        }
    }
    if (S_final != NULL) {
        memcpy(S_final, S, ns * sizeof(double));
    }
    free(S);
}

/* Gradients by reverse-mode differentiation of the forward recurrence above.
 * Laplace 3B post, "Challenge 3: Backward-pass unrolling for a sequential
 * recurrence": the backward differentiates through every sequential state
 * update. Here that is done token by token, in two passes:
 *
 *  pass 1 (forward in t): recompute S_t and set
 *      dq_t = S_t dO_t + sigmoid'(z_t) (dO_t . v_t) (a * k_t)
 *  pass 2 (backward in t): G = dL/dS_t, starting from dS_final,
 *      G <- lam G (for t < T-1), then G += q_t dO_t^T   (o_t reads S_t)
 *      dk_t = G v_t + sigmoid'(z_t) (dO_t . v_t) (a * q_t)
 *      dv_t = G^T k_t + sigmoid(z_t) dO_t
 *      da  += sigmoid'(z_t) (dO_t . v_t) (q_t * k_t)
 *  and finally dS0 = lam G (S_0 = lam S0 + k_0 v_0^T).
 */
void orc_bwd(int T, int d_k, int d_v, double lam, const double* a,
             const double* q, const double* k, const double* v,
             const double* S0, const double* dO, const double* dS_final,
             double* dq, double* dk, double* dv, double* da, double* dS0)
{
    size_t ns = (size_t)d_k * (size_t)d_v;
    double* S = (double*)calloc(ns, sizeof(double));
    double* G = (double*)calloc(ns, sizeof(double));

    /* pass 1: forward scan for dq */
    if (S0 != NULL) {
        memcpy(S, S0, ns * sizeof(double));
    }
    for (int t = 0; t < T; ++t) {
        const double* qt = q + (size_t)t * d_k;
        const double* kt = k + (size_t)t * d_k;
        const double* vt = v + (size_t)t * d_v;
        const double* dot = dO + (size_t)t * d_v;
        double* dqt = dq + (size_t)t * d_k;
        for (int i = 0; i < d_k; ++i) {
            for (int j = 0; j < d_v; ++j) {
                S[(size_t)i * d_v + j] = lam * S[(size_t)i * d_v + j] + kt[i] * vt[j];
            }
        }
        double s = sigmoid(aug_arg(d_k, a, qt, kt));
        double u = 0.0; /* dO_t . v_t */
        for (int j = 0; j < d_v; ++j) {
            u += dot[j] * vt[j];
        }
        double c = s * (1.0 - s) * u;
        for (int i = 0; i < d_k; ++i) {
            double acc = 0.0;
            for (int j = 0; j < d_v; ++j) {
                acc += S[(size_t)i * d_v + j] * dot[j];
            }
            dqt[i] = acc + ((a != NULL) ? c * a[i] * kt[i] : 0.0);
        }
    }

    /* pass 2: reverse scan for dk, dv, da, dS0 */
    if (dS_final != NULL) {
        memcpy(G, dS_final, ns * sizeof(double));
    }
    for (int t = T - 1; t >= 0; --t) {
        const double* qt = q + (size_t)t * d_k;
        const double* kt = k + (size_t)t * d_k;
        const double* vt = v + (size_t)t * d_v;
        const double* dot = dO + (size_t)t * d_v;
        double* dkt = dk + (size_t)t * d_k;
        double* dvt = dv + (size_t)t * d_v;
        if (t < T - 1) {
            for (size_t e = 0; e < ns; ++e) {
                G[e] *= lam;
            }
        }
        for (int i = 0; i < d_k; ++i) {
            for (int j = 0; j < d_v; ++j) {
                G[(size_t)i * d_v + j] += qt[i] * dot[j];
            }
        }
        double s = sigmoid(aug_arg(d_k, a, qt, kt));
        double u = 0.0;
        for (int j = 0; j < d_v; ++j) {
            u += dot[j] * vt[j];
        }
        double c = s * (1.0 - s) * u;
        for (int i = 0; i < d_k; ++i) {
            double acc = 0.0;
            for (int j = 0; j < d_v; ++j) {
                acc += G[(size_t)i * d_v + j] * vt[j];
            }
            dkt[i] = acc + ((a != NULL) ? c * a[i] * qt[i] : 0.0);
            da[i] += c * qt[i] * kt[i];
        }
        for (int j = 0; j < d_v; ++j) {
            double acc = 0.0;
            for (int i = 0; i < d_k; ++i) {
                acc += G[(size_t)i * d_v + j] * kt[i];
            }
            dvt[j] = acc + s * dot[j];
        }
    }
    if (dS0 != NULL) {
        for (size_t e = 0; e < ns; ++e) {
            dS0[e] = (T > 0) ? lam * G[e] : G[e];
        }
    }
    free(S);
    free(G);
}

/* One serving step. Laplace 3B post, "Inference optimization on Trainium2",
 * "Constant serving state": the recurrent state is fixed-size per sequence and
 * each new token is one step of the recurrence on it. */
void orc_decode_step(int d_k, int d_v, double lam, const double* a,
                     const double* q, const double* k, const double* v,
                     double* S, double* o)
{
    for (int i = 0; i < d_k; ++i) {
        for (int j = 0; j < d_v; ++j) {
            S[(size_t)i * d_v + j] = lam * S[(size_t)i * d_v + j] + k[i] * v[j];
        }
    }
    double g = sigmoid(aug_arg(d_k, a, q, k));
    for (int j = 0; j < d_v; ++j) {
        double acc = 0.0;
        for (int i = 0; i < d_k; ++i) {
            acc += S[(size_t)i * d_v + j] * q[i];
        }
        o[j] = acc + g * v[j];
    }
}

/* ------------------------------------------------------------------------
 * Convolution prologue of the mixer. Laplace 3B post, "i14 and the Laplace 3B
 * architecture": before the QKVG projection every token's (normalised)
 * residual vector goes through a depthwise causal Conv1d of width 4 with a
 * SiLU, which hands each position a 4-gram summary of its own and the three
 * previous tokens (the architecture table lists the same: depthwise causal
 * Conv1d, kernel width 4, SiLU). Channel by channel, with the filter taps
 * ordered oldest first (as a PyTorch depthwise Conv1d weight [D, 1, 4] with
 * three zeros of left padding):
 *
 *   y_t[c] = silu(b[c] + sum_{j=0..3} w[c][j] u_{t-3+j}[c]),   silu(x) = x sigmoid(x)
 *
 * For serving, the three previous inputs are the per-sequence conv state
 * ("Inference optimization on Trainium2", "Constant serving state": the fixed
 * per-sequence state that a generated token reads and updates).
 */
static double silu(double x)
{
    return x * sigmoid(x);
}

/* One sequence of L tokens. u_{-3..-1} = st[0..2] (NULL: zero); st_out (may be
 * NULL, may equal st) receives u_{L-3}, u_{L-2}, u_{L-1}, reaching back into
 * st when L < 3. */
void orc_conv_fwd(int L, int D, const double* w, const double* b, const double* u,
                  const double* st, double* y, double* st_out)
{
    for (int t = 0; t < L; ++t) {
        for (int c = 0; c < D; ++c) {
            double acc = (b != NULL) ? b[c] : 0.0;
            for (int j = 0; j < 4; ++j) {
                const int s = t - 3 + j;
                double x;
                if (s >= 0) {
                    x = u[(size_t)s * D + c];
                } else {
                    x = (st != NULL) ? st[(size_t)(3 + s) * D + c] : 0.0;
                }
                acc += w[(size_t)c * 4 + j] * x;
            }
            y[(size_t)t * D + c] = silu(acc);
        }
    }
    if (st_out != NULL) {
        double* nxt = (double*)malloc(sizeof(double) * 3 * (size_t)D);
        for (int j = 0; j < 3; ++j) {
            const int s = L - 3 + j;
            for (int c = 0; c < D; ++c) {
                double x;
                if (s >= 0) {
                    x = u[(size_t)s * D + c];
                } else {
                    x = (st != NULL) ? st[(size_t)(3 + s) * D + c] : 0.0;
                }
                nxt[(size_t)j * D + c] = x;
            }
        }
        memcpy(st_out, nxt, sizeof(double) * 3 * (size_t)D);
        free(nxt);
    }
}

/* One serving step on the conv state in place: y = silu(b + w . [st0, st1, st2, x]),
 * then the state shifts by one token. */
void orc_conv_decode_step(int D, const double* w, const double* b, const double* x,
                          double* st, double* y)
{
    for (int c = 0; c < D; ++c) {
        double acc = (b != NULL) ? b[c] : 0.0;
        acc += w[(size_t)c * 4 + 0] * st[c];
        acc += w[(size_t)c * 4 + 1] * st[(size_t)D + c];
        acc += w[(size_t)c * 4 + 2] * st[(size_t)2 * D + c];
        acc += w[(size_t)c * 4 + 3] * x[c];
        y[c] = silu(acc);
        st[c] = st[(size_t)D + c];
        st[(size_t)D + c] = st[(size_t)2 * D + c];
        st[(size_t)2 * D + c] = x[c];
    }
}

/* Mixer epilogue for ONE token. Laplace 3B post, "i14 and the Laplace 3B
 * architecture", end of the "GLA mixer" paragraph and the "Decay schedule's
 * reach" paragraph: each head's output goes through a Head RMSNorm, the heads
 * of a decay tier share that norm (its learned per-channel scale), the heads
 * are concatenated and the result is gated by SiLU(g_t).
 * Tiers are n_tiers contiguous runs of H / n_tiers heads. */
void orc_head_norm_gate(int H, int d_v, int n_tiers, double eps, const double* o,
                        const double* g, const double* gamma, double* out)
{
    const int per_tier = H / n_tiers;
    for (int h = 0; h < H; ++h) {
        const double* oh = o + (size_t)h * d_v;
        /* root mean square of this head's d_v outputs */
        double ss = 0.0;
        for (int c = 0; c < d_v; ++c) {
            ss += oh[c] * oh[c];
        }
        const double inv_rms = 1.0 / sqrt(ss / d_v + eps);
        const int tier = h / per_tier;
        for (int c = 0; c < d_v; ++c) {
            const double scale = (gamma != NULL) ? gamma[(size_t)tier * d_v + c] : 1.0;
            const double gc = g[(size_t)h * d_v + c];
            out[(size_t)h * d_v + c] = silu(gc) * (scale * oh[c] * inv_rms);
        }
    }
}

/* Gradients of the mixer epilogue for ONE token, given dout = dL/dout [H][d_v].
 * With r = sqrt(mean_c o[h][c]^2 + eps), y = o / r, s = silu(g) and the scale
 * gm = gamma[tier(h)][c] (1 when gamma is NULL), out = s gm y, so
 *   dL/dg[h][c]     = dout gm y silu'(g),    silu'(x) = sigmoid(x) (1 + x (1 - sigmoid(x)))
 *   dL/dgamma[t][c] += sum over the heads h of tier t of dout s y
 *   dL/dy[h][c]     = w = dout s gm
 *   dL/do[h][c]     = (w - y mean_c' (w y)) / r
 * (the last by differentiating y = o / r through r). dgamma is accumulated,
 * not overwritten, so that callers can sum it over tokens; NULL skips it. */
void orc_head_norm_gate_bwd(int H, int d_v, int n_tiers, double eps, const double* o,
                            const double* g, const double* gamma, const double* dout,
                            double* d_o, double* dg, double* dgamma)
{
    const int per_tier = H / n_tiers;
    for (int h = 0; h < H; ++h) {
        const double* oh = o + (size_t)h * d_v;
        double ss = 0.0;
        for (int c = 0; c < d_v; ++c) {
            ss += oh[c] * oh[c];
        }
        const double r = sqrt(ss / d_v + eps);
        const int tier = h / per_tier;
        double wy = 0.0;
        for (int c = 0; c < d_v; ++c) {
            const size_t i = (size_t)h * d_v + c;
            const double gm = (gamma != NULL) ? gamma[(size_t)tier * d_v + c] : 1.0;
            const double y = oh[c] / r;
            const double sg = sigmoid(g[i]);
            const double s = g[i] * sg;
            dg[i] = dout[i] * gm * y * sg * (1.0 + g[i] * (1.0 - sg));
            if (dgamma != NULL) {
                dgamma[(size_t)tier * d_v + c] += dout[i] * s * y;
            }
            wy += dout[i] * s * gm * y;
        }
        for (int c = 0; c < d_v; ++c) {
            const size_t i = (size_t)h * d_v + c;
            const double gm = (gamma != NULL) ? gamma[(size_t)tier * d_v + c] : 1.0;
            const double w = dout[i] * silu(g[i]) * gm;
            d_o[i] = (w - (oh[c] / r) * (wy / d_v)) / r;
        }
    }
}

/* Gradients of orc_conv_fwd for ONE sequence of L tokens, given dy [L][D] and
 * d_st_out [3][D] (the gradient of the final conv state, or NULL). With
 * x_s = u_s for s >= 0 and st[3 + s] for s < 0 (zero without st), and
 * pre_t = b + sum_j w_j x_{t-3+j}, y_t = silu(pre_t):
 *   dpre_t       = dy_t silu'(pre_t)
 *   dL/dx_s      = sum over j with 0 <= s + 3 - j < L of w_j dpre_{s+3-j}
 *                  (+ d_st_out[i] when x_s is row i of the final state, s = L - 3 + i)
 *   du_s = dL/dx_s for s >= 0;  d_st[i] = dL/dx_{i-3} (NULL: not written)
 *   dw[c][j] += sum_t dpre_t x_{t-3+j};  db[c] += sum_t dpre_t (accumulated; NULL: skipped)
 * The last two are accumulated so that callers can sum them over sequences. */
void orc_conv_bwd(int L, int D, const double* w, const double* b, const double* u,
                  const double* st, const double* dy, const double* d_st_out, double* du,
                  double* d_st, double* dw, double* db)
{
    for (int c = 0; c < D; ++c) {
        /* x_s for s = -3 .. L-1 and dpre_t for t = 0 .. L-1 of this channel */
        double* x = (double*)malloc(sizeof(double) * (size_t)(L + 3));
        double* dpre = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
        for (int s = -3; s < L; ++s) {
            x[s + 3] = (s >= 0) ? u[(size_t)s * D + c] : ((st != NULL) ? st[(size_t)(3 + s) * D + c] : 0.0);
        }
        for (int t = 0; t < L; ++t) {
            double pre = (b != NULL) ? b[c] : 0.0;
            for (int j = 0; j < 4; ++j) {
                pre += w[(size_t)c * 4 + j] * x[t + j];
            }
            const double sg = sigmoid(pre);
            dpre[t] = dy[(size_t)t * D + c] * sg * (1.0 + pre * (1.0 - sg));
            for (int j = 0; j < 4; ++j) {
                if (dw != NULL) {
                    dw[(size_t)c * 4 + j] += dpre[t] * x[t + j];
                }
            }
            if (db != NULL) {
                db[c] += dpre[t];
            }
        }
        for (int s = -3; s < L; ++s) {
            double g = 0.0;
            for (int j = 0; j < 4; ++j) {
                const int t = s + 3 - j;
                if (t >= 0 && t < L) {
                    g += w[(size_t)c * 4 + j] * dpre[t];
                }
            }
            const int i = s - (L - 3);
            if (d_st_out != NULL && i >= 0 && i < 3) {
                g += d_st_out[(size_t)i * D + c];
            }
            if (s >= 0) {
                du[(size_t)s * D + c] = g;
            } else if (d_st != NULL) {
                d_st[(size_t)(3 + s) * D + c] = g;
            }
        }
        free(x);
        free(dpre);
    }
}
