/*
 * ssd_oracle.c -- the oracle: a plain, slow, fp64 CPU implementation of the
 * Mamba-2 mixer hot path (causal depthwise conv1d + SiLU, selective-SSM scan,
 * one-token conv and state updates).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do.  It shares no code, header or constant with the HIP library.
 *
 * Every routine is the plain definition written out, token by token, with no
 * chunking, blocking or re-association: the chunked SSD scan reaches the same
 * result (up to rounding order) because it is an exact re-association of this
 * recurrence.
 *
 * Sources (web pages; cited by title and section):
 *  [P1] "Mamba 与 Nemotron 系列模型深度调研" (kenforever1 blog), section
 *       "Mamba 架构 / 1. Selective SSM 的直觉": per token the state decays by
 *       exp(A*dt) and gains dt*B*x; the output contracts the already-updated
 *       state with C and adds the skip D*x.  Section "状态契约": recurrent
 *       state [batch, heads, head_dim, state_size], conv state
 *       [batch, conv_dim, conv_kernel].
 *  [P2] walk-through of NVIDIA-Nemotron-Labs-Teacher-Chat modeling_nemotron_h.py,
 *       sections "Prefill 阶段" (causal conv writes the last 4 conv inputs into
 *       the conv state; chunked scan returns the final state) and "Decode 阶段"
 *       (conv state rolled by one with the new token in the last slot; state
 *       updated with exp(dt*A) and dt*B*x, then y = state*C + D*x).
 *  [P3] "MAX 平台 Nemotron-H 混合架构解析", section "4.5 Mamba-2 mixer 字段"
 *       (conv_dim = heads*head_dim + 2*n_groups*state; x | B | C channel order)
 *       and "5.4 NemotronHMamba2Mixer" (depthwise SiLU conv over x|B|C).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - head h uses group g(h) = h / (H/G)  (contiguous heads per group);
 *  - B enters as the Euler term dt*B*x, A as exact exp(dt*A);
 *  - y reads the state after this token's update;
 *  - the conv state keeps K columns; column 0 is overwritten by the roll and
 *    never feeds an output; the bias is optional (NULL = 0).
 *
 * Layouts (all fp64, C-contiguous):
 *  u, v        [Bt, L, CD]      conv input / output, channels last
 *  w           [CD, K]          depthwise conv taps, tap K-1 multiplies the newest token
 *  s_in, s_out [Bt, CD, K]      conv state, column K-1 = most recent input
 *  x, y        [Bt, L, H, P]
 *  Bm, Cm      [Bt, L, G, N]
 *  dt          [Bt, L, H]
 *  A, D        [H]
 *  init, fin   [Bt, H, P, N]
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* silu(z) = z * sigmoid(z)  ([P3] 5.4: the conv is a SiLU-activated depthwise conv) */
static double silu(double z) { return z / (1.0 + exp(-z)); }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Prefill conv ([P2] "Prefill 阶段"; [P3] 5.4).
 * Extended input: ut(b, tau, c) = u[b, tau, c] for 0 <= tau < L, and for the
 * K-1 tokens before the sequence, ut(b, tau, c) = s_in[b, c, K + tau]
 * (tau = -(K-1) .. -1), or 0 when s_in is NULL.
 *   v[b,t,c]     = silu(bias[c] + sum_k w[c,k] * ut(b, t-(K-1)+k, c))
 *   s_out[b,c,k] = ut(b, L-K+k, c)          (the last K conv inputs)
 * s_out must not alias s_in.
 */
static double conv_ext(const double* u, const double* s_in, int64_t L, int64_t CD,
                       int K, int64_t b, int64_t tau, int64_t c) {
    if (tau >= 0) return u[(b * L + tau) * CD + c];
    if (s_in == NULL) return 0.0;
    return s_in[(b * CD + c) * K + (K + tau)];
}

void oracle_conv1d_fwd(int64_t Bt, int64_t L, int64_t CD, int K,
                       const double* u, const double* w, const double* bias,
                       const double* s_in, double* v, double* s_out) {
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < Bt; ++b) {
        for (int64_t c = 0; c < CD; ++c) {
            for (int64_t t = 0; t < L; ++t) {
                double acc = bias ? bias[c] : 0.0;
                for (int k = 0; k < K; ++k)
                    acc += w[c * K + k] * conv_ext(u, s_in, L, CD, K, b, t - (K - 1) + k, c);
                v[(b * L + t) * CD + c] = silu(acc);
            }
            if (s_out) {
                for (int k = 0; k < K; ++k)
                    s_out[(b * CD + c) * K + k] = conv_ext(u, s_in, L, CD, K, b, L - K + k, c);
            }
        }
    }
}

/*
 * One-token conv update ([P2] "Decode 阶段": roll the window left by one, put
 * the new input in the last slot, then convolve with the taps).
 *   s[b,c,:] <- (s[b,c,1], ..., s[b,c,K-1], u[b,c])
 *   v[b,c]    = silu(bias[c] + sum_k w[c,k] * s[b,c,k])
 */
void oracle_conv1d_update(int64_t Bt, int64_t CD, int K,
                          const double* u, const double* w, const double* bias,
                          double* s, double* v) {
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < Bt; ++b) {
        for (int64_t c = 0; c < CD; ++c) {
            double* sc = s + (b * CD + c) * K;
            for (int k = 0; k + 1 < K; ++k) sc[k] = sc[k + 1];
            sc[K - 1] = u[b * CD + c];
            double acc = bias ? bias[c] : 0.0;
            for (int k = 0; k < K; ++k) acc += w[c * K + k] * sc[k];
            v[b * CD + c] = silu(acc);
        }
    }
}

/*
 * Selective-SSM scan, token by token ([P1] section 1; [P2] "Decode 阶段"
 * applied to every token in order).  For each (b, h, p), with the state row
 * S[n] = init[b,h,p,n] (0 when init is NULL) and g = h / (H/G):
 *   for t = 0 .. L-1:
 *     a     = exp(dt[b,t,h] * A[h])
 *     S[n]  = a * S[n] + dt[b,t,h] * Bm[b,t,g,n] * x[b,t,h,p]
 *     y[b,t,h,p] = sum_n S[n] * Cm[b,t,g,n] + D[h] * x[b,t,h,p]
 *   fin[b,h,p,:] = S
 * D may be NULL (no skip term); fin may be NULL.
 */
void oracle_ssm_scan(int64_t Bt, int64_t L, int H, int P, int G, int N,
                     const double* x, const double* Bm, const double* Cm,
                     const double* dt, const double* A, const double* D,
                     const double* init, double* y, double* fin) {
    const int heads_per_group = H / G;
    #pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)N);
        #pragma omp for collapse(3) schedule(static)
        for (int64_t b = 0; b < Bt; ++b) {
            for (int h = 0; h < H; ++h) {
                for (int p = 0; p < P; ++p) {
                    const int g = h / heads_per_group;
                    for (int n = 0; n < N; ++n)
                        S[n] = init ? init[(((b * H) + h) * P + p) * N + n] : 0.0;
                    for (int64_t t = 0; t < L; ++t) {
                        const double d = dt[(b * L + t) * H + h];
                        const double xv = x[((b * L + t) * H + h) * P + p];
                        const double* Bt_ = Bm + ((b * L + t) * G + g) * N;
                        const double* Ct_ = Cm + ((b * L + t) * G + g) * N;
                        const double a = exp(d * A[h]);
                        double acc = 0.0;
                        for (int n = 0; n < N; ++n) {
                            S[n] = a * S[n] + d * Bt_[n] * xv;
                            acc += S[n] * Ct_[n];
                        }
                        y[((b * L + t) * H + h) * P + p] = acc + (D ? D[h] * xv : 0.0);
                    }
                    if (fin)
                        for (int n = 0; n < N; ++n)
                            fin[(((b * H) + h) * P + p) * N + n] = S[n];
                }
            }
        }
        free(S);
    }
}

/*
 * Single-token selective state update, in place ([P2] "Decode 阶段"):
 *   a = exp(dt[b,h] * A[h]);  state[b,h,p,n] = a*state + dt*Bm[b,g,n]*x[b,h,p]
 *   y[b,h,p] = sum_n state[b,h,p,n] * Cm[b,g,n] + D[h] * x[b,h,p]
 * Layouts: state [Bt,H,P,N]; x, y [Bt,H,P]; Bm, Cm [Bt,G,N]; dt [Bt,H].
 */
void oracle_state_update(int64_t Bt, int H, int P, int G, int N, double* state,
                         const double* x, const double* Bm, const double* Cm,
                         const double* dt, const double* A, const double* D,
                         double* y) {
    const int heads_per_group = H / G;
    #pragma omp parallel for collapse(3) schedule(static)
    for (int64_t b = 0; b < Bt; ++b) {
        for (int h = 0; h < H; ++h) {
            for (int p = 0; p < P; ++p) {
                const int g = h / heads_per_group;
                const double d = dt[b * H + h];
                const double xv = x[(b * H + h) * P + p];
                const double a = exp(d * A[h]);
                double* S = state + (((b * H) + h) * P + p) * N;
                const double* Bv = Bm + (b * G + g) * N;
                const double* Cv = Cm + (b * G + g) * N;
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    S[n] = a * S[n] + d * Bv[n] * xv;
                    acc += S[n] * Cv[n];
                }
                y[(b * H + h) * P + p] = acc + (D ? D[h] * xv : 0.0);
            }
        }
    }
}
