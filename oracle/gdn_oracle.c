/*
 * Plain sequential fp64 CPU oracle of the gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library: every value here is computed
 * from its definition, token by token, in double precision, with no chunking,
 * blocking or fusion.  Callers convert every stored bf16/fp32 input exactly to
 * double before the call and compare against the double results.
 *
 * Sources (the four pages this project is built from):
 *  - metaltile-std `gated_delta.rs` (docs.rs), module doc, "Recurrence per step"
 *    and "Layouts": the gated delta rule for one token; state [B,Hv,Dv,Dk]
 *    with Dk fastest; q,k [B,Hk,Dk]; head sharing hk = hv/(Hv/Hk).
 *  - KBench `comba_decode_step` spec, spec_md and contract_md: the Comba step
 *    with a separate read key p and a query scale; state [B,H,K,V], V fastest.
 *  - pymllm `gdn_chunkwise` docs, `gdn_extend_chunkwise` parameters: packed
 *    variable-length prefill over a state pool picked by cache_indices and
 *    delimited by cu_seqlens, q/k not pre-normalised, raw gate inputs a, b
 *    with A_log and dt_bias.
 *  - regolith `gdn.metal` header comment: gate = exp(-exp(A_log) softplus(a +
 *    dt_bias)), beta = sigmoid(b), q/k L2 norm with eps 1e-6, q scaled by
 *    Dk^-1/2.
 *
 * Build: gcc -O2 -fPIC -shared -o liboracle.so gdn_oracle.c -lm
 * (no -ffast-math, no FMA contraction flags: IEEE double throughout).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/*
 * One gated delta-rule step on one value head (metaltile-std `gated_delta.rs`,
 * module documentation, "Recurrence per step").  S is the head's Dv x Dk
 * state matrix, stored row by row (S[j*Dk + i]: value index j, key index i),
 * so that the readout is y = S q.  With a = exp(g) (g the log-space gate) the
 * step is the matrix update
 *     S' = a S (I - beta k k^T) + beta v k^T,
 * which multiplies out to a rank-one correction of the decayed state:
 *     S' = a S + e k^T,   e = beta (v - a S k),
 * and the output reads the new state:
 *     y = S' q = a (S q) + (k . q) e.
 * Both products with the old state (S k and S q) are formed first, then the
 * state is overwritten.  Sk and Sq are scratch vectors of length Dv.
 */
static void gdn_head_step(double* S, const double* q, const double* k,
                          const double* v, double g, double beta, double* y,
                          int Dk, int Dv, double* Sk, double* Sq) {
  const double a = exp(g);
  double kq = 0.0;
  for (int i = 0; i < Dk; ++i) kq += k[i] * q[i];
  for (int j = 0; j < Dv; ++j) {
    const double* row = S + (size_t)j * Dk;
    double rk = 0.0, rq = 0.0;
    for (int i = 0; i < Dk; ++i) {
      rk += row[i] * k[i];
      rq += row[i] * q[i];
    }
    Sk[j] = rk;
    Sq[j] = rq;
  }
  for (int j = 0; j < Dv; ++j) {
    double* row = S + (size_t)j * Dk;
    const double e = beta * (v[j] - a * Sk[j]);
    for (int i = 0; i < Dk; ++i) row[i] = a * row[i] + e * k[i];
    y[j] = a * Sq[j] + kq * e;
  }
}

/*
 * Decode step for a dense batch (metaltile page, `mt_gated_delta_step`
 * layouts): state [B,Hv,Dv,Dk] updated in place, q,k [B,Hk,Dk],
 * v,y [B,Hv,Dv], g (log-space), beta [B,Hv].  Value head hv reads key head
 * hk = hv / (Hv/Hk) (contiguous groups, the page's DISPATCH INVARIANTS).
 * Returns 0, or -1 on an invalid shape.
 */
int oracle_gdn_step(double* state, const double* q, const double* k,
                    const double* v, const double* g, const double* beta,
                    double* y, int B, int Hk, int Hv, int Dk, int Dv) {
  if (B < 0 || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0 || Hv % Hk != 0) return -1;
  double* Sk = (double*)malloc(sizeof(double) * (size_t)Dv * 2);
  if (!Sk) return -1;
  double* Sq = Sk + Dv;
  const int group = Hv / Hk;
  for (int b = 0; b < B; ++b) {
    for (int hv = 0; hv < Hv; ++hv) {
      const int hk = hv / group;
      const size_t n = (size_t)b * Hv + hv;
      const size_t qk = ((size_t)b * Hk + hk) * Dk;
      gdn_head_step(state + n * Dv * Dk, q + qk, k + qk, v + n * Dv, g[n],
                    beta[n], y + n * Dv, Dk, Dv, Sk, Sq);
    }
  }
  free(Sk);
  return 0;
}

/*
 * x / sqrt(sum x^2 + eps), the L2 normalisation the regolith kernel applies
 * to q and k (its header comment; eps = 1e-6 there).  An all-zero row maps
 * to zero.
 */
static void l2_normalise(const double* x, double* out, int n, double eps) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  const double r = 1.0 / sqrt(ss + eps);
  for (int i = 0; i < n; ++i) out[i] = x[i] * r;
}

/*
 * Variable-length prefill over a state pool (pymllm `gdn_extend_chunkwise`
 * contract), computed token by token with no chunking:
 *   for each sequence s (tokens cu_seqlens[s] .. cu_seqlens[s+1]-1) and each
 *   value head hv, the state pool[cache_indices[s], hv] is advanced by one
 *   gated delta-rule step per token and written back in place.
 * q,k [T,Hk,Dk]; v,y [T,Hv,Dv]; g (log-space), beta [T,Hv];
 * pool [pool_size,Hv,Dv,Dk]; cache_indices [N_s]; cu_seqlens [N_s+1].
 * If l2norm != 0 the step uses k/sqrt(|k|^2+eps) and
 * scale*q/sqrt(|q|^2+eps); otherwise k and scale*q.
 * Slots not named in cache_indices are never touched.
 * Returns 0, or -1 on an invalid shape or index.
 */
int oracle_gdn_prefill(const double* q, const double* k, const double* v,
                       const double* g, const double* beta, double* pool,
                       int64_t pool_size, const int64_t* cache_indices,
                       const int64_t* cu_seqlens, int N_s, int64_t T_tot,
                       int Hk, int Hv, int Dk, int Dv, double scale, int l2norm,
                       double eps, double* y) {
  if (N_s < 0 || Hk <= 0 || Hv <= 0 || Dk <= 0 || Dv <= 0 || Hv % Hk != 0) return -1;
  if (N_s > 0 && (cu_seqlens[0] != 0 || cu_seqlens[N_s] != T_tot)) return -1;
  for (int s = 0; s < N_s; ++s) {
    if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
    if (cache_indices[s] < 0 || cache_indices[s] >= pool_size) return -1;
  }
  double* work = (double*)malloc(sizeof(double) * ((size_t)Dv * 2 + (size_t)Dk * 2));
  if (!work) return -1;
  double* Sk = work;
  double* Sq = Sk + Dv;
  double* kn = Sq + Dv;
  double* qn = kn + Dk;
  const int group = Hv / Hk;
  for (int s = 0; s < N_s; ++s) {
    const int64_t slot = cache_indices[s];
    for (int hv = 0; hv < Hv; ++hv) {
      const int hk = hv / group;
      double* S = pool + ((size_t)slot * Hv + hv) * (size_t)Dv * Dk;
      for (int64_t t = cu_seqlens[s]; t < cu_seqlens[s + 1]; ++t) {
        const double* kt = k + ((size_t)t * Hk + hk) * Dk;
        const double* qt = q + ((size_t)t * Hk + hk) * Dk;
        if (l2norm) {
          l2_normalise(kt, kn, Dk, eps);
          l2_normalise(qt, qn, Dk, eps);
        } else {
          memcpy(kn, kt, sizeof(double) * Dk);
          memcpy(qn, qt, sizeof(double) * Dk);
        }
        for (int i = 0; i < Dk; ++i) qn[i] *= scale;
        const size_t th = (size_t)t * Hv + hv;
        gdn_head_step(S, qn, kn, v + th * Dv, g[th], beta[th], y + th * Dv, Dk,
                      Dv, Sk, Sq);
      }
    }
  }
  free(work);
  return 0;
}

/*
 * One Comba step for a dense batch (KBench `comba_decode_step` specification
 * and contract).  Per (batch, head), S is the K x V state matrix stored row
 * by row (S[i*V + j]: key index i, value index j), read through its own key
 * p and written through k.  With a = exp(g) the matrix update is
 *     S' = a (I - beta k p^T) S + beta k v^T  =  a S + k u^T,
 *     u  = beta (v - a S^T p),
 * and the output reads the new state with the scaled query qs = scale q:
 *     o = S'^T qs = a (S^T qs) + (k . qs) u.
 * q, k, p [B,H,K]; v, o [B,H,V]; beta, g [B,H]; state [B,H,K,V], in place.
 * Returns 0, or -1 on an invalid shape.
 */
int oracle_comba_step(double* state, const double* q, const double* k,
                      const double* v, const double* p, const double* beta,
                      const double* g, double scale, double* o, int B, int H,
                      int K, int V) {
  if (B < 0 || H <= 0 || K <= 0 || V <= 0) return -1;
  double* col = (double*)malloc(sizeof(double) * (size_t)V * 2);
  if (!col) return -1;
  double* Stp = col;      /* S^T p  */
  double* Stq = col + V;  /* S^T qs */
  for (int b = 0; b < B; ++b) {
    for (int h = 0; h < H; ++h) {
      const size_t n = (size_t)b * H + h;
      double* S = state + n * (size_t)K * V;
      const double* qh = q + n * K;
      const double* kh = k + n * K;
      const double* ph = p + n * K;
      const double* vh = v + n * V;
      const double a = exp(g[n]);
      double kq = 0.0;
      for (int i = 0; i < K; ++i) kq += kh[i] * (scale * qh[i]);
      for (int j = 0; j < V; ++j) Stp[j] = Stq[j] = 0.0;
      for (int i = 0; i < K; ++i) {
        const double* row = S + (size_t)i * V;
        const double pi = ph[i], qi = scale * qh[i];
        for (int j = 0; j < V; ++j) {
          Stp[j] += pi * row[j];
          Stq[j] += qi * row[j];
        }
      }
      for (int j = 0; j < V; ++j) {
        const double u = beta[n] * (vh[j] - a * Stp[j]);
        Stp[j] = u;  /* from here on: u */
        o[n * V + j] = a * Stq[j] + kq * u;
      }
      for (int i = 0; i < K; ++i) {
        double* row = S + (size_t)i * V;
        for (int j = 0; j < V; ++j) row[j] = a * row[j] + kh[i] * Stp[j];
      }
    }
  }
  free(col);
  return 0;
}

/*
 * Gate prologue for prefill (pymllm `gdn_extend_chunkwise` parameters a, b,
 * A_log, dt_bias; formula from the regolith header comment), in exact fp64:
 *   g[t,h]    = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])   (log-space)
 *   beta[t,h] = 1 / (1 + exp(-b[t,h]))
 * softplus(x) = log(1 + e^x), evaluated as max(x,0) + log1p(exp(-|x|)),
 * which is the same function without overflow (no threshold).
 */
void oracle_gates(const double* a, const double* b, const double* A_log,
                  const double* dt_bias, double* g, double* beta, int64_t T,
                  int Hv) {
  for (int64_t t = 0; t < T; ++t) {
    for (int h = 0; h < Hv; ++h) {
      const size_t n = (size_t)t * Hv + h;
      const double x = a[n] + dt_bias[h];
      const double sp = (x > 0.0 ? x : 0.0) + log1p(exp(-fabs(x)));
      g[n] = -exp(A_log[h]) * sp;
      beta[n] = 1.0 / (1.0 + exp(-b[n]));
    }
  }
}

/*
 * Short causal convolution + SiLU of the layer's q/k/v channels, with a
 * rolling history per pool slot (regolith `gdn.metal`: header comment and
 * the conv/SiLU block of its kernel; 4 taps, history [channels][3] oldest
 * first).  x and out are [T][C] (C channels per token); W is [C][4], tap 3
 * weighting the current token; hist is [pool][C][3].  For each sequence s
 * (tokens cu[s] .. cu[s+1]-1) with slot = cache_indices[s], and each
 * channel c, the window at token t is (x[t-3], x[t-2], x[t-1], x[t]), where
 * inputs before the sequence's first token are the slot's history
 * (hist[0] the oldest, hist[2] the newest).  Then
 *   pre = sum_m window[m] W[c][m],   out[t][c] = pre / (1 + exp(-pre)),
 * and afterwards the slot's history holds the newest three entries of
 * (old history, the sequence's inputs), oldest first.  A zero-length
 * sequence leaves its slot untouched; other slots are never touched.
 */
int oracle_conv_silu(const double* x, const double* W, double* hist, int64_t pool,
                     const int64_t* cache_indices, const int64_t* cu, int N_s, int64_t T,
                     int C, double* out) {
  if (N_s < 0 || T < 0 || C <= 0 || pool < 0) return -1;
  for (int s = 0; s < N_s; ++s) {
    const int64_t t0 = cu[s], t1 = cu[s + 1];
    const int64_t slot = cache_indices[s];
    if (t0 < 0 || t1 < t0 || t1 > T) return -1;
    if (t1 == t0) continue;
    if (slot < 0 || slot >= pool) return -1;
    for (int c = 0; c < C; ++c) {
      double* h = hist + ((size_t)slot * C + c) * 3;
      double win[4] = {h[0], h[1], h[2], 0.0};  /* win[0..2]: the three previous inputs */
      for (int64_t t = t0; t < t1; ++t) {
        win[3] = x[(size_t)t * C + c];
        double pre = 0.0;
        for (int m = 0; m < 4; ++m) pre += win[m] * W[(size_t)c * 4 + m];
        out[(size_t)t * C + c] = pre / (1.0 + exp(-pre));
        win[0] = win[1];
        win[1] = win[2];
        win[2] = win[3];
      }
      h[0] = win[0];
      h[1] = win[1];
      h[2] = win[2];
    }
  }
  return 0;
}

/*
 * Gated RMS norm of the recurrence output (regolith `gdn.metal` header
 * comment and the kernel's output block): per (token, value head), over the
 * Dv outputs o_j of that head,
 *   y_j = o_j / sqrt(mean_j(o_j^2) + eps) * gamma[j] * sigmoid(z_j),
 * with gamma [Dv] shared by every head.  o, z, y are [T][Hv][Dv].
 */
void oracle_gated_rmsnorm(const double* o, const double* z, const double* gamma, double eps,
                          int64_t T, int Hv, int Dv, double* y) {
  for (int64_t t = 0; t < T; ++t) {
    for (int h = 0; h < Hv; ++h) {
      const size_t base = ((size_t)t * Hv + h) * Dv;
      double ss = 0.0;
      for (int j = 0; j < Dv; ++j) ss += o[base + j] * o[base + j];
      const double r = 1.0 / sqrt(ss / Dv + eps);
      for (int j = 0; j < Dv; ++j)
        y[base + j] = o[base + j] * r * gamma[j] * (1.0 / (1.0 + exp(-z[base + j])));
    }
  }
}
