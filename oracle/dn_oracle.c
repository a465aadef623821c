/*
 * dn_oracle.c -- plain fp64 CPU oracle of the gated-DeltaNet decode step.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it. It shares no code, header, table or helper with the HIP library.
 *
 * Sources (web pages; cited by title and section):
 *   [DN-GPU]  colibri PR "qwen36: run the DeltaNet layer end to end on the card
 *             (Q36_DN_GPU=1): conv, recurrence and gated norm join the two
 *             projections", section "What the PR does", Backend paragraph: the
 *             order of the steps of one decode token.
 *   [TRUNK]   colibri PR "feat(qwen36): the dense trunk places itself", section
 *             "What this adds", item 1: the fused qkv ++ z int8 projection.
 *   [FMT6]    colibri PR "cuda: fmt=6 (E8/IQ3) decode kernels, so E8 containers
 *             can reach VRAM", section "Tests": the checker is written from the
 *             description, in double precision, and shares nothing with the fast
 *             path, so a common-mode error cannot hide in both.
 *
 * Everything is computed in double. Integer weights are widened exactly; the
 * fp32 inputs are widened exactly. Each function is the plain definition of one
 * step, with no blocking, fusion or reordering. Readings where the pages are
 * silent are stated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define DNO_X_RMSNORM 1u
#define DNO_ALPHA_PER_KEY 2u
#define DNO_GATES_ON_DEVICE 4u

typedef struct {
  int d_model, n_k_heads, d_k, n_v_heads, d_v;
  int conv_k, batch, n_layers, weight_bits;
  unsigned flags;
  double eps_l2, eps_rms, q_scale;
} dno_dims;

typedef struct {
  const void *w_in;      /* int8 [R][D] or packed 4-bit [R][D/2] */
  const float *s_in;     /* [R] */
  const float *conv_w;   /* [C][K], tap K-1 multiplies the current token */
  const float *norm_w;   /* [dv] */
  const void *w_out;     /* int8 [D][V] or packed 4-bit [D][V/2] */
  const float *s_out;    /* [D] */
  const float *a_log;    /* [Hv] (DNO_GATES_ON_DEVICE) */
  const float *a_bias;   /* [Hv] (DNO_GATES_ON_DEVICE) */
} dno_layer_weights;

/* SiLU(a) = a * sigmoid(a) = a / (1 + e^-a). */
double dno_silu(double a) { return a / (1.0 + exp(-a)); }

/* One weight W[r][c] of a row-major matrix with `cols` columns.
 * 8-bit: signed bytes. 4-bit: two per byte, element 2m in the low nibble and
 * 2m+1 in the high nibble, each a 4-bit two's complement value. */
int dno_weight(const void *W, int bits, long cols, long r, long c) {
  if (bits == 8) return (int)((const int8_t *)W)[r * cols + c];
  uint8_t byte = ((const uint8_t *)W)[r * (cols / 2) + c / 2];
  int nib = (c & 1) ? (byte >> 4) : (byte & 15);
  return nib >= 8 ? nib - 16 : nib;
}

/* Per-row-scaled GEMV [TRUNK], [DN-GPU]: y[r] = s[r] * sum_c W[r][c] * x[c].
 * The scale multiplies the finished sum (one fp32 scale per row). */
void dno_gemv(int rows, int cols, const void *W, int bits, const float *s, const double *x, double *y) {
#pragma omp parallel for schedule(static)
  for (int r = 0; r < rows; ++r) {
    double acc = 0.0;
    if (bits == 8) {
      const int8_t *row = (const int8_t *)W + (long)r * cols;
      for (int c = 0; c < cols; ++c) acc += (double)row[c] * x[c];
    } else {
      const uint8_t *row = (const uint8_t *)W + (long)r * (cols / 2);
      for (int m = 0; m < cols / 2; ++m) {
        /* a nibble n is the 4-bit two's complement value (n ^ 8) - 8 */
        const int lo = row[m] & 15, hi = row[m] >> 4;
        acc += (double)((lo ^ 8) - 8) * x[2 * m];
        acc += (double)((hi ^ 8) - 8) * x[2 * m + 1];
      }
    }
    y[r] = (double)s[r] * acc;
  }
}

/* Parameter-free RMS normalisation of a layer input: y = x / sqrt(mean(x^2) + eps).
 * Reading: the pages chain layer outputs directly; without a pre-norm the chain of
 * thirty layers leaves the fp32 range, so stacks normalise each input this way. */
void dno_rms_prenorm(int n, const double *x, double eps, double *y) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += x[i] * x[i];
  double inv = 1.0 / sqrt(ss / n + eps);
  for (int i = 0; i < n; ++i) y[i] = x[i] * inv;
}

/* Depthwise causal conv + SiLU with the history advancing [DN-GPU]
 * ("causal conv + SiLU with the ring advancing").
 * hist is [K-1][C], oldest token first: hist[j] holds u_{t-(K-1)+j}.
 *   a[c] = sum_{j<K-1} w[c][j] * hist[j][c] + w[c][K-1] * u_t[c];  out[c] = silu(a[c]).
 * Then the history drops its oldest row and appends u_t. No bias (none is named). */
void dno_conv_silu(int C, int K, const float *w, double *hist, const double *u, double *out) {
  for (int c = 0; c < C; ++c) {
    double a = (double)w[(long)c * K + (K - 1)] * u[c];
    for (int j = 0; j < K - 1; ++j) a += (double)w[(long)c * K + j] * hist[(long)j * C + c];
    out[c] = dno_silu(a);
  }
  for (int j = 0; j + 1 < K - 1; ++j) memcpy(hist + (long)j * C, hist + (long)(j + 1) * C, sizeof(double) * C);
  if (K > 1) memcpy(hist + (long)(K - 2) * C, u, sizeof(double) * C);
}

/* L2 normalisation with eps inside the square root [DN-GPU]: out = v / sqrt(sum v^2 + eps). */
void dno_l2norm(int n, const double *v, double eps, double *out) {
  double ss = 0.0;
  for (int i = 0; i < n; ++i) ss += v[i] * v[i];
  double inv = 1.0 / sqrt(ss + eps);
  for (int i = 0; i < n; ++i) out[i] = v[i] * inv;
}

/* One value head's recurrence [DN-GPU]: the decay, the delta against the decayed
 * state, the write-back, then out = q^T S over the updated state.
 *   S'      = alpha * S
 *   kv[j]   = sum_i S'[i][j] * k[i]
 *   d[j]    = beta * (v[j] - kv[j])
 *   S''[i][j] = S'[i][j] + k[i] * d[j]
 *   o[j]    = q_scale * sum_i S''[i][j] * q[i]
 * S is [dk][dv], row i = key dimension, column j = value dimension. */
void dno_delta_head(int dk, int dv, double *S, const double *k, const double *v, const double *q,
                    double alpha, double beta, double q_scale, double *o) {
  for (long e = 0; e < (long)dk * dv; ++e) S[e] *= alpha;
  double *d = (double *)malloc(sizeof(double) * dv);
  for (int j = 0; j < dv; ++j) {
    double kv = 0.0;
    for (int i = 0; i < dk; ++i) kv += S[(long)i * dv + j] * k[i];
    d[j] = beta * (v[j] - kv);
  }
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += k[i] * d[j];
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * q[i];
    o[j] = q_scale * acc;
  }
  free(d);
}

/* The same recurrence with a decay per key channel, the form the linear-attention layers of the
 * other engines use ([DN-GPU], "Where this goes next": the same gated delta step, only the
 * dimensions and the gate differ). alpha[i] scales key row i of the state:
 *   S'[i][j] = alpha[i] * S[i][j]
 * and the delta, write-back and readout follow as in dno_delta_head. */
void dno_delta_head_vec(int dk, int dv, double *S, const double *k, const double *v, const double *q,
                        const double *alpha, double beta, double q_scale, double *o) {
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(long)i * dv + j] *= alpha[i];
  double *d = (double *)malloc(sizeof(double) * dv);
  for (int j = 0; j < dv; ++j) {
    double kv = 0.0;
    for (int i = 0; i < dk; ++i) kv += S[(long)i * dv + j] * k[i];
    d[j] = beta * (v[j] - kv);
  }
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(long)i * dv + j] += k[i] * d[j];
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * q[i];
    o[j] = q_scale * acc;
  }
  free(d);
}

/* softplus(y) = log(1 + e^y), written as max(y, 0) + log1p(e^-|y|) so that it neither overflows
 * nor loses the small values. */
double dno_softplus(double y) { return (y > 0.0 ? y : 0.0) + log1p(exp(-fabs(y))); }

/* The two gates of a value head from its two gate rows a, b of the in_proj output.
 * [DN-GPU] names the gates (a/b, one output per value head each) but leaves them to the engine
 * and gives no formula. Reading, stated: the decay form of gated-delta-rule layers,
 *   alpha = exp(-exp(a_log) * softplus(a + a_bias)),   beta = 1 / (1 + e^-b),
 * with a_log and a_bias per value head. alpha is in (0, 1], beta in (0, 1). */
void dno_gates(double a, double b, double a_log, double a_bias, double *alpha, double *beta) {
  *alpha = exp(-exp(a_log) * dno_softplus(a + a_bias));
  *beta = 1.0 / (1.0 + exp(-b));
}

/* Gated RMSNorm with silu(z) [DN-GPU], per value head over dv:
 *   y[j] = w[j] * o[j] / sqrt(mean(o^2) + eps) * silu(z[j]). */
void dno_gated_rmsnorm(int n, const double *o, const double *z, const float *w, double eps, double *y) {
  double ss = 0.0;
  for (int j = 0; j < n; ++j) ss += o[j] * o[j];
  double inv = 1.0 / sqrt(ss / n + eps);
  for (int j = 0; j < n; ++j) y[j] = (double)w[j] * o[j] * inv * dno_silu(z[j]);
}

/* One decode token of one layer for every sequence of the batch [DN-GPU] in the
 * page's order: in_proj GEMV, conv + SiLU, per value head L2 norms, decay, delta,
 * write-back, readout, gated RMSNorm, out_proj GEMV.
 * in_proj rows: q (Hk*dk) | k (Hk*dk) | v (Hv*dv) | z (Hv*dv) [TRUNK]; q, k, v are
 * convolved, z is not. Value head h reads key head h / (Hv/Hk).
 * With DNO_GATES_ON_DEVICE the in_proj has two more blocks, a (Hv) | b (Hv), not convolved, and
 * head h's gates come from a[h], b[h] through dno_gates; alpha and beta are then not read.
 *   S    [B][Hv][dk][dv]  (in/out)     hist [B][K-1][C] (in/out)
 *   x    [B][D]  alpha, beta [B][Hv]   out  [B][D]
 *   (with DNO_ALPHA_PER_KEY, alpha is [B][Hv][dk])                               */
int dno_layer_step(const dno_dims *d, const dno_layer_weights *W, double *S, double *hist,
                   const double *x, const float *alpha, const float *beta, double *out) {
  const int D = d->d_model, Hk = d->n_k_heads, dk = d->d_k, Hv = d->n_v_heads, dv = d->d_v;
  const int K = d->conv_k, B = d->batch;
  if (D <= 0 || Hk <= 0 || dk <= 0 || Hv <= 0 || dv <= 0 || K <= 0 || B <= 0 || Hv % Hk) return -1;
  const int gates = (d->flags & DNO_GATES_ON_DEVICE) != 0;
  if (gates && ((d->flags & DNO_ALPHA_PER_KEY) || !W->a_log || !W->a_bias)) return -1;
  const int QK = Hk * dk, V = Hv * dv, C = 2 * QK + V, R = C + V + (gates ? 2 * Hv : 0);
  double *xin = (double *)malloc(sizeof(double) * D);
  double *u = (double *)malloc(sizeof(double) * R);
  double *c = (double *)malloc(sizeof(double) * C);
  double *y = (double *)malloc(sizeof(double) * V);
  for (int b = 0; b < B; ++b) {
    if (d->flags & DNO_X_RMSNORM) dno_rms_prenorm(D, x + (long)b * D, d->eps_rms, xin);
    else memcpy(xin, x + (long)b * D, sizeof(double) * D);
    dno_gemv(R, D, W->w_in, d->weight_bits, W->s_in, xin, u);
    dno_conv_silu(C, K, W->conv_w, hist + (long)b * (K - 1) * C, u, c);
    const double *z = u + C;
    const int group = Hv / Hk;
#pragma omp parallel for schedule(static)
    for (int h = 0; h < Hv; ++h) {
      const int g = h / group;
      double *qh = (double *)malloc(sizeof(double) * dk);
      double *kh = (double *)malloc(sizeof(double) * dk);
      double *o = (double *)malloc(sizeof(double) * dv);
      dno_l2norm(dk, c + (long)g * dk, d->eps_l2, qh);
      dno_l2norm(dk, c + QK + (long)g * dk, d->eps_l2, kh);
      const double *v = c + 2 * QK + (long)h * dv;
      double *Sh = S + ((long)b * Hv + h) * dk * dv;
      if (gates) {
        double ga, gb;
        dno_gates(u[C + V + h], u[C + V + Hv + h], (double)W->a_log[h], (double)W->a_bias[h], &ga, &gb);
        dno_delta_head(dk, dv, Sh, kh, v, qh, ga, gb, d->q_scale, o);
      } else if (d->flags & DNO_ALPHA_PER_KEY) {
        double *av = (double *)malloc(sizeof(double) * dk);
        for (int i = 0; i < dk; ++i) av[i] = (double)alpha[((long)b * Hv + h) * dk + i];
        dno_delta_head_vec(dk, dv, Sh, kh, v, qh, av, (double)beta[(long)b * Hv + h], d->q_scale, o);
        free(av);
      } else {
        dno_delta_head(dk, dv, Sh, kh, v, qh, (double)alpha[(long)b * Hv + h], (double)beta[(long)b * Hv + h],
                       d->q_scale, o);
      }
      dno_gated_rmsnorm(dv, o, z + (long)h * dv, W->norm_w, d->eps_rms, y + (long)h * dv);
      free(qh); free(kh); free(o);
    }
    dno_gemv(D, V, W->w_out, d->weight_bits, W->s_out, y, out + (long)b * D);
  }
  free(xin); free(u); free(c); free(y);
  return 0;
}

/* A run of T tokens through a stack of L layers: the output of layer l is the
 * input of layer l+1; x feeds layer 0.
 *   S    [L][B][Hv][dk][dv]   hist [L][B][K-1][C]   (in/out, double)
 *   x    [T][B][D] fp32       alpha, beta [T][L][B][Hv] fp32 (alpha [T][L][B][Hv][dk] per key)
 *   out  [T][L][B][D] double (every layer's output, so a stack can be checked per layer) */
int dno_run(const dno_dims *d, const dno_layer_weights *W, double *S, double *hist, int T,
            const float *x, const float *alpha, const float *beta, double *out) {
  const int D = d->d_model, Hv = d->n_v_heads, B = d->batch, L = d->n_layers, K = d->conv_k;
  const long C = 2L * d->n_k_heads * d->d_k + (long)Hv * d->d_v;
  const long s_stride = (long)B * Hv * d->d_k * d->d_v, h_stride = (long)B * (K - 1) * C;
  double *xin = (double *)malloc(sizeof(double) * B * D);
  for (int t = 0; t < T; ++t) {
    for (long i = 0; i < (long)B * D; ++i) xin[i] = (double)x[(long)t * B * D + i];
    for (int l = 0; l < L; ++l) {
      double *o = out + ((long)t * L + l) * B * D;
      const long ab = ((long)t * L + l) * B * Hv;
      const long aa = (d->flags & DNO_ALPHA_PER_KEY) ? ab * d->d_k : ab;
      int rc = dno_layer_step(d, W + l, S + l * s_stride, hist + l * h_stride, xin, alpha + aa, beta + ab, o);
      if (rc) { free(xin); return rc; }
      memcpy(xin, o, sizeof(double) * B * D);
    }
  }
  free(xin);
  return 0;
}

/* Threads OpenMP would use (the baseline records it). */
#ifdef _OPENMP
#include <omp.h>
int dno_threads(void) { return omp_get_max_threads(); }
#else
int dno_threads(void) { return 1; }
#endif
