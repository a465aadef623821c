/* An engine loop over dn_residency.h with the real libraries (test infrastructure, run by
 * tests/test_gpu_residency.py on the card). The engine keeps the canonical host arrays, runs most
 * tokens on the card through dnr_step, and runs a token on the host (the fp64 oracle's layer step,
 * as the engine's host path) where the protocol says so: after a failed device step, and once on
 * purpose (a host step after a pull). Inputs come from files the test writes; outputs, the final
 * state and a report go back to files.
 *
 * usage: gpu_engine DIR   (DIR holds dims.txt and the arrays; see tests/test_gpu_residency.py)
 * The failures come from libdn's environment: DN_FAULT_STEP (a dn_step that fails at once) and
 * DN_FAULT_STALL (a whole-stack launch that abandons its token on the device). */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dn_residency.h"

/* the oracle's C interface (oracle/dn_oracle.c) */
typedef struct {
  int d_model, n_k_heads, d_k, n_v_heads, d_v;
  int conv_k, batch, n_layers, weight_bits;
  unsigned flags;
  double eps_l2, eps_rms, q_scale;
} dno_dims;
typedef struct {
  const void *w_in;
  const float *s_in;
  const float *conv_w;
  const float *norm_w;
  const void *w_out;
  const float *s_out;
  const float *a_log;
  const float *a_bias;
} dno_layer_weights;
int dno_layer_step(const dno_dims *d, const dno_layer_weights *W, double *S, double *hist, const double *x,
                   const float *alpha, const float *beta, double *out);

static const char *dir;

static void *load(const char *name, size_t bytes) {
  char path[1024];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  FILE *f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "cannot open %s\n", path);
    exit(2);
  }
  void *p = malloc(bytes ? bytes : 1);
  if (fread(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "short read %s\n", path);
    exit(2);
  }
  fclose(f);
  return p;
}
static void save(const char *name, const void *p, size_t bytes) {
  char path[1024];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  FILE *f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) {
    fprintf(stderr, "cannot write %s\n", path);
    exit(2);
  }
  fclose(f);
}
static void *dev_copy(const void *h, size_t bytes) {
  void *d = NULL;
  if (hipMalloc(&d, bytes) != hipSuccess || hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    fprintf(stderr, "device copy failed\n");
    exit(2);
  }
  return d;
}

int main(int argc, char **argv) {
  if (argc != 2) return 2;
  dir = argv[1];
  int D, Hk, dk, Hv, dv, K, L, T, bits;
  unsigned flags;
  double eps_l2, eps_rms, q_scale;
  {
    char path[1024];
    snprintf(path, sizeof(path), "%s/dims.txt", dir);
    FILE *f = fopen(path, "r");
    if (!f || fscanf(f, "%d %d %d %d %d %d %d %d %d %u %lf %lf %lf", &D, &Hk, &dk, &Hv, &dv, &K, &L, &T, &bits, &flags,
                     &eps_l2, &eps_rms, &q_scale) != 13)
      return 2;
    fclose(f);
  }
  const int QK = Hk * dk, V = Hv * dv, C = 2 * QK + V, R = C + V;
  const size_t rowb_in = bits == 8 ? (size_t)D : (size_t)D / 2, rowb_out = bits == 8 ? (size_t)V : (size_t)V / 2;
  const size_t s_l = (size_t)Hv * dk * dv, h_l = (size_t)(K - 1) * C;

  dno_layer_weights *hw = calloc(L, sizeof(*hw));
  dn_weights *dw = calloc(L, sizeof(*dw));
  for (int l = 0; l < L; ++l) {
    char n[64];
#define LOADW(field, name, bytes)                     \
  snprintf(n, sizeof(n), name "_%d.bin", l);          \
  hw[l].field = load(n, bytes);                       \
  dw[l].field = dev_copy(hw[l].field, bytes);
    LOADW(w_in, "w_in", R * rowb_in)
    LOADW(s_in, "s_in", sizeof(float) * R)
    LOADW(conv_w, "conv_w", sizeof(float) * C * K)
    LOADW(norm_w, "norm_w", sizeof(float) * dv)
    LOADW(w_out, "w_out", D * rowb_out)
    LOADW(s_out, "s_out", sizeof(float) * D)
#undef LOADW
  }
  float *S = load("S0.bin", sizeof(float) * L * s_l);
  float *ring = load("ring0.bin", sizeof(float) * L * h_l);
  float *S0 = load("S0.bin", sizeof(float) * L * s_l);
  float *x = load("x.bin", sizeof(float) * T * D);
  float *al = load("alpha.bin", sizeof(float) * T * L * Hv);
  float *be = load("beta.bin", sizeof(float) * T * L * Hv);

  dn_config cfg = {D, Hk, dk, Hv, dv, K, 1, L, bits, flags, (float)eps_l2, (float)eps_rms, (float)q_scale};
  dn_layer *h = NULL;
  if (dn_create(&cfg, dw, &h) != DN_OK) return 3;
  float *dx = dev_copy(x, sizeof(float) * T * D);
  float *dal = dev_copy(al, sizeof(float) * T * L * Hv);
  float *dbe = dev_copy(be, sizeof(float) * T * L * Hv);
  float *dout = NULL;
  if (hipMalloc((void **)&dout, sizeof(float) * L * D) != hipSuccess) return 3;

  dn_resident r;
  if (dnr_init(&r, h, S, ring) != DN_OK || dnr_set_checked(&r, 1) != DN_OK) return 3;

  double *outs = calloc((size_t)T * L * D, sizeof(double));
  float *ob = malloc(sizeof(float) * L * D);
  double *Sd = malloc(sizeof(double) * s_l), *Hd = malloc(sizeof(double) * (h_l ? h_l : 1));
  double *xin = malloc(sizeof(double) * D), *xo = malloc(sizeof(double) * D);
  dno_dims od = {D, Hk, dk, Hv, dv, K, 1, 1, bits, flags, eps_l2, eps_rms, q_scale};
  char where[256] = {0};
  int rcs[256];
  int host_untouched = 1;
  const int host_on_purpose = 5;  /* the engine runs this token on the host after a pull */

  for (int t = 0; t < T && t < 256; ++t) {
    int on_host = 0;
    int rc = DN_OK;
    if (t == host_on_purpose) {
      rc = dnr_pull(&r);
      on_host = 1;
    } else {
      rc = dnr_step(&r, dx + (size_t)t * D, dal + (size_t)t * L * Hv, dbe + (size_t)t * L * Hv, dout, NULL);
      if (rc == DN_OK) {
        /* the engine takes the token's output to the host (every layer's, for the test) */
        if (hipMemcpy(ob, dout, sizeof(float) * L * D, hipMemcpyDeviceToHost) != hipSuccess) return 4;
        for (size_t i = 0; i < (size_t)L * D; ++i) outs[(size_t)t * L * D + i] = ob[i];
        if (t < 3 && memcmp(S, S0, sizeof(float) * L * s_l) != 0) host_untouched = 0;
      } else {
        on_host = 1; /* the failed token runs on the host from the arrays dnr recovered */
      }
    }
    rcs[t] = rc;
    where[t] = on_host ? 'h' : 'd';
    if (on_host) {
      for (int i = 0; i < D; ++i) xin[i] = x[(size_t)t * D + i];
      for (int l = 0; l < L; ++l) {
        for (size_t i = 0; i < s_l; ++i) Sd[i] = S[l * s_l + i];
        for (size_t i = 0; i < h_l; ++i) Hd[i] = ring[l * h_l + i];
        if (dno_layer_step(&od, &hw[l], Sd, Hd, xin, al + ((size_t)t * L + l) * Hv, be + ((size_t)t * L + l) * Hv, xo))
          return 5;
        for (size_t i = 0; i < s_l; ++i) S[l * s_l + i] = (float)Sd[i];
        for (size_t i = 0; i < h_l; ++i) ring[l * h_l + i] = (float)Hd[i];
        for (int i = 0; i < D; ++i) {
          outs[((size_t)t * L + l) * D + i] = xo[i];
          xin[i] = (float)xo[i]; /* the next layer's input, as the card would pass it (fp32) */
        }
      }
      if (dnr_host_written(&r) != DN_OK) return 6;
    }
  }
  const int final_pull = dnr_pull(&r);
  save("out.bin", outs, sizeof(double) * T * L * D);
  save("S_final.bin", S, sizeof(float) * L * s_l);
  save("ring_final.bin", ring, sizeof(float) * L * h_l);
  char path[1024];
  snprintf(path, sizeof(path), "%s/report.txt", dir);
  FILE *f = fopen(path, "w");
  fprintf(f, "where %s\nrcs", where);
  for (int t = 0; t < T; ++t) fprintf(f, " %d", rcs[t]);
  fprintf(f, "\npulls %ld\npushes %ld\nhost_untouched %d\nfinal_pull %d\n", r.pulls, r.pushes, host_untouched,
          final_pull);
  fclose(f);
  dn_destroy(h);
  printf("engine done\n");
  return 0;
}
