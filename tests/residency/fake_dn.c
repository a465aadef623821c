/* A host-only stand-in for the dn.h calls that dn_residency.h uses (test infrastructure): the
 * "device" state lives in host memory, a step adds the step count to every element, and a step
 * can be told to fail after updating half of the state, as a failing device step can leave the
 * card partly advanced. */
#include <string.h>

#include "dn.h"

#define FAKE_N 64
#define FAKE_M 16

struct dn_layer {
  float S[FAKE_N], ring[FAKE_M];
  int disabled;
  long steps, fail_at;
  long sets, gets;
};

static struct dn_layer fake_handle;

dn_layer *fake_create(long fail_at) {
  memset(&fake_handle, 0, sizeof(fake_handle));
  fake_handle.fail_at = fail_at;
  return &fake_handle;
}
long fake_sets(void) { return fake_handle.sets; }
long fake_gets(void) { return fake_handle.gets; }
const float *fake_device_S(void) { return fake_handle.S; }
void fake_fail_at(long n) { fake_handle.fail_at = n; }

int dn_set_state(dn_layer *h, const float *S, const float *ring) {
  if (!h || !S) return DN_E_INVAL;
  memcpy(h->S, S, sizeof(h->S));
  if (ring) memcpy(h->ring, ring, sizeof(h->ring));
  h->disabled = 0;
  ++h->sets;
  return DN_OK;
}

int dn_get_state(dn_layer *h, float *S, float *ring) {
  if (!h || !S) return DN_E_INVAL;
  memcpy(S, h->S, sizeof(h->S));
  if (ring) memcpy(ring, h->ring, sizeof(h->ring));
  ++h->gets;
  return DN_OK;
}

static int advance(dn_layer *h, float by) {
  if (h->disabled) return DN_E_DISABLED;
  ++h->steps;
  const int fail = h->fail_at > 0 && h->steps == h->fail_at;
  for (int i = 0; i < (fail ? FAKE_N / 2 : FAKE_N); ++i) h->S[i] += by;
  for (int i = 0; i < FAKE_M; ++i) h->ring[i] = by;
  if (fail) {
    h->disabled = 1;
    return DN_E_DEVICE;
  }
  return DN_OK;
}

int dn_step(dn_layer *h, const float *x, const float *alpha, const float *beta, float *out, void *stream) {
  (void)alpha; (void)beta; (void)stream;
  if (!h || !x || !out) return DN_E_INVAL;
  return advance(h, 1.0f);
}

int dn_prefill(dn_layer *h, const float *x, int n_tokens, const float *alpha, const float *beta, float *out,
               void *stream) {
  (void)alpha; (void)beta; (void)stream;
  if (!h || !x || !out || n_tokens < 1) return DN_E_INVAL;
  return advance(h, (float)n_tokens);
}
