/* A host-only stand-in for the dn.h / dn_prefill.h calls that dn_residency.h uses (test
 * infrastructure). The "device" state lives in host memory and a step adds the step's size to every
 * element. A step can be told to fail in one of two ways, as a step of libdn can:
 *   at once  the call returns DN_E_DEVICE and nothing of the token is done (an injected failure,
 *            a launch error);
 *   late     the call returns DN_OK, the token is abandoned on the "device" (the state keeps its
 *            value from before the token, as libdn's whole-stack kernel keeps it), and the failure
 *            is reported by the next call: dn_step, or dn_get_state(h, NULL, NULL).
 * The handle latches off after a failure until dn_set_state re-arms it. */
#include <string.h>

#include "dn.h"
#include "dn_prefill.h"

#define FAKE_N 64
#define FAKE_M 16

struct dn_layer {
  float S[FAKE_N], ring[FAKE_M];
  int disabled;
  int late_err;  /* a step was abandoned: reported by the next call, and later steps do nothing */
  long steps, fail_at, fail_late_at;
  long sets, gets, checks;
};

static struct dn_layer fake_handle;

dn_layer *fake_create(long fail_at) {
  memset(&fake_handle, 0, sizeof(fake_handle));
  fake_handle.fail_at = fail_at;
  return &fake_handle;
}
long fake_sets(void) { return fake_handle.sets; }
long fake_gets(void) { return fake_handle.gets; }
long fake_checks(void) { return fake_handle.checks; }
const float *fake_device_S(void) { return fake_handle.S; }
void fake_fail_at(long n) { fake_handle.fail_at = n; }
void fake_fail_late_at(long n) { fake_handle.fail_late_at = n; }

int dn_set_state(dn_layer *h, const float *S, const float *ring) {
  if (!h || !S) return DN_E_INVAL;
  memcpy(h->S, S, sizeof(h->S));
  if (ring) memcpy(h->ring, ring, sizeof(h->ring));
  h->disabled = 0;
  h->late_err = 0;
  ++h->sets;
  return DN_OK;
}

int dn_get_state(dn_layer *h, float *S, float *ring) {
  if (!h || (!S && ring)) return DN_E_INVAL;
  if (!S) {
    ++h->checks;
    if (h->late_err) {
      h->disabled = 1;
      return DN_E_DEVICE;
    }
    return DN_OK;
  }
  memcpy(S, h->S, sizeof(h->S));
  if (ring) memcpy(ring, h->ring, sizeof(h->ring));
  ++h->gets;
  return DN_OK;
}

static int advance(dn_layer *h, float by) {
  if (h->late_err) {
    h->disabled = 1;
    return DN_E_DEVICE;
  }
  if (h->disabled) return DN_E_DISABLED;
  ++h->steps;
  if (h->fail_at > 0 && h->steps == h->fail_at) {
    h->disabled = 1;
    return DN_E_DEVICE;
  }
  if (h->fail_late_at > 0 && h->steps == h->fail_late_at) {
    h->late_err = 1;
    return DN_OK;
  }
  for (int i = 0; i < FAKE_N; ++i) h->S[i] += by;
  for (int i = 0; i < FAKE_M; ++i) h->ring[i] = by;
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
