/*
 * dn_residency.h -- host residency of a handle's recurrent state, as a thin layer over the
 * calls of dn.h and dn_prefill.h (header only: it adds no symbol to either library).
 *
 * The page "qwen36: run the DeltaNet layer end to end on the card (Q36_DN_GPU=1): conv,
 * recurrence and gated norm join the two projections", section "What the PR does", Engine
 * paragraph, keeps the engine's host arrays canonical and gives each layer two flags:
 *   fresh  the device copy matches the host arrays, so a device step needs no upload first;
 *   ahead  the device copy is newer than the host arrays, so any host use downloads first.
 * Around them: a prompt on the host pulls first; a snapshot pulls; a reset or a restore of the
 * host arrays makes the device copy stale; a failing device step pulls what the card holds and
 * the engine continues on the host.
 *
 * Here one dn_resident covers one handle (all of its layers). The engine owns the host arrays
 * S [L][B][Hv][dk][dv] and ring [L][B][K-1][C] (the layouts of dn_set_state; ring may be NULL
 * when conv_k == 1) and calls:
 *   dnr_init            after dn_create: neither flag is set, so the first device step uploads
 *   dnr_set_checked     checked mode on (1) or off (0, the default), see below
 *   dnr_pull            before reading the host arrays (host step, snapshot, prompt on the host)
 *   dnr_host_written    after writing the host arrays (host step, reset, restore); requires
 *                       that nothing was ahead, i.e. dnr_pull came first
 *   dnr_step            one device step: uploads if the device copy is not fresh, enqueues
 *                       dn_step, marks the device ahead. On a failed step it pulls what the
 *                       device holds (dn_get_state works after a failure) and returns the error,
 *                       and the engine continues on the host from those arrays.
 *   dnr_prefill         the same for dn_prefill
 *   dnr_check           wait for the device and verify every step so far (see below)
 *
 * Failures reported late. dn_step only enqueues. A failure found while the call runs (an
 * injected one, a launch error) is returned at once and nothing of that token was done. A
 * whole-stack launch that abandons its token on the device is reported by a later call; libdn
 * then keeps the state and history as they were before that token (the launch writes into a
 * second buffer that it makes current only when it completes), and every launch after it does
 * nothing. So after any failed call the host arrays hold the state after the last completed
 * device call, and `unverified` says which call that is:
 *   unverified == 0  every launched call completed: the arrays hold the state just before the
 *                    failed call, and the engine runs exactly that token on the host;
 *   unverified == k  one of the last k launched calls (counted since the last verification) was
 *                    abandoned: their outputs are not to be used, and the engine restores its own
 *                    snapshot to continue exactly.
 * In checked mode dnr_step verifies each step before it returns (one wait for the device per
 * token, as an engine that copies each token's output to the host waits anyway), so k is 0 or 1
 * and in both cases the arrays hold the state just before the failed call.
 * All return the dn.h return codes; DN_E_INVAL if the flags forbid the call (dnr_host_written
 * while the device is ahead). Single-threaded use per dn_resident.
 */
#ifndef DN_RESIDENCY_H
#define DN_RESIDENCY_H

#include <stddef.h>

#include "dn.h"
#include "dn_prefill.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  dn_layer *h;
  float *S;     /* host state, canonical */
  float *ring;  /* host conv history, canonical (NULL: not moved) */
  int fresh;    /* device copy equals the host arrays */
  int ahead;    /* device copy is newer than the host arrays */
  int checked;  /* verify every device step before dnr_step returns */
  long unverified;     /* device calls since the last verification (a check, a pull, an upload) */
  long pulls, pushes;  /* transfers so far (for the engine's accounting) */
} dn_resident;

static inline int dnr_init(dn_resident *r, dn_layer *h, float *S, float *ring) {
  if (!r || !h || !S) return DN_E_INVAL;
  r->h = h;
  r->S = S;
  r->ring = ring;
  r->fresh = 0;
  r->ahead = 0;
  r->checked = 0;
  r->unverified = 0;
  r->pulls = r->pushes = 0;
  return DN_OK;
}

static inline int dnr_set_checked(dn_resident *r, int on) {
  if (!r || !r->h) return DN_E_INVAL;
  r->checked = on != 0;
  return DN_OK;
}

/* Download if the device is ahead. The device copy stays valid (fresh) afterwards. The download
 * waits for the device, so a failure reported late shows here: DN_E_DEVICE, with the state after
 * the last completed call in the arrays and the device copy marked stale (see above). */
static inline int dnr_pull(dn_resident *r) {
  if (!r || !r->h) return DN_E_INVAL;
  if (!r->ahead) return DN_OK;
  if (r->unverified && dn_get_state(r->h, NULL, NULL) != DN_OK) {
    /* a failure reported late: take the state after the last completed call */
    int rc = dn_get_state(r->h, r->S, r->ring);
    if (rc == DN_OK) ++r->pulls;
    r->ahead = 0;
    r->fresh = 0;
    return DN_E_DEVICE;
  }
  int rc = dn_get_state(r->h, r->S, r->ring);
  if (rc != DN_OK) return rc;
  r->ahead = 0;
  r->fresh = 1;
  r->unverified = 0;
  ++r->pulls;
  return DN_OK;
}

/* Upload if the device copy is stale; dn_set_state also re-arms a handle latched by a failure. */
static inline int dnr_push(dn_resident *r) {
  if (!r || !r->h) return DN_E_INVAL;
  if (r->fresh) return DN_OK;
  int rc = dn_set_state(r->h, r->S, r->ring);
  if (rc != DN_OK) return rc;
  r->fresh = 1;
  r->ahead = 0;
  r->unverified = 0;
  ++r->pushes;
  return DN_OK;
}

/* The engine wrote the host arrays: the device copy is stale. */
static inline int dnr_host_written(dn_resident *r) {
  if (!r || !r->h || r->ahead) return DN_E_INVAL;
  r->fresh = 0;
  return DN_OK;
}

/* After a failed device call: take what the device holds (the state after the last completed
 * call) and mark the device copy stale, so that the next device call uploads (and re-arms the
 * handle). If every launched call completed, nothing is left unverified. */
static inline int dnr_recover_(dn_resident *r, int rc_fail) {
  if (dn_get_state(r->h, NULL, NULL) == DN_OK) r->unverified = 0;
  int rc = dn_get_state(r->h, r->S, r->ring);
  if (rc == DN_OK) ++r->pulls;
  r->ahead = 0;
  r->fresh = 0;
  return rc_fail;
}

/* Wait for the device and verify every device call since the last verification. On a failure the
 * host arrays receive the state after the last completed token (see above). */
static inline int dnr_check(dn_resident *r) {
  if (!r || !r->h) return DN_E_INVAL;
  if (!r->unverified) return DN_OK;
  int rc = dn_get_state(r->h, NULL, NULL);
  if (rc != DN_OK) return dnr_recover_(r, rc);
  r->unverified = 0;
  return DN_OK;
}

static inline int dnr_step(dn_resident *r, const float *x, const float *alpha, const float *beta, float *out,
                           void *hip_stream) {
  int rc = dnr_push(r);
  if (rc != DN_OK) return rc;
  rc = dn_step(r->h, x, alpha, beta, out, hip_stream);
  if (rc == DN_E_INVAL) return rc; /* nothing was launched: the flags stand */
  if (rc != DN_OK) return dnr_recover_(r, rc);
  r->ahead = 1;
  ++r->unverified;
  return r->checked ? dnr_check(r) : DN_OK;
}

static inline int dnr_prefill(dn_resident *r, const float *x, int n_tokens, const float *alpha, const float *beta,
                              float *out, void *hip_stream) {
  int rc = dnr_push(r);
  if (rc != DN_OK) return rc;
  rc = dn_prefill(r->h, x, n_tokens, alpha, beta, out, hip_stream);
  if (rc == DN_E_INVAL || rc == DN_E_NOMEM) return rc; /* nothing was launched */
  if (rc != DN_OK) return dnr_recover_(r, rc);
  r->ahead = 1;
  ++r->unverified;
  return r->checked ? dnr_check(r) : DN_OK;
}

#ifdef __cplusplus
}
#endif
#endif /* DN_RESIDENCY_H */
