/*
 * dn_residency.h -- host residency of a handle's recurrent state, as a thin layer over the
 * calls of dn.h (header only: it adds no symbol to the library).
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
 *   dnr_pull            before reading the host arrays (host step, snapshot, prompt on the host)
 *   dnr_host_written    after writing the host arrays (host step, reset, restore); requires
 *                       that nothing was ahead, i.e. dnr_pull came first
 *   dnr_step            one device step: uploads if the device copy is not fresh, enqueues
 *                       dn_step, marks the device ahead. On a failed step it pulls what the
 *                       device holds (dn_get_state works after a failure) and returns the error,
 *                       and the engine continues on the host from those arrays.
 *   dnr_prefill         the same for dn_prefill
 * All return the dn.h return codes; DN_E_INVAL if the flags forbid the call (dnr_host_written
 * while the device is ahead). Single-threaded use per dn_resident.
 */
#ifndef DN_RESIDENCY_H
#define DN_RESIDENCY_H

#include "dn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  dn_layer *h;
  float *S;     /* host state, canonical */
  float *ring;  /* host conv history, canonical (NULL: not moved) */
  int fresh;    /* device copy equals the host arrays */
  int ahead;    /* device copy is newer than the host arrays */
  long pulls, pushes;  /* transfers so far (for the engine's accounting) */
} dn_resident;

static inline int dnr_init(dn_resident *r, dn_layer *h, float *S, float *ring) {
  if (!r || !h || !S) return DN_E_INVAL;
  r->h = h;
  r->S = S;
  r->ring = ring;
  r->fresh = 0;
  r->ahead = 0;
  r->pulls = r->pushes = 0;
  return DN_OK;
}

/* Download if the device is ahead. The device copy stays valid (fresh) afterwards. */
static inline int dnr_pull(dn_resident *r) {
  if (!r || !r->h) return DN_E_INVAL;
  if (!r->ahead) return DN_OK;
  int rc = dn_get_state(r->h, r->S, r->ring);
  if (rc != DN_OK) return rc;
  r->ahead = 0;
  r->fresh = 1;
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
  ++r->pushes;
  return DN_OK;
}

/* The engine wrote the host arrays: the device copy is stale. */
static inline int dnr_host_written(dn_resident *r) {
  if (!r || !r->h || r->ahead) return DN_E_INVAL;
  r->fresh = 0;
  return DN_OK;
}

/* After a failed device call: take what the device holds, and mark the device copy stale so
 * that the next device call uploads (and re-arms the handle). */
static inline int dnr_recover_(dn_resident *r, int rc_fail) {
  r->ahead = 1;
  if (dnr_pull(r) == DN_OK) r->fresh = 0;
  return rc_fail;
}

static inline int dnr_step(dn_resident *r, const float *x, const float *alpha, const float *beta, float *out,
                           void *hip_stream) {
  int rc = dnr_push(r);
  if (rc != DN_OK) return rc;
  rc = dn_step(r->h, x, alpha, beta, out, hip_stream);
  if (rc == DN_OK) {
    r->ahead = 1;
    return DN_OK;
  }
  if (rc == DN_E_INVAL) return rc; /* nothing was launched: the flags stand */
  return dnr_recover_(r, rc);
}

static inline int dnr_prefill(dn_resident *r, const float *x, int n_tokens, const float *alpha, const float *beta,
                              float *out, void *hip_stream) {
  int rc = dnr_push(r);
  if (rc != DN_OK) return rc;
  rc = dn_prefill(r->h, x, n_tokens, alpha, beta, out, hip_stream);
  if (rc == DN_OK) {
    r->ahead = 1;
    return DN_OK;
  }
  if (rc == DN_E_INVAL || rc == DN_E_NOMEM) return rc; /* nothing was launched */
  return dnr_recover_(r, rc);
}

#ifdef __cplusplus
}
#endif
#endif /* DN_RESIDENCY_H */
