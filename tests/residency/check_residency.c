/* Drives dn_residency.h through the engine's cases against the fake calls of fake_dn.c and
 * checks the flags, the transfers and the host arrays after each (test infrastructure). */
#include <stdio.h>
#include <stdlib.h>

#include "dn_residency.h"

dn_layer *fake_create(long fail_at);
long fake_sets(void);
long fake_gets(void);
long fake_checks(void);
const float *fake_device_S(void);
void fake_fail_at(long n);
void fake_fail_late_at(long n);

#define N 64
#define M 16
static int failures = 0;
#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static int all_equal(const float *a, float v, int n) {
  for (int i = 0; i < n; ++i)
    if (a[i] != v) return 0;
  return 1;
}
static void host_set(float *S, float v) {
  for (int i = 0; i < N; ++i) S[i] = v;
}

int main(void) {
  float S[N], ring[M], x[4] = {0}, out[4];
  host_set(S, 10.0f);
  for (int i = 0; i < M; ++i) ring[i] = 0.0f;
  dn_resident r;
  dn_layer *h = fake_create(0);
  CHECK(dnr_init(&r, h, S, ring) == DN_OK && !r.fresh && !r.ahead && !r.checked && r.unverified == 0);

  /* the first device step uploads the canonical host arrays */
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK);
  CHECK(fake_sets() == 1 && r.fresh && r.ahead && r.unverified == 1 && all_equal(fake_device_S(), 11.0f, N));
  /* a fresh device copy is not uploaded again; the host arrays lag behind */
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK);
  CHECK(fake_sets() == 1 && r.unverified == 2 && all_equal(S, 10.0f, N) && all_equal(fake_device_S(), 12.0f, N));
  /* host use pulls once, after verifying the unverified steps */
  CHECK(dnr_pull(&r) == DN_OK && fake_gets() == 1 && fake_checks() == 1);
  CHECK(all_equal(S, 12.0f, N) && !r.ahead && r.fresh && r.unverified == 0);
  CHECK(dnr_pull(&r) == DN_OK && fake_gets() == 1);
  /* a host step writes the arrays: the next device step uploads them */
  host_set(S, 13.0f);
  CHECK(dnr_host_written(&r) == DN_OK && !r.fresh);
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK);
  CHECK(fake_sets() == 2 && all_equal(fake_device_S(), 14.0f, N));
  /* writing the host arrays while the device is ahead is refused (the engine must pull first) */
  CHECK(dnr_host_written(&r) == DN_E_INVAL && r.ahead);
  /* a reset of the host arrays after pulling */
  CHECK(dnr_pull(&r) == DN_OK && all_equal(S, 14.0f, N) && fake_gets() == 2);
  host_set(S, 0.0f);
  CHECK(dnr_host_written(&r) == DN_OK);
  /* a prompt on the device: uploads the reset state, then runs (steps so far: 4) */
  CHECK(dnr_prefill(&r, x, 5, NULL, NULL, out, NULL) == DN_OK);
  CHECK(fake_sets() == 3 && all_equal(fake_device_S(), 5.0f, N) && r.ahead);

  /* a device step that fails at once (step 5): nothing of the token was done; the host takes the
   * device's state, which is the state just before the token, and nothing is left unverified */
  fake_fail_at(5);
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_E_DEVICE);
  CHECK(fake_gets() == 3 && !r.ahead && !r.fresh && r.unverified == 0 && all_equal(S, 5.0f, N));
  /* the engine runs that token on the host, then the device again: the upload re-arms the handle */
  host_set(S, 6.0f);
  CHECK(dnr_host_written(&r) == DN_OK);
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK && fake_sets() == 4 && all_equal(fake_device_S(), 7.0f, N));

  /* a step abandoned on the device (step 7), unchecked: dn_step returns DN_OK, the next call reports
   * it; the host then holds the state after the last completed step, and the one unverified step
   * since the last verification is the abandoned one */
  CHECK(dnr_check(&r) == DN_OK && r.unverified == 0 && r.ahead);
  fake_fail_late_at(7);
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK && r.unverified == 1);
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_E_DEVICE);
  CHECK(fake_gets() == 4 && r.unverified == 1 && !r.ahead && !r.fresh && all_equal(S, 7.0f, N));
  host_set(S, 8.0f); /* the engine runs the abandoned token on the host */
  CHECK(dnr_host_written(&r) == DN_OK);
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK && fake_sets() == 5 && r.unverified == 1);
  CHECK(all_equal(fake_device_S(), 9.0f, N));

  /* checked mode: the step abandoned on the device (step 9) is reported by its own dnr_step, with
   * the state just before it in the host arrays */
  CHECK(dnr_set_checked(&r, 1) == DN_OK && r.checked);
  CHECK(dnr_check(&r) == DN_OK && r.unverified == 0); /* step 8, taken unchecked */
  fake_fail_late_at(9);
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_E_DEVICE);
  CHECK(fake_gets() == 5 && r.unverified == 1 && !r.ahead && !r.fresh && all_equal(S, 9.0f, N));
  host_set(S, 10.0f);
  CHECK(dnr_host_written(&r) == DN_OK);
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK && fake_sets() == 6 && r.unverified == 0 && r.ahead);
  CHECK(dnr_pull(&r) == DN_OK && all_equal(S, 11.0f, N) && fake_gets() == 6);

  /* unchecked again: a step abandoned on the device (step 11) is reported by the next pull */
  CHECK(dnr_set_checked(&r, 0) == DN_OK);
  fake_fail_late_at(11);
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK && r.ahead && r.unverified == 1);
  CHECK(dnr_pull(&r) == DN_E_DEVICE && !r.ahead && !r.fresh && all_equal(S, 11.0f, N) && fake_gets() == 7);
  CHECK(dnr_host_written(&r) == DN_OK);
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK && fake_sets() == 7 && all_equal(fake_device_S(), 12.0f, N));

  /* an invalid call launches nothing and keeps the flags */
  CHECK(dnr_step(&r, NULL, NULL, NULL, out, NULL) == DN_E_INVAL && r.ahead && r.fresh);
  CHECK(r.pushes == 7 && r.pulls == 7 && fake_sets() == 7 && fake_gets() == 7);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("residency checks passed\n");
  return 0;
}
