/* Drives dn_residency.h through the engine's cases against the fake calls of fake_dn.c and
 * checks the flags, the transfers and the host arrays after each (test infrastructure). */
#include <stdio.h>
#include <stdlib.h>

#include "dn_residency.h"

dn_layer *fake_create(long fail_at);
long fake_sets(void);
long fake_gets(void);
const float *fake_device_S(void);
void fake_fail_at(long n);

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

int main(void) {
  float S[N], ring[M], x[4] = {0}, out[4];
  for (int i = 0; i < N; ++i) S[i] = 10.0f;
  for (int i = 0; i < M; ++i) ring[i] = 0.0f;
  dn_resident r;
  dn_layer *h = fake_create(0);
  CHECK(dnr_init(&r, h, S, ring) == DN_OK && !r.fresh && !r.ahead);

  /* the first device step uploads the canonical host arrays */
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK);
  CHECK(fake_sets() == 1 && r.fresh && r.ahead && all_equal(fake_device_S(), 11.0f, N));
  /* a fresh device copy is not uploaded again; the host arrays lag behind */
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK);
  CHECK(fake_sets() == 1 && all_equal(S, 10.0f, N) && all_equal(fake_device_S(), 12.0f, N));
  /* host use pulls once */
  CHECK(dnr_pull(&r) == DN_OK && fake_gets() == 1 && all_equal(S, 12.0f, N) && !r.ahead && r.fresh);
  CHECK(dnr_pull(&r) == DN_OK && fake_gets() == 1);
  /* a host step writes the arrays: the next device step uploads them */
  for (int i = 0; i < N; ++i) S[i] += 1.0f;
  CHECK(dnr_host_written(&r) == DN_OK && !r.fresh);
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK);
  CHECK(fake_sets() == 2 && all_equal(fake_device_S(), 14.0f, N));
  /* writing the host arrays while the device is ahead is refused (the engine must pull first) */
  CHECK(dnr_host_written(&r) == DN_E_INVAL && r.ahead);
  /* a reset of the host arrays after pulling */
  CHECK(dnr_pull(&r) == DN_OK && all_equal(S, 14.0f, N));
  for (int i = 0; i < N; ++i) S[i] = 0.0f;
  CHECK(dnr_host_written(&r) == DN_OK);
  /* a prompt on the device: uploads the reset state, then runs */
  CHECK(dnr_prefill(&r, x, 5, NULL, NULL, out, NULL) == DN_OK);
  CHECK(fake_sets() == 3 && all_equal(fake_device_S(), 5.0f, N) && r.ahead);
  /* a failing device step: the host takes what the device holds (half advanced) and continues */
  fake_fail_at(5);
  const long gets0 = fake_gets();
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_E_DEVICE);
  CHECK(fake_gets() == gets0 + 1 && !r.ahead && !r.fresh);
  CHECK(all_equal(S, 6.0f, N / 2) && all_equal(S + N / 2, 5.0f, N / 2));
  /* the engine's host step, then the device again: the upload re-arms the handle */
  for (int i = 0; i < N; ++i) S[i] = 7.0f;
  CHECK(dnr_host_written(&r) == DN_OK);
  CHECK(dnr_step(&r, x, NULL, NULL, out, NULL) == DN_OK && all_equal(fake_device_S(), 8.0f, N));
  /* an invalid call launches nothing and keeps the flags */
  CHECK(dnr_step(&r, NULL, NULL, NULL, out, NULL) == DN_E_INVAL && r.ahead && r.fresh);
  CHECK(r.pushes == 4 && r.pulls == 3 && fake_sets() == 4 && fake_gets() == 3);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("residency checks passed\n");
  return 0;
}
