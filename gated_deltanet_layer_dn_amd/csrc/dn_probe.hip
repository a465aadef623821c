// Measurement only (libdn_probe): the read-stream and read-modify-write ceilings of this device's
// HBM, the figures the decode steps' achieved bandwidth is set against next to the vendor peak. Not
// part of the decode path and not linked into libdn.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dn_probe.h"

#define DN_API extern "C" __attribute__((visibility("default")))

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int PROBE_THREADS = 256;

// Every thread streams 16-byte pieces with PROBE_UNROLL nontemporal loads in flight, grid-stride,
// and folds them into one word, which the block writes so the loads are not dropped.
template <int PROBE_UNROLL>
__global__ __launch_bounds__(PROBE_THREADS) void k_read_stream(const v4u* __restrict__ p, size_t n16,
                                                               unsigned* __restrict__ sink) {
  const size_t step = (size_t)gridDim.x * PROBE_THREADS;
  unsigned acc = 0;
  size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
  for (; i + (PROBE_UNROLL - 1) * step < n16; i += PROBE_UNROLL * step) {
    v4u v[PROBE_UNROLL];
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * step);
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += step) {
    const v4u v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  __shared__ unsigned red[PROBE_THREADS];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned a = 0;
    for (int t = 0; t < PROBE_THREADS; ++t) a ^= red[t];
    sink[blockIdx.x] = a;
  }
}

// In place: every thread reads PROBE_UNROLL nontemporal 16-byte pieces, grid-stride, and writes
// each back (scaled by one, so the values stay) with nontemporal stores.
template <int PROBE_UNROLL>
__global__ __launch_bounds__(PROBE_THREADS) void k_rmw_stream(v4u* __restrict__ p, size_t n16, float one) {
  const size_t step = (size_t)gridDim.x * PROBE_THREADS;
  size_t i = (size_t)blockIdx.x * PROBE_THREADS + threadIdx.x;
  typedef float v4f __attribute__((ext_vector_type(4)));
  for (; i + (PROBE_UNROLL - 1) * step < n16; i += PROBE_UNROLL * step) {
    v4f v[PROBE_UNROLL];
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) v[u] = __builtin_bit_cast(v4f, __builtin_nontemporal_load(p + i + u * step));
#pragma unroll
    for (int u = 0; u < PROBE_UNROLL; ++u) __builtin_nontemporal_store(__builtin_bit_cast(v4u, v[u] * one), p + i + u * step);
  }
  for (; i < n16; i += step) {
    const v4f v = __builtin_bit_cast(v4f, __builtin_nontemporal_load(p + i));
    __builtin_nontemporal_store(__builtin_bit_cast(v4u, v * one), p + i);
  }
}

}  // namespace

DN_API int dn_probe_rmw_stream(void* buf, size_t bytes, int blocks, int in_flight, void* hip_stream) {
  if (!buf || blocks < 1 || blocks > DN_PROBE_MAX_BLOCKS || (bytes & 15u) || (reinterpret_cast<uintptr_t>(buf) & 15u))
    return -1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  v4u* p = static_cast<v4u*>(buf);
  if (in_flight == 4) hipLaunchKernelGGL(k_rmw_stream<4>, dim3(blocks), dim3(PROBE_THREADS), 0, st, p, bytes / 16, 1.0f);
  else if (in_flight == 8) hipLaunchKernelGGL(k_rmw_stream<8>, dim3(blocks), dim3(PROBE_THREADS), 0, st, p, bytes / 16, 1.0f);
  else if (in_flight == 16) hipLaunchKernelGGL(k_rmw_stream<16>, dim3(blocks), dim3(PROBE_THREADS), 0, st, p, bytes / 16, 1.0f);
  else return -1;
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

DN_API int dn_probe_read_stream(const void* buf, size_t bytes, unsigned* sink, int blocks, int in_flight,
                                void* hip_stream) {
  if (!buf || !sink || blocks < 1 || blocks > DN_PROBE_MAX_BLOCKS || (bytes & 15u) ||
      (reinterpret_cast<uintptr_t>(buf) & 15u))
    return -1;
  const hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  const v4u* p = static_cast<const v4u*>(buf);
  if (in_flight == 4) hipLaunchKernelGGL(k_read_stream<4>, dim3(blocks), dim3(PROBE_THREADS), 0, st, p, bytes / 16, sink);
  else if (in_flight == 8) hipLaunchKernelGGL(k_read_stream<8>, dim3(blocks), dim3(PROBE_THREADS), 0, st, p, bytes / 16, sink);
  else if (in_flight == 16) hipLaunchKernelGGL(k_read_stream<16>, dim3(blocks), dim3(PROBE_THREADS), 0, st, p, bytes / 16, sink);
  else return -1;
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
