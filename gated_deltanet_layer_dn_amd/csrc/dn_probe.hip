// Measurement only (libdn_probe): the read-stream and read-modify-write ceilings of this device's
// HBM, the figures the decode steps' achieved bandwidth is set against next to the vendor peak, and
// the latency of a hand-off between workgroups, the figure that bounds the whole-stack kernel. Not
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


// ---------------------------------------------------------------------------------------------
// Hand-off latency between workgroups. 768 threads per workgroup: waves 0..3 measure, waves 4..11
// optionally stream nontemporal reads (the weight stream of the whole-stack kernel) until the
// measuring waves are done. Words are stored with relaxed agent-scope atomics and polled with
// device-coherent (sc1) loads, as the whole-stack kernel's hand-offs are; every wait is bounded
// (cap rounds, then *err is counted and the wave stops).
constexpr int XW_THREADS = 768;
constexpr int XW_SC1 = 16;  // cache policy of a device-coherent load

__device__ __forceinline__ int xw_xcd() { return (int)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | (3 << 11)) & 7); }
__device__ __forceinline__ __amdgpu_buffer_rsrc_t xw_rsrc(const void* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

struct XchgArgs {
  int mode, arg, rounds, sif;
  unsigned* words;
  const v4u* stream;
  size_t stream_n16;
  unsigned long long* ticks;
  unsigned* err;
  unsigned* sink;
  unsigned cap;
};

__global__ __launch_bounds__(XW_THREADS) void k_exchange(const XchgArgs a) {
  __shared__ int done_waves, stop;
  __shared__ char hold[90 * 1024];  // one workgroup per compute unit
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wg = blockIdx.x, nwg = gridDim.x;
  if (tid == 0) {
    done_waves = 0;
    stop = 0;
    hold[wg & 1023] = 0;
  }
  __syncthreads();
  if (wave < 4) {
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    bool ok = true;
    if (a.mode == 0) {
      // ping: workgroup 0 and workgroup arg pass a round number back and forth
      if (wave == 0 && lane == 0 && (wg == 0 || wg == a.arg)) {
        const auto rs = xw_rsrc(a.words, 512);
        const int mine = wg == 0 ? 0 : 256, theirs = wg == 0 ? 256 : 0;
        for (int r = 1; r <= a.rounds && ok; ++r) {
          if (wg == 0) __hip_atomic_store(a.words + mine / 4, (unsigned)r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          for (unsigned it = 0;; ++it) {
            asm volatile("" ::: "memory");
            if (__builtin_amdgcn_raw_buffer_load_b32(rs, theirs, 0, XW_SC1) == (unsigned)r) break;
            if (it >= a.cap) {
              ok = false;
              break;
            }
          }
          if (wg != 0) __hip_atomic_store(a.words + mine / 4, (unsigned)r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (wg == 0) {
          a.ticks[0] = __builtin_amdgcn_s_memrealtime() - t0;
          __hip_atomic_store(a.words + 128, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // pings done
        }
        if (!ok) atomicAdd(a.err, 1u);
      }
      // every measuring wave holds its workgroup's stream until the pings are done (bounded)
      if (lane == 0) {
        const auto rs = xw_rsrc(a.words, 1024);
        for (unsigned it = 0; it < a.cap; ++it) {
          asm volatile("" ::: "memory");
          if (__builtin_amdgcn_raw_buffer_load_b32(rs, 512, 0, XW_SC1) != 0u) break;
          __builtin_amdgcn_s_sleep(10);
        }
      }
    } else {
      // all-gather of arg words: workgroup w owns words [w per, (w + 1) per), stored as 16-byte
      // stores into 8 replicas (one per XCD); every workgroup polls its XCD's replica, each of the
      // four waves a quarter; the rounds alternate between two copies of the replicas
      const int per = a.arg / nwg, nq = a.arg / 1024;
      for (int r = 1; r <= a.rounds && ok; ++r) {
        const int b = r & 1;
        for (unsigned it = 0; __hip_atomic_load(&done_waves, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < 4 * (r - 1);
             ++it) {
          __builtin_amdgcn_s_sleep(1);
          if (it >= a.cap) {
            ok = false;
            break;
          }
        }
        if (!__all(ok)) break;
        if (wave == 0 && lane < 2 * per) {  // per/4 lanes per replica
          const int rep = lane / (per / 4), q = lane % (per / 4);
          const auto rs = xw_rsrc(a.words + ((size_t)b * 8 + rep) * a.arg, 4u * a.arg);
          const v4u v = {(unsigned)r, (unsigned)r, (unsigned)r, (unsigned)r};
          __builtin_amdgcn_raw_buffer_store_b128(v, rs, (wg * per + 4 * q) * 4, 0, XW_SC1);
        }
        const auto prs = xw_rsrc(a.words + ((size_t)b * 8 + xw_xcd()) * a.arg, 4u * a.arg);
        unsigned pend = (1u << nq) - 1u;
        for (unsigned it = 0; __any(pend != 0); ++it) {
          asm volatile("" ::: "memory");
          v4u q[8];
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if ((pend >> i) & 1) q[i] = __builtin_amdgcn_raw_buffer_load_b128(prs, (4 * tid + 1024 * i) * 4, 0, XW_SC1);
#pragma unroll
          for (int i = 0; i < 8; ++i)
            if (((pend >> i) & 1) && q[i][0] == (unsigned)r && q[i][1] == (unsigned)r && q[i][2] == (unsigned)r &&
                q[i][3] == (unsigned)r)
              pend &= ~(1u << i);
          if (it >= a.cap) {
            ok = false;
            break;
          }
        }
        if (!__all(ok)) break;
        if (lane == 0) __hip_atomic_fetch_add(&done_waves, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      if (tid == 0) a.ticks[wg] = __builtin_amdgcn_s_memrealtime() - t0;
      if (lane == 0 && !__all(ok)) atomicAdd(a.err, 1u);
    }
    if (lane == 0) __hip_atomic_store(&stop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  } else if (a.sif > 0) {
    // background read stream: a.sif nontemporal 16-byte loads in flight per lane, until a measuring
    // wave of this workgroup is done (at most 2^20 loads per lane)
    const size_t stride = (size_t)nwg * 8 * 64, base = ((size_t)wg * 8 + (wave - 4)) * 64 + lane;
    size_t i = base;
    unsigned acc = 0;
    for (int n = 0; n < (1 << 20); ++n) {
      if ((n & 15) == 0 && __hip_atomic_load(&stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) break;
      if (i >= a.stream_n16) i = base;
      const v4u v = __builtin_nontemporal_load(a.stream + i);
      acc ^= v[0] ^ v[3];
      i += stride;
      if (a.sif == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | 0);
      else if (a.sif == 2) __builtin_amdgcn_s_waitcnt(0x0F70 | 1);
      else if (a.sif == 3) __builtin_amdgcn_s_waitcnt(0x0F70 | 2);
      else __builtin_amdgcn_s_waitcnt(0x0F70 | 3);
    }
    a.sink[wg * 8 + (wave - 4)] = acc;
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

DN_API int dn_probe_exchange(int mode, int arg, int rounds, int stream_in_flight, unsigned* words, size_t words_bytes,
                             const void* stream_buf, size_t stream_bytes, unsigned long long* ticks, unsigned* err,
                             unsigned* sink, int nwg, void* hip_stream) {
  if (!words || !ticks || !err || !sink || nwg < 2 || nwg > DN_PROBE_XCHG_MAX_WG || rounds < 1 || rounds > 100000 ||
      stream_in_flight < 0 || stream_in_flight > 4 || (stream_in_flight > 0 && (!stream_buf || stream_bytes < 16)) ||
      (reinterpret_cast<uintptr_t>(words) & 15u) || (reinterpret_cast<uintptr_t>(stream_buf) & 15u))
    return -1;
  if (stream_in_flight > 0 && stream_bytes / 16 < (size_t)nwg * 8 * 64) return -1;
  if (mode == 0) {
    if (arg < 1 || arg >= nwg || words_bytes < 1024) return -1;
  } else if (mode == 1) {
    if (arg < 1024 || arg > 8192 || (arg & 1023) || arg % (4 * nwg) || 2 * (arg / nwg) > 64 ||
        words_bytes < (size_t)2 * 8 * arg * 4)
      return -1;
  } else {
    return -1;
  }
  XchgArgs a{mode, arg, rounds, stream_in_flight, words, static_cast<const v4u*>(stream_buf), stream_bytes / 16,
             ticks, err, sink, 1u << 20};
  hipLaunchKernelGGL(k_exchange, dim3(nwg), dim3(XW_THREADS), 0, reinterpret_cast<hipStream_t>(hip_stream), a);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
