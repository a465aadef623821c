// Batched decode: B >= 2 independent sequences stepped together through each layer (the
// per-layer step of page "qwen36: run the DeltaNet layer end to end on the card", section "What
// the PR does", Backend paragraph, applied to every sequence of the batch).
//
// With a batch the two projections are skinny GEMMs (M weight rows x B sequences x K), so they run
// on the int8 matrix cores (v_mfma_i32_16x16x64_i8); the recurrence is a pure stream over the B x
// Hv state tiles.
//
//  * k_bsplit: the activations of a step split once into three int8 terms per (sequence,
//    128-column chunk), v ~= s1 (h + (m + l/254)/254) with s1 = max|v|/127 over the chunk, stored
//    in the GEMM's fragment order.
//  * k_bgemm: partial sums over a K range of KR columns (split-K across workgroups) for 64*MF
//    weight rows and 64 sequences. Each MFMA accumulates exact int32 products; a chunk's three sums
//    are combined in double with the chunk's scale. Fragments reach LDS by direct-to-LDS copies,
//    double-buffered; weight fragments stream into registers one chunk ahead.
//  * k_bepi: adds the KS partial sums in a fixed order and finishes each row: row scale, optional
//    input pre-norm factor, and for in_proj rows r < C the causal conv over the history plus SiLU.
//  * k_bstate: one workgroup per (value head, sequence): L2 norms of q and k in double, decay,
//    delta rule against the decayed state, readout over the updated state and the gated RMSNorm
//    with silu(z); the head's 128 outputs are one chunk of out_proj's input, split in place. Thread t holds rows 16(t/32)..+15 x columns 4(t%32)..+3 of the 128 x 128 tile
//    in registers: one coalesced read and one write of the tile.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dn_internal.h"
#include "dn_tsplit_norm.h"

namespace dn {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// s_waitcnt with vmcnt <= n and the other counters unconstrained
#define DN_VMCNT_WAIT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | (n))

constexpr int KC = 128;  // activation columns staged per chunk (2 MFMA k-steps of 64)
constexpr int KSC = KC / 64;  // k-steps per chunk
constexpr int NT = 64;   // sequences per workgroup: 4 MFMA column fragments of 16

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Two packed 4-bit weights per byte (element 2m low nibble, 2m+1 high) -> four signed bytes
// holding 16*w in k order, from one 16-bit half.
__device__ __forceinline__ int nib4(unsigned h16) {
  const unsigned y = (h16 & 0xFFu) | ((h16 & 0xFF00u) << 8);
  return (int)(((y << 4) & 0x00F000F0u) | ((y & 0x00F000F0u) << 8));
}

// Workgroup barrier over LDS data only. __syncthreads() carries a fence that waits for every
// outstanding global access of the wave (vmcnt counts loads too), which would make the next chunk's
// copies and weight loads complete before the current chunk's MFMAs start; this waits only for the
// wave's LDS accesses, and each wave waits for its own direct-to-LDS copies with an explicit vmcnt.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Split v (|v| <= 127 s1) into three int8 terms.
__device__ __forceinline__ void split3(float v, float inv1, float s1, float inv2, float s2, float inv3, int& h,
                                       int& m, int& l) {
  const float hf = fminf(fmaxf(rintf(v * inv1), -127.f), 127.f);
  const float r1 = fmaf(-s1, hf, v);
  const float mf = fminf(fmaxf(rintf(r1 * inv2), -127.f), 127.f);
  const float r2 = fmaf(-s2, mf, r1);
  const float lf = fminf(fmaxf(rintf(r2 * inv3), -127.f), 127.f);
  h = (int)hf;
  m = (int)mf;
  l = (int)lf;
}

// Three-term int8 split of the activations, once per (sequence, 128-column chunk), written in
// the order the GEMM's LDS fragments take: for column block nb and chunk c a 24 KB block
// [term][k-step][column fragment][lane][16 bytes] (lane = sequence % 16 + 16 * (16-column group of
// the k-step)), the chunk's scale per sequence, and its sum of squares (for the input pre-norm).
__global__ __launch_bounds__(64) void k_bsplit(const BSplitArgs a) {
  // one wave per 16 sequences of a chunk: blockIdx.y = 4 * (block of 64 sequences) + group of 16
  const int tid = threadIdx.x, c = blockIdx.x, nb = blockIdx.y >> 2;
  const int NC = gridDim.x;
  // sequence nb*64 + sb, columns 32 sq4 .. +31 of the chunk
  const int sb = 16 * (blockIdx.y & 3) + (tid >> 2), sq4 = tid & 3;
  const int b = nb * NT + sb;
  const bool valid = b < a.B;
  const float* arow = a.act + (size_t)(valid ? b : 0) * a.act_stride + c * KC + 32 * sq4;
  v4f xv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) xv[i] = valid ? reinterpret_cast<const v4f*>(arow)[i] : v4f{0.f, 0.f, 0.f, 0.f};
  float mx = 0.f, ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mx = fmaxf(mx, fabsf(xv[i][e]));
      ss = fmaf(xv[i][e], xv[i][e], ss);
    }
  // the four threads of a sequence are the lanes of one quad
  mx = fmaxf(mx, dpp_f<0xB1>(mx));
  mx = fmaxf(mx, dpp_f<0x4E>(mx));
  ss += dpp_f<0xB1>(ss);
  ss += dpp_f<0x4E>(ss);
  float s1 = mx * (1.0f / 127.0f);
  if (!(s1 > 0.f)) s1 = 1.0f;
  const float inv1 = 1.0f / s1, s2 = s1 * (1.0f / 254.0f), inv2 = 1.0f / s2, inv3 = 254.0f / s2;
  const size_t blk = (size_t)nb * NC + c;
  if (sq4 == 0) {
    a.sc[blk * NT + sb] = s1;
    if (valid) a.ssq[(size_t)b * NC + c] = ss;
  }
  v4i* xs = static_cast<v4i*>(a.xs) + blk * (3 * KSC * 4 * 64);
  // columns 32 sq4 + 16 gg: k-step sq4 / 2, 16-column group 2 (sq4 % 2) + gg -> lane
  // (sb % 16) + 16 * group of column fragment sb / 16
#pragma unroll
  for (int gg = 0; gg < 2; ++gg) {
    int hw[4], mw[4], lw[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      int h0, m0, l0, h1, m1, l1, h2, m2, l2, h3, m3, l3;
      const v4f v = xv[4 * gg + d];
      split3(v[0], inv1, s1, inv2, s2, inv3, h0, m0, l0);
      split3(v[1], inv1, s1, inv2, s2, inv3, h1, m1, l1);
      split3(v[2], inv1, s1, inv2, s2, inv3, h2, m2, l2);
      split3(v[3], inv1, s1, inv2, s2, inv3, h3, m3, l3);
      hw[d] = (h0 & 0xFF) | ((h1 & 0xFF) << 8) | ((h2 & 0xFF) << 16) | ((h3 & 0xFF) << 24);
      mw[d] = (m0 & 0xFF) | ((m1 & 0xFF) << 8) | ((m2 & 0xFF) << 16) | ((m3 & 0xFF) << 24);
      lw[d] = (l0 & 0xFF) | ((l1 & 0xFF) << 8) | ((l2 & 0xFF) << 16) | ((l3 & 0xFF) << 24);
    }
    const int f = sb >> 4, ln = (sb & 15) + 16 * (2 * (sq4 & 1) + gg), ks2 = sq4 >> 1;
    xs[((0 * KSC + ks2) * 4 + f) * 64 + ln] = v4i{hw[0], hw[1], hw[2], hw[3]};
    xs[((1 * KSC + ks2) * 4 + f) * 64 + ln] = v4i{mw[0], mw[1], mw[2], mw[3]};
    xs[((2 * KSC + ks2) * 4 + f) * 64 + ln] = v4i{lw[0], lw[1], lw[2], lw[3]};
  }
}

// Whole-row three-term split (library GEMM input): one workgroup per row t. The row's maximum and
// sum of squares are reduced in a fixed order; the terms go to xs[i][t][k], four columns per thread
// per pass, rows read twice (the second pass hits the cache).
__global__ __launch_bounds__(256) void k_tsplit(const TSplitArgs a) {
  __shared__ float rmx[4], rss[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, t = blockIdx.x;
  const int K = a.K;
  const float* row = a.act + (size_t)t * a.act_stride;
  float mx = 0.f, ss = 0.f;
  for (int c = 4 * tid; c < K; c += 1024) {
    const v4f v = *reinterpret_cast<const v4f*>(row + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mx = fmaxf(mx, fabsf(v[e]));
      ss = fmaf(v[e], v[e], ss);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o));
    ss += __shfl_xor(ss, o);
  }
  if (lane == 0) {
    rmx[wave] = mx;
    rss[wave] = ss;
  }
  __syncthreads();
  mx = fmaxf(fmaxf(rmx[0], rmx[1]), fmaxf(rmx[2], rmx[3]));
  ss = (rss[0] + rss[1]) + (rss[2] + rss[3]);
  float s1 = mx * (1.0f / 127.0f);
  if (!(s1 > 0.f)) s1 = 1.0f;
  const float inv1 = 1.0f / s1, s2 = s1 * (1.0f / 254.0f), inv2 = 1.0f / s2, inv3 = 254.0f / s2;
  if (tid == 0) {
    a.s1[t] = s1;
    a.ssq[t] = ss;
  }
  const size_t plane = (size_t)a.T * K;
  int8_t* xh = a.xs + (size_t)t * K;
  for (int c = 4 * tid; c < K; c += 1024) {
    const v4f v = *reinterpret_cast<const v4f*>(row + c);
    int h[4], m[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split3(v[e], inv1, s1, inv2, s2, inv3, h[e], m[e], l[e]);
    auto pack = [](const int (&q)[4]) {
      return (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) | ((q[3] & 0xFF) << 24);
    };
    *reinterpret_cast<int*>(xh + c) = pack(h);
    *reinterpret_cast<int*>(xh + plane + c) = pack(m);
    *reinterpret_cast<int*>(xh + 2 * plane + c) = pack(l);
  }
}

// k_tsplit of the readout rows with the gated RMSNorm fused in front: thread i holds columns
// 1024 p + 4 i .. +3 of pass p, so a head's 128 columns are 32 consecutive lanes of one pass; the
// normalised, gated row stays in registers for the split.
__global__ __launch_bounds__(256) void k_tsplit_norm(const TSplitNormArgs a) {
  constexpr int NP = 8;  // passes of 1024 columns (K <= 8192)
  __shared__ float rmx[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, t = blockIdx.x;
  const int K = a.sp.K;
  const float* row = a.sp.act + (size_t)t * a.sp.act_stride;
  const float* zr = a.z + (size_t)t * a.z_stride;
  v4f y[NP];
  float mx = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c = 1024 * p + 4 * tid;
    y[p] = v4f{0.f, 0.f, 0.f, 0.f};
    if (c < K) {  // K is a multiple of 128, so a head's 32 lanes are all in or all out
      const v4f o = *reinterpret_cast<const v4f*>(row + c);
      const v4f z = *reinterpret_cast<const v4f*>(zr + c);
      const v4f w = *reinterpret_cast<const v4f*>(a.norm_w + (c & 127));
      float ss = (o[0] * o[0] + o[1] * o[1]) + (o[2] * o[2] + o[3] * o[3]);
#pragma unroll
      for (int m = 1; m < 32; m <<= 1) ss += __shfl_xor(ss, m);
      const float inv = rsqrtf(ss / 128.0f + a.eps);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float g = z[e] / (1.0f + __expf(-z[e]));  // silu(z)
        y[p][e] = w[e] * o[e] * inv * g;
        mx = fmaxf(mx, fabsf(y[p][e]));
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
  if (lane == 0) rmx[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(rmx[0], rmx[1]), fmaxf(rmx[2], rmx[3]));
  float s1 = mx * (1.0f / 127.0f);
  if (!(s1 > 0.f)) s1 = 1.0f;
  const float inv1 = 1.0f / s1, s2 = s1 * (1.0f / 254.0f), inv2 = 1.0f / s2, inv3 = 254.0f / s2;
  if (tid == 0) a.sp.s1[t] = s1;
  const size_t plane = (size_t)a.sp.T * K;
  int8_t* xh = a.sp.xs + (size_t)t * K;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c = 1024 * p + 4 * tid;
    if (c < K) {
      int h[4], m[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) split3(y[p][e], inv1, s1, inv2, s2, inv3, h[e], m[e], l[e]);
      auto pack = [](const int (&q)[4]) {
        return (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) | ((q[3] & 0xFF) << 24);
      };
      *reinterpret_cast<int*>(xh + c) = pack(h);
      *reinterpret_cast<int*>(xh + plane + c) = pack(m);
      *reinterpret_cast<int*>(xh + 2 * plane + c) = pack(l);
    }
  }
}

// Split-K GEMM on the pre-split activations: partial sums of one K range for 64 MF rows and 64
// sequences. Each 128-column chunk (24 KB of fragments + 64 scales) is copied straight into LDS
// with direct-to-LDS loads, double-buffered, while the next chunk's weight fragments stream into
// registers.
template <int BITS, int MF, int NKS>
__global__ __launch_bounds__(256) void k_bgemm(const BGemmArgs a) {
  constexpr int NCHUNK = NKS / KSC;
  constexpr int FRAGS = 3 * KSC * 4 * 64;  // v4i per chunk block (24 KB)
  constexpr int PER_WAVE = FRAGS / 64 / 4;  // 1 KB direct-to-LDS loads per wave per chunk
  static_assert(NCHUNK % 2 == 0, "chunks run in pairs");
  // two separate buffers, so that the compiler can tell the copies into one from the reads of the
  // other and keeps the next chunk's copies in flight while the current chunk is read
  __shared__ v4i xs0[FRAGS], xs1[FRAGS];
  __shared__ float scl0[NT], scl1[NT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = blockIdx.x, ks = blockIdx.y, nb = blockIdx.z;
  const int M = a.M, K = a.K, B = a.B;
  const int NC = K / KC;
  const int k0 = ks * (NKS * 64);
  const int c0 = k0 / KC;
  const int r0 = rb * 64 * MF + wave * 16 * MF;

  typedef v4i Frag[KSC][MF];
  // A fragments (weights): row r0 + 16 mf + lane%16, k = 64 s + 16 (lane/16) + byte
  auto load_a = [&](int c, Frag& A) {
#pragma unroll
    for (int s = 0; s < KSC; ++s)
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        const size_t row = (size_t)(r0 + 16 * mf + (lane & 15));
        const int kk = k0 + 64 * (KSC * c + s) + 16 * (lane >> 4);
        if (BITS == 8) {
          A[s][mf] =
              __builtin_nontemporal_load(reinterpret_cast<const v4i*>(static_cast<const int8_t*>(a.W) + row * K + kk));
        } else {
          const v2u p = __builtin_nontemporal_load(
              reinterpret_cast<const v2u*>(static_cast<const uint8_t*>(a.W) + row * (K / 2) + kk / 2));
          A[s][mf] = v4i{nib4(p.x & 0xFFFFu), nib4(p.x >> 16), nib4(p.y & 0xFFFFu), nib4(p.y >> 16)};
        }
      }
  };
  // copy chunk c's fragments and scales into LDS buffer X, S
  auto stage = [&](int c, v4i* X, float* S) {
    const size_t blk = (size_t)nb * NC + c0 + c;
    const v4i* src = static_cast<const v4i*>(a.xs) + blk * FRAGS;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = wave * PER_WAVE + i;  // 1 KB piece
      __builtin_amdgcn_global_load_lds(src + q * 64 + lane, X + q * 64, 16, 0, 0);
    }
    if (wave == 0) __builtin_amdgcn_global_load_lds(a.sc + blk * NT + lane, S, 4, 0, 0);
  };

  float facc[MF][4][4];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) facc[mf][f][v] = 0.f;

  Frag A0, A1;
  stage(0, xs0, scl0);
  load_a(0, A0);
  // one chunk: request the next chunk into the other buffer, wait for this one, run its MFMAs
  auto chunk = [&](int c, const Frag& A, Frag& Anext, const v4i* X, const float* S, v4i* Xn, float* Sn) {
    if (c + 1 < NCHUNK) {
      stage(c + 1, Xn, Sn);
      load_a(c + 1, Anext);
      // loads issued after this chunk's: the next chunk's pieces (+ its scales on wave 0) and weights
      if (wave == 0) DN_VMCNT_WAIT(PER_WAVE + 1 + KSC * MF);
      else DN_VMCNT_WAIT(PER_WAVE + KSC * MF);
    } else {
      DN_VMCNT_WAIT(0);
    }
    lds_barrier();  // every wave's pieces of chunk c are in LDS
    v4i acc[3][MF][4];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[t][mf][f] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < KSC; ++s)
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const v4i bf = X[((t * KSC + s) * 4 + f) * 64 + lane];
#pragma unroll
          for (int mf = 0; mf < MF; ++mf)
            acc[t][mf][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[s][mf], bf, acc[t][mf][f], 0, 0, 0);
        }
    // fold the chunk into the float sums with each sequence's scale (column lane % 16 of fragment f);
    // a chunk's sums are below 2^22 in magnitude: exact in fp32, combined in fp32
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const float s1b = S[16 * f + (lane & 15)] * (BITS == 4 ? 1.0f / 16.0f : 1.0f);
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float d = (float)acc[0][mf][f][v] +
                          fmaf((float)acc[2][mf][f][v], 1.0f / 254.0f, (float)acc[1][mf][f][v]) * (1.0f / 254.0f);
          facc[mf][f][v] = fmaf(s1b, d, facc[mf][f][v]);
        }
    }
    lds_barrier();  // buffer c % 2 is refilled two chunks later
  };
  // rolled loop over chunk pairs (ping-pong weight and LDS buffers), so only two chunks of weights
  // are live
#pragma clang loop unroll(disable)
  for (int c = 0; c < NCHUNK; c += 2) {
    chunk(c, A0, A1, xs0, scl0, xs1, scl1);
    chunk(c + 1, A1, A0, xs1, scl1, xs0, scl0);
  }

  // partial sums: lane holds rows r0 + 16 mf + 4 (lane/16) .. +3 of sequence nb*64 + 16 f + lane%16
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int b = nb * NT + 16 * f + (lane & 15);
    if (b < B)
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
        *reinterpret_cast<v4f*>(a.part + ((size_t)ks * B + b) * M + r0 + 16 * mf + 4 * (lane >> 4)) =
            v4f{facc[mf][f][0], facc[mf][f][1], facc[mf][f][2], facc[mf][f][3]};
  }
}

// Split-K GEMM, all loads up front. A workgroup of 4*NRB waves owns one K range of KR columns, 64
// sequences and NRB blocks of 64 weight rows (wave w: 16 rows of block w/4). It first copies the K
// range's split activations (3 x 64 x KR bytes) into LDS with direct-to-LDS loads and waits for
// them alone (the compiler orders every later LDS read after all loads that precede it, so no
// weight load may be in flight at that point); then each wave requests its whole K range of
// weight fragments at once and runs the MFMAs as they arrive.
//
// SPLIT: the workgroup splits its K range of the fp32 activations itself (as k_bsplit does, into the
// same LDS fragment order): eight waves load the slice with plain loads, every wave then requests
// its weights, and the split waits only for the activation loads, so the two latencies overlap.
template <int BITS, int NRB, int KR, bool SPLIT>
__global__ __launch_bounds__(256 * NRB) void k_bgemm2(const BGemmArgs a) {
  constexpr int NW = 4 * NRB;              // waves
  constexpr int NKS = KR / 64;             // k-steps
  constexpr int NCHUNK = KR / KC;          // 128-column chunks (one split scale each)
  constexpr int FRAGS = 3 * KSC * 4 * 64;  // v4i per chunk block (24 KB)
  constexpr int PIECES = NCHUNK * FRAGS / 64;  // 1 KB direct-to-LDS copies
  static_assert(PIECES % NW == 0, "");
  __shared__ v4i xs[NCHUNK][FRAGS];
  __shared__ float scl[NCHUNK][NT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rg = blockIdx.x, ks = blockIdx.y, nb = blockIdx.z;
  const int M = a.M, K = a.K, B = a.B;
  const int NC = K / KC;
  const int k0 = ks * KR, c0 = k0 / KC;
  const int row0 = (rg * NRB + wave / 4) * 64 + 16 * (wave & 3);

  static_assert(!SPLIT || (BITS == 8 && NCHUNK * 64 * 4 <= 256 * NRB), "split: 4 threads per (sequence, chunk)");
  // SPLIT: thread (chunk sc, sequence sb, quarter sq4) holds columns 32 sq4 .. +31 of the chunk
  const bool splitter = SPLIT && tid < NCHUNK * 64 * 4;
  const int sc_ = tid >> 8, sb = (tid >> 2) & 63, sq4 = tid & 3;
  const int bs = nb * NT + sb;
  const bool bvalid = bs < B;
  v4f xv[8];
  if constexpr (SPLIT) {
    if (splitter) {
      // rows past the batch load row 0 (unconditional loads, no branches between them) and are
      // zeroed once they arrive
      const float* arow = a.act + (size_t)(bvalid ? bs : 0) * a.act_stride + k0 + sc_ * KC + 32 * sq4;
#pragma unroll
      for (int i = 0; i < 8; ++i) xv[i] = reinterpret_cast<const v4f*>(arow)[i];
    }
  } else {
    const v4i* src = static_cast<const v4i*>(a.xs) + ((size_t)nb * NC + c0) * FRAGS;
    v4i* dst = &xs[0][0];
#pragma unroll
    for (int i = 0; i < PIECES / NW; ++i) {
      const int q = wave * (PIECES / NW) + i;  // 1 KB piece of the K range's contiguous blocks
      __builtin_amdgcn_global_load_lds(src + q * 64 + lane, dst + q * 64, 16, 0, 0);
    }
    if (wave == 0)
#pragma unroll
      for (int c = 0; c < NCHUNK; ++c)
        __builtin_amdgcn_global_load_lds(a.sc + ((size_t)nb * NC + c0 + c) * NT + lane, &scl[c][0], 4, 0, 0);
    DN_VMCNT_WAIT(0);
    __syncthreads();
  }
  v4i A[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const size_t row = (size_t)(row0 + (lane & 15));
    const int kk = k0 + 64 * s + 16 * (lane >> 4);
    if (BITS == 8) {
      A[s] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(static_cast<const int8_t*>(a.W) + row * K + kk));
    } else {
      const v2u p = __builtin_nontemporal_load(
          reinterpret_cast<const v2u*>(static_cast<const uint8_t*>(a.W) + row * (K / 2) + kk / 2));
      A[s] = v4i{nib4(p.x & 0xFFFFu), nib4(p.x >> 16), nib4(p.y & 0xFFFFu), nib4(p.y >> 16)};
    }
  }
  if constexpr (SPLIT) {
    // the activation loads are older than the weight loads: waiting for xv leaves the weights in
    // flight
    if (splitter) {
      if (!bvalid)
#pragma unroll
        for (int i = 0; i < 8; ++i) xv[i] = v4f{0.f, 0.f, 0.f, 0.f};
      float mx = 0.f, ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          mx = fmaxf(mx, fabsf(xv[i][e]));
          ss = fmaf(xv[i][e], xv[i][e], ss);
        }
      mx = fmaxf(mx, dpp_f<0xB1>(mx));
      mx = fmaxf(mx, dpp_f<0x4E>(mx));
      ss += dpp_f<0xB1>(ss);
      ss += dpp_f<0x4E>(ss);
      float s1 = mx * (1.0f / 127.0f);
      if (!(s1 > 0.f)) s1 = 1.0f;
      const float inv1 = 1.0f / s1, s2 = s1 * (1.0f / 254.0f), inv2 = 1.0f / s2, inv3 = 254.0f / s2;
      if (sq4 == 0) {
        scl[sc_][sb] = s1;
        if (rg == 0 && bvalid) a.ssq[(size_t)bs * NC + c0 + sc_] = ss;
      }
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        int hw[4], mw[4], lw[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          int h0, m0, l0, h1, m1, l1, h2, m2, l2, h3, m3, l3;
          const v4f v = xv[4 * gg + d];
          split3(v[0], inv1, s1, inv2, s2, inv3, h0, m0, l0);
          split3(v[1], inv1, s1, inv2, s2, inv3, h1, m1, l1);
          split3(v[2], inv1, s1, inv2, s2, inv3, h2, m2, l2);
          split3(v[3], inv1, s1, inv2, s2, inv3, h3, m3, l3);
          hw[d] = (h0 & 0xFF) | ((h1 & 0xFF) << 8) | ((h2 & 0xFF) << 16) | ((h3 & 0xFF) << 24);
          mw[d] = (m0 & 0xFF) | ((m1 & 0xFF) << 8) | ((m2 & 0xFF) << 16) | ((m3 & 0xFF) << 24);
          lw[d] = (l0 & 0xFF) | ((l1 & 0xFF) << 8) | ((l2 & 0xFF) << 16) | ((l3 & 0xFF) << 24);
        }
        const int f = sb >> 4, ln = (sb & 15) + 16 * (2 * (sq4 & 1) + gg), ks2 = sq4 >> 1;
        xs[sc_][((0 * KSC + ks2) * 4 + f) * 64 + ln] = v4i{hw[0], hw[1], hw[2], hw[3]};
        xs[sc_][((1 * KSC + ks2) * 4 + f) * 64 + ln] = v4i{mw[0], mw[1], mw[2], mw[3]};
        xs[sc_][((2 * KSC + ks2) * 4 + f) * 64 + ln] = v4i{lw[0], lw[1], lw[2], lw[3]};
      }
    }
    lds_barrier();  // the staged terms and scales; the weight loads stay in flight
  }

  float facc[4][4];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) facc[f][v] = 0.f;
#pragma unroll
  for (int c = 0; c < NCHUNK; ++c) {
    v4i acc[3][4];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int f = 0; f < 4; ++f) acc[t][f] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < KSC; ++s) {
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int f = 0; f < 4; ++f)
          acc[t][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[KSC * c + s], xs[c][((t * KSC + s) * 4 + f) * 64 + lane],
                                                            acc[t][f], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // one k-step's fragments in registers at a time
    }
    // a chunk's sums are below 2^22 in magnitude: exact in fp32, combined in fp32
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const float s1b = scl[c][16 * f + (lane & 15)] * (BITS == 4 ? 1.0f / 16.0f : 1.0f);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float d = (float)acc[0][f][v] +
                         fmaf((float)acc[2][f][v], 1.0f / 254.0f, (float)acc[1][f][v]) * (1.0f / 254.0f);
        facc[f][v] = fmaf(s1b, d, facc[f][v]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // one chunk's accumulators live at a time
  }
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const int b = nb * NT + 16 * f + (lane & 15);
    if (b < B)
      *reinterpret_cast<v4f*>(a.part + ((size_t)ks * B + b) * M + row0 + 4 * (lane >> 4)) =
          v4f{facc[f][0], facc[f][1], facc[f][2], facc[f][3]};
  }
}

// Three-term split of whole activation rows for the whole-K projection: one workgroup per sequence,
// one scale per row (s1 = max|v| / 127 over all K columns, as the single-sequence path splits its
// input), written in the fragment order of k_bsplit; the row's scale goes to sc [block][64] and its
// sum of squares (for the input pre-norm) to ssq [B].
__global__ __launch_bounds__(256) void k_bsplit_row(const BSplitArgs a) {
  constexpr int NP = 8;  // passes of 1024 columns (K <= 8192)
  __shared__ float rmx[4], rss[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, b = blockIdx.x;
  const int K = a.K, NC = K / KC, nb = b / NT, sb = b % NT;
  const float* row = a.act + (size_t)b * a.act_stride;
  v4f v[NP];
  float mx = 0.f, ss = 0.f;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int c = 4 * tid + 1024 * p;
    v[p] = c < K ? *reinterpret_cast<const v4f*>(row + c) : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mx = fmaxf(mx, fabsf(v[p][e]));
      ss = fmaf(v[p][e], v[p][e], ss);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o));
    ss += __shfl_xor(ss, o);
  }
  if (lane == 0) {
    rmx[wave] = mx;
    rss[wave] = ss;
  }
  __syncthreads();
  mx = fmaxf(fmaxf(rmx[0], rmx[1]), fmaxf(rmx[2], rmx[3]));
  ss = (rss[0] + rss[1]) + (rss[2] + rss[3]);
  float s1 = mx * (1.0f / 127.0f);
  if (!(s1 > 0.f)) s1 = 1.0f;
  const float inv1 = 1.0f / s1, s2 = s1 * (1.0f / 254.0f), inv2 = 1.0f / s2, inv3 = 254.0f / s2;
  if (tid == 0) {
    a.sc[(size_t)nb * NT + sb] = s1;
    a.ssq[b] = ss;
  }
  int8_t* xs = static_cast<int8_t*>(a.xs);
  const int f = sb >> 4;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int k0 = 4 * tid + 1024 * p;
    if (k0 >= K) break;
    int h[4], m[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split3(v[p][e], inv1, s1, inv2, s2, inv3, h[e], m[e], l[e]);
    // column k0 .. k0+3: chunk c, k-step ks, 16-column group g, bytes (k0 % 16) .. +3 of lane
    // (sb % 16) + 16 g of column fragment f
    const int c = k0 / KC, kk = k0 % KC, ks = kk / 64, gq = (kk % 64) / 16;
    const size_t frag0 = ((size_t)(nb * NC + c) * (3 * KSC * 4 * 64)) * 16 + (kk % 16);
    const int ln = (sb & 15) + 16 * gq;
    auto pack = [](const int (&q)[4]) {
      return (q[0] & 0xFF) | ((q[1] & 0xFF) << 8) | ((q[2] & 0xFF) << 16) | ((q[3] & 0xFF) << 24);
    };
    *reinterpret_cast<int*>(xs + frag0 + (size_t)(((0 * KSC + ks) * 4 + f) * 64 + ln) * 16) = pack(h);
    *reinterpret_cast<int*>(xs + frag0 + (size_t)(((1 * KSC + ks) * 4 + f) * 64 + ln) * 16) = pack(m);
    *reinterpret_cast<int*>(xs + frag0 + (size_t)(((2 * KSC + ks) * 4 + f) * 64 + ln) * 16) = pack(l);
  }
}

// vmcnt(n) for n < 64 (the counter's low four bits and its high two), expcnt and lgkmcnt not waited
constexpr int vm_imm(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }
// chunk xor permutation of the staged weight rows (row r of a 16-row tile): the operand reads of a
// group of 16 lanes (rows 0..15, one 16-byte chunk each) meet every LDS bank once
__device__ __forceinline__ int bp_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
typedef __attribute__((address_space(3))) void bp_lds_t;

// Copy wave: publish in LDS that n chunks of its K quarter have landed. The store is written out by
// hand: the compiler would otherwise wait for every direct-to-LDS load in flight before it.
__device__ __forceinline__ void bp_publish(int* ready, int n) {
#if defined(__HIP_DEVICE_COMPILE__)  // (the host pass has no LDS address space)
  const unsigned at = (unsigned)(uintptr_t)(__attribute__((address_space(3))) int*)ready;
  asm volatile("ds_write_b32 %0, %1" ::"v"(at), "v"(n) : "memory");
#endif
}

// Whole-K projection with the epilogue fused (no partial sums), 8-bit weights: a workgroup owns 16*RT
// weight rows and 64 sequences, in twelve waves.
//  * Copy waves 8..11: wave 8 + q requests its share of the epilogue's conv history, then the whole
//    K quarter q of the workgroup's weight rows (CPW chunks of 128 columns) straight into LDS at
//    once, each load instruction 8 whole rows of 128 bytes, and publishes in LDS how many of its
//    chunks have landed. So every HBM read of the kernel is in flight from the start.
//  * MFMA waves 0..7: wave w takes K quarter w % 4 for the 32 sequences of half w / 4. The split
//    activations (k_bsplit_row, one scale per row; the same few hundred KB for every workgroup,
//    L2-resident) stream into registers two k-steps ahead; each k-step's weight fragments are read
//    from LDS once its chunk is published. The two halves read the same staged weights.
// Each wave keeps exact int32 sums of the three terms over its whole K quarter (at most
// 127 * 127 * 1024 < 2^24 in magnitude: exact in fp32 too) and folds them once; the four K quarters'
// sums meet in LDS (over the staged weights) and are added in quarter order; then each
// (row, sequence) gets k_bepi's epilogue.
template <int RT, int CPW>
__global__ __launch_bounds__(768) void k_bproj(const BGemmArgs g, const BEpiArgs e) {
  constexpr int ROWS = 16 * RT, NF = 2;  // sequence tiles of 16 per MFMA wave
  constexpr int WT = 2 * RT;             // load instructions (8 rows x 128 bytes) per weight chunk
  constexpr int WQ = CPW * WT * 1024;    // LDS bytes of one K quarter's weights
  // the history: 3 NT segments (slot, sequence) of ROWS channels, 16 bytes (4 channels) per lane, SEGI
  // whole segments per load instruction; NRW instructions per copy wave
  constexpr int LPS = ROWS / 4, SEGI = 64 / LPS, NSEG = 3 * NT;
  constexpr int NRI = (NSEG + SEGI - 1) / SEGI, NRW = (NRI + 3) / 4;
  // the quarter sums: rows padded to ROWS + 4 (16-byte writes of 8 lanes meet every bank once)
  constexpr int RP = ROWS + 4, REG0 = WQ > 4 * NT * RP ? WQ : 4 * NT * RP;  // floats before the history
  static_assert(NRW + CPW * WT + 3 <= 63, "");  // loads in flight per copy wave
  // dynamic LDS (bproj_lds_bytes): [weights 4 WQ bytes, later the quarter sums 4*NT*RP floats (REG0
  // floats for both) | history 3*NT*ROWS | taps 4*ROWS | scales 64 | sums of squares NT | 256 for the
  // history loads past its end] floats. The direct-to-LDS
  // copies write it behind the compiler's back, which it must not assume to be unwritten.
  extern __shared__ float bproj_lds[];
  __shared__ int wready[4];
  char* const wl = reinterpret_cast<char*>(bproj_lds);
  float(*red)[NT][RP] = reinterpret_cast<float(*)[NT][RP]>(bproj_lds);  // [4]
  float(*ring_l)[NT][ROWS] = reinterpret_cast<float(*)[NT][ROWS]>(bproj_lds + REG0);  // [3]
  float* cw_l = bproj_lds + REG0 + 3 * NT * ROWS;
  float* s_l = cw_l + 4 * ROWS;
  float* ssq_l = s_l + 64;
  float* spare_l = ssq_l + NT;
  // wave index uniform (scalar): the direct-to-LDS destinations derive from it
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = blockIdx.x, nb = blockIdx.y;
  const int M = g.M, K = g.K, B = g.B, NC = K / KC;
  const int row0 = rb * ROWS;
  const bool conv = e.conv_w != nullptr;
  const bool hist = conv && row0 < e.C;
  const int Kc = e.Kc, C = e.C;
  if (tid < 4) wready[tid] = 0;
  __syncthreads();

  v4i acc[RT][3][NF];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[rt][t][f] = v4i{0, 0, 0, 0};
  const int kq = wave & 3, f0 = NF * ((wave >> 2) & 1);
  float s1[NF];

  if (wave >= 8) {
    // copy wave q = kq. First the epilogue's inputs (their count varies; the waits below count only
    // the weight loads issued later), addresses clamped into range.
    if (kq == 0) {
      __builtin_amdgcn_global_load_lds(e.s + min(row0 + lane, M - 1), s_l, 4, 0, 0);
      __builtin_amdgcn_global_load_lds(e.ssq + min(nb * NT + lane, B - 1), ssq_l, 4, 0, 0);
    }
    for (int i = kq - 1; hist && i >= 0 && i < ROWS * 4 / 64; i += 3) {
      const int idx = 64 * i + lane, rl = idx / 4, q = idx % 4;
      __builtin_amdgcn_global_load_lds(e.conv_w + (size_t)min(row0 + rl, C - 1) * Kc + min(q, Kc - 1), cw_l + 64 * i, 4, 0, 0);
    }
    // the history: instruction n takes segments SEGI n .. +SEGI-1 (lane l: segment SEGI n + l / LPS,
    // channels 4 (l % LPS) .. +3); lanes past the segments stay idle. Slots past the taps, channels
    // past C and workgroups without history copy weight bytes instead (into slots nothing reads);
    // instructions past the last segment, into the spare area.
    for (int m = 0; m < NRW; ++m) {
      const int n = kq + 4 * m, seg = SEGI * n + lane / LPS, ch = row0 + 4 * (lane % LPS);
      const int j = seg / NT, bl = seg % NT;
      const float* src = reinterpret_cast<const float*>(g.W);
      if (hist && j < Kc - 1 && ch < C)
        src = e.ring + ((size_t)min(nb * NT + bl, B - 1) * (Kc - 1) + j) * C + ch;
      float* dst = n < NRI ? &ring_l[0][0][0] + SEGI * ROWS * n : spare_l;
      if (lane < SEGI * LPS && (n >= NRI || seg < NSEG)) __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    }
    // the K quarter's weights: instruction (chunk c, group gi) fills rows 8 gi .. +7 of the chunk,
    // lane l row 8 gi + l / 8, 16-byte chunk (l % 8) ^ bp_swz(row % 16); rows past M read row M-1
    const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(g.W), (short)0, (int)((size_t)M * K), 0x00020000);
    int woff[WT];
#pragma unroll
    for (int gi = 0; gi < WT; ++gi)
      woff[gi] = min(row0 + 8 * gi + (lane >> 3), M - 1) * K + 16 * ((lane & 7) ^ bp_swz(8 * (gi & 1) + (lane >> 3)));
    auto copy = [&](int c, int gi) {
#if defined(__HIP_DEVICE_COMPILE__)  // (the host pass rejects this form and then drops the kernel's stub)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsW, (bp_lds_t*)(wl + ((kq * CPW + c) * WT + gi) * 1024), 16,
                                               woff[gi], (kq * CPW + c) * KC, 0, 0);
#endif
    };
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int gi = 0; gi < WT; ++gi) copy(c, gi);
    // chunk c has landed once at most the later chunks' loads remain
    static_assert(CPW <= 4, "");
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
      switch (CPW - 1 - c) {
        case 0: __builtin_amdgcn_s_waitcnt(vm_imm(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(vm_imm(WT)); break;
        case 2: __builtin_amdgcn_s_waitcnt(vm_imm(2 * WT)); break;
        default: __builtin_amdgcn_s_waitcnt(vm_imm(3 * WT)); break;
      }
      bp_publish(&wready[kq], c + 1);
    }
  } else {
    // buffer loads of the split activations: one VGPR offset, the chunk and k-step offsets in scalars
    const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void*>(g.xs), (short)0, (int)((size_t)(nb + 1) * NC * 24576), 0x00020000);
    const int xofs = 16 * lane + f0 * 1024;
    const int xblk = nb * NC * 24576;
#pragma unroll
    for (int f = 0; f < NF; ++f) s1[f] = g.sc[(size_t)nb * NT + 16 * (f0 + f) + (lane & 15)];
    v4i X[2][3][NF];
    auto load_x = [&](int ks, int buf) {
      const int c = kq * CPW + ks / KSC, s = ks % KSC;
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int f = 0; f < NF; ++f)
          X[buf][t][f] = __builtin_bit_cast(
              v4i, __builtin_amdgcn_raw_buffer_load_b128(xrs, xofs + ((t * KSC + s) * 4 + f) * 1024, xblk + c * 24576, 0));
    };
    // operand reads within a chunk's 2 KB row tile: lane l, row l % 16, 16-byte chunk 4 s + l / 16
    const int rr = lane & 15, rd0 = 16 * (64 * (rr >> 3) + 8 * (rr & 7) + ((lane >> 4) ^ bp_swz(rr)));
    const int rd1 = rd0 ^ 64;
    // Two k-steps of activations in flight. The scheduler would sink each load next to its first
    // use; the barriers keep the lead.
    load_x(0, 0);
    load_x(1, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < CPW * KSC; ++ks) {
      const int c = ks / KSC, s = ks % KSC, buf = ks & 1;
      if (s == 0) {
        while (__hip_atomic_load(&wready[kq], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) <= c)
          __builtin_amdgcn_s_sleep(1);
        asm volatile("" ::: "memory");  // the chunk's weights are read after its publication
      }
      const char* wb = wl + (kq * CPW + c) * WT * 1024 + (s ? rd1 : rd0);
      v4i A[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) A[rt] = *reinterpret_cast<const v4i*>(wb + rt * 2048);
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int t = 0; t < 3; ++t)
            acc[rt][t][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[rt], X[buf][t][f], acc[rt][t][f], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 2 < CPW * KSC) load_x(ks + 2, buf);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __syncthreads();  // every wave is done with the staged weights; every copy has landed
  if (wave < 8) {
    // fold the three exact term sums with the row scale; the MFMA output layout: lane holds sequence
    // 16 f + lane % 16, rows 16 rt + 4 (lane / 16) + v
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        v4f dv;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float d = (float)acc[rt][0][f][v] +
                          fmaf((float)acc[rt][2][f][v], 1.0f / 254.0f, (float)acc[rt][1][f][v]) * (1.0f / 254.0f);
          dv[v] = s1[f] * d;
        }
        *reinterpret_cast<v4f*>(&red[kq][16 * (f0 + f) + (lane & 15)][16 * rt + 4 * (lane >> 4)]) = dv;
      }
  }
  __syncthreads();

  // epilogue: a thread per sequence and 4 consecutive rows (16-byte LDS reads and stores; rows
  // fastest across threads, so the history and output stores are coalesced)
  for (int idx = tid; idx < NT * ROWS / 4; idx += 768) {
    const int bl = idx / (ROWS / 4), rl = 4 * (idx % (ROWS / 4));
    const int r = row0 + rl, b = nb * NT + bl;
    if (r >= M || b >= B) continue;
    const v4f q0 = *reinterpret_cast<const v4f*>(&red[0][bl][rl]), q1 = *reinterpret_cast<const v4f*>(&red[1][bl][rl]);
    const v4f q2 = *reinterpret_cast<const v4f*>(&red[2][bl][rl]), q3 = *reinterpret_cast<const v4f*>(&red[3][bl][rl]);
    const v4f sv = *reinterpret_cast<const v4f*>(s_l + rl);
    const float pf = e.prenorm ? rsqrtf(ssq_l[bl] / (float)K + e.eps) : 1.0f;
    v4f u, o;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const float sum = ((q0[v] + q1[v]) + q2[v]) + q3[v];
      u[v] = sv[v] * pf * sum;
    }
    o = u;
    if (conv && r < C) {
      v4f h[3];
#pragma unroll
      for (int q = 0; q < 3; ++q) h[q] = *reinterpret_cast<const v4f*>(&ring_l[q][bl][rl]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const v4f tap = *reinterpret_cast<const v4f*>(cw_l + 4 * (rl + v));
        float acc2 = 0.f;
#pragma unroll
        for (int q = 0; q < 3; ++q)
          if (q < Kc - 1) acc2 = fmaf(tap[q], h[q][v], acc2);
        acc2 = fmaf(tap[min(3, Kc - 1)], u[v], acc2);
        o[v] = silu(acc2);
      }
      float* rg = e.ring + (size_t)b * (Kc - 1) * C + r;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (q + 1 < Kc - 1) *reinterpret_cast<v4f*>(rg + (size_t)q * C) = h[q + 1];
      if (Kc > 1) *reinterpret_cast<v4f*>(rg + (size_t)(Kc - 2) * C) = u;
    }
    *reinterpret_cast<v4f*>(e.out + (size_t)b * e.out_stride + r) = o;
  }
}

// Finish the rows: add the K-range partial sums in order, row scale, input pre-norm factor, and for
// rows r < C the causal conv over the history (oldest first) plus SiLU, advancing the history.
template <int NB>
__global__ __launch_bounds__(256) void k_bepi(const BEpiArgs a) {
  const int r = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  if (r >= a.M) return;
  // partials are requested NB at a time (NB >= the count when it is at most 16) before they are
  // added, in a fixed order
  float sum = 0.f;
  if (a.terms) {
    // exact sums of the three terms, folded in double with the row's split scale
    const size_t plane = (size_t)a.B * a.M, at = (size_t)b * a.M + r;
    const int d0 = a.terms[at], d1 = a.terms[plane + at], d2 = a.terms[2 * plane + at];
    sum = (float)((double)a.s1[b] * ((double)d0 + ((double)d1 + (double)d2 * (1.0 / 254.0)) * (1.0 / 254.0)));
  } else {
    for (int k0 = 0; k0 < a.KS; k0 += NB) {
      float pv[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) pv[k] = k0 + k < a.KS ? a.part[((size_t)(k0 + k) * a.B + b) * a.M + r] : 0.f;
#pragma unroll
      for (int k = 0; k < NB; ++k)
        if (k0 + k < a.KS) sum += pv[k];
    }
  }
  float scale = a.s[r];
  if (a.prenorm) {
    float ss = 0.f;
    for (int c0 = 0; c0 < a.NC; c0 += 16) {
      float sv[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) sv[c] = c0 + c < a.NC ? a.ssq[(size_t)b * a.NC + c0 + c] : 0.f;
#pragma unroll
      for (int c = 0; c < 16; ++c)
        if (c0 + c < a.NC) ss += sv[c];
    }
    scale *= rsqrtf(ss / (float)a.K + a.eps);
  }
  const float u = scale * sum;
  float o = u;
  if (a.conv_w && r < a.C) {
    const int Kc = a.Kc, C = a.C;
    const float* cw = a.conv_w + (size_t)r * Kc;
    float* rg = a.ring + (size_t)b * (Kc - 1) * C + r;
    float prev[3] = {0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < Kc - 1) prev[j] = rg[(size_t)j * C];
    float acc = cw[Kc - 1] * u;
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < Kc - 1) acc = fmaf(cw[j], prev[j], acc);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (j + 1 < Kc - 1) rg[(size_t)j * C] = prev[j + 1];
    if (Kc > 1) rg[(size_t)(Kc - 2) * C] = u;
    o = silu(acc);
  }
  a.out[(size_t)b * a.out_stride + r] = o;
}

// One (value head, sequence) per workgroup; 128 x 128 state tile. PK: one decay per key row.
template <bool PK>
__global__ __launch_bounds__(256) void k_bstate(const BStateArgs a) {
  constexpr int DK = 128, DV = 128;
  __shared__ float qs[DK], kks[DK], dl[DV], als[PK ? DK : 1];
  __shared__ float red[8][DV];
  __shared__ double dred[4][2];
  __shared__ float fred[2];
  __shared__ __attribute__((aligned(16))) int8_t ybytes[3][DV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, b = blockIdx.y;
  const int cg = tid & 31, rg = tid >> 5;
  float* Sb = a.S + ((size_t)b * a.Hv + h) * DK * DV;
  // Every barrier below hands over LDS data only (lds_barrier): the state tile's stores are not
  // waited for, so the workgroup goes on with the readout while they drain.
  // The tile through a buffer resource: one offset register per lane, the row steps in scalars (the
  // addresses of sixteen loads and stores held in registers would cost a workgroup per CU).
  // Non-temporal: with the plain policy a single layer's states stay in the last-level cache from
  // one step to the next (39 us), but states that do not fit it, as in a stack of layers, take
  // 61 us against 50 for the non-temporal form on MI355X.
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(Sb, (short)0, DK * DV * 4, 0x00020000);
  const int soff = (16 * rg * DV + 4 * cg) * 4;
  v4f s[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(srs, soff, r * DV * 4, 2));

  const float* ub = a.u + (size_t)b * a.R;
  const int g = h / (a.Hv / a.Hk);
  float vv = 0.f, zz = 0.f, nwv = 0.f;
  double sq = 0.0, sk = 0.0;
  if (tid < DK) {
    // (the norm weight too: a load issued after the tile's stores would wait for them to complete)
    nwv = a.norm_w[tid];
    const float q = ub[g * DK + tid], k = ub[a.QK + g * DK + tid];
    qs[tid] = q;
    kks[tid] = k;
    sq = (double)q * q;
    sk = (double)k * k;
    vv = ub[2 * a.QK + h * DV + tid];
    zz = ub[a.C + h * DV + tid];
    if constexpr (PK) als[tid] = a.alpha[((size_t)b * a.Hv + h) * DK + tid];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sq += __shfl_xor(sq, o);
    sk += __shfl_xor(sk, o);
  }
  if (lane == 0) {
    dred[wave][0] = sq;
    dred[wave][1] = sk;
  }
  lds_barrier();
  // L2 norms in double, eps inside the sqrt (waves 0 and 1 hold the 128 rows)
  const float qn = (float)((double)a.q_scale / sqrt((dred[0][0] + dred[1][0]) + (double)a.eps_l2));
  const float kn = (float)(1.0 / sqrt((dred[0][1] + dred[1][1]) + (double)a.eps_l2));
  const float alpha = PK ? 0.f : a.alpha[(size_t)b * a.Hv + h], beta = a.beta[(size_t)b * a.Hv + h];

  // decay, then (decayed S)^T k for this thread's 4 columns over its 16 rows
  float kvp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float kr = kks[16 * rg + r] * kn;
    const float ar = PK ? als[16 * rg + r] : alpha;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[r][j] *= ar;
      kvp[j] = fmaf(s[r][j], kr, kvp[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) red[rg][4 * cg + j] = kvp[j];
  lds_barrier();
  if (tid < DV) {
    float kv = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) kv += red[i][tid];
    dl[tid] = beta * (vv - kv);
  }
  lds_barrier();
  // delta rule write, then the readout over the updated state
  float op[4] = {0.f, 0.f, 0.f, 0.f};
  float d4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) d4[j] = dl[4 * cg + j];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float kr = kks[16 * rg + r] * kn, qr = qs[16 * rg + r] * qn;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s[r][j] = fmaf(kr, d4[j], s[r][j]);
      op[j] = fmaf(s[r][j], qr, op[j]);
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, s[r]), srs, soff, r * DV * 4, 2);
#pragma unroll
  for (int j = 0; j < 4; ++j) red[rg][4 * cg + j] = op[j];
  lds_barrier();
  float o = 0.f, o2 = 0.f;
  if (tid < DV) {
#pragma unroll
    for (int i = 0; i < 8; ++i) o += red[i][tid];
    o2 = o * o;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) o2 += __shfl_xor(o2, off);
  if (lane == 0 && wave < 2) fred[wave] = o2;
  lds_barrier();
  float yv = 0.f;
  if (tid < DV) {
    const float inv = rsqrtf((fred[0] + fred[1]) / (float)DV + a.eps_rms);
    yv = nwv * o * inv * silu(zz);
  }
  // This head's 128 readout columns are one 128-column chunk of the out_proj input of sequence b:
  // split it into three int8 terms in the GEMM's fragment order (as k_bsplit does).
  float mx = fabsf(yv);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  lds_barrier();  // fred is reused
  if (lane == 0 && wave < 2) fred[wave] = mx;
  lds_barrier();
  float s1 = fmaxf(fred[0], fred[1]) * (1.0f / 127.0f);
  if (!(s1 > 0.f)) s1 = 1.0f;
  if (tid < DV) {
    const float inv1 = 1.0f / s1, s2 = s1 * (1.0f / 254.0f), inv2 = 1.0f / s2, inv3 = 254.0f / s2;
    int hq, mq, lq;
    split3(yv, inv1, s1, inv2, s2, inv3, hq, mq, lq);
    ybytes[0][tid] = (int8_t)hq;
    ybytes[1][tid] = (int8_t)mq;
    ybytes[2][tid] = (int8_t)lq;
  }
  lds_barrier();
  const int sb = b % NT;
  const size_t blk = (size_t)(b / NT) * a.Hv + h;  // column block of 64 sequences, chunk h
  if (tid < 3 * 8) {
    // 16 columns 16 p .. +15 of term t: k-step p / 4, 16-column group p % 4
    const int t = tid >> 3, p = tid & 7;
    const int ln = (sb & 15) + 16 * (p & 3), f = sb >> 4, ks2 = p >> 2;
    static_cast<v4i*>(a.xs)[blk * (3 * KSC * 4 * 64) + ((t * KSC + ks2) * 4 + f) * 64 + ln] =
        *reinterpret_cast<const v4i*>(&ybytes[t][16 * p]);
  }
  if (tid == 0) a.sc[blk * NT + sb] = s1;
}

template <int BITS, int MF, int NKS>
hipError_t go_bgemm(const BGemmArgs& a, hipStream_t st) {
  const dim3 grid(a.M / (64 * MF), a.K / (NKS * 64), (a.B + NT - 1) / NT);
  hipLaunchKernelGGL((k_bgemm<BITS, MF, NKS>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int BITS>
hipError_t bgemm_bits(const BGemmArgs& a, int mf, hipStream_t st) {
  const int nks = a.KR / 64;
  if (mf == 1) {
    if (nks == 16) return go_bgemm<BITS, 1, 16>(a, st);
    if (nks == 8) return go_bgemm<BITS, 1, 8>(a, st);
    if (nks == 4) return go_bgemm<BITS, 1, 4>(a, st);
  }
  return hipErrorInvalidValue;
}

// staged weights (4 K quarters of cpw chunks x 2 rt load instructions of 1 KB) or the padded quarter
// sums, history, taps, scales, sums of squares, spare
constexpr size_t bproj_lds_bytes(int rt, int cpw) {
  return sizeof(float) * ((cpw * 2 * rt * 1024 > 4 * NT * (16 * rt + 4) ? cpw * 2 * rt * 1024 : 4 * NT * (16 * rt + 4)) +
                          3 * NT * 16 * rt + 4 * 16 * rt + 64 + NT + 256);
}

template <int RT, int CPW>
hipError_t go_bproj(const BGemmArgs& g, const BEpiArgs& e, hipStream_t st) {
  constexpr size_t lds = bproj_lds_bytes(RT, CPW);
  static_assert(lds <= 160 * 1024, "");
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_bproj<RT, CPW>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  const dim3 grid((g.M + 16 * RT - 1) / (16 * RT), (g.B + NT - 1) / NT);
  hipLaunchKernelGGL((k_bproj<RT, CPW>), grid, dim3(768), lds, st, g, e);
  return hipGetLastError();
}

template <int RT>
hipError_t bproj_rt(const BGemmArgs& g, const BEpiArgs& e, hipStream_t st) {
  switch (g.K / (4 * KC)) {
    case 2: return go_bproj<RT, 2>(g, e, st);
    case 4: return go_bproj<RT, 4>(g, e, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool bgemm_shape_ok(int M, int K, int mf, int kr) {
  return M > 0 && K > 0 && mf == 1 && M % (64 * mf) == 0 && (kr == 256 || kr == 512 || kr == 1024) && K % kr == 0;
}

hipError_t launch_bsplit_row(const BSplitArgs& a, hipStream_t st) {
  if (a.K % 1024 || a.K > 8192 || a.act_stride % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bsplit_row, dim3(a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bsplit(const BSplitArgs& a, hipStream_t st) {
  if (a.K % KC) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_bsplit, dim3(a.K / KC, 4 * ((a.B + NT - 1) / NT)), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bgemm(const BGemmArgs& a, int bits, int mf, hipStream_t st) {
  if (!bgemm_shape_ok(a.M, a.K, mf, a.KR)) return hipErrorInvalidValue;
  return bits == 8 ? bgemm_bits<8>(a, mf, st) : bgemm_bits<4>(a, mf, st);
}

template <int BITS, int NRB, int KR>
hipError_t go_bgemm2(const BGemmArgs& a, hipStream_t st) {
  const dim3 grid(a.M / (64 * NRB), a.K / KR, (a.B + NT - 1) / NT);
  if (a.act) {
    if constexpr (BITS == 8 && KR == 256 && NRB >= 2)
      hipLaunchKernelGGL((k_bgemm2<BITS, NRB, KR, true>), grid, dim3(256 * NRB), 0, st, a);
    else
      return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((k_bgemm2<BITS, NRB, KR, false>), grid, dim3(256 * NRB), 0, st, a);
  }
  return hipGetLastError();
}

template <int BITS, int KR>
hipError_t bgemm2_kr(const BGemmArgs& a, int nrb, hipStream_t st) {
  if (nrb == 3) return go_bgemm2<BITS, 3, KR>(a, st);
  if (nrb == 2) return go_bgemm2<BITS, 2, KR>(a, st);
  if (nrb == 1) return go_bgemm2<BITS, 1, KR>(a, st);
  return hipErrorInvalidValue;
}

template <int BITS>
hipError_t bgemm2_bits(const BGemmArgs& a, int nrb, hipStream_t st) {
  if (a.KR == 512) return bgemm2_kr<BITS, 512>(a, nrb, st);
  if (a.KR == 256) return bgemm2_kr<BITS, 256>(a, nrb, st);
  return hipErrorInvalidValue;
}

bool bgemm2_shape_ok(int M, int K, int nrb, int kr) {
  return M > 0 && K > 0 && nrb >= 1 && nrb <= 3 && M % (64 * nrb) == 0 && (kr == 256 || kr == 512) && K % kr == 0;
}

hipError_t launch_bgemm2(const BGemmArgs& a, int bits, int nrb, hipStream_t st) {
  if (!bgemm2_shape_ok(a.M, a.K, nrb, a.KR)) return hipErrorInvalidValue;
  return bits == 8 ? bgemm2_bits<8>(a, nrb, st) : bgemm2_bits<4>(a, nrb, st);
}

hipError_t launch_tsplit(const TSplitArgs& a, hipStream_t st) {
  if (a.T < 1 || a.K < 4 || a.K % 4 || a.act_stride % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tsplit, dim3(a.T), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_tsplit_norm(const TSplitNormArgs& a, hipStream_t st) {
  if (a.sp.T < 1 || a.sp.K < 128 || a.sp.K % 128 || a.sp.K > 8192 || a.sp.act_stride % 4 || a.z_stride % 4 ||
      reinterpret_cast<uintptr_t>(a.z) % 16 || reinterpret_cast<uintptr_t>(a.sp.act) % 16)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tsplit_norm, dim3(a.sp.T), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bepi(const BEpiArgs& a, hipStream_t st) {
  const dim3 grid((a.M + 255) / 256, a.B);
  if (a.KS <= 4) hipLaunchKernelGGL(k_bepi<4>, grid, dim3(256), 0, st, a);
  else if (a.KS <= 8) hipLaunchKernelGGL(k_bepi<8>, grid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(k_bepi<16>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bstate(const BStateArgs& a, hipStream_t st) {
  if (a.alpha_per_key)
    hipLaunchKernelGGL(k_bstate<true>, dim3(a.Hv, a.B), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(k_bstate<false>, dim3(a.Hv, a.B), dim3(256), 0, st, a);
  return hipGetLastError();
}

// The whole-K projection (8-bit weights) takes K = 4 * CPW * 128 with CPW 2 or 4 (every wave two or
// four chunks) and row tiles of 48 rows when M leaves at least one workgroup per compute unit's worth
// of them, else of 32.
bool bproj_shape_ok(int M, int K, int* rt) {
  if (M <= 0 || K <= 0 || K % (4 * KC) || (K / (4 * KC) != 2 && K / (4 * KC) != 4)) return false;
  *rt = M >= 48 * 256 ? 3 : 2;
  return true;
}

hipError_t launch_bproj(const BGemmArgs& g, const BEpiArgs& e, int bits, int rt, hipStream_t st) {
  int want = 0;
  // (the history and the output move in 16-byte pieces: 4 rows)
  if (bits != 8 || !bproj_shape_ok(g.M, g.K, &want) || (rt != 2 && rt != 3) || (e.conv_w && e.C % 4) || g.M % 4 ||
      e.out_stride % 4)
    return hipErrorInvalidValue;
  return rt == 2 ? bproj_rt<2>(g, e, st) : bproj_rt<3>(g, e, st);
}

}  // namespace dn
