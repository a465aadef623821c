// HIP kernels of the gated-DeltaNet decode step for CDNA4 (gfx950).
//
// Steps (page "qwen36: run the DeltaNet layer end to end on the card", section "What the PR
// does", Backend paragraph): in_proj GEMV -> causal conv + SiLU with the history advancing ->
// per value head L2 norms (double, eps inside the sqrt) -> decay -> delta against the decayed
// state -> write-back -> out = q^T S over the updated state -> gated RMSNorm with silu(z) ->
// out_proj GEMV.
//
// GEMV arithmetic. The weights are exact small integers. The activation vector is split into
// three int8 terms, x ~= s1*(x0 + (x1 + x2/254)/254) with s1 = max|x|/127, so that each row's
// dot product is three exact int32 dot products (v_dot4_i32_i8 / sdot4) combined in double.
// The split leaves |x - xhat| <= s1/(2*254^2) per element, below 1e-7 of the dot product's
// magnitude for Gaussian activations (the level of fp32 rounding), and cuts the VALU work per
// weight byte from two instructions (convert + FMA) to three quarters.
#include <hip/hip_runtime.h>
#include <cmath>

#include "dn_internal.h"

namespace dn {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int sdot4(int a, int b, int c) { return __builtin_amdgcn_sdot4(a, b, c, false); }

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Workgroup barrier that waits only for the wave's LDS accesses (__syncthreads() would also wait
// for every outstanding global load, the weight rows requested ahead included).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Reductions over a 256-thread workgroup (4 waves). `buf` holds 4 elements; every thread
// gets the result. Fixed order, so results are run-to-run identical.
template <typename T>
__device__ __forceinline__ T block_sum(T v, T* buf) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) buf[wave] = v;
  __syncthreads();
  return (buf[0] + buf[1]) + (buf[2] + buf[3]);
}
__device__ __forceinline__ float block_max(float v, float* buf) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) buf[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(buf[0], buf[1]), fmaxf(buf[2], buf[3]));
}

// Position of column c in the staged int8 activations. For 4-bit weights each packed dword
// holds columns 8m..8m+7 as nibbles (low nibble first); masking gives the even columns in one
// dword and the odd columns in another, so the activations are staged even-first per group of 8.
template <int BITS>
__device__ __forceinline__ int x_pos(int c) {
  if (BITS == 8) return c;
  return (c & ~7) | ((c & 1) << 2) | ((c >> 1) & 3);
}

// ---------------------------------------------------------------------------------------------
// GEMV: one wave streams RB rows at a time; each lane loads NCH 16-byte chunks per row (chunk
// index lane + 64k), so one load instruction covers 1 KiB of one row. Grid-stride over rows.
// ---------------------------------------------------------------------------------------------
template <int BITS, int NCH, int RB>
__global__ __launch_bounds__(256) void k_gemv(const GemvArgs a) {
  extern __shared__ int smem[];  // staged x: three int8 terms, [cols] bytes each
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float hinv[64];
  const int b = blockIdx.y;
  const float* xb = a.x + (size_t)b * a.x_stride;

  // The input row (and, for a gated readout, its heads' partial sums of squares) is requested
  // first, then the wave's first RB weight rows: vector loads complete in order, so the staging
  // below waits only for the input while the weight rows' HBM latency overlaps it (its barriers
  // wait only for LDS).
  const int nchunk = (BITS == 8 ? a.cols : a.cols / 2) >> 4;
  const v4i* W = reinterpret_cast<const v4i*>(a.W);
  v4i w[RB][NCH];
  // (branch-free: an out-of-range piece reads piece 0 and is zeroed, so the compiler can count
  // the loads in flight exactly instead of waiting for all of them at the next use of any load)
  auto load_rows = [&](int r0) {
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int k = 0; k < NCH; ++k) {
        const int c = lane + 64 * k, r = r0 + i;
        const bool in = r < a.rows && c < nchunk;
        const v4i v = __builtin_nontemporal_load(&W[in ? (size_t)r * nchunk + c : 0]);
        w[i][k] = in ? v : v4i{0, 0, 0, 0};
      }
  };
  // 0. with head_ssq: x is a gated readout whose per-head RMS factors are still to be applied;
  // head h's factor from its head_nb (at most HNB) partial sums of squares, thread h
  constexpr int HNB = 16;
  const bool hn = a.head_ssq != nullptr;
  const int nheads = hn ? a.cols / a.head_dim : 0;
  float hp[HNB];
  {
    // (issued unconditionally, from x itself when there are no partials, and masked where they are
    // summed, so that no wait for them is placed before the loads below)
    const int nb = hn ? a.head_nb : 1;
    const float* p = hn ? a.head_ssq + ((size_t)b * nheads + (tid < nheads ? tid : 0)) * a.head_nb : xb;
#pragma unroll
    for (int k = 0; k < HNB; ++k) hp[k] = p[k < nb ? k : 0];
  }
  // 1. x into registers (XR values per thread, one read), its sum of squares (pre-norm) and
  // max |x| (split scale), reduced together
  constexpr int XR = (BITS == 8 ? 4 : 8) * NCH;  // cols <= 256 XR
  __shared__ float red2[4][2];
  float xr[XR];
#pragma unroll
  for (int m = 0; m < XR; ++m) {
    const int c = tid + 256 * m;
    const float v = xb[c < a.cols ? c : 0];
    xr[m] = c < a.cols ? v : 0.f;
  }
  load_rows((blockIdx.x * 4 + wave) * RB);
  if (hn) {
    if (tid < nheads) {
      float sp = 0.f;
#pragma unroll
      for (int k = 0; k < HNB; ++k) sp += k < a.head_nb ? hp[k] : 0.f;
      hinv[tid] = rsqrtf(sp / (float)a.head_dim + a.head_eps);
    }
    lds_sync();
#pragma unroll
    for (int m = 0; m < XR; ++m) {
      const int c = tid + 256 * m;
      if (c < a.cols) xr[m] *= hinv[c / a.head_dim];
    }
  }
  float ss = 0.f, mx = 0.f;
#pragma unroll
  for (int m = 0; m < XR; ++m) {
    ss = fmaf(xr[m], xr[m], ss);
    mx = fmaxf(mx, fabsf(xr[m]));
  }
  ss = wave_sum(ss);
  mx = wave_max(mx);
  if (lane == 0) {
    red2[wave][0] = ss;
    red2[wave][1] = mx;
  }
  lds_sync();
  ss = (red2[0][0] + red2[1][0]) + (red2[2][0] + red2[3][0]);
  mx = fmaxf(fmaxf(red2[0][1], red2[1][1]), fmaxf(red2[2][1], red2[3][1]));
  const float scale = a.prenorm ? rsqrtf(ss / (float)a.cols + a.eps) : 1.0f;
  float s1 = mx * scale * (1.0f / 127.0f);
  if (!(s1 > 0.f)) s1 = 1.0f;
  const float inv1 = 1.0f / s1, s2 = s1 * (1.0f / 254.0f), inv2 = 1.0f / s2;
  const float s3 = s2 * (1.0f / 254.0f), inv3 = 1.0f / s3;

  // 2. split x into three int8 terms, staged in LDS. Each term rounds by adding 1.5 * 2^23 to the
  // clamped quotient (ties to even, as rintf): the integer lands in the low mantissa bits, whose
  // low byte is the int8 term.
  int8_t* xh8 = reinterpret_cast<int8_t*>(smem);
  int8_t* xm8 = xh8 + a.cols;
  int8_t* xl8 = xm8 + a.cols;
  constexpr float BIAS = 12582912.0f;
  int sum_h = 0, sum_m = 0, sum_l = 0;
#pragma unroll
  for (int m = 0; m < XR; ++m) {
    const int c = tid + 256 * m;
    if (c < a.cols) {
      const float v = xr[m] * scale;
      const float th = __builtin_amdgcn_fmed3f(v * inv1, -127.f, 127.f) + BIAS, h = th - BIAS;
      const float r1 = fmaf(-s1, h, v);
      const float tm = __builtin_amdgcn_fmed3f(r1 * inv2, -127.f, 127.f) + BIAS, mm = tm - BIAS;
      const float r2 = fmaf(-s2, mm, r1);
      const float tl = __builtin_amdgcn_fmed3f(r2 * inv3, -127.f, 127.f) + BIAS;
      const int p = x_pos<BITS>(c);
      xh8[p] = (int8_t)__float_as_uint(th);
      xm8[p] = (int8_t)__float_as_uint(tm);
      xl8[p] = (int8_t)__float_as_uint(tl);
      if (BITS == 4) {
        sum_h += (int)h;
        sum_m += (int)mm;
        sum_l += (int)(tl - BIAS);
      }
    }
  }
  if (BITS == 4) {
    // three block sums in one pass over LDS
    sum_h = wave_sum(sum_h);
    sum_m = wave_sum(sum_m);
    sum_l = wave_sum(sum_l);
    __shared__ int redh[3][4];
    if (lane == 0) {
      redh[0][wave] = sum_h;
      redh[1][wave] = sum_m;
      redh[2][wave] = sum_l;
    }
    lds_sync();
    sum_h = (redh[0][0] + redh[0][1]) + (redh[0][2] + redh[0][3]);
    sum_m = (redh[1][0] + redh[1][1]) + (redh[1][2] + redh[1][3]);
    sum_l = (redh[2][0] + redh[2][1]) + (redh[2][2] + redh[2][3]);
  } else {
    lds_sync();
  }

  // 3. stream rows (the first RB are in flight already)
  const v4i* XH = reinterpret_cast<const v4i*>(xh8);
  const v4i* XM = reinterpret_cast<const v4i*>(xm8);
  const v4i* XL = reinterpret_cast<const v4i*>(xl8);
  const int wave_stride = gridDim.x * 4 * RB;
  for (int r0 = (blockIdx.x * 4 + wave) * RB; r0 < a.rows; r0 += wave_stride) {
    if (r0 != (blockIdx.x * 4 + wave) * RB) load_rows(r0);
    int ah[RB], am[RB], al[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) ah[i] = am[i] = al[i] = 0;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int c = lane + 64 * k;
      if (c < nchunk) {
        if (BITS == 8) {
          const v4i xh = XH[c], xm = XM[c], xl = XL[c];
#pragma unroll
          for (int i = 0; i < RB; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ah[i] = sdot4(w[i][k][e], xh[e], ah[i]);
              am[i] = sdot4(w[i][k][e], xm[e], am[i]);
              al[i] = sdot4(w[i][k][e], xl[e], al[i]);
            }
          }
        } else {
          const v4i xh0 = XH[2 * c], xh1 = XH[2 * c + 1], xm0 = XM[2 * c], xm1 = XM[2 * c + 1];
          const v4i xl0 = XL[2 * c], xl1 = XL[2 * c + 1];
          const int xhE[4] = {xh0[0], xh0[2], xh1[0], xh1[2]}, xhO[4] = {xh0[1], xh0[3], xh1[1], xh1[3]};
          const int xmE[4] = {xm0[0], xm0[2], xm1[0], xm1[2]}, xmO[4] = {xm0[1], xm0[3], xm1[1], xm1[3]};
          const int xlE[4] = {xl0[0], xl0[2], xl1[0], xl1[2]}, xlO[4] = {xl0[1], xl0[3], xl1[1], xl1[3]};
#pragma unroll
          for (int i = 0; i < RB; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // nibble n (two's complement w) xor 8 gives w + 8 in 0..15
              const unsigned p = (unsigned)w[i][k][e] ^ 0x88888888u;
              const int lo = (int)(p & 0x0F0F0F0Fu), hi = (int)((p >> 4) & 0x0F0F0F0Fu);
              ah[i] = sdot4(lo, xhE[e], ah[i]);
              ah[i] = sdot4(hi, xhO[e], ah[i]);
              am[i] = sdot4(lo, xmE[e], am[i]);
              am[i] = sdot4(hi, xmO[e], am[i]);
              al[i] = sdot4(lo, xlE[e], al[i]);
              al[i] = sdot4(hi, xlO[e], al[i]);
            }
          }
        }
      }
    }
    float mine = 0.f;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      int th = wave_sum(ah[i]), tm = wave_sum(am[i]), tl = wave_sum(al[i]);
      if (BITS == 4) {
        th -= 8 * sum_h;
        tm -= 8 * sum_m;
        tl -= 8 * sum_l;
      }
      const float dot = (float)((double)s1 * ((double)th + ((double)tm + (double)tl * (1.0 / 254.0)) * (1.0 / 254.0)));
      if (lane == i) mine = dot;
    }
    const int r = r0 + lane;
    if (lane < RB && r < a.rows) {
      const float u = a.s[r] * mine;
      float* ob = a.out + (size_t)b * a.out_stride;
      if (a.conv_w != nullptr && r < a.C) {
        const int K = a.K;
        const float* cw = a.conv_w + (size_t)r * K;
        float* rg = a.ring + (size_t)b * (K - 1) * a.C + r;
        float hist[3] = {0.f, 0.f, 0.f};
        float acc = cw[K - 1] * u;
#pragma unroll
        for (int j = 0; j < 3; ++j)
          if (j < K - 1) {
            hist[j] = rg[(size_t)j * a.C];
            acc = fmaf(cw[j], hist[j], acc);
          }
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (j + 1 < K - 1) rg[(size_t)j * a.C] = hist[j + 1];
        if (K > 1) rg[(size_t)(K - 2) * a.C] = u;
        ob[r] = silu(acc);
      } else {
        ob[r] = u;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Value head: one workgroup per (head, sequence). Column chunks of 64 (one column per lane);
// the four waves split the key rows i = wave + 4t.
// ---------------------------------------------------------------------------------------------
template <int DKMAX>
__global__ __launch_bounds__(256) void k_head(const HeadArgs a) {
  constexpr int TPR = DKMAX / 4;  // key rows per thread
  __shared__ float qs[256], ks[256], os[256], als[256];
  __shared__ float red[4][64];
  __shared__ double redd[4];
  __shared__ float redf[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, b = blockIdx.y;
  const int g = h / (a.Hv / a.Hk);
  const int dk = a.dk, dv = a.dv, QK = a.Hk * dk;
  const float* ub = a.u + (size_t)b * a.R;
  const float* q = ub + (size_t)g * dk;
  const float* k = ub + QK + (size_t)g * dk;
  const float* v = ub + 2 * QK + (size_t)h * dv;
  const float* z = ub + a.C + (size_t)h * dv;

  // L2 norms in double, eps inside the sqrt
  double sq = 0.0, sk = 0.0;
  const float* ah = a.alpha + ((size_t)b * a.Hv + h) * (a.alpha_per_key ? dk : 1);
  for (int i = tid; i < dk; i += 256) {
    const float qv = q[i], kv = k[i];
    qs[i] = qv;
    ks[i] = kv;
    als[i] = ah[a.alpha_per_key ? i : 0];
    sq += (double)qv * qv;
    sk += (double)kv * kv;
  }
  sq = block_sum(sq, redd);
  sk = block_sum(sk, redd);
  const float qn = (float)((double)a.q_scale / sqrt(sq + (double)a.eps_l2));
  const float kn = (float)(1.0 / sqrt(sk + (double)a.eps_l2));
  __syncthreads();
  for (int i = tid; i < dk; i += 256) {
    qs[i] *= qn;
    ks[i] *= kn;
  }
  __syncthreads();

  const float beta = a.beta[(size_t)b * a.Hv + h];
  float* S = a.S + ((size_t)b * a.Hv + h) * dk * dv;
  for (int j0 = 0; j0 < dv; j0 += 64) {
    const int j = j0 + lane;
    const bool jv = j < dv;
    float s[TPR];
    float kvp = 0.f;
#pragma unroll
    for (int t = 0; t < TPR; ++t) {
      const int i = wave + 4 * t;
      s[t] = 0.f;
      if (i < dk && jv) {
        s[t] = als[i] * S[(size_t)i * dv + j];
        kvp = fmaf(s[t], ks[i], kvp);
      }
    }
    red[wave][lane] = kvp;
    __syncthreads();
    const float kv = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
    __syncthreads();
    const float delta = jv ? beta * (v[j] - kv) : 0.f;
    float op = 0.f;
#pragma unroll
    for (int t = 0; t < TPR; ++t) {
      const int i = wave + 4 * t;
      if (i < dk && jv) {
        s[t] = fmaf(ks[i], delta, s[t]);
        S[(size_t)i * dv + j] = s[t];
        op = fmaf(s[t], qs[i], op);
      }
    }
    red[wave][lane] = op;
    __syncthreads();
    const float o = (red[0][lane] + red[1][lane]) + (red[2][lane] + red[3][lane]);
    if (wave == 0 && jv) os[j] = o;
    __syncthreads();
  }

  // gated RMSNorm over dv with silu(z)
  float ssq = 0.f;
  for (int j = tid; j < dv; j += 256) ssq = fmaf(os[j], os[j], ssq);
  ssq = block_sum(ssq, redf);
  const float inv = rsqrtf(ssq / (float)dv + a.eps_rms);
  float* yb = a.y + (size_t)b * a.Hv * dv + (size_t)h * dv;
  for (int j = tid; j < dv; j += 256) yb[j] = a.norm_w[j] * os[j] * inv * silu(z[j]);
}

// ---------------------------------------------------------------------------------------------
// Value head, split by columns: one workgroup per (head, block of 16 value columns, sequence), so
// that a single sequence's states stream through many compute units (one workgroup per head
// leaves most of them idle). The columns of a head's state are independent but for the gated
// RMSNorm, which needs the head's sum of o^2: each block writes its columns' w o silu(z) and its
// partial sum, and the out_proj GEMV applies the head's 1/rms when it stages its input.
// Thread t: column 16 cb + t % 16, key rows t / 16 + 16 m.
// ---------------------------------------------------------------------------------------------
template <int DKMAX>
__global__ __launch_bounds__(256) void k_head_cols(const HeadArgs a) {
  constexpr int RPT = DKMAX / 16;  // key rows per thread
  __shared__ float qs[DKMAX], ks[DKMAX], als[DKMAX];
  __shared__ float red[16][17];
  __shared__ double redd[4];
  const int tid = threadIdx.x, jl = tid & 15, rg = tid >> 4;
  const int nb = a.dv / 16, h = blockIdx.x / nb, cb = blockIdx.x % nb, b = blockIdx.y;
  const int g = h / (a.Hv / a.Hk);
  const int dk = a.dk, dv = a.dv, QK = a.Hk * dk, j = 16 * cb + jl;
  const float* ub = a.u + (size_t)b * a.R;
  const float* q = ub + (size_t)g * dk;
  const float* k = ub + QK + (size_t)g * dk;
  const float* ah = a.alpha + ((size_t)b * a.Hv + h) * (a.alpha_per_key ? dk : 1);

  // the state block's loads first (their latency under the norms): rows rg + 16 m, column j
  float* S = a.S + ((size_t)b * a.Hv + h) * dk * dv + j;
  float s[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + 16 * m;
    s[m] = i < dk ? S[(size_t)i * dv] : 0.f;
  }
  // L2 norms in double, eps inside the sqrt
  double sq = 0.0, sk = 0.0;
  for (int i = tid; i < dk; i += 256) {
    const float qv = q[i], kv = k[i];
    qs[i] = qv;
    ks[i] = kv;
    als[i] = ah[a.alpha_per_key ? i : 0];
    sq += (double)qv * qv;
    sk += (double)kv * kv;
  }
  sq = block_sum(sq, redd);
  sk = block_sum(sk, redd);
  const float qn = (float)((double)a.q_scale / sqrt(sq + (double)a.eps_l2));
  const float kn = (float)(1.0 / sqrt(sk + (double)a.eps_l2));

  // decay; (decayed S)^T k^ of column j over this thread's rows, then over the row groups
  float kvp = 0.f;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + 16 * m;
    if (i < dk) {
      s[m] *= als[i];
      kvp = fmaf(s[m], ks[i] * kn, kvp);
    }
  }
  red[rg][jl] = kvp;
  __syncthreads();
  float kv = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) kv += red[r][jl];
  const float delta = a.beta[(size_t)b * a.Hv + h] * (ub[2 * QK + (size_t)h * dv + j] - kv);
  // delta rule and the readout over the updated state
  float op = 0.f;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + 16 * m;
    if (i < dk) {
      s[m] = fmaf(ks[i] * kn, delta, s[m]);
      S[(size_t)i * dv] = s[m];
      op = fmaf(s[m], qs[i] * qn, op);
    }
  }
  __syncthreads();  // every read of red is done
  red[rg][jl] = op;
  __syncthreads();
  if (tid < 16) {
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) o += red[r][tid];
    const float z = ub[a.C + (size_t)h * dv + j];
    a.y[(size_t)b * a.Hv * dv + (size_t)h * dv + j] = a.norm_w[j] * o * silu(z);
    float o2 = o * o;
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) o2 += __shfl_xor(o2, off, 16);
    if (tid == 0) a.ssq[((size_t)b * a.Hv + h) * nb + cb] = o2;
  }
}

// ---------------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------------
template <int BITS, int NCH, int RB>
static hipError_t go_gemv(const GemvArgs& a, hipStream_t st) {
  const int rows_per_block = 4 * RB;
  int grid = (a.rows + rows_per_block - 1) / rows_per_block;
  if (grid > 2048) grid = 2048;
  const size_t lds = 3 * (size_t)a.cols;
  hipLaunchKernelGGL((k_gemv<BITS, NCH, RB>), dim3(grid, a.batch), dim3(256), lds, st, a);
  return hipGetLastError();
}

// rows per wave (RB) by 16-byte chunks per lane and row (NCH): 8 KiB of weights in flight per wave
// for rows of up to 2048 and 4096 bytes (measured against 16 KiB: 48-value-head stack 915 -> 871 us per
// token, heads of 256 836 -> 756 us; a row is reduced by one wave either way, so results are the same)
#ifndef DN_GEMV_RB2
#define DN_GEMV_RB2 4
#endif
#ifndef DN_GEMV_RB4
#define DN_GEMV_RB4 2
#endif
#ifndef DN_GEMV_RB8
#define DN_GEMV_RB8 2
#endif
template <int BITS>
static hipError_t gemv_bits(const GemvArgs& a, hipStream_t st) {
  const int nchunk = (BITS == 8 ? a.cols : a.cols / 2) >> 4;
  const int nch = (nchunk + 63) / 64;
  if (nch <= 1) return go_gemv<BITS, 1, 8>(a, st);
  if (nch <= 2) return go_gemv<BITS, 2, DN_GEMV_RB2>(a, st);
  if (nch <= 4) return go_gemv<BITS, 4, DN_GEMV_RB4>(a, st);
  if (nch <= 8) return go_gemv<BITS, 8, DN_GEMV_RB8>(a, st);
  if (nch <= 16) return go_gemv<BITS, 16, 1>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_gemv(const GemvArgs& a, int bits, hipStream_t st) {
  // the input row is held in registers, at most 256 (4 NCH or, 4-bit, 8 NCH) columns per thread;
  // a gated readout's head factors come from at most 16 partial sums for each of at most 64 heads
  if (a.cols > 16384) return hipErrorInvalidValue;
  if (a.head_ssq && (a.head_nb > 16 || a.head_dim < 1 || a.cols / a.head_dim > 64)) return hipErrorInvalidValue;
  return bits == 8 ? gemv_bits<8>(a, st) : gemv_bits<4>(a, st);
}

template <int DKMAX>
static hipError_t go_head(const HeadArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_head<DKMAX>), dim3(a.Hv, a.batch), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int DKMAX>
static hipError_t go_head_cols(const HeadArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_head_cols<DKMAX>), dim3(a.Hv * (a.dv / 16), a.batch), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_head(const HeadArgs& a, hipStream_t st) {
  if (a.ssq) {
    if (a.dv % 16 || a.dk % 16) return hipErrorInvalidValue;
    if (a.dk <= 64) return go_head_cols<64>(a, st);
    if (a.dk <= 128) return go_head_cols<128>(a, st);
    if (a.dk <= 256) return go_head_cols<256>(a, st);
    return hipErrorInvalidValue;
  }
  if (a.dk <= 16) return go_head<16>(a, st);
  if (a.dk <= 32) return go_head<32>(a, st);
  if (a.dk <= 64) return go_head<64>(a, st);
  if (a.dk <= 128) return go_head<128>(a, st);
  if (a.dk <= 256) return go_head<256>(a, st);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------------------------
// Gates on the card (DN_GATES_ON_DEVICE): one workgroup per input row n. The row is staged in LDS
// (RMS-normalised when asked), each wave takes gate rows w, w+4, ... and reduces its fp32 dot
// product; row h < Hv gives alpha[n][h], row Hv + h gives beta[n][h].
// ---------------------------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(256) void k_gates(const GateArgs a) {
  extern __shared__ float xr[];  // [D]
  __shared__ float redf[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = blockIdx.x, D = a.D;
  const float* xb = a.x + (size_t)n * a.x_stride;
  float ss = 0.f;
  for (int c = tid; c < D; c += 256) {
    const float v = xb[c];
    xr[c] = v;
    ss = fmaf(v, v, ss);
  }
  ss = block_sum(ss, redf);  // its barriers also publish xr
  const float inv = a.prenorm ? rsqrtf(ss / (float)D + a.eps) : 1.0f;
  constexpr int COLS = BITS == 8 ? 16 : 32;  // columns per 16-byte chunk
  const size_t rowbytes = BITS == 8 ? (size_t)D : (size_t)D / 2;
  for (int r = wave; r < 2 * a.Hv; r += 4) {
    const uint8_t* wr = static_cast<const uint8_t*>(a.W) + (size_t)r * rowbytes;
    float acc = 0.f;
    for (int c0 = COLS * lane; c0 < D; c0 += 64 * COLS) {
      const v4i w = *reinterpret_cast<const v4i*>(wr + (BITS == 8 ? c0 : c0 / 2));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned p = (unsigned)w[e];
        if (BITS == 8) {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc = fmaf((float)(int8_t)(p >> (8 * q)), xr[c0 + 4 * e + q], acc);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int nib = (int)((p >> (4 * q)) & 15u);
            acc = fmaf((float)((nib ^ 8) - 8), xr[c0 + 8 * e + q], acc);
          }
        }
      }
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      const float u = a.s[r] * inv * acc;
      if (r < a.Hv) a.alpha[(size_t)n * a.Hv + r] = dn_gate_alpha(u, a.a_log[r], a.a_bias[r]);
      else a.beta[(size_t)n * a.Hv + (r - a.Hv)] = dn_gate_beta(u);
    }
  }
}

hipError_t launch_gates(const GateArgs& a, int bits, hipStream_t st) {
  if (a.N < 1 || a.D < 1 || a.D > 16384 || a.D % (bits == 8 ? 16 : 32)) return hipErrorInvalidValue;
  const size_t lds = sizeof(float) * a.D;
  // the widest rows (64 KiB of x) with the kernel's static LDS exceed the default per-launch limit
  const void* fn = bits == 8 ? reinterpret_cast<const void*>(&k_gates<8>) : reinterpret_cast<const void*>(&k_gates<4>);
  if (lds > 48 * 1024)
    if (hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds); e != hipSuccess)
      return e;
  if (bits == 8) hipLaunchKernelGGL(k_gates<8>, dim3(a.N), dim3(256), lds, st, a);
  else hipLaunchKernelGGL(k_gates<4>, dim3(a.N), dim3(256), lds, st, a);
  return hipGetLastError();
}

// Buffer 0 made current (see launch_persist_settle): the copy runs only if buffer 1 is current.
__global__ void k_settle_copy(const float* __restrict__ s1, float* __restrict__ s0, size_t n_s,
                              const float* __restrict__ r1, float* __restrict__ r0, size_t n_ring, const Ctl* ctl) {
  if (!(ctl->parity & 1u)) return;
  const size_t step = (size_t)gridDim.x * blockDim.x;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n_s; e += step) s0[e] = s1[e];
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n_ring; e += step) r0[e] = r1[e];
}
__global__ void k_settle_flag(Ctl* ctl) {
  if (threadIdx.x == 0) ctl->parity = 0u;
}

hipError_t launch_persist_settle(float* const S[2], float* const ring[2], size_t n_s, size_t n_ring, Ctl* ctl,
                                 hipStream_t st) {
  hipLaunchKernelGGL(k_settle_copy, dim3(1024), dim3(256), 0, st, S[1], S[0], n_s, ring[1], ring[0], n_ring, ctl);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(k_settle_flag, dim3(1), dim3(64), 0, st, ctl);
  return hipGetLastError();
}

}  // namespace dn
