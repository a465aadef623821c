// Prefill: a prompt of T tokens of one sequence through a layer, with the recurrence taken in
// chunks of 64 tokens. The per-token step is the one of page "qwen36: run the DeltaNet layer end to
// end on the card", section "What the PR does", Backend paragraph (in_proj, conv + SiLU with the
// history advancing, L2 norms of q and k with eps inside the sqrt, decay, delta rule against the
// decayed state, readout over the updated state, gated RMSNorm with silu(z), out_proj); the page
// keeps a prompt (more than one token) on the CPU, and this file is that prompt pass on the card.
//
// The projections are the batched path's int8 GEMMs with the tokens as the columns. This file
// holds the parts that differ from decode:
//  * k_pconv: the in_proj epilogue, with the causal conv running along the tokens (the history
//    supplies the values before token 0).
//  * k_pintra + k_pscan: the gated delta rule over a chunk of tokens j = 0..63 with the state S0
//    at its start. With g_j the product of the decays up to token j of the chunk, the step's
//    corrections d_j = beta_j (v_j - (decayed state)^T k_j) satisfy
//        d_j + sum_{m<j} beta_j (g_j / g_m) (k_j . k_m) d_m = beta_j (v_j - g_j S0^T k_j),
//    a unit lower-triangular system (I + A) D = diag(beta) (V - diag(g) K S0). With
//    Tm = (I + A)^-1, W = Tm diag(beta g) K and Uv = Tm diag(beta) V, D = Uv - W S0. The readout
//    over the updated state is o_j = g_j S0^T q_j + sum_{m<=j} (g_j / g_m) (q_j . k_m) d_m, and the
//    state after the chunk is g_last S0 + sum_m (g_last / g_m) k_m d_m^T. This is the per-token
//    step rewritten, not an approximation: it agrees with it up to rounding.
//    k_pintra computes the parts that do not depend on S0 (Tm, W, Uv, the decayed q and k, the
//    masked q.k products) for every (head, chunk) in parallel; k_pscan carries the state through
//    the chunks for one (head, 16 value columns), the columns of S being independent.
//  * k_pnorm: the gated RMSNorm of every (token, head).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "dn_internal.h"

namespace dn {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int DK = 128, DV = 128, CT = PF_CT;
constexpr int OFF_W = 0, OFF_UV = CT * DK, OFF_QG = 2 * CT * DK, OFF_KT = 3 * CT * DK, OFF_P = 4 * CT * DK,
              OFF_G = 4 * CT * DK + CT * CT;
constexpr int TR = 32;  // tokens per thread in k_pconv
constexpr int LD = DK + 4;  // padded LDS row of 128 floats (keeps 16-byte alignment)

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

// Workgroup barrier that waits only for this wave's LDS accesses. A __syncthreads() also waits for
// every outstanding global access, here the readout's stores of the chunk; the scan's barriers
// order LDS data between waves and no global data.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float prenorm_of(const PConvArgs& a, int t) {
  if (!a.prenorm) return 1.0f;
  float ss = 0.f;
  for (int c = 0; c < a.NC; ++c) ss += a.ssq[(size_t)t * a.NC + c];
  return rsqrtf(ss / (float)a.K + a.eps);
}

// One thread per (row, run of TR tokens): pre-conv values from the K-range partial sums in a fixed
// order (all of the run's loads issued before any store), the conv over a window slid along the
// run, SiLU; the thread whose run ends the prompt writes the new history.
__global__ __launch_bounds__(256) void k_pconv(const PConvArgs a) {
  __shared__ float pn[TR];
  const int r = blockIdx.x * 256 + threadIdx.x;
  const int t0 = blockIdx.y * TR, nt = min(TR, a.T - t0);
  if ((int)threadIdx.x < nt) pn[threadIdx.x] = prenorm_of(a, t0 + threadIdx.x);
  __syncthreads();
  if (r >= a.M) return;
  const float sr = a.s[r];
  const float* __restrict__ part = a.part;
  float* __restrict__ out = a.out;
  auto pre = [&](int t, float f) {
    if (a.terms) {
      // exact sums of the three terms, folded in double with the token's split scale
      const size_t plane = (size_t)a.T * a.M, at = (size_t)t * a.M + r;
      const int d0 = a.terms[at], d1 = a.terms[plane + at], d2 = a.terms[2 * plane + at];
      return sr * f * (float)((double)a.s1[t] * ((double)d0 + ((double)d1 + (double)d2 * (1.0 / 254.0)) * (1.0 / 254.0)));
    }
    float pv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) pv[k] = k < a.KS ? part[((size_t)k * a.T + t) * a.M + r] : 0.f;
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < a.KS) sum += pv[k];
    for (int k = 4; k < a.KS; ++k) sum += part[((size_t)k * a.T + t) * a.M + r];
    return sr * f * sum;
  };
  float u[TR];
#pragma unroll
  for (int i = 0; i < TR; ++i) u[i] = i < nt ? pre(t0 + i, pn[i]) : 0.f;
  if (r >= a.C) {  // z rows: no conv
#pragma unroll
    for (int i = 0; i < TR; ++i)
      if (i < nt) out[(size_t)(t0 + i) * a.M + r] = u[i];
    return;
  }
  const int K = a.Kc;
  float w[4], hist[3] = {0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = j < K ? a.conv_w[(size_t)r * K + j] : 0.f;
  // hist[j]: pre-conv value of token t0 - (K-1) + j (oldest first); negative tokens from the history
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < K - 1) {
      const int tok = t0 - (K - 1) + j;
      hist[j] = tok >= 0 ? pre(tok, prenorm_of(a, tok)) : a.ring_in[(size_t)(tok + K - 1) * a.C + r];
    }
#pragma unroll
  for (int i = 0; i < TR; ++i) {
    if (i < nt) {
      float acc = w[K - 1] * u[i];
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < K - 1) acc = fmaf(w[j], hist[j], acc);
      out[(size_t)(t0 + i) * a.M + r] = silu(acc);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (j + 1 < K - 1) hist[j] = hist[j + 1];
      if (K > 1) hist[K - 2] = u[i];
    }
  }
  if (t0 + nt == a.T)
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < K - 1) a.ring_out[(size_t)j * a.C + r] = hist[j];
}

typedef int pc_v4i __attribute__((ext_vector_type(4)));

// k_pconv on the library GEMM's exact term sums, four adjacent rows per thread: 16-byte loads and
// stores, and every load unconditional (a token past the prompt reads the last token's row and is
// not stored), so the loads of a run of tokens are all in flight together.
constexpr int TR4 = 16;
__global__ __launch_bounds__(256) void k_pconv4(const PConvArgs a) {
  __shared__ float pn[TR4 + 3];  // pre-norm factors of tokens t0 - 3 .. t0 + TR4 - 1
  const int r = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int t0 = blockIdx.y * TR4, nt = min(TR4, a.T - t0);
  if ((int)threadIdx.x < TR4 + 3) {
    const int tok = t0 - 3 + (int)threadIdx.x;
    pn[threadIdx.x] = tok >= 0 && tok < a.T ? prenorm_of(a, tok) : 0.f;
  }
  __syncthreads();
  if (r >= a.M) return;
  float sr[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sr[e] = a.s[r + e];
  const size_t plane = (size_t)a.T * a.M;
  auto pre4 = [&](int t, float f, float (&o)[4]) {
    const size_t at = (size_t)t * a.M + r;
    const pc_v4i d0 = *reinterpret_cast<const pc_v4i*>(a.terms + at);
    const pc_v4i d1 = *reinterpret_cast<const pc_v4i*>(a.terms + plane + at);
    const pc_v4i d2 = *reinterpret_cast<const pc_v4i*>(a.terms + 2 * plane + at);
    const double s1 = (double)a.s1[t];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = sr[e] * f * (float)(s1 * ((double)d0[e] + ((double)d1[e] + (double)d2[e] * (1.0 / 254.0)) * (1.0 / 254.0)));
  };
  float u[TR4][4];
#pragma unroll
  for (int i = 0; i < TR4; ++i) pre4(min(t0 + i, a.T - 1), pn[3 + i], u[i]);
  if (r >= a.C) {  // z rows: no conv
#pragma unroll
    for (int i = 0; i < TR4; ++i)
      if (i < nt) *reinterpret_cast<v4f*>(a.out + (size_t)(t0 + i) * a.M + r) = v4f{u[i][0], u[i][1], u[i][2], u[i][3]};
    return;
  }
  const int K = a.Kc;
  float w[4][4], hist[3][4] = {};
#pragma unroll
  for (int e = 0; e < 4; ++e)
#pragma unroll
    for (int j = 0; j < 4; ++j) w[e][j] = j < K ? a.conv_w[(size_t)(r + e) * K + j] : 0.f;
  // hist[j]: pre-conv values of token t0 - (K-1) + j (oldest first); negative tokens from the history
#pragma unroll
  for (int j = 0; j < 3; ++j)
    if (j < K - 1) {
      const int tok = t0 - (K - 1) + j;
      if (tok >= 0) {
        pre4(tok, pn[3 - (K - 1) + j], hist[j]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) hist[j][e] = a.ring_in[(size_t)(tok + K - 1) * a.C + r + e];
      }
    }
#pragma unroll
  for (int i = 0; i < TR4; ++i) {
    if (i < nt) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float acc = w[e][K - 1] * u[i][e];
#pragma unroll
        for (int j = 0; j < 3; ++j)
          if (j < K - 1) acc = fmaf(w[e][j], hist[j][e], acc);
        y[e] = silu(acc);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          if (j + 1 < K - 1) hist[j][e] = hist[j + 1][e];
        if (K > 1) hist[K - 2][e] = u[i][e];
      }
      *reinterpret_cast<v4f*>(a.out + (size_t)(t0 + i) * a.M + r) = v4f{y[0], y[1], y[2], y[3]};
    }
  }
  if (t0 + nt == a.T)
#pragma unroll
    for (int j = 0; j < 3; ++j)
      if (j < K - 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) a.ring_out[(size_t)j * a.C + r + e] = hist[j][e];
}

// One workgroup per (value head, chunk): the chunk terms that do not depend on the incoming state.
// The 64 x 64 and 64 x 128 products run on the fp32 matrix cores (lane layout and permuted sum
// index as in k_pscan); the unit lower-triangular solve runs in the first wave (lane = column)
// while the other three form the masked q.k products.
__global__ __launch_bounds__(256) void k_pintra(const PIntraArgs a) {
  __shared__ __attribute__((aligned(16))) float sQ[CT][LD], sK[CT][LD], sV[CT][LD];
  __shared__ float sA[CT][CT + 1];  // A, then Tm = (I + A)^-1 in place
  __shared__ double slg[CT];
  __shared__ float sb[CT], sbg[CT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int h = blockIdx.x, c = blockIdx.y;
  const int g = h / (a.Hv / a.Hk);
  const int t0 = c * CT, nj = min(CT, a.T - t0);
  float* out = a.cw + ((size_t)h * a.NCH + c) * PF_CHUNK_FLOATS;

  // q, k (L2-normalised, norms accumulated in double, eps inside the sqrt) and v of the chunk's
  // tokens; four threads per token, rows of tokens past the prompt are zero
  {
    const int j = tid >> 2, p = tid & 3;
    const bool live = j < nj;
    const float* ur = a.u + (size_t)(t0 + (live ? j : 0)) * a.R;
    v4f qv[8], kv[8], vv[8];
    double sq = 0.0, sk = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int col = 4 * (p + 4 * e);
      const v4f z4 = {0.f, 0.f, 0.f, 0.f};
      qv[e] = live ? *reinterpret_cast<const v4f*>(ur + g * DK + col) : z4;
      kv[e] = live ? *reinterpret_cast<const v4f*>(ur + a.QK + g * DK + col) : z4;
      vv[e] = live ? *reinterpret_cast<const v4f*>(ur + 2 * a.QK + h * DV + col) : z4;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        sq += (double)qv[e][q] * qv[e][q];
        sk += (double)kv[e][q] * kv[e][q];
      }
    }
    sq += __shfl_xor(sq, 1);
    sq += __shfl_xor(sq, 2);
    sk += __shfl_xor(sk, 1);
    sk += __shfl_xor(sk, 2);
    const float qn = (float)((double)a.q_scale / sqrt(sq + (double)a.eps_l2));
    const float kn = (float)(1.0 / sqrt(sk + (double)a.eps_l2));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int col = 4 * (p + 4 * e);
      *reinterpret_cast<v4f*>(&sQ[j][col]) = qv[e] * qn;
      *reinterpret_cast<v4f*>(&sK[j][col]) = kv[e] * kn;
      *reinterpret_cast<v4f*>(&sV[j][col]) = vv[e];
    }
  }
  // gates; slg = running sum of log decay within the chunk, in double so that the difference of
  // two sums (the log of the decay between two tokens) keeps fp32 accuracy however strong the
  // decays are; a decay of 0 is clamped to e^-80 (below 1e-34, so what it multiplies vanishes)
  if (wave == 0) {
    const bool live = lane < nj;
    const size_t gi = (size_t)(t0 + lane) * a.gstride + h;
    const float al = live ? a.alpha[gi] : 1.0f;
    const float be = live ? a.beta[gi] : 0.0f;
    double lg = (double)fmaxf(logf(al), -80.0f);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double v = __shfl_up(lg, o);
      if (lane >= o) lg += v;
    }
    slg[lane] = lg;
    sb[lane] = be;
    sbg[lane] = be * expf((float)lg);
  }
  __syncthreads();

  // decayed q rows, k rows weighted by the decay to the chunk's end, the chunk's total decay
  {
    const double lgl = slg[nj - 1];
    for (int e = tid; e < CT * (DK / 4); e += 256) {
      const int j = e / (DK / 4), i4 = (e % (DK / 4)) * 4;
      const v4f q = *reinterpret_cast<const v4f*>(&sQ[j][i4]), k = *reinterpret_cast<const v4f*>(&sK[j][i4]);
      *reinterpret_cast<v4f*>(out + OFF_QG + j * DK + i4) = q * expf((float)slg[j]);
      *reinterpret_cast<v4f*>(out + OFF_KT + j * DK + i4) = j < nj ? k * expf((float)(lgl - slg[j])) : v4f{0.f, 0.f, 0.f, 0.f};
    }
    if (tid == 0) out[OFF_G] = expf((float)lgl);
  }

  // 64 x 64 tile (rt, ct) of X K^T for X = sQ or sK (sum over 128 columns, permuted)
  auto tile_xk = [&](const float (*X)[LD], int rt, int ct) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 32; ++st)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(X[16 * rt + li][32 * lk + st], sK[16 * ct + li][32 * lk + st], acc,
                                                 0, 0, 0);
    return acc;
  };
  // A = strictly lower part of diag(beta) (g_j/g_m) K K^T: wave w forms row tile w
  for (int ct = 0; ct < 4; ++ct) {
    const v4f gt = ct <= wave ? tile_xk(sK, wave, ct) : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = 16 * wave + 4 * lk + v, m = 16 * ct + li;
      sA[j][m] = m < j ? sb[j] * expf((float)(slg[j] - slg[m])) * gt[v] : 0.f;
    }
  }
  __syncthreads();

  if (wave == 0) {
    // Tm = (I + A)^-1 by forward substitution; lane `col` solves column col, then Tm overwrites A
    const int col = lane;
    float tc[CT];
#pragma unroll
    for (int j = 0; j < CT; ++j) {
      // four interleaved partial sums, so each row's dependent chain is a quarter as long
      float v[4] = {j == col ? 1.0f : 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < j; ++m) v[m & 3] = fmaf(-sA[j][m], tc[m], v[m & 3]);
      tc[j] = (v[0] + v[1]) + (v[2] + v[3]);
    }
#pragma unroll
    for (int j = 0; j < CT; ++j) sA[j][col] = tc[j];
  } else {
    // P = lower part (with the diagonal) of (g_j/g_m) Q K^T; the 10 tiles with ct <= rt over the
    // three other waves, zeros above
    for (int t = wave - 1; t < 16; t += 3) {
      const int rt = t >> 2, ct = t & 3;
      const v4f qt = ct <= rt ? tile_xk(sQ, rt, ct) : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 16 * rt + 4 * lk + v, m = 16 * ct + li;
        out[OFF_P + j * CT + m] = m <= j ? expf((float)(slg[j] - slg[m])) * qt[v] : 0.f;
      }
    }
  }
  __syncthreads();

  // W = Tm diag(beta g) K and Uv = Tm diag(beta) V: wave w forms rows 16w..16w+15, all columns
  {
    float aw[16], au[16];
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int m = 16 * lk + st;
      const float tm = sA[16 * wave + li][m];
      aw[st] = tm * sbg[m];
      au[st] = tm * sb[m];
    }
    for (int ct = 0; ct < 8; ++ct) {
      v4f wacc = {0.f, 0.f, 0.f, 0.f}, uacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        const int m = 16 * lk + st;
        wacc = __builtin_amdgcn_mfma_f32_16x16x4f32(aw[st], sK[m][16 * ct + li], wacc, 0, 0, 0);
        uacc = __builtin_amdgcn_mfma_f32_16x16x4f32(au[st], sV[m][16 * ct + li], uacc, 0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 16 * wave + 4 * lk + v;
        out[OFF_W + j * DK + 16 * ct + li] = wacc[v];
        out[OFF_UV + j * DV + 16 * ct + li] = uacc[v];
      }
    }
  }
}

// One workgroup per (value head, block of 16 value columns): the state block is carried through
// the chunks in order; each chunk gives D = Uv - W S, the readout Qg S + P D and the next state
// g_last S + Kt^T D. The products run on the fp32 matrix cores (v_mfma_f32_16x16x4_f32: lane l
// holds A[l%16][k] and B[k][l%16] with k = l/16, and D[4(l/16)+v][l%16]). The sum index is
// permuted so that every lane reads contiguous runs: at step s, lane group k = l/16 covers column
// 32k + s of a 128-long sum and 16k + s of a 64-long one, on both operands. Wave w owns rows
// 16w..16w+15 of D and of the readout, and rows 32w..32w+31 of the next state; the state block
// also sits in every wave's registers as the B operand, refreshed through LDS after each chunk.
__global__ __launch_bounds__(256) void k_pscan(const PScanArgs a) {
  __shared__ __attribute__((aligned(16))) float sS[DK][16], sD[CT][16];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, h = blockIdx.x, b = blockIdx.y;
  const int li = lane & 15, lk = lane >> 4;
  float* Sh = a.S + (size_t)h * DK * DV;
  for (int e = tid; e < DK * 16; e += 256) {
    if (a.transposed) {
      const int cc = e / DK, i = e % DK;  // stored [dv][dk]
      sS[i][cc] = Sh[(size_t)(16 * b + cc) * DK + i];
    } else {
      const int i = e / 16, cc = e % 16;
      sS[i][cc] = Sh[(size_t)i * DV + 16 * b + cc];
    }
  }
  __syncthreads();
  float bS[32];
#pragma unroll
  for (int st = 0; st < 32; ++st) bS[st] = sS[32 * lk + st][li];
  for (int c = 0; c < a.NCH; ++c) {
    const float* cw = a.cw + ((size_t)h * a.NCH + c) * PF_CHUNK_FLOATS;
    const int t0 = c * CT, nj = min(CT, a.T - t0);
    // A operands of this wave: rows 16w + li of W, Qg, P; columns 32w + 16tau + li of Kt^T
    float aW[32], aQ[32], aP[16], aK[2][16];
    {
      const float* wr = cw + OFF_W + (16 * w + li) * DK + 32 * lk;
      const float* qr = cw + OFF_QG + (16 * w + li) * DK + 32 * lk;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const v4f x = *reinterpret_cast<const v4f*>(wr + 4 * q), y = *reinterpret_cast<const v4f*>(qr + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          aW[4 * q + e] = -x[e];
          aQ[4 * q + e] = y[e];
        }
      }
      const float* pr = cw + OFF_P + (16 * w + li) * CT + 16 * lk;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f x = *reinterpret_cast<const v4f*>(pr + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) aP[4 * q + e] = x[e];
      }
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int st = 0; st < 16; ++st) aK[tau][st] = cw[OFF_KT + (16 * lk + st) * DK + 32 * w + 16 * tau + li];
    }
    const float gl = cw[OFF_G];
    // D = Uv - W S for rows 16w.., started from Uv
    v4f dacc;
#pragma unroll
    for (int v = 0; v < 4; ++v) dacc[v] = cw[OFF_UV + (16 * w + 4 * lk + v) * DV + 16 * b + li];
#pragma unroll
    for (int st = 0; st < 32; ++st) dacc = __builtin_amdgcn_mfma_f32_16x16x4f32(aW[st], bS[st], dacc, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) sD[16 * w + 4 * lk + v][li] = dacc[v];
    lds_barrier();
    float bD[16];
#pragma unroll
    for (int st = 0; st < 16; ++st) bD[st] = sD[16 * lk + st][li];
    // readout Qg S + P D
    v4f oacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 32; ++st) oacc = __builtin_amdgcn_mfma_f32_16x16x4f32(aQ[st], bS[st], oacc, 0, 0, 0);
#pragma unroll
    for (int st = 0; st < 16; ++st) oacc = __builtin_amdgcn_mfma_f32_16x16x4f32(aP[st], bD[st], oacc, 0, 0, 0);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = 16 * w + 4 * lk + v;
      if (j < nj) a.o[(size_t)(t0 + j) * a.V + h * DV + 16 * b + li] = oacc[v];
    }
    // next state, rows 32w + 16tau + 4lk + v
    v4f sacc[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
      for (int v = 0; v < 4; ++v) sacc[tau][v] = gl * sS[32 * w + 16 * tau + 4 * lk + v][li];
#pragma unroll
      for (int st = 0; st < 16; ++st)
        sacc[tau] = __builtin_amdgcn_mfma_f32_16x16x4f32(aK[tau][st], bD[st], sacc[tau], 0, 0, 0);
    }
    lds_barrier();  // every read of the old state block and of D is done
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int v = 0; v < 4; ++v) sS[32 * w + 16 * tau + 4 * lk + v][li] = sacc[tau][v];
    lds_barrier();
#pragma unroll
    for (int st = 0; st < 32; ++st) bS[st] = sS[32 * lk + st][li];
  }
  for (int e = tid; e < DK * 16; e += 256) {
    if (a.transposed) {
      const int cc = e / DK, ii = e % DK;
      Sh[(size_t)(16 * b + cc) * DK + ii] = sS[ii][cc];
    } else {
      const int ii = e / 16, cc = e % 16;
      Sh[(size_t)ii * DV + 16 * b + cc] = sS[ii][cc];
    }
  }
}

// Gated RMSNorm of one (token, value head), in place.
__global__ __launch_bounds__(128) void k_pnorm(const PNormArgs a) {
  __shared__ float red[2];
  const int t = blockIdx.x, h = blockIdx.y, j = threadIdx.x;
  float* op = a.o + (size_t)t * a.V + h * DV + j;
  const float o = *op;
  const float z = a.u[(size_t)t * a.R + a.C + h * DV + j];
  float s = o * o;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if ((j & 63) == 0) red[j >> 6] = s;
  __syncthreads();
  const float inv = rsqrtf((red[0] + red[1]) / (float)DV + a.eps_rms);
  *op = a.norm_w[j] * o * inv * silu(z);
}

}  // namespace

hipError_t launch_pconv(const PConvArgs& a, hipStream_t st) {
  if (a.terms && a.M % 4 == 0 && a.C % 4 == 0 && reinterpret_cast<uintptr_t>(a.terms) % 16 == 0 &&
      reinterpret_cast<uintptr_t>(a.out) % 16 == 0) {
    hipLaunchKernelGGL(k_pconv4, dim3((a.M / 4 + 255) / 256, (a.T + TR4 - 1) / TR4), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_pconv, dim3((a.M + 255) / 256, (a.T + TR - 1) / TR), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pintra(const PIntraArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_pintra, dim3(a.Hv, a.NCH), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pscan(const PScanArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_pscan, dim3(a.Hv, DV / 16), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_pnorm(const PNormArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_pnorm, dim3(a.T, a.V / DV), dim3(128), 0, st, a);
  return hipGetLastError();
}

}  // namespace dn
