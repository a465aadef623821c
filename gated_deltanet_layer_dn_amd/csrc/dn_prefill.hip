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
// The chunk terms are stored in the order k_pscan's lanes read them (every load instruction of the
// scan then reads 1 KB in one piece): 16-byte units, unit u holding four consecutive values.
//   W, Qg [64][128]: element (row, col) in unit ((row/16) 8 + (col%32)/4) 64 + row%16 + 16 (col/32)
//   P [64][64]:      element (row, col) in unit ((row/16) 4 + (col%16)/4) 64 + row%16 + 16 (col/16)
//   Kt (k weighted by the decay to the chunk's end, token tok, key column i): unit
//                    ((i/32) 2 + (i/16)%2) 4 + (tok%16)/4) 64 + i%16 + 16 (tok/16), value tok % 4
//   Uv [64][128]:    element (row, col) in unit ((col/16) 4 + row/16) 64 + col%16 + 16 ((row%16)/4),
//                    value row % 4
constexpr int TR = 32;  // tokens per thread in k_pconv
constexpr int LD = DK + 4;  // padded LDS row of 128 floats (keeps 16-byte alignment)

// SiLU with the hardware reciprocal (within an ulp of the quotient)
__device__ __forceinline__ float silu(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

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

// k_pconv on the exact term sums of the three-term GEMM (folded here in double with the token's
// scale), or on sums the GEMM already folded the same way (one K range), four adjacent rows per
// thread: 16-byte loads and stores, and every load unconditional (a token past the prompt reads the
// last token's row and is not stored), so the loads of a run of tokens are all in flight together.
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
    if (!a.terms) {  // the sums already folded (one K range)
      const v4f p = *reinterpret_cast<const v4f*>(a.part + at);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = sr[e] * f * p[e];
      return;
    }
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
// The 64 x 64 and 64 x 128 products run on the fp32 matrix cores (lane layout as in k_pscan); the
// unit lower-triangular inverse goes in 16 x 16 blocks: the four diagonal blocks by substitution in
// the first wave (lane = column) while the other three form the masked q.k products, then the
// blocks below the diagonal by matrix-core products.
__global__ __launch_bounds__(256) void k_pintra(const PIntraArgs a) {
  __shared__ __attribute__((aligned(16))) float sQ[CT][LD], sK[CT][LD], sV[CT][LD];
  __shared__ float sA[CT][CT + 1];  // A
  __shared__ float sT[CT][CT + 1];  // Tm = (I + A)^-1 (lower triangular)
  __shared__ __attribute__((aligned(16))) float sPs[CT][CT + 4];  // P, staged for whole-unit stores
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

  // decayed q rows, k rows weighted by the decay to the chunk's end (stored transposed, [dk][token],
  // the layout k_pscan reads), the chunk's total decay
  {
    const double lgl = slg[nj - 1];
    // one 16-byte unit per thread and step, consecutive threads on consecutive units
    for (int u = tid; u < CT * DK / 4; u += 256) {
      const int ul = u & 63, j = 16 * (u >> 9) + (ul & 15), i4 = 32 * (ul >> 4) + 4 * ((u >> 6) & 7);
      const v4f q = *reinterpret_cast<const v4f*>(&sQ[j][i4]);
      *reinterpret_cast<v4f*>(out + OFF_QG + 4 * u) = q * expf((float)slg[j]);
    }
    for (int u = tid; u < CT * DK / 4; u += 256) {
      const int ul = u & 63, i = 32 * (u >> 9) + 16 * ((u >> 8) & 1) + (ul & 15);
      const int tok0 = 16 * (ul >> 4) + 4 * ((u >> 6) & 3);
      v4f kv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tk = tok0 + e;
        kv[e] = tk < nj ? sK[tk][i] * expf((float)(lgl - slg[tk])) : 0.f;
      }
      *reinterpret_cast<v4f*>(out + OFF_KT + 4 * u) = kv;
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

  // Tm = (I + A)^-1 in 16 x 16 blocks: the diagonal blocks by forward substitution (wave 0, lane l
  // column l % 16 of block l / 16) while the other waves form P; then the blocks below the diagonal,
  // one diagonal of blocks after the other, on the matrix cores:
  //   T_ij = -T_ii sum_{j <= k < i} A_ik T_kj
  if (wave == 0) {
    const int r0 = 16 * (lane >> 4), c = lane & 15;
    float tc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float v0 = r == c ? 1.0f : 0.0f, v1 = 0.0f;  // two interleaved partial sums
#pragma unroll
      for (int m = 0; m < r; ++m) {
        if (m & 1) v1 = fmaf(-sA[r0 + r][r0 + m], tc[m], v1);
        else v0 = fmaf(-sA[r0 + r][r0 + m], tc[m], v0);
      }
      tc[r] = v0 + v1;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) sT[r0 + r][r0 + c] = tc[r];
  } else {
    // P = lower part (with the diagonal) of (g_j/g_m) Q K^T; the 10 tiles with ct <= rt over the
    // three other waves, zeros above
    for (int t = wave - 1; t < 16; t += 3) {
      const int rt = t >> 2, ct = t & 3;
      const v4f qt = ct <= rt ? tile_xk(sQ, rt, ct) : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 16 * rt + 4 * lk + v, m = 16 * ct + li;
        sPs[j][m] = m <= j ? expf((float)(slg[j] - slg[m])) * qt[v] : 0.f;
      }
    }
  }
  __syncthreads();
  // P in the scan's order, one whole 16-byte unit per thread and step
  for (int u = tid; u < CT * CT / 4; u += 256) {
    const int ul = u & 63, j = 16 * (u >> 8) + (ul & 15), m4 = 16 * (ul >> 4) + 4 * ((u >> 6) & 3);
    *reinterpret_cast<v4f*>(out + OFF_P + 4 * u) = *reinterpret_cast<const v4f*>(&sPs[j][m4]);
  }
  // 16 x 16 products with the sum index 4 s + k at step s (lane group k = l / 16)
  for (int L = 1; L < 4; ++L) {
    if (wave < 4 - L) {
      const int i = wave + L, j = wave;
      v4f x = {0.f, 0.f, 0.f, 0.f};
      for (int k = j; k < i; ++k)
#pragma unroll
        for (int st = 0; st < 4; ++st)
          x = __builtin_amdgcn_mfma_f32_16x16x4f32(sA[16 * i + li][16 * k + 4 * st + lk],
                                                   sT[16 * k + 4 * st + lk][16 * j + li], x, 0, 0, 0);
      // T_ii x: x's rows 4 k + v sit in this lane's x[v], so the sum index here is 4 k + s
      v4f y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        y = __builtin_amdgcn_mfma_f32_16x16x4f32(sT[16 * i + li][16 * i + 4 * lk + st], x[st], y, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 4; ++v) sT[16 * i + 4 * lk + v][16 * j + li] = -y[v];
    }
    __syncthreads();
  }

  // W = Tm diag(beta g) K and Uv = Tm diag(beta) V. Tm is lower triangular: row tile rt sums over
  // the first 16 (rt + 1) rows of K and V only. Wave w forms column tiles 2w and 2w + 1 of every
  // row tile (the same number of products on every wave). Every operand is read into registers
  // first (Tm's nonzero blocks scaled, 40 steps, and a column tile's K and V rows), so the products
  // of a column tile issue back to back.
  {
    float aw[40], au[40];  // step st of row tile rt at index 2 rt (rt + 1) + st
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int st = 0; st < 4 * (rt + 1); ++st) {
        const int m = 4 * st + lk;
        const float tm = sT[16 * rt + li][m];
        aw[2 * rt * (rt + 1) + st] = tm * sbg[m];
        au[2 * rt * (rt + 1) + st] = tm * sb[m];
      }
#pragma unroll
    for (int cl = 0; cl < 2; ++cl) {
      const int ct = 2 * wave + cl;
      float bk[16], bv[16];
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        bk[st] = sK[4 * st + lk][16 * ct + li];
        bv[st] = sV[4 * st + lk][16 * ct + li];
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        v4f wacc = {0.f, 0.f, 0.f, 0.f}, uacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4 * (rt + 1); ++st) {
          wacc = __builtin_amdgcn_mfma_f32_16x16x4f32(aw[2 * rt * (rt + 1) + st], bk[st], wacc, 0, 0, 0);
          uacc = __builtin_amdgcn_mfma_f32_16x16x4f32(au[2 * rt * (rt + 1) + st], bv[st], uacc, 0, 0, 0);
        }
        // W staged in sQ (free since P), written in the scan's order below
#pragma unroll
        for (int v = 0; v < 4; ++v) sQ[16 * rt + 4 * lk + v][16 * ct + li] = wacc[v];
        // rows 16 rt + 4 lk + v, column 16 ct + li: one whole unit of the Uv order per lane
        *reinterpret_cast<v4f*>(out + OFF_UV + 4 * ((ct * 4 + rt) * 64 + lane)) = uacc;
      }
    }
  }
  __syncthreads();
  for (int u = tid; u < CT * DK / 4; u += 256) {
    const int ul = u & 63, j = 16 * (u >> 9) + (ul & 15), c4 = 32 * (ul >> 4) + 4 * ((u >> 6) & 7);
    *reinterpret_cast<v4f*>(out + OFF_W + 4 * u) = *reinterpret_cast<const v4f*>(&sQ[j][c4]);
  }
}

// One workgroup per (value head, block of 16 value columns): the state block is carried through
// the chunks in order; each chunk gives D = Uv - W S, the next state g_last S + Kt^T D and the
// readout Qg S + P D. The products run on the fp32 matrix cores (v_mfma_f32_16x16x4_f32: lane l
// holds A[l%16][k] and B[k][l%16] with k = l/16, and D[4(l/16)+v][l%16]). The sum index is
// permuted so that every lane reads contiguous runs: at step s, lane group k = l/16 covers column
// 32k + s of a 128-long sum and 16k + s of a 64-long one, on both operands. Wave w owns rows
// 16w..16w+15 of D and of the readout, and rows 32w..32w+31 of the next state; the state block
// also sits in every wave's registers as the B operand, refreshed through LDS after each chunk.
// The chain from one state to the next is D, then the next state; the next chunk's chain operands
// are loaded while a chunk computes, and the readout's products go after the state's (their
// operands requested at the chunk's start), filling the matrix pipe while the new state block
// passes through LDS.
struct PScanOps {  // a chunk's operands on the chain from one state to the next
  float aW[32], aK[2][16];  // rows 16w + li of W; columns 32w + 16tau + li of Kt^T
  float uv[4];              // Uv rows 16w + 4lk + v, column 16b + li
  float gl;                 // the chunk's total decay
};
struct PScanRead {  // a chunk's readout operands
  float aQ[32], aP[16];  // rows 16w + li of Qg, P
};

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
  // loads only (no arithmetic on the loaded values, which would wait for them at once); part: 1 W,
  // 2 Kt, 4 Uv and the decay
  auto load_ops = [&](int c, PScanOps& o, int part) {
    const float* cw = a.cw + ((size_t)h * a.NCH + c) * PF_CHUNK_FLOATS;
    if (part & 1) {
    const float* wr = cw + OFF_W + 4 * (w * 8 * 64 + lane);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const v4f x = *reinterpret_cast<const v4f*>(wr + 256 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) o.aW[4 * q + e] = x[e];
    }
    }
    if (part & 2) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const float* kr = cw + OFF_KT + 4 * ((w * 2 + tau) * 4 * 64 + lane);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f x = *reinterpret_cast<const v4f*>(kr + 256 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) o.aK[tau][4 * q + e] = x[e];
      }
    }
    }
    if (part & 4) {
    const v4f x = *reinterpret_cast<const v4f*>(cw + OFF_UV + 4 * ((b * 4 + w) * 64 + lane));
#pragma unroll
    for (int v = 0; v < 4; ++v) o.uv[v] = x[v];
    o.gl = cw[OFF_G];
    }
  };
  auto load_read = [&](int c, PScanRead& o) {
    const float* cw = a.cw + ((size_t)h * a.NCH + c) * PF_CHUNK_FLOATS;
    const float* qr = cw + OFF_QG + 4 * (w * 8 * 64 + lane);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const v4f y = *reinterpret_cast<const v4f*>(qr + 256 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) o.aQ[4 * q + e] = y[e];
    }
    const float* pr = cw + OFF_P + 4 * (w * 4 * 64 + lane);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4f x = *reinterpret_cast<const v4f*>(pr + 256 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) o.aP[4 * q + e] = x[e];
    }
  };
  __syncthreads();
  float bS[32];
#pragma unroll
  for (int st = 0; st < 32; ++st) bS[st] = sS[32 * lk + st][li];
  // one chunk; `last`: the prompt's last chunk, which may be ragged (the others are whole, so their
  // loads and stores are unconditional and the waits for them exact)
  auto chunk = [&](int c, const PScanOps& o, PScanOps& nx, bool last) {
    // the readout operands of this chunk (needed after the chain's products) are requested first,
    // the next chunk's chain operands (needed a whole chunk later) in three parts between this chunk's
    // products: all at once, the loads would hold the wave's issue while the memory pipe takes them
    PScanRead rd;
    load_read(c, rd);
    const int cn = min(c + 1, a.NCH - 1);
    load_ops(cn, nx, 1);
    __builtin_amdgcn_sched_barrier(0);
    const int t0 = c * CT, nj = min(CT, a.T - t0);
    // D = Uv - W S for rows 16w..
    v4f dacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 32; ++st) dacc = __builtin_amdgcn_mfma_f32_16x16x4f32(o.aW[st], bS[st], dacc, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_ops(cn, nx, 2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < 4; ++v) sD[16 * w + 4 * lk + v][li] = o.uv[v] - dacc[v];
    lds_barrier();
    float bD[16];
#pragma unroll
    for (int st = 0; st < 16; ++st) bD[st] = sD[16 * lk + st][li];
    // next state, rows 32w + 16tau + 4lk + v: on the chain, so first
    v4f sacc[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int v = 0; v < 4; ++v) sacc[tau][v] = o.gl * sS[32 * w + 16 * tau + 4 * lk + v][li];
#pragma unroll
    for (int st = 0; st < 16; ++st)
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
        sacc[tau] = __builtin_amdgcn_mfma_f32_16x16x4f32(o.aK[tau][st], bD[st], sacc[tau], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_ops(cn, nx, 4);
    __builtin_amdgcn_sched_barrier(0);
    // readout Qg S + P D: off the chain
    v4f oacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 32; ++st) oacc = __builtin_amdgcn_mfma_f32_16x16x4f32(rd.aQ[st], bS[st], oacc, 0, 0, 0);
#pragma unroll
    for (int st = 0; st < 16; ++st) oacc = __builtin_amdgcn_mfma_f32_16x16x4f32(rd.aP[st], bD[st], oacc, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();  // every read of the old state block and of D is done
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int v = 0; v < 4; ++v) sS[32 * w + 16 * tau + 4 * lk + v][li] = sacc[tau][v];
    lds_barrier();
#pragma unroll
    for (int st = 0; st < 32; ++st) bS[st] = sS[32 * lk + st][li];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = 16 * w + 4 * lk + v;
      if (!last || j < nj) a.o[(size_t)(t0 + j) * a.V + h * DV + 16 * b + li] = oacc[v];
    }
  };
  PScanOps o0, o1;
  load_ops(0, o0, 7);
  int c = 0;
  for (; c + 2 < a.NCH; c += 2) {
    chunk(c, o0, o1, false);
    chunk(c + 1, o1, o0, false);
  }
  if (c + 1 < a.NCH) {
    chunk(c, o0, o1, false);
    chunk(c + 1, o1, o0, true);
  } else {
    chunk(c, o0, o1, true);
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

typedef int pg_v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void pg_lds_t;

// k_pgemm: a workgroup of eight waves owns 256 weight rows and 64 tokens (x 3 terms); wave w the rows
// 64 (w % 4) .. +63 (four 16-row tiles) against the 32 tokens of half w / 4 and their three terms:
// 4 x 2 x 3 MFMA tiles (v_mfma_i32_16x16x64_i8), 96 accumulators. K advances in stages of 128
// columns, two LDS buffers: while a stage's products run, the next stage goes from memory straight
// into the other buffer (buffer loads with the LDS bit, no registers between). A stage holds 28 tiles
// of 16 rows (or tokens) x 128 columns, 2 KB each: 16 weight tiles, then 3 terms x 4 token tiles.
// Each load instruction covers 8 whole rows of 128 bytes (lane l: row l / 8, 16-byte chunk
// (l % 8) ^ PG_SWZ(row)), so every cache line fetched is used whole; the xor permutation of the
// chunks makes the operand reads (lane l: row l % 16, chunk 4 k + l / 16 of k-step k) hit every LDS
// bank once per group of 16 lanes. One barrier per stage.
constexpr int PG_ROWS = 256, PG_TOK = 64, PG_KC = 128, PG_WAVES = 8;
constexpr int PG_AT = PG_ROWS / 16, PG_XT = 3 * (PG_TOK / 16);  // weight and token tiles per stage
constexpr int PG_TILE = 2048, PG_STAGE = (PG_AT + PG_XT) * PG_TILE;
constexpr int PG_NI = (PG_AT + PG_XT) * 2 / PG_WAVES;  // load instructions per wave per stage: 7

__device__ __forceinline__ int pg_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ void pg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

constexpr int PG_PLD = PG_ROWS + 4;  // padded row of the conv epilogue's staging ([64 tokens][256 rows])

template <bool CONV>
__global__ __launch_bounds__(512) void k_pgemm(const PGemmArgs a) {
  __shared__ pg_v4i sq[2][PG_STAGE / 16];
  // wave index uniform (scalar): which tile each of its loads fills derives from it
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = wave & 3, th = wave >> 2;  // row group of 64, token half of 32
  const int row0 = blockIdx.x * PG_ROWS, t0 = blockIdx.y * PG_TOK;
  const int NS = a.K / PG_KC;
  const __amdgpu_buffer_rsrc_t rsW =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a.W), (short)0, (int)((size_t)a.M * a.K), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsX =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(a.X), (short)0, (int)((size_t)3 * a.T * a.K), 0x00020000);
  // load instruction g = 7 w + i of a stage fills rows 8 (g % 2) .. +7 of tile g / 2; rows and tokens
  // past the end are clamped (their sums are never stored); per-lane byte offsets at the stage's
  // first column
  int off[PG_NI];
#pragma unroll
  for (int i = 0; i < PG_NI; ++i) {
    const int g = PG_NI * wave + i, r = 8 * (g & 1) + (lane >> 3), c = (lane & 7) ^ pg_swz(r);
    if (g < 2 * PG_AT) {
      off[i] = min(row0 + 16 * (g >> 1) + r, a.M - 1) * a.K + 16 * c;
    } else {
      const int xt = (g - 2 * PG_AT) >> 1, term = xt >> 2, tt = xt & 3;
      off[i] = (term * a.T + min(t0 + 16 * tt + r, a.T - 1)) * a.K + 16 * c;
    }
  }
  auto issue = [&](int stage) {
    char* const base = reinterpret_cast<char*>(sq[stage & 1]);
#pragma unroll
    for (int i = 0; i < PG_NI; ++i) {
      const int g = PG_NI * wave + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(g < 2 * PG_AT ? rsW : rsX, (pg_lds_t*)(base + 1024 * g), 16, off[i],
                                               stage * PG_KC, 0, 0);
    }
  };
  // operand reads within a tile: byte offsets of lane l's chunk for k-steps 0 and 1
  const int rr = lane & 15, rd0 = 16 * (64 * (rr >> 3) + 8 * (rr & 7) + ((lane >> 4) ^ pg_swz(rr)));
  const int rd1 = rd0 ^ 64;
  struct Ops { pg_v4i A[4], X[3][2]; };
  auto read = [&](int stage, int rd, Ops& o) {
    const char* const base = reinterpret_cast<const char*>(sq[stage & 1]) + rd;
#pragma unroll
    for (int r = 0; r < 4; ++r) o.A[r] = *reinterpret_cast<const pg_v4i*>(base + (4 * rg + r) * PG_TILE);
#pragma unroll
    for (int term = 0; term < 3; ++term)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        o.X[term][tt] = *reinterpret_cast<const pg_v4i*>(base + (PG_AT + 4 * term + 2 * th + tt) * PG_TILE);
  };
  pg_v4i acc[4][2][3];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int term = 0; term < 3; ++term) acc[r][tt][term] = pg_v4i{0, 0, 0, 0};
  auto mfma = [&](const Ops& o) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int term = 0; term < 3; ++term)
          acc[r][tt][term] = __builtin_amdgcn_mfma_i32_16x16x64_i8(o.A[r], o.X[term][tt], acc[r][tt][term], 0, 0, 0);
  };
  issue(0);
  for (int st = 0; st < NS; ++st) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of stage st have landed
    pg_barrier();  // every wave's loads of stage st landed; every wave is done with stage st - 1's buffer
    if (st + 1 < NS) issue(st + 1);
    Ops o0, o1;
    read(st, rd0, o0);
    read(st, rd1, o1);
    __builtin_amdgcn_sched_barrier(0);  // all reads first: the second k-step's arrive under the first's products
    mfma(o0);
    mfma(o1);
  }
  // epilogue: lane holds token t0 + 32 th + 16 tt + lane % 16, rows 16 r + 4 (lane / 16) + v of the
  // wave's four row tiles; the three terms folded in double with the token's scale (as k_pconv
  // folds the library GEMM's sums), four consecutive rows per 16-byte store
  // the epilogue's scalars first, all requested together: the token scales, the row scales of the
  // lane's 16 rows (four runs of four), the pre-norm sums
  float s1v[2], ssqv[2];
  v4f srow[4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int tc = min(t0 + 32 * th + 16 * tt + (lane & 15), a.T - 1);
    s1v[tt] = a.s1[tc];
    ssqv[tt] = CONV ? a.ssq[tc] : 0.f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r)
    srow[r] = a.s ? *reinterpret_cast<const v4f*>(a.s + min(row0 + 64 * rg + 16 * r + 4 * (lane >> 4), a.M - 4))
                  : v4f{1.f, 1.f, 1.f, 1.f};
  if constexpr (!CONV) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = t0 + 32 * th + 16 * tt + (lane & 15);
      const double s1 = (double)s1v[tt];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = row0 + 64 * rg + 16 * r + 4 * (lane >> 4);
        v4f o;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          o[v] = (float)(s1 * ((double)acc[r][tt][0][v] +
                               ((double)acc[r][tt][1][v] + (double)acc[r][tt][2][v] * (1.0 / 254.0)) * (1.0 / 254.0)));
          if (a.s) o[v] = srow[r][v] * o[v];  // out_proj: the row scale (k_bepi's last step)
        }
        if (t < a.T) {
          if (m + 3 < a.M) {
            *reinterpret_cast<v4f*>(a.out + (size_t)t * a.M + m) = o;
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
              if (m + v < a.M) a.out[(size_t)t * a.M + m + v] = o[v];
          }
        }
        __builtin_amdgcn_sched_barrier(0);  // one tile's doubles live at a time
      }
    }
  } else {
    // in_proj: pre-conv values (the fold times the row scale and the token's pre-norm factor, as
    // k_pconv computes them) staged in LDS as [64 tokens][256 rows] over the stage buffers, which every
    // wave is done with; the edge tokens' values also to global memory
    float(*sP)[PG_PLD] = reinterpret_cast<float(*)[PG_PLD]>(&sq[0][0]);
    pg_barrier();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int tl = 32 * th + 16 * tt + (lane & 15), t = t0 + tl;
      const double s1 = (double)s1v[tt];
      const float f = a.prenorm ? rsqrtf(ssqv[tt] / (float)a.K + a.eps) : 1.0f;
      const bool edge_t = t < a.T && (tl < 3 || tl >= PG_TOK - 3 || t >= a.T - 3);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = 64 * rg + 16 * r + 4 * (lane >> 4), m = row0 + rl;
        v4f o;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float fold = (float)(s1 * ((double)acc[r][tt][0][v] +
                                           ((double)acc[r][tt][1][v] + (double)acc[r][tt][2][v] * (1.0 / 254.0)) *
                                               (1.0 / 254.0)));
          o[v] = srow[r][v] * f * fold;
        }
        *reinterpret_cast<v4f*>(&sP[tl][rl]) = o;
        if (edge_t && m < a.M) *reinterpret_cast<v4f*>(a.edge + (size_t)t * a.M + m) = o;  // M % 4 == 0
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
    pg_barrier();
    // thread: row rl, tokens 32 h2 .. +31 of the tile; rows < C: conv over the previous Kc - 1
    // tokens and SiLU, in k_pconv's order of operations, for tokens whose history is in the tile
    const int rl = threadIdx.x & (PG_ROWS - 1), j0 = 32 * (threadIdx.x / PG_ROWS), m = row0 + rl;
    if (m < a.M) {
      if (m >= a.C) {
        for (int i = 0; i < 32; ++i)
          if (t0 + j0 + i < a.T) a.out[(size_t)(t0 + j0 + i) * a.M + m] = sP[j0 + i][rl];
      } else {
        const int Kc = a.Kc;
        float w[4], hist[3] = {0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = q < Kc ? a.conv_w[(size_t)m * Kc + q] : 0.f;
#pragma unroll
        for (int q = 0; q < 3; ++q)
          if (q < Kc - 1 && j0 - (Kc - 1) + q >= 0) hist[q] = sP[j0 - (Kc - 1) + q][rl];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int j = j0 + i;
          const float u = sP[j][rl];
          float accv = w[Kc - 1] * u;
#pragma unroll
          for (int q = 0; q < 3; ++q)
            if (q < Kc - 1) accv = fmaf(w[q], hist[q], accv);
          if (j >= 3 && t0 + j < a.T) a.out[(size_t)(t0 + j) * a.M + m] = silu(accv);
#pragma unroll
          for (int q = 0; q < 2; ++q)
            if (q + 1 < Kc - 1) hist[q] = hist[q + 1];
          if (Kc > 1) hist[Kc - 2] = u;
        }
      }
    }
  }
}

// The first three tokens of each 64-token tile after k_pgemm's conv epilogue (rows < C): the conv
// over the edge buffer's pre-conv values (tokens before the prompt from the history) and SiLU, in
// k_pconv's order of operations; the last tile's workgroups also leave the new history.
__global__ __launch_bounds__(256) void k_pconv_edge(const PConvArgs a) {
  const int r = blockIdx.x * 256 + threadIdx.x, t0 = PG_TOK * blockIdx.y;
  if (r >= a.C) return;
  const int Kc = a.Kc;
  float w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) w[q] = q < Kc ? a.conv_w[(size_t)r * Kc + q] : 0.f;
  auto pre = [&](int tok) {
    return tok >= 0 ? a.part[(size_t)tok * a.M + r] : a.ring_in[(size_t)(tok + Kc - 1) * a.C + r];
  };
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int t = t0 + i;
    if (t < a.T) {
      float acc = w[Kc - 1] * a.part[(size_t)t * a.M + r];
#pragma unroll
      for (int q = 0; q < 3; ++q)
        if (q < Kc - 1) acc = fmaf(w[q], pre(t - (Kc - 1) + q), acc);
      a.out[(size_t)t * a.M + r] = silu(acc);
    }
  }
  if (blockIdx.y == gridDim.y - 1)
#pragma unroll
    for (int q = 0; q < 3; ++q)
      if (q < Kc - 1) a.ring_out[(size_t)q * a.C + r] = pre(a.T - (Kc - 1) + q);
}
}  // namespace

hipError_t launch_pconv(const PConvArgs& a, hipStream_t st) {
  const void* in4 = a.terms ? static_cast<const void*>(a.terms) : a.KS == 1 ? static_cast<const void*>(a.part) : nullptr;
  if (in4 && a.M % 4 == 0 && a.C % 4 == 0 && reinterpret_cast<uintptr_t>(in4) % 16 == 0 &&
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

bool pgemm_shape_ok(int M, int K, int T) {
  return M >= 1 && T >= 1 && K >= PG_KC && K % PG_KC == 0 && M % 4 == 0 &&
         (size_t)M * K < (1u << 31) && (size_t)3 * T * K < (1u << 31);
}

hipError_t launch_pgemm(const PGemmArgs& a, hipStream_t st) {
  if (!pgemm_shape_ok(a.M, a.K, a.T) || reinterpret_cast<uintptr_t>(a.out) % 16) return hipErrorInvalidValue;
  const dim3 grid((a.M + PG_ROWS - 1) / PG_ROWS, (a.T + PG_TOK - 1) / PG_TOK);
  if (a.conv) {
    if (a.Kc < 1 || a.Kc > 4 || a.C > a.M || reinterpret_cast<uintptr_t>(a.edge) % 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_pgemm<true>, grid, dim3(64 * PG_WAVES), 0, st, a);
  } else {
    hipLaunchKernelGGL(k_pgemm<false>, grid, dim3(64 * PG_WAVES), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_pconv_edge(const PConvArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(k_pconv_edge, dim3((a.C + 255) / 256, (a.T + PG_TOK - 1) / PG_TOK), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace dn
