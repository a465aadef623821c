// Internal interface between the C-ABI host code and the HIP kernels of libdn.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

#include "dn.h"

namespace dn {

// Per-row-scaled GEMV over a batch: out[b][r] = s[r] * sum_c W[r][c] * xin[b][c], where xin
// is x (optionally RMS-normalised). With `conv` set, rows r < C also run the depthwise causal
// conv + SiLU against the history ring[b][K-1][C] and advance it.
struct GemvArgs {
  const void* W;        // [rows][cols] int8 or [rows][cols/2] packed int4
  const float* s;       // [rows]
  const float* x;       // [B][x_stride]
  float* out;           // [B][out_stride]
  int rows, cols, batch;
  int x_stride, out_stride;
  int prenorm;          // RMS-normalise x first
  float eps;
  // conv epilogue (used when conv_w != nullptr)
  const float* conv_w;  // [C][K]
  float* ring;          // [B][K-1][C], oldest first
  int C, K;
};

// One value head per workgroup: L2 norms, decay, delta rule, readout, gated RMSNorm.
struct HeadArgs {
  const float* u;       // [B][R]: post-conv q | k | v, then raw z
  float* S;             // [B][Hv][dk][dv]
  const float* alpha;   // [B][Hv]
  const float* beta;    // [B][Hv]
  const float* norm_w;  // [dv]
  float* y;             // [B][Hv*dv]
  int Hk, Hv, dk, dv, R, C, batch;
  float eps_l2, eps_rms, q_scale;
};

hipError_t launch_gemv(const GemvArgs& a, int bits, hipStream_t st);
hipError_t launch_head(const HeadArgs& a, hipStream_t st);

}  // namespace dn
