// The prefill projections with 8-bit weights as plain int8 x int8 -> int32 library GEMMs
// (hipBLASLt): D = W X^T with W the projection's rows [M][K] and X the three int8 terms of every
// token's input [3T][K] (see k_tsplit), D [3T][M] int32. The integer sums are exact, so the result
// does not depend on the algorithm the library picks; the fold of the three terms, the scales and
// the conv run in this library's own epilogue kernels.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstdint>
#include <new>

#include "dn_internal.h"

namespace dn {

namespace {
constexpr size_t LT_WS_BYTES = 32u << 20;  // workspace the library may use per GEMM

struct LtShape {
  hipblasLtMatmulDesc_t md = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo{};
  size_t ws = 0;
  int M = 0, N = 0, K = 0;
  bool ok = false;
};

void release(LtShape& s) {
  if (s.la) (void)hipblasLtMatrixLayoutDestroy(s.la);
  if (s.lb) (void)hipblasLtMatrixLayoutDestroy(s.lb);
  if (s.lc) (void)hipblasLtMatrixLayoutDestroy(s.lc);
  if (s.md) (void)hipblasLtMatmulDescDestroy(s.md);
  s = LtShape{};
}
}  // namespace

struct LtCtx {
  hipblasLtHandle_t h = nullptr;
  void* ws = nullptr;
  LtShape shape[2];
};

LtCtx* lt_create() {
  LtCtx* c = new (std::nothrow) LtCtx();
  if (!c) return nullptr;
  if (hipblasLtCreate(&c->h) != HIPBLAS_STATUS_SUCCESS) {
    delete c;
    return nullptr;
  }
  if (hipMalloc(&c->ws, LT_WS_BYTES) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipblasLtDestroy(c->h);
    delete c;
    return nullptr;
  }
  return c;
}

void lt_destroy(LtCtx* c) {
  if (!c) return;
  for (LtShape& s : c->shape) release(s);
  if (c->ws) (void)hipFree(c->ws);
  if (c->h) (void)hipblasLtDestroy(c->h);
  delete c;
}

bool lt_prepare(LtCtx* c, int slot, int M, int N, int K) {
  if (!c || slot < 0 || slot > 1 || M < 1 || N < 1 || K < 1) return false;
  LtShape& s = c->shape[slot];
  if (s.md && s.M == M && s.N == N && s.K == K) return s.ok;
  release(s);
  s.M = M;
  s.N = N;
  s.K = K;
  // Column-major view: D (M x N, ld M) = A^T (A: K x M, ld K, the row-major weights) * B (K x N, ld K,
  // the row-major terms).
  const int32_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  bool ok = hipblasLtMatmulDescCreate(&s.md, HIPBLAS_COMPUTE_32I, HIP_R_32I) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(s.md, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatmulDescSetAttribute(s.md, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&s.la, HIP_R_8I, K, M, K) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&s.lb, HIP_R_8I, K, N, K) == HIPBLAS_STATUS_SUCCESS;
  ok = ok && hipblasLtMatrixLayoutCreate(&s.lc, HIP_R_32I, M, N, M) == HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulPreference_t pref = nullptr;
  ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
  const uint64_t ws = LT_WS_BYTES;
  ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &ws, sizeof(ws)) ==
                 HIPBLAS_STATUS_SUCCESS;
  hipblasLtMatmulHeuristicResult_t res[1];
  int n = 0;
  ok = ok && hipblasLtMatmulAlgoGetHeuristic(c->h, s.md, s.la, s.lb, s.lc, s.lc, pref, 1, res, &n) ==
                 HIPBLAS_STATUS_SUCCESS;
  if (pref) (void)hipblasLtMatmulPreferenceDestroy(pref);
  ok = ok && n >= 1 && res[0].state == HIPBLAS_STATUS_SUCCESS && res[0].workspaceSize <= LT_WS_BYTES;
  if (ok) {
    s.algo = res[0].algo;
    s.ws = res[0].workspaceSize;
  }
  s.ok = ok;
  return ok;
}

hipError_t lt_gemm_i8(LtCtx* c, int slot, const void* W, const int8_t* X, int32_t* D, hipStream_t st) {
  if (!c || slot < 0 || slot > 1 || !c->shape[slot].ok) return hipErrorInvalidValue;
  LtShape& s = c->shape[slot];
  const int32_t alpha = 1, beta = 0;
  const hipblasStatus_t r = hipblasLtMatmul(c->h, s.md, &alpha, W, s.la, X, s.lb, &beta, D, s.lc, D, s.lc, &s.algo,
                                            c->ws, s.ws, st);
  return r == HIPBLAS_STATUS_SUCCESS ? hipSuccess : hipErrorLaunchFailure;
}

}  // namespace dn
