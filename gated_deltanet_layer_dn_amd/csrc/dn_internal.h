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
  // when set, x is a gated readout still to be scaled per head of head_dim columns by
  // 1/sqrt(sum of head_ssq [B][cols/head_dim][head_nb] / head_dim + head_eps)
  const float* head_ssq;
  int head_dim, head_nb;
  float head_eps;
};

// One value head per workgroup: L2 norms, decay, delta rule, readout, gated RMSNorm.
struct HeadArgs {
  const float* u;       // [B][R]: post-conv q | k | v, then raw z
  float* S;             // [B][Hv][dk][dv]
  const float* alpha;   // [B][Hv], or [B][Hv][dk] with alpha_per_key
  const float* beta;    // [B][Hv]
  const float* norm_w;  // [dv]
  float* y;             // [B][Hv*dv]
  int Hk, Hv, dk, dv, R, C, batch;
  int alpha_per_key;    // 1: key row i of head h decays by alpha[b][h][i]
  float eps_l2, eps_rms, q_scale;
  // when set (dk, dv multiples of 16): the column-split kernel, one workgroup per 16 value columns;
  // y gets w o silu(z) without the head's 1/rms and ssq [B][Hv][dv/16] the blocks' sums of o^2
  float* ssq;
};

hipError_t launch_gemv(const GemvArgs& a, int bits, hipStream_t st);
hipError_t launch_head(const HeadArgs& a, hipStream_t st);

// The two gates of each value head from the in_proj's gate rows a | b (DN_GATES_ON_DEVICE):
// alpha = exp(-exp(a_log) * softplus(a + a_bias)), beta = 1 / (1 + exp(-b)).
__device__ __forceinline__ float dn_softplus(float y) { return fmaxf(y, 0.f) + log1pf(expf(-fabsf(y))); }
__device__ __forceinline__ float dn_gate_alpha(float a, float a_log, float a_bias) {
  return expf(-expf(a_log) * dn_softplus(a + a_bias));
}
__device__ __forceinline__ float dn_gate_beta(float b) { return 1.0f / (1.0f + expf(-b)); }

// Gates for N input rows (tokens or sequences): u = s[r] * prenorm(x) . W[r] for the 2 Hv gate
// rows, then alpha[n][h] from row h and beta[n][h] from row Hv + h.
struct GateArgs {
  const float* x;        // [N][x_stride], D columns used
  int x_stride, N, D;
  int prenorm;           // RMS-normalise x first
  float eps;
  const void* W;         // the gate rows: [2 Hv][D] int8 or [2 Hv][D/2] packed int4
  const float* s;        // [2 Hv]
  const float* a_log;    // [Hv]
  const float* a_bias;   // [Hv]
  int Hv;
  float* alpha;          // [N][Hv]
  float* beta;           // [N][Hv]
};
hipError_t launch_gates(const GateArgs& a, int bits, hipStream_t st);

// ---- batched path (B >= 2): int8-MFMA projections and a streaming state kernel ----
// act[b][k] split into three int8 terms per (sequence, 128-column chunk), in the GEMM's fragment order.
struct BSplitArgs {
  const float* act;      // [B][act_stride], K columns used
  int act_stride;
  int K, B;
  void* xs;              // [ceil(B/64)][K/128] blocks of 24 KB
  float* sc;             // [ceil(B/64)][K/128][64] split scales
  float* ssq;            // [B][K/128] sums of squares
};
// part[ks][b][r] = sum over the ks-th K range of W[r][k] * act[b][k], for M rows.
struct BGemmArgs {
  const void* W;         // [M][K] int8 or [M][K/2] packed int4
  const void* xs;        // split activations (BSplitArgs::xs)
  const float* sc;       // their scales (BSplitArgs::sc)
  float* part;           // [K/KR][B][M]
  int M, K, B, KR;
  // When act is set (8-bit weights, 256-column K ranges, two or three row blocks) the GEMM splits
  // its own K range of act [B][act_stride] instead of reading xs / sc, and the workgroups of the
  // first row block write the chunk sums of squares to ssq [B][K/128].
  const float* act;
  int act_stride;
  float* ssq;
};
// out[b][r] = epilogue(s[r] * sum_ks part[ks][b][r]).
struct BEpiArgs {
  const float* part;
  int KS, M, B;
  const int32_t* terms;  // instead of part when set: [3][B][M] exact sums of the three int8 terms
  const float* s1;       // [B] their per-row split scales (with terms)
  const float* s;        // [M]
  const float* ssq;      // [B][NC] (pre-norm only)
  int NC, K, prenorm;    // the pre-norm factor is 1/sqrt(sum ssq / K + eps)
  float eps;
  const float* conv_w;   // [C][Kc] or nullptr: rows r < C get the causal conv + SiLU
  float* ring;           // [B][Kc-1][C], oldest first
  int C, Kc;
  float* out;            // [B][out_stride]
  int out_stride;
};
struct BStateArgs {
  const float* u;        // [B][R]: post-conv q | k | v, then raw z
  float* S;              // [B][Hv][128][128]
  const float* alpha;    // [B][Hv], or [B][Hv][128] with alpha_per_key
  const float* beta;     // [B][Hv]
  const float* norm_w;   // [128]
  void* xs;              // out: the gated readout split for out_proj (BSplitArgs::xs layout, K = V)
  float* sc;             // out: its scales
  int B, Hk, Hv, R, C, QK, V;
  float eps_l2, eps_rms, q_scale;
  int alpha_per_key;     // 1: key row i of head h decays by alpha[b][h][i]
};
bool bgemm_shape_ok(int M, int K, int mf, int kr);
hipError_t launch_bsplit(const BSplitArgs& a, hipStream_t st);
hipError_t launch_bgemm(const BGemmArgs& a, int bits, int mf, hipStream_t st);
// all loads up front: K range KR (256 or 512), NRB (1..3) blocks of 64 rows per workgroup
bool bgemm2_shape_ok(int M, int K, int nrb, int kr);
hipError_t launch_bgemm2(const BGemmArgs& a, int bits, int nrb, hipStream_t st);
hipError_t launch_bepi(const BEpiArgs& a, hipStream_t st);
// The three-term split of whole rows (one scale per row) for the whole-K projection: xs as for
// launch_bsplit, sc [ceil(B/64)][64] row scales, ssq [B] row sums of squares; K a multiple of 1024.
hipError_t launch_bsplit_row(const BSplitArgs& a, hipStream_t st);
// out[b][r] = epilogue(s[r] * sum_k W[r][k] act[b][k]) over the whole K in one kernel: a
// workgroup takes 16*RT rows and 64 sequences, its eight waves a quarter of K and half of the
// sequences each (act split by launch_bsplit_row). g supplies W, xs, sc, M, K, B; e the epilogue
// (part and KS unused; ssq the row sums of launch_bsplit_row).
bool bproj_shape_ok(int M, int K, int* rt);
hipError_t launch_bproj(const BGemmArgs& g, const BEpiArgs& e, int bits, int rt, hipStream_t st);
hipError_t launch_bstate(const BStateArgs& a, hipStream_t st);

// Whole-row three-term split for the library GEMMs: row t of act becomes
// act[t][k] ~= s1[t] (h + (m + l/254)/254) with s1[t] = max_k |act[t][k]| / 127, the terms stored
// term-major as xs[i][t][k] (i = 0, 1, 2 for h, m, l), and ssq[t] = sum_k act[t][k]^2.
struct TSplitArgs {
  const float* act;      // [T][act_stride], K columns used
  int act_stride, K, T;  // K a multiple of 1024
  int8_t* xs;            // [3][T][K]
  float* s1;             // [T]
  float* ssq;            // [T]
};
hipError_t launch_tsplit(const TSplitArgs& a, hipStream_t st);

// int8 x int8 -> int32 library GEMMs (dn_lt.cpp): D [N][M] = W [M][K] (row-major int8) times
// X [N][K] (row-major int8), exact. Two shape slots per context (in_proj, out_proj); lt_prepare
// returns false when the library has no algorithm for the shape.
struct LtCtx;
LtCtx* lt_create();
void lt_destroy(LtCtx* c);
bool lt_prepare(LtCtx* c, int slot, int M, int N, int K);
hipError_t lt_gemm_i8(LtCtx* c, int slot, const void* W, const int8_t* X, int32_t* D, hipStream_t st);

// ---- prefill: T tokens of one sequence through a layer, chunkwise (128 x 128 state tiles) ----
// in_proj epilogue along the tokens: u[t][r] = s[r] * prenorm(t) * sum_ks part[ks][t][r], then for
// rows r < C the causal conv over the history (ring_in, oldest first) and the previous tokens, SiLU.
struct PConvArgs {
  const float* part;     // [KS][T][M]
  int KS, T, M;
  const int32_t* terms;  // instead of part when set: [3][T][M] exact sums of the three int8 terms
  const float* s1;       // [T] their per-token split scales (with terms)
  const float* s;        // [M]
  const float* ssq;      // [T][NC] sums of squares of the layer input per 128-column chunk
  int NC, K, prenorm;    // pre-norm factor 1/sqrt(sum ssq / K + eps)
  float eps;
  const float* conv_w;   // [C][Kc]
  const float* ring_in;  // [Kc-1][C]
  float* ring_out;       // [Kc-1][C]: the last Kc-1 pre-conv values after token T-1
  int C, Kc;
  float* out;            // [T][M]: post-conv q | k | v, raw z
};
// Chunk-local terms of the gated delta rule for (value head, chunk of 64 tokens).
struct PIntraArgs {
  const float* u;        // [T][R] post-conv q | k | v, raw z
  int T, R, QK, Hv, Hk;
  const float* alpha;    // token t, head h at alpha[t * gstride + h]
  const float* beta;
  int gstride;
  float eps_l2, q_scale;
  int NCH;               // chunks: ceil(T / 64)
  float* cw;             // per (h, chunk): W, Uv, Qg, Kt [64][128] each, P [64][64], gamma
};
// Sequential pass over the chunks for (value head, block of 16 value columns).
struct PScanArgs {
  const float* cw;       // PIntraArgs::cw
  float* S;              // the layer's state: [Hv][128][128] ([dk][dv]), or [Hv][dv][dk] if transposed
  int transposed;
  int T, Hv, NCH, V;
  float* o;              // [T][V] readout
};
// Gated RMSNorm per (token, value head): y = w * o / rms(o) * silu(z), in place over o.
struct PNormArgs {
  float* o;              // [T][V] readout in, gated output out
  const float* u;        // [T][R] (z at column C + h * 128)
  const float* norm_w;   // [128]
  int T, R, C, V;
  float eps_rms;
};
constexpr int PF_CT = 64;                                   // tokens per chunk
constexpr size_t PF_CHUNK_FLOATS = 4 * 64 * 128 + 64 * 64 + 4;  // per (head, chunk) in PIntraArgs::cw
hipError_t launch_pconv(const PConvArgs& a, hipStream_t st);
hipError_t launch_pintra(const PIntraArgs& a, hipStream_t st);
hipError_t launch_pscan(const PScanArgs& a, hipStream_t st);
hipError_t launch_pnorm(const PNormArgs& a, hipStream_t st);
// The prompt projections with 8-bit weights as one int8 matrix-core GEMM with the fold of the three
// terms in its epilogue: out[t][m] = s1[t] * (D0 + (D1 + D2 / 254) / 254), Dτ = sum_k W[m][k] X[τ][t][k]
// exact in int32, folded in double. X is k_tsplit's [3][T][K]; out has the layout of a single
// K-range partial sum ([1][T][M]) for k_pconv / k_bepi. K a multiple of 128, M of 4, M K and 3 T K
// below 2^31 (32-bit byte offsets); out 16-byte aligned.
struct PGemmArgs {
  const int8_t* W;  // [M][K]
  const int8_t* X;  // [3][T][K]
  const float* s1;  // [T]
  float* out;       // [T][M]
  int M, K, T;
  // in_proj epilogue when conv != 0 (what k_pconv does after the library GEMM): pre-conv values
  // s[m] f(t) sum (f the pre-norm factor 1/sqrt(ssq[t] / K + eps) if prenorm, else 1), then for rows
  // m < C the causal conv over the previous Kc - 1 tokens and SiLU, into out, for every token whose
  // history lies in its 64-token tile (local index >= 3); rows m >= C get the pre-conv value. The
  // pre-conv values of each tile's first and last three tokens and of the prompt's last three go to
  // edge ([T][M], other tokens' rows untouched) for k_pconv_edge, which finishes the first three.
  int conv;
  const float* s;       // [M] row scales; without conv, when set: out[t][m] = s[m] * the fold (the
                        // out_proj rows finished, as k_bepi finishes them)
  const float* ssq;     // [T] sums of squares of the layer input (one chunk: k_tsplit's)
  int prenorm;
  float eps;
  const float* conv_w;  // [C][Kc]
  int C, Kc;
  float* edge;          // [T][M]
};
bool pgemm_shape_ok(int M, int K, int T);
hipError_t launch_pgemm(const PGemmArgs& a, hipStream_t st);
// After k_pgemm's conv epilogue: the first three tokens of every 64-token tile (rows < C) from the
// edge values and, before the prompt, the history; and the new history (the last Kc - 1 pre-conv
// values). part = the edge buffer, out = k_pgemm's out; s, terms, ssq unused.
hipError_t launch_pconv_edge(const PConvArgs& a, hipStream_t st);

// ---- whole-stack kernel (single sequence, 128 x 128 state tiles) ----
struct LayerW {
  const void* w_in;
  const float* s_in;
  const float* conv_w;
  const float* norm_w;
  const void* w_out;
  const float* s_out;
  const float* a_log;    // [Hv] (gates on the device)
  const float* a_bias;   // [Hv]
};

// Control words of one handle in device memory: the tag base of the next launch, the count of
// workgroups that finished the current launch, a sticky error flag, and which of the two state and
// history buffers holds the current ones (a launch reads that one, writes the other, and the last
// workgroup to finish makes the written one current only if no workgroup failed).
struct Ctl {
  unsigned epoch;
  unsigned done;
  unsigned error;
  unsigned parity;
};

struct PersistArgs {
  const LayerW* layers;  // [L], device memory
  float* S[2];           // two buffers of [L][Hv][dv][dk] (each head's state stored transposed)
  float* ring[2];        // two buffers of [L][K-1][C], oldest first
  const float* x;        // [D]
  const float* alpha;    // [L][Hv], or [L][Hv][128] with alpha_per_key
  const float* beta;     // [L][Hv]
  float* out;            // [L][D]
  unsigned* X;           // [8][D]  layer output, self-tagged 32-bit words, one copy per XCD
  uint64_t* U;           // [R (+ 2 Hv)]  tagged in_proj output (post-conv q|k|v, raw z, raw gate rows)
  unsigned* G;           // [8][V + 512] gated readout and partial sums of squares of the readout,
                         // self-tagged 32-bit words, in four segments [V/4 columns | partials of
                         // those heads], one copy per XCD
  Ctl* ctl;
  unsigned* err_host;          // host-mapped pinned word: the launch's error flag, written by the last workgroup
  unsigned long long* timers;  // instrumented builds only: [NWG][L][32] phase timestamps
  int L, R, C, QK, K, Hk, Hv;
  unsigned flags;
  float eps_l2, eps_rms, q_scale;
  int alpha_per_key;     // 1: key row i of head h decays by alpha[l][h][i] (at most PK_MAXL layers)
  int gates;             // 1: gates from the in_proj rows R .. R + 2 Hv (U holds them after the R rows)
  unsigned spin_cap;     // poll rounds a hand-off may take before the launch aborts (PERSIST_SPIN_CAP)
};
constexpr int PK_MAXL = 32;  // layers of a whole-stack launch with one decay per key channel
// Poll rounds of one hand-off before the launch gives up (a round is about 1 us, so about a second):
// far beyond any exchange of a launch whose workgroups are all resident, short enough that a grid
// that cannot become resident fails in about a second.
constexpr unsigned PERSIST_SPIN_CAP = 1u << 20;

struct PersistShape {
  int batch, D, V, R, dk, dv, Hv, K, bits;
  int L, alpha_per_key, gates;
};

bool persist_supported(const PersistShape& s, int nwg);
hipError_t persist_occupancy(const PersistShape& s, int* blocks_per_cu);
// coop: launch cooperatively (every workgroup resident at once, or the launch fails)
hipError_t launch_persist(const PersistArgs& a, const PersistShape& s, int nwg, bool coop, hipStream_t st);
hipError_t launch_state_tile(const float* src, float* dst, int L, int Hv, int dk, int dv, bool to_tiled,
                             hipStream_t st);
// Make buffer 0 the current one: copy buffer 1 of the state (n_s floats) and of the history (n_ring
// floats) into buffer 0 if ctl->parity says buffer 1 is current, then set the parity to 0. For work
// that updates the state in place (prompts) on a whole-stack handle.
hipError_t launch_persist_settle(float* const S[2], float* const ring[2], size_t n_s, size_t n_ring, Ctl* ctl,
                                 hipStream_t st);

}  // namespace dn
