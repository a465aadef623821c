// C-ABI host side of libdn: handle lifecycle, validation, state movement, launch sequence of
// dn_step. The handle's layout is in dn_handle.h (shared with libdn_prefill).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "dn.h"
#include "dn_handle.h"
#include "dn_internal.h"

#define DN_API extern "C" __attribute__((visibility("default")))

using dn::DeviceScope;
using dn::fail;
using dn::host_err;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int validate(const dn_config* c) {
  if (!c) return DN_E_INVAL;
  if (c->weight_bits != 8 && c->weight_bits != 4) return DN_E_INVAL;
  const int col_mult = c->weight_bits == 8 ? 16 : 32;
  if (c->d_model <= 0 || c->d_model > 16384 || c->d_model % col_mult) return DN_E_INVAL;
  if (c->n_k_heads <= 0 || c->n_v_heads <= 0 || c->n_v_heads > 64) return DN_E_INVAL;
  if (c->n_v_heads % c->n_k_heads) return DN_E_INVAL;
  if (c->d_k <= 0 || c->d_k > 256 || c->d_v <= 0 || c->d_v > 256) return DN_E_INVAL;
  const long V = (long)c->n_v_heads * c->d_v;
  if (V % col_mult || V > 16384) return DN_E_INVAL;
  if (c->conv_k < 1 || c->conv_k > 4) return DN_E_INVAL;
  if (c->batch < 1 || c->batch > 1024) return DN_E_INVAL;
  if (c->n_layers < 1 || c->n_layers > 256) return DN_E_INVAL;
  if (c->flags & ~(DN_X_RMSNORM | DN_ALPHA_PER_KEY | DN_GATES_ON_DEVICE)) return DN_E_INVAL;
  if ((c->flags & DN_ALPHA_PER_KEY) && (c->flags & DN_GATES_ON_DEVICE)) return DN_E_INVAL;
  if (!(c->eps_l2 >= 0.f) || !(c->eps_rms >= 0.f)) return DN_E_INVAL;
  return DN_OK;
}

template <typename T>
void dfree(T*& p) {
  if (p) (void)hipFree(p);
  p = nullptr;
}

void free_all(dn_layer* h) {
  dfree(h->S);
  dfree(h->ring);
  dfree(h->u);
  dfree(h->y);
  dfree(h->yssq);
  dfree(h->gal);
  dfree(h->gbe);
  dfree(h->S_alt);
  dfree(h->ring_alt);
  dfree(h->d_layers);
  dfree(h->X);
  dfree(h->U);
  dfree(h->G);
  dfree(h->ctl);
  dfree(h->stage);
  if (h->err_host) (void)hipHostFree(h->err_host);
  h->err_host = nullptr;
  dfree(h->timers);
  dfree(h->part);
  dfree(h->xs);
  dfree(h->sc);
  dfree(h->ssq);
  if (h->ext && h->ext_free) h->ext_free(h->ext);
  h->ext = nullptr;
  h->ext_free = nullptr;
}

// GEMM shape for an M x K projection: the all-loads-up-front kernel with 256-column K ranges and
// NRB blocks of 64 rows (3 for in_proj, 2 for out_proj when the row count allows), else the chunked
// kernel. Measured on MI355X at 64 sequences: in_proj 14.7 us (chunked 18.9), out_proj 6.9 us (9.1).
#ifndef DN_BGEMM_KR_IN
// K range of the in_proj GEMM's workgroups (256 or 512). 512 halves the split-K partial sums but
// leaves one workgroup per compute unit: 107 against 97 us per step at 64 sequences on MI355X.
#define DN_BGEMM_KR_IN 256
#endif
void pick_gemm(int M, int K, int* mf, int* kr, bool* up, int which) {
  *kr = 0;
  const int kr2 = which == 1 ? DN_BGEMM_KR_IN : 256;
  for (int n : {which == 1 ? 3 : 2, 2, 1})
    if (!*kr && dn::bgemm2_shape_ok(M, K, n, kr2)) { *mf = n; *kr = kr2; *up = true; }
  if (*kr) return;
  *mf = 1;
  for (int c : {1024, 512, 256})
    if (!*kr && dn::bgemm_shape_ok(M, K, 1, c)) *kr = c;
  *up = false;
  (void)which;
}

// Set up the batched path when the shape allows it: the in_proj GEMM takes 64-row blocks and the
// largest K range of 1024/512/256 columns that divides d_model (few partial sums); out_proj, with
// few rows, takes 64-row blocks and 256-column K ranges so that enough workgroups stream its
// weights (measured on MI355X at 64 sequences: in_proj 22 -> 16.5 us against 128-row blocks,
// out_proj 14.5 -> 8.8 us against 1024-column ranges).
int setup_batched(dn_layer* h) {
  const dn_config& c = h->cfg;
  const char* force = std::getenv("DN_LAYER_KERNELS");
  if ((force && std::atoi(force) != 0) || c.batch < 2 || c.d_k != 128 || c.d_v != 128) return DN_OK;
  const int D = c.d_model, R = h->R, V = h->V;
  int mf1 = 1, kr1 = 0, mf2 = 1, kr2 = 0;
  bool up1 = false, up2 = false;
  pick_gemm(R, D, &mf1, &kr1, &up1, 1);
  pick_gemm(D, V, &mf2, &kr2, &up2, 2);
  if (!kr1 || !kr2) return DN_OK;
  const size_t B = c.batch, nb = (B + 63) / 64, nc = std::max(D, V) / 128;
  const size_t part_elems = std::max((size_t)(D / kr1) * B * R, (size_t)(V / kr2) * B * D);
  bool ok = hipMalloc(&h->part, sizeof(float) * part_elems) == hipSuccess;
  ok = ok && hipMalloc(&h->xs, (size_t)24576 * nb * nc) == hipSuccess;
  ok = ok && hipMalloc(&h->sc, sizeof(float) * 64 * nb * nc) == hipSuccess;
  ok = ok && hipMalloc(&h->ssq, sizeof(float) * B * nc) == hipSuccess;
  if (!ok) return DN_E_NOMEM;
  h->mf1 = mf1; h->kr1 = kr1; h->mf2 = mf2; h->kr2 = kr2; h->up1 = up1; h->up2 = up2;
  // in_proj, with enough rows for every compute unit, as one whole-K kernel with its epilogue.
  // DN_BPROJ=0 keeps the split-K GEMM and the separate epilogue; DN_BPROJ=1 takes the whole-K
  // kernel for every shape it supports (fewer rows too).
  int rt = 0;
  const char* bp = std::getenv("DN_BPROJ");
  const int bpv = bp ? std::atoi(bp) : -1;
  if (bpv != 0 && c.weight_bits == 8 && dn::bproj_shape_ok(R, D, &rt) && (rt == 3 || bpv == 1)) h->rt1 = rt;
  h->batched = true;
  return DN_OK;
}

// Set up the whole-stack kernel when the shape allows it: hand-off buffers, control words,
// the device copy of the weight table, and the staging buffer of the tiled state.
int setup_persist(dn_layer* h) {
  const dn_config& c = h->cfg;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, h->device) != hipSuccess) return DN_E_DEVICE;
  h->nwg = prop.multiProcessorCount;
  dn::PersistShape& ps = h->ps;
  ps.batch = c.batch; ps.D = c.d_model; ps.V = h->V; ps.R = h->R; ps.dk = c.d_k; ps.dv = c.d_v;
  ps.Hv = c.n_v_heads; ps.K = c.conv_k; ps.bits = c.weight_bits;
  ps.L = c.n_layers; ps.alpha_per_key = (c.flags & DN_ALPHA_PER_KEY) ? 1 : 0; ps.gates = h->gates ? 1 : 0;
  const char* force = std::getenv("DN_LAYER_KERNELS");
  if ((force && std::atoi(force) != 0) || !dn::persist_supported(ps, h->nwg)) return DN_OK;
  int per_cu = 0;
  if (dn::persist_occupancy(ps, &per_cu) != hipSuccess || per_cu < 1) return DN_OK;
  const size_t L = c.n_layers;
  bool ok = hipMalloc(&h->d_layers, sizeof(dn::LayerW) * L) == hipSuccess;
  ok = ok && hipMalloc(&h->S_alt, sizeof(float) * L * h->s_elems) == hipSuccess;
  ok = ok && hipMalloc(&h->ring_alt, sizeof(float) * (L * h->ring_elems + 1)) == hipSuccess;
  ok = ok && hipMalloc(&h->X, sizeof(unsigned) * 8 * (c.d_model)) == hipSuccess;
  const size_t u_words = h->R + (h->gates ? 2 * c.n_v_heads : 0);
  ok = ok && hipMalloc(&h->U, sizeof(uint64_t) * u_words) == hipSuccess;
  ok = ok && hipMalloc(&h->G, sizeof(unsigned) * 8 * (h->V + 512)) == hipSuccess;
  ok = ok && hipMalloc(&h->ctl, sizeof(dn::Ctl)) == hipSuccess;
  ok = ok && hipMalloc(&h->stage, sizeof(float) * L * h->s_elems) == hipSuccess;
  ok = ok && hipHostMalloc(&h->err_host, sizeof(unsigned), hipHostMallocMapped | hipHostMallocCoherent) == hipSuccess;
  ok = ok && hipHostGetDevicePointer(reinterpret_cast<void**>(&h->err_dev), h->err_host, 0) == hipSuccess;
#ifdef DN_PHASE_TIMERS
  ok = ok && hipMalloc(&h->timers, sizeof(unsigned long long) * h->nwg * L * 32) == hipSuccess;
  ok = ok && hipMemset(h->timers, 0, sizeof(unsigned long long) * h->nwg * L * 32) == hipSuccess;
#endif
  if (!ok) return DN_E_NOMEM;
  // The kernel's waits between workgroups need every workgroup resident at once. An ordinary launch
  // gets that on a device with no other work (one workgroup per compute unit, occupancy checked
  // above); where other work may share the device, a launch whose grid cannot become resident ends
  // through the bounded waits, leaves the state of the last completed token and is reported.
  // DN_PERSIST_LAUNCH=cooperative makes the runtime start the grid only when all of it fits, at
  // about 20 us more per launch on MI355X.
  int coop = 0;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, h->device) != hipSuccess) coop = 0;
  const char* lm = std::getenv("DN_PERSIST_LAUNCH");
  h->coop = coop != 0 && lm && std::strcmp(lm, "cooperative") == 0;
  std::vector<dn::LayerW> lw(L);
  for (size_t l = 0; l < L; ++l)
    lw[l] = dn::LayerW{h->w[l].w_in,  h->w[l].s_in,  h->w[l].conv_w, h->w[l].norm_w,
                       h->w[l].w_out, h->w[l].s_out, h->w[l].a_log,  h->w[l].a_bias};
  const dn::Ctl ctl0{1u, 0u, 0u, 0u};
  ok = hipMemcpy(h->d_layers, lw.data(), sizeof(dn::LayerW) * L, hipMemcpyHostToDevice) == hipSuccess;
  ok = ok && hipMemset(h->X, 0, sizeof(unsigned) * 8 * (c.d_model)) == hipSuccess;
  ok = ok && hipMemset(h->U, 0, sizeof(uint64_t) * u_words) == hipSuccess;
  ok = ok && hipMemset(h->G, 0, sizeof(unsigned) * 8 * (h->V + 512)) == hipSuccess;
  ok = ok && hipMemcpy(h->ctl, &ctl0, sizeof(ctl0), hipMemcpyHostToDevice) == hipSuccess;
  if (!ok) return DN_E_DEVICE;
  *h->err_host = 0;
  h->persist = true;
  return DN_OK;
}

// The hand-off state of the whole-stack kernel as dn_create leaves it: buffers zeroed, tag base 1,
// no error. The x and gated-readout words carry only their tag mod 4, and after an aborted launch
// words of any of its layers may remain; some of those would match the tags the next launch's
// first polls wait for, so re-arming the handle starts the exchange state afresh.
int reset_handoff(dn_layer* h) {
  const dn_config& c = h->cfg;
  const size_t u_words = h->R + (h->gates ? 2 * c.n_v_heads : 0);
  const dn::Ctl ctl0{1u, 0u, 0u, 0u};
  bool ok = hipMemset(h->X, 0, sizeof(unsigned) * 8 * (c.d_model)) == hipSuccess;
  ok = ok && hipMemset(h->U, 0, sizeof(uint64_t) * u_words) == hipSuccess;
  ok = ok && hipMemset(h->G, 0, sizeof(unsigned) * 8 * (h->V + 512)) == hipSuccess;
  ok = ok && hipMemcpy(h->ctl, &ctl0, sizeof(ctl0), hipMemcpyHostToDevice) == hipSuccess;
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  if (!ok) return DN_E_DEVICE;
  *h->err_host = 0;
  return DN_OK;
}

}  // namespace

DN_API int dn_create(const dn_config* cfg, const dn_weights* w, dn_layer** out) {
  if (!out) return DN_E_INVAL;
  *out = nullptr;
  if (validate(cfg) != DN_OK || !w) return DN_E_INVAL;
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dn_weights& x = w[l];
    if (!x.w_in || !x.s_in || !x.conv_w || !x.norm_w || !x.w_out || !x.s_out) return DN_E_INVAL;
    if (!aligned16(x.w_in) || !aligned16(x.w_out)) return DN_E_INVAL;
    if (!aligned16(x.s_in) || !aligned16(x.s_out)) return DN_E_INVAL;
    if ((cfg->flags & DN_GATES_ON_DEVICE) && (!x.a_log || !x.a_bias)) return DN_E_INVAL;
  }
  dn_layer* h = new (std::nothrow) dn_layer();
  if (!h) return DN_E_NOMEM;
  h->cfg = *cfg;
  h->w.assign(w, w + cfg->n_layers);
  if (hipGetDevice(&h->device) != hipSuccess) {
    delete h;
    return DN_E_DEVICE;
  }
  const int QK = cfg->n_k_heads * cfg->d_k;
  h->V = cfg->n_v_heads * cfg->d_v;
  h->C = 2 * QK + h->V;
  h->R = h->C + h->V;
  h->gates = (cfg->flags & DN_GATES_ON_DEVICE) != 0;
  const size_t L = cfg->n_layers, B = cfg->batch;
  h->s_elems = B * cfg->n_v_heads * (size_t)cfg->d_k * cfg->d_v;
  h->ring_elems = B * (size_t)(cfg->conv_k - 1) * h->C;
  bool ok = hipMalloc(&h->S, sizeof(float) * L * h->s_elems) == hipSuccess;
  ok = ok && hipMalloc(&h->ring, sizeof(float) * (L * h->ring_elems + 1)) == hipSuccess;
  ok = ok && hipMalloc(&h->u, sizeof(float) * B * h->R) == hipSuccess;
  ok = ok && hipMalloc(&h->y, sizeof(float) * B * h->V) == hipSuccess;
  if (cfg->d_k % 16 == 0 && cfg->d_v % 16 == 0 && cfg->d_k <= 256 && cfg->n_v_heads <= 64)
    ok = ok && hipMalloc(&h->yssq, sizeof(float) * B * cfg->n_v_heads * (cfg->d_v / 16)) == hipSuccess;
  if (h->gates) {
    ok = ok && hipMalloc(&h->gal, sizeof(float) * B * cfg->n_v_heads) == hipSuccess;
    ok = ok && hipMalloc(&h->gbe, sizeof(float) * B * cfg->n_v_heads) == hipSuccess;
  }
  if (!ok) {
    (void)hipGetLastError();
    free_all(h);
    delete h;
    return DN_E_NOMEM;
  }
  ok = hipMemset(h->S, 0, sizeof(float) * L * h->s_elems) == hipSuccess;
  ok = ok && hipMemset(h->ring, 0, sizeof(float) * (L * h->ring_elems + 1)) == hipSuccess;
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    free_all(h);
    delete h;
    return DN_E_DEVICE;
  }
  if (int rc = setup_persist(h); rc != DN_OK) {
    (void)hipGetLastError();
    free_all(h);
    delete h;
    return rc;
  }
  if (int rc = setup_batched(h); rc != DN_OK) {
    (void)hipGetLastError();
    free_all(h);
    delete h;
    return rc;
  }
  if (hipDeviceSynchronize() != hipSuccess) {
    free_all(h);
    delete h;
    return DN_E_DEVICE;
  }
  if (const char* e = std::getenv("DN_FAULT_STEP")) h->fault_step = std::atol(e);
  if (const char* e = std::getenv("DN_FAULT_STALL")) h->fault_stall = std::atol(e);
  if (const char* e = std::getenv("DN_SYNC_DEBUG")) h->sync_debug = std::atoi(e) != 0;
  if (const char* e = std::getenv("DN_VERBOSE"); e && std::atoi(e) != 0) h->verbose = true;
  if (h->verbose)
    std::fprintf(stderr, "[dn] handle: %d layer(s), batch %d: %s%s\n", cfg->n_layers, cfg->batch,
                 h->persist ? "whole-stack kernel" : h->batched ? "batched kernels" : "per-layer kernels",
                 h->persist   ? (h->coop ? ", cooperative launch" : ", ordinary launch")
                 : h->batched ? (h->rt1 ? ", in_proj whole-K" : ", in_proj split-K")
                              : "");
  *out = h;
  return DN_OK;
}

DN_API int dn_set_state(dn_layer* h, const float* S, const float* ring) {
  if (!h || !S) return DN_E_INVAL;
  DeviceScope dev(h->device);
  if (!dev.ok() || hipDeviceSynchronize() != hipSuccess) return DN_E_DEVICE;
  const size_t L = h->cfg.n_layers;
  if (h->persist) {
    if (hipMemcpy(h->stage, S, sizeof(float) * L * h->s_elems, hipMemcpyDefault) != hipSuccess) return DN_E_DEVICE;
    if (dn::launch_state_tile(h->stage, h->S, (int)L, h->cfg.n_v_heads, h->cfg.d_k, h->cfg.d_v, true, nullptr) !=
        hipSuccess)
      return DN_E_DEVICE;
    if (reset_handoff(h) != DN_OK) return DN_E_DEVICE;
  } else if (hipMemcpy(h->S, S, sizeof(float) * L * h->s_elems, hipMemcpyDefault) != hipSuccess) {
    return DN_E_DEVICE;
  }
  if (ring && h->ring_elems &&
      hipMemcpy(h->ring, ring, sizeof(float) * L * h->ring_elems, hipMemcpyDefault) != hipSuccess)
    return DN_E_DEVICE;
  if (hipDeviceSynchronize() != hipSuccess) return DN_E_DEVICE;
  h->disabled = false;
  return DN_OK;
}

DN_API int dn_get_state(dn_layer* h, float* S, float* ring) {
  if (!h || (!S && ring)) return DN_E_INVAL;
  DeviceScope dev(h->device);
  if (!dev.ok()) return DN_E_DEVICE;
  if (!S) {
    // status only: every launch so far has completed after the wait, so the whole-stack kernel's
    // host-mapped error word is final
    if (hipDeviceSynchronize() != hipSuccess) return fail(h, DN_E_DEVICE);
    if (h->persist && host_err(h)) return fail(h, DN_E_DEVICE);
    return DN_OK;
  }
  (void)hipDeviceSynchronize();  // a failed step may have left an error; copy what the device holds
  (void)hipGetLastError();
  const size_t L = h->cfg.n_layers;
  const float* ring_cur = h->ring;
  if (h->persist) {
    // the current one of the two buffers (a failed launch left it as before its token)
    dn::Ctl ctl{};
    if (hipMemcpy(&ctl, h->ctl, sizeof(ctl), hipMemcpyDeviceToHost) != hipSuccess) return DN_E_DEVICE;
    const float* S_cur = (ctl.parity & 1u) ? h->S_alt : h->S;
    ring_cur = (ctl.parity & 1u) ? h->ring_alt : h->ring;
    if (dn::launch_state_tile(S_cur, h->stage, (int)L, h->cfg.n_v_heads, h->cfg.d_k, h->cfg.d_v, false, nullptr) !=
            hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
      return DN_E_DEVICE;
    if (hipMemcpy(S, h->stage, sizeof(float) * L * h->s_elems, hipMemcpyDefault) != hipSuccess) return DN_E_DEVICE;
  } else if (hipMemcpy(S, h->S, sizeof(float) * L * h->s_elems, hipMemcpyDefault) != hipSuccess) {
    return DN_E_DEVICE;
  }
  if (ring && h->ring_elems &&
      hipMemcpy(ring, ring_cur, sizeof(float) * L * h->ring_elems, hipMemcpyDefault) != hipSuccess)
    return DN_E_DEVICE;
  return hipDeviceSynchronize() == hipSuccess ? DN_OK : DN_E_DEVICE;
}

namespace {
// One batched projection: split the activations, split-K MFMA GEMM, epilogue; or, with rt > 0,
// split the activations and run the whole-K kernel that ends in the epilogue.
// act == nullptr: the activations are already split (the state kernel splits the gated readout).
int batched_proj(dn_layer* h, const void* W, const float* s, const float* act, int K, int M, int mf, int kr, bool up,
                 bool prenorm, const float* conv_w, float* ring, float* outp, int out_stride, hipStream_t st,
                 int rt = 0) {
  const dn_config& c = h->cfg;
  if (rt > 0) {
    if (act) {
      dn::BSplitArgs sp{};
      sp.act = act; sp.act_stride = K; sp.K = K; sp.B = c.batch; sp.xs = h->xs; sp.sc = h->sc; sp.ssq = h->ssq;
      if (dn::launch_bsplit_row(sp, st) != hipSuccess) return DN_E_DEVICE;
    }
    dn::BGemmArgs g{};
    g.W = W; g.xs = h->xs; g.sc = h->sc; g.M = M; g.K = K; g.B = c.batch;
    dn::BEpiArgs e{};
    e.M = M; e.B = c.batch; e.s = s; e.ssq = h->ssq; e.NC = K / 128; e.K = K; e.prenorm = prenorm ? 1 : 0;
    e.eps = c.eps_rms; e.conv_w = conv_w; e.ring = ring; e.C = h->C; e.Kc = c.conv_k; e.out = outp;
    e.out_stride = out_stride;
    if (dn::launch_bproj(g, e, c.weight_bits, rt, st) != hipSuccess) return DN_E_DEVICE;
    if (h->sync_debug && hipStreamSynchronize(st) != hipSuccess) return DN_E_DEVICE;
    return DN_OK;
  }
  // the up-front GEMM splits its own K range of the activations (8-bit weights, 256-column ranges,
  // at least two row blocks); otherwise a separate split kernel runs first
  const bool fuse = act && up && c.weight_bits == 8 && kr == 256 && mf >= 2;
  if (act && !fuse) {
    dn::BSplitArgs sp{};
    sp.act = act; sp.act_stride = K; sp.K = K; sp.B = c.batch; sp.xs = h->xs; sp.sc = h->sc; sp.ssq = h->ssq;
    if (dn::launch_bsplit(sp, st) != hipSuccess) return DN_E_DEVICE;
  }
  dn::BGemmArgs g{};
  g.W = W; g.xs = h->xs; g.sc = h->sc; g.part = h->part; g.M = M; g.K = K; g.B = c.batch; g.KR = kr;
  if (fuse) {
    g.act = act; g.act_stride = K; g.ssq = h->ssq;
  }
  if ((up ? dn::launch_bgemm2(g, c.weight_bits, mf, st) : dn::launch_bgemm(g, c.weight_bits, mf, st)) != hipSuccess)
    return DN_E_DEVICE;
  dn::BEpiArgs e{};
  e.part = h->part; e.KS = K / kr; e.M = M; e.B = c.batch; e.s = s;
  e.ssq = h->ssq; e.NC = K / 128; e.K = K; e.prenorm = prenorm ? 1 : 0; e.eps = c.eps_rms;
  e.conv_w = conv_w; e.ring = ring; e.C = h->C; e.Kc = c.conv_k; e.out = outp; e.out_stride = out_stride;
  if (dn::launch_bepi(e, st) != hipSuccess) return DN_E_DEVICE;
  if (h->sync_debug && hipStreamSynchronize(st) != hipSuccess) return DN_E_DEVICE;
  return DN_OK;
}
}  // namespace


DN_API int dn_step(dn_layer* h, const float* x, const float* alpha, const float* beta, float* out, void* hip_stream) {
  if (!h || !x || !out) return DN_E_INVAL;
  if (!h->gates && (!alpha || !beta)) return DN_E_INVAL;
  if (h->disabled) return DN_E_DISABLED;
  const dn_config& c = h->cfg;
  const size_t L = c.n_layers, B = c.batch, D = c.d_model;
  // out must not overlap x
  const char* xb = reinterpret_cast<const char*>(x);
  const char* ob = reinterpret_cast<const char*>(out);
  if (ob < xb + sizeof(float) * B * D && xb < ob + sizeof(float) * L * B * D) return DN_E_INVAL;
  ++h->steps;
  if (h->fault_step > 0 && h->steps == h->fault_step) return fail(h, DN_E_FAULT);
  DeviceScope dev(h->device);
  if (!dev.ok()) return fail(h, DN_E_DEVICE);
  hipStream_t st = reinterpret_cast<hipStream_t>(hip_stream);
  if (h->persist) {
    if (host_err(h)) {  // a completed launch reported a stalled hand-off
      if (h->verbose) std::fprintf(stderr, "[dn] dn_step: an earlier whole-stack launch abandoned its token\n");
      return fail(h, DN_E_DEVICE);
    }
    dn::PersistArgs a{};
    a.layers = h->d_layers; a.x = x; a.alpha = alpha; a.beta = beta; a.out = out;
    a.S[0] = h->S; a.S[1] = h->S_alt; a.ring[0] = h->ring; a.ring[1] = h->ring_alt;
    a.X = h->X; a.U = h->U; a.G = h->G; a.ctl = h->ctl; a.err_host = h->err_dev; a.timers = h->timers;
    a.L = (int)L; a.R = h->R; a.C = h->C; a.QK = c.n_k_heads * c.d_k; a.K = c.conv_k;
    a.Hk = c.n_k_heads; a.Hv = c.n_v_heads; a.flags = c.flags;
    a.eps_l2 = c.eps_l2; a.eps_rms = c.eps_rms; a.q_scale = c.q_scale;
    a.alpha_per_key = (c.flags & DN_ALPHA_PER_KEY) ? 1 : 0;
    a.gates = h->gates ? 1 : 0;
    // an injected stall: every hand-off gets a single poll round, so the launch aborts through its
    // own error path (reported by the next call) as soon as one exchange is not already complete
    a.spin_cap = (h->fault_stall > 0 && h->steps == h->fault_stall) ? 0u : dn::PERSIST_SPIN_CAP;
    // a cooperative launch cannot be recorded into a graph here: under capture the launch is an
    // ordinary one, and co-residency rests on the device being otherwise idle when it replays
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipError_t e = hipStreamIsCapturing(st, &cap); e != hipSuccess) {
      if (h->verbose) std::fprintf(stderr, "[dn] dn_step: stream capture query failed: %s\n", hipGetErrorString(e));
      return fail(h, DN_E_DEVICE);
    }
    const bool coop = h->coop && cap == hipStreamCaptureStatusNone;
    hipError_t e = dn::launch_persist(a, h->ps, h->nwg, coop, st);
    if (e != hipSuccess && coop) {
      // The runtime may refuse a cooperative launch (for one, while another process on the device
      // holds the global wave sync its cooperative launches use). Nothing was launched: the handle
      // falls back to ordinary launches, whose co-residency rests on the device being otherwise idle
      // and whose bounded waits end a launch that cannot be resident.
      (void)hipGetLastError();
      if (h->verbose)
        std::fprintf(stderr, "[dn] dn_step: cooperative launch refused (%s); ordinary launches from now on\n",
                     hipGetErrorString(e));
      h->coop = false;
      e = dn::launch_persist(a, h->ps, h->nwg, false, st);
    }
    if (e != hipSuccess) {
      if (h->verbose) std::fprintf(stderr, "[dn] dn_step: launch failed: %s\n", hipGetErrorString(e));
      return fail(h, DN_E_DEVICE);
    }
    if (h->sync_debug && (hipStreamSynchronize(st) != hipSuccess || host_err(h))) return fail(h, DN_E_DEVICE);
    return DN_OK;
  }
  const int pk = (c.flags & DN_ALPHA_PER_KEY) ? 1 : 0;
  const size_t a_layer = B * c.n_v_heads * (pk ? (size_t)c.d_k : 1);  // alpha elements per layer
  if (h->batched) {
    const int QK = c.n_k_heads * c.d_k;
    for (size_t l = 0; l < L; ++l) {
      const dn_weights& w = h->w[l];
      if (int rc = batched_proj(h, w.w_in, w.s_in, l == 0 ? x : out + (l - 1) * B * D, (int)D, h->R, h->mf1, h->kr1,
                                h->up1, (c.flags & DN_X_RMSNORM) != 0, w.conv_w, h->ring + l * h->ring_elems, h->u, h->R, st,
                                h->rt1);
          rc != DN_OK)
        return fail(h, rc);
      dn::BStateArgs bs{};
      bs.u = h->u; bs.S = h->S + l * h->s_elems;
      if (h->gates) {
        if (dn::launch_layer_gates(h, l, l == 0 ? x : out + (l - 1) * B * D, (int)B, h->gal, h->gbe, st) != hipSuccess)
          return fail(h, DN_E_DEVICE);
        bs.alpha = h->gal; bs.beta = h->gbe;
      } else {
        bs.alpha = alpha + l * a_layer; bs.beta = beta + l * B * c.n_v_heads;
      }
      bs.alpha_per_key = pk;
      bs.norm_w = w.norm_w; bs.xs = h->xs; bs.sc = h->sc;
      bs.B = (int)B; bs.Hk = c.n_k_heads; bs.Hv = c.n_v_heads; bs.R = h->R; bs.C = h->C; bs.QK = QK; bs.V = h->V;
      bs.eps_l2 = c.eps_l2; bs.eps_rms = c.eps_rms; bs.q_scale = c.q_scale;
      if (dn::launch_bstate(bs, st) != hipSuccess) return fail(h, DN_E_DEVICE);
      if (h->sync_debug && hipStreamSynchronize(st) != hipSuccess) return fail(h, DN_E_DEVICE);
      if (int rc = batched_proj(h, w.w_out, w.s_out, nullptr, h->V, (int)D, h->mf2, h->kr2, h->up2, false, nullptr, nullptr,
                                out + l * B * D, (int)D, st);
          rc != DN_OK)
        return fail(h, rc);
      if (h->sync_debug && hipStreamSynchronize(st) != hipSuccess) return fail(h, DN_E_DEVICE);
    }
    return DN_OK;
  }
  for (size_t l = 0; l < L; ++l) {
    const dn_weights& w = h->w[l];
    const float* xl = l == 0 ? x : out + (l - 1) * B * D;
    dn::GemvArgs gi{};
    gi.W = w.w_in; gi.s = w.s_in; gi.x = xl; gi.out = h->u;
    gi.rows = h->R; gi.cols = (int)D; gi.batch = (int)B;
    gi.x_stride = (int)D; gi.out_stride = h->R;
    gi.prenorm = (c.flags & DN_X_RMSNORM) ? 1 : 0; gi.eps = c.eps_rms;
    gi.conv_w = w.conv_w; gi.ring = h->ring + l * h->ring_elems; gi.C = h->C; gi.K = c.conv_k;
    if (dn::launch_gemv(gi, c.weight_bits, st) != hipSuccess) return fail(h, DN_E_DEVICE);
    if (h->sync_debug && hipStreamSynchronize(st) != hipSuccess) return fail(h, DN_E_DEVICE);

    dn::HeadArgs ha{};
    ha.u = h->u; ha.S = h->S + l * h->s_elems;
    if (h->gates) {
      if (dn::launch_layer_gates(h, l, xl, (int)B, h->gal, h->gbe, st) != hipSuccess) return fail(h, DN_E_DEVICE);
      ha.alpha = h->gal; ha.beta = h->gbe;
    } else {
      ha.alpha = alpha + l * a_layer; ha.beta = beta + l * B * c.n_v_heads;
    }
    ha.alpha_per_key = pk;
    ha.norm_w = w.norm_w; ha.y = h->y;
    ha.Hk = c.n_k_heads; ha.Hv = c.n_v_heads; ha.dk = c.d_k; ha.dv = c.d_v;
    ha.R = h->R; ha.C = h->C; ha.batch = (int)B;
    ha.eps_l2 = c.eps_l2; ha.eps_rms = c.eps_rms; ha.q_scale = c.q_scale;
    ha.ssq = h->yssq;  // the column-split kernel when the shape allows it
    if (dn::launch_head(ha, st) != hipSuccess) return fail(h, DN_E_DEVICE);
    if (h->sync_debug && hipStreamSynchronize(st) != hipSuccess) return fail(h, DN_E_DEVICE);

    dn::GemvArgs go{};
    go.W = w.w_out; go.s = w.s_out; go.x = h->y; go.out = out + l * B * D;
    go.rows = (int)D; go.cols = h->V; go.batch = (int)B;
    go.x_stride = h->V; go.out_stride = (int)D;
    go.prenorm = 0; go.eps = 0.f;
    go.conv_w = nullptr; go.ring = nullptr; go.C = 0; go.K = 0;
    if (h->yssq) {  // the heads' 1/rms, from the column blocks' sums of squares
      go.head_ssq = h->yssq; go.head_dim = c.d_v; go.head_nb = c.d_v / 16; go.head_eps = c.eps_rms;
    }
    if (dn::launch_gemv(go, c.weight_bits, st) != hipSuccess) return fail(h, DN_E_DEVICE);
    if (h->sync_debug && hipStreamSynchronize(st) != hipSuccess) return fail(h, DN_E_DEVICE);
  }
  return DN_OK;
}

DN_API void dn_destroy(dn_layer* h) {
  if (!h) return;
  DeviceScope dev(h->device);
  (void)hipDeviceSynchronize();
#ifdef DN_PHASE_TIMERS
  if (const char* path = std::getenv("DN_PHASE_TIMERS"); path && h->timers) {
    std::vector<unsigned long long> t((size_t)h->nwg * h->cfg.n_layers * 32);
    if (hipMemcpy(t.data(), h->timers, t.size() * sizeof(t[0]), hipMemcpyDeviceToHost) == hipSuccess) {
      if (FILE* f = std::fopen(path, "wb")) {
        std::fwrite(t.data(), sizeof(t[0]), t.size(), f);
        std::fclose(f);
      }
    }
  }
#endif
  free_all(h);
  delete h;
}
