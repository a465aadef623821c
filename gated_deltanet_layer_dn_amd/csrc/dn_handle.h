// The handle's layout, shared by the host code of libdn (dn_api.cpp: the five calls of the
// per-layer object) and of libdn_prefill (dn_prefill_api.cpp: prompts through a handle). Both
// libraries are built together from these sources, so a handle created by one is read by the
// other with the same layout.
//
// The handle is the per-layer device object of page "qwen36: run the DeltaNet layer end to end
// on the card" (section "What the PR does", Backend and Tier paragraphs): it owns the conv
// history, the recurrent state and one token's scratch; the state moves only through
// dn_set_state / dn_get_state, and dn_get_state still works after a failed step.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

#include "dn.h"
#include "dn_internal.h"

struct dn_layer {
  dn_config cfg;
  std::vector<dn_weights> w;
  int device = 0;
  int R = 0, C = 0, V = 0;  // R: in_proj rows q|k|v|z (gate rows, if any, follow them)
  bool gates = false;       // DN_GATES_ON_DEVICE: 2 Hv gate rows after the R rows
  float* gal = nullptr;     // [B][Hv] scratch: gates computed on the card (per-layer and batched paths)
  float* gbe = nullptr;
  size_t s_elems = 0;     // per layer: B*Hv*dk*dv
  size_t ring_elems = 0;  // per layer: B*(K-1)*C
  float* S = nullptr;     // [L][B][Hv][dk][dv] ([L][Hv][dv][dk] with the whole-stack kernel)
  float* ring = nullptr;  // [L][B][K-1][C], oldest first
  float* u = nullptr;     // [B][R] scratch: post-conv q|k|v, raw z
  float* y = nullptr;     // [B][V] scratch: gated RMSNorm output
  float* yssq = nullptr;  // [B][Hv][dv/16] scratch: the readout's partial sums of squares
  // whole-stack kernel (single sequence, 128 x 128 state tiles)
  bool persist = false;
  int nwg = 0;
  bool coop = false;        // launched cooperatively (the runtime places every workgroup at once)
  float* S_alt = nullptr;   // the second state buffer: a launch reads the current one (Ctl::parity)
  float* ring_alt = nullptr;  // and writes the other; a launch that fails leaves the current one intact
  dn::PersistShape ps{};
  dn::LayerW* d_layers = nullptr;
  unsigned* X = nullptr;    // hand-off buffers: layer output and gated readout in self-tagged
                            // 32-bit words, in_proj output in 64-bit tagged words
  uint64_t* U = nullptr;
  unsigned* G = nullptr;
  dn::Ctl* ctl = nullptr;
  float* stage = nullptr;   // canonical-layout staging of the state for set/get
  unsigned* err_host = nullptr;  // pinned host word the whole-stack kernel writes its error flag to
  unsigned* err_dev = nullptr;   // the same word as the device addresses it
  unsigned long long* timers = nullptr;  // instrumented builds: phase timestamps of the last step
  // batched path (B >= 2, 128 x 128 state tiles): MFMA projections with split-K partial sums
  bool batched = false;
  int mf1 = 0, kr1 = 0, mf2 = 0, kr2 = 0;  // rows per workgroup / 64 and K range of in_proj, out_proj
  bool up1 = false, up2 = false;           // the projection uses the all-loads-up-front GEMM (NRB = mf)
  int rt1 = 0;                             // in_proj as one whole-K kernel with 16*rt1-row tiles (0: split-K GEMM)
  float* part = nullptr;                   // split-K partial sums
  void* xs = nullptr;                      // activations split into int8 terms, fragment order
  float* sc = nullptr;                     // their per-(sequence, 128-column chunk) scales
  float* ssq = nullptr;                    // per-(sequence, chunk) sums of squares (input pre-norm)
  // the prompt path's own state (libdn_prefill), released by dn_destroy through ext_free
  void* ext = nullptr;
  void (*ext_free)(void*) = nullptr;
  bool disabled = false;
  long steps = 0;
  long fault_step = 0;    // 1-based step to fail (0 = never)
  long fault_stall = 0;   // 1-based step whose whole-stack launch may not wait in any hand-off (0 = never)
  bool sync_debug = false;
  bool verbose = false;   // DN_VERBOSE=1: the path at creation, and the HIP error of a failed launch
};

namespace dn {

// Makes the handle's device current for the duration of a call and restores the caller's current
// device on every return path, so that no entry point changes the calling thread's device.
class DeviceScope {
 public:
  explicit DeviceScope(int dev) {
    if (hipGetDevice(&prev_) != hipSuccess) {
      prev_ = -1;
      ok_ = false;
      return;
    }
    ok_ = prev_ == dev || hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceScope() {
    int cur = -1;
    if (prev_ >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev_) (void)hipSetDevice(prev_);
  }
  bool ok() const { return ok_; }
  DeviceScope(const DeviceScope&) = delete;
  DeviceScope& operator=(const DeviceScope&) = delete;

 private:
  int prev_ = -1;
  bool ok_ = false;
};

// The whole-stack kernel stores its error flag into host memory at the end of each launch; the
// host reads it without synchronising, so a failure is seen at the first call after that launch.
inline unsigned host_err(const dn_layer* h) { return *reinterpret_cast<volatile const unsigned*>(h->err_host); }

// A failed step latches the handle off until dn_set_state re-arms it.
inline int fail(dn_layer* h, int rc) {
  h->disabled = true;
  return rc;
}

// Gates of N input rows of layer l (DN_GATES_ON_DEVICE) into alpha_out/beta_out [N][Hv].
inline hipError_t launch_layer_gates(const dn_layer* h, size_t l, const float* xl, int N, float* alpha_out,
                                     float* beta_out, hipStream_t st) {
  const dn_config& c = h->cfg;
  const dn_weights& w = h->w[l];
  const size_t rowbytes = c.weight_bits == 8 ? (size_t)c.d_model : (size_t)c.d_model / 2;
  GateArgs g{};
  g.x = xl; g.x_stride = c.d_model; g.N = N; g.D = c.d_model;
  g.prenorm = (c.flags & DN_X_RMSNORM) ? 1 : 0; g.eps = c.eps_rms;
  g.W = static_cast<const uint8_t*>(w.w_in) + (size_t)h->R * rowbytes; g.s = w.s_in + h->R;
  g.a_log = w.a_log; g.a_bias = w.a_bias; g.Hv = c.n_v_heads;
  g.alpha = alpha_out; g.beta = beta_out;
  return launch_gates(g, c.weight_bits, st);
}

}  // namespace dn
