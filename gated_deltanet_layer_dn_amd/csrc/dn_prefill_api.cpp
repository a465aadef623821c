// C-ABI host side of libdn_prefill: a prompt of T tokens through a handle made by libdn's
// dn_create (include/dn_prefill.h). The page keeps prompts on the CPU (page "qwen36: run the
// DeltaNet layer end to end on the card", section "What the PR does", Engine paragraph: a prompt,
// S > 1, keeps the batched CPU path); this is the same per-token computation on the card, with the
// recurrence evaluated in chunks of 64 tokens.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <new>
#include <string>

#include "dn.h"
#include "dn_handle.h"
#include "dn_internal.h"
#include "dn_prefill.h"
#include "dn_tsplit_norm.h"

#define DN_API extern "C" __attribute__((visibility("default")))

using dn::DeviceScope;
using dn::fail;
using dn::host_err;

namespace {

// Scratch of one prefill call, carved out of one buffer.
struct PfBufs {
  void* xs;     // split activations of the prompt (fragment blocks, or [3][T][K] for the library GEMM)
  float* sc;    // their scales
  float* ssq;   // their per-chunk sums of squares
  float* part;  // GEMM K-range partial sums [KS][T][M], or the three terms' int32 sums [3][T][M]
  float* u;     // [T][R] post-conv in_proj output
  float* cw;    // chunk terms of the recurrence
  float* o;     // [T][V] readout, then gated output
  float* ring;  // the new conv history of a layer
  float* al;    // [T][Hv] gates computed on the card
  float* be;
};

// K range of a prefill GEMM: the widest of 1024, 512, 256 columns that divides K.
int pf_kr(int K) { return K % 1024 == 0 ? 1024 : K % 512 == 0 ? 512 : 256; }

// Byte size of the scratch for prompts of up to T tokens; with base != nullptr also the pieces,
// each 256-byte aligned, carved from base.
size_t pf_layout(const dn_layer* h, int T, char* base, PfBufs* b) {
  const dn_config& c = h->cfg;
  const size_t D = c.d_model, V = h->V, R = h->R;
  const size_t nb = ((size_t)T + 63) / 64, nch = ((size_t)T + dn::PF_CT - 1) / dn::PF_CT;
  const size_t ncmax = std::max(D, V) / 128;
  // both GEMM paths: K-range partial sums (hand-written GEMM) or the three terms' int32 sums
  // (library GEMM); split activations in fragment blocks or as [3][T][K]
  const size_t part = (size_t)T * std::max(std::max((D / pf_kr((int)D)) * R, (V / pf_kr((int)V)) * D),
                                           3 * std::max(R, D));
  const size_t xs_bytes = std::max(nb * ncmax * 24576, 3 * (size_t)T * std::max(D, V));
  const size_t ring = std::max<size_t>(1, (size_t)(c.conv_k - 1) * h->C);
  const size_t gates = h->gates ? (size_t)T * c.n_v_heads : 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += (bytes + 255) & ~(size_t)255;
    return p;
  };
  PfBufs t{};
  t.xs = take(xs_bytes);
  t.sc = reinterpret_cast<float*>(take(sizeof(float) * std::max(nb * ncmax * 64, (size_t)T)));
  t.ssq = reinterpret_cast<float*>(take(sizeof(float) * T * ncmax));
  t.part = reinterpret_cast<float*>(take(sizeof(float) * part));
  t.u = reinterpret_cast<float*>(take(sizeof(float) * T * R));
  t.cw = reinterpret_cast<float*>(take(sizeof(float) * c.n_v_heads * nch * dn::PF_CHUNK_FLOATS));
  t.o = reinterpret_cast<float*>(take(sizeof(float) * T * V));
  t.ring = reinterpret_cast<float*>(take(sizeof(float) * ring));
  t.al = reinterpret_cast<float*>(take(sizeof(float) * gates));
  t.be = reinterpret_cast<float*>(take(sizeof(float) * gates));
  if (b) *b = t;
  return off;
}

// GEMM paths of the projections with 8-bit weights (4-bit weights always take the split-K one):
//   PF_GEMM_AUTO    the fused hand-written GEMM where its shape constraints hold, else the library
//                   GEMM where the library has an algorithm for the shape, else split-K
//   PF_GEMM_FUSED   int8 MFMA GEMM over the three terms with their fold in its epilogue (k_pgemm),
//                   where its shape constraints hold, else split-K
//   PF_GEMM_LIBRARY the library's int8 GEMM over the three terms, folded by the next kernel, where
//                   the library has an algorithm for the shape, else split-K
//   PF_GEMM_SPLITK  the hand-written split-K GEMM on fragment blocks with a separate reduction
enum { PF_GEMM_AUTO = 0, PF_GEMM_FUSED, PF_GEMM_LIBRARY, PF_GEMM_SPLITK };

int gemm_from_env() {
  const char* v = std::getenv("DN_PREFILL_GEMM");
  if (!v) return PF_GEMM_AUTO;
  const std::string m(v);
  return m == "fused" ? PF_GEMM_FUSED : m == "library" ? PF_GEMM_LIBRARY : m == "splitk" ? PF_GEMM_SPLITK : PF_GEMM_AUTO;
}

// The prompt path's state kept in the handle: scratch sized for the longest prompt so far (grown,
// never shrunk) and the library GEMMs of 8-bit projections (created at the first prefill).
struct PrefillExt {
  int cap = 0;
  void* buf = nullptr;
  dn::LtCtx* lt = nullptr;
  bool lt_tried = false;
  int gemm = 0;          // DN_PREFILL_GEMM: the projections' GEMM path (PF_GEMM_*)
  bool verbose = false;  // DN_VERBOSE=1: print the projection path of each call
};

void ext_free(void* p) {
  PrefillExt* e = static_cast<PrefillExt*>(p);
  if (!e) return;
  if (e->buf) (void)hipFree(e->buf);
  dn::lt_destroy(e->lt);
  delete e;
}

PrefillExt* ext_of(dn_layer* h) {
  if (!h->ext) {
    PrefillExt* e = new (std::nothrow) PrefillExt();
    if (!e) return nullptr;
    e->gemm = gemm_from_env();
    if (const char* v = std::getenv("DN_VERBOSE")) e->verbose = std::atoi(v) != 0;
    h->ext = e;
    h->ext_free = ext_free;
  }
  return static_cast<PrefillExt*>(h->ext);
}

int pf_reserve(dn_layer* h, PrefillExt* e, int T) {
  if (T <= e->cap) return DN_OK;
  if (e->buf) (void)hipFree(e->buf);
  e->buf = nullptr;
  e->cap = 0;
  if (hipMalloc(&e->buf, pf_layout(h, T, nullptr, nullptr)) != hipSuccess) return DN_E_NOMEM;
  e->cap = T;
  return DN_OK;
}

// Checks shared by the prefill entry points; DN_OK if the call may proceed.
int pf_check(dn_layer* h, const float* x, int n_tokens, const float* alpha, const float* beta, const float* out) {
  if (!h || !x || !out || n_tokens < 1 || n_tokens > DN_PREFILL_MAX_TOKENS) return DN_E_INVAL;
  if (!h->gates && (!alpha || !beta)) return DN_E_INVAL;
  if (h->disabled) return DN_E_DISABLED;
  const dn_config& c = h->cfg;
  const size_t L = c.n_layers, D = c.d_model, T = n_tokens, B = c.batch;
  if (c.d_k != 128 || c.d_v != 128 || (c.flags & DN_ALPHA_PER_KEY) || D % 256 || h->V % 256) return DN_E_INVAL;
  const char* xb = reinterpret_cast<const char*>(x);
  const char* ob = reinterpret_cast<const char*>(out);
  if (ob < xb + sizeof(float) * B * T * D && xb < ob + sizeof(float) * L * B * T * D) return DN_E_INVAL;
  return DN_OK;
}

// The prompt through every layer on the given scratch. gemm: PF_GEMM_*; lt: the library GEMM
// context, or nullptr (no library GEMM).
int pf_run(dn_layer* h, const PfBufs& pb, int gemm, dn::LtCtx* lt, bool verbose, const float* x, int n_tokens,
           const float* alpha, const float* beta, float* out, hipStream_t st) {
  const dn_config& c = h->cfg;
  const size_t L = c.n_layers, D = c.d_model, T = n_tokens, B = c.batch;
  const int QK = c.n_k_heads * c.d_k, V = h->V, R = h->R, K = c.conv_k;
  const int nch = (n_tokens + dn::PF_CT - 1) / dn::PF_CT;
  const int kr_in = pf_kr((int)D), kr_out = pf_kr(V);
  auto check = [&]() { return !h->sync_debug || hipStreamSynchronize(st) == hipSuccess; };
  // 8-bit weights: the projections as int8 GEMMs over the three terms of every token (the fused
  // hand-written one or the library's), each where its shape constraints hold; else split-K
  const bool w8 = c.weight_bits == 8;
  const bool fu_in = w8 && gemm != PF_GEMM_LIBRARY && gemm != PF_GEMM_SPLITK && dn::pgemm_shape_ok(R, (int)D, n_tokens);
  const bool fu_out = w8 && gemm != PF_GEMM_LIBRARY && gemm != PF_GEMM_SPLITK && dn::pgemm_shape_ok((int)D, V, n_tokens);
  const bool lib_ok = w8 && lt && (gemm == PF_GEMM_AUTO || gemm == PF_GEMM_LIBRARY);
  const bool lt_in = !fu_in && lib_ok && dn::lt_prepare(lt, 0, R, 3 * n_tokens, (int)D);
  const bool lt_out = !fu_out && lib_ok && dn::lt_prepare(lt, 1, (int)D, 3 * n_tokens, V);
  const bool tri_in = fu_in || lt_in, tri_out = fu_out || lt_out;  // [3][T][K] split, sums folded
  if (verbose)
    std::fprintf(stderr, "[dn] prefill of %d token(s): in_proj %s, out_proj %s\n", n_tokens,
                 fu_in ? "fused int8 GEMM" : lt_in ? "library int8 GEMM" : "split-K int8 GEMM",
                 fu_out ? "fused int8 GEMM after the fused norm-and-split"
                 : lt_out ? "library int8 GEMM after the fused norm-and-split" : "split-K int8 GEMM");
  if (h->persist) {
    // the prompt updates the state and history in place: make the first of the whole-stack
    // kernel's two buffers the current one
    float* const Sb[2] = {h->S, h->S_alt};
    float* const Rb[2] = {h->ring, h->ring_alt};
    if (dn::launch_persist_settle(Sb, Rb, L * h->s_elems, L * h->ring_elems, h->ctl, st) != hipSuccess)
      return fail(h, DN_E_DEVICE);
  }
  int8_t* const tx = static_cast<int8_t*>(pb.xs);
  int32_t* const td = reinterpret_cast<int32_t*>(pb.part);
  const size_t ring_seq = (size_t)(K - 1) * h->C, s_seq = (size_t)c.n_v_heads * c.d_k * c.d_v;
  // the sequences of a batch one after the other, each through every layer; out[l][b] is layer l's
  // output for sequence b and layer l+1's input
  for (size_t sb = 0; sb < B; ++sb)
  for (size_t l = 0; l < L; ++l) {
    const dn_weights& w = h->w[l];
    const float* xl = l == 0 ? x + sb * T * D : out + ((l - 1) * B + sb) * T * D;
    float* const ring_l = h->ring + l * h->ring_elems + sb * ring_seq;
    // in_proj: split the prompt's inputs, int8 GEMM over the tokens, conv along the tokens (the
    // fused GEMM's epilogue does the conv within each 64-token tile, k_pconv_edge the tiles' first
    // three tokens; else k_pconv after the GEMM)
    dn::PConvArgs pc{};
    if (tri_in) {
      dn::TSplitArgs sp{xl, (int)D, (int)D, n_tokens, tx, pb.sc, pb.ssq};
      if (dn::launch_tsplit(sp, st) != hipSuccess) return fail(h, DN_E_DEVICE);
      if (fu_in) {
        dn::PGemmArgs g{static_cast<const int8_t*>(w.w_in), tx, pb.sc, pb.u, R, (int)D, n_tokens};
        g.conv = 1; g.s = w.s_in; g.ssq = pb.ssq; g.prenorm = (c.flags & DN_X_RMSNORM) ? 1 : 0; g.eps = c.eps_rms;
        g.conv_w = w.conv_w; g.C = h->C; g.Kc = K; g.edge = pb.part;
        if (dn::launch_pgemm(g, st) != hipSuccess) return fail(h, DN_E_DEVICE);
        pc.part = pb.part; pc.KS = 1;
      } else {
        if (dn::lt_gemm_i8(lt, 0, w.w_in, tx, td, st) != hipSuccess) return fail(h, DN_E_DEVICE);
        pc.terms = td; pc.s1 = pb.sc; pc.KS = 0;
      }
      pc.NC = 1;
    } else {
      dn::BSplitArgs sp{xl, (int)D, (int)D, n_tokens, pb.xs, pb.sc, pb.ssq};
      if (dn::launch_bsplit(sp, st) != hipSuccess) return fail(h, DN_E_DEVICE);
      dn::BGemmArgs gi{w.w_in, pb.xs, pb.sc, pb.part, R, (int)D, n_tokens, kr_in};
      if (dn::launch_bgemm(gi, c.weight_bits, 1, st) != hipSuccess) return fail(h, DN_E_DEVICE);
      pc.part = pb.part; pc.KS = (int)D / kr_in; pc.NC = (int)D / 128;
    }
    pc.T = n_tokens; pc.M = R;
    pc.s = w.s_in; pc.ssq = pb.ssq; pc.K = (int)D;
    pc.prenorm = (c.flags & DN_X_RMSNORM) ? 1 : 0; pc.eps = c.eps_rms;
    pc.conv_w = w.conv_w; pc.ring_in = ring_l; pc.ring_out = pb.ring;
    pc.C = h->C; pc.Kc = K; pc.out = pb.u;
    if ((fu_in ? dn::launch_pconv_edge(pc, st) : dn::launch_pconv(pc, st)) != hipSuccess) return fail(h, DN_E_DEVICE);
    if (K > 1 && hipMemcpyAsync(ring_l, pb.ring, sizeof(float) * ring_seq, hipMemcpyDeviceToDevice, st) != hipSuccess)
      return fail(h, DN_E_DEVICE);
    if (!check()) return fail(h, DN_E_DEVICE);
    // recurrence in chunks, then the gated RMSNorm
    dn::PIntraArgs pi{};
    pi.u = pb.u; pi.T = n_tokens; pi.R = R; pi.QK = QK; pi.Hv = c.n_v_heads; pi.Hk = c.n_k_heads;
    if (h->gates) {
      if (dn::launch_layer_gates(h, l, xl, n_tokens, pb.al, pb.be, st) != hipSuccess) return fail(h, DN_E_DEVICE);
      pi.alpha = pb.al; pi.beta = pb.be; pi.gstride = c.n_v_heads;
    } else {
      pi.alpha = alpha + (l * B + sb) * c.n_v_heads; pi.beta = beta + (l * B + sb) * c.n_v_heads;
      pi.gstride = (int)(L * B) * c.n_v_heads;
    }
    pi.eps_l2 = c.eps_l2; pi.q_scale = c.q_scale; pi.NCH = nch; pi.cw = pb.cw;
    if (dn::launch_pintra(pi, st) != hipSuccess) return fail(h, DN_E_DEVICE);
    dn::PScanArgs ps{};
    ps.cw = pb.cw; ps.S = h->S + l * h->s_elems + sb * s_seq; ps.transposed = h->persist ? 1 : 0;
    ps.T = n_tokens; ps.Hv = c.n_v_heads; ps.NCH = nch; ps.V = V; ps.o = pb.o;
    if (dn::launch_pscan(ps, st) != hipSuccess) return fail(h, DN_E_DEVICE);
    // the gated RMSNorm: its own pass, or fused into the split for the library GEMM (the readout
    // rows and z are aligned, V, R and C being multiples of 128; V <= 64 heads x 128 = 8192 columns)
    if (!tri_out) {
      dn::PNormArgs pn{pb.o, pb.u, w.norm_w, n_tokens, R, h->C, V, c.eps_rms};
      if (dn::launch_pnorm(pn, st) != hipSuccess) return fail(h, DN_E_DEVICE);
    }
    if (!check()) return fail(h, DN_E_DEVICE);
    // out_proj
    dn::BEpiArgs e{};
    if (tri_out) {
      dn::TSplitArgs so{pb.o, V, V, n_tokens, tx, pb.sc, pb.ssq};
      const dn::TSplitNormArgs sn{so, pb.u + h->C, R, w.norm_w, c.eps_rms};
      if (dn::launch_tsplit_norm(sn, st) != hipSuccess) return fail(h, DN_E_DEVICE);
      if (fu_out) {
        // the GEMM's epilogue applies the row scale and writes the layer's output: no k_bepi
        dn::PGemmArgs g{static_cast<const int8_t*>(w.w_out), tx, pb.sc, out + (l * B + sb) * T * D, (int)D, V, n_tokens};
        g.s = w.s_out;
        if (dn::launch_pgemm(g, st) != hipSuccess) return fail(h, DN_E_DEVICE);
      } else {
        if (dn::lt_gemm_i8(lt, 1, w.w_out, tx, td, st) != hipSuccess) return fail(h, DN_E_DEVICE);
        e.terms = td; e.s1 = pb.sc; e.KS = 0;
      }
    } else {
      dn::BSplitArgs so{pb.o, V, V, n_tokens, pb.xs, pb.sc, pb.ssq};
      if (dn::launch_bsplit(so, st) != hipSuccess) return fail(h, DN_E_DEVICE);
      dn::BGemmArgs go{w.w_out, pb.xs, pb.sc, pb.part, (int)D, V, n_tokens, kr_out};
      if (dn::launch_bgemm(go, c.weight_bits, 1, st) != hipSuccess) return fail(h, DN_E_DEVICE);
      e.part = pb.part; e.KS = V / kr_out;
    }
    e.M = (int)D; e.B = n_tokens; e.s = w.s_out;
    e.out = out + (l * B + sb) * T * D; e.out_stride = (int)D;
    if (!fu_out && dn::launch_bepi(e, st) != hipSuccess) return fail(h, DN_E_DEVICE);
    if (!check()) return fail(h, DN_E_DEVICE);
  }
  return DN_OK;
}

}  // namespace

DN_API int dn_prefill(dn_layer* h, const float* x, int n_tokens, const float* alpha, const float* beta, float* out,
                      void* hip_stream) {
  if (int rc = pf_check(h, x, n_tokens, alpha, beta, out); rc != DN_OK) return rc;
  DeviceScope dev(h->device);
  if (!dev.ok()) return fail(h, DN_E_DEVICE);
  if (h->persist && host_err(h)) return fail(h, DN_E_DEVICE);
  PrefillExt* e = ext_of(h);
  if (!e) return DN_E_NOMEM;
  if (int rc = pf_reserve(h, e, n_tokens); rc != DN_OK) {
    (void)hipGetLastError();  // the failed allocation's error; the handle stays usable
    return rc;
  }
  if (h->cfg.weight_bits == 8 && (e->gemm == PF_GEMM_AUTO || e->gemm == PF_GEMM_LIBRARY) && !e->lt_tried) {
    e->lt_tried = true;
    e->lt = dn::lt_create();
  }
  PfBufs pb{};
  pf_layout(h, n_tokens, static_cast<char*>(e->buf), &pb);
  return pf_run(h, pb, e->gemm, e->lt, e->verbose, x, n_tokens, alpha, beta, out,
                reinterpret_cast<hipStream_t>(hip_stream));
}

// ---- prompts without allocation (dn_prefill_noalloc) ----
//
// The scratch lives in a file-scope device array, one per device the library runs on, held until
// the process ends. Host code reaches it only through the address hipGetSymbolAddress gives on that
// device (the array's name is a host-side stand-in, not a device address).
namespace {

__device__ __align__(256) unsigned char scratch[DN_PREFILL_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The device address of this device's scratch array, looked up once per device with that device
// current (the caller's DeviceScope); nullptr if the lookup fails.
void* scratch_on(int device) {
  if (device < 0 || device >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[device] = p;
  }
  return g_scratch_ptr[device];
}

}  // namespace

DN_API int dn_prefill_noalloc(dn_layer* h, const float* x, int n_tokens, const float* alpha, const float* beta,
                              float* out, void* hip_stream) {
  if (int rc = pf_check(h, x, n_tokens, alpha, beta, out); rc != DN_OK) return rc;
  const size_t need = pf_layout(h, n_tokens, nullptr, nullptr);
  if (need > (size_t)DN_PREFILL_NOALLOC_SCRATCH_BYTES) {
    if (h->verbose)
      std::fprintf(stderr,
                   "[dn] dn_prefill_noalloc: %d tokens need %zu bytes of scratch, more than the %d bytes it has;"
                   " pass fewer tokens per call\n",
                   n_tokens, need, DN_PREFILL_NOALLOC_SCRATCH_BYTES);
    return DN_E_INVAL;
  }
  DeviceScope dev(h->device);
  if (!dev.ok()) return fail(h, DN_E_DEVICE);
  if (h->persist && host_err(h)) return fail(h, DN_E_DEVICE);
  char* base = static_cast<char*>(scratch_on(h->device));
  if (!base) return fail(h, DN_E_DEVICE);
  PfBufs pb{};
  pf_layout(h, n_tokens, base, &pb);
  if (h->verbose) std::fprintf(stderr, "[dn] dn_prefill_noalloc: %zu bytes of the device's scratch array\n", need);
  // no library GEMM here: its path gives the fused GEMM's results bit for bit, so that one stands in
  const int gemm = gemm_from_env() == PF_GEMM_LIBRARY ? PF_GEMM_FUSED : gemm_from_env();
  return pf_run(h, pb, gemm, nullptr, h->verbose, x, n_tokens, alpha, beta, out, reinterpret_cast<hipStream_t>(hip_stream));
}
