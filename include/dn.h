/*
 * dn.h -- C ABI of the gated-DeltaNet decode step on MI355X (gfx950).
 *
 * One handle holds what the page "qwen36: run the DeltaNet layer end to end on
 * the card (Q36_DN_GPU=1): conv, recurrence and gated norm join the two
 * projections" (section "What the PR does", Backend paragraph) puts in one
 * per-layer device object: the short-conv history, the recurrent state
 * [vh x kdim x vdim], and one token's scratch, with the weights alongside. A
 * handle may hold a stack of n_layers such layers (n_layers = 1 is exactly the
 * page's object); dn_step then runs one decode token through all of them, the
 * output of layer l feeding layer l+1 on the device.
 *
 * Five entry points mirror the page's five optional backend calls (the
 * "Verified" section counts them): create, set_state, get_state, step, destroy.
 * dn_strerror is static inline, so libdn exports exactly these five. Prompts go
 * through a handle on the card with the separate library libdn_prefill
 * (include/dn_prefill.h); the page leaves prompts to the CPU.
 *
 * All sizes are element counts. All matrices are row-major and C-contiguous.
 * The library never synchronises the device inside dn_step.
 *
 * Devices. A handle lives on the HIP device that was current at dn_create. Every other call
 * makes that device current for its own duration and restores the caller's current device
 * before it returns; a stream passed in must belong to the handle's device.
 */
#ifndef DN_H
#define DN_H

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define DN_OK          0
#define DN_E_INVAL    -1  /* bad dimensions, NULL or misaligned pointer */
#define DN_E_NOMEM    -2  /* device allocation failed */
#define DN_E_DEVICE   -3  /* a HIP error at launch or copy; the handle latches off */
#define DN_E_DISABLED -4  /* dn_step after a failed step; dn_set_state re-arms */
#define DN_E_FAULT    -5  /* injected failure (environment DN_FAULT_STEP=n fails the n-th dn_step, 1-based) */

/* Environment read by dn_create:
 *   DN_FAULT_STEP=n     fail the n-th dn_step of the handle before it launches anything
 *   DN_FAULT_STALL=n    whole-stack handles: the n-th dn_step's launch gives every hand-off between
 *                       workgroups a single poll round, so it aborts through the kernel's own error
 *                       path unless every exchange is already complete; the next call reports it
 *   DN_SYNC_DEBUG=1     synchronise after every launch and check for errors
 *   DN_LAYER_KERNELS=1  use the per-layer kernels even where the whole-stack kernel applies
 *   DN_VERBOSE=1        print which path the handle uses to stderr, and the HIP error of a failed launch
 *   DN_PERSIST_LAUNCH=cooperative
 *                       launch the whole-stack kernel cooperatively: the runtime starts it only when
 *                       the whole grid can be resident (about 20 us more per launch on MI355X; not
 *                       while the stream is being captured into a graph)
 *
 * Execution paths. A single-sequence handle (batch 1) with d_k = d_v = 128 and supported widths
 * runs each dn_step as one whole-stack kernel launch with one workgroup per compute unit, whose
 * workgroups wait for one another; they must all be resident at once, which an otherwise idle
 * device gives (two such steps must not run concurrently on one device: issue them on one stream).
 * If other work keeps part of the grid from starting for about a second, the launch gives up: it
 * leaves the state and history of the last completed token, later launches do nothing, and the
 * failure is reported (DN_E_DEVICE) by the next dn_step or by dn_get_state(h, NULL, NULL).
 * Other shapes run three kernels per layer. */

/* dn_config.flags */
#define DN_X_RMSNORM 1u   /* RMS-normalise each layer's input, x / sqrt(mean(x^2) + eps_rms) (stack pre-norm) */
/* One decay per key channel instead of one per head: key row i of value head h's state is
 * multiplied by alpha[l][b][h][i] before the delta step. This is the gate of the other engines'
 * linear-attention layers, which run the same gated delta step with other dimensions and gates
 * (page "qwen36: run the DeltaNet layer end to end on the card", section "Where this goes next").
 * alpha becomes [L][B][Hv][dk]. Single-sequence handles then run the per-layer kernels instead
 * of the whole-stack kernel. */
#define DN_ALPHA_PER_KEY 2u
/* Gates computed on the card. The page keeps the two gates (a/b, one output per value head each)
 * in the engine and passes them in (page "qwen36: run the DeltaNet layer end to end on the card",
 * section "What the PR does", Backend paragraph); in a stack run by one launch per token each
 * layer's gates depend on that layer's input, which exists only on the device. With this flag
 * the in_proj has two more row blocks after z, a (Hv rows) | b (Hv rows), per-row scaled like the
 * others and not convolved, and value head h of every sequence takes
 *   alpha = exp(-exp(a_log[h]) * softplus(a[h] + a_bias[h])),   beta = 1 / (1 + exp(-b[h]))
 * (softplus(y) = log(1 + e^y)). The page gives no formula; this is the decay form of
 * gated-delta-rule layers, stated as this library's reading. dn_step and dn_prefill then ignore
 * their alpha and beta arguments, which may be NULL. Not combinable with DN_ALPHA_PER_KEY. */
#define DN_GATES_ON_DEVICE 4u

typedef struct dn_layer dn_layer; /* opaque */

typedef struct {
  int d_model;      /* D: model width. Multiple of 16 (8-bit weights) or 32 (4-bit weights), <= 16384 */
  int n_k_heads;    /* Hk: key heads; n_v_heads % n_k_heads == 0 */
  int d_k;          /* dk: key head dim, 1..256 */
  int n_v_heads;    /* Hv: value heads, 1..64; value head h reads key head h / (Hv/Hk) */
  int d_v;          /* dv: value head dim, 1..256; Hv*dv a multiple of 16 (8-bit) or 32 (4-bit) */
  int conv_k;       /* K: causal conv kernel size, 1..4 */
  int batch;        /* B: independent sequences stepped together, 1..1024 */
  int n_layers;     /* L: layers in the stack, 1..256 */
  int weight_bits;  /* 8 (int8) or 4 (packed signed int4) */
  unsigned flags;   /* DN_X_RMSNORM, DN_ALPHA_PER_KEY, DN_GATES_ON_DEVICE (not with DN_ALPHA_PER_KEY), or 0 */
  float eps_l2;     /* eps inside the sqrt of the q/k L2 norms (1e-6) */
  float eps_rms;    /* eps of the gated RMSNorm and of the input pre-norm (1e-6) */
  float q_scale;    /* multiplies the readout q^T S (1.0) */
} dn_config;

/* One layer's weights: DEVICE pointers, BORROWED (the caller keeps them alive and
 * unchanged until dn_destroy), 16-byte aligned.
 *   R = 2*Hk*dk + 2*Hv*dv in_proj rows, ordered q (Hk*dk) | k (Hk*dk) | v (Hv*dv) | z (Hv*dv)
 *   ("qkv ++ z", page "feat(qwen36): the dense trunk places itself", section "What this adds"),
 *   and with DN_GATES_ON_DEVICE 2*Hv more rows a (Hv) | b (Hv);
 *   C = 2*Hk*dk + Hv*dv convolved channels (q, k, v); z is not convolved.
 * 8-bit weights are signed bytes; 4-bit weights are two per byte, element 2m in the
 * low nibble and 2m+1 in the high nibble, 4-bit two's complement. */
typedef struct {
  const void  *w_in;    /* [R][D] int8, or [R][D/2] packed int4 */
  const float *s_in;    /* [R] per-row scale: u[r] = s_in[r] * sum_c w_in[r][c] x[c] */
  const float *conv_w;  /* [C][K] depthwise taps; tap K-1 multiplies the current token */
  const float *norm_w;  /* [dv] gated RMSNorm weight, shared by all value heads */
  const void  *w_out;   /* [D][Hv*dv] int8, or [D][Hv*dv/2] packed int4 */
  const float *s_out;   /* [D] per-row scale */
  const float *a_log;   /* [Hv] decay gate parameters with DN_GATES_ON_DEVICE, else ignored (may be NULL) */
  const float *a_bias;  /* [Hv] */
} dn_weights;

/* Create a handle for cfg->n_layers layers; w points to n_layers dn_weights (host
 * memory, read during the call). The handle owns the state, the conv history and
 * the scratch (device memory on the current HIP device); state and history start
 * at zero. Returns DN_OK and *out, or DN_E_INVAL / DN_E_NOMEM / DN_E_DEVICE with
 * *out = NULL. */
int dn_create(const dn_config *cfg, const dn_weights *w, dn_layer **out);

/* Copy the state in (page "qwen36: run the DeltaNet layer end to end on the card", section
 * "What the PR does", Tier paragraph: the host copy of the state moves to and from the card with
 * set/get_state). S: [L][B][Hv][dk][dv] fp32; ring: [L][B][K-1][C] fp32, oldest token first (NULL
 * leaves the history unchanged). Host or device pointers, read during the call (not retained).
 * Synchronous: waits for all work on the device first. Re-arms a latched handle, and restarts the
 * whole-stack kernel's exchange state between workgroups as dn_create leaves it.
 * Returns DN_OK, DN_E_INVAL (NULL handle or S) or DN_E_DEVICE. */
int dn_set_state(dn_layer *h, const float *S, const float *ring);

/* Copy the state out, same layouts as dn_set_state (ring may be NULL). Host or device pointers,
 * written during the call. Synchronous: waits for all work on the device first. Valid after a
 * failed step: it returns what the device holds (page "qwen36: run the DeltaNet layer end to end
 * on the card", section "What the PR does", Tier paragraph: get_state works after a failed step).
 * With S and ring both NULL it copies nothing and only reports, after that wait, whether every
 * dn_step launched so far completed: DN_E_DEVICE (and the handle latches off) if a whole-stack
 * launch abandoned its token, else DN_OK. This is the synchronous form of the report the next
 * dn_step would otherwise give.
 * Returns DN_OK, DN_E_INVAL (NULL handle, or S NULL with ring not NULL) or DN_E_DEVICE. */
int dn_get_state(dn_layer *h, float *S, float *ring);

/* One decode token for every sequence, through every layer (page "qwen36: run the
 * DeltaNet layer end to end on the card", section "What the PR does": in_proj GEMV,
 * causal conv + SiLU with the history advancing, per value head L2 norms of q and k
 * with eps inside the sqrt, decay, delta rule against the decayed state, write-back,
 * out = q^T S over the updated state, gated RMSNorm with silu(z), out_proj GEMV).
 * DEVICE pointers:
 *   x            [B][D]        input of layer 0
 *   alpha, beta  [L][B][Hv]    per-head decay (multiplies S) and delta-rule step size;
 *                              alpha is [L][B][Hv][dk] with DN_ALPHA_PER_KEY; not read (may
 *                              be NULL) with DN_GATES_ON_DEVICE
 *   out          [L][B][D]     out[l] is layer l's output and layer l+1's input;
 *                              out[L-1] is the stack's output. Must not overlap x.
 * hip_stream: a hipStream_t (NULL = the default stream). Enqueue only: returns
 * before the work completes. Returns DN_OK, DN_E_INVAL, DN_E_DISABLED, DN_E_FAULT
 * or DN_E_DEVICE (the last two latch the handle off). A whole-stack launch whose
 * workgroups stop waiting for one another (a bounded wait ran out) abandons the
 * token and records an error in host memory at its end; the first dn_step after that
 * launch has completed returns DN_E_DEVICE. */
int dn_step(dn_layer *h, const float *x, const float *alpha, const float *beta, float *out, void *hip_stream);

/* Free everything the handle owns, including what libdn_prefill keeps in it (waits for the device
 * first); the borrowed weights stay the caller's. The end of the page's per-layer object (page
 * "qwen36: run the DeltaNet layer end to end on the card", section "What the PR does", Backend
 * paragraph). NULL-safe. */
void dn_destroy(dn_layer *h);

static inline const char *dn_strerror(int rc) {
  switch (rc) {
    case DN_OK: return "ok";
    case DN_E_INVAL: return "invalid argument";
    case DN_E_NOMEM: return "out of device memory";
    case DN_E_DEVICE: return "device error";
    case DN_E_DISABLED: return "layer disabled after a failed step";
    case DN_E_FAULT: return "injected fault";
    default: return "unknown error";
  }
}

#ifdef __cplusplus
}
#endif
#endif /* DN_H */
