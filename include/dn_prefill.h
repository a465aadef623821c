/*
 * dn_prefill.h -- C ABI of libdn_prefill: prompts through a gated-DeltaNet handle on the card.
 *
 * The page "qwen36: run the DeltaNet layer end to end on the card (Q36_DN_GPU=1): conv, recurrence
 * and gated norm join the two projections" keeps a prompt (more than one token) on the CPU (section
 * "What the PR does", Engine paragraph); this library runs the same per-token computation for a
 * whole prompt on the card, through a handle made by libdn's dn_create (include/dn.h). It is a
 * separate library so that libdn exports exactly the page's five calls. Load libdn first: the
 * handle, its state and its history are libdn's, and dn_destroy releases what this library keeps
 * in the handle.
 */
#ifndef DN_PREFILL_H
#define DN_PREFILL_H

#include "dn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Prefill: run a prompt of T tokens of ONE sequence through every layer (all T tokens
 * through layer 0, then layer 1, ...), starting from the state and conv history the
 * handle holds and leaving them after the last prompt token, so that dn_step continues
 * the sequence. Each token gets exactly the decode step of dn_step (page "qwen36: run
 * the DeltaNet layer end to end on the card", section "What the PR does", Backend paragraph);
 * the recurrence is evaluated in chunks of 64 tokens, which is the per-token step rewritten
 * and agrees with it up to rounding.
 * Requires d_k == d_v == 128, a scalar decay (no DN_ALPHA_PER_KEY), d_model and n_v_heads * d_v
 * multiples of 256. With batch B > 1 every sequence gets a prompt of the same T tokens.
 * DEVICE pointers:
 *   x            [B][T][D]     the prompts' inputs of layer 0, one sequence after the other
 *   alpha, beta  [T][L][B][Hv] per token, the gates of dn_step (not read, may be NULL, with
 *                              DN_GATES_ON_DEVICE)
 *   out          [L][B][T][D]  out[l][b] is layer l's output for sequence b's tokens and layer
 *                              l+1's input. Must not overlap x.
 * T = n_tokens, 1..DN_PREFILL_MAX_TOKENS per call; a longer prompt goes in several calls, each
 * continuing from the state the previous one left. The handle keeps scratch memory sized for the
 * longest prompt seen so far (allocated here, freed by dn_destroy).
 * Projections with 8-bit weights: this library's int8 matrix-core GEMM over the three int8 terms of
 * each input row, the terms folded in its epilogue; the environment variable DN_PREFILL_GEMM, read at
 * a handle's first prefill, selects another path for comparison: "library" (the GPU BLAS library's
 * int8 GEMM over the same terms, folded by the next kernel the same way: results equal the default's
 * bit for bit) or "splitk" (split-K GEMM on fragment blocks, as for 4-bit weights).
 * hip_stream: a hipStream_t (NULL = the default stream). Enqueue only. Returns DN_OK,
 * DN_E_INVAL (shape or arguments not supported; the handle stays usable), DN_E_NOMEM,
 * DN_E_DISABLED or DN_E_DEVICE (latches the handle off, as a failed dn_step does). */
#define DN_PREFILL_MAX_TOKENS 65535
int dn_prefill(dn_layer *h, const float *x, int n_tokens, const float *alpha, const float *beta, float *out,
               void *hip_stream);

/* dn_prefill without any allocation, for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid it. Same arguments, layouts, state
 * handling and return codes as dn_prefill, and the same computation in the same kernels (never the
 * library GEMM, whose workspace and setup would allocate): results equal those of dn_prefill bit for
 * bit.
 * Its scratch is one static device array of DN_PREFILL_NOALLOC_SCRATCH_BYTES per device the library
 * runs on, held until the process ends; the call calls no allocator (neither HIP's nor a library's).
 * A call whose scratch would exceed the array returns DN_E_INVAL without launching anything (and,
 * with DN_VERBOSE=1, says how many bytes it needed): pass the prompt in pieces of fewer tokens, each
 * call continuing from the state the previous one left. For the 30-layer stack's layer shape (d_model
 * 2048, 16 x 128 key and 32 x 128 value heads) a call takes up to about 200 tokens.
 * Every call on one device shares that device's array, which keeps the last call's contents (nothing
 * in it needs to start at zero): calls that overlap in time on one device race and must not be
 * issued (use one stream per device, or order them). */
#define DN_PREFILL_NOALLOC_SCRATCH_BYTES (64 << 20)
int dn_prefill_noalloc(dn_layer *h, const float *x, int n_tokens, const float *alpha, const float *beta, float *out,
                       void *hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* DN_PREFILL_H */
