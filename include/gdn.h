/*
 * libgdn: the gated delta rule on AMD Instinct MI355X (gfx950).
 *
 * The gated delta rule is the recurrent mixer of the Qwen3.5 / Qwen3-Next hybrid
 * blocks (Qwen3.5 text encyclopedia page, note "The DeltaNet mixer"; Qwen3-Next
 * encyclopedia page, note "The DeltaNet mixer fuses its projections per key head").
 * Per value head it keeps a float32 state S of shape [d_k, d_v] and, per token t,
 *
 *     S <- exp(g_t) S                        g_t: the token's log decay ("decays")
 *     S <- S + k_t (beta_t (v_t - S^T k_t))^T  beta_t: the write strength ("betas")
 *     o_t = S^T q_t                          read after the write
 *
 * where q_t and k_t are optionally L2-normalised in the kernel (GDN_QK_L2NORM:
 * x / sqrt(sum x^2 + 1e-6)) and q_t is multiplied by `scale` (the pages use
 * 1/sqrt(128)).  Query/key heads are shared by groups of value heads the way
 * repeat_interleave shares them: value head h reads query/key head
 * h / (H_v / H_qk).  The call shapes mirror the pages' kernel call: q, k, v
 * (elements 0-2), g, beta, initial_state in; the output and the state leaving
 * the layer out, or the state after every token (Qwen3.5 text encyclopedia
 * page, value table of model.layers[i].linear_attn).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *    never allocates, frees or synchronises: it validates on the host, enqueues
 *    its kernels on `stream`, and returns.
 *  - Tensors are dense and row-major in exactly the layouts stated below.
 *  - Validation runs on the host before any launch: on failure the call
 *    returns a status, records a message for gdn_last_error(), and writes
 *    nothing.  A failed launch returns GDN_ERR_HIP.  Device faults surface at
 *    the caller's next synchronisation.  No C++ exception crosses this ABI.
 *  - Calls are reentrant; gdn_last_error() is per host thread.
 *  - Alignment: pointers read or written with 16-byte vector accesses must be
 *    16-byte aligned (chunked paths: q, k, v, states, workspace; decode step:
 *    state); o to 4 of its elements (every path); every other pointer to its
 *    element size.  A misaligned pointer returns GDN_ERR_ALIGN.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL                        */
  GDN_ERR_SHAPE = 2,       /* a size is negative, zero where it may not be, or
                              H_v is not a multiple of H_qk                      */
  GDN_ERR_DTYPE = 3,       /* unknown dtype / o_dtype value                     */
  GDN_ERR_UNSUPPORTED = 4, /* valid, but no kernel is built for this (d_k, d_v,
                              chunk, dtype) combination                          */
  GDN_ERR_ALIAS = 5,       /* an output overlaps an input it may not overlap    */
  GDN_ERR_ALIGN = 6,       /* a pointer is not 16-byte aligned                  */
  GDN_ERR_WORKSPACE = 7,   /* workspace missing or smaller than the query says  */
  GDN_ERR_HIP = 8          /* a HIP launch failed                               */
} gdn_status;

/* Element types.  GDN_F32 = float32, GDN_BF16 = bfloat16. */
enum { GDN_F32 = 0, GDN_BF16 = 1 };

/* flags */
enum { GDN_QK_L2NORM = 1u << 0 };

typedef struct {
  int32_t B;       /* rows; with cu_seqlens B must be 1                          */
  int32_t T;       /* tokens per row; with cu_seqlens, the total token count     */
  int32_t H_qk;    /* query/key heads                                             */
  int32_t H_v;     /* value heads, a multiple of H_qk                             */
  int32_t d_k;     /* key width                                                   */
  int32_t d_v;     /* value width                                                 */
  int32_t chunk;   /* tokens per chunk of the chunked path (ignored by the step)  */
  float scale;     /* multiplies q (after the optional L2 norm)                   */
  int32_t dtype;   /* element type of q, k, v: GDN_F32 or GDN_BF16                */
  int32_t o_dtype; /* element type of o: GDN_F32 or GDN_BF16                      */
  uint32_t flags;  /* GDN_QK_L2NORM                                               */
} gdn_shape;

/*
 * Built kernel set (anything else returns GDN_ERR_UNSUPPORTED):
 *   chunked paths:  dtype GDN_BF16 with d_k = 128, chunk in {32, 64}, d_v in {16, 32, ..., 128};
 *                   dtype GDN_F32  with d_k in {16, 128}, chunk in {16, 32, 64},
 *                                  d_v in {16, 32, ..., 128}.
 *                   (bf16 MFMA contracts over 32 elements: bf16 needs d_k = 128.)
 *   decode step:    d_k in {16, 128}, d_v in {16, 128}, either dtype.
 *
 * Range of the bf16 path at chunk 64 (gdn_chunk_fwd, gdn_chunk_fwd_noalloc,
 * gdn_states_fwd, gdn_states_fwd_strided): its matrix products take fp16
 * operands.  q and k enter as fp16 (exact for bf16 values of magnitude in
 * [6.1e-5, 65504]; smaller ones keep an absolute error below 3e-8, larger ones
 * become infinities), and so do the state S and the per-chunk values derived
 * from v (X = V - diag(e^G) K S, U = T diag(beta) X), each of which must stay
 * below 65504 in magnitude: with |v| up to ~1e3 and decays and write strengths
 * in their usual ranges they stay far inside.  A value past the range turns into
 * an infinity or NaN that reaches o or the final state; the call then sets bit 1
 * (value 2) of the int32 status word at the start of the workspace and its
 * results are invalid.  Bit 0 (value 1) reports a malformed cu_seqlens array.
 * The fp32 path, the bf16 path at chunk 32 and the decode step compute in fp32
 * and have no such limit (their status word only ever holds bit 0).
 */

/*
 * gdn_chunk_fwd: the chunked prompt path (the pages' "prompt's chunked" kernel).
 *
 *   q, k           [B, T, H_qk, d_k]  dtype
 *   v              [B, T, H_v, d_v]   dtype
 *   g, beta        [B, T, H_v]        float32; g is a log decay (<= 0, -inf
 *                                     resets the state; a NaN makes that head's
 *                                     o and state non-finite from its token on,
 *                                     on the bf16 chunk-64 path possibly from
 *                                     earlier tokens of its chunk, and sets bit 1
 *                                     of the status word), beta the write strength
 *   initial_state  [N, H_v, d_k, d_v] float32, or NULL for a zero state
 *   cu_seqlens     int32 [N+1] on the device, or NULL.  Non-NULL packs N
 *                  sequences on one row (B == 1): sequence n owns tokens
 *                  [cu[n], cu[n+1]), no state crosses a boundary (the pages'
 *                  split-point convention for packed rows).  cu[0] == 0,
 *                  non-decreasing, cu[N] == T.  A device array violating this
 *                  makes every kernel of the call a no-op and sets the status
 *                  word at the start of the workspace to nonzero.
 *   num_seqs       N when cu_seqlens is given (ignored otherwise; N = B)
 *   o              [B, T, H_v, d_v]   o_dtype (written)
 *   final_state    [N, H_v, d_k, d_v] float32, or NULL (not written).  It may be
 *                  the same pointer as initial_state (in-place continuation of
 *                  a cache buffer); any other overlap with an input is refused.
 *   workspace      device scratch of at least gdn_chunk_fwd_workspace() bytes,
 *                  contents undefined on entry and exit.  It holds the per-chunk
 *                  triangular factors between the two launches of the call.
 */
gdn_status gdn_chunk_fwd(const gdn_shape *s, const void *q, const void *k,
                         const void *v, const float *g, const float *beta,
                         const float *initial_state, const int32_t *cu_seqlens,
                         int32_t num_seqs, void *o, float *final_state,
                         void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Workspace bytes gdn_chunk_fwd needs for this shape; num_seqs is N when the
   call will pass cu_seqlens, else 0.  Returns 0 if the shape is invalid.  It is
   also what gdn_chunk_fwd_gated needs. */
size_t gdn_chunk_fwd_workspace(const gdn_shape *s, int32_t num_seqs);

/*
 * gdn_chunk_fwd_gated: gdn_chunk_fwd followed by the mixer's output norm, the
 * norm(y, gate = silu(z)) with gain `weight` that the mixer applies to the rule's
 * output (Qwen3.5 text encyclopedia page, note "The DeltaNet mixer"): per token and
 * value head, over that head's d_v values,
 *     out = weight * o / sqrt(mean(o^2) + eps) * silu(z).
 *   Arguments as gdn_chunk_fwd's, with o replaced by
 *   z              [B, T, H_v, d_v]   dtype (the gate input), aligned to 4 elements
 *   weight         [d_v] float32, 16-byte aligned
 *   eps            >= 0
 *   out            [B, T, H_v, d_v]   o_dtype (written); must not overlap any input
 *   d_v must be one of 16, 32, 64, 128, 256 (the norm's widths).
 * Where the chain runs one workgroup per (sequence, value head) -- bf16 inputs at
 * chunk 64 with d_v = 128 in dense rows (no cu_seqlens) once sequences x value heads
 * reach the GPU's compute-unit count -- the norm is applied in the chain's output
 * stage and o itself is never written.  Elsewhere (packed sequences there split each
 * head's columns over two workgroups) the chain writes o into `out` and the norm then
 * runs in place over it (one more pass over out and z; with a bf16 out, o is then
 * rounded to bf16 before the norm reads it, so the result carries two roundings
 * instead of one).
 * The status word at the start of the workspace is as for gdn_chunk_fwd (in the fused
 * case its bit 1 flags a non-finite normed output instead of a non-finite o).
 */
gdn_status gdn_chunk_fwd_gated(const gdn_shape *s, const void *q, const void *k,
                               const void *v, const float *g, const float *beta,
                               const float *initial_state, const int32_t *cu_seqlens,
                               int32_t num_seqs, const void *z, const float *weight,
                               float eps, void *out, float *final_state,
                               void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * gdn_chunk_fwd_noalloc: gdn_chunk_fwd for callers that cannot allocate device
 * memory -- code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It takes no workspace: its kernels use a static device array
 * of GDN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends, and the call allocates nothing (no hipMalloc, no
 * allocating library routine).  The caller still passes every input and output,
 * as for gdn_chunk_fwd, with the same meaning, layout and ownership.
 *
 *   Limit: a shape whose gdn_chunk_fwd_workspace() exceeds
 *          GDN_NOALLOC_SCRATCH_BYTES returns GDN_ERR_WORKSPACE and writes nothing.
 *   Sharing: every call on one GPU uses that GPU's one array, which keeps the
 *          last call's contents; calls that overlap in time on one GPU (two
 *          streams, two threads) race and must be serialised by the caller.
 *   Status: a bad cu_seqlens array sets the status word at the start of the
 *          static array (not readable through this ABI); the kernels then do
 *          nothing, as in gdn_chunk_fwd.
 *   The first call on a device looks the array's address up once (a host-side
 *   runtime query, no allocation); a failure there returns GDN_ERR_HIP.
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_chunk_fwd_noalloc(const gdn_shape *s, const void *q, const void *k,
                                 const void *v, const float *g, const float *beta,
                                 const float *initial_state, const int32_t *cu_seqlens,
                                 int32_t num_seqs, void *o, float *final_state,
                                 hipStream_t stream);

/*
 * gdn_recurrent_step: one decode token per sequence (the pages' "decode step's
 * recurrent" kernel).  s->T must be 1.
 *
 *   q, k    [B, 1, H_qk, d_k]  dtype
 *   v       [B, 1, H_v, d_v]   dtype
 *   g, beta [B, 1, H_v]        float32
 *   state   [B, H_v, d_k, d_v] float32, read and updated IN PLACE
 *   o       [B, 1, H_v, d_v]   o_dtype (written); must not overlap state
 */
gdn_status gdn_recurrent_step(const gdn_shape *s, const void *q, const void *k,
                              const void *v, const float *g, const float *beta,
                              float *state, void *o, hipStream_t stream);

/*
 * gdn_states_fwd: gdn_chunk_fwd plus the state after every token (the pages'
 * `states`, [batch seq heads key_dim value_dim] float32, produced by their
 * token-by-token route).
 *
 *   states  [B, T, H_v, d_k, d_v] float32 (written); must not overlap any
 *           other argument.  states[.., t, h] is S after token t of its
 *           sequence, so the last token's entry equals final_state.
 * Other arguments as gdn_chunk_fwd; o and final_state may be NULL here.
 */
gdn_status gdn_states_fwd(const gdn_shape *s, const void *q, const void *k,
                          const void *v, const float *g, const float *beta,
                          const float *initial_state, const int32_t *cu_seqlens,
                          int32_t num_seqs, void *o, float *states,
                          float *final_state, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes gdn_states_fwd needs (num_seqs as for gdn_chunk_fwd_workspace). */
size_t gdn_states_fwd_workspace(const gdn_shape *s, int32_t num_seqs);

/*
 * gdn_states_fwd_strided: gdn_states_fwd keeping only some tokens' states.
 * The Qwen3.5 text encyclopedia page gives both the per-token `states` [batch
 * seq heads key_dim value_dim], at 1-3 MiB per token per block (note
 * "Loading"), and `state`, the state after one token, read by iterating over
 * the prompt's tokens (value table of model.layers[i].linear_attn); this call
 * writes the states of a token range at a stride, and only those.
 *
 *   t_begin, t_end, t_step  the tokens kept are t_begin, t_begin + t_step, ...
 *                           < t_end of every row, indexed along the T axis of
 *                           the [B, T] token layout (with cu_seqlens: along the
 *                           one packed row).  0 <= t_begin <= t_end <= T and
 *                           t_step >= 1, else GDN_ERR_SHAPE.
 *   states  [B, n, H_v, d_k, d_v] float32 (written), n = ceil((t_end - t_begin)
 *           / t_step): states[b, i, h] is S after token t_begin + i t_step of
 *           row b.  May be NULL only when n == 0; must not overlap any other
 *           argument.
 * o and final_state are complete, as in gdn_states_fwd; the workspace is the one
 * gdn_states_fwd_workspace returns.  t_begin = 0, t_end = T, t_step = 1 gives
 * gdn_states_fwd.  Only the kept states are written to memory: the state write,
 * the bulk of the call's traffic, shrinks in proportion.
 */
gdn_status gdn_states_fwd_strided(const gdn_shape *s, const void *q, const void *k,
                                  const void *v, const float *g, const float *beta,
                                  const float *initial_state, const int32_t *cu_seqlens,
                                  int32_t num_seqs, void *o, float *states, int32_t t_begin,
                                  int32_t t_end, int32_t t_step, float *final_state,
                                  void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * The mixer's steps around the delta rule (Qwen3.5 text encyclopedia page,
 * note "The DeltaNet mixer"; Qwen3-Next encyclopedia page, same note), for
 * channel c, token t and value head h, sigma the logistic function:
 *
 *   before:  xc[t,c] = sum_{i<4} w[c,i] x[t-3+i,c], causal and one filter per
 *            channel; q, k, v are xc sigma(xc) on the q, k and v channels;
 *            beta = sigma(b); g = -e^{A_log} ln(1 + e^{a + dt_bias})
 *   kernel:  the gated delta rule above on q, k, v, g, beta
 *   after:   out[t,h,:] = weight * y / sqrt(mean(y^2) + eps) * z sigma(z), over
 *            the d_v outputs y of one value head and its gate input z
 *
 * The module listing on the first page gives the convolution as depthwise, kernel
 * size 4, padding 3, no bias; the note "The readout is the plain projection"
 * gives the output norm's gain as its weight (not 1 + weight).
 */

/*
 * gdn_gated_norm: the output norm, per (token, value head) over its d_v values:
 *
 *     out = weight * y / sqrt(mean(y^2) + eps) * silu(z),   silu(x) = x sigmoid(x)
 *
 *   y       [B, T, H_v, d_v]  s->o_dtype (the o of gdn_chunk_fwd / gdn_states_fwd)
 *   z       [B, T, H_v, d_v]  s->dtype   (the gate's input, in_proj_z's output)
 *   weight  [d_v]             float32, shared by the heads
 *   eps     >= 0 (the family's norms use 1e-6)
 *   out     [B, T, H_v, d_v]  s->o_dtype (written); may be y itself (in place),
 *           must not overlap z or weight
 * Uses s->B, T, H_v, d_v, dtype, o_dtype; built for d_v in {16, 32, 64, 128, 256}.
 * y, z and out are read and written 4 elements at a time (aligned to 4 elements),
 * weight as float4 (16-byte aligned).
 */
gdn_status gdn_gated_norm(const gdn_shape *s, const void *y, const void *z,
                          const float *weight, float eps, void *out,
                          hipStream_t stream);

/*
 * gdn_recurrent_step_gated: gdn_recurrent_step with the output norm fused into
 * the step kernel: writes out = gdn_gated_norm of the step's o, which never
 * reaches memory.
 *
 *   z       [B, 1, H_v, d_v]  dtype
 *   weight  [d_v]             float32
 *   out     [B, 1, H_v, d_v]  o_dtype (written); must not overlap any input
 * Other arguments as gdn_recurrent_step.
 */
gdn_status gdn_recurrent_step_gated(const gdn_shape *s, const void *q, const void *k,
                                    const void *v, const float *g, const float *beta,
                                    float *state, const void *z, const float *weight,
                                    float eps, void *out, hipStream_t stream);

/*
 * gdn_mixer_prologue: the steps before the delta rule, in one pass over x.
 *
 *   x               [B, T, C] dtype, C = 2 H_qk d_k + H_v d_v: in_proj_qkv's output,
 *                   channels q (H_qk d_k), then k (H_qk d_k), then v (H_v d_v)
 *   conv_w          [C, 4] float32, the depthwise causal filter; tap 3 multiplies the
 *                   current token, tap i the token 3 - i before it
 *   conv_state_in   [N, C, 3] float32, the three inputs before each sequence (oldest
 *                   first), or NULL for zeros
 *   conv_state_out  [N, C, 3] float32 (written): the last three inputs each sequence
 *                   has seen, counting its conv_state_in; or NULL.  It may be
 *                   conv_state_in itself (in-place update of a decode cache)
 *   a, b            [B, T, H_v] float32: in_proj_a and in_proj_b outputs
 *   A_log, dt_bias  [H_v] float32
 *   cu_seqlens, num_seqs as gdn_chunk_fwd (N = num_seqs if cu_seqlens else B);
 *                   a decode step is B rows of T = 1 with conv_state_in/out
 *   q, k            [B, T, H_qk, d_k] dtype (written): silu(conv(x)) split
 *   v               [B, T, H_v, d_v]  dtype (written)
 *   g, beta         [B, T, H_v] float32 (written)
 * q and k leave unnormalised and unscaled: the delta-rule entry points apply the
 * l2 norm (GDN_QK_L2NORM) and the scale.  Needs d_k and d_v multiples of 4; x,
 * q, k, v aligned to 4 elements, conv_w to 16 bytes.  No output may overlap an
 * input, except conv_state_out == conv_state_in exactly.
 */
gdn_status gdn_mixer_prologue(const gdn_shape *s, const void *x, const float *conv_w,
                              const float *conv_state_in, float *conv_state_out,
                              const float *a, const float *b, const float *A_log,
                              const float *dt_bias, const int32_t *cu_seqlens,
                              int32_t num_seqs, void *q, void *k, void *v, float *g,
                              float *beta, hipStream_t stream);

/*
 * gdn_set_timing_events: benchmark instrumentation.  While `events` is
 * non-NULL, every gdn_chunk_fwd / gdn_states_fwd call made on this host thread
 * records events[0] on its stream before its first kernel and events[i] right
 * after its i-th kernel, for i < n: plan (1), prep (2), carry (3) and, on the
 * states path, stream (4).  hipEventElapsedTime(events[i-1], events[i]) is then
 * the duration of kernel i.  The events are owned by the caller; passing NULL
 * turns the hook off.  Returns GDN_ERR_SHAPE if n < 0.
 */
gdn_status gdn_set_timing_events(hipEvent_t *events, int n);

/* Static text for a status code. */
const char *gdn_status_string(gdn_status st);

/* Detail of the last failed call on this host thread ("" if none). */
const char *gdn_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
