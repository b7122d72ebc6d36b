// Host-side interface between the C ABI layer (gdn_api.cpp) and the kernel
// translation units: the workspace layout and the launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Problem description after validation (all sizes non-negative, H_v % H_qk == 0).
struct Problem {
  int B, T, H_qk, H_v, d_k, d_v, C;
  int N;              // sequences: num_seqs with cu_seqlens, else B
  int T_tot;          // tokens on the packed axis: B * T
  int max_chunks;     // upper bound on the chunk count (grid size of the chunk-parallel phase)
  float scale;
  int dtype, o_dtype; // GDN_F32 / GDN_BF16
  bool l2norm;
  bool packed;        // cu_seqlens given
};

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
// The plan kernel orders at most this many sequences by length (O(N^2) ranks).
constexpr int kOrderMaxSeqs = 4096;
inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace of the chunked paths, carved out of the caller's buffer:
//   status      int32            plan result: 0 ok, nonzero = bad cu_seqlens
//   seq_start   int32 [N+1]      token offset of each sequence (cu_seqlens or n*T)
//   chunk_first int32 [N+1]      global index of each sequence's first chunk
//   order       int32 [N+1]      sequences by decreasing chunk count (plan kernel)
//   tb          f32 [max_chunks, H_v, C, C]   T diag(beta), T = (I + A)^-1
//   pm          f32 [max_chunks, H_v, C, C]   scale * (decay mask o Q K^T)
//   eg          f32 [max_chunks, H_v, C]      exp(G_r)          (G: in-chunk cumsum of g)
//   eb          f32 [max_chunks, H_v, C]      exp(G_last - G_r)
//   (the general path keeps tb, pm, eg, eb; the fused bf16 path keeps instead,
//    in MFMA fragment order -- see gdn_fused.hip)
//   tt          [H_v, max_chunks, fused_t_bytes()]   T diag(beta) (fp16 hi/lo) and
//                                                    the chain's per-token factors
//   kk          [H_qk, max_chunks, fused_k_bytes()]  K and Q (fp16)
//   pf          [H_v, max_chunks, fused_p_bytes()]   P (fp16 hi/lo), split head-wide chains only
//   (states path only)
//   u           f32 [T_tot, H_v, d_v]        per-token write vectors
//   sc          f32 [max_chunks, H_v, d_k, d_v]  state at each chunk start
struct Workspace {
  int32_t *status = nullptr;
  int32_t *seq_start = nullptr;
  int32_t *chunk_first = nullptr;
  int32_t *order = nullptr;
  float *tb = nullptr, *pm = nullptr, *eg = nullptr, *eb = nullptr;
  unsigned char *tt = nullptr;  // fused bf16 path: T diag(beta) fragments and factors per (value head, chunk)
  unsigned char *kk = nullptr;  // fused bf16 path: key and query fragments per (query/key head, chunk)
  unsigned char *pf = nullptr;  // fused bf16 path, split head-wide chains: P fragments per (value head, chunk)
  float *u = nullptr, *sc = nullptr;
  size_t bytes = 0;
};

// Size of the static device scratch that gdn_chunk_fwd_noalloc uses as its workspace
// (gdn_noalloc.hip), and its device address on the current device (looked up once
// per device; the array's host-side name is never passed to a kernel).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void **ptr);

// Computes the layout; with base == nullptr only `bytes` is meaningful.
Workspace workspace_layout(const Problem &p, bool states, void *base);

// Launchers: return hipSuccess or the launch error.  Pointers are device pointers.
struct ChunkArgs {
  const void *q, *k, *v;
  const float *g, *beta, *s0;
  const int32_t *cu;   // may be null (dense rows)
  void *o;             // may be null (states path)
  float *final_state;  // may be null
  float *states;       // states path only
  // states path: keep the tokens t_lo, t_lo + t_step, ... < t_hi of every row
  // (the T axis of [B, T]; with cu_seqlens, of the one packed row); states then
  // holds n_sel = ceil((t_hi - t_lo) / t_step) tokens per row
  int t_lo = 0, t_hi = 0, t_step = 1, n_sel = 0;
  Workspace ws;
  hipEvent_t *events = nullptr;  // optional timing hook: recorded around each launch
  int n_events = 0;
  // gated output (chunk path only, where fused_wide(): o <- nw * o / sqrt(mean(o^2) + eps) * silu(z))
  const void *z = nullptr;
  const float *nw = nullptr;
  float eps = 0.0f;
};
hipError_t launch_chunk_path(const Problem &p, const ChunkArgs &a, bool states, hipStream_t stream);

// Pieces shared by the chunked paths (gdn_chunk.hip): the plan kernel, the
// per-token states stream, and the timing hook.
hipError_t launch_plan(const Problem &p, const ChunkArgs &a, hipStream_t stream);
// Dense rows (no cu_seqlens) need no plan: their geometry is n T and n ceil(T / C).
inline bool dense_rows(const Problem &p) { return !p.packed && p.T > 0; }
struct Seqs;
hipError_t launch_states_stream(const Problem &p, const ChunkArgs &a, const Seqs &sq, hipStream_t stream);
inline void mark_event(const ChunkArgs &a, int i, hipStream_t st) {
  if (a.events && i < a.n_events) (void)hipEventRecord(a.events[i], st);
}
// The fused bf16 chunked path (gdn_fused.hip): d_k = 128, C = 64; bytes of its
// per-(value head, chunk) workspace slot.
hipError_t launch_fused_path(const Problem &p, const ChunkArgs &a, bool states, hipStream_t stream);
size_t fused_t_bytes();
size_t fused_k_bytes();
size_t fused_p_bytes();
// True when the fused path runs the head-wide chains for this problem: one workgroup per
// (sequence, value head), or two per head (half its columns each) for packed sequences.
bool fused_wide(const Problem &p);
// True when the solve also forms P for the chain (the split head-wide chains); the whole-head
// chains form it themselves.
bool fused_solve_p(const Problem &p);

// True when a chunked-path kernel is built for this problem.
bool chunk_path_supported(const Problem &p);

struct StepArgs {
  const void *q, *k, *v;
  const float *g, *beta;
  float *state;
  void *o;
  // optional fused output norm: o <- weight * o / sqrt(mean(o^2) + eps) * silu(z)
  const void *z = nullptr;
  const float *weight = nullptr;
  float eps = 0.0f;
};
hipError_t launch_recurrent_step(const Problem &p, const StepArgs &a, hipStream_t stream);
bool step_supported(const Problem &p);

// The mixer's steps around the delta rule (gdn_mixer.hip).
struct NormArgs {
  const void *y;        // [T_tot, H_v, d_v] o_dtype
  const void *z;        // [T_tot, H_v, d_v] dtype
  const float *weight;  // [d_v]
  float eps;
  void *out;            // [T_tot, H_v, d_v] o_dtype, may be y
};
bool norm_supported(const Problem &p);
hipError_t launch_gated_norm(const Problem &p, const NormArgs &a, hipStream_t stream);

struct PrologueArgs {
  const void *x;          // [T_tot, 2 H_qk d_k + H_v d_v] dtype
  const float *conv_w;    // [channels, 4]
  const float *cs_in;     // [N, channels, 3] or null
  float *cs_out;          // [N, channels, 3] or null; may be cs_in
  const float *a, *b;     // [T_tot, H_v]
  const float *A_log, *dt_bias;  // [H_v]
  const int32_t *cu;      // cu_seqlens or null
  void *q, *k, *v;        // dtype
  float *g, *beta;        // [T_tot, H_v]
};
bool prologue_supported(const Problem &p);
hipError_t launch_prologue(const Problem &p, const PrologueArgs &a, hipStream_t stream);

}  // namespace gdn
