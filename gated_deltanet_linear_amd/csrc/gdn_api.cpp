// The C ABI of libgdn (include/gdn.h): host-side validation, workspace
// carving and dispatch to the HIP kernels.  Nothing here allocates, frees or
// synchronises; every check runs before the first launch, so a refused call
// writes nothing.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <exception>
#include <string>

#include "gdn.h"
#include "gdn_internal.hpp"

static_assert(GDN_NOALLOC_SCRATCH_BYTES == gdn::kNoAllocScratchBytes, "the header states the static scratch size");

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t *g_events = nullptr;
thread_local int g_n_events = 0;

gdn_status fail(gdn_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(gdn_status_string(st)) + ": " + buf;
  return st;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

struct Arg {
  const void *p;
  const char *name;
  size_t align;
};

// Every non-NULL pointer must be aligned to what its kernel reads or writes it with.
template <size_t N> gdn_status check_alignment(const Arg (&args)[N]) {
  for (const Arg &a : args)
    if (a.p && !aligned(a.p, a.align)) return fail(GDN_ERR_ALIGN, "%s is not %zu-byte aligned", a.name, a.align);
  return GDN_OK;
}

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi)
  Span() = default;
  Span(const void *p, size_t bytes) : lo(reinterpret_cast<uintptr_t>(p)), hi(lo + bytes) {}
  bool empty() const { return lo == hi || lo == 0; }
  bool overlaps(const Span &o) const { return !empty() && !o.empty() && lo < o.hi && o.lo < hi; }
};

size_t esize(int dt) { return dt == GDN_BF16 ? 2 : 4; }

// Shape checks shared by every entry point; fills p.  mode: 0 chunked path, 1 decode
// step (T == 1), 2 token-wise mixer steps (no chunk).
gdn_status check_shape(const gdn_shape *s, bool packed, int32_t num_seqs, int mode, gdn::Problem &p) {
  const bool step = mode == 1;
  if (!s) return fail(GDN_ERR_NULL, "shape is NULL");
  if (s->dtype != GDN_F32 && s->dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "dtype %d", s->dtype);
  if (s->o_dtype != GDN_F32 && s->o_dtype != GDN_BF16) return fail(GDN_ERR_DTYPE, "o_dtype %d", s->o_dtype);
  if (s->B < 0 || s->T < 0) return fail(GDN_ERR_SHAPE, "B=%d T=%d", s->B, s->T);
  if (s->H_qk <= 0 || s->H_v <= 0 || s->H_v % s->H_qk != 0)
    return fail(GDN_ERR_SHAPE, "H_qk=%d H_v=%d (H_v must be a positive multiple of H_qk)", s->H_qk, s->H_v);
  if (s->d_k <= 0 || s->d_v <= 0) return fail(GDN_ERR_SHAPE, "d_k=%d d_v=%d", s->d_k, s->d_v);
  if (s->flags & ~(uint32_t)GDN_QK_L2NORM) return fail(GDN_ERR_SHAPE, "unknown flags 0x%x", s->flags);
  if (!(s->scale == s->scale)) return fail(GDN_ERR_SHAPE, "scale is NaN");
  if (step) {
    if (s->T != 1) return fail(GDN_ERR_SHAPE, "the decode step takes T == 1, got %d", s->T);
  } else if (mode == 0 && s->chunk <= 0) {
    return fail(GDN_ERR_SHAPE, "chunk=%d", s->chunk);
  }
  if (packed) {
    if (s->B != 1) return fail(GDN_ERR_SHAPE, "packed sequences need B == 1, got %d", s->B);
    if (num_seqs < 0) return fail(GDN_ERR_SHAPE, "num_seqs=%d", num_seqs);
  }
  const int64_t T_tot = (int64_t)s->B * s->T;
  // Every flat index a kernel forms must fit comfortably (token counts in int32).
  if (T_tot > (1LL << 30)) return fail(GDN_ERR_SHAPE, "B*T=%lld too large", (long long)T_tot);
  p.B = s->B;
  p.T = s->T;
  p.H_qk = s->H_qk;
  p.H_v = s->H_v;
  p.d_k = s->d_k;
  p.d_v = s->d_v;
  p.C = mode == 0 ? s->chunk : 1;
  p.packed = packed;
  p.N = packed ? num_seqs : s->B;
  p.T_tot = (int)T_tot;
  p.scale = s->scale;
  p.dtype = s->dtype;
  p.o_dtype = s->o_dtype;
  p.l2norm = (s->flags & GDN_QK_L2NORM) != 0;
  p.max_chunks = 0;
  if (mode == 0) {
    const int64_t mc = packed ? (T_tot + p.C - 1) / p.C + p.N : (int64_t)p.B * ((p.T + p.C - 1) / p.C);
    if (mc * p.H_v > (1LL << 30)) return fail(GDN_ERR_SHAPE, "too many chunks");
    p.max_chunks = (int)mc;
  }
  return GDN_OK;
}

struct Tensors {
  Span q, k, v, g, beta, s0, cu, o, states, fin, ws;
};

Tensors spans(const gdn::Problem &p, const void *q, const void *k, const void *v, const float *g,
              const float *beta, const float *s0, const int32_t *cu, const void *o, const float *states,
              size_t states_tokens, const float *fin, const void *ws, size_t ws_bytes) {
  const size_t T = p.T_tot, es = esize(p.dtype);
  const size_t state_bytes = (size_t)p.N * p.H_v * p.d_k * p.d_v * sizeof(float);
  Tensors t;
  t.q = Span(q, T * p.H_qk * p.d_k * es);
  t.k = Span(k, T * p.H_qk * p.d_k * es);
  t.v = Span(v, T * p.H_v * p.d_v * es);
  t.g = Span(g, T * p.H_v * sizeof(float));
  t.beta = Span(beta, T * p.H_v * sizeof(float));
  t.s0 = Span(s0, state_bytes);
  t.cu = Span(cu, ((size_t)p.N + 1) * sizeof(int32_t));
  t.o = Span(o, T * p.H_v * p.d_v * esize(p.o_dtype));
  t.states = Span(states, states_tokens * p.H_v * p.d_k * p.d_v * sizeof(float));
  t.fin = Span(fin, state_bytes);
  t.ws = Span(ws, ws_bytes);
  return t;
}

gdn_status chunked_common(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                          int32_t num_seqs, void *o, float *states, float *final_state, void *workspace,
                          size_t workspace_bytes, hipStream_t stream, bool with_states, int32_t t_begin = 0,
                          int32_t t_end = -1, int32_t t_step = 1, const void *z = nullptr,
                          const float *norm_w = nullptr, float eps = 0.0f, bool gated = false) {
  gdn::Problem p;
  gdn_status st = check_shape(s, cu_seqlens != nullptr, num_seqs, 0, p);
  if (st != GDN_OK) return st;
  // the token selection of the states path (all tokens unless strided)
  if (t_end < 0) t_end = p.T;
  if (with_states && (t_begin < 0 || t_end > p.T || t_begin > t_end || t_step < 1))
    return fail(GDN_ERR_SHAPE, "token selection [%d, %d) step %d is not within [0, %d) with step >= 1", t_begin,
                t_end, t_step, p.T);
  const int32_t n_sel = with_states ? (t_end - t_begin + t_step - 1) / t_step : 0;
  if (!gdn::chunk_path_supported(p))
    return fail(GDN_ERR_UNSUPPORTED, "no chunked kernel for dtype=%d d_k=%d d_v=%d chunk=%d", p.dtype, p.d_k,
                p.d_v, p.C);
  const bool any_tokens = p.T_tot > 0;
  if (any_tokens && (!q || !k || !v || !g || !beta)) return fail(GDN_ERR_NULL, "q, k, v, g and beta are required");
  if (!with_states && any_tokens && !o) return fail(GDN_ERR_NULL, "o is required");
  if (with_states && n_sel > 0 && p.B > 0 && !states) return fail(GDN_ERR_NULL, "states is required");
  if (gated) {
    if (!gdn::norm_supported(p)) return fail(GDN_ERR_UNSUPPORTED, "no output norm for d_v=%d", p.d_v);
    if (!(eps >= 0.0f) || eps > 1e30f) return fail(GDN_ERR_SHAPE, "eps=%g", (double)eps);
    if (any_tokens && (!z || !norm_w)) return fail(GDN_ERR_NULL, "z and weight are required");
  }
  const gdn::Workspace need = gdn::workspace_layout(p, with_states, nullptr);
  if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need.bytes);
  if (workspace_bytes < need.bytes)
    return fail(GDN_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need.bytes);
  // q, k, v rows are read with 16-byte vector loads, states written with 16-byte
  // stores, o written 4 elements at a time, the workspace read as float4;
  // everything else is scalar.
  const Arg args[] = {{q, "q", 16},           {k, "k", 16},
                      {v, "v", 16},           {g, "g", 4},
                      {beta, "beta", 4},      {initial_state, "initial_state", 4},
                      {cu_seqlens, "cu_seqlens", 4}, {o, "o", 4 * esize(p.o_dtype)},
                      {states, "states", 16}, {final_state, "final_state", 4},
                      {workspace, "workspace", 16}};
  if ((st = check_alignment(args)) != GDN_OK) return st;
  if (gated) {
    const Arg gargs[] = {{z, "z", 4 * esize(p.dtype)}, {norm_w, "weight", 16}};
    if ((st = check_alignment(gargs)) != GDN_OK) return st;
  }

  const Tensors t = spans(p, q, k, v, g, beta, initial_state, cu_seqlens, o, states,
                          with_states ? (size_t)p.B * n_sel : 0, final_state, workspace, workspace_bytes);
  const Span ins[] = {t.q, t.k, t.v, t.g, t.beta, t.s0, t.cu};
  const char *in_names[] = {"q", "k", "v", "g", "beta", "initial_state", "cu_seqlens"};
  struct Out {
    Span s;
    const char *name;
  } outs[] = {{t.o, "o"}, {t.states, "states"}, {t.fin, "final_state"}, {t.ws, "workspace"}};
  for (const Out &x : outs) {
    for (int i = 0; i < 7; ++i) {
      if (!x.s.overlaps(ins[i])) continue;
      // The one permitted overlap: final_state == initial_state exactly.
      const bool inplace = (&x == &outs[2]) && i == 5 && x.s.lo == ins[i].lo && x.s.hi == ins[i].hi;
      if (!inplace) return fail(GDN_ERR_ALIAS, "%s overlaps %s", x.name, in_names[i]);
    }
  }
  for (int a = 0; a < 4; ++a)
    for (int b = a + 1; b < 4; ++b)
      if (outs[a].s.overlaps(outs[b].s)) return fail(GDN_ERR_ALIAS, "%s overlaps %s", outs[a].name, outs[b].name);
  if (gated) {
    const Span sz(z, (size_t)p.T_tot * p.H_v * p.d_v * esize(p.dtype)), sw(norm_w, (size_t)p.d_v * sizeof(float));
    for (const Out &x : outs) {
      if (x.s.overlaps(sz)) return fail(GDN_ERR_ALIAS, "%s overlaps z", x.name);
      if (x.s.overlaps(sw)) return fail(GDN_ERR_ALIAS, "%s overlaps weight", x.name);
    }
  }

  gdn::ChunkArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.s0 = initial_state;
  a.cu = cu_seqlens;
  a.o = o;
  a.final_state = final_state;
  a.states = states;
  a.t_lo = t_begin;
  a.t_hi = t_end;
  a.t_step = t_step;
  a.n_sel = n_sel;
  a.ws = gdn::workspace_layout(p, with_states, workspace);
  a.events = g_events;
  a.n_events = g_n_events;
  // The output norm runs inside the chain where one workgroup holds a whole value head
  // (the head-wide chains on dense rows; packed sequences split each head's columns
  // over two workgroups); elsewhere it follows the chain, in place over o.
  const bool fused_norm = gated && !with_states && p.dtype == GDN_BF16 && !p.packed && gdn::fused_wide(p);
  if (fused_norm) {
    a.z = z;
    a.nw = norm_w;
    a.eps = eps;
  }
  hipError_t e = gdn::launch_chunk_path(p, a, with_states, stream);
  if (e == hipSuccess && gated && !fused_norm && any_tokens) {
    gdn::NormArgs na{o, z, norm_w, eps, o};
    e = gdn::launch_gated_norm(p, na, stream);
  }
  if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
  g_last_error.clear();
  return GDN_OK;
}

}  // namespace

extern "C" {

const char *gdn_status_string(gdn_status st) {
  switch (st) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
  }
  return "GDN_UNKNOWN_STATUS";
}

const char *gdn_last_error(void) { return g_last_error.c_str(); }

int gdn_version(void) { return 100; }

gdn_status gdn_set_timing_events(hipEvent_t *events, int n) {
  if (n < 0) return fail(GDN_ERR_SHAPE, "n=%d", n);
  g_events = events;
  g_n_events = events ? n : 0;
  return GDN_OK;
}

static size_t workspace_query(const gdn_shape *s, int32_t num_seqs, bool states) {
  try {
    const std::string keep = g_last_error;  // a query never changes the last error
    gdn::Problem p;
    const gdn_status st = check_shape(s, num_seqs > 0, num_seqs, 0, p);
    g_last_error = keep;
    if (st != GDN_OK) return 0;
    return gdn::workspace_layout(p, states, nullptr).bytes;
  } catch (...) {
    return 0;
  }
}

size_t gdn_chunk_fwd_workspace(const gdn_shape *s, int32_t num_seqs) { return workspace_query(s, num_seqs, false); }

size_t gdn_states_fwd_workspace(const gdn_shape *s, int32_t num_seqs) { return workspace_query(s, num_seqs, true); }

gdn_status gdn_chunk_fwd(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                         int32_t num_seqs, void *o, float *final_state, void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  try {
    return chunked_common(s, q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, o, nullptr, final_state,
                          workspace, workspace_bytes, stream, false);
  } catch (const std::exception &e) {
    return fail(GDN_ERR_HIP, "internal error: %s", e.what());
  } catch (...) {
    return fail(GDN_ERR_HIP, "internal error");
  }
}

gdn_status gdn_chunk_fwd_gated(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                               const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                               int32_t num_seqs, const void *z, const float *weight, float eps, void *out,
                               float *final_state, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    return chunked_common(s, q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, out, nullptr, final_state,
                          workspace, workspace_bytes, stream, false, 0, -1, 1, z, weight, eps, true);
  } catch (const std::exception &e) {
    return fail(GDN_ERR_HIP, "internal error: %s", e.what());
  } catch (...) {
    return fail(GDN_ERR_HIP, "internal error");
  }
}

gdn_status gdn_chunk_fwd_noalloc(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                                 int32_t num_seqs, void *o, float *final_state, hipStream_t stream) {
  try {
    gdn::Problem p;
    gdn_status st = check_shape(s, cu_seqlens != nullptr, num_seqs, 0, p);
    if (st != GDN_OK) return st;
    const size_t need = gdn::workspace_layout(p, false, nullptr).bytes;
    if (need > gdn::kNoAllocScratchBytes)
      return fail(GDN_ERR_WORKSPACE,
                  "this call needs %zu bytes of scratch; gdn_chunk_fwd_noalloc's static scratch holds %zu "
                  "(GDN_NOALLOC_SCRATCH_BYTES): use gdn_chunk_fwd with a workspace",
                  need, gdn::kNoAllocScratchBytes);
    void *ws = nullptr;
    const hipError_t e = gdn::noalloc_scratch(&ws);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
    return chunked_common(s, q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, o, nullptr, final_state, ws,
                          gdn::kNoAllocScratchBytes, stream, false);
  } catch (const std::exception &e) {
    return fail(GDN_ERR_HIP, "internal error: %s", e.what());
  } catch (...) {
    return fail(GDN_ERR_HIP, "internal error");
  }
}

gdn_status gdn_states_fwd(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                          const float *beta, const float *initial_state, const int32_t *cu_seqlens,
                          int32_t num_seqs, void *o, float *states, float *final_state, void *workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  try {
    return chunked_common(s, q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, o, states, final_state,
                          workspace, workspace_bytes, stream, true);
  } catch (const std::exception &e) {
    return fail(GDN_ERR_HIP, "internal error: %s", e.what());
  } catch (...) {
    return fail(GDN_ERR_HIP, "internal error");
  }
}

gdn_status gdn_states_fwd_strided(const gdn_shape *s, const void *q, const void *k, const void *v,
                                  const float *g, const float *beta, const float *initial_state,
                                  const int32_t *cu_seqlens, int32_t num_seqs, void *o, float *states,
                                  int32_t t_begin, int32_t t_end, int32_t t_step, float *final_state,
                                  void *workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    return chunked_common(s, q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, o, states, final_state,
                          workspace, workspace_bytes, stream, true, t_begin, t_end, t_step);
  } catch (const std::exception &e) {
    return fail(GDN_ERR_HIP, "internal error: %s", e.what());
  } catch (...) {
    return fail(GDN_ERR_HIP, "internal error");
  }
}

gdn_status gdn_recurrent_step(const gdn_shape *s, const void *q, const void *k, const void *v, const float *g,
                              const float *beta, float *state, void *o, hipStream_t stream) {
  try {
    gdn::Problem p;
    gdn_status st = check_shape(s, false, 0, 1, p);
    if (st != GDN_OK) return st;
    if (!gdn::step_supported(p))
      return fail(GDN_ERR_UNSUPPORTED, "no decode kernel for d_k=%d d_v=%d", p.d_k, p.d_v);
    if (p.B > 0 && (!q || !k || !v || !g || !beta || !state || !o))
      return fail(GDN_ERR_NULL, "q, k, v, g, beta, state and o are required");
    // The state is read and written as float4, o written 4 elements at a time.
    const Arg args[] = {{q, "q", esize(p.dtype)}, {k, "k", esize(p.dtype)},   {v, "v", esize(p.dtype)},
                        {g, "g", 4},              {beta, "beta", 4},          {state, "state", 16},
                        {o, "o", 4 * esize(p.o_dtype)}};
    if ((st = check_alignment(args)) != GDN_OK) return st;
    const Tensors t = spans(p, q, k, v, g, beta, nullptr, nullptr, o, nullptr, 0, nullptr, nullptr, 0);
    const Span sst(state, (size_t)p.B * p.H_v * p.d_k * p.d_v * sizeof(float));
    const Span ins[] = {t.q, t.k, t.v, t.g, t.beta};
    const char *in_names[] = {"q", "k", "v", "g", "beta"};
    for (int i = 0; i < 5; ++i) {
      if (sst.overlaps(ins[i])) return fail(GDN_ERR_ALIAS, "state overlaps %s", in_names[i]);
      if (t.o.overlaps(ins[i])) return fail(GDN_ERR_ALIAS, "o overlaps %s", in_names[i]);
    }
    if (t.o.overlaps(sst)) return fail(GDN_ERR_ALIAS, "o overlaps state");
    gdn::StepArgs a{q, k, v, g, beta, state, o};
    const hipError_t e = gdn::launch_recurrent_step(p, a, stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    g_last_error.clear();
    return GDN_OK;
  } catch (...) {
    return fail(GDN_ERR_HIP, "internal error");
  }
}

gdn_status gdn_recurrent_step_gated(const gdn_shape *s, const void *q, const void *k, const void *v,
                                    const float *g, const float *beta, float *state, const void *z,
                                    const float *weight, float eps, void *out, hipStream_t stream) {
  try {
    gdn::Problem p;
    gdn_status st = check_shape(s, false, 0, 1, p);
    if (st != GDN_OK) return st;
    if (!gdn::step_supported(p))
      return fail(GDN_ERR_UNSUPPORTED, "no decode kernel for d_k=%d d_v=%d", p.d_k, p.d_v);
    if (!(eps >= 0.0f) || eps > 1e30f) return fail(GDN_ERR_SHAPE, "eps=%g", (double)eps);
    if (p.B > 0 && (!q || !k || !v || !g || !beta || !state || !z || !weight || !out))
      return fail(GDN_ERR_NULL, "q, k, v, g, beta, state, z, weight and out are required");
    const Arg args[] = {{q, "q", esize(p.dtype)}, {k, "k", esize(p.dtype)},     {v, "v", esize(p.dtype)},
                        {g, "g", 4},              {beta, "beta", 4},            {state, "state", 16},
                        {z, "z", esize(p.dtype)}, {weight, "weight", 4},        {out, "out", 4 * esize(p.o_dtype)}};
    if ((st = check_alignment(args)) != GDN_OK) return st;
    const Tensors t = spans(p, q, k, v, g, beta, nullptr, nullptr, out, nullptr, 0, nullptr, nullptr, 0);
    const Span sst(state, (size_t)p.B * p.H_v * p.d_k * p.d_v * sizeof(float));
    const Span sz(z, (size_t)p.B * p.H_v * p.d_v * esize(p.dtype)), sw(weight, (size_t)p.d_v * sizeof(float));
    const Span ins[] = {t.q, t.k, t.v, t.g, t.beta, sz, sw};
    const char *in_names[] = {"q", "k", "v", "g", "beta", "z", "weight"};
    for (int i = 0; i < 7; ++i) {
      if (sst.overlaps(ins[i])) return fail(GDN_ERR_ALIAS, "state overlaps %s", in_names[i]);
      if (t.o.overlaps(ins[i])) return fail(GDN_ERR_ALIAS, "out overlaps %s", in_names[i]);
    }
    if (t.o.overlaps(sst)) return fail(GDN_ERR_ALIAS, "out overlaps state");
    gdn::StepArgs a{q, k, v, g, beta, state, out, z, weight, eps};
    const hipError_t e = gdn::launch_recurrent_step(p, a, stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    g_last_error.clear();
    return GDN_OK;
  } catch (...) {
    return fail(GDN_ERR_HIP, "internal error");
  }
}

gdn_status gdn_gated_norm(const gdn_shape *s, const void *y, const void *z, const float *weight, float eps,
                          void *out, hipStream_t stream) {
  try {
    gdn::Problem p;
    gdn_status st = check_shape(s, false, 0, 2, p);
    if (st != GDN_OK) return st;
    if (!gdn::norm_supported(p)) return fail(GDN_ERR_UNSUPPORTED, "no norm kernel for d_v=%d", p.d_v);
    if (!(eps >= 0.0f) || eps > 1e30f) return fail(GDN_ERR_SHAPE, "eps=%g", (double)eps);
    const size_t rows = (size_t)p.T_tot * p.H_v;
    if (rows > 0 && (!y || !z || !weight || !out)) return fail(GDN_ERR_NULL, "y, z, weight and out are required");
    const Arg args[] = {{y, "y", 4 * esize(p.o_dtype)},
                        {z, "z", 4 * esize(p.dtype)},
                        {weight, "weight", 16},
                        {out, "out", 4 * esize(p.o_dtype)}};
    if ((st = check_alignment(args)) != GDN_OK) return st;
    const Span sy(y, rows * p.d_v * esize(p.o_dtype)), so(out, rows * p.d_v * esize(p.o_dtype));
    const Span sz(z, rows * p.d_v * esize(p.dtype)), sw(weight, (size_t)p.d_v * sizeof(float));
    if (so.overlaps(sy) && !(so.lo == sy.lo && so.hi == sy.hi))
      return fail(GDN_ERR_ALIAS, "out overlaps y other than exactly (in place)");
    if (so.overlaps(sz)) return fail(GDN_ERR_ALIAS, "out overlaps z");
    if (so.overlaps(sw)) return fail(GDN_ERR_ALIAS, "out overlaps weight");
    gdn::NormArgs a{y, z, weight, eps, out};
    const hipError_t e = gdn::launch_gated_norm(p, a, stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    g_last_error.clear();
    return GDN_OK;
  } catch (...) {
    return fail(GDN_ERR_HIP, "internal error");
  }
}

gdn_status gdn_mixer_prologue(const gdn_shape *s, const void *x, const float *conv_w,
                              const float *conv_state_in, float *conv_state_out, const float *a_in,
                              const float *b_in, const float *A_log, const float *dt_bias,
                              const int32_t *cu_seqlens, int32_t num_seqs, void *q, void *k, void *v,
                              float *g, float *beta, hipStream_t stream) {
  try {
    gdn::Problem p;
    gdn_status st = check_shape(s, cu_seqlens != nullptr, num_seqs, 2, p);
    if (st != GDN_OK) return st;
    if (!gdn::prologue_supported(p))
      return fail(GDN_ERR_UNSUPPORTED, "no prologue kernel for d_k=%d d_v=%d (multiples of 4)", p.d_k, p.d_v);
    if (p.packed && p.T_tot > 0 && p.N < 1) return fail(GDN_ERR_SHAPE, "num_seqs=%d with tokens", p.N);
    const size_t T = p.T_tot, es = esize(p.dtype);
    const size_t nq = (size_t)p.H_qk * p.d_k, nv = (size_t)p.H_v * p.d_v, Cch = 2 * nq + nv;
    if (Cch > (1u << 28)) return fail(GDN_ERR_SHAPE, "%zu channels", Cch);
    if (T > 0 && (!x || !conv_w || !a_in || !b_in || !A_log || !dt_bias || !q || !k || !v || !g || !beta))
      return fail(GDN_ERR_NULL, "x, conv_w, a, b, A_log, dt_bias, q, k, v, g and beta are required");
    const Arg args[] = {{x, "x", 4 * es},         {conv_w, "conv_w", 16},    {conv_state_in, "conv_state_in", 4},
                        {conv_state_out, "conv_state_out", 4}, {a_in, "a", 4}, {b_in, "b", 4},
                        {A_log, "A_log", 4},     {dt_bias, "dt_bias", 4},   {cu_seqlens, "cu_seqlens", 4},
                        {q, "q", 4 * es},        {k, "k", 4 * es},          {v, "v", 4 * es},
                        {g, "g", 4},             {beta, "beta", 4}};
    if ((st = check_alignment(args)) != GDN_OK) return st;
    const size_t cs_bytes = (size_t)p.N * Cch * 3 * sizeof(float);
    const Span ins[] = {Span(x, T * Cch * es),
                        Span(conv_w, Cch * 4 * sizeof(float)),
                        Span(conv_state_in, cs_bytes),
                        Span(a_in, T * p.H_v * sizeof(float)),
                        Span(b_in, T * p.H_v * sizeof(float)),
                        Span(A_log, (size_t)p.H_v * sizeof(float)),
                        Span(dt_bias, (size_t)p.H_v * sizeof(float)),
                        Span(cu_seqlens, ((size_t)p.N + 1) * sizeof(int32_t))};
    const char *in_names[] = {"x", "conv_w", "conv_state_in", "a", "b", "A_log", "dt_bias", "cu_seqlens"};
    struct Out {
      Span s;
      const char *name;
    } outs[] = {{Span(q, T * nq * es), "q"},
                {Span(k, T * nq * es), "k"},
                {Span(v, T * nv * es), "v"},
                {Span(g, T * p.H_v * sizeof(float)), "g"},
                {Span(beta, T * p.H_v * sizeof(float)), "beta"},
                {Span(conv_state_out, cs_bytes), "conv_state_out"}};
    for (int o = 0; o < 6; ++o) {
      for (int i = 0; i < 8; ++i) {
        if (!outs[o].s.overlaps(ins[i])) continue;
        const bool inplace = o == 5 && i == 2 && outs[o].s.lo == ins[i].lo && outs[o].s.hi == ins[i].hi;
        if (!inplace) return fail(GDN_ERR_ALIAS, "%s overlaps %s", outs[o].name, in_names[i]);
      }
      for (int o2 = o + 1; o2 < 6; ++o2)
        if (outs[o].s.overlaps(outs[o2].s)) return fail(GDN_ERR_ALIAS, "%s overlaps %s", outs[o].name, outs[o2].name);
    }
    gdn::PrologueArgs a{x, conv_w, conv_state_in, conv_state_out, a_in, b_in, A_log, dt_bias, cu_seqlens,
                        q, k, v, g, beta};
    const hipError_t e = gdn::launch_prologue(p, a, stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "launch failed: %s", hipGetErrorString(e));
    g_last_error.clear();
    return GDN_OK;
  } catch (...) {
    return fail(GDN_ERR_HIP, "internal error");
  }
}

}  // extern "C"
