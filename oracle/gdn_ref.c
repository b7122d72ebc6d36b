/*
 * gdn_ref: the fp64 CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product (libgdn,
 * HIP on gfx950) never calls it, links it, or shares code with it.
 *
 * What it computes: the plain token-by-token recurrence of the gated delta
 * rule, in double precision, one (sequence, value head) at a time.  It is
 * written from the pages' statement of the mixer, not from any kernel:
 *
 *   - Qwen3.5 text encyclopedia page, "The DeltaNet mixer" note: the kernel is
 *     called as delta_rule(l2norm(q)/sqrt(128), l2norm(k), v, g, beta) and
 *     returns (y, state); each token keeps decays.exp() of the state; betas is
 *     the write strength; the query/key heads are repeat_interleave'd up to the
 *     value heads, so value head h reads query/key head h / (H_v / H_qk).
 *   - same page, value table of model.layers[i].linear_attn: state_input is
 *     None at the start of a prompt (a zero state), state_output is the state
 *     leaving the layer, and states is the state after every token.
 *   - Qwen3-Next encyclopedia page, same note: decays are float32 and <= 0.
 *
 * The update itself is the gated form of the delta (Widrow-Hoff) rule on a
 * linear associative memory S in R^{d_k x d_v}:
 *
 *      S  <- exp(g_t) * S                     (decay: the token keeps exp(g))
 *      e   = S^T k_t                          (what the memory predicts for k)
 *      S  <- S + k_t (beta_t (v_t - e))^T     (delta-rule write, strength beta)
 *      o_t = S^T q_t                          (read after the write)
 *
 * with k_t, q_t optionally L2-normalised as x / sqrt(sum x^2 + 1e-6) and q_t
 * then multiplied by `scale`.  A decay of g = -inf gives exp(g) = 0 exactly,
 * i.e. the state is reset before that token's write.
 *
 * Inputs are float32 (bf16 data is passed upcast, which is exact); all
 * arithmetic is double.  No -ffast-math: the build keeps IEEE semantics.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GDN_REF_OK 0
#define GDN_REF_EINVAL 1
#define GDN_REF_ENOMEM 2

int gdn_ref_version(void) { return 1; }

/* One (sequence, value head) unit: runs tokens [t0, t1) of the packed axis. */
static void run_unit(int64_t t0, int64_t t1, int64_t h, int64_t hi, int64_t n,
                     int64_t H_qk, int64_t H_v, int64_t d_k, int64_t d_v,
                     int64_t n_heads, const float *q, const float *k,
                     const float *v, const float *g, const float *beta,
                     const double *s0, double scale, int l2norm, double *o,
                     double *s_final, double *states, double *S, double *kk,
                     double *qq, double *e) {
  const int64_t group = H_v / H_qk; /* value heads per query/key head */
  const int64_t j = h / group;      /* repeat_interleave: heads gj..gj+g-1 <- j */
  const int64_t dkv = d_k * d_v;

  if (s0)
    memcpy(S, s0 + (n * H_v + h) * dkv, sizeof(double) * (size_t)dkv);
  else
    memset(S, 0, sizeof(double) * (size_t)dkv);

  for (int64_t t = t0; t < t1; ++t) {
    const float *kt = k + (t * H_qk + j) * d_k;
    const float *qt = q + (t * H_qk + j) * d_k;
    const float *vt = v + (t * H_v + h) * d_v;
    for (int64_t i = 0; i < d_k; ++i) {
      kk[i] = (double)kt[i];
      qq[i] = (double)qt[i];
    }
    if (l2norm) {
      double sk = 0.0, sq = 0.0;
      for (int64_t i = 0; i < d_k; ++i) {
        sk += kk[i] * kk[i];
        sq += qq[i] * qq[i];
      }
      const double rk = 1.0 / sqrt(sk + 1e-6), rq = 1.0 / sqrt(sq + 1e-6);
      for (int64_t i = 0; i < d_k; ++i) {
        kk[i] *= rk;
        qq[i] *= rq;
      }
    }
    for (int64_t i = 0; i < d_k; ++i) qq[i] *= scale;

    const double alpha = exp((double)g[t * H_v + h]); /* exp(-inf) == 0 */
    const double b = (double)beta[t * H_v + h];

    /* decay */
    for (int64_t x = 0; x < dkv; ++x) S[x] *= alpha;
    /* prediction e = S^T k */
    for (int64_t c = 0; c < d_v; ++c) e[c] = 0.0;
    for (int64_t i = 0; i < d_k; ++i) {
      const double ki = kk[i];
      const double *row = S + i * d_v;
      for (int64_t c = 0; c < d_v; ++c) e[c] += row[c] * ki;
    }
    /* delta, written with strength beta: S += k (beta (v - e))^T */
    for (int64_t c = 0; c < d_v; ++c) e[c] = b * ((double)vt[c] - e[c]);
    for (int64_t i = 0; i < d_k; ++i) {
      const double ki = kk[i];
      double *row = S + i * d_v;
      for (int64_t c = 0; c < d_v; ++c) row[c] += ki * e[c];
    }
    /* read after the write: o = S^T q */
    if (o) {
      double *ot = o + (t * H_v + h) * d_v;
      for (int64_t c = 0; c < d_v; ++c) ot[c] = 0.0;
      for (int64_t i = 0; i < d_k; ++i) {
        const double qi = qq[i];
        const double *row = S + i * d_v;
        for (int64_t c = 0; c < d_v; ++c) ot[c] += row[c] * qi;
      }
    }
    if (states)
      memcpy(states + (t * n_heads + hi) * dkv, S, sizeof(double) * (size_t)dkv);
  }
  if (s_final)
    memcpy(s_final + (n * H_v + h) * dkv, S, sizeof(double) * (size_t)dkv);
}

/*
 * Runs the recurrence over n_seq sequences packed on one token axis.
 *
 *   cu      [n_seq+1]   token offsets: sequence n owns tokens [cu[n], cu[n+1])
 *                       (the split-point convention of the pages' packed rows);
 *                       a dense [B, T] batch is cu = {0, T, 2T, ..., B*T}.
 *   q, k    [T_tot, H_qk, d_k]  float32
 *   v       [T_tot, H_v,  d_v]  float32
 *   g, beta [T_tot, H_v]        float32 (g is a log decay, <= 0, may be -inf)
 *   s0      [n_seq, H_v, d_k, d_v] double, or NULL for a zero initial state
 *   heads   [n_heads] value heads to compute, or NULL for all H_v heads
 *   o       [T_tot, H_v, d_v] double or NULL; only the listed heads are written
 *   s_final [n_seq, H_v, d_k, d_v] double or NULL; only listed heads written
 *   states  [T_tot, n_heads, d_k, d_v] double or NULL: the state after every
 *           token, indexed by position in `heads` (by h when heads is NULL)
 *   nthreads <= 0 means all available threads.
 * Returns 0 on success, GDN_REF_EINVAL on a bad argument, GDN_REF_ENOMEM.
 */
int gdn_ref_forward(int64_t n_seq, const int64_t *cu, int64_t H_qk, int64_t H_v,
                    int64_t d_k, int64_t d_v, const float *q, const float *k,
                    const float *v, const float *g, const float *beta,
                    const double *s0, double scale, int l2norm,
                    const int64_t *heads, int64_t n_heads, double *o,
                    double *s_final, double *states, int nthreads) {
  if (n_seq < 0 || !cu || H_qk <= 0 || H_v <= 0 || H_v % H_qk || d_k <= 0 ||
      d_v <= 0)
    return GDN_REF_EINVAL;
  if (!heads) n_heads = H_v;
  if (n_heads < 0) return GDN_REF_EINVAL;
  for (int64_t n = 0; n < n_seq; ++n)
    if (cu[n + 1] < cu[n]) return GDN_REF_EINVAL;
  if (heads)
    for (int64_t x = 0; x < n_heads; ++x)
      if (heads[x] < 0 || heads[x] >= H_v) return GDN_REF_EINVAL;
  if (cu[n_seq] > cu[0] && (!q || !k || !v || !g || !beta))
    return GDN_REF_EINVAL;

  const int64_t units = n_seq * n_heads;
  int failed = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
#endif
  {
    const size_t per = (size_t)(d_k * d_v + 2 * d_k + d_v);
    double *buf = (double *)malloc(sizeof(double) * per);
    if (!buf) {
      failed = 1;
    } else {
      double *S = buf, *kk = S + d_k * d_v, *qq = kk + d_k, *e = qq + d_k;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
      for (int64_t u = 0; u < units; ++u) {
        const int64_t n = u / n_heads, hi = u % n_heads;
        const int64_t h = heads ? heads[hi] : hi;
        run_unit(cu[n], cu[n + 1], h, hi, n, H_qk, H_v, d_k, d_v, n_heads, q, k,
                 v, g, beta, s0, scale, l2norm, o, s_final, states, S, kk, qq,
                 e);
      }
      free(buf);
    }
  }
  (void)nthreads;
  return failed ? GDN_REF_ENOMEM : GDN_REF_OK;
}

/* Number of threads the library would use for nthreads <= 0. */
int gdn_ref_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
