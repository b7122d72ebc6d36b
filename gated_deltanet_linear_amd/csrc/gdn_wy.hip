// The bf16 chunked path of libgdn (d_k = 128, chunk C = 64): gdn_chunk_fwd and
// gdn_states_fwd on bf16 q, k, v.
//
// It computes the gated delta rule of the pages (Qwen3.5 text encyclopedia
// page, note "The DeltaNet mixer") in the UT / WY chunk form, arranged so that
// the sequential part -- the carry of the state S from chunk to chunk -- holds
// only the products that depend on S.  Per (chunk, value head), with the
// in-chunk cumulative log decay G_r = g_0 + ... + g_r:
//
//   A[r,i] = beta_r e^{G_r - G_i} (k_r . k_i), i < r       T = (I + A)^{-1}
//   P[r,i] = e^{G_r - G_i} (q_r . k_i), i <= r
//   W      = T diag(beta e^G) K        (C x d_k)       prep, all chunks at once
//   U'     = T diag(beta) V            (C x d_v)       prep, all chunks at once
//   U      = U' - W S                                  chain
//   O      = diag(e^G) Q S + P U                       chain
//   S     <- e^{G_last} S + K^T diag(e^{G_last - G}) U chain
//
// U' - W S is T diag(beta) (V - diag(e^G) K S), the tokens' write vectors of
// the token recursion.  With l2norm, k and q carry their row norms as factors
// inside W, P and the per-token vectors, and K, Q themselves stay the exact
// bf16 inputs.
//
// Launch sequence: plan (gdn_chunk.hip), prep (chunk, value head), chain
// (sequence, value head, block of 16 NB value columns), and on the states path
// the per-token stream (gdn_chunk.hip).
//
// Chain: 4 waves per block.  Wave w keeps rows [32w, 32w + 32) of the S block
// in registers, and computes the token tile [16w, 16w + 16) of U and O.  Per
// chunk it publishes its S rows in LDS (bf16 hi/lo), forms U = U' - W S and
// Q S for its token tile, publishes U, then updates its S rows with K^T U and
// finishes its O rows with P U: two barriers per chunk.  Every operand that
// does not depend on S is loaded from the workspace straight into registers,
// two chunks ahead, in the lane order of the MFMA that consumes it; nothing
// but S and U passes through LDS.
//
// MFMA lane order (v_mfma_f32_16x16x32_bf16): lane l feeds row l%16 of A and
// column l%16 of B, and 8 contraction indices given by the group l/16.  The
// accumulator holds rows 4(l/16) + i, i < 4, of column l%16.  Here the 8
// contraction indices of group g in step s are {32s + 4g + i, 32s + 16 + 4g + i},
// i < 4: the rows that lane l holds in the accumulators of two vertically
// adjacent tiles.  So S (rows of d_k) and U (rows of tokens) become B operands
// without any transposition, and every workspace operand is stored in that
// order.
//
// Precision: as on the fp32 path, products of computed values (S, W, U, P)
// enter MFMA as bf16 hi/lo pairs (hi*hi + hi*lo + lo*hi); q, k, v enter once.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn.h"

namespace gdn {
namespace {

constexpr int DK = 128, C = 64;
constexpr int LDQ = DK + 8;  // q, k rows (bf16)
constexpr int LDT = C + 8;   // K^T, V^T, T', T'' rows (bf16)
constexpr int LDF = C + 4;   // fp32 C x C
constexpr float kFloor = -1.0e4f;

__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ bf16x8 as_bf(const u32x4 &x) { return __builtin_bit_cast(bf16x8, x); }

// Two fp32 values -> one packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest
// even), and the pair's halves back as fp32.
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, bf16x2_t));
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// x = hi + lo + O(2^-17 |x|) for the 4 values of a.
__device__ __forceinline__ void split4(const f32x4 &a, u32x2 &hi, u32x2 &lo) {
  const uint32_t h0 = pk_bf16(a[0], a[1]), h1 = pk_bf16(a[2], a[3]);
  hi = u32x2{h0, h1};
  lo = u32x2{pk_bf16(a[0] - bf_lo(h0), a[1] - bf_hi(h0)), pk_bf16(a[2] - bf_lo(h1), a[3] - bf_hi(h1))};
}
// The 8 values {a[0..3], b[0..3]} as one bf16x8 hi and one lo fragment.
__device__ __forceinline__ void split8(const f32x4 &a, const f32x4 &b, u32x4 &hi, u32x4 &lo) {
  u32x2 ah, al, bh, bl;
  split4(a, ah, al);
  split4(b, bh, bl);
  hi = u32x4{ah[0], ah[1], bh[0], bh[1]};
  lo = u32x4{al[0], al[1], bl[0], bl[1]};
}
__device__ __forceinline__ u32x4 cat(const u32x2 &a, const u32x2 &b) { return u32x4{a[0], a[1], b[0], b[1]}; }
template <bool BF> __device__ __forceinline__ auto out_cvt(float x) {
  if constexpr (BF) return f2bf(x);
  else return x;
}

// ---------------------------------------------------------------------------
// prep: one (chunk, value head) per block of 4 waves.  Wave w owns token tile
// [16w, 16w + 16): its rows of P, W and U'.  One LDS region (36 KiB, four
// blocks per CU) holds in turn the q, k rows, then A and T (fp32), then K^T and
// V^T (bf16).
// ---------------------------------------------------------------------------
struct PrepSmem {
  static constexpr int RA = 2 * C * LDQ * 2, RB = 2 * C * LDF * 4, RC = (DK + 128) * LDT * 2;
  static constexpr int R = RA > RB ? (RA > RC ? RA : RC) : (RB > RC ? RB : RC);
  alignas(16) unsigned char r[R];
  alignas(16) double gam[C];
  float beta[C], rq[C], rk[C], eg[C];
};

__global__ __launch_bounds__(256) void wy_prep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const int32_t *__restrict__ status,
    const int32_t *__restrict__ seq_start, const int32_t *__restrict__ chunk_first,
    unsigned char *__restrict__ wf, unsigned char *__restrict__ pf, float *__restrict__ uf,
    float *__restrict__ fac, unsigned char *__restrict__ ktf, unsigned char *__restrict__ qf, int N, int H_qk,
    int H_v, int d_v, int MC, float scale, int l2norm) {
  __shared__ PrepSmem sm;
  if (*status) return;
  const int c = blockIdx.x;
  if (c >= chunk_first[N]) return;
  const int n = find_seq(chunk_first, N, c);
  const int t0 = seq_start[n] + (c - chunk_first[n]) * C;
  const int len = min(C, seq_start[n + 1] - t0);
  const int h = blockIdx.y, R = H_v / H_qk, j = h / R;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t slot = (int64_t)h * MC + c;  // head-major: one head's chunks are contiguous
  uint16_t *sq = reinterpret_cast<uint16_t *>(sm.r), *sk = sq + C * LDQ;

  // Every global load of the chunk is issued before the first use.  Rows past
  // the chunk's length read a valid row and are replaced by zeros when stored.
  const int VV = d_v / 8;
  u32x4 qv[4], kv[4], vv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int x = tid + 256 * i, r = min(x >> 4, len - 1), cv = x & 15;
    const int64_t off = ((int64_t)(t0 + r) * H_qk + j) * DK + cv * 8;
    qv[i] = *reinterpret_cast<const u32x4 *>(q + off);
    kv[i] = *reinterpret_cast<const u32x4 *>(k + off);
    const int xv = min(x, C * VV - 1), rv = min(xv / VV, len - 1);
    vv[i] = *reinterpret_cast<const u32x4 *>(v + ((int64_t)(t0 + rv) * H_v + h) * d_v + (xv % VV) * 8);
  }
  const int tl = min(lane, len - 1);
  const float graw = g[(int64_t)(t0 + tl) * H_v + h], braw = beta[(int64_t)(t0 + tl) * H_v + h];
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int x = tid + 256 * i, r = x >> 4, cv = x & 15;
    *reinterpret_cast<u32x4 *>(sq + r * LDQ + cv * 8) = r < len ? qv[i] : zero;
    *reinterpret_cast<u32x4 *>(sk + r * LDQ + cv * 8) = r < len ? kv[i] : zero;
  }
  // In-chunk cumulative decay (fp64) and write strengths; zero past the length.
  if (w == 3) {
    const double gv = lane < len ? (double)fmaxf(graw, kFloor) : 0.0;
    const double gm = wave_inclusive_scan(gv, lane);
    sm.gam[lane] = gm;
    sm.eg[lane] = expf((float)gm);
    sm.beta[lane] = lane < len ? braw : 0.f;
  }
  __syncthreads();
  // Q fragments, once per (chunk, query/key head): item (token tile w, d_k step
  // s, lane) = Q[16w + l%16][{32s + 4g + i, 32s + 16 + 4g + i}].
  if (h % R == 0) {
    u32x4 *Q4 = reinterpret_cast<u32x4 *>(qf + ((int64_t)j * MC + c) * kWyQBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int it = tid + 256 * i, ln = it & 63, ws = it >> 6;
      const uint16_t *row = sq + (16 * (ws >> 2) + (ln & 15)) * LDQ + 32 * (ws & 3) + 4 * (ln >> 4);
      Q4[it] = cat(*reinterpret_cast<const u32x2 *>(row), *reinterpret_cast<const u32x2 *>(row + 16));
    }
  }
  if (tid < 2 * C) {
    const int r = tid % C;
    float rn = 1.f;
    if (l2norm) {
      const uint16_t *row = (tid < C ? sq : sk) + r * LDQ;
      float ss = 0.f;
      for (int i = 0; i < DK; ++i) {
        const float a = bf2f(row[i]);
        ss += a * a;
      }
      rn = 1.0f / sqrtf(ss + 1e-6f);
    }
    if (tid < C) sm.rq[r] = rn * scale;
    else sm.rk[r] = rn;
  }
  // Gram tiles, 5 per wave, kept in registers: wave w takes the w + 1 tiles
  // (K Q^T)[16 ni.., 16 w..], ni <= w, whose accumulators hold P's rows of token
  // tile w in the carry's lane order, and 4 - w of the 10 lower tiles of K K^T.
  constexpr int kKKFirst[4] = {0, 4, 7, 9};
  f32x4 acc[5];
  int kmi[5], kni[5];
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    const bool isp = m <= w;
    int mi = w, ni = m;
    if (!isp) {
      const int t = kKKFirst[w] + (m - w - 1);
      mi = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
      ni = t - mi * (mi + 1) / 2;
    }
    kmi[m] = mi;
    kni[m] = ni;
    // isp: A = K rows of tile ni, B = Q rows of tile w.  else: A = K tile mi, B = K tile ni.
    const uint16_t *Ab = sk + ((isp ? ni : mi) * 16 + lr) * LDQ + 8 * lg;
    const uint16_t *Bb = (isp ? sq + (w * 16 + lr) * LDQ : sk + (ni * 16 + lr) * LDQ) + 8 * lg;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += 32) a = mfma_bf16(ld8(Ab + k0), ld8(Bb + k0), a);
    acc[m] = a;
  }
  __syncthreads();  // the q, k rows are dead; the region holds A and T from here

  float *A = reinterpret_cast<float *>(sm.r), *Tm = A + C * LDF;
  {
    u32x4 *P4 = reinterpret_cast<u32x4 *>(pf + slot * kWyPBytes);
    const int r = 16 * w + lr;  // P row of this lane
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      if (m <= w) {
        // P[r][16m + 4lg + i] = rq_r rk_i e^{G_r - G_i} (q_r . k_i), i <= r
        f32x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ci = 16 * m + 4 * lg + e;
          pv[e] = ci <= r ? sm.rq[r] * sm.rk[ci] * expf((float)(sm.gam[r] - sm.gam[ci])) * acc[m][e] : 0.f;
        }
        u32x2 hi, lo;
        split4(pv, hi, lo);
        // fragment (w, st = m / 2): elements 0-3 from tile 2st, 4-7 from tile 2st + 1
        u32x2 *P2 = reinterpret_cast<u32x2 *>(P4 + ((w * 2 + (m >> 1)) * 2) * 64 + lane) + (m & 1);
        P2[0] = hi;
        P2[128] = lo;  // the lo plane is 64 lanes (1 KiB) further
        if ((m & 1) == 0 && m == w) {  // tile 2st + 1 is above the diagonal: zero
          P2[1] = u32x2{0u, 0u};
          P2[129] = u32x2{0u, 0u};
        }
      } else {
        // A[r][i] = beta_r rk_r rk_i e^{G_r - G_i} (k_r . k_i), i < r
        const int mi = kmi[m], ni = kni[m];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 16 * mi + 4 * lg + e, ci = 16 * ni + lr;
          A[rr * LDF + ci] = ci < rr ? sm.beta[rr] * sm.rk[rr] * sm.rk[ci] *
                                           expf((float)(sm.gam[rr] - sm.gam[ci])) * acc[m][e]
                                     : 0.f;
        }
      }
    }
  }
  // Per-token factors: e^G q-norm (scale included), e^{G_last - G} k-norm, e^{G_last}.
  if (tid < C) {
    float *F = fac + slot * kWyFac;
    const double gl = sm.gam[len - 1];
    F[tid] = sm.eg[tid] * sm.rq[tid];
    F[C + tid] = tid < len ? expf((float)(gl - sm.gam[tid])) * sm.rk[tid] : 0.f;
    if (tid == 0) F[2 * C] = expf((float)gl);
  }
  __syncthreads();

  // T = (I + A)^{-1}.  Diagonal 16x16 blocks by forward substitution: lane
  // 16 b + cc owns column cc of block b.
  if (w == 0) {
    const int bb = lane >> 4, cc = lane & 15;
    const float *Ab = A + (bb * 16) * LDF + bb * 16;
    float col[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = (r == cc) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) s -= Ab[r * LDF + m] * col[m];
      col[r] = s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Tm[(bb * 16 + r) * LDF + bb * 16 + cc] = col[r];
  }
  __syncthreads();
  // Below the diagonal, wave jb fills block column jb from the top down:
  //   T_ib,jb = -T_ib,ib * Y,  Y = sum_{m=jb}^{ib-1} A_ib,m T_m,jb     (fp32 MFMA 16x16x4)
  // Y's MFMA feeds contraction index 4s + l/16 in step s; the second product
  // feeds 4(l/16) + s, which makes its B operand in step s this lane's own
  // accumulator element Y[4(l/16) + s][l%16].
  if (w < 3) {
    const int jb = w;
    for (int ib = jb + 1; ib < 4; ++ib) {
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      for (int m = jb; m < ib; ++m) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          y = mfma_f32(A[(16 * ib + lr) * LDF + 16 * m + 4 * s + lg], Tm[(16 * m + 4 * s + lg) * LDF + 16 * jb + lr], y);
      }
      f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) t = mfma_f32(Tm[(16 * ib + lr) * LDF + 16 * ib + 4 * lg + s], y[s], t);
#pragma unroll
      for (int e = 0; e < 4; ++e) Tm[(16 * ib + 4 * lg + e) * LDF + 16 * jb + lr] = -t[e];
    }
  }
  __syncthreads();

  // This wave's fragments of T' = T diag(beta e^G k-norm) and T'' = T diag(beta)
  // (rows of token tile w, columns 32 st + 8 lg .. + 7), bf16 hi/lo.  T' is the
  // B operand of W^T = K^T T'^T and T'' the A operand of U' = T'' V.
  u32x4 t1h[2], t1l[2], t2h[2], t2l[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    if (st <= (w >> 1)) {
      const int r = 16 * w + lr;
      f32x4 a1, b1, a2, b2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ci = 32 * st + 8 * lg + e;
        const float t = ci <= r ? Tm[r * LDF + ci] * sm.beta[ci] : 0.f;
        const float t1 = t * sm.eg[ci] * sm.rk[ci];
        if (e < 4) {
          a2[e] = t;
          a1[e] = t1;
        } else {
          b2[e - 4] = t;
          b1[e - 4] = t1;
        }
      }
      split8(a1, b1, t1h[st], t1l[st]);
      split8(a2, b2, t2h[st], t2l[st]);
    }
  }
  __syncthreads();  // A and T are dead; the region holds K^T and V^T from here
  uint16_t *kt = reinterpret_cast<uint16_t *>(sm.r), *vt = kt + DK * LDT;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int x = tid + 256 * i, r = x >> 4, cv = x & 15;
    const u32x4 b = r < len ? kv[i] : zero;
#pragma unroll
    for (int e = 0; e < 8; ++e) kt[(cv * 8 + e) * LDT + r] = (uint16_t)(b[e >> 1] >> (16 * (e & 1)));
    if (x < C * VV) {
      const int rv = x / VV, cvv = x % VV;
      const u32x4 c4 = rv < len ? vv[i] : zero;
#pragma unroll
      for (int e = 0; e < 8; ++e) vt[(cvv * 8 + e) * LDT + rv] = (uint16_t)(c4[e >> 1] >> (16 * (e & 1)));
    }
  }
  __syncthreads();

  // W^T = K^T T'^T for token tile w, by d_k step s: the tiles of d_k rows 32s..
  // and 32s+16.. give this lane W[16w + l%16][{32s + 4g + i, 32s + 16 + 4g + i}].
  {
    u32x4 *W4 = reinterpret_cast<u32x4 *>(wf + slot * kWyWBytes) + w * 8 * 64 + lane;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st <= (w >> 1)) {  // T' is lower triangular
          const int ko = 32 * st + 8 * lg;
          const bf16x8 a0 = ld8(kt + (32 * s + lr) * LDT + ko), a1 = ld8(kt + (32 * s + 16 + lr) * LDT + ko);
          acc0 = mfma_bf16(a0, as_bf(t1h[st]), acc0);
          acc0 = mfma_bf16(a0, as_bf(t1l[st]), acc0);
          acc1 = mfma_bf16(a1, as_bf(t1h[st]), acc1);
          acc1 = mfma_bf16(a1, as_bf(t1l[st]), acc1);
        }
      }
      u32x4 hi, lo;
      split8(acc0, acc1, hi, lo);
      W4[(s * 2 + 0) * 64] = hi;
      W4[(s * 2 + 1) * 64] = lo;
    }
  }
  // U' = T'' V for token tile w, by value column tile ct, in accumulator order.
  {
    const int NCT = d_v / 16;
    f32x4 *U4 = reinterpret_cast<f32x4 *>(uf + slot * (int64_t)(C * d_v)) + w * NCT * 64 + lane;
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st <= (w >> 1)) {
          const bf16x8 b = ld8(vt + (16 * ct + lr) * LDT + 32 * st + 8 * lg);
          a = mfma_bf16(as_bf(t2h[st]), b, a);
          a = mfma_bf16(as_bf(t2l[st]), b, a);
        }
      }
      U4[ct * 64] = a;
    }
  }
  // K^T fragments, once per (chunk, query/key head): item (d_k tile mt, token
  // step st, lane) = K^T[16 mt + l%16][{32 st + 4g + i, 32 st + 16 + 4g + i}].
  if (h % R == 0) {
    u32x4 *K4 = reinterpret_cast<u32x4 *>(ktf + ((int64_t)j * MC + c) * kWyKtBytes);
    for (int it = tid; it < 16 * 64; it += 256) {
      const int ln = it & 63, ms = it >> 6, mt = ms >> 1, st = ms & 1;
      const uint16_t *row = kt + (16 * mt + (ln & 15)) * LDT + 32 * st + 4 * (ln >> 4);
      K4[it] = cat(*reinterpret_cast<const u32x2 *>(row), *reinterpret_cast<const u32x2 *>(row + 16));
    }
  }
}

// ---------------------------------------------------------------------------
// chain: one (sequence, value head, 16 NB-column block of S) per block of 4 waves.
// ---------------------------------------------------------------------------
// The operands of one chunk that do not depend on S, held in registers.
template <int NB> struct ChainOps {
  u32x4 w[4][2];   // W hi/lo: token tile of this wave, d_k steps 0..3
  u32x4 q[4];      // q rows of the token tile, d_k steps 0..3
  u32x4 kt[2][2];  // K^T: this wave's two d_k tiles, token steps 0..1
  u32x4 p[2][2];   // P hi/lo: token tile of this wave, token steps 0..1
  f32x4 u[NB];     // U' tiles
  f32x4 fq, fu;    // e^G q-norm, e^{G_last - G} k-norm for the 4 rows of this lane
  float el;        // e^{G_last}
};

template <int NB, bool STATES, bool OBF16>
__global__ __launch_bounds__(256) void wy_chain_kernel(
    const uint16_t *__restrict__ q, const float *__restrict__ s0, const int32_t *__restrict__ status,
    const int32_t *__restrict__ seq_start, const int32_t *__restrict__ chunk_first,
    const unsigned char *__restrict__ wf, const unsigned char *__restrict__ pf, const float *__restrict__ uf,
    const float *__restrict__ fac, const unsigned char *__restrict__ ktf, const unsigned char *__restrict__ qf,
    void *__restrict__ o,
    float *__restrict__ fin, float *__restrict__ uw, float *__restrict__ scw, int N, int H_qk, int H_v,
    int d_v, int MC, int units, int grid) {
  // S rows and U rows as published by their owner wave, in the owner's lane order.
  __shared__ u32x4 sx[NB][4][2][64];
  __shared__ u32x2 ux[NB][4][2][64];
  __shared__ u32x2 u2x[NB][4][2][64];
  constexpr int LDO = 16 * NB + 4;  // O tile rows, fp32 (the pad spreads rows over the banks)
  __shared__ float ot[4][16 * LDO];
  if (*status) return;
  const int u = xcd_remap(blockIdx.x, grid);
  if (u >= units) return;
  const int NJB = d_v / (16 * NB), NCT = d_v / 16;
  const int jb = u % NJB, h = (u / NJB) % H_v, n = u / (NJB * H_v);
  const int j = h / (H_v / H_qk);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int col0 = jb * 16 * NB;
  const int64_t sbase = (int64_t)(n * H_v + h) * DK;

  // S[mt][nb] holds rows 32w + 16mt + 4lg + i, column col0 + 16nb + lr.
  f32x4 S[2][NB];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      S[mt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (s0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[mt][nb][i] = s0[(sbase + 32 * w + 16 * mt + 4 * lg + i) * d_v + col0 + 16 * nb + lr];
      }
    }

  const int c_begin = chunk_first[n], c_end = chunk_first[n + 1];
  const int s_begin = seq_start[n], s_end = seq_start[n + 1];
  // Drain the initial-state loads here, so that inside the chunk loop the
  // vector-memory counter covers only the operand prefetches.
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

  // Where chunk c's operands live, for this lane.
  struct Src {
    const u32x4 *w, *kt, *p, *q;
    const f32x4 *u;
    const float *f;
  };
  auto src = [&](int c) {
    Src a;
    const int64_t slot = (int64_t)h * MC + c;
    a.w = reinterpret_cast<const u32x4 *>(wf + slot * kWyWBytes) + w * 8 * 64 + lane;
    a.kt = reinterpret_cast<const u32x4 *>(ktf + ((int64_t)j * MC + c) * kWyKtBytes) + 2 * w * 2 * 64 + lane;
    a.p = reinterpret_cast<const u32x4 *>(pf + slot * kWyPBytes) + w * 2 * 2 * 64 + lane;
    a.q = reinterpret_cast<const u32x4 *>(qf + ((int64_t)j * MC + c) * kWyQBytes) + w * 4 * 64 + lane;
    a.u = reinterpret_cast<const f32x4 *>(uf + slot * (int64_t)(C * d_v)) + (w * NCT + jb * NB) * 64 + lane;
    a.f = fac + slot * kWyFac;
    return a;
  };
  auto load_wq = [&](ChainOps<NB> &op, const Src &a, int s) {
    op.w[s][0] = a.w[(s * 2 + 0) * 64];
    op.w[s][1] = a.w[(s * 2 + 1) * 64];
    op.q[s] = a.q[s * 64];
  };
  auto load_uf = [&](ChainOps<NB> &op, const Src &a) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) op.u[nb] = a.u[nb * 64];
    op.fq = *reinterpret_cast<const f32x4 *>(a.f + 16 * w + 4 * lg);
    op.fu = *reinterpret_cast<const f32x4 *>(a.f + C + 16 * w + 4 * lg);
    op.el = a.f[2 * C];
  };
  auto load_kt = [&](ChainOps<NB> &op, const Src &a, int mt) {
    op.kt[mt][0] = a.kt[(mt * 2 + 0) * 64];
    op.kt[mt][1] = a.kt[(mt * 2 + 1) * 64];
  };
  auto load_p = [&](ChainOps<NB> &op, const Src &a) {
#pragma unroll
    for (int st = 0; st < 2; ++st)
      if (st <= (w >> 1))  // P is lower triangular: token tiles 0, 1 use step 0 only
#pragma unroll
        for (int pl = 0; pl < 2; ++pl) op.p[st][pl] = a.p[(st * 2 + pl) * 64];
  };
  // Scheduling groups (instruction classes for __builtin_amdgcn_sched_group_barrier).
  constexpr int kMFMA = 0x008, kVMR = 0x020, kDSR = 0x100;

  // One chunk; the operands of chunk `cn` are loaded behind it, each group of
  // registers right after its last use here, interleaved with the MFMAs so that
  // the loads stream while the matrix cores work.
  auto chunk = [&](ChainOps<NB> &op, int c, int cn) {
    const int t0 = s_begin + (c - c_begin) * C;
    const int len = min(C, s_end - t0);
    const Src nx = src(cn);
    // 1. publish this wave's S rows (the B operand of d_k step w)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      u32x4 hi, lo;
      split8(S[0][nb], S[1][nb], hi, lo);
      sx[nb][w][0][lane] = hi;
      sx[nb][w][1][lane] = lo;
      if constexpr (STATES) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            scw[(((int64_t)c * H_v + h) * DK + 32 * w + 16 * mt + 4 * lg + i) * d_v + col0 + 16 * nb + lr] =
                S[mt][nb][i];
      }
    }
    __syncthreads();
    // 2. W S and Q S for token tile w; W and q of the next chunk stream in behind
    f32x4 aw[NB], aq[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) aw[nb] = aq[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bf16x8 sh = as_bf(sx[nb][s][0][lane]), sl = as_bf(sx[nb][s][1][lane]);
        aw[nb] = mfma_bf16(as_bf(op.w[s][0]), sh, aw[nb]);
        aw[nb] = mfma_bf16(as_bf(op.w[s][0]), sl, aw[nb]);
        aw[nb] = mfma_bf16(as_bf(op.w[s][1]), sh, aw[nb]);
        aq[nb] = mfma_bf16(as_bf(op.q[s]), sh, aq[nb]);
        aq[nb] = mfma_bf16(as_bf(op.q[s]), sl, aq[nb]);
      }
      load_wq(op, nx, s);
      __builtin_amdgcn_sched_group_barrier(kDSR, 2 * NB, 0);
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        __builtin_amdgcn_sched_group_barrier(kMFMA, NB, 0);
        __builtin_amdgcn_sched_group_barrier(kVMR, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kMFMA, 2 * NB, 0);
    }
    // 3. U = U' - W S and U'' = diag(e^{G_last - G} k-norm) U; publish both
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const f32x4 uv = op.u[nb] - aw[nb];
      const f32x4 u2 = uv * op.fu;
      u32x2 hi, lo;
      split4(uv, hi, lo);
      ux[nb][w][0][lane] = hi;
      ux[nb][w][1][lane] = lo;
      split4(u2, hi, lo);
      u2x[nb][w][0][lane] = hi;
      u2x[nb][w][1][lane] = lo;
      aq[nb] *= op.fq;
      if constexpr (STATES) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * w + 4 * lg + i;
          if (r < len) uw[((int64_t)(t0 + r) * H_v + h) * d_v + col0 + 16 * nb + lr] = uv[i];
        }
      }
    }
    const float el = op.el;
    load_uf(op, nx);
    __syncthreads();
    // 4. S <- e^{G_last} S + K^T U'' for this wave's rows; U', the factors and
    //    K^T of the next chunk stream in behind
    bf16x8 bh[NB][2], bl[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bh[nb][st] = as_bf(cat(u2x[nb][2 * st][0][lane], u2x[nb][2 * st + 1][0][lane]));
        bl[nb][st] = as_bf(cat(u2x[nb][2 * st][1][lane], u2x[nb][2 * st + 1][1][lane]));
      }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        S[mt][nb] *= el;
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          S[mt][nb] = mfma_bf16(as_bf(op.kt[mt][st]), bh[nb][st], S[mt][nb]);
          S[mt][nb] = mfma_bf16(as_bf(op.kt[mt][st]), bl[nb][st], S[mt][nb]);
        }
      }
      load_kt(op, nx, mt);
    }
    __builtin_amdgcn_sched_group_barrier(kDSR, 8 * NB, 0);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(kMFMA, NB, 0);
      if (k == 3 || k == 7) __builtin_amdgcn_sched_group_barrier(kVMR, 2, 0);
    }
    //    O = e^G q-norm (Q S) + P U for token tile w; P of the next chunk behind it
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st <= (w >> 1)) {  // P is lower triangular
          const bf16x8 bh2 = as_bf(cat(ux[nb][2 * st][0][lane], ux[nb][2 * st + 1][0][lane]));
          const bf16x8 bl2 = as_bf(cat(ux[nb][2 * st][1][lane], ux[nb][2 * st + 1][1][lane]));
          aq[nb] = mfma_bf16(as_bf(op.p[st][0]), bh2, aq[nb]);
          aq[nb] = mfma_bf16(as_bf(op.p[st][0]), bl2, aq[nb]);
          aq[nb] = mfma_bf16(as_bf(op.p[st][1]), bh2, aq[nb]);
        }
      }
    }
    load_p(op, nx);
    if (o) {
      // The O tile goes through LDS so that each lane stores 4 consecutive
      // columns of one row: lane l takes row l%16 and columns 4(l/16) + 16 m.
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) ot[w][(4 * lg + i) * LDO + 16 * nb + lr] = aq[nb][i];
      __builtin_amdgcn_wave_barrier();
      const int r = 16 * w + lr;  // row of the chunk
      if (r < len) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(&ot[w][lr * LDO + 4 * lg]);
        const int64_t ob = ((int64_t)(t0 + r) * H_v + h) * d_v + col0 + 4 * lg;
#pragma unroll
        for (int m = 0; m < NB; ++m) {
          const f32x4 x = src[4 * m];
          if constexpr (OBF16) {
            *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(o) + ob + 16 * m) =
                u32x2{pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3])};
          } else {
            *reinterpret_cast<f32x4 *>(static_cast<float *>(o) + ob + 16 * m) = x;
          }
        }
      }
    }
  };

  // One register set.  The first chunk is peeled, so that the loop is entered
  // with the same memory operations in flight as on its back edge (the
  // compiler's wait counts are then exact).  Past the last chunk the loads
  // repeat the last chunk (always valid memory) and go unused.
  if (c_begin < c_end) {
    ChainOps<NB> op;
    {
      const Src a = src(c_begin);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) load_wq(op, a, s4);
      load_uf(op, a);
      load_kt(op, a, 0);
      load_kt(op, a, 1);
      load_p(op, a);
    }
    chunk(op, c_begin, min(c_begin + 1, c_end - 1));
    for (int c = c_begin + 1; c < c_end; ++c) chunk(op, c, min(c + 1, c_end - 1));
  }

  if (fin) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fin[(sbase + 32 * w + 16 * mt + 4 * lg + i) * d_v + col0 + 16 * nb + lr] = S[mt][nb][i];
  }
}

template <int NB, bool STATES, bool OBF16>
hipError_t run_wy(const Problem &p, const ChunkArgs &a, hipStream_t st) {
  const Workspace &w = a.ws;
  mark_event(a, 0, st);
  hipError_t e = launch_plan(p, a, st);
  if (e != hipSuccess) return e;
  mark_event(a, 1, st);
  const uint16_t *q = static_cast<const uint16_t *>(a.q), *k = static_cast<const uint16_t *>(a.k),
                 *v = static_cast<const uint16_t *>(a.v);
  if (p.max_chunks > 0 && p.H_v > 0) {
    hipLaunchKernelGGL(wy_prep_kernel, dim3(p.max_chunks, p.H_v), dim3(256), 0, st, q, k, v, a.g, a.beta,
                       w.status, w.seq_start, w.chunk_first, w.wf, w.pf, w.uf, w.fac, w.ktf, w.qf, p.N,
                       p.H_qk, p.H_v, p.d_v, p.max_chunks, p.scale, p.l2norm ? 1 : 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  mark_event(a, 2, st);
  const int units = p.N * p.H_v * (p.d_v / (16 * NB));
  if (units > 0) {
    const int grid = (units + 7) / 8 * 8;
    hipLaunchKernelGGL((wy_chain_kernel<NB, STATES, OBF16>), dim3(grid), dim3(256), 0, st, q, a.s0, w.status,
                       w.seq_start, w.chunk_first, w.wf, w.pf, w.uf, w.fac, w.ktf, w.qf, a.o, a.final_state, w.u,
                       w.sc, p.N, p.H_qk, p.H_v, p.d_v, p.max_chunks, units, grid);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  mark_event(a, 3, st);
  if constexpr (STATES) {
    if ((e = launch_states_stream(p, a, st)) != hipSuccess) return e;
    mark_event(a, 4, st);
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_wy_path(const Problem &p, const ChunkArgs &a, bool states, hipStream_t st) {
  if (p.d_k != DK || p.C != C || p.d_v % 32 != 0 || p.d_v > 128) return hipErrorInvalidValue;
  const bool ob = p.o_dtype == GDN_BF16;
  if (states) return ob ? run_wy<1, true, true>(p, a, st) : run_wy<1, true, false>(p, a, st);
  return ob ? run_wy<1, false, true>(p, a, st) : run_wy<1, false, false>(p, a, st);
}

}  // namespace gdn
