// The bf16 chunked path of libgdn (d_k = 128, chunk C = 64): gdn_chunk_fwd and
// gdn_states_fwd on bf16 q, k, v.
//
// It computes the gated delta rule of the pages (Qwen3.5 text encyclopedia
// page, note "The DeltaNet mixer") in the UT / WY chunk form, arranged so that
// the sequential part -- the carry of the state S from chunk to chunk -- holds
// only the products that depend on S.  Per (chunk, value head), with the
// in-chunk cumulative log decay G_r = g_0 + ... + g_r, normalised keys
// K^ = diag(rk) K and scaled queries Q^ = diag(rq) Q (rq = scale, times the
// row's inverse norm with GDN_QK_L2NORM; rk = 1 or that norm):
//
//   A[r,i] = beta_r e^{G_r - G_i} (k^_r . k^_i), i < r      T = (I + A)^{-1}
//   P[r,i] = e^{G_r - G_i} (q^_r . k^_i), i <= r            R = P T
//   W      = T diag(beta e^G) K^          (C x d_k)  \
//   U'     = T diag(beta) V               (C x d_v)   | prep, all chunks
//   Q'     = diag(e^G) Q^ - R diag(beta e^G) K^         | at once
//   O'     = R diag(beta) V                            /
//   U      = U' - W S                                  chain
//   O      = Q' S + O'                                 chain
//   S     <- e^{G_last} S + K^^T diag(e^{G_last - G}) U chain
//
// U' - W S is T diag(beta) (V - diag(e^G) K^ S), the tokens' write vectors of
// the token recursion, and Q' S + O' = diag(e^G) Q^ S + P U: the output's
// intra-chunk part P U' is formed in prep at full precision, and the chain's
// output needs S alone.
//
// Launch sequence: plan (gdn_chunk.hip), prep (chunk, value head), chain
// (sequence, value head, block of 16 NB value columns), and on the states path
// the per-token stream (gdn_chunk.hip).
//
// Chain: 8 waves per block.  Waves 0-3 carry the state: wave w keeps rows
// [32w, 32w + 32) of the S block in registers and forms U for the token tile
// [16w, 16w + 16); waves 4-7 form O from the S that the state waves publish in
// LDS: two barriers per chunk.  Every operand that does not depend on S is
// loaded from the workspace straight into registers, one chunk ahead, in the
// lane order of the MFMA that consumes it; nothing but S and U passes through
// LDS.
//
// MFMA lane order (v_mfma_f32_16x16x32_{bf16,f16}): lane l feeds row l%16 of A
// and column l%16 of B, and 8 contraction indices given by the group l/16.  The
// accumulator holds rows 4(l/16) + i, i < 4, of column l%16.  Here the 8
// contraction indices of group g in step s are {32s + 4g + i, 32s + 16 + 4g + i},
// i < 4: the rows that lane l holds in the accumulators of two vertically
// adjacent tiles.  So S (rows of d_k) and U (rows of tokens) become B operands
// without any transposition, and every workspace operand is stored in that
// order.
//
// Precision.  Prep: q, k, v enter bf16 MFMA exactly; computed fp32 operands
// (T, P, R and their diagonal scalings) enter as bf16 hi/lo pairs (hi*hi +
// hi*lo + lo*hi).  Chain: its operands are fp16 (11 significant bits): W, Q'
// and S once, K^ once (exact for the bf16 inputs in fp16's normal range), and
// the write vectors diag(e^{G_last - G}) U as an fp16 hi/lo pair, which keeps
// the state's own rounding at ~2^-22 per chunk.  A numpy emulation of this
// placement on the 4096-token prefill laws gives max |dO| ~2e-3 x RMS(o) and a
// final-state error ~1e-7 (6e-5 with slow decays), against single-fp16 P U
// (6e-3 x RMS), which is why the P U' product stays in prep.  fp16's range
// bounds the carried values: |S|, |W| and |Q'| entries must stay below 65504.
#include <atomic>
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn.h"

namespace gdn {
namespace {

constexpr int DK = 128, C = 64;
constexpr int LDQ = DK + 8;  // q, k rows (bf16)
constexpr int LDT = C + 2;   // K^T, V^T rows (bf16): an odd number of words spreads the
                             // transposing 2-byte stores over the LDS banks
constexpr int LDF = C + 4;   // fp32 C x C
constexpr float kFloor = -1.0e4f;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8 ld8(const uint16_t *p) { return *reinterpret_cast<const bf16x8 *>(p); }
// bf16 elements p[0..3] and p[16..19] (4-byte aligned): the split contraction order.
__device__ __forceinline__ bf16x8 ld8s(const uint16_t *p) {
  const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
  return __builtin_bit_cast(bf16x8, u32x4{q[0], q[1], q[8], q[9]});
}
// e^x on the hardware exponential (v_exp_f32 of x log2 e): relative error a few
// ulp for the decay arguments met here (|x| below a few hundred).
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ bf16x8 as_bf(const u32x4 &x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ f16x8 as_h(const u32x4 &x) { return __builtin_bit_cast(f16x8, x); }
__device__ __forceinline__ f32x4 mfma_f16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h(a), as_h(b), c, 0, 0, 0);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two fp32 values -> one packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest
// even), and the pair's halves back as fp32.
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, bf16x2_t));
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
// The same for fp16 (v_cvt_pk_f16_f32, round to nearest even).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_f16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, f16x2_t));
}
__device__ __forceinline__ f32x2_t unpk_f16(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
}

// x = hi + lo + O(2^-17 |x|) for the 4 values of a (bf16).
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
// fp16: the 4 values of a once, and as hi + lo (x = hi + lo + O(2^-22 |x|) in
// fp16's normal range).
__device__ __forceinline__ u32x2 h16x4(const f32x4 &a) { return u32x2{pk_f16(a[0], a[1]), pk_f16(a[2], a[3])}; }
__device__ __forceinline__ u32x4 h16x8(const f32x4 &a, const f32x4 &b) {
  return u32x4{pk_f16(a[0], a[1]), pk_f16(a[2], a[3]), pk_f16(b[0], b[1]), pk_f16(b[2], b[3])};
}
__device__ __forceinline__ void split4h(const f32x4 &a, u32x2 &hi, u32x2 &lo) {
  hi = h16x4(a);
  const f32x2_t h0 = unpk_f16(hi[0]), h1 = unpk_f16(hi[1]);
  lo = u32x2{pk_f16(a[0] - h0[0], a[1] - h0[1]), pk_f16(a[2] - h1[0], a[3] - h1[1])};
}

// ---------------------------------------------------------------------------
// prep: one (chunk, value head) per block of 4 waves.  Wave w owns token tile
// [16w, 16w + 16): its rows of P, R, W, U', Q' and O'.  One LDS region (36 KiB,
// four blocks per CU) holds in turn the q, k rows, then A and T (fp32), then
// K^T and V^T (bf16).
// ---------------------------------------------------------------------------
struct PrepSmem {
  static constexpr int RA = 2 * C * LDQ * 2, RB = 2 * C * LDF * 4, RC = (DK + 128) * LDT * 2;
  static constexpr int R = RA > RB ? (RA > RC ? RA : RC) : (RB > RC ? RB : RC);
  alignas(16) unsigned char r[R];
  alignas(16) double gam[C];
  alignas(16) float beta[C], rq[C], rk[C], eg[C];
  alignas(16) float bek[C];  // beta e^G k-norm: the column scaling of T' and R'
};

__global__ __launch_bounds__(256) void wy_prep_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const Seqs seqs,
    unsigned char *__restrict__ wf, unsigned char *__restrict__ qf, float *__restrict__ uf,
    float *__restrict__ of, float *__restrict__ fac, unsigned char *__restrict__ ktf, int H_qk, int H_v,
    int d_v, int MC, float scale, int l2norm) {
  __shared__ PrepSmem sm;
  if (seqs.bad()) return;
  // Chunks run last to first, so that the chain's first chunks are the ones
  // written last (still in the Infinity Cache, and in L2 below); within a chunk,
  // the value heads are ordered so that the block of head h lands on the XCD of
  // the chain group that reads it (workgroups are dealt to the 8 XCDs round
  // robin; the chain puts (sequence n, query/key head j) on XCD (n H_qk + j) % 8).
  const int cpos = blockIdx.x / H_v, p = blockIdx.x % H_v;
  const int nch = seqs.chunks();
  if (cpos >= nch) return;
  const int c = nch - 1 - cpos;
  const int n = seqs.seq_of(c);
  const int t0 = seqs.start(n) + (c - seqs.first(n)) * C;
  const int len = min(C, seqs.start(n + 1) - t0);
  const int R = H_v / H_qk;
  int h = p;
  if (H_qk % 8 == 0 && H_v % 8 == 0) {
    const int x = p & 7, kk = p >> 3;  // XCD of this block, and its rank among the chunk's blocks there
    h = (x + 8 * (kk / R)) * R + kk % R;
  }
  const int j = h / R;
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
  // 1/|q_r| (times the scale) and 1/|k_r| from the loaded rows: the 16 loads of
  // row r sit on 16 neighbouring lanes, whose shuffle sum gives the row's sum of
  // squares.  Rows past the length hold the last row (finite; their q, k rows
  // are zero in LDS).
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float s2q = 0.f, s2k = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float q0 = bf_lo(qv[i][e]), q1 = bf_hi(qv[i][e]), k0 = bf_lo(kv[i][e]), k1 = bf_hi(kv[i][e]);
      s2q += q0 * q0 + q1 * q1;
      s2k += k0 * k0 + k1 * k1;
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      s2q += __shfl_xor(s2q, o);
      s2k += __shfl_xor(s2k, o);
    }
    if ((lane & 15) == 0) {
      const int r = (tid + 256 * i) >> 4;
      sm.rq[r] = (l2norm ? 1.0f / sqrtf(s2q + 1e-6f) : 1.f) * scale;
      sm.rk[r] = l2norm ? 1.0f / sqrtf(s2k + 1e-6f) : 1.f;
    }
  }
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int x = tid + 256 * i, r = x >> 4, cv = x & 15;
    *reinterpret_cast<u32x4 *>(sq + r * LDQ + cv * 8) = r < len ? qv[i] : zero;
    *reinterpret_cast<u32x4 *>(sk + r * LDQ + cv * 8) = r < len ? kv[i] : zero;
  }
  // In-chunk cumulative decay (fp64) and write strengths; zero past the length.
  if (w == 3) {
    const double gv = lane < len ? (double)floor_keep_nan(graw, kFloor) : 0.0;
    const double gm = wave_inclusive_scan(gv, lane);
    sm.gam[lane] = gm;
    sm.eg[lane] = fexp((float)gm);
    sm.beta[lane] = lane < len ? braw : 0.f;
  }
  __syncthreads();
  // Gram tiles, 5 per wave, kept in registers: wave w takes the w + 1 tiles
  // (K Q^T)[16 ni.., 16 w..], ni <= w, whose accumulators hold P's rows of token
  // tile w (lane: row 16w + l%16, columns 16 ni + 4(l/16) + i), and 4 - w of the
  // 10 lower tiles of K K^T.
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
    const int r = 16 * w + lr;  // P row of this lane
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      if (m <= w) {
        // P[r][16m + 4lg + i] = rq_r rk_i e^{G_r - G_i} (q_r . k_i), i <= r; kept in acc[m]
        const int c0 = 16 * m + 4 * lg;
        const f32x4 rkc = *reinterpret_cast<const f32x4 *>(sm.rk + c0);
        const double gr = sm.gam[r];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[m][e] = c0 + e <= r ? sm.rq[r] * rkc[e] * fexp((float)(gr - sm.gam[c0 + e])) * acc[m][e] : 0.f;
      } else {
        // A[r][i] = beta_r rk_r rk_i e^{G_r - G_i} (k_r . k_i), i < r
        const int mi = kmi[m], ni = kni[m];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int rr = 16 * mi + 4 * lg + e, ci = 16 * ni + lr;
          A[rr * LDF + ci] = ci < rr ? sm.beta[rr] * sm.rk[rr] * sm.rk[ci] *
                                           fexp((float)(sm.gam[rr] - sm.gam[ci])) * acc[m][e]
                                     : 0.f;
        }
      }
    }
  }
  // Per-token factors of the carry: e^{G_last - G} (zero past the length), e^{G_last}.
  if (tid < C) {
    sm.bek[tid] = sm.beta[tid] * sm.eg[tid] * sm.rk[tid];
    float *F = fac + slot * kWyFac;
    const double gl = sm.gam[len - 1];
    F[tid] = tid < len ? fexp((float)(gl - sm.gam[tid])) : 0.f;
    if (tid == 0) F[C] = fexp((float)gl);
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
  // accumulator element Y[4(l/16) + s][l%16].  Blocks above the diagonal are
  // never written: every reader below masks them.
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

  // This lane's row of T (row 16w + l%16, token step st in the split order
  // {32 st + 4g + i, 32 st + 16 + 4g + i}; zero above the diagonal), kept in
  // registers across the barrier that retires T.
  const int rw = 16 * w + lr;
  f32x4 ta[2], tb[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    ta[st] = tb[st] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (st <= (w >> 1)) {
      const int i0 = 32 * st + 4 * lg;
      const f32x4 x0 = *reinterpret_cast<const f32x4 *>(Tm + rw * LDF + i0);
      const f32x4 x1 = *reinterpret_cast<const f32x4 *>(Tm + rw * LDF + i0 + 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ta[st][e] = i0 + e <= rw ? x0[e] : 0.f;
        tb[st][e] = i0 + 16 + e <= rw ? x1[e] : 0.f;
      }
    }
  }
  // R = P T for the rows of token tile w, as the tiles nt <= w of R^T = T^T P^T
  // (contraction over tokens in the split order).  The B operand P^T is this
  // lane's own P accumulators: P[16w + l%16][32 st + 4g + i] = acc[2st][i] and
  // [.. + 16] = acc[2st + 1][i].  racc[nt][i] = R[16w + l%16][16 nt + 4g + i].
  f32x4 racc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) racc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    if (2 * st <= w) {
      const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
      u32x4 ph, pl;
      split8(acc[2 * st], 2 * st + 1 <= w ? acc[2 * st + 1] : z4, ph, pl);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (nt <= w && nt <= 2 * st + 1) {
          const int nn = 16 * nt + lr;
          f32x4 xa, xb;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i0 = 32 * st + 4 * lg + e, i1 = i0 + 16;
            xa[e] = i0 >= nn ? Tm[i0 * LDF + nn] : 0.f;  // T is lower triangular
            xb[e] = i1 >= nn ? Tm[i1 * LDF + nn] : 0.f;
          }
          u32x4 th, tl;
          split8(xa, xb, th, tl);
          racc[nt] = mfma_bf16(as_bf(th), as_bf(ph), racc[nt]);
          racc[nt] = mfma_bf16(as_bf(th), as_bf(pl), racc[nt]);
          racc[nt] = mfma_bf16(as_bf(tl), as_bf(ph), racc[nt]);
        }
      }
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
  // This lane's query row for Q' (row 16w + l%16, d_k {32s + 4g + i, 32s + 16 + 4g + i}),
  // read again from global memory (the chunk's rows are in L2).
  u32x2 qa[4], qb[4];
  {
    const uint16_t *qrow = q + ((int64_t)(t0 + min(rw, len - 1)) * H_qk + j) * DK + 4 * lg;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qa[s] = *reinterpret_cast<const u32x2 *>(qrow + 32 * s);
      qb[s] = *reinterpret_cast<const u32x2 *>(qrow + 32 * s + 16);
    }
  }
  __syncthreads();

  // Row fragments (token tile w, token step st, split order), bf16 hi/lo, with
  // the column scalings of the four products below:
  //   diag(beta e^G k-norm): T' for W, R' for Q';   diag(beta): T'' for U', R'' for O'.
  auto frag = [&](const f32x4 &xa, const f32x4 &xb, int st, bool dk, u32x4 &hi, u32x4 &lo) {
    const float *sc = (dk ? sm.bek : sm.beta) + 32 * st + 4 * lg;
    split8(xa * *reinterpret_cast<const f32x4 *>(sc), xb * *reinterpret_cast<const f32x4 *>(sc + 16), hi, lo);
  };
  // W^T = K^T T'^T and (R' K)^T = K^T R'^T for token tile w, by d_k step s: the
  // tiles of d_k rows 32s.. and 32s+16.. give this lane row 16w + l%16 at d_k
  // {32s + 4g + i, 32s + 16 + 4g + i}, the chain's A-operand order.  Both are
  // stored as fp16; Q' = e^G q-norm scale Q - R' K.
  {
    u32x4 t1h[2], t1l[2], r1h[2], r1l[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (st <= (w >> 1)) {
        frag(ta[st], tb[st], st, true, t1h[st], t1l[st]);
        frag(racc[2 * st], racc[2 * st + 1], st, true, r1h[st], r1l[st]);
      }
    }
    u32x4 *W4 = reinterpret_cast<u32x4 *>(wf + slot * kWyWBytes) + w * 4 * 64 + lane;
    u32x4 *Q4 = reinterpret_cast<u32x4 *>(qf + slot * kWyQBytes) + w * 4 * 64 + lane;
    const float fq = sm.eg[rw] * sm.rq[rw];
    const bool live = rw < len;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, x0 = acc0, x1 = acc0;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st <= (w >> 1)) {  // T' and R' are lower triangular
          const bf16x8 a0 = ld8s(kt + (32 * s + lr) * LDT + 32 * st + 4 * lg);
          const bf16x8 a1 = ld8s(kt + (32 * s + 16 + lr) * LDT + 32 * st + 4 * lg);
          acc0 = mfma_bf16(a0, as_bf(t1h[st]), acc0);
          acc0 = mfma_bf16(a0, as_bf(t1l[st]), acc0);
          acc1 = mfma_bf16(a1, as_bf(t1h[st]), acc1);
          acc1 = mfma_bf16(a1, as_bf(t1l[st]), acc1);
          x0 = mfma_bf16(a0, as_bf(r1h[st]), x0);
          x0 = mfma_bf16(a0, as_bf(r1l[st]), x0);
          x1 = mfma_bf16(a1, as_bf(r1h[st]), x1);
          x1 = mfma_bf16(a1, as_bf(r1l[st]), x1);
        }
      }
      W4[s * 64] = h16x8(acc0, acc1);
      f32x4 y0, y1;
      y0[0] = bf_lo(qa[s][0]); y0[1] = bf_hi(qa[s][0]); y0[2] = bf_lo(qa[s][1]); y0[3] = bf_hi(qa[s][1]);
      y1[0] = bf_lo(qb[s][0]); y1[1] = bf_hi(qb[s][0]); y1[2] = bf_lo(qb[s][1]); y1[3] = bf_hi(qb[s][1]);
      const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
      Q4[s * 64] = h16x8(live ? y0 * fq - x0 : z4, live ? y1 * fq - x1 : z4);
    }
  }
  // U' = T'' V and O' = R'' V for token tile w, by value column tile ct, in
  // accumulator order (fp32).
  {
    u32x4 t2h[2], t2l[2], r2h[2], r2l[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      if (st <= (w >> 1)) {
        frag(ta[st], tb[st], st, false, t2h[st], t2l[st]);
        frag(racc[2 * st], racc[2 * st + 1], st, false, r2h[st], r2l[st]);
      }
    }
    const int NCT = d_v / 16;
    f32x4 *U4 = reinterpret_cast<f32x4 *>(uf + slot * (int64_t)(C * d_v)) + w * NCT * 64 + lane;
    f32x4 *O4 = reinterpret_cast<f32x4 *>(of + slot * (int64_t)(C * d_v)) + w * NCT * 64 + lane;
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = a;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        if (st <= (w >> 1)) {
          const bf16x8 bs = ld8s(vt + (16 * ct + lr) * LDT + 32 * st + 4 * lg);
          a = mfma_bf16(as_bf(t2h[st]), bs, a);
          a = mfma_bf16(as_bf(t2l[st]), bs, a);
          b = mfma_bf16(as_bf(r2h[st]), bs, b);
          b = mfma_bf16(as_bf(r2l[st]), bs, b);
        }
      }
      U4[ct * 64] = a;
      O4[ct * 64] = b;
    }
  }
  // K^^T fragments (fp16, normalised keys), once per (chunk, query/key head):
  // item (d_k tile mt, token step st, lane) = K^^T[16 mt + l%16][{32 st + 4g + i,
  // 32 st + 16 + 4g + i}].
  if (h % R == 0) {
    u32x4 *K4 = reinterpret_cast<u32x4 *>(ktf + ((int64_t)j * MC + c) * kWyKtBytes);
    for (int it = tid; it < 16 * 64; it += 256) {
      const int ln = it & 63, ms = it >> 6, mt = ms >> 1, st = ms & 1;
      const int t = 32 * st + 4 * (ln >> 4);
      const uint32_t *r32 = reinterpret_cast<const uint32_t *>(kt + (16 * mt + (ln & 15)) * LDT + t);
      f32x4 a = {bf_lo(r32[0]), bf_hi(r32[0]), bf_lo(r32[1]), bf_hi(r32[1])};
      f32x4 b = {bf_lo(r32[8]), bf_hi(r32[8]), bf_lo(r32[9]), bf_hi(r32[9])};
      if (l2norm) {
        a *= *reinterpret_cast<const f32x4 *>(sm.rk + t);
        b *= *reinterpret_cast<const f32x4 *>(sm.rk + t + 16);
      }
      K4[it] = h16x8(a, b);
    }
  }
}

// ---------------------------------------------------------------------------
// chain: one (sequence, value head, block of 16 NB columns of S) per block of
// 8 waves.  Waves 0-3 carry the state: wave w keeps rows [32w, 32w + 32) of
// the S block in registers and forms the write vectors U of token tile [16w,
// 16w + 16).  Waves 4-7 produce the output: wave 4 + w computes O for token
// tile w from the published S.  Per chunk c:
//
//   state waves                          output waves
//   publish S (fp16) -> sx
//   ---------------------------- barrier 1 ----------------------------
//   U = U' - W S, U'' -> u2x (hi/lo)     O = Q' S + O' (from sx), store O
//   ---------------------------- barrier 2 ----------------------------
//   S <- e^{G_last} S + K^^T U''
//
// Every wave is done with sx and u2x of chunk c once it has passed the barrier
// after its last read, so one buffer of each suffices.  Every operand that does
// not depend on S is loaded from the workspace straight into registers ahead of
// its use (the state waves' one chunk ahead, each group right after its last
// use, interleaved with the MFMAs of its phase).
//
// NB = 1 gives the most blocks (the latency of one long sequence is spread over
// every CU); NB = 2 and 4 cut the operand loads per column of S by 2 and 4, for
// launches that fill the GPU with blocks either way (many sequences, or many
// heads).
// ---------------------------------------------------------------------------
template <int NB> struct StateOps {
  u32x4 w[4];      // W (fp16) of token tile w, d_k steps 0..3
  u32x4 kt[2][2];  // K^^T (fp16) of this wave's two d_k tiles, token steps 0..1
  f32x4 u[NB];     // U' tiles
  f32x4 fu;        // e^{G_last - G} of this lane's 4 rows
  float el;        // e^{G_last}
};
template <int NB> struct OutOps {
  u32x4 q[4];      // Q' (fp16) of token tile w, d_k steps 0..3
  f32x4 o[NB];     // O' tiles
  uint32_t pf[2];  // words of the L2 warm-up loads, consumed a chunk later
};

template <bool STATES, bool OBF16, int NB, bool WARM>
__global__ __launch_bounds__(512) void wy_chain_kernel(
    const float *__restrict__ s0, const Seqs sq, const unsigned char *__restrict__ wf,
    const unsigned char *__restrict__ qf, const float *__restrict__ uf, const float *__restrict__ of,
    const float *__restrict__ fac, const unsigned char *__restrict__ ktf, void *__restrict__ o,
    float *__restrict__ fin, float *__restrict__ uw, float *__restrict__ scw, int H_qk, int H_v, int d_v,
    int MC, int groups) {
  // S as published by its owner wave (the B operand of d_k step w), one
  // 16-column tile nb after the other.  u2x: the two token tiles of token step
  // st side by side, so a reader takes its 8 contraction indices with one
  // 16-byte load.
  __shared__ u32x4 sx[4][NB][64];
  __shared__ u32x4 u2x[NB][2][2][64];
  constexpr int LDO = 20;  // O tile rows, fp32 (the pad spreads rows over the banks)
  __shared__ float ot[4][16 * LDO];
  if (sq.bad()) return;
  const int NCT = d_v / 16;         // 16-column tiles of S
  const int NCB = NCT / NB;         // column blocks
  // groups: (sequence, query/key head), whose value heads share K^T too
  const int u = xcd_group_remap(blockIdx.x, NCB * (H_v / H_qk), groups);
  if (u < 0) return;
  const int jb = u % NCB, h = (u / NCB) % H_v, n = u / (NCB * H_v);
  const int j = h / (H_v / H_qk);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = wave & 3;
  const int lr = lane & 15, lg = lane >> 4;
  const int col0 = jb * 16 * NB;
  const int64_t sbase = (int64_t)(n * H_v + h) * DK;
  const int c_begin = sq.first(n), c_end = sq.first(n + 1);
  const int s_begin = sq.start(n), s_end = sq.start(n + 1);
  const int64_t hslot = (int64_t)h * MC, jslot = (int64_t)j * MC;
  constexpr int kMFMA = 0x008, kVMR = 0x020, kDSR = 0x100;  // scheduling-group classes

  if (wave < 4) {
    // ------------------------------ state waves ------------------------------
    // S[nb][mt] holds rows 32w + 16mt + 4lg + i, column col0 + 16nb + lr.
    f32x4 S[NB][2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        S[nb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (s0) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S[nb][mt][i] = s0[(sbase + 32 * w + 16 * mt + 4 * lg + i) * d_v + col0 + 16 * nb + lr];
        }
      }
    // Drain the initial-state loads, so that inside the chunk loop the
    // vector-memory counter covers only the operand prefetches.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

    auto wp = [&](int c) {
      return reinterpret_cast<const u32x4 *>(wf + (hslot + c) * kWyWBytes) + w * 4 * 64 + lane;
    };
    auto kp = [&](int c) {
      return reinterpret_cast<const u32x4 *>(ktf + (jslot + c) * kWyKtBytes) + 2 * w * 2 * 64 + lane;
    };
    auto load_uf = [&](StateOps<NB> &op, int c) {
      const f32x4 *U4 = reinterpret_cast<const f32x4 *>(uf + (hslot + c) * (int64_t)(C * d_v));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) op.u[nb] = U4[(w * NCT + jb * NB + nb) * 64 + lane];
      const float *F = fac + (hslot + c) * kWyFac;
      op.fu = *reinterpret_cast<const f32x4 *>(F + 16 * w + 4 * lg);
      op.el = F[C];
    };

    auto chunk = [&](StateOps<NB> &op, int c, int cn) {
      const int t0 = s_begin + (c - c_begin) * C;
      const int len = min(C, s_end - t0);
      // 1. publish this wave's S rows (the B operand of d_k step w)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        sx[w][nb][lane] = h16x8(S[nb][0], S[nb][1]);
        if constexpr (STATES) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              scw[(((int64_t)c * H_v + h) * DK + 32 * w + 16 * mt + 4 * lg + i) * d_v + col0 + 16 * nb + lr] =
                  S[nb][mt][i];
        }
      }
      __syncthreads();  // 1
      // 2. U = U' - W S for token tile w (two accumulators: even and odd d_k steps)
      const u32x4 *W4 = wp(cn);
      f32x4 a0[NB], a1[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) a0[nb] = a1[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const u32x4 sv = sx[s][nb][lane];
          if (s & 1) a1[nb] = mfma_f16(op.w[s], sv, a1[nb]);
          else a0[nb] = mfma_f16(op.w[s], sv, a0[nb]);
        }
        op.w[s] = W4[s * 64];
        __builtin_amdgcn_sched_group_barrier(kDSR, NB, 0);
        __builtin_amdgcn_sched_group_barrier(kMFMA, NB, 0);
        __builtin_amdgcn_sched_group_barrier(kVMR, 1, 0);
      }
      //    U'' = diag(e^{G_last - G}) U; publish U'' (fp16 hi/lo)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const f32x4 uv = op.u[nb] - (a0[nb] + a1[nb]);
        const f32x4 u2 = uv * op.fu;
        u32x2 hi, lo;
        split4h(u2, hi, lo);
        reinterpret_cast<u32x2 *>(&u2x[nb][w >> 1][0][lane])[w & 1] = hi;
        reinterpret_cast<u32x2 *>(&u2x[nb][w >> 1][1][lane])[w & 1] = lo;
        if constexpr (STATES) {
          // the write vectors of rows t0 .. t0 + len
          const auto rs = rows_rsrc(uw + (int64_t)t0 * H_v * d_v, (int64_t)len * H_v * d_v * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = uv[i];  // (a bit cast of the vector element itself would read element 0)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs,
                                                  (((16 * w + 4 * lg + i) * H_v + h) * d_v + col0 + 16 * nb + lr) * 4,
                                                  0, 0);
          }
        }
      }
      const float el = op.el;
      load_uf(op, cn);
      __syncthreads();  // 2
      // 3. S <- e^{G_last} S + K^^T U'' for this wave's rows
      u32x4 bh[NB][2], bl[NB][2];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          bh[nb][st] = u2x[nb][st][0][lane];
          bl[nb][st] = u2x[nb][st][1][lane];
        }
      const u32x4 *K4 = kp(cn);
      f32x4 ah[NB][2], al[NB][2];  // K^^T U''_hi and K^^T U''_lo: independent chains
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) ah[nb][mt] = al[nb][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 2; ++st) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            ah[nb][mt] = mfma_f16(op.kt[mt][st], bh[nb][st], ah[nb][mt]);
            al[nb][mt] = mfma_f16(op.kt[mt][st], bl[nb][st], al[nb][mt]);
          }
          op.kt[mt][st] = K4[(mt * 2 + st) * 64];
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) S[nb][mt] = S[nb][mt] * el + (ah[nb][mt] + al[nb][mt]);
      __builtin_amdgcn_sched_group_barrier(kDSR, 4 * NB, 0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        __builtin_amdgcn_sched_group_barrier(kMFMA, 2 * NB, 0);
        __builtin_amdgcn_sched_group_barrier(kVMR, 1, 0);
      }
    };

    if (c_begin < c_end) {
      StateOps<NB> op;
      {
        const u32x4 *W4 = wp(c_begin), *K4 = kp(c_begin);
#pragma unroll
        for (int s = 0; s < 4; ++s) op.w[s] = W4[s * 64];
        load_uf(op, c_begin);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int st = 0; st < 2; ++st) op.kt[mt][st] = K4[(mt * 2 + st) * 64];
      }
      // The first chunk is peeled, so that the loop is entered with the same
      // loads in flight as on its back edge (the compiler's wait counts are then
      // exact).  Past the last chunk the loads repeat it and go unused.
      chunk(op, c_begin, min(c_begin + 1, c_end - 1));
      for (int c = c_begin + 1; c < c_end; ++c) chunk(op, c, min(c + 1, c_end - 1));
    }
    if (fin) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            fin[(sbase + 32 * w + 16 * mt + 4 * lg + i) * d_v + col0 + 16 * nb + lr] = S[nb][mt][i];
    }
  } else {
    // ------------------------------ output waves -----------------------------
    // O for chunk c is formed between the chunk's two barriers, while the state
    // waves form U (the output needs S alone).  It is stored through a small LDS
    // transpose, so that each lane writes 4 consecutive columns of one row with
    // one 16-byte store (a quarter of the store instructions of the accumulator
    // layout's 4-byte ones; the vector-memory path is shared by all 8 waves).
    // The next chunk's operands are loaded right after the MFMAs that consume
    // this chunk's, and the stores carry no branch (see rows_rsrc), so the wait
    // for them covers those loads alone.
    auto qp = [&](int c) {
      return reinterpret_cast<const u32x4 *>(qf + (hslot + c) * kWyQBytes) + w * 4 * 64 + lane;
    };
    auto load_out = [&](OutOps<NB> &op, int c) {
      const u32x4 *Q4 = qp(c);
#pragma unroll
      for (int s = 0; s < 4; ++s) op.q[s] = Q4[s * 64];
      const f32x4 *O4 = reinterpret_cast<const f32x4 *>(of + (hslot + c) * (int64_t)(C * d_v));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) op.o[nb] = O4[(w * NCT + jb * NB + nb) * 64 + lane];
    };

    // L2 warm-up (WARM: 16-column chains that fill every CU): every chunk the output
    // waves load one word of each 128-byte line this chain reads two chunks later
    // (its 1/NCB share of the W, Q' and K^T lines all column blocks of its head
    // read, its own U' and O' lines, the decay factors), so that those lines are
    // in the XCD's L2 when the operand loads come.  The loaded words are consumed
    // one chunk later, so no wait is added.
    constexpr int kWarmAhead = 2;
    const int ol = (wave - 4) * 64 + lane;
    const int nS = 3 * 128 / NCB, nU = 32 * NB, nL = nS + 2 * nU + 4;
    const int last_c = c_end - 1;
    auto pf_ptr = [&](int cp, int L) -> const uint32_t * {
      L = min(L, nL - 1);
      const int ls = jb + NCB * min(L, nS - 1), reg = ls >> 7;
      const unsigned char *ps = (reg == 0 ? wf + (hslot + cp) * kWyWBytes
                                 : reg == 1 ? qf + (hslot + cp) * kWyQBytes
                                            : ktf + (jslot + cp) * kWyKtBytes) + (ls & 127) * 128;
      const int lu = min(max(L - nS, 0), 2 * nU - 1), x = lu % nU;
      const float *ub = (lu < nU ? uf : of) + (hslot + cp) * (int64_t)(C * d_v);
      const unsigned char *pu = reinterpret_cast<const unsigned char *>(ub) +
                                (int64_t)((x / (8 * NB)) * NCT + jb * NB) * 1024 + (x % (8 * NB)) * 128;
      const unsigned char *pfac = reinterpret_cast<const unsigned char *>(fac + (hslot + cp) * kWyFac) +
                                  min(max(L - nS - 2 * nU, 0) * 128, 316);
      return reinterpret_cast<const uint32_t *>(L < nS ? ps : L < nS + 2 * nU ? pu : pfac);
    };
    auto chunk = [&](OutOps<NB> &op, int c, int cn) {
      const int t0 = s_begin + (c - c_begin) * C;
      const int len = min(C, s_end - t0);
      __syncthreads();  // 1
      // O = Q' S + O' for token tile w, from the S published for this chunk
      f32x4 ao[NB], ao2[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        ao[nb] = op.o[nb];
        ao2[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const u32x4 sv = sx[s][nb][lane];
          if (s & 1) ao2[nb] = mfma_f16(op.q[s], sv, ao2[nb]);
          else ao[nb] = mfma_f16(op.q[s], sv, ao[nb]);
        }
      load_out(op, cn);
      if constexpr (WARM) {
        asm volatile("" ::"v"(op.pf[0]), "v"(op.pf[1]));
        const int cp = min(c + kWarmAhead, last_c);
        op.pf[0] = *pf_ptr(cp, ol);
        op.pf[1] = *pf_ptr(cp, ol + 256);
      }
      {
        // rows t0 .. t0 + len of o (no row without o)
        const int esz = OBF16 ? 2 : 4;
        const auto rs = rows_rsrc(o ? static_cast<unsigned char *>(o) + (int64_t)t0 * H_v * d_v * esz : nullptr,
                                  o ? (int64_t)len * H_v * d_v * esz : 0);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const f32x4 x = ao[nb] + ao2[nb];
#pragma unroll
          for (int i = 0; i < 4; ++i) ot[w][(4 * lg + i) * LDO + lr] = x[i];
          __builtin_amdgcn_wave_barrier();
          const f32x4 y = *reinterpret_cast<const f32x4 *>(&ot[w][lr * LDO + 4 * lg]);
          __builtin_amdgcn_wave_barrier();
          // lane l: row 16w + l%16, columns col0 + 16nb + 4(l/16) ..
          const int off = (((16 * w + lr) * H_v + h) * d_v + col0 + 16 * nb + 4 * lg) * esz;
          if constexpr (OBF16)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{pk_bf16(y[0], y[1]), pk_bf16(y[2], y[3])}, rs, off, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y), rs, off, 0, 0);
        }
      }
      __syncthreads();  // 2
    };

    if (c_begin < c_end) {
      OutOps<NB> op;
      load_out(op, c_begin);
      if constexpr (WARM) {
        op.pf[0] = *pf_ptr(min(c_begin + kWarmAhead, last_c), ol);
        op.pf[1] = *pf_ptr(min(c_begin + kWarmAhead, last_c), ol + 256);
      }
      // First chunk peeled, as on the state waves; past the last chunk the
      // loads repeat it and go unused.
      chunk(op, c_begin, min(c_begin + 1, c_end - 1));
      for (int c = c_begin + 1; c < c_end; ++c) chunk(op, c, min(c + 1, c_end - 1));
    }
  }
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

template <bool STATES, bool OBF16, int NB>
hipError_t launch_chain(const Problem &p, const ChunkArgs &a, const Seqs &sq, hipStream_t st) {
  const Workspace &w = a.ws;
  const int groups = p.N * p.H_qk, ncb = p.d_v / (16 * NB);
  if (groups == 0 || ncb == 0) return hipSuccess;
  const int grid = xcd_group_grid(ncb * (p.H_v / p.H_qk), groups);
  // The L2 warm-up pays where 16-column chains occupy every CU; with fewer
  // chains than CUs (or wider blocks) it costs more than it saves.
  const bool warm = NB == 1 && (int64_t)p.N * p.H_v * ncb >= device_cus();
  if (warm)
    hipLaunchKernelGGL((wy_chain_kernel<STATES, OBF16, NB, NB == 1>), dim3(grid), dim3(512), 0, st, a.s0, sq, w.wf,
                       w.qf, w.uf, w.of, w.fac, w.ktf, a.o, a.final_state, w.u, w.sc, p.H_qk, p.H_v, p.d_v,
                       p.max_chunks, groups);
  else
    hipLaunchKernelGGL((wy_chain_kernel<STATES, OBF16, NB, false>), dim3(grid), dim3(512), 0, st, a.s0, sq, w.wf,
                       w.qf, w.uf, w.of, w.fac, w.ktf, a.o, a.final_state, w.u, w.sc, p.H_qk, p.H_v, p.d_v,
                       p.max_chunks, groups);
  return hipGetLastError();
}

template <bool STATES, bool OBF16>
hipError_t run_wy(const Problem &p, const ChunkArgs &a, hipStream_t st) {
  const Workspace &w = a.ws;
  mark_event(a, 0, st);
  hipError_t e;
  const bool dense = dense_rows(p);
  if (!dense && (e = launch_plan(p, a, st)) != hipSuccess) return e;
  mark_event(a, 1, st);
  const Seqs sq{w.status, w.seq_start, w.chunk_first, p.N, dense ? p.T : 0, dense ? ceil_div(p.T, C) : 0};
  const uint16_t *q = static_cast<const uint16_t *>(a.q), *k = static_cast<const uint16_t *>(a.k),
                 *v = static_cast<const uint16_t *>(a.v);
  if (p.max_chunks > 0 && p.H_v > 0) {
    hipLaunchKernelGGL(wy_prep_kernel, dim3(p.max_chunks * p.H_v), dim3(256), 0, st, q, k, v, a.g, a.beta,
                       sq, w.wf, w.qf, w.uf, w.of, w.fac, w.ktf, p.H_qk, p.H_v, p.d_v, p.max_chunks, p.scale,
                       p.l2norm ? 1 : 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  mark_event(a, 2, st);
  // Column blocks of 16, 32 or 64 columns: the width doubles while the narrower
  // blocks would outnumber the CUs (wider blocks load each chunk's W, K^T and Q'
  // once for more columns; narrower ones spread a few long chains over more
  // CUs, but two of them sharing a CU each run slower than one wider block).
  const int64_t chains16 = (int64_t)p.N * p.H_v * (p.d_v / 16), cus = (int64_t)device_cus();
  const int nb = chains16 > cus ? (p.d_v % 64 == 0 && chains16 / 2 > cus ? 4 : 2) : 1;
  e = nb == 4 ? launch_chain<STATES, OBF16, 4>(p, a, sq, st)
      : nb == 2 ? launch_chain<STATES, OBF16, 2>(p, a, sq, st)
                : launch_chain<STATES, OBF16, 1>(p, a, sq, st);
  if (e != hipSuccess) return e;
  mark_event(a, 3, st);
  if constexpr (STATES) {
    if ((e = launch_states_stream(p, a, sq, st)) != hipSuccess) return e;
    mark_event(a, 4, st);
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_wy_path(const Problem &p, const ChunkArgs &a, bool states, hipStream_t st) {
  if (p.d_k != DK || p.C != C || p.d_v % 32 != 0 || p.d_v > 128) return hipErrorInvalidValue;
  const bool ob = p.o_dtype == GDN_BF16;
  if (states) return ob ? run_wy<true, true>(p, a, st) : run_wy<true, false>(p, a, st);
  return ob ? run_wy<false, true>(p, a, st) : run_wy<false, false>(p, a, st);
}

}  // namespace gdn
