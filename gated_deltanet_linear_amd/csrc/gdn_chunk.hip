// The chunked paths of libgdn: the pieces every input type shares (the plan
// kernel, the per-token states stream, the launchers and the workspace
// layout) and the general path (fp32 inputs at every supported size, bf16 at
// chunk 32); bf16 inputs at chunk 64 take the fused path of gdn_fused.hip.
//
// What is computed is the gated delta rule of the pages (Qwen3.5 text
// encyclopedia page, note "The DeltaNet mixer"; value table of
// model.layers[i].linear_attn) over chunks of C tokens.  Per value head, with
// the in-chunk cumulative log decay G_r = g_0 + ... + g_r and S the state at
// the chunk start, the token recurrence unrolls to (UT / WY form):
//
//   A[r,i] = beta_r e^{G_r - G_i} (k_r . k_i), i < r    strictly lower
//   T      = (I + A)^{-1}                                unit lower
//   U      = T diag(beta) (V - diag(e^G) K S)            the tokens' write vectors
//   O      = diag(e^G) Q S + P U,  P[r,i] = e^{G_r-G_i} (q_r . k_i), i <= r
//   S     <- e^{G_last} S + K^T diag(e^{G_last - G}) U
//
// fp32 launch sequence on the caller's stream:
//   plan   (1 workgroup)  sequence starts and chunk numbering from cu_seqlens
//   prep   (chunk, qk head)  K K^T and Q K^T on MFMA, the fp32 triangular solve,
//                           T diag(beta), P and the decay vectors -> workspace.
//                           Both value heads of a query/key head share K K^T, Q K^T.
//   carry  (sequence, value head, column block of S)  walks the chunks of one
//                           sequence in order with its S block in registers:
//                           [Q;K] S, T diag(beta) X, P U and K^T U on fp32 MFMA.
//                           The delta rule acts on each column of S on its own,
//                           so column blocks are independent chains.
//   stream (states path only)  S after every token from the chunk-start
//                           state and the write vectors: S <- e^g S + k u^T,
//                           branch-free 16-byte buffer stores.
//
// Decays are summed in fp64 and every factor e^{G_r - G_i} is formed from a
// difference with r >= i, so it never overflows; g is clamped to -1e4, which
// keeps -inf (a reset) finite and still gives exp() == 0 for every factor that
// spans it.
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn.h"

namespace gdn {

constexpr float kGFloor = -1.0e4f;

// ---------------------------------------------------------------------------
// plan: sequence starts, the first global chunk of every sequence, and the
// sequences ordered by length.
// ---------------------------------------------------------------------------
__global__ void plan_kernel(const int32_t *__restrict__ cu, int N, int T, int T_tot, int C,
                            int max_chunks, int32_t *__restrict__ status,
                            int32_t *__restrict__ seq_start, int32_t *__restrict__ chunk_first,
                            int32_t *__restrict__ order) {
  __shared__ int bad_s;
  if (threadIdx.x == 0) {
    int bad = 0, acc = 0, prev = 0;
    for (int n = 0; n <= N; ++n) {
      const int s = cu ? cu[n] : n * T;
      if ((n == 0 && s != 0) || s < prev || s > T_tot) bad = 1;
      seq_start[n] = s;
      chunk_first[n] = acc;
      if (n < N) {
        const int e = cu ? cu[n + 1] : (n + 1) * T;
        if (e >= s) acc += (e - s + C - 1) / C;
      }
      prev = s;
    }
    if (N >= 0 && (cu ? cu[N] : N * T) != T_tot) bad = 1;
    if (acc > max_chunks) bad = 1;
    *status = bad;
    bad_s = bad;
  }
  __syncthreads();
  // The sequences by decreasing chunk count (ties by index), so that the longest
  // chains start first; past kOrderMaxSeqs sequences, their own order.
  if (!order || bad_s) return;
  for (int n = threadIdx.x; n < N; n += blockDim.x) {
    int rank = n;
    if (N <= kOrderMaxSeqs) {
      const int ln = chunk_first[n + 1] - chunk_first[n];
      rank = 0;
      for (int m = 0; m < N; ++m) {
        const int lm = chunk_first[m + 1] - chunk_first[m];
        rank += lm > ln || (lm == ln && m < n);
      }
    }
    order[rank] = n;
  }
}

// Operand storage of a policy: bf16 path -> uint16_t (computed values as hi/lo
// pairs), fp32 path -> float (single arrays, exact fp32 MFMA).
// ---------------------------------------------------------------------------
// Operand policies.  bf16 path: inputs are bf16 (uint16_t storage) and every
// computed operand is a bf16 hi/lo pair; fp32 path: fp32 everywhere, exact
// fp32 MFMA.  Fr<BF> loads one MFMA operand fragment from LDS:
//   row(): lane l takes row l%16 of a [M][ld] array whose contraction index is
//          contiguous, contraction slice k0 + 8(l/16) .. (+4(l/16) for fp32);
//   col(): lane l takes column l%16 of a [K][ld] array (contraction = row
//          index), the same contraction slice, gathered element by element.
// A and B fragments of one MFMA use the same slice assignment, so they agree
// on which contraction index each lane group feeds.
// ---------------------------------------------------------------------------
template <typename TIn> struct Pol {
  static constexpr bool BF = std::is_same<TIn, uint16_t>::value;
  using CT = typename std::conditional<BF, uint16_t, float>::type;
  static constexpr int PAD = BF ? 8 : 4;  // row padding in elements (16 bytes)
  static constexpr int VEC = 16 / sizeof(TIn);
};

template <bool BF> struct Fr;
template <> struct Fr<true> {
  using T = bf16x8;
  static constexpr int KS = 32;
  static __device__ __forceinline__ T row(const uint16_t *base, int ld, int lane, int k0) {
    return *reinterpret_cast<const bf16x8 *>(base + (lane & 15) * ld + k0 + 8 * (lane >> 4));
  }
  static __device__ __forceinline__ T col(const uint16_t *base, int ld, int lane, int k0) {
    const uint16_t *p = base + (k0 + 8 * (lane >> 4)) * ld + (lane & 15);
    uint4 u;
    u.x = (uint32_t)p[0] | ((uint32_t)p[ld] << 16);
    u.y = (uint32_t)p[2 * ld] | ((uint32_t)p[3 * ld] << 16);
    u.z = (uint32_t)p[4 * ld] | ((uint32_t)p[5 * ld] << 16);
    u.w = (uint32_t)p[6 * ld] | ((uint32_t)p[7 * ld] << 16);
    return __builtin_bit_cast(bf16x8, u);
  }
  static __device__ __forceinline__ f32x4 mma(const f32x4 &acc, const T &a, const T &b) {
    return mfma_bf16(a, b, acc);
  }
};
template <> struct Fr<false> {
  using T = f32x4;
  static constexpr int KS = 16;
  static __device__ __forceinline__ T row(const float *base, int ld, int lane, int k0) {
    return *reinterpret_cast<const f32x4 *>(base + (lane & 15) * ld + k0 + 4 * (lane >> 4));
  }
  static __device__ __forceinline__ T col(const float *base, int ld, int lane, int k0) {
    const float *p = base + (k0 + 4 * (lane >> 4)) * ld + (lane & 15);
    return f32x4{p[0], p[ld], p[2 * ld], p[3 * ld]};
  }
  static __device__ __forceinline__ f32x4 mma(f32x4 acc, const T &a, const T &b) {
    acc = mfma_f32(a[0], b[0], acc);
    acc = mfma_f32(a[1], b[1], acc);
    acc = mfma_f32(a[2], b[2], acc);
    return mfma_f32(a[3], b[3], acc);
  }
};

// Stores 4 fp32 values as 4 consecutive elements: split into hi at ph and lo
// at pl (bf16 path) or as they are at ph (fp32 path).
template <bool BF, typename CT>
__device__ __forceinline__ void put4(CT *ph, CT *pl, const f32x4 &v) {
  if constexpr (BF) {
    uint16_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split_bf16(v[i], h[i], l[i]);
    uint2 H, L;
    H.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    H.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
    L.x = (uint32_t)l[0] | ((uint32_t)l[1] << 16);
    L.y = (uint32_t)l[2] | ((uint32_t)l[3] << 16);
    *reinterpret_cast<uint2 *>(ph) = H;
    *reinterpret_cast<uint2 *>(pl) = L;
  } else {
    (void)pl;
    *reinterpret_cast<f32x4 *>(ph) = v;
  }
}

// The per-chunk triangular factors in the workspace: for each (chunk, value
// head) slot, 4*C*C bytes.  bf16 path: a hi plane then a lo plane of C x C
// bf16 (row-major); fp32 path: one C x C fp32 plane.
template <typename CT, int C>
__device__ __forceinline__ CT *plane(unsigned char *base, int64_t slot) {
  return reinterpret_cast<CT *>(base + slot * (int64_t)(4 * C * C));
}

// ---------------------------------------------------------------------------
// prep: per (chunk, query/key head): K K^T and Q K^T once, then for each value
// head of the group the decays, A, T = (I + A)^{-1}, T diag(beta) and P.
// ---------------------------------------------------------------------------
template <typename TIn, int DK, int C> struct PrepSmem {
  static constexpr int LDQ = DK + Pol<TIn>::PAD;
  static constexpr int LDC = C + 4;
  static constexpr int QKB = 2 * C * LDQ * (int)sizeof(TIn);
  static constexpr int TRB = 2 * C * LDC * (int)sizeof(float);
  static constexpr int UB = QKB > TRB ? QKB : TRB;
  alignas(16) unsigned char u[UB];  // q, k while loading; A, T once K K^T and Q K^T exist
  alignas(16) float G[C * LDC];     // K K^T (lower tiles)
  alignas(16) float QK[C * LDC];    // Q K^T (lower tiles)
  alignas(16) double gam[C];
  float beta[C], rq[C], rk[C];
  __device__ TIn *q() { return reinterpret_cast<TIn *>(u); }
  __device__ TIn *k() { return q() + C * LDQ; }
  __device__ float *A() { return reinterpret_cast<float *>(u); }
  __device__ float *T() { return A() + C * LDC; }
};

template <typename TIn, int DK, int C>
__global__ __launch_bounds__(256) void prep_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const float *__restrict__ g,
    const float *__restrict__ beta, const int32_t *__restrict__ status,
    const int32_t *__restrict__ seq_start, const int32_t *__restrict__ chunk_first,
    unsigned char *__restrict__ tbw, unsigned char *__restrict__ pmw, float *__restrict__ eg,
    float *__restrict__ eb, int N, int H_qk, int H_v, float scale, int l2norm) {
  using P = Pol<TIn>;
  using F = Fr<P::BF>;
  using CT = typename P::CT;
  using S = PrepSmem<TIn, DK, C>;
  constexpr int LDQ = S::LDQ, LDC = S::LDC, VEC = P::VEC, VPR = DK / VEC, NB = C / 16;
  static_assert(C % 16 == 0 && C <= 64 && DK % F::KS == 0, "prep tiling");
  __shared__ S sm;

  if (*status) return;
  const int c = blockIdx.x;
  if (c >= chunk_first[N]) return;
  const int n = find_seq(chunk_first, N, c);
  const int t0 = seq_start[n] + (c - chunk_first[n]) * C;
  const int len = min(C, seq_start[n + 1] - t0);
  const int j = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  TIn *sq = sm.q(), *sk = sm.k();

  // q, k rows of this chunk (zero beyond len).
  for (int x = tid; x < C * VPR; x += 256) {
    const int r = x / VPR, cv = x % VPR;
    uint4 qv = {0u, 0u, 0u, 0u}, kv = {0u, 0u, 0u, 0u};
    if (r < len) {
      const int64_t off = ((int64_t)(t0 + r) * H_qk + j) * DK + cv * VEC;
      qv = *reinterpret_cast<const uint4 *>(q + off);
      kv = *reinterpret_cast<const uint4 *>(k + off);
    }
    *reinterpret_cast<uint4 *>(sq + r * LDQ + cv * VEC) = qv;
    *reinterpret_cast<uint4 *>(sk + r * LDQ + cv * VEC) = kv;
  }
  __syncthreads();
  if (tid < 2 * C) {
    const int r = tid % C;
    float rn = 1.f;
    if (l2norm) {
      const TIn *row = (tid < C ? sq : sk) + r * LDQ;
      float ss = 0.f;
      for (int i = 0; i < DK; ++i) {
        const float a = Elem<TIn>::get(row, i);
        ss += a * a;
      }
      rn = 1.0f / sqrtf(ss + 1e-6f);
    }
    if (tid < C) sm.rq[r] = rn * scale;
    else sm.rk[r] = rn;
  }
  // K K^T and Q K^T: the lower 16x16 tiles (diagonal included) on MFMA.
  constexpr int NTRI = NB * (NB + 1) / 2;
  for (int t = wave; t < 2 * NTRI; t += 4) {
    const bool isq = t >= NTRI;
    const int tt = isq ? t - NTRI : t;
    int mi = 0;
    while ((mi + 1) * (mi + 2) / 2 <= tt) ++mi;
    const int ni = tt - mi * (mi + 1) / 2;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const TIn *Ab = (isq ? sq : sk) + mi * 16 * LDQ;
    const TIn *Bb = sk + ni * 16 * LDQ;
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += F::KS) acc = F::mma(acc, F::row(Ab, LDQ, lane, k0), F::row(Bb, LDQ, lane, k0));
    float *D = isq ? sm.QK : sm.G;
#pragma unroll
    for (int i = 0; i < 4; ++i) D[(mi * 16 + 4 * lg + i) * LDC + ni * 16 + lr] = acc[i];
  }
  __syncthreads();  // q and k are dead from here; their space holds A and T

  float *A = sm.A(), *Tm = sm.T();
  const int R = H_v / H_qk;
  for (int rr = 0; rr < R; ++rr) {
    const int h = j * R + rr;
    const int64_t slot = (int64_t)c * H_v + h;
    if (wave == 0) {
      double gv = 0.0;
      float bv = 0.f;
      if (lane < len) {
        gv = (double)floor_keep_nan(g[(int64_t)(t0 + lane) * H_v + h], kGFloor);
        bv = beta[(int64_t)(t0 + lane) * H_v + h];
      }
      const double gam = wave_inclusive_scan(gv, lane);
      if (lane < C) {
        sm.gam[lane] = gam;
        sm.beta[lane] = bv;
      }
    }
    __syncthreads();
    // A (strictly lower) to LDS; P (lower, diagonal included) to the workspace.
    CT *pph = plane<CT, C>(pmw, slot), *ppl = pph + C * C;
    for (int x4 = tid; x4 < C * C / 4; x4 += 256) {
      const int r = (4 * x4) / C, i0 = (4 * x4) % C;
      f32x4 av, pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        float a = 0.f, p = 0.f;
        if (i <= r) {
          const float dec = expf((float)(sm.gam[r] - sm.gam[i]));
          p = sm.rq[r] * sm.rk[i] * dec * sm.QK[r * LDC + i];
          if (i < r) a = sm.beta[r] * dec * sm.rk[r] * sm.rk[i] * sm.G[r * LDC + i];
        }
        av[e] = a;
        pv[e] = p;
      }
      *reinterpret_cast<f32x4 *>(A + r * LDC + i0) = av;
      put4<P::BF>(pph + 4 * x4, ppl + 4 * x4, pv);
    }
    if (tid < C) {
      eg[slot * C + tid] = expf((float)sm.gam[tid]);
      eb[slot * C + tid] = expf((float)(sm.gam[C - 1] - sm.gam[tid]));
    }
    __syncthreads();

    // T = (I + A)^{-1}.  Diagonal 16x16 blocks by forward substitution: lane
    // 16 b + c owns column c of block b.
    if (wave == 0 && lane < C) {
      const int bb = lane >> 4, cc = lane & 15;
      const float *Ab = A + (bb * 16) * LDC + bb * 16;
      float col[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = (r == cc) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) s -= Ab[r * LDC + m] * col[m];
        col[r] = s;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) Tm[(bb * 16 + r) * LDC + bb * 16 + cc] = col[r];
    }
    __syncthreads();
    // Below the diagonal, wave j fills block column j from the top down:
    //   T_ij = -T_ii * Y,  Y = sum_{m=j}^{i-1} A_im T_mj      (fp32 MFMA 16x16x4)
    // Y's MFMA takes contraction slot l/16 = index 4s + l/16 of step s; the
    // second product takes index 4(l/16) + s instead, which makes the B operand
    // of step s this lane's own accumulator element Y[4(l/16) + s][l%16].
    if (wave < NB - 1) {
      const int jb = wave;
      for (int ib = jb + 1; ib < NB; ++ib) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        for (int m = jb; m < ib; ++m) {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            y = mfma_f32(A[(16 * ib + lr) * LDC + 16 * m + 4 * s + lg],
                         Tm[(16 * m + 4 * s + lg) * LDC + 16 * jb + lr], y);
        }
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) t = mfma_f32(Tm[(16 * ib + lr) * LDC + 16 * ib + 4 * lg + s], y[s], t);
#pragma unroll
        for (int e = 0; e < 4; ++e) Tm[(16 * ib + 4 * lg + e) * LDC + 16 * jb + lr] = -t[e];
      }
    }
    __syncthreads();
    CT *tph = plane<CT, C>(tbw, slot), *tpl = tph + C * C;
    for (int x4 = tid; x4 < C * C / 4; x4 += 256) {
      const int r = (4 * x4) / C, i0 = (4 * x4) % C;
      f32x4 tv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + e;
        tv[e] = (i <= r) ? Tm[r * LDC + i] * sm.beta[i] : 0.f;
      }
      put4<P::BF>(tph + 4 * x4, tpl + 4 * x4, tv);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// carry: one (sequence, value head, DVB-column block of S) walks its chunks in
// order.  8 waves; every chunk's shared operands (q, k, v block, T diag(beta),
// P, decays) are fetched into registers while the previous chunk computes,
// then staged in LDS.  Per chunk, three barrier-separated phases:
//   1. [Q;K] S (waves 0-3: Q row tiles, waves 4-7: K row tiles, all column
//      tiles each, so A fragments are reused); X = V - e^G (K S) -> LDS
//   2. U = T diag(beta) X, one output tile per wave -> LDS (U and U'')
//   3. O = e^G Q S + P U (waves 0-3, from their own Q S);
//      S <- e^{G_last} S + K^T U'' (every wave its own S tiles; K^T fragments
//      are gathered from row-major K)
// ---------------------------------------------------------------------------
template <typename TIn, int DK, int C, int DVB> struct CarrySmem {
  using CT = typename Pol<TIn>::CT;
  static constexpr bool BF = Pol<TIn>::BF;
  static constexpr int PAD = Pol<TIn>::PAD;
  static constexpr int LDQ = DK + PAD;   // Q, K      [C][LDQ]
  static constexpr int LDST = DK + PAD;  // S^T       [DVB][LDST]
  static constexpr int LDX = C + PAD;    // Tb, P     [C][LDX];  X^T, U^T, U2^T [DVB][LDX]
  static constexpr int LO = BF ? 1 : 0;  // lo halves exist only on the bf16 path
  alignas(16) TIn q[C * LDQ];
  alignas(16) TIn k[C * LDQ];
  alignas(16) CT tbh[C * LDX];
  alignas(16) CT tbl[LO ? C * LDX : 4];
  alignas(16) CT ph[C * LDX];
  alignas(16) CT pl[LO ? C * LDX : 4];
  alignas(16) TIn v[C * DVB];
  alignas(16) CT sth[DVB * LDST];
  alignas(16) CT stl[LO ? DVB * LDST : 4];
  alignas(16) CT xth[DVB * LDX];
  alignas(16) CT xtl[LO ? DVB * LDX : 4];
  alignas(16) CT uth[DVB * LDX];
  alignas(16) CT utl[LO ? DVB * LDX : 4];
  alignas(16) CT u2h[DVB * LDX];
  alignas(16) CT u2l[LO ? DVB * LDX : 4];
  alignas(16) float eg[C], eb[C], rq[C], rk[C];
};

// The 16-byte vectors one chunk brings in, numbered: Q rows, K rows, T diag(beta)
// planes, P planes, the v block, e^G, e^{G_last - G}.
template <typename TIn, int DK, int C, int DVB> struct ChunkVecs {
  using CT = typename Pol<TIn>::CT;
  static constexpr int EQ = 16 / sizeof(TIn), EC = 16 / sizeof(CT);
  static constexpr int NPLANES = Pol<TIn>::BF ? 2 : 1;
  static constexpr int QROW = DK / EQ, VROW = DVB / EQ;
  static constexpr int NQ = C * QROW, NPL = C * C / EC, NTB = NPLANES * NPL, NVV = C * VROW, NE = C / 4;
  static constexpr int B_K = NQ, B_TB = 2 * NQ, B_PM = B_TB + NTB, B_V = B_PM + NTB, B_EG = B_V + NVV,
                       B_EB = B_EG + NE, TOTAL = B_EB + NE;
};

// Next-chunk prefetch into registers.  Every register slot belongs to one
// region (Q rows, K rows, the T diag(beta) planes, the P planes, the v block,
// the decay vectors), so the loads carry no divergent branches: a branch join
// would make the compiler wait for every load in flight.  Rows past the chunk's
// length are loaded from row 0 (always valid) and zeroed when stashed.
template <typename TIn, int DK, int C, int DVB, int NT>
struct Fetch {
  using V = ChunkVecs<TIn, DK, C, DVB>;
  using SM = CarrySmem<TIn, DK, C, DVB>;
  using CT = typename SM::CT;
  static constexpr int SQ = (V::NQ + NT - 1) / NT, ST = (V::NTB + NT - 1) / NT, SV = (V::NVV + NT - 1) / NT,
                       SE = (2 * V::NE + NT - 1) / NT;
  u32x4 rq[SQ], rk[SQ], rt[ST], rp[ST], rv[SV], re[SE];
  int len;

  __device__ __forceinline__ void load(const TIn *q, const TIn *k, const TIn *v, const unsigned char *tbw,
                                       const unsigned char *pmw, const float *egw, const float *ebw, int t0,
                                       int len_, int64_t slot, int j, int h, int H_qk, int H_v, int d_v,
                                       int col0, int tid) {
    len = len_;
#pragma unroll
    for (int i = 0; i < SQ; ++i) {
      const int y = tid + i * NT;
      if (y < V::NQ) {
        int row = y / V::QROW;
        row = row < len ? row : 0;
        const int64_t off = ((int64_t)(t0 + row) * H_qk + j) * DK + (y % V::QROW) * V::EQ;
        rq[i] = *reinterpret_cast<const u32x4 *>(q + off);
        rk[i] = *reinterpret_cast<const u32x4 *>(k + off);
      }
    }
    const u32x4 *tb = reinterpret_cast<const u32x4 *>(tbw + slot * (int64_t)(4 * C * C));
    const u32x4 *pm = reinterpret_cast<const u32x4 *>(pmw + slot * (int64_t)(4 * C * C));
#pragma unroll
    for (int i = 0; i < ST; ++i) {
      const int y = tid + i * NT;
      if (y < V::NTB) {
        rt[i] = tb[y];
        rp[i] = pm[y];
      }
    }
#pragma unroll
    for (int i = 0; i < SV; ++i) {
      const int y = tid + i * NT;
      if (y < V::NVV) {
        int row = y / V::VROW;
        row = row < len ? row : 0;
        rv[i] = *reinterpret_cast<const u32x4 *>(v + ((int64_t)(t0 + row) * H_v + h) * d_v + col0 +
                                                 (y % V::VROW) * V::EQ);
      }
    }
#pragma unroll
    for (int i = 0; i < SE; ++i) {
      const int y = tid + i * NT;
      if (y < 2 * V::NE) {
        const float *src = (y < V::NE ? egw : ebw) + slot * C;
        re[i] = reinterpret_cast<const u32x4 *>(src)[y % V::NE];
      }
    }
  }

  __device__ __forceinline__ void stash(SM &sm, int tid) const {
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < SQ; ++i) {
      const int y = tid + i * NT;
      if (y < V::NQ) {
        const int row = y / V::QROW, at = row * SM::LDQ + (y % V::QROW) * V::EQ;
        *reinterpret_cast<u32x4 *>(sm.q + at) = row < len ? rq[i] : zero;
        *reinterpret_cast<u32x4 *>(sm.k + at) = row < len ? rk[i] : zero;
      }
    }
#pragma unroll
    for (int i = 0; i < ST; ++i) {
      const int y = tid + i * NT;
      if (y < V::NTB) {
        const int pl = y / V::NPL, w = y % V::NPL;
        const int at = ((w * V::EC) / C) * SM::LDX + (w * V::EC) % C;
        *reinterpret_cast<u32x4 *>((pl ? sm.tbl : sm.tbh) + at) = rt[i];
        *reinterpret_cast<u32x4 *>((pl ? sm.pl : sm.ph) + at) = rp[i];
      }
    }
#pragma unroll
    for (int i = 0; i < SV; ++i) {
      const int y = tid + i * NT;
      if (y < V::NVV) {
        const int row = y / V::VROW;
        *reinterpret_cast<u32x4 *>(sm.v + row * DVB + (y % V::VROW) * V::EQ) = row < len ? rv[i] : zero;
      }
    }
#pragma unroll
    for (int i = 0; i < SE; ++i) {
      const int y = tid + i * NT;
      if (y < 2 * V::NE) *reinterpret_cast<u32x4 *>((y < V::NE ? sm.eg : sm.eb) + 4 * (y % V::NE)) = re[i];
    }
  }
};

template <typename TIn, int DK, int C, int DVB, bool STATES, bool OBF16>
__global__ __launch_bounds__(512) void carry_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ s0, const int32_t *__restrict__ status,
    const int32_t *__restrict__ seq_start, const int32_t *__restrict__ chunk_first,
    const unsigned char *__restrict__ tbw, const unsigned char *__restrict__ pmw,
    const float *__restrict__ egw, const float *__restrict__ ebw, void *__restrict__ o,
    float *__restrict__ fin, float *__restrict__ uw, float *__restrict__ scw, int N, int H_qk, int H_v,
    int d_v, float scale, int l2norm, int groups) {
  using P = Pol<TIn>;
  using F = Fr<P::BF>;
  using SM = CarrySmem<TIn, DK, C, DVB>;
  using CT = typename SM::CT;
  constexpr bool BF = P::BF;
  constexpr int NT = 512, KS = F::KS;
  constexpr int LDQ = SM::LDQ, LDST = SM::LDST, LDX = SM::LDX;
  constexpr int NMT = DK / 16, NNT = DVB / 16, NST = NMT * NNT, SPW = (NST + 7) / 8;
  constexpr int NRT = C / 16;
  static_assert(C % KS == 0 && DK % KS == 0 && DVB % 16 == 0 && NRT <= 4, "carry tiling");
  __shared__ SM sm;

  if (*status) return;
  const int NJB = d_v / DVB;
  const int u = xcd_group_remap(blockIdx.x, NJB * (H_v / H_qk), groups);  // (sequence, q/k head)
  if (u < 0) return;
  const int jb = u % NJB, h = (u / NJB) % H_v, n = u / (NJB * H_v);
  const int j = h / (H_v / H_qk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int col0 = jb * DVB;

  // This wave's tiles of the S block: tile id wave + 8 s -> (row tile, col tile).
  f32x4 S[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    S[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int t = wave + 8 * s;
    if (t < NST && s0) {
      const int mi = t / NNT, ni = t % NNT;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[s][i] = s0[((int64_t)(n * H_v + h) * DK + mi * 16 + 4 * lg + i) * d_v + col0 + ni * 16 + lr];
    }
  }

  const int c_begin = chunk_first[n], c_end = chunk_first[n + 1];
  const int s_begin = seq_start[n], s_end = seq_start[n + 1];
  Fetch<TIn, DK, C, DVB, NT> pre;
  if (c_begin < c_end)
    pre.load(q, k, v, tbw, pmw, egw, ebw, s_begin, min(C, s_end - s_begin), (int64_t)c_begin * H_v + h, j, h,
             H_qk, H_v, d_v, col0, tid);

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = s_begin + (c - c_begin) * C;
    const int len = min(C, s_end - t0);
    const int64_t slot = (int64_t)c * H_v + h;
    __syncthreads();  // the previous chunk is done with every LDS buffer
    pre.stash(sm, tid);
    if (!l2norm && tid < C) {
      sm.rq[tid] = scale;
      sm.rk[tid] = 1.f;
    }
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int t = wave + 8 * s;
      if (t < NST) {
        const int mi = t / NNT, ni = t % NNT;
        const int cn = ni * 16 + lr, rk0 = mi * 16 + 4 * lg;
        put4<BF>(sm.sth + cn * LDST + rk0, sm.stl + (BF ? cn * LDST + rk0 : 0), S[s]);
        if constexpr (STATES) {
#pragma unroll
          for (int i = 0; i < 4; ++i) scw[(slot * DK + rk0 + i) * d_v + col0 + cn] = S[s][i];
        }
      }
    }
    __syncthreads();
    if (c + 1 < c_end)  // in flight while this chunk computes
      pre.load(q, k, v, tbw, pmw, egw, ebw, t0 + C, min(C, s_end - t0 - C), slot + H_v, j, h, H_qk, H_v, d_v,
               col0, tid);
    if (l2norm) {
      if (tid < 2 * C) {
        const int r = tid % C;
        const TIn *row = (tid < C ? sm.q : sm.k) + r * LDQ;
        float ss = 0.f;
        for (int i = 0; i < DK; ++i) {
          const float a = Elem<TIn>::get(row, i);
          ss += a * a;
        }
        const float rn = 1.0f / sqrtf(ss + 1e-6f);
        if (tid < C) sm.rq[r] = rn * scale;
        else sm.rk[r] = rn;
      }
      __syncthreads();
    }

    // Phase 1: [Q;K] S.  Waves 0-3 take Q row tiles, waves 4-7 K row tiles.
    const bool isq = wave < 4;
    const int mt = wave & 3;
    f32x4 qsc[NNT];
    if (mt < NRT) {
      f32x4 acc[NNT];
#pragma unroll
      for (int ni = 0; ni < NNT; ++ni) acc[ni] = f32x4{0.f, 0.f, 0.f, 0.f};
      const TIn *Ab = (isq ? sm.q : sm.k) + mt * 16 * LDQ;
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += KS) {
        const auto a = F::row(Ab, LDQ, lane, k0);
#pragma unroll
        for (int ni = 0; ni < NNT; ++ni) {
          acc[ni] = F::mma(acc[ni], a, F::row(sm.sth + ni * 16 * LDST, LDST, lane, k0));
          if constexpr (BF) acc[ni] = F::mma(acc[ni], a, F::row(sm.stl + ni * 16 * LDST, LDST, lane, k0));
        }
      }
#pragma unroll
      for (int ni = 0; ni < NNT; ++ni) {
        if (isq) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = mt * 16 + 4 * lg + i;
            qsc[ni][i] = acc[ni][i] * sm.eg[r] * sm.rq[r];
          }
        } else {
          f32x4 xv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = mt * 16 + 4 * lg + i;
            xv[i] = Elem<TIn>::get(sm.v, r * DVB + ni * 16 + lr) - sm.eg[r] * sm.rk[r] * acc[ni][i];
          }
          const int cn = ni * 16 + lr, r0 = mt * 16 + 4 * lg;
          put4<BF>(sm.xth + cn * LDX + r0, sm.xtl + (BF ? cn * LDX + r0 : 0), xv);
        }
      }
    }
    __syncthreads();

    // Phase 2: U = T diag(beta) X (lower triangular: row tile m needs columns < 16 (m + 1)).
    for (int t = wave; t < NRT * NNT; t += 8) {
      const int um = t / NNT, un = t % NNT;
      f32x4 ua = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += KS) {
        if (k0 < 16 * (um + 1)) {
          const auto ah = F::row(sm.tbh + um * 16 * LDX, LDX, lane, k0);
          const auto bh = F::row(sm.xth + un * 16 * LDX, LDX, lane, k0);
          ua = F::mma(ua, ah, bh);
          if constexpr (BF) {
            ua = F::mma(ua, ah, F::row(sm.xtl + un * 16 * LDX, LDX, lane, k0));
            ua = F::mma(ua, F::row(sm.tbl + um * 16 * LDX, LDX, lane, k0), bh);
          }
        }
      }
      f32x4 u2;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = um * 16 + 4 * lg + i;
        u2[i] = sm.eb[r] * sm.rk[r] * ua[i];
        if constexpr (STATES) {
          if (r < len) uw[((int64_t)(t0 + r) * H_v + h) * d_v + col0 + un * 16 + lr] = ua[i];
        }
      }
      const int cn = un * 16 + lr, r0 = um * 16 + 4 * lg;
      put4<BF>(sm.uth + cn * LDX + r0, sm.utl + (BF ? cn * LDX + r0 : 0), ua);
      put4<BF>(sm.u2h + cn * LDX + r0, sm.u2l + (BF ? cn * LDX + r0 : 0), u2);
    }
    __syncthreads();

    // Phase 3a: O = e^G Q S + P U for this wave's Q row tile; rows < len are stored.
    if (isq && mt < NRT) {
      f32x4 oa[NNT];
#pragma unroll
      for (int ni = 0; ni < NNT; ++ni) oa[ni] = qsc[ni];
#pragma unroll
      for (int k0 = 0; k0 < C; k0 += KS) {
        if (k0 < 16 * (mt + 1)) {
          const auto ah = F::row(sm.ph + mt * 16 * LDX, LDX, lane, k0);
          typename F::T al;
          if constexpr (BF) al = F::row(sm.pl + mt * 16 * LDX, LDX, lane, k0);
#pragma unroll
          for (int ni = 0; ni < NNT; ++ni) {
            const auto bh = F::row(sm.uth + ni * 16 * LDX, LDX, lane, k0);
            oa[ni] = F::mma(oa[ni], ah, bh);
            if constexpr (BF) {
              oa[ni] = F::mma(oa[ni], ah, F::row(sm.utl + ni * 16 * LDX, LDX, lane, k0));
              oa[ni] = F::mma(oa[ni], al, bh);
            }
          }
        }
      }
      if (o) {
#pragma unroll
        for (int ni = 0; ni < NNT; ++ni) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = mt * 16 + 4 * lg + i;
            if (r < len) {
              const int64_t oi = ((int64_t)(t0 + r) * H_v + h) * d_v + col0 + ni * 16 + lr;
              if constexpr (OBF16) reinterpret_cast<uint16_t *>(o)[oi] = f2bf(oa[ni][i]);
              else reinterpret_cast<float *>(o)[oi] = oa[ni][i];
            }
          }
        }
      }
    }
    // Phase 3b: S <- e^{G_last} S + K^T diag(e^{G_last - G}) U.
    const float elast = sm.eg[C - 1];
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int t = wave + 8 * s;
      if (t < NST) {
        const int mi = t / NNT, ni = t % NNT;
        S[s] *= elast;
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += KS) {
          const auto a = F::col(sm.k + mi * 16, LDQ, lane, k0);
          S[s] = F::mma(S[s], a, F::row(sm.u2h + ni * 16 * LDX, LDX, lane, k0));
          if constexpr (BF) S[s] = F::mma(S[s], a, F::row(sm.u2l + ni * 16 * LDX, LDX, lane, k0));
        }
      }
    }
  }

  if (fin) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) {
      const int t = wave + 8 * s;
      if (t < NST) {
        const int mi = t / NNT, ni = t % NNT;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fin[((int64_t)(n * H_v + h) * DK + mi * 16 + 4 * lg + i) * d_v + col0 + ni * 16 + lr] = S[s][i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// stream: the state after every token, S <- e^{g_t} S + k_t u_t^T, from the
// chunk-start state and the write vectors of the carry phase.  Workgroup =
// (chunk, value head, block of RS * SRPT rows of S); a thread owns 4 columns of
// SRPT rows (rows rl + RS i), so that each wave store covers consecutive rows,
// and streams them out token by token with 16-byte stores.  The stores are
// plain (cached) ones: on the 4 GiB readout they write ~5% faster than
// non-temporal stores of the same pattern.
// Only the selected tokens are stored: tl = t_lo + j t_step < t_hi, tl the
// token's index in its row of rowT tokens, to states[row * n_sel + j]; a chunk
// with no selected token is skipped.
// ---------------------------------------------------------------------------
template <typename TIn, int C, int SRPT>
__global__ __launch_bounds__(256) void stream_kernel(
    const TIn *__restrict__ k, const float *__restrict__ g, const float *__restrict__ uw,
    const float *__restrict__ scw, const Seqs sq, float *__restrict__ states, int H_qk, int H_v, int d_k,
    int d_v, int l2norm, int rowT, int t_lo, int t_hi, int t_step, int n_sel) {
  extern __shared__ float ssm[];  // u [C][d_v], kk [C][RS][SRPT], alpha [C]
  static_assert(SRPT % 4 == 0 || SRPT == 1, "k factors are read 4 at a time");
  if (sq.bad()) return;
  const int c = blockIdx.x;
  if (c >= sq.chunks()) return;
  const int n = sq.seq_of(c);
  const int t0 = sq.start(n) + (c - sq.first(n)) * C;
  const int len = min(C, sq.start(n + 1) - t0);
  const int h = blockIdx.y, j = h / (H_v / H_qk);
  // the chunk's tokens lie in one row: row b, in-row indices tl0 .. tl0 + len
  const int brow = t0 / rowT, tl0 = t0 - brow * rowT;
  int r_end;  // tokens of the chunk to step through: up to its last selected one
  {
    const int f = max(t_lo, tl0), e = min(t_hi, tl0 + len);
    const int first = t_lo + (f - t_lo + t_step - 1) / t_step * t_step;  // first selected in-row index >= f
    if (first >= e) return;
    r_end = t_lo + (e - 1 - t_lo) / t_step * t_step - tl0 + 1;
  }
  const int CGn = d_v / 4, RS = 256 / CGn, SR = RS * SRPT;
  const int row0 = blockIdx.z * SR;
  const int tid = threadIdx.x, cg = tid % CGn, rl = tid / CGn;
  float *us = ssm, *kk = ssm + C * d_v, *al = kk + C * SR;
  const int64_t slot = (int64_t)c * H_v + h;
  // The chunk-start state is loaded first; it is not needed before the barrier.
  // Rows past d_k (and the tail threads when 256 % (d_v / 4) != 0) read row
  // d_k - 1: computed, never stored.
  f32x4 Sv[SRPT];
#pragma unroll
  for (int i = 0; i < SRPT; ++i) {
    const int row = min(row0 + rl + RS * i, d_k - 1);
    Sv[i] = *reinterpret_cast<const f32x4 *>(scw + (slot * d_k + row) * d_v + 4 * cg);
  }
  for (int x = tid; x < len * CGn; x += 256) {
    const int r = x / CGn, cc = x % CGn;
    *reinterpret_cast<f32x4 *>(us + r * d_v + 4 * cc) =
        *reinterpret_cast<const f32x4 *>(uw + ((int64_t)(t0 + r) * H_v + h) * d_v + 4 * cc);
  }
  if (tid < len) al[tid] = expf(g[(int64_t)(t0 + tid) * H_v + h]);
  if (row0 + SR > d_k)  // factors of rows past d_k are zero
    for (int x = tid; x < C * SR; x += 256) {
      const int y = x % SR;
      if (row0 + y / SRPT + RS * (y % SRPT) >= d_k) kk[x] = 0.f;
    }
  // Key rows: 16-byte loads, VPR of them per row on VPR neighbouring lanes (a
  // power of two that divides the wave), whose shuffle sum gives |k_r|^2; each
  // factor k_r[row] (times 1/|k_r| with l2norm) goes to kk[r][rr][i] for
  // row = row0 + rr + RS i.
  constexpr int VE = 16 / sizeof(TIn);
  const int VPR = d_k / VE;
  for (int base = 0; base < C * VPR; base += 256) {  // uniform trip count: every lane shuffles
    const int v = base + tid, r = v / VPR, part = v % VPR;
    float e[VE];
    if (r < len) {
      const TIn *src = k + ((int64_t)(t0 + r) * H_qk + j) * d_k + part * VE;
      if constexpr (std::is_same_v<TIn, float>) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(src);
#pragma unroll
        for (int q = 0; q < 4; ++q) e[q] = x[q];
      } else {
        const u32x4 x = *reinterpret_cast<const u32x4 *>(src);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          e[2 * q] = __uint_as_float(x[q] << 16);
          e[2 * q + 1] = __uint_as_float(x[q] & 0xffff0000u);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < VE; ++q) e[q] = 0.f;
    }
    float rk = 1.f;
    if (l2norm) {
      float ss = 0.f;
#pragma unroll
      for (int q = 0; q < VE; ++q) ss += e[q] * e[q];
      for (int o = 1; o < VPR; o <<= 1) ss += __shfl_xor(ss, o);
      rk = 1.0f / sqrtf(ss + 1e-6f);
    }
    if (r < len) {
#pragma unroll
      for (int q = 0; q < VE; ++q) {
        const int loc = part * VE + q - row0;
        if (loc >= 0 && loc < SR) kk[r * SR + (loc % RS) * SRPT + loc / RS] = e[q] * rk;
      }
    }
  }
  __syncthreads();
  if (rl >= RS) return;  // tail threads when 256 % (d_v / 4) != 0
  const int64_t sstride = (int64_t)H_v * d_k * d_v;  // one token
  float *const head0 = states + (int64_t)h * d_k * d_v;
  // Byte offsets in a token's d_k x d_v block of this head: the thread's first
  // row, and from one of its rows to the next.  Rows past d_k lie outside the
  // block, so their stores are dropped by the buffer's range check.
  const int off0 = ((row0 + rl) * d_v + 4 * cg) * 4, roff = RS * d_v * 4;
  for (int r = 0; r < r_end; ++r) {
    const f32x4 uv = *reinterpret_cast<const f32x4 *>(us + r * d_v + 4 * cg);
    const float a = al[r];
    float kf[SRPT];
    if constexpr (SRPT == 1) {
      kf[0] = kk[r * SR + rl];
    } else {
#pragma unroll
      for (int i4 = 0; i4 < SRPT; i4 += 4) {
        const f32x4 k4 = *reinterpret_cast<const f32x4 *>(kk + r * SR + rl * SRPT + i4);
#pragma unroll
        for (int e = 0; e < 4; ++e) kf[i4 + e] = k4[e];
      }
    }
#pragma unroll
    for (int i = 0; i < SRPT; ++i) Sv[i] = a * Sv[i] + kf[i] * uv;
    const int tl = tl0 + r;
    if (tl >= t_lo && tl < t_hi && (tl - t_lo) % t_step == 0) {  // uniform over the block
      const auto rs = rows_rsrc(head0 + ((int64_t)brow * n_sel + (tl - t_lo) / t_step) * sstride,
                                (int64_t)d_k * d_v * 4);
#pragma unroll
      for (int i = 0; i < SRPT; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, Sv[i]), rs, off0 + i * roff, 0, 2);
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
hipError_t launch_plan(const Problem &p, const ChunkArgs &a, hipStream_t st) {
  const Workspace &w = a.ws;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, st, a.cu, p.N, p.T, p.T_tot, p.C, p.max_chunks,
                     w.status, w.seq_start, w.chunk_first, w.order);
  return hipGetLastError();
}

template <typename TIn, int C, int SRPT>
static hipError_t stream_t(const Problem &p, const ChunkArgs &a, const Seqs &sq, hipStream_t st) {
  const Workspace &w = a.ws;
  const int CGn = p.d_v / 4, SR = (256 / CGn) * SRPT;
  const int zb = ceil_div(p.d_k, SR);
  if (p.max_chunks > 0 && p.H_v > 0 && zb > 0) {
    const size_t shm = sizeof(float) * ((size_t)C * p.d_v + (size_t)C * SR + C);
    if (a.n_sel <= 0) return hipSuccess;
    const int rowT = p.packed ? p.T_tot : p.T;
    hipLaunchKernelGGL((stream_kernel<TIn, C, SRPT>), dim3(p.max_chunks, p.H_v, zb), dim3(256), shm, st,
                       static_cast<const TIn *>(a.k), a.g, w.u, w.sc, sq, a.states, p.H_qk, p.H_v, p.d_k, p.d_v,
                       p.l2norm ? 1 : 0, rowT, a.t_lo, a.t_hi, a.t_step, a.n_sel);
    return hipGetLastError();
  }
  return hipSuccess;
}

// Rows per thread: as many as keep the row block within d_k (16, 4 or 1).
template <typename TIn, int C>
static hipError_t stream_rows(const Problem &p, const ChunkArgs &a, const Seqs &sq, hipStream_t st) {
  const int RS = 256 / (p.d_v / 4);
  if (RS * 16 <= p.d_k) return stream_t<TIn, C, 16>(p, a, sq, st);
  if (RS * 4 <= p.d_k) return stream_t<TIn, C, 4>(p, a, sq, st);
  return stream_t<TIn, C, 1>(p, a, sq, st);
}

hipError_t launch_states_stream(const Problem &p, const ChunkArgs &a, const Seqs &sq, hipStream_t st) {
  if (p.dtype == GDN_BF16) {
    if (p.C == 64) return stream_rows<uint16_t, 64>(p, a, sq, st);
    if (p.C == 32) return stream_rows<uint16_t, 32>(p, a, sq, st);
  } else {
    if (p.C == 64) return stream_rows<float, 64>(p, a, sq, st);
    if (p.C == 32) return stream_rows<float, 32>(p, a, sq, st);
    if (p.C == 16) return stream_rows<float, 16>(p, a, sq, st);
  }
  return hipErrorInvalidValue;
}

template <typename TIn, int DK, int C, int DVB, bool STATES, bool OBF16>
static hipError_t run_t(const Problem &p, const ChunkArgs &a, hipStream_t st) {
  const Workspace &w = a.ws;
  mark_event(a, 0, st);
  hipError_t e = launch_plan(p, a, st);
  if (e != hipSuccess) return e;
  mark_event(a, 1, st);
  const TIn *q = static_cast<const TIn *>(a.q), *k = static_cast<const TIn *>(a.k),
            *v = static_cast<const TIn *>(a.v);
  if (p.max_chunks > 0 && p.H_qk > 0) {
    hipLaunchKernelGGL((prep_kernel<TIn, DK, C>), dim3(p.max_chunks, p.H_qk), dim3(256), 0, st, q, k, a.g,
                       a.beta, w.status, w.seq_start, w.chunk_first, reinterpret_cast<unsigned char *>(w.tb),
                       reinterpret_cast<unsigned char *>(w.pm), w.eg, w.eb, p.N, p.H_qk, p.H_v, p.scale,
                       p.l2norm ? 1 : 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  mark_event(a, 2, st);
  const int groups = p.N * p.H_qk;
  if (groups > 0 && p.d_v > 0) {
    const int grid = xcd_group_grid(p.d_v / DVB * (p.H_v / p.H_qk), groups);
    hipLaunchKernelGGL((carry_kernel<TIn, DK, C, DVB, STATES, OBF16>), dim3(grid), dim3(512), 0, st, q, k, v,
                       a.s0, w.status, w.seq_start, w.chunk_first, reinterpret_cast<const unsigned char *>(w.tb),
                       reinterpret_cast<const unsigned char *>(w.pm), w.eg, w.eb, a.o,
                       a.final_state, w.u, w.sc, p.N, p.H_qk, p.H_v, p.d_v, p.scale, p.l2norm ? 1 : 0, groups);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  mark_event(a, 3, st);
  if constexpr (STATES) {
    const Seqs sq{w.status, w.seq_start, w.chunk_first, p.N, 0, 0};
    if ((e = launch_states_stream(p, a, sq, st)) != hipSuccess) return e;
    mark_event(a, 4, st);
  }
  return hipSuccess;
}

template <typename TIn, int DK, int C, int DVB>
static hipError_t run_cfg(const Problem &p, const ChunkArgs &a, bool states, hipStream_t st) {
  const bool ob = p.o_dtype == GDN_BF16;
  if (states) return ob ? run_t<TIn, DK, C, DVB, true, true>(p, a, st) : run_t<TIn, DK, C, DVB, true, false>(p, a, st);
  return ob ? run_t<TIn, DK, C, DVB, false, true>(p, a, st) : run_t<TIn, DK, C, DVB, false, false>(p, a, st);
}

bool chunk_path_supported(const Problem &p) {
  // d_v <= 128 keeps the states stream's LDS staging (C x d_v fp32) within 64 KiB.
  if (p.d_v > 128) return false;
  if (p.dtype == GDN_BF16) {
    if (p.d_k != 128) return false;  // bf16 MFMA contracts over 32: d_k and C multiples of 32
    return (p.C == 64 || p.C == 32) && p.d_v % 16 == 0;
  }
  return (p.d_k == 16 || p.d_k == 128) && (p.C == 16 || p.C == 32 || p.C == 64) && p.d_v % 16 == 0;
}

// fp32 inputs at every supported (d_k, chunk), and bf16 inputs at chunk 32, take the
// general path of this file (fp32: exact fp32 MFMA; bf16: hi/lo bf16 operands); bf16
// at chunk 64 takes the fused path of gdn_fused.hip.
template <typename TIn, int DK>
static hipError_t run_chunk(const Problem &p, const ChunkArgs &a, bool states, hipStream_t st) {
  if constexpr (std::is_same<TIn, float>::value) {
    if (p.C == 16) return run_cfg<TIn, DK, 16, 16>(p, a, states, st);
  }
  if (p.C == 32) return run_cfg<TIn, DK, 32, 16>(p, a, states, st);
  if constexpr (std::is_same<TIn, float>::value) {
    if (p.C == 64) return run_cfg<TIn, DK, 64, 16>(p, a, states, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_path(const Problem &p, const ChunkArgs &a, bool states, hipStream_t st) {
  if (!chunk_path_supported(p)) return hipErrorInvalidValue;
  if (p.dtype == GDN_BF16) {
    if (p.C == 64) return launch_fused_path(p, a, states, st);
    return run_chunk<uint16_t, 128>(p, a, states, st);
  }
  return p.d_k == 16 ? run_chunk<float, 16>(p, a, states, st) : run_chunk<float, 128>(p, a, states, st);
}

Workspace workspace_layout(const Problem &p, bool states, void *base) {
  Workspace w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes, 256);
    return at;
  };
  const size_t st = take(sizeof(int32_t));
  const size_t ss = take(sizeof(int32_t) * ((size_t)p.N + 1));
  const size_t cf = take(sizeof(int32_t) * ((size_t)p.N + 1));
  const size_t od = take(sizeof(int32_t) * ((size_t)p.N + 1));
  const size_t cc = (size_t)p.max_chunks * p.H_v;
  const bool fused = p.dtype == GDN_BF16 && p.C == 64;  // the path of gdn_fused.hip
  size_t tb = 0, pm = 0, eg = 0, eb = 0, tt = 0, kk = 0, pf = 0;
  const bool wide = fused && fused_solve_p(p);  // the solve forms P for these chains
  if (fused) {
    tt = take(fused_t_bytes() * cc);
    kk = take(fused_k_bytes() * (size_t)p.max_chunks * p.H_qk);
    if (wide) pf = take(fused_p_bytes() * cc);
  } else {
    tb = take(sizeof(float) * cc * p.C * p.C);
    pm = take(sizeof(float) * cc * p.C * p.C);
    eg = take(sizeof(float) * cc * p.C);
    eb = take(sizeof(float) * cc * p.C);
  }
  size_t uo = 0, so = 0;
  if (states) {
    uo = take(sizeof(float) * (size_t)p.T_tot * p.H_v * p.d_v);
    so = take(sizeof(float) * cc * p.d_k * p.d_v);
  }
  w.bytes = off;
  if (base) {
    char *b = static_cast<char *>(base);
    w.status = reinterpret_cast<int32_t *>(b + st);
    w.seq_start = reinterpret_cast<int32_t *>(b + ss);
    w.chunk_first = reinterpret_cast<int32_t *>(b + cf);
    w.order = reinterpret_cast<int32_t *>(b + od);
    if (fused) {
      w.tt = reinterpret_cast<unsigned char *>(b + tt);
      w.kk = reinterpret_cast<unsigned char *>(b + kk);
      if (wide) w.pf = reinterpret_cast<unsigned char *>(b + pf);
    } else {
      w.tb = reinterpret_cast<float *>(b + tb);
      w.pm = reinterpret_cast<float *>(b + pm);
      w.eg = reinterpret_cast<float *>(b + eg);
      w.eb = reinterpret_cast<float *>(b + eb);
    }
    if (states) {
      w.u = reinterpret_cast<float *>(b + uo);
      w.sc = reinterpret_cast<float *>(b + so);
    }
  }
  return w;
}

}  // namespace gdn
