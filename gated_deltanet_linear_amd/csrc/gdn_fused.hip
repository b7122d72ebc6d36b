// The bf16 chunked path of libgdn (d_k = 128, chunk C = 64): gdn_chunk_fwd and
// gdn_states_fwd on bf16 q, k, v, in two launches.
//
// It computes the gated delta rule of the pages (Qwen3.5 text encyclopedia
// page, note "The DeltaNet mixer") in the UT / WY chunk form.  Per (chunk,
// value head), with the in-chunk cumulative log decay G_r = g_0 + ... + g_r,
// the raw keys K and queries Q (rk_r, rq_r: the row scalings of the optional
// in-kernel l2 norm, rq also carrying the scale), and S the state at the chunk
// start:
//
//   A[r,i] = beta_r rk_r rk_i e^{G_r - G_i} (k_r . k_i), i < r,  T = (I + A)^{-1}
//   X      = V - diag(e^G rk) K S
//   U      = T diag(beta) X                           the tokens' write vectors
//   P[r,i] = rq_r rk_i e^{G_r - G_i} (q_r . k_i), i <= r
//   O      = diag(e^G rq) Q S + P U
//   S     <- e^{G_last} S + K^T diag(e^{G_last - G} rk) U
//
// solve (chunk, query/key head): the keys' and queries' fp16 MFMA fragments and
//   norms once, K K^T once for the value heads that share the keys, then per
//   value head the decays, A, the fp32 triangular solve, T~ = T diag(beta) as
//   fp16 hi/lo MFMA fragments, and the per-token decay factors the chain uses.
//   These are all that passes between the two launches: 14 KiB per (value head,
//   chunk) and 32 KiB per (query/key head, chunk).
// chain (sequence, value head, block of 16 NB columns of S): walks the chunks
//   of one sequence in order.  v, the Q K^T products, the carry and the output
//   are formed here.  Wave roles:
//     copy   (1 wave)   copies chunk c+1's K, Q and T~ fragments and factors from
//                       the workspace straight into its LDS stage (global -> LDS
//                       loads, no registers), and moves its v to the accumulator
//                       order (an identity MFMA; v's loads run a chunk ahead);
//     carry  (NB waves) wave j keeps columns [16j, 16j + 16) of the block's S
//                       (all d_k rows, fp32) in registers and runs K S, X,
//                       T~ X, U'' and K^T U'' for chunk c with no barrier:
//                       every accumulator feeds the next MFMA as its operand
//                       through the contraction order below, and K^T comes from
//                       the K fragments by transposed LDS reads;
//     output (2 waves)  form P from Q K^T and Q S for chunk c, and P U for chunk
//                       c-1 (whose U the carry published before the last
//                       barrier), and store o of chunk c-1: wave 0 token tiles
//                       {0, 3}, wave 1 {1, 2};
//     stream (with the states kept for at least half of the tokens) step the
//                       block's columns of S through every token from the same
//                       published U and store each kept state; each column block
//                       then runs as two blocks, one per half of S's rows.
//   One barrier per chunk, ordering LDS only; nothing else synchronises the waves.
// wide chain (sequence, value head), where sequences x value heads fill every CU:
//   eight column waves each carry one 16-column tile and form its output, with P
//   formed by the copy wave; optionally with the mixer's output norm applied in place
//   of o.  Packed sequences split each head over two workgroups of four column waves,
//   which take P from the solve.
//
// MFMA lane order (v_mfma_f32_16x16x32_f16): lane l feeds row l%16 of A and
// column l%16 of B, and 8 contraction indices chosen by the group g = l/16.
// The accumulator holds rows 4g + i, i < 4, of column l%16.  The contraction
// indices of group g in step s are {32s + 4g + i, 32s + 16 + 4g + i}, i < 4:
// exactly the rows lane l holds in the accumulators of two vertically adjacent
// 16-row tiles.  So S (rows of d_k), X, U and U'' (rows of tokens) become B
// operands in place, and P (from the accumulators of K Q^T) an A operand.
//
// Precision (a numpy emulation of this placement on the 4096-token prefill
// laws gave max|dO| ~5e-4 x RMS(o) and a final-state error ~2e-7, 1e-3 and
// 4e-5 with slow decays): q, k enter fp16 MFMA exactly (bf16 values in fp16's
// normal range); S enters once in fp16; T~, X, P, U and U'' as fp16 hi/lo
// pairs (hi*hi + hi*lo + lo*hi where both sides are split).  Single-fp16 X
// and U cost ~5e-3 x RMS on o and ~2e-4 on a state left by a short last chunk.  fp16's range
// bounds the carried operands: a value of S, X, U or U'' beyond 65504 becomes an
// infinity that reaches o or the final state, and any non-finite o or final-state
// value sets bit 1 of the workspace status word (the results are then invalid).
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn.h"

namespace gdn {
namespace {

constexpr int DK = 128, C = 64;
constexpr float kFloor = -1.0e4f;
constexpr int LDK = DK + 8;  // solve: k rows (bf16)
constexpr int LDF = C + 4;   // solve: fp32 C x C

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f16x8 as_h(const u32x4 &x) { return __builtin_bit_cast(f16x8, x); }
__device__ __forceinline__ f32x4 mfma_h(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h(a), as_h(b), c, 0, 0, 0);
}
// e^x on the hardware exponential (v_exp_f32 of x log2 e): a few ulp for the
// decay arguments met here.
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
// Two fp32 values -> one packed fp16 pair (v_cvt_pk_f16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pk_f16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, f16x2_t));
}
__device__ __forceinline__ f32x2_t unpk_f16(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
}
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x, y}, bf16x2_t));
}
// The 8 values {a[0..3], b[0..3]} as one fp16 fragment.
__device__ __forceinline__ u32x4 h16x8(const f32x4 &a, const f32x4 &b) {
  return u32x4{pk_f16(a[0], a[1]), pk_f16(a[2], a[3]), pk_f16(b[0], b[1]), pk_f16(b[2], b[3])};
}
// ... and as hi + lo (x = hi + lo + O(2^-22 |x|) in fp16's normal range).
__device__ __forceinline__ void split8h(const f32x4 &a, const f32x4 &b, u32x4 &hi, u32x4 &lo) {
  hi = h16x8(a, b);
  const f32x2_t h0 = unpk_f16(hi[0]), h1 = unpk_f16(hi[1]), h2 = unpk_f16(hi[2]), h3 = unpk_f16(hi[3]);
  lo = u32x4{pk_f16(a[0] - h0[0], a[1] - h0[1]), pk_f16(a[2] - h1[0], a[3] - h1[1]),
             pk_f16(b[0] - h2[0], b[1] - h2[1]), pk_f16(b[2] - h3[0], b[3] - h3[1])};
}
// 8 bf16 values (two 8-byte words) as one fp16 fragment: exact for values in
// fp16's normal range (|x| in [2^-14, 65504]); smaller ones round to fp16's
// subnormals, larger ones overflow (the range check catches what follows).
__device__ __forceinline__ u32x4 bf8_to_h(const u32x2 &a, const u32x2 &b) {
  return u32x4{pk_f16(bf_lo(a[0]), bf_hi(a[0])), pk_f16(bf_lo(a[1]), bf_hi(a[1])),
               pk_f16(bf_lo(b[0]), bf_hi(b[0])), pk_f16(bf_lo(b[1]), bf_hi(b[1]))};
}
// Workgroup barrier that orders LDS accesses only.  Every exchange between the
// chain kernel's waves goes through LDS; their global loads and stores are
// private (the o and states stores, the T~ loads), so a barrier need not wait for
// them -- a full __syncthreads() would hold each chunk for a global memory round
// trip.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One 16-byte global -> LDS load per lane (global_load_lds_dwordx4): lane l's 16
// bytes at src (its own address) land at lds + 16 l; lds is the same for the wave.
__device__ __forceinline__ void lds_copy16(const void *src, void *lds) {
  __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// Waits until at most N vector-memory operations of the wave are outstanding
// (vmcnt(N); they complete in issue order), which covers global -> LDS loads: the
// compiler does not track those for LDS readers in other waves.  The signal fences
// keep memory accesses on their side.
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0f70 | N);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Sum over the 16 lanes of each DPP row (lanes 16g .. 16g + 15), in every lane:
// rotations by 8, 4, 2 and 1 within the row.
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
  return x;
}
__device__ __forceinline__ float silu_f(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
// The value x of lane `src` (0 .. 63), through the LDS crossbar (no memory access).
__device__ __forceinline__ float lane_read(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * src, __builtin_bit_cast(int, x)));
}
// Four consecutive output values at byte offset off of a row range: 16 bytes (fp32) or
// 8 bytes (bf16, rounded to nearest even).
// Cache policy of the chain's streamed outputs (o and the per-token states): non-temporal,
// so that they drain to memory during the kernel instead of sitting dirty in L2 at its
// end (prefill 116 -> 115 us, states 773 -> 757 us).  The head-wide chain's o stores keep
// the default policy: streamed, its calls measured 2-3% slower.
constexpr int kNT = 2;
template <bool OBF16>
__device__ __forceinline__ void store_o4(__amdgpu_buffer_rsrc_t r, int off, const f32x4 &x) {
  if constexpr (OBF16)
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3])}, r, off, 0, 0);
  else
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}

// The 6 lower fragments of a C x C lower-triangular A operand: (row tile m,
// token step s) with 32 s <= 16 m + 15.
__device__ __forceinline__ constexpr int tri_frag(int m, int s) { return m < 2 ? m : 2 * m - 2 + s; }
constexpr int kTriFrags = 6;
// The K and Q fragments sit in the workspace (and LDS) with lane l's 16 bytes in slot
// kf_slot(l): bit 3 flips in the odd 16-lane groups.  The fragment readers stay free of
// LDS bank conflicts and the transposed reads of K (below) conflict only 2-way.
__device__ __forceinline__ constexpr int kf_slot(int x) { return x ^ (((x >> 4) & 1) << 3); }
// ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives as element e the 16-bit
// value in position i%4 of the 4 that lane 4e + i/4 of its group addressed.
__device__ __forceinline__ u32x2 lds_read_tr16(const void *p) {
  typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4_t;
  const auto *lp = (const __attribute__((address_space(3))) fp16x4_t *)(p);
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                       const_cast<__attribute__((address_space(3))) fp16x4_t *>(lp)));
}
// Per (value head, chunk): the T~ hi and lo fragments, then the chain's per-token
// factors as rows of C floats: G log2(e) (G the in-chunk cumulative decay), e^G rk,
// e^{G_last - G} rk (zero past the chunk's length), e^G rq, rk, rq, and a row whose
// first entry is e^{G_last}.
constexpr size_t kTFragBytes = 2 * kTriFrags * 64 * 16;
enum { FAC_GL2 = 0, FAC_EKR, FAC_FKR, FAC_EQR, FAC_RK, FAC_RQ, FAC_EL, kFacRows = 8 };
constexpr size_t kTBytes = kTFragBytes + kFacRows * C * 4;
// Per (value head, chunk), split head-wide chains only: P's hi/lo A fragments, as T~'s.
constexpr size_t kPBytes = 2 * kTriFrags * 64 * 16;
// Per (query/key head, chunk): 16 K fragments, then 16 Q fragments (fp16).
constexpr size_t kKFragBytes = 16 * 64 * 16;
constexpr size_t kKBytes = 2 * kKFragBytes;

// ---------------------------------------------------------------------------
// solve: one (chunk, query/key head) per block of 4 waves; K K^T once, then per
// value head of the group the decays, A, T = (I + A)^{-1} and the fragments of
// T~ = T diag(beta).  About 37 KiB of LDS: four blocks share a CU.
// ---------------------------------------------------------------------------
struct SolveSmem {
  alignas(16) float ra[C * LDF];  // key rows (bf16, row stride LDK) until K K^T is formed, then A
  alignas(16) float rt[C * LDF];  // query rows until their fragments are out, then T
  alignas(16) f32x4 y[2][64];     // the solve's exchange: Y of row block 2, column blocks 0 and 1
  alignas(16) double gam[C];
  alignas(16) float beta[C], rk[C], rq[C];
};
static_assert(sizeof(float) * C * LDF >= sizeof(uint16_t) * C * LDK, "key and query rows fit the A and T regions");

// One 16x16 block product on fp32 MFMA, accumulated: acc += X_{ib,m} Y_{m,jb}, where X
// and Y are C x C row-major LDS matrices (row stride LDF); step s contracts index
// 4s + l/16.  The result holds rows 4(l/16) + i of column l%16.
__device__ __forceinline__ f32x4 block_mm(const float *X, const float *Y, int ib, int m, int jb, int lr, int lg,
                                          f32x4 acc) {
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = mfma_f32(X[(16 * ib + lr) * LDF + 16 * m + 4 * s + lg], Y[(16 * m + 4 * s + lg) * LDF + 16 * jb + lr], acc);
  return acc;
}
// acc += X_{ib,m} Z for a 16x16 block Z held as an accumulator (z[s]: rows 4(l/16) + s of
// column l%16): step s contracts index 4(l/16) + s, which is this lane's own z[s].
__device__ __forceinline__ f32x4 block_mm_acc(const float *X, int ib, int m, const f32x4 &z, int lr, int lg,
                                              f32x4 acc) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = mfma_f32(X[(16 * ib + lr) * LDF + 16 * m + 4 * lg + s], z[s], acc);
  return acc;
}

template <bool WP>  // WP: also P's fragments, for split head-wide chains
__global__ __launch_bounds__(256) void solve_kernel(const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
                                                    const float *__restrict__ g, const float *__restrict__ beta,
                                                    const Seqs seqs, int32_t *__restrict__ status,
                                                    unsigned char *__restrict__ tt, unsigned char *__restrict__ kk,
                                                    unsigned char *__restrict__ pf, int H_qk, int H_v, int MC,
                                                    float scale, int l2norm) {
  __shared__ SolveSmem sm;
  if (blockIdx.x == 0 && threadIdx.x == 0 && seqs.T != 0) *status = 0;  // dense rows: no plan kernel clears it
  if (seqs.bad()) return;
  const int nch = seqs.chunks();
  // The query/key heads of one chunk share an XCD: they read the same rows of g and
  // beta (a few bytes each per row), which that XCD's L2 then fetches once.
  const int u = xcd_group_remap(blockIdx.x, H_qk, MC);
  if (u < 0) return;
  const int cpos = u / H_qk, j = u % H_qk;
  if (cpos >= nch) return;
  // Chunks run last to first: the chain's first chunks are the ones written last.
  const int c = nch - 1 - cpos;
  const int n = seqs.seq_of(c);
  const int t0 = seqs.start(n) + (c - seqs.first(n)) * C;
  const int len = min(C, seqs.start(n + 1) - t0);
  const int R = H_v / H_qk;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  uint16_t *sk = reinterpret_cast<uint16_t *>(sm.ra), *sq = reinterpret_cast<uint16_t *>(sm.rt);
  float *A = sm.ra, *T = sm.rt;

  // Wave 3 holds the decays and write strengths of the next value head (lane = token),
  // loaded one head ahead.
  float graw = 0.f, braw = 0.f;
  auto load_gb = [&](int rr) {
    const int tl = min(lane, len - 1), h = j * R + rr;
    graw = g[(int64_t)(t0 + tl) * H_v + h];
    braw = beta[(int64_t)(t0 + tl) * H_v + h];
  };
  if (w == 3) load_gb(0);

  // Key and query rows: 16 lanes per row, 16-byte loads; |k_r|^2 and |q_r|^2 from
  // shuffle sums.  Rows past the chunk's length are zero.
  {
    u32x4 kv[4], qv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = tid + 256 * i, r = min(x >> 4, len - 1), cv = x & 15;
      const int64_t off = ((int64_t)(t0 + r) * H_qk + j) * DK + cv * 8;
      // read once: non-temporal, so that the L2 keeps this kernel's outputs for the chain
      kv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(k + off));
      qv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(q + off));
    }
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s2 = 0.f, t2 = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s2 += bf_lo(kv[i][e]) * bf_lo(kv[i][e]) + bf_hi(kv[i][e]) * bf_hi(kv[i][e]);
        t2 += bf_lo(qv[i][e]) * bf_lo(qv[i][e]) + bf_hi(qv[i][e]) * bf_hi(qv[i][e]);
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        s2 += __shfl_xor(s2, o);
        t2 += __shfl_xor(t2, o);
      }
      const int x = tid + 256 * i, r = x >> 4, cv = x & 15;
      if (cv == 0) {
        sm.rk[r] = l2norm ? 1.0f / sqrtf(s2 + 1e-6f) : 1.f;
        sm.rq[r] = l2norm ? scale / sqrtf(t2 + 1e-6f) : scale;
      }
      *reinterpret_cast<u32x4 *>(sk + r * LDK + cv * 8) = r < len ? kv[i] : zero;
      *reinterpret_cast<u32x4 *>(sq + r * LDK + cv * 8) = r < len ? qv[i] : zero;
    }
  }
  __syncthreads();
  // The keys' and queries' fp16 fragments for the chain (raw rows: the norms are
  // row scalings there).  Fragment 4m + s, lane l (slot kf_slot(l)): token 16m + l%16
  // at d_k {32s + 4g + i, 32s + 16 + 4g + i}: K is the A operand of K S and of K Q^T,
  // Q the A operand of Q S and the B operand of K Q^T.
  {
    unsigned char *dst = kk + ((int64_t)j * MC + c) * kKBytes;
    u32x4 *kfr = reinterpret_cast<u32x4 *>(dst), *qfr = reinterpret_cast<u32x4 *>(dst + kKFragBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int it = tid + 256 * i, f = it >> 6, ln = it & 63, r = ln & 15, gg = ln >> 4;
      const int m = f >> 2, s = f & 3, at = (16 * m + r) * LDK + 32 * s + 4 * gg;
      const int slot = (f << 6) | kf_slot(ln);
      kfr[slot] = bf8_to_h(*reinterpret_cast<const u32x2 *>(sk + at), *reinterpret_cast<const u32x2 *>(sk + at + 16));
      qfr[slot] = bf8_to_h(*reinterpret_cast<const u32x2 *>(sq + at), *reinterpret_cast<const u32x2 *>(sq + at + 16));
    }
  }
  // K K^T, the 10 lower 16x16 tiles (wave w: tiles w, w + 4, w + 8), kept in registers.
  f32x4 gt[3];
  int tmi[3], tni[3];
#pragma unroll
  for (int qq = 0; qq < 3; ++qq) {
    const int t = w + 4 * qq;
    const int mi = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
    const int ni = t - mi * (mi + 1) / 2;
    tmi[qq] = mi;
    tni[qq] = ni;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    if (t < 10) {
      const uint16_t *Ab = sk + (mi * 16 + lr) * LDK + 8 * lg, *Bb = sk + (ni * 16 + lr) * LDK + 8 * lg;
#pragma unroll
      for (int k0 = 0; k0 < DK; k0 += 32)
        a = mfma_bf16(*reinterpret_cast<const bf16x8 *>(Ab + k0), *reinterpret_cast<const bf16x8 *>(Bb + k0), a);
    }
    gt[qq] = a;
  }
  // For split head-wide chains, K Q^T for P: wave w takes query tile m = w, key tiles ni <= m:
  // D(ni, m) holds, in lane l, query 16m + l%16 at keys 16ni + 4g + i, the A operand of
  // P U once the key tiles are paired (2s, 2s + 1).
  f32x4 gp[4];
#pragma unroll
  for (int ni = 0; ni < 4; ++ni) gp[ni] = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (WP) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      if (ni <= w) {
        const uint16_t *Ab = sk + (ni * 16 + lr) * LDK + 8 * lg, *Bb = sq + (w * 16 + lr) * LDK + 8 * lg;
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += 32)
          gp[ni] = mfma_bf16(*reinterpret_cast<const bf16x8 *>(Ab + k0), *reinterpret_cast<const bf16x8 *>(Bb + k0), gp[ni]);
      }
    }
  }
  __syncthreads();  // the key and query rows are dead: ra holds A and rt holds T from here

  for (int rr = 0; rr < R; ++rr) {
    const int h = j * R + rr;
    unsigned char *slot = tt + ((int64_t)h * MC + c) * kTBytes;
    if (w == 3) {
      // Decays: the in-chunk cumulative sum in fp64 (g = -inf floored to a finite
      // reset), then the chain's factors of this value head.
      const double gv = lane < len ? (double)floor_keep_nan(graw, kFloor) : 0.0;
      const double gam = wave_inclusive_scan(gv, lane);
      const double glast = __shfl(gam, len - 1);
      sm.gam[lane] = gam;
      sm.beta[lane] = lane < len ? braw : 0.f;
      float *fac = reinterpret_cast<float *>(slot + kTFragBytes);
      const float eg = fexp((float)gam), rkv = sm.rk[lane], rqv = sm.rq[lane];
      fac[FAC_GL2 * C + lane] = (float)(gam * 1.4426950408889634);
      fac[FAC_EKR * C + lane] = eg * rkv;
      fac[FAC_FKR * C + lane] = lane < len ? fexp((float)(glast - gam)) * rkv : 0.f;
      fac[FAC_EQR * C + lane] = eg * rqv;
      fac[FAC_RK * C + lane] = rkv;
      fac[FAC_RQ * C + lane] = rqv;
      fac[FAC_EL * C + lane] = lane == 0 ? fexp((float)glast) : 0.f;
      fac[(FAC_EL + 1) * C + lane] = 0.f;
      if (rr + 1 < R) load_gb(rr + 1);
    }
    __syncthreads();
    // A[r][i] = beta_r rk_r rk_i e^{G_r - G_i} (k_r . k_i), i < r (zero elsewhere in the
    // diagonal blocks; blocks above the diagonal are never read)
#pragma unroll
    for (int qq = 0; qq < 3; ++qq) {
      if (w + 4 * qq < 10) {
        const int i = 16 * tni[qq] + lr;
        const double gi = sm.gam[i];
        const float rki = sm.rk[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * tmi[qq] + 4 * lg + e;
          A[r * LDF + i] = i < r ? sm.beta[r] * sm.rk[r] * rki * fexp((float)(sm.gam[r] - gi)) * gt[qq][e] : 0.f;
        }
      }
    }
    __syncthreads();
    // T = (I + A)^{-1} of the unit lower-triangular I + A, by blocks of 16.
    // Diagonal blocks by forward substitution: lane 16 b + cc owns column cc of block b.
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
      for (int r = 0; r < 16; ++r) T[(bb * 16 + r) * LDF + bb * 16 + cc] = col[r];
    }
    __syncthreads();
    // Then by the block inverse of a lower-triangular matrix, L21 = -T22 A21 T11:
    // first within the two 32-row halves (waves 0 and 1: blocks (1,0) and (3,2)),
    // then the lower-left 32 x 32 quarter (wave w: block (2 + w/2, w%2)), whose row
    // block 3 takes row block 2's Y = A21 T11 from its wave through LDS.
    if (w < 2) {
      const int ib = 2 * w + 1, jb = 2 * w;
      const f32x4 y = block_mm(A, T, ib, jb, jb, lr, lg, f32x4{0.f, 0.f, 0.f, 0.f});
      const f32x4 t = block_mm_acc(T, ib, ib, y, lr, lg, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int e = 0; e < 4; ++e) T[(16 * ib + 4 * lg + e) * LDF + 16 * jb + lr] = -t[e];
    }
    __syncthreads();
    {
      const int ib = 2 + (w >> 1), jb = w & 1;
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
      for (int m = jb; m < 2; ++m) y = block_mm(A, T, ib, m, jb, lr, lg, y);
      if (ib == 2) sm.y[jb][lane] = y;
      __syncthreads();
      f32x4 t = block_mm_acc(T, ib, ib, y, lr, lg, f32x4{0.f, 0.f, 0.f, 0.f});
      if (ib == 3) t = block_mm_acc(T, 3, 2, sm.y[jb][lane], lr, lg, t);
#pragma unroll
      for (int e = 0; e < 4; ++e) T[(16 * ib + 4 * lg + e) * LDF + 16 * jb + lr] = -t[e];
    }
    __syncthreads();
    // T~ = T diag(beta) as A fragments (row tile m = w, token step s <= m / 2), fp16 hi/lo:
    // lane l: row 16 m + l%16, tokens {32 s + 4g + i, 32 s + 16 + 4g + i}; zero above the diagonal.
    {
      const int m = w, r = 16 * m + lr;
      u32x4 *dst = reinterpret_cast<u32x4 *>(slot);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s <= (m >> 1)) {
          const int i0 = 32 * s + 4 * lg;
          const f32x4 x0 = *reinterpret_cast<const f32x4 *>(T + r * LDF + i0);
          const f32x4 x1 = *reinterpret_cast<const f32x4 *>(T + r * LDF + i0 + 16);
          const f32x4 b0 = *reinterpret_cast<const f32x4 *>(sm.beta + i0);
          const f32x4 b1 = *reinterpret_cast<const f32x4 *>(sm.beta + i0 + 16);
          f32x4 a, b;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = i0 + e <= r ? x0[e] * b0[e] : 0.f;
            b[e] = i0 + 16 + e <= r ? x1[e] * b1[e] : 0.f;
          }
          u32x4 hi, lo;
          split8h(a, b, hi, lo);
          const int f = tri_frag(m, s);
          dst[(2 * f) * 64 + lane] = hi;
          dst[(2 * f + 1) * 64 + lane] = lo;
        }
      }
    }
    // P[r][i] = rq_r rk_i e^{G_r - G_i} (q_r . k_i), i <= r, as fp16 hi/lo A fragments
    // (row tile m = w), for split head-wide chains
    if constexpr (WP) {
      const int m = w, r = 16 * m + lr;
      const double gr = sm.gam[r];
      const float rq = sm.rq[r];
      f32x4 d[4];
#pragma unroll
      for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * ni + 4 * lg + e;
          d[ni][e] = (ni <= m && i <= r) ? rq * sm.rk[i] * fexp((float)(gr - sm.gam[i])) * gp[ni][e] : 0.f;
        }
      }
      u32x4 *dst = reinterpret_cast<u32x4 *>(pf + ((int64_t)h * MC + c) * kPBytes);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s <= (m >> 1)) {
          u32x4 hi, lo;
          split8h(d[2 * s], d[2 * s + 1], hi, lo);
          const int f = tri_frag(m, s);
          dst[(2 * f) * 64 + lane] = hi;
          dst[(2 * f + 1) * 64 + lane] = lo;
        }
      }
    }
    __syncthreads();  // gam, beta, A and T are reused by the next value head
  }
}

// ---------------------------------------------------------------------------
// chain: one (sequence, value head, block of 16 NB columns of S) per workgroup
// of NB + 3 waves, and stream_waves(NB) more with the per-token states streamed here
// (see the head of the file).
// ---------------------------------------------------------------------------
template <int NB> struct ChainStage {
  u32x4 kf[16][64];     // K, A operand of K S and K Q^T: fragment 4m + s, slot kf_slot(l) (copied)
  u32x4 qf[16][64];     // Q, A operand of Q S, B operand of K Q^T: fragment 4m + s, slot kf_slot(l) (copied)
  u32x4 tf[2 * kTriFrags][64];  // T~ hi/lo: fragment 2 tri_frag(m, s) + (0 hi, 1 lo) (copied)
  f32x4 vv[NB][4][64];  // V in accumulator order: column tile, token tile, lane (formed by the copy wave)
  float fac[kFacRows][C];  // the per-token factors (copied): FAC_GL2 ... FAC_EL
};
template <int NB> struct ChainSmem {
  ChainStage<NB> st[2];
  u32x4 sx[2][NB][4][64];  // S at the chunk start, B operand (d_k step s), fp16, double buffered
  f32x4 uf[2][NB][4][64];  // U of a chunk in accumulator order (column tile, token tile), fp32, double buffered
};
// With the per-token states each (column block) runs as kStateHalves blocks, one per
// half of S's d_k rows, whose stream_waves(NB) stream waves step that half of the block's
// 16 NB columns; stream wave w keeps the keys of its rows as pairs, kp[w][t][p] = fp16
// {K[t][2p'], K[t][2p' + 1]} for its p-th pair p' (rows padded by 4 words).
constexpr int kStateHalves = 2;
__host__ __device__ constexpr int stream_waves(int NB) { return NB == 1 ? 2 : 4; }
template <int NB> struct ChainSmemStates : ChainSmem<NB> {
  static constexpr int SW = stream_waves(NB), PW = DK / kStateHalves / 2 / SW;  // waves, key pairs per wave
  uint32_t kp[SW][C][PW + 4];
};

// The per-token states, by mode SM: SM_WRITE writes what the stream kernel expands (each
// chunk's start state into scw, the tokens' write vectors into uw); SM_STREAM streams them
// here: stream_waves(NB) more waves step the block's columns of S token by token,
// S <- e^{g_t} S + k_t u_t^T, from U as the carry publishes it, and store the state
// after every selected token: tl = t_lo + j t_step < t_hi (tl the token's index in
// its row of rowT tokens) to states[row * n_sel + j].
enum { SM_NONE = 0, SM_WRITE = 1, SM_STREAM = 2 };
template <int NB, int SM, bool OBF16>
__global__ __launch_bounds__(64 * (NB + 3 + (SM == SM_STREAM ? stream_waves(NB) : 0))) void chain_kernel(
    const uint16_t *__restrict__ v, const float *__restrict__ s0, const Seqs sq, const unsigned char *__restrict__ tt,
    const unsigned char *__restrict__ kk, int32_t *__restrict__ status, void *__restrict__ o,
    float *__restrict__ fin, float *__restrict__ uw, float *__restrict__ scw, float *__restrict__ states, int H_qk,
    int H_v, int d_v, int MC, int groups, int rowT, int t_lo, int t_hi, int t_step, int n_sel) {
  constexpr bool STATES = SM == SM_STREAM;
  __shared__ std::conditional_t<STATES, ChainSmemStates<NB>, ChainSmem<NB>> sm;
  if (sq.bad()) return;
  const int NCB = d_v / (16 * NB);
  // with the states, each column block runs once per half of S's rows (rh): both carry
  // the state; the first writes o and the final state, each streams its half's states
  constexpr int RH = STATES ? kStateHalves : 1;
  const int u0 = xcd_group_remap(blockIdx.x, RH * NCB * (H_v / H_qk), groups);
  if (u0 < 0) return;
  const int rh = u0 % RH, u = u0 / RH;
  // packed sequences are taken longest first (the plan's order)
  const int jb = u % NCB, h = (u / NCB) % H_v, n = sq.by_length(u / (NCB * H_v));
  const int j = h / (H_v / H_qk);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int col0 = jb * 16 * NB;
  const int c_begin = sq.first(n), c_end = sq.first(n + 1);
  const int s_begin = sq.start(n), s_end = sq.start(n + 1);
  const int nit = c_end - c_begin;
  // Waves are dealt to the CU's four SIMDs in order (wave i on SIMD i % 4): with one
  // carry wave every role has a SIMD of its own.
  const int ROLE_OUT = NB, ROLE_COPY = NB + 2;

  if (wave < NB) {
    // ------------------------------ carry waves ------------------------------
    const int jt = wave, cc = col0 + 16 * jt + lr;
    const int pl = kf_slot(lane);                                                // this lane's fragment slot
    const int tslot = kf_slot(4 * (lane >> 4) + ((lane >> 2) & 3) + 16 * (lane & 3));  // its transposed-read slot
    const int64_t sbase = (int64_t)(n * H_v + h) * DK;
    f32x4 S[8];  // S[mt]: rows 16 mt + 4g + i, column cc
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[mt][i] = s0 ? s0[(sbase + 16 * mt + 4 * lg + i) * d_v + cc] : 0.f;
    }
    u32x4 sb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      sb[s] = h16x8(S[2 * s], S[2 * s + 1]);
      sm.sx[0][jt][s][lane] = sb[s];
    }
    lds_barrier();
    for (int it = 0; it < nit; ++it) {
      const ChainStage<NB> &P = sm.st[it & 1];
      const int c = c_begin + it;
      if constexpr (SM == SM_WRITE) {
        // the state at the chunk start
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            scw[(((int64_t)c * H_v + h) * DK + 16 * mt + 4 * lg + i) * d_v + cc] = S[mt][i];
      }
      // K's fragments for K S, then the K^T fragments of K^T U'' (below), read now so
      // that their latency passes under K S and T~ X.  Fragment (mt, st): lane (g, r) holds K[32 st + 4g + i][16 mt
      // + r] and K[32 st + 16 + 4g + i][16 mt + r], i < 4: two transposed reads of the K
      // fragments, where lane (g, 4e + q) of its group addresses token 32 st (+16) + 4g
      // + e at d_k 16 mt + 4q, i.e. K fragment 4(2 st (+1)) + mt/2, lane 4g + e + 16q,
      // half mt%2.
      // (With the per-token states the store stream sets the pace: the fragments are
      // read where they are used, leaving registers for more stream waves.)
      auto ktr = [&](int mt, int st) {
        const unsigned char *b = reinterpret_cast<const unsigned char *>(&P.kf[8 * st + (mt >> 1)][tslot]) + 8 * (mt & 1);
        const u32x2 lo = lds_read_tr16(b), hi = lds_read_tr16(b + 4 * 64 * 16);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      u32x4 kfr[16];
      u32x4 ktf[8][2];
      if constexpr (!STATES) {
#pragma unroll
        for (int f = 0; f < 16; ++f) kfr[f] = P.kf[f][pl];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int st = 0; st < 2; ++st) ktf[mt][st] = ktr(mt, st);
        __builtin_amdgcn_sched_barrier(0);
      }
      // K S: token tile m, four d_k steps
      f32x4 ks[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) ks[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int m = 0; m < 4; ++m) ks[m] = mfma_h(STATES ? P.kf[4 * m + s][pl] : kfr[4 * m + s], sb[s], ks[m]);
      // X = V - diag(e^G rk) K S
      f32x4 x[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 e = *reinterpret_cast<const f32x4 *>(&P.fac[FAC_EKR][16 * m + 4 * lg]);
        x[m] = P.vv[jt][m][lane] - e * ks[m];
      }
      u32x4 xh0, xl0, xh1, xl1;
      split8h(x[0], x[1], xh0, xl0);
      split8h(x[2], x[3], xh1, xl1);
      // U = T~ X (lower triangular: token tile m needs steps s <= m / 2)
      f32x4 uacc[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int f0 = 2 * tri_frag(m, 0);
        f32x4 a = mfma_h(P.tf[f0][lane], xh0, f32x4{0.f, 0.f, 0.f, 0.f});
        a = mfma_h(P.tf[f0][lane], xl0, a);
        a = mfma_h(P.tf[f0 + 1][lane], xh0, a);
        if (m >= 2) {
          const int f1 = 2 * tri_frag(m, 1);
          a = mfma_h(P.tf[f1][lane], xh1, a);
          a = mfma_h(P.tf[f1][lane], xl1, a);
          a = mfma_h(P.tf[f1 + 1][lane], xh1, a);
        }
        uacc[m] = a;
      }
      // publish U (fp32) for the output (and stream) waves' next iteration
#pragma unroll
      for (int m = 0; m < 4; ++m) sm.uf[it & 1][jt][m][lane] = uacc[m];
      if constexpr (SM == SM_WRITE) {
        // the tokens' write vectors, rows t0 .. t0 + len
        const int t0 = s_begin + it * C;
        const int len = min(C, s_end - t0);
        const auto rs = rows_rsrc(uw + (int64_t)t0 * H_v * d_v, (int64_t)len * H_v * d_v * 4);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(uacc[m][i]), rs,
                                                  (((16 * m + 4 * lg + i) * H_v + h) * d_v + cc) * 4, 0, 0);
      }
      // U'' = diag(e^{G_last - G} rk) U as fp16 hi/lo
      f32x4 u2[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        u2[m] = uacc[m] * *reinterpret_cast<const f32x4 *>(&P.fac[FAC_FKR][16 * m + 4 * lg]);
      }
      u32x4 uh0, ul0, uh1, ul1;
      split8h(u2[0], u2[1], uh0, ul0);
      split8h(u2[2], u2[3], uh1, ul1);
      // S <- e^{G_last} S + K^T U'' (the decayed state seeds the accumulator)
      const float el = P.fac[FAC_EL][0];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const u32x4 k0 = STATES ? ktr(mt, 0) : ktf[mt][0], k1 = STATES ? ktr(mt, 1) : ktf[mt][1];
        f32x4 a = S[mt] * el;
        a = mfma_h(k0, uh0, a);
        a = mfma_h(k0, ul0, a);
        a = mfma_h(k1, uh1, a);
        S[mt] = mfma_h(k1, ul1, a);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sb[s] = h16x8(S[2 * s], S[2 * s + 1]);
        sm.sx[(it + 1) & 1][jt][s][lane] = sb[s];
      }
      lds_barrier();
    }
    if (fin && rh == 0) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) fin[(sbase + 16 * mt + 4 * lg + i) * d_v + cc] = S[mt][i];
    }
    // a non-finite final state flags the call (an fp16 overflow of any carried operand ends here)
    bool bad = false;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) bad |= !__builtin_isfinite(S[mt][i]);
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(status, 2);
  } else if (wave < ROLE_COPY) {
    // ------------------------------ output waves -----------------------------
    // Wave 0 takes token tiles {0, 3}, wave 1 {1, 2}: five K Q^T tiles each.  The
    // tiles are compile-time constants of each wave's code path.  Iteration it forms
    // chunk it's P and Q S into registers, and finishes chunk it-1 with P U from the
    // U the carry waves published before the barrier.
    bool bad = false;
    const int fs = kf_slot(lane);  // this lane's fragment slot
    auto out_role = [&](auto m0c, auto m1c) {
      constexpr int M0 = decltype(m0c)::value, M1 = decltype(m1c)::value;
      constexpr int esz = OBF16 ? 2 : 4;
      u32x4 ph[2][2], pl[2][2];   // P of the pending chunk, fp16 hi/lo (token tile, key step)
      f32x4 qs[2][NB];            // its diag(e^G rq) Q S
      int pt0 = 0, plen = 0;      // its first token and length
      // o = diag(e^G rq) Q S + P U for the pending chunk, from U in buffer ub
      auto finish = [&](int ub) {
        const auto rs = rows_rsrc(o ? static_cast<unsigned char *>(o) + (int64_t)pt0 * H_v * d_v * esz : nullptr,
                                  o ? (int64_t)plen * H_v * d_v * esz : 0);
#pragma unroll
        for (int jt = 0; jt < NB; ++jt) {
          u32x4 uh[2], ul[2];
#pragma unroll
          for (int s = 0; s < 2; ++s)
            split8h(sm.uf[ub][jt][2 * s][lane], sm.uf[ub][jt][2 * s + 1][lane], uh[s], ul[s]);
#pragma unroll
          for (int a = 0; a < 2; ++a) {
            const int m = a == 0 ? M0 : M1;
            f32x4 acc = qs[a][jt];
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              if (s == 0 || m >= 2) {
                acc = mfma_h(ph[a][s], uh[s], acc);
                acc = mfma_h(ph[a][s], ul[s], acc);
                acc = mfma_h(pl[a][s], uh[s], acc);
              }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) bad |= !__builtin_isfinite(acc[i]);
            // lane: column col0 + 16 jt + l%16, rows 16 m + 4g + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int off = (((16 * m + 4 * lg + i) * H_v + h) * d_v + col0 + 16 * jt + lr) * esz;
              const float xv = acc[i];
              if constexpr (OBF16)
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pk_bf16(xv, 0.f) & 0xffffu), rs, off, 0, kNT);
              else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(xv), rs, off, 0, kNT);
            }
          }
        }
      };
      lds_barrier();
      for (int it = 0; it < nit; ++it) {
        if (it > 0) finish((it - 1) & 1);
        const ChainStage<NB> &P = sm.st[it & 1];
        // P for the two token tiles: D(ni, m) = K_ni Q_m^T holds, in lane l, query row
        // 16 m + l%16 at keys 16 ni + 4g + i: for the pair of key tiles (2 st, 2 st + 1)
        // the A operand of P U in the contraction order.  Scaled rq_r rk_i e^{G_r - G_i}, i <= r.
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int m = a == 0 ? M0 : M1;
          const int r = 16 * m + lr;
          const float gr = P.fac[FAC_GL2][r];
          const float rq = P.fac[FAC_RQ][r];
          f32x4 d[4];
#pragma unroll
          for (int ni = 0; ni < 4; ++ni) {
            d[ni] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (ni <= m) {
#pragma unroll
              for (int s = 0; s < 4; ++s) d[ni] = mfma_h(P.kf[4 * ni + s][fs], P.qf[4 * m + s][fs], d[ni]);
              const f32x4 rkc = *reinterpret_cast<const f32x4 *>(&P.fac[FAC_RK][16 * ni + 4 * lg]);
              const f32x4 gc = *reinterpret_cast<const f32x4 *>(&P.fac[FAC_GL2][16 * ni + 4 * lg]);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int i = 16 * ni + 4 * lg + e;
                d[ni][e] = i <= r ? rq * rkc[e] * __builtin_amdgcn_exp2f(gr - gc[e]) * d[ni][e] : 0.f;
              }
            }
          }
          split8h(d[0], d[1], ph[a][0], pl[a][0]);
          if (m >= 2) split8h(d[2], d[3], ph[a][1], pl[a][1]);
          // diag(e^G rq) Q S for this token tile, every column tile
          const f32x4 eq = *reinterpret_cast<const f32x4 *>(&P.fac[FAC_EQR][16 * m + 4 * lg]);
#pragma unroll
          for (int jt = 0; jt < NB; ++jt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma_h(P.qf[4 * m + s][fs], sm.sx[it & 1][jt][s][lane], acc);
            qs[a][jt] = acc * eq;
          }
        }
        pt0 = s_begin + it * C;
        plen = min(C, s_end - pt0);
        lds_barrier();
      }
      if (nit > 0) finish((nit - 1) & 1);
    };
    if (rh != 0) {  // o is the first row half's: here only the barriers
      lds_barrier();
      for (int it = 0; it < nit; ++it) lds_barrier();
    } else if (wave == ROLE_OUT) {
      out_role(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{});
    } else {
      out_role(std::integral_constant<int, 1>{}, std::integral_constant<int, 2>{});
    }
    // rows past a chunk's length hold finite values that are never stored; a
    // non-finite stored row is what the range check reports
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(status, 2);
  } else if (wave == ROLE_COPY) {
    // ------------------------------ copy wave --------------------------------
    // K, Q, T~ fragments and the factors of chunk c into stage b: global -> LDS loads,
    // lane l's 16 bytes to the block's slot l.  Then V in accumulator order, by an
    // identity MFMA (exact) on v's bf16 rows, which this wave loads a chunk ahead (rows
    // past the length read as zeros).
    // A = v's rows (token 16m + l%16, columns 4g .. 4g + 3 in the first half of the
    // step), B selects column n = l%16: D[4g + i][n] = v[16m + 4g + i][n].
    u32x4 vsel;
    {
      uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * lg + e == lr) wv[e >> 1] |= 0x3f80u << (16 * (e & 1));  // bf16 1.0
      vsel = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
    // v's rows of chunk c: two register sets, each in flight across one barrier
    // (plain arrays selected at compile time: a copy between them would wait for the loads)
    u32x2 va0[NB][4], va1[NB][4];
    auto vload = [&](u32x2 (&va)[NB][4], int c) {
      const int t0 = s_begin + (c - c_begin) * C;
      const int len = min(C, s_end - t0);
      const auto rv = rows_rsrc(const_cast<uint16_t *>(v) + (int64_t)t0 * H_v * d_v, (int64_t)len * H_v * d_v * 2);
#pragma unroll
      for (int jt = 0; jt < NB; ++jt)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          va[jt][m] = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                         rv, (((16 * m + lr) * H_v + h) * d_v + col0 + 16 * jt + 4 * lg) * 2, 0, 0));
    };
    // stage b <- chunk c; vcur holds chunk c's v rows, vnext receives chunk c + 1's
    auto prep = [&](int b, int c, u32x2 (&vcur)[NB][4], u32x2 (&vnext)[NB][4]) {
      ChainStage<NB> &S = sm.st[b];
      const u32x4 *ksrc = reinterpret_cast<const u32x4 *>(kk + ((int64_t)j * MC + c) * kKBytes) + lane;
      const u32x4 *tsrc = reinterpret_cast<const u32x4 *>(tt + ((int64_t)h * MC + c) * kTBytes) + lane;
#pragma unroll
      for (int f = 0; f < 16; ++f) lds_copy16(ksrc + f * 64, &S.kf[f][0]);
#pragma unroll
      for (int f = 0; f < 16; ++f) lds_copy16(ksrc + (16 + f) * 64, &S.qf[f][0]);
#pragma unroll
      for (int f = 0; f < 2 * kTriFrags; ++f) lds_copy16(tsrc + f * 64, &S.tf[f][0]);
      static_assert(kFacRows * C * 4 == 2 * 64 * 16, "the factors are two 1 KiB copies");
      lds_copy16(tsrc + 2 * kTriFrags * 64, &S.fac[0][0]);
      lds_copy16(tsrc + (2 * kTriFrags + 1) * 64, &S.fac[4][0]);
      // the next chunk's v rows are issued last: the wait below leaves only them in flight
      if (c + 1 < c_end) {
        vload(vnext, c + 1);
        wait_vm<4 * NB>();
      } else {
        wait_vm<0>();
      }
#pragma unroll
      for (int jt = 0; jt < NB; ++jt)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          S.vv[jt][m][lane] = mfma_bf16(__builtin_bit_cast(bf16x8, u32x4{vcur[jt][m][0], vcur[jt][m][1], 0u, 0u}),
                                        __builtin_bit_cast(bf16x8, vsel), f32x4{0.f, 0.f, 0.f, 0.f});
    };
    if (nit > 0) {
      vload(va0, c_begin);
      prep(0, c_begin, va0, va1);
    }
    lds_barrier();
    // iteration it prepares chunk it + 1 (stage (it + 1) & 1; its v rows in va[(it + 1) & 1])
    for (int it = 0; it < nit; it += 2) {
      if (it + 1 < nit) prep(1, c_begin + it + 1, va1, va0);
      lds_barrier();
      if (it + 1 >= nit) break;
      if (it + 2 < nit) prep(0, c_begin + it + 2, va0, va1);
      lds_barrier();
    }
  } else if constexpr (STATES) {
    // ------------------------------ stream waves -----------------------------
    // The block's 128 x 16 NB slice of S, in fp32, stepped through every token.  Lane
    // l of stream wave w owns RPL consecutive rows at columns col0 + 4cq .. + 3 (cq =
    // l % CQ), so that each store instruction writes whole 16 NB-column row segments
    // (a 128-byte line at NB = 2).  Iteration it steps through chunk it - 1, with the
    // U the carry published in the previous iteration (one chunk behind, as the output
    // waves), then copies chunk it's keys (the stage's exact fp16 K fragments), decays
    // e^{g_t} and key norms out of the stage: each wave into its own key region, so
    // stepping and copying need no order between the waves.
    constexpr int SW = stream_waves(NB), CQ = 4 * NB, RR = 64 / CQ, WR = DK / RH / SW, RPL = WR / RR;
    static_assert(RPL % 2 == 0 && RPL <= 8 && WR % 16 == 0, "a lane's rows are whole key pairs");
    const int sw = wave - (ROLE_COPY + 1);
    const int cq = lane % CQ, rr = lane / CQ;
    const int rb = DK / RH * rh + WR * sw;  // this wave's rows rb .. rb + WR
    const int row0 = rb + RPL * rr;         // the lane's first row; its pairs start at pl0 in its wave's region
    const int pl0 = RPL / 2 * rr;
    f32x4 Sr[RPL];
#pragma unroll
    for (int e = 0; e < RPL; ++e) {
      Sr[e] = s0 ? *reinterpret_cast<const f32x4 *>(s0 + ((int64_t)(n * H_v + h) * DK + row0 + e) * d_v + col0 + 4 * cq)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // e^{g_t} and rk_t of token t = lane: the chunk being copied and the one being stepped
    float al_next = 0.f, rk_next = 0.f, al_cur = 0.f, rk_cur = 0.f;
    auto capture = [&](int it) {
      const ChainStage<NB> &P = sm.st[it & 1];
      // this wave's rows rb .. rb + WR, 16 at a time (row block h16 = 2 st + half):
      // lane (g, r) of fragment (m, st) holds token 16m + r at d_k 32st + 4g + i (words
      // 0, 1) and 32st + 16 + 4g + i (words 2, 3), i.e. in words 2 half, 2 half + 1 the
      // pairs of rows 16 h16 + 4g, 16 h16 + 4g + 2
      const int r = lane & 15, g = lane >> 4;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int hb = 0; hb < WR / 16; ++hb) {
          const int h16 = rb / 16 + hb, st = h16 >> 1, half = h16 & 1;
          const u32x4 x = P.kf[4 * m + st][kf_slot(lane)];
          *reinterpret_cast<u32x2 *>(&sm.kp[sw][16 * m + r][8 * hb + 2 * g]) =
              half ? u32x2{x[2], x[3]} : u32x2{x[0], x[1]};
        }
      // e^{g_t} as the difference of the cumulative decays (log2 e units), rk_t
      const float gl = P.fac[FAC_GL2][lane], glp = lane > 0 ? P.fac[FAC_GL2][lane - 1] : 0.f;
      al_next = __builtin_amdgcn_exp2f(gl - glp);
      rk_next = P.fac[FAC_RK][lane];
    };
    const float *head0 = states + (int64_t)h * DK * d_v;
    const int64_t sstride = (int64_t)H_v * DK * d_v;  // one token
    const int off0 = (row0 * d_v + col0 + 4 * cq) * 4;
    typedef uint32_t kpair_t __attribute__((ext_vector_type(RPL / 2)));
    // one token: S <- e^{g_t} S + k_t u_t^T on this lane's rows (key pairs kw, fp16)
    auto token = [&](int t, const f32x4 &uu, const kpair_t &kw) {
      const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, al_cur), t));
      const float rkt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rk_cur), t));
#pragma unroll
      for (int e = 0; e < RPL; ++e) {
        const uint32_t w = kw[e / 2];
        const float ke = (float)__builtin_bit_cast(__fp16, (uint16_t)(e % 2 ? w >> 16 : w & 0xffffu)) * rkt;
#pragma unroll
        for (int c = 0; c < 4; ++c) Sr[e][c] = __builtin_fmaf(Sr[e][c], a, ke * uu[c]);
      }
    };
    auto store = [&](const float *dst) {
      const auto rs = rows_rsrc(const_cast<float *>(dst), (int64_t)DK * d_v * 4);
#pragma unroll
      for (int e = 0; e < RPL; ++e)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, Sr[e]), rs, off0 + e * d_v * 4, 0, kNT);
    };
    // U of tokens 4tq .. 4tq + 3 at this lane's columns (token tile tq/4, lane group
    // tq%4: u4[c][i] is token 4tq + i, column 4cq + c) and their key pairs
    auto load4 = [&](int b, int tq, f32x4 (&u4)[4], kpair_t (&k4)[4]) {
#pragma unroll
      for (int c = 0; c < 4; ++c) u4[c] = sm.uf[b][cq >> 2][tq >> 2][16 * (tq & 3) + 4 * (cq & 3) + c];
#pragma unroll
      for (int i = 0; i < 4; ++i) k4[i] = *reinterpret_cast<const kpair_t *>(&sm.kp[sw][4 * tq + i][pl0]);
    };
    auto step_tokens = [&](int it) {
      const int b = it & 1;
      const int t0 = s_begin + it * C;
      const int len = min(C, s_end - t0);
      // the chunk's tokens lie in one row: row brow, in-row indices tl0 .. tl0 + len;
      // the next selected one is tl_sel = t_lo + j t_step (advanced as tokens pass, so
      // the loop divides once per chunk)
      const int brow = t0 / rowT, tl0 = t0 - brow * rowT;
      int j = tl0 <= t_lo ? 0 : (tl0 - t_lo + t_step - 1) / t_step;
      int tl_sel = t_lo + j * t_step;
      const float *dst = head0 + ((int64_t)brow * n_sel + j) * sstride;  // state j's head block
      // every token of a whole chunk kept: no test per token
      const bool all = len == C && t_step == 1 && t_lo <= tl0 && tl0 + C <= t_hi;
      auto group = [&](int tq, const f32x4 (&u4)[4], const kpair_t (&k4)[4]) {
        if (all) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            token(4 * tq + i, f32x4{u4[0][i], u4[1][i], u4[2][i], u4[3][i]}, k4[i]);
            store(dst);
            dst += sstride;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = 4 * tq + i;
            if (t >= len) break;
            token(t, f32x4{u4[0][i], u4[1][i], u4[2][i], u4[3][i]}, k4[i]);
            if (tl0 + t == tl_sel && tl_sel < t_hi) {  // uniform over the block
              store(dst);
              dst += sstride;
              tl_sel += t_step;
            }
          }
        }
      };
      // two register sets, each loaded a group ahead of its use (plain arrays: a copy
      // between them would wait for the loads)
      const int ng = (len + 3) / 4;
      f32x4 ua[4], ub[4];
      kpair_t ka[4], kb[4];
      load4(b, 0, ua, ka);
      for (int tq = 0; tq < ng; tq += 2) {
        if (tq + 1 < ng) load4(b, tq + 1, ub, kb);
        group(tq, ua, ka);
        if (tq + 1 >= ng) break;
        if (tq + 2 < ng) load4(b, tq + 2, ua, ka);
        group(tq + 1, ub, kb);
      }
    };
    lds_barrier();
    for (int it = 0; it < nit; ++it) {
      if (it > 0) step_tokens(it - 1);
      capture(it);  // after the step: the key region holds one chunk
      al_cur = al_next;
      rk_cur = rk_next;
      lds_barrier();
    }
    if (nit > 0) step_tokens(nit - 1);
  }
}

// ---------------------------------------------------------------------------
// wide chain: one (sequence, value head) per workgroup of WC + 1 waves (WC = 8), or,
// for packed sequences of unequal lengths, two workgroups per head with half its
// columns each (WC = 4), for workloads whose sequences x value heads fill every CU
// (d_v = 128).  Column wave w owns one 16-column tile of S and runs, for chunk c,
// both the carry (K S, X, T~ X, K^T U'') and the tile's output diag(e^G rq) Q S + P U
// from its own S and U registers (the output as its transpose, so that each lane
// stores four consecutive columns); wave WC copies chunk c + 1's K, Q, T~ fragments,
// factors and v rows into the other LDS stage and, for whole heads, forms P from K and
// Q there (for split heads the solve forms P and the wave copies it).  One
// barrier per chunk.  A chunk's fragments reach LDS once per workgroup, where the
// narrow chain fetches them once per 16 or 32 columns.  With GATED (whole heads only)
// the output norm is applied here (below).
// ---------------------------------------------------------------------------
constexpr int kWideCols = 8;                  // 16-column tiles of a head (d_v = 128)
constexpr int kTPW = 1;                       // tiles per column wave
constexpr int kWideWaves = kWideCols / kTPW;  // column waves
struct WideStage {
  u32x4 kf[16][64];             // K fragments, slot kf_slot(l) (copied)
  u32x4 qf[16][64];             // Q fragments, slot kf_slot(l) (copied)
  u32x4 tf[2 * kTriFrags][64];  // T~ hi/lo (copied)
  u32x4 pf[2 * kTriFrags][64];  // P hi/lo: fragment 2 tri_frag(m, s) + (0 hi, 1 lo) (copied; formed by the solve)
  u32x4 vr[16][64];             // v rows (bf16): row r's 16-byte chunk k in slot 16 r + (k ^ r % 16) (copied)
  float fac[kFacRows][C];       // the per-token factors (copied)
};
struct WideSmem {
  WideStage st[2];
  float red[2][C][kWideCols];  // gated output: each tile's share of each token's sum of squares
};

// GATED: o is not stored; the kernel writes weight * o / sqrt(mean(o^2) + eps) * silu(z)
// instead, the mean over the head's d_v values.  The tiles' waves leave their shares of
// each chunk's sums of squares in LDS and finish the chunk's output after the barrier
// that closes its step, so the sums need no wait of their own.
template <bool STATES, bool OBF16, bool GATED, int WC>
__global__ __launch_bounds__(64 * (WC + 1)) void wide_kernel(
    const uint16_t *__restrict__ v, const float *__restrict__ s0, const Seqs sq, const unsigned char *__restrict__ tt,
    const unsigned char *__restrict__ kk, const unsigned char *__restrict__ pfw, int32_t *__restrict__ status,
    void *__restrict__ o, float *__restrict__ fin, float *__restrict__ uw, float *__restrict__ scw, int H_qk,
    int H_v, int MC, int groups, const uint16_t *__restrict__ zg, const float *__restrict__ nw, float eps) {
  __shared__ WideSmem sm;
  if (sq.bad()) return;
  constexpr int d_v = 16 * kWideCols;
  // WC column waves per block: the head's columns in NP parts (one block each, on one XCD)
  constexpr int NP = kWideWaves / WC;
  static_assert(NP * WC == kWideWaves && (!GATED || NP == 1), "the gated output needs the whole head in a block");
  // P: formed by the copy wave where a block holds the whole head (its chunks are long enough
  // to hide the work), else formed by the solve and copied
  constexpr bool PIB = NP == 1;
  // (sequence, query/key head) groups of H_v / H_qk value heads, longest sequences first
  const int u0 = xcd_group_remap(blockIdx.x, NP * (H_v / H_qk), groups);
  if (u0 < 0) return;
  const int part = u0 % NP, u = u0 / NP;
  const int h = u % H_v, n = sq.by_length(u / H_v);
  const int j = h / (H_v / H_qk);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int fs = kf_slot(lane);
  const int c_begin = sq.first(n), c_end = sq.first(n + 1);
  const int s_begin = sq.start(n), s_end = sq.start(n + 1);
  const int nit = c_end - c_begin;

  if (wave < WC) {
    // ---------------------------- column waves -------------------------------
    // Wave w owns the kTPW 16-column tiles jt = kTPW (WC part + w) + t; each operand read
    // from LDS feeds all of them.
    const int jw = WC * part + wave;
    const int tslot = kf_slot(4 * (lane >> 4) + ((lane >> 2) & 3) + 16 * (lane & 3));  // transposed-read slot
    const int64_t sbase = (int64_t)(n * H_v + h) * DK;
    int cc[kTPW];
#pragma unroll
    for (int t = 0; t < kTPW; ++t) cc[t] = 16 * (kTPW * jw + t) + lr;
    f32x4 S[kTPW][8];  // S[t][mt]: rows 16 mt + 4g + i, column cc[t]
    u32x4 sb[kTPW][4];
#pragma unroll
    for (int t = 0; t < kTPW; ++t) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[t][mt][i] = s0 ? s0[(sbase + 16 * mt + 4 * lg + i) * d_v + cc[t]] : 0.f;
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) sb[t][s] = h16x8(S[t][2 * s], S[t][2 * s + 1]);
    }
    // v in accumulator order by an identity MFMA on its bf16 rows (token 16m + l%16,
    // columns 4g .. 4g + 3 in the first half of the step; B selects column l%16).
    u32x4 vsel;
    {
      uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * lg + e == lr) wv[e >> 1] |= 0x3f80u << (16 * (e & 1));  // bf16 1.0
      vsel = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
    constexpr int esz = OBF16 ? 2 : 4;
    bool bad = false;
    // gated output: this lane's 4 columns of the tile, their gains, and the o and z of
    // the chunk whose output waits for the barrier that closed its step
    const int c0 = 16 * kTPW * jw + 4 * lg;
    f32x4 wg = {0.f, 0.f, 0.f, 0.f};
    if constexpr (GATED) wg = *reinterpret_cast<const f32x4 *>(nw + c0);
    f32x4 ok[4] = {};
    u32x2 zk[4] = {};
    // Chunk it's normed output.  It runs inside step it + 1, between U = T~ X and that
    // chunk's output stage (which overwrites ok and zk), without a branch around it so
    // that its arithmetic can interleave with the step's MFMAs; `live` false (no chunk
    // before the first) stores nothing: the row range is empty.
    auto finish = [&](int it, bool live) {
      const int t0 = s_begin + it * C;
      const int len = live ? min(C, s_end - t0) : 0;
      // token 16g + l%16 = lane: its sum of squares over the head, then 1 / RMS
      const f32x4 ra = *reinterpret_cast<const f32x4 *>(&sm.red[it & 1][lane][0]);
      const f32x4 rb = *reinterpret_cast<const f32x4 *>(&sm.red[it & 1][lane][4]);
      const float tot = ((ra[0] + ra[1]) + (ra[2] + ra[3])) + ((rb[0] + rb[1]) + (rb[2] + rb[3]));
      const float inv = rsqrtf(tot * (1.0f / d_v) + eps);
      const auto ro = rows_rsrc(o && live ? static_cast<unsigned char *>(o) + (int64_t)t0 * H_v * d_v * esz : nullptr,
                                o ? (int64_t)len * H_v * d_v * esz : 0);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float r = lane_read(inv, 16 * m + lr);  // token 16m + l%16
        const f32x4 zf = {__uint_as_float(zk[m][0] << 16), __uint_as_float(zk[m][0] & 0xffff0000u),
                          __uint_as_float(zk[m][1] << 16), __uint_as_float(zk[m][1] & 0xffff0000u)};
        f32x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = wg[i] * (ok[m][i] * r) * silu_f(zf[i]);
        bad |= lr < len - 16 * m &&
               !(__builtin_isfinite(y[0]) && __builtin_isfinite(y[1]) && __builtin_isfinite(y[2]) && __builtin_isfinite(y[3]));
        store_o4<OBF16>(ro, (((16 * m + lr) * H_v + h) * d_v + c0) * esz, y);
      }
    };
    auto step = [&](int it) {
      const int c = c_begin + it;
      const WideStage &P = sm.st[it & 1];
      const int t0 = s_begin + it * C;
      const int len = min(C, s_end - t0);
      if constexpr (STATES) {
        // the state at the chunk start
#pragma unroll
        for (int t = 0; t < kTPW; ++t)
#pragma unroll
          for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              scw[(((int64_t)c * H_v + h) * DK + 16 * mt + 4 * lg + i) * d_v + cc[t]] = S[t][mt][i];
      }
      // K S: token tile m, four d_k steps
      f32x4 ks[kTPW][4];
#pragma unroll
      for (int t = 0; t < kTPW; ++t)
#pragma unroll
        for (int m = 0; m < 4; ++m) ks[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const u32x4 kfr = P.kf[4 * m + s][fs];
#pragma unroll
          for (int t = 0; t < kTPW; ++t) ks[t][m] = mfma_h(kfr, sb[t][s], ks[t][m]);
        }
      // X = V - diag(e^G rk) K S, V: row 16m + l%16, columns 16 jt + 4g .. + 3 (half g%2 of
      // v row chunk 2 jt + g/2) moved to accumulator order
      u32x4 xh[kTPW][2], xl[kTPW][2];
#pragma unroll
      for (int t = 0; t < kTPW; ++t) {
        const int jt = kTPW * jw + t;
        f32x4 x[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int r = 16 * m + lr;
          const u32x2 vr = *reinterpret_cast<const u32x2 *>(
              reinterpret_cast<const unsigned char *>(&P.vr[0][0]) + (16 * r + ((2 * jt + (lg >> 1)) ^ lr)) * 16 +
              8 * (lg & 1));
          const f32x4 vv = mfma_bf16(__builtin_bit_cast(bf16x8, u32x4{vr[0], vr[1], 0u, 0u}),
                                     __builtin_bit_cast(bf16x8, vsel), f32x4{0.f, 0.f, 0.f, 0.f});
          const f32x4 e = *reinterpret_cast<const f32x4 *>(&P.fac[FAC_EKR][16 * m + 4 * lg]);
          x[m] = vv - e * ks[t][m];
        }
        split8h(x[0], x[1], xh[t][0], xl[t][0]);
        split8h(x[2], x[3], xh[t][1], xl[t][1]);
      }
      // U = T~ X (lower triangular: token tile m needs steps s <= m / 2)
      f32x4 uacc[kTPW][4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int t = 0; t < kTPW; ++t) uacc[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (s == 0 || m >= 2) {
            const int f = 2 * tri_frag(m, s);
            const u32x4 th = P.tf[f][lane], tl = P.tf[f + 1][lane];
#pragma unroll
            for (int t = 0; t < kTPW; ++t) {
              uacc[t][m] = mfma_h(th, xh[t][s], uacc[t][m]);
              uacc[t][m] = mfma_h(th, xl[t][s], uacc[t][m]);
              uacc[t][m] = mfma_h(tl, xh[t][s], uacc[t][m]);
            }
          }
        }
      }
      if constexpr (STATES) {
        // the tokens' write vectors, rows t0 .. t0 + len
        const auto rs = rows_rsrc(uw + (int64_t)t0 * H_v * d_v, (int64_t)len * H_v * d_v * 4);
#pragma unroll
        for (int t = 0; t < kTPW; ++t)
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float xv = uacc[t][m][i];
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(xv), rs,
                                                    (((16 * m + 4 * lg + i) * H_v + h) * d_v + cc[t]) * 4, 0, 0);
            }
      }
      if constexpr (GATED) finish(it - 1, it > 0);  // the previous chunk's normed output
      // The output first (its registers are free again for the state update):
      // o = diag(e^G rq) Q S + P U for these tiles, as its transpose (S^T Q^T + U^T P^T:
      // the same fragments with the MFMA operands swapped), so that lane (g, l%16) holds
      // token 16m + l%16 at the tile's columns 4g .. 4g + 3.
      u32x4 pu_h[kTPW][2], pu_l[kTPW][2];
#pragma unroll
      for (int t = 0; t < kTPW; ++t) {
        split8h(uacc[t][0], uacc[t][1], pu_h[t][0], pu_l[t][0]);
        split8h(uacc[t][2], uacc[t][3], pu_h[t][1], pu_l[t][1]);
      }
      f32x4 ot[kTPW][4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int t = 0; t < kTPW; ++t) ot[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u32x4 qf = P.qf[4 * m + s][fs];
#pragma unroll
          for (int t = 0; t < kTPW; ++t) ot[t][m] = mfma_h(sb[t][s], qf, ot[t][m]);
        }
        const float eq = P.fac[FAC_EQR][16 * m + lr];
#pragma unroll
        for (int t = 0; t < kTPW; ++t) ot[t][m] = ot[t][m] * eq;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (s == 0 || m >= 2) {
            const int f = 2 * tri_frag(m, s);
            const u32x4 ph = P.pf[f][lane], pl = P.pf[f + 1][lane];
#pragma unroll
            for (int t = 0; t < kTPW; ++t) {
              ot[t][m] = mfma_h(pu_h[t][s], ph, ot[t][m]);
              ot[t][m] = mfma_h(pu_l[t][s], ph, ot[t][m]);
              ot[t][m] = mfma_h(pu_h[t][s], pl, ot[t][m]);
            }
          }
        }
      }
      if constexpr (GATED) {
        static_assert(kTPW == 1, "the gated output is kept for one tile per wave");
        // Kept for the norm after this step's closing barrier: o (ot), the gate z of the
        // same elements, and this tile's share of each token's sum of squares in
        // red[it % 2][token][tile] -- summed over the lane's 4 columns, then over the 4
        // lane groups (lanes l, l ^ 16, l ^ 32); lane (g, l%16) writes token 16g + l%16.
        const auto rz = rows_rsrc(const_cast<uint16_t *>(zg) + (int64_t)t0 * H_v * d_v, (int64_t)len * H_v * d_v * 2);
        f32x4 sq;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          zk[m] = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_raw_buffer_load_b64(rz, (((16 * m + lr) * H_v + h) * d_v + c0) * 2, 0, 0));
          ok[m] = ot[0][m];
          sq[m] = ot[0][m][0] * ot[0][m][0] + ot[0][m][1] * ot[0][m][1] + ot[0][m][2] * ot[0][m][2] +
                  ot[0][m][3] * ot[0][m][3];
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) sq[m] += lane_read(sq[m], lane ^ 16);
#pragma unroll
        for (int m = 0; m < 4; ++m) sq[m] += lane_read(sq[m], lane ^ 32);
        sm.red[it & 1][lane][wave] = lg == 0 ? sq[0] : lg == 1 ? sq[1] : lg == 2 ? sq[2] : sq[3];
      } else {
        const auto ro = rows_rsrc(o ? static_cast<unsigned char *>(o) + (int64_t)t0 * H_v * d_v * esz : nullptr,
                                  o ? (int64_t)len * H_v * d_v * esz : 0);
#pragma unroll
        for (int t = 0; t < kTPW; ++t)
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            bad |= lr < len - 16 * m && !(__builtin_isfinite(ot[t][m][0]) && __builtin_isfinite(ot[t][m][1]) &&
                                            __builtin_isfinite(ot[t][m][2]) && __builtin_isfinite(ot[t][m][3]));
            store_o4<OBF16>(ro, (((16 * m + lr) * H_v + h) * d_v + 16 * (kTPW * jw + t) + 4 * lg) * esz, ot[t][m]);
          }
      }
      // U'' = diag(e^{G_last - G} rk) U and S <- e^{G_last} S + K^T U''
      u32x4 uh[kTPW][2], ul[kTPW][2];
#pragma unroll
      for (int t = 0; t < kTPW; ++t) {
        f32x4 u2[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          u2[m] = uacc[t][m] * *reinterpret_cast<const f32x4 *>(&P.fac[FAC_FKR][16 * m + 4 * lg]);
        split8h(u2[0], u2[1], uh[t][0], ul[t][0]);
        split8h(u2[2], u2[3], uh[t][1], ul[t][1]);
      }
      // The K^T fragment (mt, st) by two transposed reads of the K fragments: lane
      // (g, 4e + q) of a group addresses token 32 st (+16) + 4g + e at d_k 16 mt + 4q,
      // i.e. K fragment 4(2 st (+1)) + mt/2, lane 4g + e + 16q, half mt%2.
      auto ktf = [&](int mt, int st) {
        const unsigned char *b = reinterpret_cast<const unsigned char *>(&P.kf[8 * st + (mt >> 1)][tslot]) + 8 * (mt & 1);
        const u32x2 lo = lds_read_tr16(b), hi = lds_read_tr16(b + 4 * 64 * 16);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      const float el = P.fac[FAC_EL][0];
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const u32x4 k0 = ktf(mt, 0), k1 = ktf(mt, 1);
#pragma unroll
        for (int t = 0; t < kTPW; ++t) {
          f32x4 a = S[t][mt] * el;
          a = mfma_h(k0, uh[t][0], a);
          a = mfma_h(k0, ul[t][0], a);
          a = mfma_h(k1, uh[t][1], a);
          S[t][mt] = mfma_h(k1, ul[t][1], a);
        }
      }
#pragma unroll
      for (int t = 0; t < kTPW; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) sb[t][s] = h16x8(S[t][2 * s], S[t][2 * s + 1]);
      lds_barrier();
    };
    lds_barrier();
    for (int it = 0; it < nit; ++it) step(it);
    if constexpr (GATED) {
      if (nit > 0) finish(nit - 1, true);
    }
    if (fin) {
#pragma unroll
      for (int t = 0; t < kTPW; ++t)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) fin[(sbase + 16 * mt + 4 * lg + i) * d_v + cc[t]] = S[t][mt][i];
    }
    // a non-finite stored o or final state flags the call (an fp16 overflow of a carried operand)
#pragma unroll
    for (int t = 0; t < kTPW; ++t)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) bad |= !__builtin_isfinite(S[t][mt][i]);
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) atomicOr(status, 2);
  } else {
    // ------------------------------ copy wave --------------------------------
    // K, Q, T~, P fragments, the factors and the v rows of chunk c into stage b: global
    // -> LDS loads, lane l's 16 bytes to the block's slot l.
    auto prep = [&](int b, int c) {
      WideStage &S = sm.st[b];
      const u32x4 *ksrc = reinterpret_cast<const u32x4 *>(kk + ((int64_t)j * MC + c) * kKBytes) + lane;
      const u32x4 *tsrc = reinterpret_cast<const u32x4 *>(tt + ((int64_t)h * MC + c) * kTBytes) + lane;
#pragma unroll
      for (int f = 0; f < 16; ++f) lds_copy16(ksrc + f * 64, &S.kf[f][0]);
#pragma unroll
      for (int f = 0; f < 16; ++f) lds_copy16(ksrc + (16 + f) * 64, &S.qf[f][0]);
#pragma unroll
      for (int f = 0; f < 2 * kTriFrags; ++f) lds_copy16(tsrc + f * 64, &S.tf[f][0]);
      if constexpr (!PIB) {
        const u32x4 *psrc = reinterpret_cast<const u32x4 *>(pfw + ((int64_t)h * MC + c) * kPBytes) + lane;
#pragma unroll
        for (int f = 0; f < 2 * kTriFrags; ++f) lds_copy16(psrc + f * 64, &S.pf[f][0]);
      }
      lds_copy16(tsrc + 2 * kTriFrags * 64, &S.fac[0][0]);
      lds_copy16(tsrc + (2 * kTriFrags + 1) * 64, &S.fac[4][0]);
      // v rows: instruction f, lane l -> row 4f + l/16, slot l%16, which holds the row's
      // chunk (l%16) ^ (row % 16); rows past the length repeat its last row (their
      // products are zero: T~ has no entries there and the factors are zero)
      {
        const int t0 = s_begin + (c - c_begin) * C;
        const int len = min(C, s_end - t0);
#pragma unroll
        for (int f = 0; f < 16; ++f) {
          const int row = 4 * f + (lane >> 4), r = min(row, len - 1), k = (lane & 15) ^ (row & 15);
          lds_copy16(reinterpret_cast<const unsigned char *>(v) + (((int64_t)(t0 + r) * H_v + h) * d_v + 8 * k) * 2,
                     &S.vr[f][0]);
        }
      }
      wait_vm<0>();
      if constexpr (!PIB) return;
      // P of chunk c from its K and Q fragments (now in the stage): for query tile m, the Gram
      // K_ni Q_m^T of key tiles ni <= m holds, in lane l, query row 16m + l%16 at keys 16ni +
      // 4g + i; scaled by rq_r rk_i e^{G_r - G_i} (i <= r, else zero) it is, as fp16 hi/lo,
      // the A operand of P U for key steps s <= m / 2
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int r = 16 * m + lr;
        const float gr = S.fac[FAC_GL2][r], rq = S.fac[FAC_RQ][r];
        u32x4 qf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[s] = S.qf[4 * m + s][fs];
        f32x4 d[4];
#pragma unroll
        for (int ni = 0; ni < 4; ++ni) {
          d[ni] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (ni <= m) {
#pragma unroll
            for (int s = 0; s < 4; ++s) d[ni] = mfma_h(S.kf[4 * ni + s][fs], qf[s], d[ni]);
            const f32x4 rkc = *reinterpret_cast<const f32x4 *>(&S.fac[FAC_RK][16 * ni + 4 * lg]);
            const f32x4 gc = *reinterpret_cast<const f32x4 *>(&S.fac[FAC_GL2][16 * ni + 4 * lg]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 16 * ni + 4 * lg + e;
              d[ni][e] = i <= r ? rq * rkc[e] * __builtin_amdgcn_exp2f(gr - gc[e]) * d[ni][e] : 0.f;
            }
          }
        }
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          if (st <= (m >> 1)) {
            u32x4 hi, lo;
            split8h(d[2 * st], d[2 * st + 1], hi, lo);
            const int f = tri_frag(m, st);
            S.pf[2 * f][lane] = hi;
            S.pf[2 * f + 1][lane] = lo;
          }
        }
      }
    };
    if (nit > 0) prep(0, c_begin);
    lds_barrier();
    for (int it = 0; it < nit; ++it) {
      if (it + 1 < nit) prep((it + 1) & 1, c_begin + it + 1);
      lds_barrier();
    }
  }
}

template <bool STATES, bool OBF16, bool GATED, int WC>
hipError_t launch_wide(const Problem &p, const ChunkArgs &a, const Seqs &sq, hipStream_t st) {
  const Workspace &w = a.ws;
  const int groups = p.N * p.H_qk;
  if (groups == 0) return hipSuccess;
  const int grid = xcd_group_grid(kWideWaves / WC * (p.H_v / p.H_qk), groups);
  hipLaunchKernelGGL((wide_kernel<STATES, OBF16, GATED, WC>), dim3(grid), dim3(64 * (WC + 1)), 0, st,
                     static_cast<const uint16_t *>(a.v), a.s0, sq, w.tt, w.kk, w.pf, w.status, a.o, a.final_state,
                     w.u, w.sc, p.H_qk, p.H_v, p.max_chunks, groups, static_cast<const uint16_t *>(a.z), a.nw,
                     a.eps);
  return hipGetLastError();
}

template <int NB, int SM, bool OBF16>
hipError_t launch_chain(const Problem &p, const ChunkArgs &a, const Seqs &sq, hipStream_t st) {
  constexpr bool STATES = SM == SM_STREAM;
  const Workspace &w = a.ws;
  const int groups = p.N * p.H_qk, ncb = p.d_v / (16 * NB);
  if (groups == 0 || ncb == 0) return hipSuccess;
  const int rowT = p.packed ? p.T_tot : p.T;
  const int grid = xcd_group_grid((STATES ? kStateHalves : 1) * ncb * (p.H_v / p.H_qk), groups);
  hipLaunchKernelGGL((chain_kernel<NB, SM, OBF16>), dim3(grid), dim3(64 * (NB + 3 + (STATES ? stream_waves(NB) : 0))),
                     0, st, static_cast<const uint16_t *>(a.v), a.s0, sq, w.tt, w.kk, w.status, a.o, a.final_state,
                     w.u, w.sc, a.states, p.H_qk, p.H_v, p.d_v, p.max_chunks, groups, rowT, a.t_lo, a.t_hi, a.t_step, a.n_sel);
  return hipGetLastError();
}

// Compute units of the current device (looked up once per device).
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cached[dev] = n;
  return n;
}

template <bool STATES, bool OBF16>
hipError_t run_fused(const Problem &p, const ChunkArgs &a, hipStream_t st) {
  const Workspace &w = a.ws;
  mark_event(a, 0, st);
  hipError_t e;
  const bool dense = dense_rows(p);
  if (!dense && (e = launch_plan(p, a, st)) != hipSuccess) return e;
  mark_event(a, 1, st);
  const Seqs sq{w.status, w.seq_start, w.chunk_first, p.N, dense ? p.T : 0, dense ? ceil_div(p.T, C) : 0, w.order};
  if (p.max_chunks > 0 && p.H_qk > 0) {
    const dim3 sgrid(xcd_group_grid(p.H_qk, p.max_chunks));
    if (w.pf)
      hipLaunchKernelGGL(solve_kernel<true>, sgrid, dim3(256), 0, st, static_cast<const uint16_t *>(a.q),
                         static_cast<const uint16_t *>(a.k), a.g, a.beta, sq, w.status, w.tt, w.kk, w.pf, p.H_qk,
                         p.H_v, p.max_chunks, p.scale, p.l2norm ? 1 : 0);
    else
      hipLaunchKernelGGL(solve_kernel<false>, sgrid, dim3(256), 0, st, static_cast<const uint16_t *>(a.q),
                         static_cast<const uint16_t *>(a.k), a.g, a.beta, sq, w.status, w.tt, w.kk, w.pf, p.H_qk,
                         p.H_v, p.max_chunks, p.scale, p.l2norm ? 1 : 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  mark_event(a, 2, st);
  // A whole value head per workgroup once sequences x value heads fill every CU;
  // else two column tiles per workgroup (their carries share the stage and P) once
  // the single-tile grid would fill every CU twice over; one below that.
  // The per-token states: streamed by the chain itself when at least half of each row's
  // tokens are kept (32-column blocks where d_v allows, whose state rows are whole
  // 128-byte lines); else, and behind the head-wide chain, the chain writes the chunk-start
  // states and write vectors and the stream kernel expands only the chunks and tokens
  // that the selection needs.
  const long blocks1 = (long)p.N * p.H_v * (p.d_v / 16);
  const bool wide = fused_wide(p);
  const bool in_chain = STATES && !wide && 2L * a.n_sel >= (p.packed ? p.T_tot : p.T);
  const bool two = p.d_v % 32 == 0 && (in_chain || blocks1 >= 2L * cu_count());
  if (wide) {
    // Packed sequences of unequal lengths: each head in two blocks of half its columns,
    // so that a chunk of the longest sequences takes less time and the shorter
    // sequences' blocks fill the CUs (the norm needs the whole head in one block)
    if (!STATES && a.z)
      e = launch_wide<false, OBF16, true, kWideWaves>(p, a, sq, st);
    else if (p.packed)
      e = launch_wide<STATES, OBF16, false, kWideWaves / 2>(p, a, sq, st);
    else
      e = launch_wide<STATES, OBF16, false, kWideWaves>(p, a, sq, st);
  } else if constexpr (STATES) {
    if (in_chain)
      e = two ? launch_chain<2, SM_STREAM, OBF16>(p, a, sq, st) : launch_chain<1, SM_STREAM, OBF16>(p, a, sq, st);
    else
      e = two ? launch_chain<2, SM_WRITE, OBF16>(p, a, sq, st) : launch_chain<1, SM_WRITE, OBF16>(p, a, sq, st);
  } else {
    e = two ? launch_chain<2, SM_NONE, OBF16>(p, a, sq, st) : launch_chain<1, SM_NONE, OBF16>(p, a, sq, st);
  }
  if (e != hipSuccess) return e;
  mark_event(a, 3, st);
  if constexpr (STATES) {
    if (!in_chain && (e = launch_states_stream(p, a, sq, st)) != hipSuccess) return e;
    mark_event(a, 4, st);
  }
  return hipSuccess;
}

}  // namespace

size_t fused_t_bytes() { return kTBytes; }
size_t fused_p_bytes() { return kPBytes; }
bool fused_wide(const Problem &p) {
  return p.dtype == GDN_BF16 && p.C == C && p.d_k == DK && p.d_v == 16 * kWideCols &&
         (long)p.N * p.H_v >= cu_count();
}
bool fused_solve_p(const Problem &p) { return fused_wide(p) && p.packed; }
size_t fused_k_bytes() { return kKBytes; }

hipError_t launch_fused_path(const Problem &p, const ChunkArgs &a, bool states, hipStream_t st) {
  if (p.d_k != DK || p.C != C || p.d_v % 16 != 0 || p.d_v > 128) return hipErrorInvalidValue;
  const bool ob = p.o_dtype == GDN_BF16;
  if (states) return ob ? run_fused<true, true>(p, a, st) : run_fused<true, false>(p, a, st);
  return ob ? run_fused<false, true>(p, a, st) : run_fused<false, false>(p, a, st);
}

}  // namespace gdn
