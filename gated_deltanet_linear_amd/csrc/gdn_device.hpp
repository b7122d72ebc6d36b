// Device-side building blocks for libgdn on gfx950 (CDNA4): element types,
// bf16 hi/lo splitting, 16x16 MFMA tile products over LDS operands, and
// wavefront reductions.  Used by every kernel of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // raw 16-byte vector
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));  // raw 8-byte vector

constexpr int kWave = 64;

// A raw buffer resource over `bytes` bytes at p (32-bit data format): buffer
// stores at offsets past the end are dropped by the hardware.  The kernels mask
// rows past a ragged end this way instead of with a branch: a branch around a
// store leaves the compiler unable to count the outstanding vector-memory
// operations past it (it then waits for all of them before the next load is
// used), and a run of stores each behind its own exec-mask branch issues
// measurably slower than the same stores unguarded.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(void *p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, (int)bytes, 0x00020000);
}

// ---------------------------------------------------------------------------
// bf16 <-> f32.  Storage of bf16 data is uint16_t; conversions round to
// nearest even (gfx950's v_cvt_pk_bf16_f32).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t x) {
  return __builtin_bit_cast(float, (uint32_t)x << 16);
}
__device__ __forceinline__ uint16_t f2bf(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
// x == hi + lo + O(2^-17 |x|): hi is x rounded to bf16, lo the rounded residual.
__device__ __forceinline__ void split_bf16(float x, uint16_t &hi, uint16_t &lo) {
  const __bf16 h = (__bf16)x;
  hi = __builtin_bit_cast(uint16_t, h);
  lo = f2bf(x - (float)h);
}

// Element loads of the input tensors (q, k, v): float32 or bf16 storage.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float get(const float *p, int64_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float get(const uint16_t *p, int64_t i) { return bf2f(p[i]); }
};

// ---------------------------------------------------------------------------
// 16x16 output tiles on MFMA.
//
// Accumulator layout (v_mfma_f32_16x16x{4f32,32_bf16}): lane l holds rows
// 4*(l/16) + i, i = 0..3, of column l%16.  Operands are read from LDS with the
// contraction index contiguous: A as [M][lda] (row m of the tile at A + m*lda)
// and B as [N][ldb] (column n of the tile at B + n*ldb).  Lane l feeds row
// l%16 of A and column l%16 of B; the 16 lanes of group l/16 cover one
// contiguous slice of the contraction index.  Which slice a group feeds does
// not matter for the result as long as A and B use the same assignment, which
// both helpers below do.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// acc += A[0:16, 0:kmax) * B[0:kmax, 0:16] with bf16 operands.  A and B each are
// one bf16 array (exact values) or a hi/lo pair (an fp32 value split in two);
// SA / SB say which.  The hi*lo cross terms are summed, lo*lo is dropped.
// K is the compile-time extent; kmax <= K (a multiple of 32) trims the loop
// where the rest of the contraction is known to be zero.
template <int K, bool SA, bool SB>
__device__ __forceinline__ void tile_bf16(f32x4 &acc, const uint16_t *Ah, const uint16_t *Al, int lda,
                                          const uint16_t *Bh, const uint16_t *Bl, int ldb, int lane,
                                          int kmax = K) {
  static_assert(K % 32 == 0, "bf16 MFMA contraction is a multiple of 32");
  const int r = lane & 15, g = lane >> 4;
  const uint16_t *pa = Ah + r * lda + 8 * g;
  const uint16_t *pb = Bh + r * ldb + 8 * g;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 32) {
    if (k0 < kmax) {
      const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(pa + k0);
      const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(pb + k0);
      acc = mfma_bf16(ah, bh, acc);
      if constexpr (SB) {
        const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(Bl + r * ldb + 8 * g + k0);
        acc = mfma_bf16(ah, bl, acc);
      }
      if constexpr (SA) {
        const bf16x8 al = *reinterpret_cast<const bf16x8 *>(Al + r * lda + 8 * g + k0);
        acc = mfma_bf16(al, bh, acc);
      }
    }
  }
}

// acc += A[0:16, 0:kmax) * B[0:kmax, 0:16] with fp32 operands (exact products).
template <int K>
__device__ __forceinline__ void tile_f32(f32x4 &acc, const float *A, int lda, const float *B, int ldb,
                                         int lane, int kmax = K) {
  static_assert(K % 16 == 0, "fp32 MFMA contraction is a multiple of 16");
  const int r = lane & 15, g = lane >> 4;
  const float *pa = A + r * lda + 4 * g;
  const float *pb = B + r * ldb + 4 * g;
#pragma unroll
  for (int k0 = 0; k0 < K; k0 += 16) {
    if (k0 < kmax) {
      const float4 a = *reinterpret_cast<const float4 *>(pa + k0);
      const float4 b = *reinterpret_cast<const float4 *>(pb + k0);
      acc = mfma_f32(a.x, b.x, acc);
      acc = mfma_f32(a.y, b.y, acc);
      acc = mfma_f32(a.z, b.z, acc);
      acc = mfma_f32(a.w, b.w, acc);
    }
  }
}

// ---------------------------------------------------------------------------
// Wavefront helpers.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_xor(float x, int mask) { return __shfl_xor(x, mask, kWave); }

// Inclusive prefix sum over the 64 lanes of a wavefront, in double precision.
__device__ __forceinline__ double wave_inclusive_scan(double x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

// Sequence n owning global chunk c: chunk_first[n] <= c < chunk_first[n+1].
__device__ __forceinline__ int find_seq(const int32_t *chunk_first, int N, int c) {
  int lo = 0, hi = N;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (chunk_first[mid] <= c) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Where sequences and their chunks start.  Dense rows (no cu_seqlens, T > 0):
// row n starts at token n T and its chunks at n ceil(T / C), no tables needed;
// packed rows: the tables and the status word the plan kernel wrote, and
// optionally its order of the sequences by decreasing chunk count.
struct Seqs {
  const int32_t *status, *seq_start, *chunk_first;
  int N;    // sequences
  int T;    // > 0: dense rows of T tokens; 0: use the tables
  int cpr;  // chunks per dense row
  const int32_t *order = nullptr;  // packed rows: sequence of rank i by length (or null)
  // the i-th sequence by decreasing length (dense rows: all alike, the i-th)
  __device__ __forceinline__ int by_length(int i) const { return (T || !order) ? i : order[i]; }
  __device__ __forceinline__ bool bad() const { return T == 0 && *status != 0; }
  __device__ __forceinline__ int chunks() const { return T ? N * cpr : chunk_first[N]; }
  __device__ __forceinline__ int seq_of(int c) const { return T ? c / cpr : find_seq(chunk_first, N, c); }
  __device__ __forceinline__ int first(int n) const { return T ? n * cpr : chunk_first[n]; }
  __device__ __forceinline__ int start(int n) const { return T ? n * T : seq_start[n]; }
};

// blockIdx -> logical work item u = g * per + r, for work made of `groups`
// groups of `per` items that share their operands (the column blocks of the
// value heads of one (sequence, query/key head)).  Workgroups are dealt to the 8 XCDs round robin; this keeps
// each group on one XCD, whose L2 then serves the group's shared reads, and
// deals the groups themselves round robin, so that the first groups in u order
// (the first sequences) spread over every XCD.  The grid is
// 8 ceil(groups / 8) per blocks; padding blocks get -1.
__device__ __forceinline__ int xcd_group_remap(int bid, int per, int groups) {
  const int x = bid & 7, i = bid >> 3;
  const int g = (i / per) * 8 + x;
  return g < groups ? g * per + i % per : -1;
}
inline int xcd_group_grid(int per, int groups) { return (groups + 7) / 8 * 8 * per; }

// max(x, lo) that keeps a NaN a NaN (fmaxf would return lo): the decay floor turns
// g = -inf into a finite reset, while a NaN decay propagates as it does through the
// oracle, the decode step and the states stream.
__device__ __forceinline__ float floor_keep_nan(float x, float lo) { return x < lo ? lo : x; }

// Non-temporal 16-byte store (streamed output that is not read back soon).
__device__ __forceinline__ void store_nt(float4 *p, const float4 &v) {
  __builtin_nontemporal_store(v.x, &p->x);
  __builtin_nontemporal_store(v.y, &p->y);
  __builtin_nontemporal_store(v.z, &p->z);
  __builtin_nontemporal_store(v.w, &p->w);
}

}  // namespace gdn
