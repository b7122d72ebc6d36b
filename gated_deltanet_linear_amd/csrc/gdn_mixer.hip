// The DeltaNet mixer's steps around the delta rule (Qwen3.5 text encyclopedia
// page, note "The DeltaNet mixer"; Qwen3-Next encyclopedia page, same note),
// in this library's notation, for channel c, token t and value head h:
//
//   prologue:  xc[t,c]  = sum_{i<4} w[c,i] x[t-3+i,c]  (causal, one filter per channel)
//              (q|k|v)[t,c] = xc[t,c] sigma(xc[t,c])    channels split q, then k, then v
//              beta[t,h] = sigma(b[t,h]),  g[t,h] = -e^{A_log[h]} ln(1 + e^{a[t,h] + dt_bias[h]})
//   epilogue:  out[t,h,:] = weight * y / sqrt(mean(y^2) + eps) * z sigma(z)
//                           over one value head's d_v outputs y = y[t,h,:], z = z[t,h,:]
//
// All three are elementwise or nearly so, bound by HBM: one pass over their
// inputs and outputs, 16-byte (fp32) or 8-byte (bf16) accesses per lane on
// consecutive channels.  The decode step fuses the epilogue into its own
// kernel (gdn_step.hip); these kernels serve the prompt paths.
#include <algorithm>
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn.h"

namespace gdn {
namespace {

__device__ __forceinline__ f32x4 load4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ f32x4 load4(const uint16_t *p) {
  const u32x2 u = *reinterpret_cast<const u32x2 *>(p);
  return f32x4{bf2f((uint16_t)(u.x & 0xffffu)), bf2f((uint16_t)(u.x >> 16)), bf2f((uint16_t)(u.y & 0xffffu)),
               bf2f((uint16_t)(u.y >> 16))};
}
__device__ __forceinline__ void store4(float *p, const f32x4 &x) { *reinterpret_cast<f32x4 *>(p) = x; }
__device__ __forceinline__ void store4(uint16_t *p, const f32x4 &x) {
  *reinterpret_cast<u32x2 *>(p) = u32x2{(uint32_t)f2bf(x[0]) | ((uint32_t)f2bf(x[1]) << 16),
                                        (uint32_t)f2bf(x[2]) | ((uint32_t)f2bf(x[3]) << 16)};
}
// The same, non-temporal: a final output that nothing reads back soon.
__device__ __forceinline__ void store4_nt(float *p, const f32x4 &x) {
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
}
__device__ __forceinline__ void store4_nt(uint16_t *p, const f32x4 &x) {
  __builtin_nontemporal_store(u32x2{(uint32_t)f2bf(x[0]) | ((uint32_t)f2bf(x[1]) << 16),
                                    (uint32_t)f2bf(x[2]) | ((uint32_t)f2bf(x[3]) << 16)},
                              reinterpret_cast<u32x2 *>(p));
}
// x sigmoid(x) with the hardware reciprocal (1 ulp): a division's exact rounding
// buys nothing for values that are then stored as bf16 or compared at 1e-5.
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// ---------------------------------------------------------------------------
// Gated RMS norm: one row = one (token, value head), DV values; DV/4 lanes per
// row, 4 consecutive values per lane, so a row never spans two waves.
// ---------------------------------------------------------------------------
template <typename TY, typename TZ, int DV>
__global__ __launch_bounds__(256) void gated_norm_kernel(const TY *__restrict__ y, const TZ *__restrict__ z,
                                                         const float *__restrict__ w, float eps, TY *out,
                                                         int64_t rows) {
  constexpr int LPR = DV / 4;
  static_assert(DV % 4 == 0 && 64 % LPR == 0, "a row must sit in one wave");
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = gid / LPR;
  const int c = (int)(gid % LPR) * 4;
  const bool ok = r < rows;
  const f32x4 yv = ok ? load4(y + r * DV + c) : f32x4{0.f, 0.f, 0.f, 0.f};
  float ss = yv[0] * yv[0] + yv[1] * yv[1] + yv[2] * yv[2] + yv[3] * yv[3];
#pragma unroll
  for (int m = 1; m < LPR; m <<= 1) ss += wave_xor(ss, m);  // every lane takes part
  if (!ok) return;
  const float rs = rsqrtf(ss * (1.0f / DV) + eps);
  const f32x4 zv = load4(z + r * DV + c);
  const f32x4 wv = load4(w + c);
  f32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = wv[i] * (yv[i] * rs) * silu(zv[i]);
  store4_nt(out + r * DV + c, o);
}

template <typename TY, typename TZ>
hipError_t launch_norm_t(const Problem &p, const NormArgs &a, hipStream_t st) {
  const int64_t rows = (int64_t)p.T_tot * p.H_v;
  if (rows == 0) return hipSuccess;
  const TY *y = static_cast<const TY *>(a.y);
  const TZ *z = static_cast<const TZ *>(a.z);
  TY *o = static_cast<TY *>(a.out);
  const int64_t threads = rows * (p.d_v / 4);
  const dim3 grid((unsigned)((threads + 255) / 256));
  switch (p.d_v) {
    case 16: hipLaunchKernelGGL((gated_norm_kernel<TY, TZ, 16>), grid, dim3(256), 0, st, y, z, a.weight, a.eps, o, rows); break;
    case 32: hipLaunchKernelGGL((gated_norm_kernel<TY, TZ, 32>), grid, dim3(256), 0, st, y, z, a.weight, a.eps, o, rows); break;
    case 64: hipLaunchKernelGGL((gated_norm_kernel<TY, TZ, 64>), grid, dim3(256), 0, st, y, z, a.weight, a.eps, o, rows); break;
    case 128: hipLaunchKernelGGL((gated_norm_kernel<TY, TZ, 128>), grid, dim3(256), 0, st, y, z, a.weight, a.eps, o, rows); break;
    case 256: hipLaunchKernelGGL((gated_norm_kernel<TY, TZ, 256>), grid, dim3(256), 0, st, y, z, a.weight, a.eps, o, rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prologue, part 1: causal depthwise convolution of width 4 and SiLU.
// Thread (channel group of 4, run of kRun tokens): the three previous inputs
// of its 4 channels ride along in registers, and are reset from the sequence's
// convolution state (or zeros) wherever a sequence starts.  Consecutive
// threads take consecutive channel groups of the same token.  Unless the
// convolution state is updated in place, the same launch also writes each
// sequence's outgoing state (at its last token) and the gates.
// ---------------------------------------------------------------------------
constexpr int kRun = 16;

struct SeqRows {
  const int32_t *cu;  // cu_seqlens, or nullptr for dense rows of rowT tokens
  int N, rowT, T_tot;
  // Start of sequence n, clamped into [0, T_tot] (a bad device array must not
  // send an access out of bounds).
  __device__ __forceinline__ int start(int n) const {
    const int s = cu ? cu[n] : n * rowT;
    return min(max(s, 0), T_tot);
  }
  __device__ __forceinline__ int seq_of(int t) const { return cu ? find_seq(cu, N, t) : t / rowT; }
};

// The 4 channels of T at p: their raw bytes (8 for bf16, 16 for fp32), and
// unpacked to floats.
template <typename T>
using Raw4 = typename std::conditional<std::is_same<T, float>::value, u32x4, u32x2>::type;
template <typename T> __device__ __forceinline__ Raw4<T> ld4raw(const T *p) {
  return *reinterpret_cast<const Raw4<T> *>(p);
}
template <typename T> __device__ __forceinline__ void unpack4(const Raw4<T> &r, f32x4 &o) {
  if constexpr (std::is_same<T, float>::value) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = r[e];  // (a bit cast of the vector element itself reads element 0)
      o[e] = __builtin_bit_cast(float, u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t u = r[e];
      o[2 * e] = __builtin_bit_cast(float, u << 16);
      o[2 * e + 1] = __builtin_bit_cast(float, u & 0xffff0000u);
    }
  }
}

// The gates of item r = (token, value head): g = -exp(A_log) softplus(a + dt_bias),
// beta = sigmoid(b).
__device__ __forceinline__ void gate_item(int64_t r, int H_v, const float *__restrict__ a,
                                          const float *__restrict__ b, const float *__restrict__ A_log,
                                          const float *__restrict__ dt_bias, float *__restrict__ g,
                                          float *__restrict__ beta) {
  const int h = (int)(r % H_v);
  const float av = a[r] + dt_bias[h];
  const float sp = av > 20.0f ? av : log1pf(__expf(av));  // softplus
  g[r] = -__expf(A_log[h]) * sp;
  beta[r] = 1.0f / (1.0f + __expf(-b[r]));
}

template <typename T>
__global__ __launch_bounds__(256) void conv_silu_kernel(const T *__restrict__ x, const float *__restrict__ cw,
                                                        const float *__restrict__ cs_in, const SeqRows sr,
                                                        int Cch, int nq, int nv, T *__restrict__ q,
                                                        T *__restrict__ k, T *__restrict__ v,
                                                        float *__restrict__ cs_out, const float *__restrict__ a,
                                                        const float *__restrict__ b, const float *__restrict__ A_log,
                                                        const float *__restrict__ dt_bias, int H_v,
                                                        float *__restrict__ g, float *__restrict__ beta) {
  // Gates, when this launch carries them: one flat loop over every thread.
  if (g) {
    const int64_t n_gate = (int64_t)sr.T_tot * H_v, nthr = (int64_t)gridDim.x * gridDim.y * 256;
    for (int64_t r = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 256 + threadIdx.x; r < n_gate; r += nthr)
      gate_item(r, H_v, a, b, A_log, dt_bias, g, beta);
  }
  const int g4 = blockIdx.x * 256 + threadIdx.x;
  const int c = 4 * g4;
  if (c >= Cch) return;
  f32x4 wt[4];  // wt[i][j]: tap i of channel c + j (tap 3 multiplies the current token)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x4 wc = load4(cw + (int64_t)(c + j) * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) wt[i][j] = wc[i];
  }
  T *dst;
  int64_t ld;
  if (c < nq) {
    dst = q + c;
    ld = nq;
  } else if (c < 2 * nq) {
    dst = k + (c - nq);
    ld = nq;
  } else {
    dst = v + (c - 2 * nq);
    ld = nv;
  }
  // the three inputs before token t of sequence n, oldest first
  f32x4 h0, h1, h2;
  auto reset = [&](int n, int t) {
    const int s = sr.start(n);
    f32x4 hv[3];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int tt = t - 3 + i;
      if (tt >= s) {
        hv[i] = load4(x + (int64_t)tt * Cch + c);
      } else {
        const int j = tt - s + 3;  // index into the sequence's state, in [0, 3) for a sane array
        hv[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (cs_in && j >= 0)
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[i][e] = cs_in[((int64_t)n * Cch + c + e) * 3 + j];
      }
    }
    h0 = hv[0];
    h1 = hv[1];
    h2 = hv[2];
  };
  // Outgoing state of an empty sequence: its incoming state (or zeros); the
  // other sequences' states are written at their last token below.
  if (cs_out && blockIdx.y == 0) {
    for (int n = 0; n < sr.N; ++n) {
      const int s = sr.start(n), e = n + 1 < sr.N ? sr.start(n + 1) : sr.T_tot;
      if (e > s) continue;
#pragma unroll
      for (int i = 0; i < 12; ++i)
        cs_out[((int64_t)n * Cch + c) * 3 + i] = cs_in ? cs_in[((int64_t)n * Cch + c) * 3 + i] : 0.0f;
    }
  }
  const int runs = (sr.T_tot + kRun - 1) / kRun;
  for (int run = blockIdx.y; run < runs; run += gridDim.y) {
    const int t0 = run * kRun, t1 = min(t0 + kRun, sr.T_tot);
    int n = sr.seq_of(t0);
    int next = n + 1 < sr.N ? sr.start(n + 1) : sr.T_tot;
    reset(n, t0);
    // The next kAhead tokens' inputs are in flight while a token is computed and
    // stored (raw bytes, unpacked at use; reads past the run repeat its last
    // token and go unused).  Without them each token would wait for its own
    // load and for the store before it.
    constexpr int kAhead = 4;
    Raw4<T> ring[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) ring[i] = ld4raw<T>(x + (int64_t)min(t0 + i, t1 - 1) * Cch + c);
#pragma unroll
    for (int i = 0; i < kRun; ++i) {
      const int t = t0 + i;
      if (t < t1) {
        if (t >= next) {  // a sequence starts here (skip the empty ones)
          while (n + 1 < sr.N && sr.start(n + 1) <= t) ++n;
          next = n + 1 < sr.N ? sr.start(n + 1) : sr.T_tot;
          reset(n, t);
        }
        f32x4 xt;
        unpack4<T>(ring[i % kAhead], xt);
        if (i + kAhead < kRun) ring[i % kAhead] = ld4raw<T>(x + (int64_t)min(t + kAhead, t1 - 1) * Cch + c);
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = silu(wt[0][j] * h0[j] + wt[1][j] * h1[j] + wt[2][j] * h2[j] + wt[3][j] * xt[j]);
        store4(dst + (int64_t)t * ld, o);
        h0 = h1;
        h1 = h2;
        h2 = xt;
        if (cs_out && t + 1 == next) {  // the sequence's last token: its last three inputs
          float *so = cs_out + ((int64_t)n * Cch + c) * 3;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            so[3 * e] = h0[e];
            so[3 * e + 1] = h1[e];
            so[3 * e + 2] = h2[e];
          }
        }
      }
    }
  }
}

// Prologue, part 2, for an in-place state update or no tokens (after part 1,
// which reads the incoming states): each sequence's outgoing convolution state,
// then the gates.  One flat loop over N * Cch state items and T_tot * H_v gate
// items.
template <typename T>
__global__ __launch_bounds__(256) void prologue_tail_kernel(const T *__restrict__ x, const float *cs_in,
                                                            float *cs_out, const SeqRows sr, int Cch,
                                                            const float *__restrict__ a,
                                                            const float *__restrict__ b,
                                                            const float *__restrict__ A_log,
                                                            const float *__restrict__ dt_bias, int H_v,
                                                            float *__restrict__ g, float *__restrict__ beta) {
  const int64_t n_state = cs_out ? (int64_t)sr.N * Cch : 0;
  const int64_t n_gate = (int64_t)sr.T_tot * H_v;
  for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < n_state + n_gate;
       it += (int64_t)gridDim.x * 256) {
    if (it < n_state) {
      const int n = (int)(it / Cch), c = (int)(it % Cch);
      const int s = sr.start(n), e = n + 1 < sr.N ? sr.start(n + 1) : sr.T_tot;
      const int L = max(e - s, 0);
      float nv[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int i = L + j;  // index into [incoming state (3); the sequence's inputs (L)]
        if (i >= 3) nv[j] = Elem<T>::get(x, (int64_t)(s + i - 3) * Cch + c);
        else nv[j] = cs_in ? cs_in[((int64_t)n * Cch + c) * 3 + i] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 3; ++j) cs_out[((int64_t)n * Cch + c) * 3 + j] = nv[j];  // after all reads
    } else {
      gate_item(it - n_state, H_v, a, b, A_log, dt_bias, g, beta);
    }
  }
}

template <typename T>
hipError_t launch_prologue_t(const Problem &p, const PrologueArgs &a, hipStream_t st) {
  const int nq = p.H_qk * p.d_k, nv = p.H_v * p.d_v, Cch = 2 * nq + nv;
  const SeqRows sr{a.cu, p.N, p.T, p.T_tot};
  const T *x = static_cast<const T *>(a.x);
  // The convolution kernel also writes the outgoing states and the gates, except
  // where the states are updated in place (every incoming state must be read
  // before any is written: a second kernel does both then) or there are no tokens.
  const bool fuse = p.T_tot > 0 && (a.cs_out == nullptr || a.cs_out != a.cs_in);
  if (p.T_tot > 0) {
    const int runs = (p.T_tot + kRun - 1) / kRun;
    const dim3 grid((unsigned)((Cch / 4 + 255) / 256), (unsigned)std::min(runs, 65535));
    hipLaunchKernelGGL((conv_silu_kernel<T>), grid, dim3(256), 0, st, x, a.conv_w, a.cs_in, sr, Cch, nq, nv,
                       static_cast<T *>(a.q), static_cast<T *>(a.k), static_cast<T *>(a.v),
                       fuse ? a.cs_out : nullptr, a.a, a.b, a.A_log, a.dt_bias, p.H_v, fuse ? a.g : nullptr,
                       a.beta);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fuse) return e;
  }
  const int64_t items = (a.cs_out ? (int64_t)p.N * Cch : 0) + (int64_t)p.T_tot * p.H_v;
  if (items > 0) {
    const unsigned blocks = (unsigned)std::min<int64_t>((items + 255) / 256, 8192);
    hipLaunchKernelGGL((prologue_tail_kernel<T>), dim3(blocks), dim3(256), 0, st, x, a.cs_in, a.cs_out, sr, Cch,
                       a.a, a.b, a.A_log, a.dt_bias, p.H_v, a.g, a.beta);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

bool norm_supported(const Problem &p) {
  return p.d_v == 16 || p.d_v == 32 || p.d_v == 64 || p.d_v == 128 || p.d_v == 256;
}

hipError_t launch_gated_norm(const Problem &p, const NormArgs &a, hipStream_t st) {
  const bool yb = p.o_dtype == GDN_BF16, zb = p.dtype == GDN_BF16;
  if (yb) return zb ? launch_norm_t<uint16_t, uint16_t>(p, a, st) : launch_norm_t<uint16_t, float>(p, a, st);
  return zb ? launch_norm_t<float, uint16_t>(p, a, st) : launch_norm_t<float, float>(p, a, st);
}

bool prologue_supported(const Problem &p) { return p.d_k % 4 == 0 && p.d_v % 4 == 0; }

hipError_t launch_prologue(const Problem &p, const PrologueArgs &a, hipStream_t st) {
  return p.dtype == GDN_BF16 ? launch_prologue_t<uint16_t>(p, a, st) : launch_prologue_t<float>(p, a, st);
}

}  // namespace gdn
