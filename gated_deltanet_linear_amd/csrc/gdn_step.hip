// gdn_recurrent_step: one decode token per sequence, state updated in place.
//
// This is the pages' "decode step's recurrent" kernel (Qwen3.5 text
// encyclopedia page, value table of model.layers[i].linear_attn): for every
// (sequence b, value head h) it reads the 128 x 128 fp32 state once, and writes
// it once:
//
//   e = S^T k,  r = S^T q          column reductions over d_k of the OLD state
//   a = exp(g), d = beta (v - a e)  prediction of the decayed state a S
//   S <- a S + k d^T                in place
//   o = a r + (k . q) d             = S_new^T q, read after the write
//
// and, in the gated variant, the mixer's output norm on the spot (the same
// page's note "The DeltaNet mixer": norm(y, gate=silu(z)) with gain weight):
//
//   o <- weight * o / sqrt(mean(o^2) + eps) * silu(z)   over the head's d_v values
//
// The step is a pure HBM stream (0.74 FLOP per byte): one workgroup per
// (b, h) of up to 1024 threads; each thread keeps a 4-column x (d_k / row
// groups)-row strip of S in registers between the read and the write, so S
// crosses HBM exactly twice.  Loads and stores are 16 bytes per lane, and each
// wave instruction touches two whole 512-byte rows of S.  The loads are plain
// and the stores non-temporal: on 256 sequences x 32 heads that pairing steps
// ~9% faster than non-temporal loads and stores, and plain stores are slower
// with either kind of load.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"
#include "gdn.h"

namespace gdn {

template <int DK, int DV> struct StepCfg {
  static constexpr int CG = DV / 4;                                   // float4 column groups
  static constexpr int NT = (DK * DV / 4 < 1024) ? DK * DV / 4 : 1024;  // threads
  static constexpr int RG = NT / CG;                                  // row groups
  static constexpr int RPT = DK / RG;                                 // rows per thread
  static constexpr int NW = (NT + 63) / 64;                           // waves
  static_assert(DV % 4 == 0 && CG <= 64 && NT % CG == 0 && DK % RG == 0, "step tiling");
  static_assert(NT % 64 == 0 || NT == CG * RG, "whole waves");
};

template <int DK, int DV, typename TIn, bool OBF16, bool GN>
__global__ __launch_bounds__((StepCfg<DK, DV>::NT)) void step_kernel(
    const TIn *__restrict__ q, const TIn *__restrict__ k, const TIn *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, float *__restrict__ state,
    void *__restrict__ o, int H_qk, int H_v, float scale, int l2norm, const TIn *__restrict__ z,
    const float *__restrict__ wn, float eps) {
  using Cfg = StepCfg<DK, DV>;
  constexpr int CG = Cfg::CG, RG = Cfg::RG, RPT = Cfg::RPT, NW = Cfg::NW;

  const int bh = blockIdx.x;  // b * H_v + h
  const int b = bh / H_v, h = bh - b * H_v;
  const int j = h / (H_v / H_qk);  // repeat_interleave head sharing
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cg = tid % CG, rg = tid / CG;

  __shared__ float ks[DK], qs[DK];
  __shared__ float red[NW][2][DV];
  __shared__ float sc3[3];

  // Issue the state strip loads first: they are the long pole.
  float *Sp = state + (int64_t)bh * DK * DV;
  f32x4 S[RPT];
#pragma unroll
  for (int s = 0; s < RPT; ++s)
    S[s] = *reinterpret_cast<const f32x4 *>(Sp + (int64_t)(rg + RG * s) * DV + 4 * cg);

  const int64_t qk_off = ((int64_t)b * H_qk + j) * DK;
  for (int i = tid; i < DK; i += Cfg::NT) {
    ks[i] = Elem<TIn>::get(k, qk_off + i);
    qs[i] = Elem<TIn>::get(q, qk_off + i);
  }
  const float alpha = expf(g[bh]);  // exp(-inf) == 0: a reset
  const float bta = beta[bh];
  f32x4 vv;
  {
    const int64_t vo = (int64_t)bh * DV + 4 * cg;
    vv = f32x4{Elem<TIn>::get(v, vo), Elem<TIn>::get(v, vo + 1), Elem<TIn>::get(v, vo + 2),
               Elem<TIn>::get(v, vo + 3)};
  }
  // The output norm's gate input and gain for this lane's 4 columns, loaded with
  // the state so that their latency is not added at the end (every row group
  // loads them; the lanes of row group 0 use them).
  f32x4 zc = {0.f, 0.f, 0.f, 0.f}, wc = zc;
  if constexpr (GN) {
    const int64_t zo = (int64_t)bh * DV + 4 * cg;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      zc[c] = Elem<TIn>::get(z, zo + c);
      wc[c] = wn[4 * cg + c];
    }
  }
  __syncthreads();

  // Norms and k.q (wave 0), shared through LDS.
  if (wave == 0) {
    float sk = 0.f, sq = 0.f, skq = 0.f;
    for (int i = lane; i < DK; i += 64) {
      const float a = ks[i], c = qs[i];
      sk += a * a;
      sq += c * c;
      skq += a * c;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      sk += wave_xor(sk, m);
      sq += wave_xor(sq, m);
      skq += wave_xor(skq, m);
    }
    if (lane == 0) {
      const float rk = l2norm ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f;
      const float rq = (l2norm ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f) * scale;
      sc3[0] = rk;
      sc3[1] = rq;
      sc3[2] = skq * rk * rq;  // k_hat . q_hat
    }
  }
  __syncthreads();
  const float rk = sc3[0], rq = sc3[1], kq = sc3[2];

  // Column partial sums of the old state against k_hat and q_hat.
  f32x4 e = {0.f, 0.f, 0.f, 0.f}, r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < RPT; ++s) {
    const int row = rg + RG * s;
    const float kk = ks[row] * rk, qq = qs[row] * rq;
    e += S[s] * kk;
    r += S[s] * qq;
  }
  // Reduce over the row groups of this wave (lanes sharing cg), then over waves.
#pragma unroll
  for (int m = CG; m < 64; m <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      e[c] += wave_xor(e[c], m);
      r[c] += wave_xor(r[c], m);
    }
  }
  if (NW > 1) {
    if (lane < CG) {
      *reinterpret_cast<f32x4 *>(&red[wave][0][4 * cg]) = e;
      *reinterpret_cast<f32x4 *>(&red[wave][1][4 * cg]) = r;
    }
    __syncthreads();
    e = *reinterpret_cast<const f32x4 *>(&red[0][0][4 * cg]);
    r = *reinterpret_cast<const f32x4 *>(&red[0][1][4 * cg]);
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      e += *reinterpret_cast<const f32x4 *>(&red[w][0][4 * cg]);
      r += *reinterpret_cast<const f32x4 *>(&red[w][1][4 * cg]);
    }
  }

  const f32x4 d = bta * (vv - alpha * e);  // delta of the decayed state
  // Write back a S + k_hat d^T.
#pragma unroll
  for (int s = 0; s < RPT; ++s) {
    const int row = rg + RG * s;
    const float kk = ks[row] * rk;
    __builtin_nontemporal_store(alpha * S[s] + kk * d, reinterpret_cast<f32x4 *>(Sp + (int64_t)row * DV + 4 * cg));
  }
  if (rg == 0) {
    f32x4 out = alpha * r + kq * d;
    if constexpr (GN) {
      // the head's d_v outputs sit in lanes 0 .. CG-1 of wave 0, 4 per lane
      float ss = out[0] * out[0] + out[1] * out[1] + out[2] * out[2] + out[3] * out[3];
#pragma unroll
      for (int m = 1; m < CG; m <<= 1) ss += wave_xor(ss, m);
      const float rs = rsqrtf(ss * (1.0f / DV) + eps);
#pragma unroll
      for (int c = 0; c < 4; ++c) out[c] = wc[c] * (out[c] * rs) * (zc[c] / (1.0f + __expf(-zc[c])));
    }
    if constexpr (OBF16) {
      uint16_t *op = reinterpret_cast<uint16_t *>(o) + (int64_t)bh * DV + 4 * cg;
      uint2 pk;
      pk.x = (uint32_t)f2bf(out[0]) | ((uint32_t)f2bf(out[1]) << 16);
      pk.y = (uint32_t)f2bf(out[2]) | ((uint32_t)f2bf(out[3]) << 16);
      *reinterpret_cast<uint2 *>(op) = pk;
    } else {
      *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(o) + (int64_t)bh * DV + 4 * cg) = out;
    }
  }
}

template <int DK, int DV, typename TIn, bool OBF16>
static hipError_t launch_step_t(const Problem &p, const StepArgs &a, hipStream_t st) {
  const int grid = p.B * p.H_v;
  if (grid == 0) return hipSuccess;
  if (a.z) {
    hipLaunchKernelGGL((step_kernel<DK, DV, TIn, OBF16, true>), dim3(grid), dim3(StepCfg<DK, DV>::NT), 0, st,
                       static_cast<const TIn *>(a.q), static_cast<const TIn *>(a.k),
                       static_cast<const TIn *>(a.v), a.g, a.beta, a.state, a.o, p.H_qk, p.H_v, p.scale,
                       p.l2norm ? 1 : 0, static_cast<const TIn *>(a.z), a.weight, a.eps);
  } else {
    hipLaunchKernelGGL((step_kernel<DK, DV, TIn, OBF16, false>), dim3(grid), dim3(StepCfg<DK, DV>::NT), 0, st,
                       static_cast<const TIn *>(a.q), static_cast<const TIn *>(a.k),
                       static_cast<const TIn *>(a.v), a.g, a.beta, a.state, a.o, p.H_qk, p.H_v, p.scale,
                       p.l2norm ? 1 : 0, static_cast<const TIn *>(nullptr), static_cast<const float *>(nullptr),
                       0.0f);
  }
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_step_dims(const Problem &p, const StepArgs &a, hipStream_t st) {
  const bool ob = p.o_dtype == GDN_BF16;
  if (p.dtype == GDN_BF16)
    return ob ? launch_step_t<DK, DV, uint16_t, true>(p, a, st) : launch_step_t<DK, DV, uint16_t, false>(p, a, st);
  return ob ? launch_step_t<DK, DV, float, true>(p, a, st) : launch_step_t<DK, DV, float, false>(p, a, st);
}

bool step_supported(const Problem &p) {
  return (p.d_k == 16 || p.d_k == 128) && (p.d_v == 16 || p.d_v == 128);
}

hipError_t launch_recurrent_step(const Problem &p, const StepArgs &a, hipStream_t st) {
  if (p.d_k == 128 && p.d_v == 128) return launch_step_dims<128, 128>(p, a, st);
  if (p.d_k == 16 && p.d_v == 16) return launch_step_dims<16, 16>(p, a, st);
  if (p.d_k == 16 && p.d_v == 128) return launch_step_dims<16, 128>(p, a, st);
  if (p.d_k == 128 && p.d_v == 16) return launch_step_dims<128, 16>(p, a, st);
  return hipErrorInvalidValue;
}

}  // namespace gdn
