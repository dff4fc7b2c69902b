// Decode backward ("FLARE++: Low-rank attention with dynamic attention
// routing", appendix on context parallelism, FLARE++ backward paragraph: each
// token's local decoder contributes to the gradient of the replicated latent
// keys, and the latent values' gradient is the sum of the decoders'
// contributions).  For Y[n] = softmax_m(s Xq[n].Klat[m]) Z and an output
// gradient dY:
//   A = softmax over the M latents,  dA = dY Z^T,  delta[n] = sum_m A dA,
//   dT = A (dA - delta),  dXq = s dT Klat,  dKlat = s dT^T Xq,  dZ = A^T dY.
// Two passes: the token side (softmax over the latents is lane-local) writes
// dXq and each token's log2-normaliser and delta; the latent side streams the
// tokens again and sums dZ and dKlat per token chunk, which a fixed-order
// reduction adds up.
#include "common.h"
#include "kernels.h"

namespace flare {

namespace {
template <typename T>
__device__ __forceinline__ float ld1(const T* p) {
  if constexpr (sizeof(T) == 2) return bf16_to_f32(*p); else return *p;
}
template <typename T>
__device__ __forceinline__ void st1(T* p, float v) {
  if constexpr (sizeof(T) == 2) *p = to_bf16(v); else *p = v;
}
}  // namespace

// ---------------------------------------------------------------------------
// General vector kernels (float32, or shapes without a matrix-core variant).
// ---------------------------------------------------------------------------
// Token side: one wave per token, lanes over head dims; three passes over the
// latents (normaliser, delta, dXq) recompute the dot products.
template <typename TIn>
__global__ __launch_bounds__(256) void dbwd_tok_generic_kernel(const DecBwdArgs a) {
  constexpr int MAXDL = 4;   // D <= 256
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t total = (int64_t)a.B * a.H * a.N;
  if (tok >= total) return;
  const int n = (int)(tok % a.N);
  const int64_t bh = tok / a.N;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int D = a.D, M = a.M;
  const bool valid = !a.token_mask || a.token_mask[(int64_t)b * a.N + n] != 0;
  const int64_t srow = bh * a.stats_stride + n;
  TIn* dx = static_cast<TIn*>(a.dXq) + tok * D;
  if (!valid) {
    for (int d = lane; d < D; d += 64) st1(dx + d, 0.f);
    if (lane == 0) {
      a.lse2[srow] = __builtin_huge_valf();   // weights exp2(t - inf) = 0 on the latent side
      a.delta[srow] = 0.f;
    }
    return;
  }
  const TIn* Kl = static_cast<const TIn*>(a.Klat) + (int64_t)b * a.klat_bstride + (int64_t)h * M * D;
  const float* Zb = a.Z + bh * (int64_t)M * D;
  float x[MAXDL], g[MAXDL];
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    x[j] = d < D ? ld1(static_cast<const TIn*>(a.Xq) + tok * D + d) : 0.f;
    g[j] = d < D ? ld1(static_cast<const TIn*>(a.dY) + tok * D + d) : 0.f;
  }
  auto score = [&](int m) {   // log2 units
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < MAXDL; ++j) {
      const int d = lane + 64 * j;
      if (d < D) t = __builtin_fmaf(x[j], ld1(Kl + (int64_t)m * D + d), t);
    }
    return wave_sum(t) * a.scale_log2;
  };
  auto dgrad = [&](int m) {
    float t = 0.f;
#pragma unroll
    for (int j = 0; j < MAXDL; ++j) {
      const int d = lane + 64 * j;
      if (d < D) t = __builtin_fmaf(g[j], Zb[(int64_t)m * D + d], t);
    }
    return wave_sum(t);
  };
  float mx = kNegInf, l = 0.f;
  for (int m = 0; m < M; ++m) {
    const float t = score(m);
    const float nm = fmaxf(mx, t);
    l = l * exp2f(mx - nm) + exp2f(t - nm);
    mx = nm;
  }
  const float lse2 = mx + log2f(l);
  float delta = 0.f;
  for (int m = 0; m < M; ++m) delta = __builtin_fmaf(exp2f(score(m) - lse2), dgrad(m), delta);
  float acc[MAXDL] = {0.f, 0.f, 0.f, 0.f};
  for (int m = 0; m < M; ++m) {
    const float dt = exp2f(score(m) - lse2) * (dgrad(m) - delta);
#pragma unroll
    for (int j = 0; j < MAXDL; ++j) {
      const int d = lane + 64 * j;
      if (d < D) acc[j] = __builtin_fmaf(dt, ld1(Kl + (int64_t)m * D + d), acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    if (d < D) st1(dx + d, a.scale * acc[j]);
  }
  if (lane == 0) {
    a.lse2[srow] = lse2;
    a.delta[srow] = delta;
  }
}

// Latent side: one wave per latent row, over every valid token.
template <typename TIn>
__global__ __launch_bounds__(256) void dbwd_lat_generic_kernel(const DecBwdArgs a) {
  constexpr int MAXDL = 4;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)a.B * a.H * a.M;
  if (row >= rows) return;
  const int m = (int)(row % a.M);
  const int64_t bh = row / a.M;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int D = a.D;
  const TIn* kr = static_cast<const TIn*>(a.Klat) + (int64_t)b * a.klat_bstride + ((int64_t)h * a.M + m) * D;
  const float* zr = a.Z + row * D;
  const TIn* Xg = static_cast<const TIn*>(a.Xq) + bh * (int64_t)a.N * D;
  const TIn* Gg = static_cast<const TIn*>(a.dY) + bh * (int64_t)a.N * D;
  const uint8_t* mk = a.token_mask ? a.token_mask + (int64_t)b * a.N : nullptr;
  float kd[MAXDL], zd[MAXDL], az[MAXDL], ak[MAXDL];
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    kd[j] = d < D ? ld1(kr + d) : 0.f;
    zd[j] = d < D ? zr[d] : 0.f;
    az[j] = ak[j] = 0.f;
  }
  for (int n = 0; n < a.N; ++n) {
    if (mk && mk[n] == 0) continue;
    float xd[MAXDL], gd[MAXDL], t = 0.f, da = 0.f;
#pragma unroll
    for (int j = 0; j < MAXDL; ++j) {
      const int d = lane + 64 * j;
      xd[j] = d < D ? ld1(Xg + (int64_t)n * D + d) : 0.f;
      gd[j] = d < D ? ld1(Gg + (int64_t)n * D + d) : 0.f;
      t = __builtin_fmaf(xd[j], kd[j], t);
      da = __builtin_fmaf(gd[j], zd[j], da);
    }
    t = wave_sum(t) * a.scale_log2;
    da = wave_sum(da);
    const float w = exp2f(t - a.lse2[bh * a.stats_stride + n]);
    const float dt = w * (da - a.delta[bh * a.stats_stride + n]);
#pragma unroll
    for (int j = 0; j < MAXDL; ++j) {
      az[j] = __builtin_fmaf(w, gd[j], az[j]);
      ak[j] = __builtin_fmaf(dt, xd[j], ak[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    if (d < D) {
      a.dZ[row * D + d] = az[j];
      a.dKlat[row * D + d] = a.scale * ak[j];
      if (a.dZ_cast) st1(static_cast<TIn*>(a.dZ_cast) + row * D + d, az[j]);
    }
  }
}

hipError_t launch_decode_bwd_generic(const DecBwdArgs& a, bool bf16, hipStream_t s) {
  const int64_t toks = (int64_t)a.B * a.H * a.N;
  const int64_t rows = (int64_t)a.B * a.H * a.M;
  if (toks > 0) {
    const unsigned g = (unsigned)((toks + 3) / 4);
    if (bf16) hipLaunchKernelGGL(dbwd_tok_generic_kernel<uint16_t>, dim3(g), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(dbwd_tok_generic_kernel<float>, dim3(g), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (rows > 0) {
    const unsigned g = (unsigned)((rows + 3) / 4);
    if (bf16) hipLaunchKernelGGL(dbwd_lat_generic_kernel<uint16_t>, dim3(g), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(dbwd_lat_generic_kernel<float>, dim3(g), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

bool decode_bwd_mfma_supported(int M, int D) { return false; }
int decode_bwd_waves(int D) { return 4; }
hipError_t launch_decode_bwd_mfma(const DecBwdArgs& a, hipStream_t s) { return hipErrorInvalidValue; }
hipError_t launch_decode_bwd_reduce(const DecBwdArgs& a, bool bf16, hipStream_t s) { return hipErrorInvalidValue; }

}  // namespace flare
