// Encoder backward with the global statistics ("FLARE++: Low-rank attention
// with dynamic attention routing", appendix on context parallelism, backward
// paragraph): the probabilities of every partition are normalised by the
// global log-normaliser L of the forward pass, P = exp(s q.k - L); the row
// term c = rowsum(dZ * Z) carries the redistribution of mass between
// partitions; dS = P (dZ.v - c); dV = P^T dZ, dK = s dS^T Q, and the query
// gradient s dS K is summed over all partitions.
#include "common.h"
#include "kernels.h"

namespace flare {

// c[row] = sum_d dZ[row, d] * Z[row, d]  (one wave per row)
template <typename TIn>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const TIn* __restrict__ dZ, const float* __restrict__ Z,
                                                         int64_t rows, int D, float* __restrict__ c) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float acc = 0.f;
  for (int d = lane; d < D; d += 64) {
    float g;
    if constexpr (sizeof(TIn) == 2) g = bf16_to_f32(dZ[row * D + d]); else g = dZ[row * D + d];
    acc = __builtin_fmaf(g, Z[row * D + d], acc);
  }
  acc = wave_sum(acc);
  if (lane == 0) c[row] = acc;
}

template <typename TIn>
__device__ __forceinline__ float ldg_(const TIn* p) {
  if constexpr (sizeof(TIn) == 2) return bf16_to_f32(*p); else return *p;
}
template <typename TIn>
__device__ __forceinline__ void stg_(TIn* p, float v) {
  if constexpr (sizeof(TIn) == 2) *p = to_bf16(v); else *p = v;
}

// ---------------------------------------------------------------------------
// General vector kernels (float32 inputs, or shapes without a matrix-core
// variant).  Float32 arithmetic throughout.
// ---------------------------------------------------------------------------
// dK, dV of one token per wave: lanes take head dims; the score and dP of each
// latent row are wave reductions.
template <typename TIn>
__global__ __launch_bounds__(256) void bwd_kv_generic_kernel(const BwdArgs a) {
  constexpr int MAXDL = 4;   // D <= 256
  const int64_t tok = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t total = (int64_t)a.B * a.H * a.N;
  if (tok >= total) return;
  const int n = (int)(tok % a.N);
  const int64_t bh = tok / a.N;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int D = a.D, M = a.M;
  TIn* dk = static_cast<TIn*>(a.dK) + tok * D;
  TIn* dv = static_cast<TIn*>(a.dV) + tok * D;
  const bool valid = !a.mask || a.mask[(int64_t)b * a.N + n] != 0;
  float kk[MAXDL], vv[MAXDL], ak[MAXDL], av[MAXDL];
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    kk[j] = (valid && d < D) ? ldg_(static_cast<const TIn*>(a.K) + tok * D + d) : 0.f;
    vv[j] = (valid && d < D) ? ldg_(static_cast<const TIn*>(a.V) + tok * D + d) : 0.f;
    ak[j] = av[j] = 0.f;
  }
  if (valid) {
    const TIn* Q = static_cast<const TIn*>(a.Q) + (int64_t)b * a.q_bstride + (int64_t)h * M * D;
    const TIn* dZ = static_cast<const TIn*>(a.dZ) + bh * (int64_t)M * D;
    const float* Lr = a.L + bh * M;
    const float* cr = a.c + bh * M;
    for (int m = 0; m < M; ++m) {
      const float Lm = Lr[m];
      if (Lm == kNegInf) continue;   // row without any valid key: no gradient
      float qd[MAXDL], gd[MAXDL], sq = 0.f, sp = 0.f;
#pragma unroll
      for (int j = 0; j < MAXDL; ++j) {
        const int d = lane + 64 * j;
        qd[j] = d < D ? ldg_(Q + (int64_t)m * D + d) : 0.f;
        gd[j] = d < D ? ldg_(dZ + (int64_t)m * D + d) : 0.f;
        sq = __builtin_fmaf(qd[j], kk[j], sq);
        sp = __builtin_fmaf(gd[j], vv[j], sp);
      }
      sq = wave_sum(sq);
      sp = wave_sum(sp);
      const float p = __expf(a.scale * sq - Lm);
      const float ds = p * (sp - cr[m]);
#pragma unroll
      for (int j = 0; j < MAXDL; ++j) {
        av[j] = __builtin_fmaf(p, gd[j], av[j]);
        ak[j] = __builtin_fmaf(ds, qd[j], ak[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    if (d < D) {
      stg_(dv + d, av[j]);
      stg_(dk + d, a.scale * ak[j]);
    }
  }
}

// dQ of one latent row per wave, summed over every valid token.
template <typename TIn>
__global__ __launch_bounds__(256) void bwd_q_generic_kernel(const BwdArgs a) {
  constexpr int MAXDL = 4;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)a.B * a.H * a.M;
  if (row >= rows) return;
  const int m = (int)(row % a.M);
  const int64_t bh = row / a.M;
  const int h = (int)(bh % a.H), b = (int)(bh / a.H);
  const int D = a.D;
  const TIn* Qr = static_cast<const TIn*>(a.Q) + (int64_t)b * a.q_bstride + ((int64_t)h * a.M + m) * D;
  const TIn* gr = static_cast<const TIn*>(a.dZ) + row * D;
  const TIn* Kg = static_cast<const TIn*>(a.K) + bh * (int64_t)a.N * D;
  const TIn* Vg = static_cast<const TIn*>(a.V) + bh * (int64_t)a.N * D;
  const uint8_t* mk = a.mask ? a.mask + (int64_t)b * a.N : nullptr;
  const float Lm = a.L[row], cm = a.c[row];
  float qd[MAXDL], gd[MAXDL], acc[MAXDL];
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    qd[j] = d < D ? ldg_(Qr + d) : 0.f;
    gd[j] = d < D ? ldg_(gr + d) : 0.f;
    acc[j] = 0.f;
  }
  if (Lm != kNegInf) {
    for (int n = 0; n < a.N; ++n) {
      if (mk && mk[n] == 0) continue;
      float kd[MAXDL], sq = 0.f, sp = 0.f;
#pragma unroll
      for (int j = 0; j < MAXDL; ++j) {
        const int d = lane + 64 * j;
        kd[j] = d < D ? ldg_(Kg + (int64_t)n * D + d) : 0.f;
        const float vd = d < D ? ldg_(Vg + (int64_t)n * D + d) : 0.f;
        sq = __builtin_fmaf(qd[j], kd[j], sq);
        sp = __builtin_fmaf(gd[j], vd, sp);
      }
      sq = wave_sum(sq);
      sp = wave_sum(sp);
      const float ds = __expf(a.scale * sq - Lm) * (sp - cm);
#pragma unroll
      for (int j = 0; j < MAXDL; ++j) acc[j] = __builtin_fmaf(ds, kd[j], acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    if (d < D) a.dQ[row * D + d] = a.scale * acc[j];
  }
}

hipError_t launch_bwd_rowdot(const void* dZ, bool bf16, const float* Z, int64_t rows, int D, float* c,
                             hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (bf16)
    hipLaunchKernelGGL(bwd_rowdot_kernel<uint16_t>, dim3(grid), dim3(256), 0, s,
                       static_cast<const uint16_t*>(dZ), Z, rows, D, c);
  else
    hipLaunchKernelGGL(bwd_rowdot_kernel<float>, dim3(grid), dim3(256), 0, s, static_cast<const float*>(dZ), Z,
                       rows, D, c);
  return hipGetLastError();
}

hipError_t launch_bwd_generic(const BwdArgs& a, bool bf16, hipStream_t s) {
  const int64_t toks = (int64_t)a.B * a.H * a.N;
  const int64_t rows = (int64_t)a.B * a.H * a.M;
  if (toks > 0) {
    const unsigned g = (unsigned)((toks + 3) / 4);
    if (bf16) hipLaunchKernelGGL(bwd_kv_generic_kernel<uint16_t>, dim3(g), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(bwd_kv_generic_kernel<float>, dim3(g), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (rows > 0) {
    const unsigned g = (unsigned)((rows + 3) / 4);
    if (bf16) hipLaunchKernelGGL(bwd_q_generic_kernel<uint16_t>, dim3(g), dim3(256), 0, s, a);
    else hipLaunchKernelGGL(bwd_q_generic_kernel<float>, dim3(g), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace flare
