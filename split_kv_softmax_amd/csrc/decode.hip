// Local decode ("FLARE++: Low-rank attention with dynamic attention routing",
// appendix on context parallelism, FLARE and FLARE++ forward paragraphs):
// every token attends over the M replicated latents, Y[n] = softmax_m(s Xq[n].Klat[m]) Z,
// with no cross-partition work.  The softmax over m is exact (all M scores of a
// token are formed before any exponential).
#include "common.h"
#include "kernels.h"

namespace flare {

// ---------------------------------------------------------------------------
// bf16 matrix-core decode.  A workgroup (4 waves) owns one (batch, head) and a
// run of tokens; each wave handles 32 tokens at a time:
//   T^T[m][n] = Klat Xq^T         (A = latent rows from LDS, B = token rows
//                                  loaded straight into registers)
//   softmax over m                 (a token's M scores sit in one lane pair)
//   Y^T[d][n] = Z^T P^T            (A = Z^T in bf16 from LDS, B = P)
// so the normalisation by the row sum is lane-local.  Klat and Z are staged in
// LDS once per workgroup.
// ---------------------------------------------------------------------------
template <int D, int MB>
__global__ __launch_bounds__(256) void decode_mfma_kernel(const DecodeArgs a) {
  constexpr int M = 32 * MB;
  constexpr int KS = D / 16;   // k-steps of the score product
  constexpr int DB = D / 32;   // 32-row blocks of Y^T
  constexpr int MS = M / 16;   // k-steps of the value product
  constexpr int KLD = D + 8;
  constexpr int ZLD = M + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Kl[M * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Zt[D * ZLD];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int nblk = (a.N + a.tokens_per_block - 1) / a.tokens_per_block;
  int bid = blockIdx.x;
  const int tb = bid % nblk;
  bid /= nblk;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int64_t bh = (int64_t)b * a.H + h;

  {  // stage latent keys (row-major) and Z (transposed, rounded to bf16)
    const uint16_t* kg = static_cast<const uint16_t*>(a.Klat) + (int64_t)b * a.klat_bstride + (int64_t)h * M * D;
    for (int f = tid; f < M * D / 8; f += 256) {
      const int row = f / (D / 8), chk = f % (D / 8);
      st16(&Kl[row * KLD + 8 * chk], ld16(kg + (int64_t)row * D + 8 * chk));
    }
    const float* zg = a.Z + bh * (int64_t)M * D;
    for (int f = tid; f < M * D; f += 256) {
      const int m = f / D, d = f % D;
      Zt[d * ZLD + m] = to_bf16(zg[f]);
    }
  }
  __syncthreads();

  const uint16_t* Xg = static_cast<const uint16_t*>(a.Xq) + bh * (int64_t)a.N * D;
  uint16_t* Yg = static_cast<uint16_t*>(a.Y) + bh * (int64_t)a.N * D;
  const uint8_t* tm = a.token_mask ? a.token_mask + (int64_t)b * a.N : nullptr;
  const float c2 = a.scale_log2;
  const int n_lo = tb * a.tokens_per_block;
  const int n_hi = min(a.N, n_lo + a.tokens_per_block);

  for (int n0 = n_lo + 32 * wave; n0 < n_hi; n0 += 128) {
    const int n = n0 + l32;
    const bool inb = n < n_hi;
    bf16x8_t xop[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      xop[ks] = inb ? __builtin_bit_cast(bf16x8_t, ld16(Xg + (int64_t)n * D + 16 * ks + 8 * hh))
                    : bf16x8_t{};
    f32x16_t t[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      t[mb] = f32x16_t{};
      const uint16_t* krow = &Kl[(32 * mb + swap23(l32)) * KLD + 8 * hh];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        t[mb] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(krow + 16 * ks)),
                             xop[ks], t[mb]);
    }
    float mx = t[0][0];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, t[mb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float nmc = -mx * c2;
    float lsum = 0.f;
    bf16x8_t pk[MS];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = fast_exp2(__builtin_fmaf(t[mb][8 * g + j], c2, nmc));
          lsum += p[j];
        }
        u32x4_t w;
        w[0] = pack_bf16x2(p[0], p[1]);
        w[1] = pack_bf16x2(p[2], p[3]);
        w[2] = pack_bf16x2(p[4], p[5]);
        w[3] = pack_bf16x2(p[6], p[7]);
        pk[2 * mb + g] = __builtin_bit_cast(bf16x8_t, w);
      }
    lsum += __shfl_xor(lsum, 32, 64);
    f32x16_t y[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      y[db] = f32x16_t{};
      const uint16_t* zrow = &Zt[(32 * db + l32) * ZLD + 8 * hh];
#pragma unroll
      for (int ks = 0; ks < MS; ++ks)
        y[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(zrow + 16 * ks)),
                             pk[ks], y[db]);
    }
    const bool keep = inb && (!tm || tm[n] != 0);
    const float inv = 1.f / lsum;
    if (inb) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x2_t w;
          if (keep) {
            w[0] = pack_bf16x2(y[db][4 * q] * inv, y[db][4 * q + 1] * inv);
            w[1] = pack_bf16x2(y[db][4 * q + 2] * inv, y[db][4 * q + 3] * inv);
          } else {
            w = u32x2_t{0u, 0u};
          }
          *reinterpret_cast<u32x2_t*>(Yg + (int64_t)n * D + 32 * db + 8 * q + 4 * hh) = w;
        }
    }
  }
}

bool decode_mfma_supported(int M, int D) {
  // register budget: the M scores and D outputs of 32 tokens per wave
  if (D == 64) return M == 32 || M == 64 || M == 128 || M == 256;
  if (D == 128) return M == 32 || M == 64 || M == 128;
  return false;
}

template <int D, int MB>
static hipError_t launch_dec_t(const DecodeArgs& a, hipStream_t s) {
  const int64_t nblk = (a.N + a.tokens_per_block - 1) / a.tokens_per_block;
  const int64_t grid = nblk * a.H * a.B;
  hipLaunchKernelGGL((decode_mfma_kernel<D, MB>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s) {
  if (a.D == 64) {
    switch (a.M) {
      case 32: return launch_dec_t<64, 1>(a, s);
      case 64: return launch_dec_t<64, 2>(a, s);
      case 128: return launch_dec_t<64, 4>(a, s);
      case 256: return launch_dec_t<64, 8>(a, s);
    }
  } else if (a.D == 128) {
    switch (a.M) {
      case 32: return launch_dec_t<128, 1>(a, s);
      case 64: return launch_dec_t<128, 2>(a, s);
      case 128: return launch_dec_t<128, 4>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// General vector decode (float32, or bf16 shapes without a matrix-core
// variant): one wave per token; lanes take latent rows for the scores and
// head dimensions for the output.  Float32 arithmetic throughout.
// ---------------------------------------------------------------------------
template <typename TIn>
__device__ __forceinline__ float ldx(const TIn* p);
template <>
__device__ __forceinline__ float ldx<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ldx<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <typename TOut>
__device__ __forceinline__ void stx(TOut* p, float v);
template <>
__device__ __forceinline__ void stx<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void stx<uint16_t>(uint16_t* p, float v) { *p = to_bf16(v); }

template <typename TIn>
__global__ __launch_bounds__(256) void decode_generic_kernel(const DecodeArgs a) {
  constexpr int MAXL = 4;   // M <= 256 and D <= 256
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)blockIdx.x * 4 + wave;   // flattened (b, h, n)
  const int64_t total = (int64_t)a.B * a.H * a.N;
  if (tok >= total) return;
  const int n = (int)(tok % a.N);
  const int64_t bh = tok / a.N;
  const int h = (int)(bh % a.H);
  const int b = (int)(bh / a.H);
  const int D = a.D, M = a.M;
  const TIn* xr = static_cast<const TIn*>(a.Xq) + tok * D;
  const TIn* kl = static_cast<const TIn*>(a.Klat) + (int64_t)b * a.klat_bstride + (int64_t)h * M * D;
  const float* zg = a.Z + bh * (int64_t)M * D;
  TIn* yr = static_cast<TIn*>(a.Y) + tok * D;
  if (a.token_mask && a.token_mask[(int64_t)b * a.N + n] == 0) {
    for (int d = lane; d < D; d += 64) stx(yr + d, 0.f);
    return;
  }
  float sc[MAXL];
  float mx = kNegInf;
#pragma unroll
  for (int j = 0; j < MAXL; ++j) {
    const int m = lane + 64 * j;
    sc[j] = kNegInf;
    if (m < M) {
      float d = 0.f;
      for (int i = 0; i < D; ++i) d = __builtin_fmaf(ldx(xr + i), ldx(kl + (int64_t)m * D + i), d);
      sc[j] = d;
      mx = fmaxf(mx, d);
    }
  }
  mx = wave_max(mx);
  float ls = 0.f;
#pragma unroll
  for (int j = 0; j < MAXL; ++j) {
    sc[j] = (lane + 64 * j < M) ? fast_exp2((sc[j] - mx) * a.scale_log2) : 0.f;
    ls += sc[j];
  }
  ls = wave_sum(ls);
  float acc[MAXL];
#pragma unroll
  for (int j = 0; j < MAXL; ++j) acc[j] = 0.f;
#pragma unroll
  for (int j = 0; j < MAXL; ++j) {
    for (int i = 0; i < 64; ++i) {
      const int m = 64 * j + i;
      if (m >= M) break;
      const float pm = __shfl(sc[j], i, 64);
#pragma unroll
      for (int jj = 0; jj < MAXL; ++jj) {
        const int d = lane + 64 * jj;
        if (d < D) acc[jj] = __builtin_fmaf(pm, zg[(int64_t)m * D + d], acc[jj]);
      }
    }
  }
  const float inv = 1.f / ls;
#pragma unroll
  for (int jj = 0; jj < MAXL; ++jj) {
    const int d = lane + 64 * jj;
    if (d < D) stx(yr + d, acc[jj] * inv);
  }
}

hipError_t launch_decode_generic(const DecodeArgs& a, bool bf16, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.H * a.N;
  const int64_t grid = (total + 3) / 4;
  if (bf16)
    hipLaunchKernelGGL(decode_generic_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(decode_generic_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace flare
