// Encoder kernels: per-partition (O_r, L_r) states of softmax attention of M
// latent rows over the tokens of one chunk ("FLARE++: Low-rank attention with
// dynamic attention routing", appendix on context parallelism: the local-shard
// encoder between eq. 18 and eq. 23, which streams the shard's keys and values
// through an online softmax and returns both the normalised output and the
// log-normaliser; an attention row with no valid key returns (0, -inf)).
//
// The online softmax keeps, per row, the running maximum m of the raw dot
// products, the running sum l of exp(s (q.k - m)) and the unnormalised output
// acc; a new block of scores with maximum m' rescales l and acc by
// exp(s (m - m')) (the online-softmax merge of "Ring vs. Tree Attention").
// Exponentials are taken as exp2 of scores pre-multiplied by s log2(e); the
// returned log-normaliser is natural: L = s m + ln l.
#include "common.h"
#include "kernels.h"

namespace flare {

// ---------------------------------------------------------------------------
// bf16 matrix-core encoder.  One workgroup = one (batch, head, chunk) and all
// M = 32*NW latent rows, so each K/V byte is read from HBM exactly once.
// Wave w owns rows [32w, 32w+32).  Per 64-token tile:
//   S^T[n][m] = K_tile Q_w^T      (A = K rows from LDS, B = Q from registers)
//   online softmax over n          (the 32 scores of a row live in one lane
//                                   pair, so the row max needs one exchange)
//   O^T[d][m] += V_tile^T P^T      (A = V^T from LDS, B = P from registers)
// The result column of both products is the latent row, so the per-row
// rescale and normalisation are lane-local.
// ---------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) void encode_mfma_kernel(const EncodeArgs a) {
  constexpr int T = 64 * NW;
  constexpr int TILE = 64;
  constexpr int KS = D / 16;             // k-steps of the score product
  constexpr int DB = D / 32;             // 32-row blocks of O^T
  constexpr int KLD = D + 8;             // LDS row stride of K (elements)
  constexpr int VLD = TILE + 8;          // LDS row stride of V^T (elements)
  constexpr int KITEMS = TILE * D / 8;   // 16-byte pieces of a K tile
  constexpr int VITEMS = (TILE / 2) * (D / 8);  // row pairs x 16-byte pieces of a V tile
  constexpr int KI = (KITEMS + T - 1) / T;
  constexpr int VI = (VITEMS + T - 1) / T;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[TILE * KLD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VLD];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int nch = a.tab.nchunks;
  int bid = blockIdx.x;
  const int c = bid % nch;
  bid /= nch;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int t_begin = a.tab.bnd[c], t_end = a.tab.bnd[c + 1];
  const int64_t bh = (int64_t)b * a.H + h;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + bh * (int64_t)a.N * D;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + bh * (int64_t)a.N * D;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + (int64_t)b * a.q_bstride +
                       (int64_t)h * a.M * D;
  const uint8_t* mk = a.mask ? a.mask + (int64_t)b * a.N : nullptr;

  // Q rows of this wave as the B operand: column j = latent row 32w + j.
  bf16x8_t qop[KS];
  {
    const uint16_t* qrow = Qg + (int64_t)(32 * wave + l32) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qop[ks] = __builtin_bit_cast(bf16x8_t, ld16(qrow + 16 * ks));
  }

  const int ntiles = (t_end - t_begin + TILE - 1) / TILE;

  // validity of the 64 tokens of a tile as a wave-uniform bit mask
  auto range_bits = [&](int t0) -> uint64_t {
    const int n = t_end - t0;
    return n >= 64 ? ~0ull : ((1ull << n) - 1ull);
  };
  auto load_mask_byte = [&](int t0) -> int {
    const int t = t0 + lane;
    return (mk && t < t_end) ? (int)mk[t] : 1;
  };
  auto bits_from_byte = [&](int t0, int byte) -> uint64_t {
    uint64_t rb = range_bits(t0);
    if (!mk) return rb;
    return rb & (uint64_t)__ballot(byte != 0);
  };

  u32x4_t kreg[KI];
  u32x4_t vreg[VI][2];
  auto issue_loads = [&](int t0, uint64_t bits) {
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int f = i * T + tid;
      const int row = f / (D / 8), chk = f % (D / 8);
      if (f < KITEMS && ((bits >> row) & 1ull))
        kreg[i] = ld16(Kg + (int64_t)(t0 + row) * D + 8 * chk);
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int f = i * T + tid;
      const int pr = f / (D / 8), chk = f % (D / 8);
      if (f < VITEMS) {
        if ((bits >> (2 * pr)) & 1ull) vreg[i][0] = ld16(Vg + (int64_t)(t0 + 2 * pr) * D + 8 * chk);
        if ((bits >> (2 * pr + 1)) & 1ull) vreg[i][1] = ld16(Vg + (int64_t)(t0 + 2 * pr + 1) * D + 8 * chk);
      }
    }
  };
  auto store_lds = [&](uint64_t bits) {
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int f = i * T + tid;
      const int row = f / (D / 8), chk = f % (D / 8);
      if (f < KITEMS) st16(&Ks[row * KLD + 8 * chk], kreg[i]);
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int f = i * T + tid;
      const int pr = f / (D / 8), chk = f % (D / 8);
      if (f < VITEMS) {
        // padding and out-of-chunk rows are zero so that P = 0 never meets NaN
        const u32x4_t r0 = ((bits >> (2 * pr)) & 1ull) ? vreg[i][0] : u32x4_t{0, 0, 0, 0};
        const u32x4_t r1 = ((bits >> (2 * pr + 1)) & 1ull) ? vreg[i][1] : u32x4_t{0, 0, 0, 0};
        uint32_t* dst = reinterpret_cast<uint32_t*>(&Vt[(8 * chk) * VLD + 2 * pr]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          dst[(2 * j) * (VLD / 2)] = __builtin_amdgcn_perm(r1[j], r0[j], 0x05040100u);
          dst[(2 * j + 1) * (VLD / 2)] = __builtin_amdgcn_perm(r1[j], r0[j], 0x07060302u);
        }
      }
    }
  };

  f32x16_t o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x16_t{};
  float m_run = kNegInf;   // running max of raw dot products of row 32w + l32
  float l_run = 0.f;       // this lane half's share of the running sum
  const float c2 = a.scale_log2;

  uint64_t bits_cur = 0;
  int mbyte = 1;
  if (ntiles > 0) {
    bits_cur = bits_from_byte(t_begin, load_mask_byte(t_begin));
    if (bits_cur) issue_loads(t_begin, bits_cur);
    if (ntiles > 1) mbyte = load_mask_byte(t_begin + TILE);
  }

  for (int it = 0; it < ntiles; ++it) {
    const int t0 = t_begin + it * TILE;
    __syncthreads();
    if (bits_cur) store_lds(bits_cur);
    __syncthreads();
    uint64_t bits_next = 0;
    if (it + 1 < ntiles) {
      bits_next = bits_from_byte(t0 + TILE, mbyte);
      if (bits_next) issue_loads(t0 + TILE, bits_next);
      if (it + 2 < ntiles) mbyte = load_mask_byte(t0 + 2 * TILE);
    }
    if (bits_cur) {
      // ---- scores S^T for the two 32-token blocks
      f32x16_t s[2];
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2) {
        s[b2] = f32x16_t{};
        const uint16_t* krow = &Ks[(32 * b2 + swap23(l32)) * KLD + 8 * hh];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          s[b2] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(krow + 16 * ks)),
                               qop[ks], s[b2]);
      }
      // register r of lane half hh in block b2 holds token 32*b2 + 16*(r/8) + 8*hh + r%8
      if (bits_cur != ~0ull) {
        const uint64_t lb = bits_cur >> (8 * hh);
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int tk = 32 * b2 + 16 * (r >> 3) + (r & 7);
            if (!((lb >> tk) & 1ull)) s[b2][r] = kNegInf;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float nmc = -m_use * c2;
      if (__ballot(m_new != m_run)) {
        const float alpha = fast_exp2(m_run * c2 + nmc);   // 0 when m_run = -inf
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) o[i] *= alpha;
      }
      m_run = m_new;
      bf16x8_t pk[4];
      float lsum = 0.f;
#pragma unroll
      for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            p[j] = fast_exp2(__builtin_fmaf(s[b2][8 * g + j], c2, nmc));
            lsum += p[j];
          }
          u32x4_t w;
          w[0] = pack_bf16x2(p[0], p[1]);
          w[1] = pack_bf16x2(p[2], p[3]);
          w[2] = pack_bf16x2(p[4], p[5]);
          w[3] = pack_bf16x2(p[6], p[7]);
          pk[2 * b2 + g] = __builtin_bit_cast(bf16x8_t, w);
        }
      l_run += lsum;
      // ---- O^T += V^T P^T ; k-step ks covers tokens 16ks .. 16ks+15
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vrow = &Vt[(32 * db + l32) * VLD + 8 * hh];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          o[db] = mfma32x32x16(__builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(vrow + 16 * ks)),
                               pk[ks], o[db]);
      }
    }
    bits_cur = bits_next;
  }

  // ---- normalise and store this chunk's state
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const bool empty = !(l_tot > 0.f);
  const float inv = empty ? 0.f : 1.f / l_tot;
  const int slot = a.tab.slot[c];
  float* Ob;
  float* Lb;
  if (slot < 0) {
    const int r = -slot - 1;
    Ob = a.O_part + (((int64_t)r * a.B + b) * a.H + h) * (int64_t)a.M * D;
    Lb = a.L_part + (((int64_t)r * a.B + b) * a.H + h) * (int64_t)a.M;
  } else {
    Ob = a.ws_O + (((int64_t)slot * a.B + b) * a.H + h) * (int64_t)a.M * D;
    Lb = a.ws_L + (((int64_t)slot * a.B + b) * a.H + h) * (int64_t)a.M;
  }
  const int m = 32 * wave + l32;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4_t v = {o[db][4 * q] * inv, o[db][4 * q + 1] * inv, o[db][4 * q + 2] * inv, o[db][4 * q + 3] * inv};
      *reinterpret_cast<f32x4_t*>(Ob + (int64_t)m * D + 32 * db + 8 * q + 4 * hh) = v;
    }
  if (hh == 0) Lb[m] = empty ? kNegInf : (m_run * a.scale + __logf(l_tot));
}

bool encode_mfma_supported(int M, int D) {
  return (D == 64 || D == 128) && M % 32 == 0 && M >= 32 && M <= 256;
}

template <int D, int NW>
static hipError_t launch_mfma_t(const EncodeArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.tab.nchunks * a.H * a.B;
  hipLaunchKernelGGL((encode_mfma_kernel<D, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_encode_mfma(const EncodeArgs& a, hipStream_t s) {
  const int NW = a.M / 32;
  if (a.D == 64) {
    switch (NW) {
      case 1: return launch_mfma_t<64, 1>(a, s);
      case 2: return launch_mfma_t<64, 2>(a, s);
      case 3: return launch_mfma_t<64, 3>(a, s);
      case 4: return launch_mfma_t<64, 4>(a, s);
      case 5: return launch_mfma_t<64, 5>(a, s);
      case 6: return launch_mfma_t<64, 6>(a, s);
      case 7: return launch_mfma_t<64, 7>(a, s);
      case 8: return launch_mfma_t<64, 8>(a, s);
    }
  } else if (a.D == 128) {
    switch (NW) {
      case 1: return launch_mfma_t<128, 1>(a, s);
      case 2: return launch_mfma_t<128, 2>(a, s);
      case 3: return launch_mfma_t<128, 3>(a, s);
      case 4: return launch_mfma_t<128, 4>(a, s);
      case 5: return launch_mfma_t<128, 5>(a, s);
      case 6: return launch_mfma_t<128, 6>(a, s);
      case 7: return launch_mfma_t<128, 7>(a, s);
      case 8: return launch_mfma_t<128, 8>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Single latent row (M = 1), bf16: split-KV decoding attention of one query
// against a chunk of keys.  This is a streaming dot-product/axpy over the
// chunk (HBM-bound, one flop pair per byte), done on the vector ALUs: a group
// of D/8 lanes owns one key at a time (16 contiguous bytes per lane, so a wave
// reads whole rows), reduces the dot product across its lanes, and keeps its
// own online-softmax state; the 256/(D/8) group states are merged in LDS.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void encode_q1_kernel(const EncodeArgs a) {
  constexpr int LPK = D / 8;          // lanes per key
  constexpr int G = 256 / LPK;        // key groups per workgroup
  constexpr int U = 4;                // keys per group per iteration
  __shared__ float sm_m[G], sm_l[G];
  __shared__ float sm_acc[G][D];

  const int tid = threadIdx.x;
  const int g = tid / LPK, lig = tid % LPK;
  const int nch = a.tab.nchunks;
  int bid = blockIdx.x;
  const int c = bid % nch;
  bid /= nch;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int t_begin = a.tab.bnd[c], t_end = a.tab.bnd[c + 1];
  const int64_t bh = (int64_t)b * a.H + h;
  const uint16_t* Kg = static_cast<const uint16_t*>(a.K) + bh * (int64_t)a.N * D + 8 * lig;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.V) + bh * (int64_t)a.N * D + 8 * lig;
  const uint16_t* Qg = static_cast<const uint16_t*>(a.Q) + (int64_t)b * a.q_bstride + (int64_t)h * D + 8 * lig;
  const uint8_t* mk = a.mask ? a.mask + (int64_t)b * a.N : nullptr;
  const float c2 = a.scale_log2;

  float q[8];
  {
    const u32x4_t w = ld16(Qg);
#pragma unroll
    for (int j = 0; j < 4; ++j) { q[2 * j] = bf16lo(w[j]); q[2 * j + 1] = bf16hi(w[j]); }
  }
  float m_run = kNegInf, l_run = 0.f, acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;

  for (int base = t_begin; base < t_end; base += G * U) {
    u32x4_t kw[U], vw[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = base + g + G * u;
      ok[u] = t < t_end;
      if (ok[u] && mk) ok[u] = mk[t] != 0;
      if (ok[u]) {
        kw[u] = ld16(Kg + (int64_t)t * D);
        vw[u] = ld16(Vg + (int64_t)t * D);
      } else {
        kw[u] = u32x4_t{0, 0, 0, 0};
        vw[u] = u32x4_t{0, 0, 0, 0};
      }
    }
    float sc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        d = __builtin_fmaf(q[2 * j], bf16lo(kw[u][j]), d);
        d = __builtin_fmaf(q[2 * j + 1], bf16hi(kw[u][j]), d);
      }
#pragma unroll
      for (int o = LPK / 2; o >= 1; o >>= 1) d += __shfl_xor(d, o, 64);
      sc[u] = ok[u] ? d : kNegInf;
    }
    float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float nmc = -m_use * c2;
    const float alpha = fast_exp2(m_run * c2 + nmc);
    float p[U];
#pragma unroll
    for (int u = 0; u < U; ++u) p[u] = fast_exp2(__builtin_fmaf(sc[u], c2, nmc));
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float e = acc[2 * j] * alpha, f = acc[2 * j + 1] * alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        e = __builtin_fmaf(p[u], bf16lo(vw[u][j]), e);
        f = __builtin_fmaf(p[u], bf16hi(vw[u][j]), f);
      }
      acc[2 * j] = e;
      acc[2 * j + 1] = f;
    }
    m_run = m_new;
  }
  if (lig == 0) { sm_m[g] = m_run; sm_l[g] = l_run; }
#pragma unroll
  for (int j = 0; j < 8; ++j) sm_acc[g][8 * lig + j] = acc[j];
  __syncthreads();

  const int slot = a.tab.slot[c];
  float* Ob;
  float* Lb;
  if (slot < 0) {
    const int r = -slot - 1;
    Ob = a.O_part + (((int64_t)r * a.B + b) * a.H + h) * (int64_t)D;
    Lb = a.L_part + (((int64_t)r * a.B + b) * a.H + h);
  } else {
    Ob = a.ws_O + (((int64_t)slot * a.B + b) * a.H + h) * (int64_t)D;
    Lb = a.ws_L + (((int64_t)slot * a.B + b) * a.H + h);
  }
  float M = kNegInf;
  for (int i = 0; i < G; ++i) M = fmaxf(M, sm_m[i]);
  const float Mu = (M == kNegInf) ? 0.f : M;
  float l = 0.f;
  for (int i = 0; i < G; ++i) l += sm_l[i] * fast_exp2((sm_m[i] - Mu) * c2);
  const bool empty = !(l > 0.f);
  if (tid < D) {
    float o = 0.f;
    for (int i = 0; i < G; ++i) o += sm_acc[i][tid] * fast_exp2((sm_m[i] - Mu) * c2);
    Ob[tid] = empty ? 0.f : o / l;
  }
  if (tid == 0) *Lb = empty ? kNegInf : (M * a.scale + __logf(l));
}

bool encode_q1_supported(int M, int D) { return M == 1 && (D == 32 || D == 64 || D == 128); }

hipError_t launch_encode_q1(const EncodeArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.tab.nchunks * a.H * a.B;
  switch (a.D) {
    case 32: hipLaunchKernelGGL(encode_q1_kernel<32>, dim3((unsigned)grid), dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL(encode_q1_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(encode_q1_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// General vector encoder (float32 inputs, or bf16 shapes without a matrix-core
// variant).  One wave per (batch, head, chunk, latent row); a 64-token tile
// gives one score per lane, then lanes switch to head dimensions to
// accumulate the weighted values.  All arithmetic is float32.
// ---------------------------------------------------------------------------
template <typename TIn>
__device__ __forceinline__ float ldv(const TIn* p);
template <>
__device__ __forceinline__ float ldv<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ldv<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename TIn>
__global__ __launch_bounds__(256) void encode_generic_kernel(const EncodeArgs a) {
  constexpr int MAXDL = 4;  // D <= 256
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int nch = a.tab.nchunks;
  const int mgroups = (a.M + 3) / 4;
  int bid = blockIdx.x;
  const int c = bid % nch;
  bid /= nch;
  const int mg = bid % mgroups;
  bid /= mgroups;
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int m = 4 * mg + wave;
  if (m >= a.M) return;
  const int D = a.D;
  const int t_begin = a.tab.bnd[c], t_end = a.tab.bnd[c + 1];
  const int64_t bh = (int64_t)b * a.H + h;
  const TIn* Kg = static_cast<const TIn*>(a.K) + bh * (int64_t)a.N * D;
  const TIn* Vg = static_cast<const TIn*>(a.V) + bh * (int64_t)a.N * D;
  const TIn* Qr = static_cast<const TIn*>(a.Q) + (int64_t)b * a.q_bstride + ((int64_t)h * a.M + m) * D;
  const uint8_t* mk = a.mask ? a.mask + (int64_t)b * a.N : nullptr;
  const float c2 = a.scale_log2;

  float m_run = kNegInf, l_run = 0.f, acc[MAXDL];
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) acc[j] = 0.f;

  for (int t0 = t_begin; t0 < t_end; t0 += 64) {
    const int t = t0 + lane;
    bool ok = t < t_end;
    if (ok && mk) ok = mk[t] != 0;
    float sdot = kNegInf;
    if (ok) {
      const TIn* kr = Kg + (int64_t)t * D;
      float d = 0.f;
      for (int i = 0; i < D; ++i) d = __builtin_fmaf(ldv(Qr + i), ldv(kr + i), d);
      sdot = d;
    }
    const uint64_t okmask = __ballot(ok);
    const float mx = wave_max(sdot);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float nmc = -m_use * c2;
    const float alpha = fast_exp2(m_run * c2 + nmc);
    const float p = ok ? fast_exp2(__builtin_fmaf(sdot, c2, nmc)) : 0.f;
    l_run = l_run * alpha + wave_sum(p);
#pragma unroll
    for (int j = 0; j < MAXDL; ++j) acc[j] *= alpha;
    for (int i = 0; i < 64; ++i) {
      const float pi = __shfl(p, i, 64);
      if (!((okmask >> i) & 1ull)) continue;
      const TIn* vr = Vg + (int64_t)(t0 + i) * D;
#pragma unroll
      for (int j = 0; j < MAXDL; ++j) {
        const int d = lane + 64 * j;
        if (d < D) acc[j] = __builtin_fmaf(pi, ldv(vr + d), acc[j]);
      }
    }
    m_run = m_new;
  }
  const int slot = a.tab.slot[c];
  float* Ob;
  float* Lb;
  if (slot < 0) {
    const int r = -slot - 1;
    Ob = a.O_part + ((((int64_t)r * a.B + b) * a.H + h) * a.M + m) * (int64_t)D;
    Lb = a.L_part + (((int64_t)r * a.B + b) * a.H + h) * a.M + m;
  } else {
    Ob = a.ws_O + ((((int64_t)slot * a.B + b) * a.H + h) * a.M + m) * (int64_t)D;
    Lb = a.ws_L + (((int64_t)slot * a.B + b) * a.H + h) * a.M + m;
  }
  const bool empty = !(l_run > 0.f);
  const float inv = empty ? 0.f : 1.f / l_run;
#pragma unroll
  for (int j = 0; j < MAXDL; ++j) {
    const int d = lane + 64 * j;
    if (d < D) Ob[d] = acc[j] * inv;
  }
  if (lane == 0) *Lb = empty ? kNegInf : (m_run * a.scale + __logf(l_run));
}

hipError_t launch_encode_generic(const EncodeArgs& a, bool bf16, hipStream_t s) {
  const int64_t grid = (int64_t)a.tab.nchunks * ((a.M + 3) / 4) * a.H * a.B;
  if (bf16)
    hipLaunchKernelGGL(encode_generic_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(encode_generic_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace flare
