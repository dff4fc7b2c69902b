// C ABI of libflare: argument validation, work decomposition and launches.
// Declarations and their contract are in include/flare.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/flare.h"
#include "kernels.h"

using namespace flare;

namespace {

thread_local std::string g_err;

flare_status fail(flare_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

flare_status hip_fail(hipError_t e, const char* what) {
  return fail(FLARE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(flare_dtype dt) { return dt == FLARE_BF16 ? 2 : 4; }

// ---------------------------------------------------------------- validation
flare_status check_common(flare_dtype dt, int B, int H, int N, int M, int D) {
  if (dt != FLARE_F32 && dt != FLARE_BF16) return fail(FLARE_EINVAL, "unknown dtype %d", (int)dt);
  if (B < 0 || H < 0 || N < 0 || M < 0 || D < 0)
    return fail(FLARE_EINVAL, "negative size (B=%d H=%d N=%d M=%d D=%d)", B, H, N, M, D);
  if (D % 4 != 0 || D < 4 || D > 256)
    return fail(FLARE_EUNSUPPORTED, "head dimension D=%d unsupported (need D %% 4 == 0, 4 <= D <= 256)", D);
  return FLARE_OK;
}

flare_status check_offsets(int N, int R, const int64_t* off) {
  if (R < 1) return fail(FLARE_EINVAL, "R=%d partitions; need R >= 1", R);
  if (!off) return fail(FLARE_EINVAL, "offsets is NULL");
  if (off[0] != 0) return fail(FLARE_EINVAL, "offsets[0]=%lld, must be 0", (long long)off[0]);
  for (int r = 0; r < R; ++r)
    if (off[r + 1] < off[r])
      return fail(FLARE_EINVAL, "offsets not sorted: offsets[%d]=%lld > offsets[%d]=%lld (partitions must be disjoint)",
                  r, (long long)off[r], r + 1, (long long)off[r + 1]);
  if (off[R] != N) return fail(FLARE_EINVAL, "offsets[R]=%lld must equal N=%d", (long long)off[R], N);
  return FLARE_OK;
}

// ------------------------------------------------------------ work planning
enum class EncKind { Mfma, Q1, Generic };

EncKind encode_kind(flare_dtype dt, int M, int D, bool masked) {
  if (dt == FLARE_BF16 && (encode_mfma_supported(M, D) || encode_ilv_used(M, D, masked))) return EncKind::Mfma;
  if (dt == FLARE_BF16 && encode_q1_supported(M, D)) return EncKind::Q1;
  return EncKind::Generic;
}

struct Chunk {
  int32_t lo, hi;
  int part;
};

struct EncodePlan {
  EncKind kind;
  std::vector<Chunk> chunks;
  std::vector<int> first_chunk;   // per partition, index into chunks; size R+1
  std::vector<int16_t> slot;      // per chunk
  int nslots = 0;
  size_t mw_bytes = 0;    // validity words of the padding mask (matrix-core path)
  int64_t mw_stride = 0;  // words per batch row
  size_t o_bytes = 0;     // partial outputs of split partitions
  size_t order_bytes = 0; // heavy-first launch order (masked matrix-core path)
  size_t ws_bytes = 0;
};

int round_up(int x, int m) { return (x + m - 1) / m * m; }

// Chunk length for a partition of n tokens.
int chunk_len_for(EncKind kind, int B, int H, int R, int M, int D, int64_t max_part, bool masked) {
  if (max_part <= 0) return 1;
  switch (kind) {
    case EncKind::Mfma: {
      // Enough workgroups for one full round of resident workgroups over the
      // 256 CUs, but long enough chunks that the partial states stay a few
      // percent of the K/V bytes (state bytes / K,V bytes = 2M / chunk_len).
      const int64_t base = (int64_t)B * H * R;
      const int64_t target = 256 * (int64_t)encode_mfma_per_cu(M, D, masked);
      const int split = (int)std::max<int64_t>(1, (target + base - 1) / base);
      int len = round_up((int)((max_part + split - 1) / split), 64);
      const int min_len = std::max(1024, 32 * M);
      if (split > 1 && len < min_len) len = min_len;
      return std::max(len, 64);
    }
    case EncKind::Q1:
      return 4096;
    default: {
      // The vector kernel walks a chunk's 64-token tiles one after another
      // (latency-bound), so aim for about 2048 workgroups (one per chunk and
      // group of four latent rows), with chunks of at least 128 tokens.
      const int64_t base = (int64_t)B * H * R * ((M + 3) / 4);
      const int64_t split = std::max<int64_t>(1, (2048 + base - 1) / base);
      const int len = round_up((int)((max_part + split - 1) / split), 64);
      return std::max(len, 128);
    }
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

EncodePlan plan_encode(flare_dtype dt, int B, int H, int N, int M, int D, int R, const int64_t* off, bool masked) {
  EncodePlan p;
  p.kind = encode_kind(dt, M, D, masked);
  int64_t max_part = 0;
  for (int r = 0; r < R; ++r) max_part = std::max<int64_t>(max_part, off[r + 1] - off[r]);
  const int len = chunk_len_for(p.kind, B, H, R, M, D, max_part, masked);
  p.first_chunk.resize(R + 1);
  for (int r = 0; r < R; ++r) {
    p.first_chunk[r] = (int)p.chunks.size();
    const int64_t lo = off[r], hi = off[r + 1];
    const int64_t n = hi - lo;
    if (n <= 0) continue;
    const int64_t k = (n + len - 1) / len;
    // equal pieces rounded up to whole 64-token tiles
    const int64_t piece = ((n + k - 1) / k + 63) / 64 * 64;
    for (int64_t t = lo; t < hi; t += piece) p.chunks.push_back({(int32_t)t, (int32_t)std::min<int64_t>(hi, t + piece), r});
  }
  p.first_chunk[R] = (int)p.chunks.size();
  p.slot.resize(p.chunks.size());
  for (int r = 0; r < R; ++r) {
    const int a = p.first_chunk[r], b = p.first_chunk[r + 1];
    if (b - a == 1) {
      p.slot[a] = (int16_t)(-(r + 1));
    } else {
      for (int i = a; i < b; ++i) p.slot[i] = (int16_t)(p.nslots++);
    }
  }
  const size_t per = (size_t)B * H * M;
  if (masked && p.kind == EncKind::Mfma) {
    p.mw_stride = (N + 63) / 64 + 1;     // one spare word for tiles that straddle the end
    p.mw_bytes = align256((size_t)B * p.mw_stride * sizeof(uint64_t));
  }
  if (p.nslots) p.o_bytes = align256((size_t)p.nslots * per * D * sizeof(float));
  const size_t l_bytes = p.nslots ? align256((size_t)p.nslots * per * sizeof(float)) : 0;
  const int launch_chunks = std::min<int>(kMaxChunks, (int)p.chunks.size());
  if (p.mw_bytes && launch_chunks > 0 && (int64_t)B * launch_chunks <= kMaxOrderItems)
    p.order_bytes = align256((size_t)B * H * launch_chunks * sizeof(int32_t));
  p.ws_bytes = p.mw_bytes + p.o_bytes + l_bytes + p.order_bytes;
  return p;
}

bool plan_fits(const EncodePlan& p, int R) {
  // slots and partition indices must fit the 16-bit table entries
  return p.nslots < 32767 && R < 32767;
}

}  // namespace

// =============================================================== C ABI
extern "C" {

const char* flare_last_error(void) { return g_err.c_str(); }

const char* flare_version(void) { return "libflare 0.1 (gfx950)"; }

size_t flare_encode_workspace_size(flare_dtype dtype, int B, int H, int N, int M, int D, int R,
                                   const int64_t* offsets, int masked) {
  const std::string saved = g_err;
  if (check_common(dtype, B, H, N, M, D) != FLARE_OK || check_offsets(N, R, offsets) != FLARE_OK) {
    g_err = saved;
    return 0;
  }
  return plan_encode(dtype, B, H, N, M, D, R, offsets, masked != 0).ws_bytes;
}

}  // extern "C"

namespace {

// Outputs of the merged form (flare_encode_merge); null: states only.
struct MergeOut {
  uint32_t* counters;
  float* Z;
  float* L;
  void* Z_bf16;
};

flare_status merge_states(int R, int64_t rows, int D, const float* O_part, const float* L_part, float* Z, float* L,
                          void* Z_bf16, hipStream_t s) {
  FoldArgs f;
  memset(&f, 0, sizeof(f));
  f.in_O = O_part;
  f.in_L = L_part;
  f.out_O = Z;
  f.out_L = L;
  f.out_bf16 = static_cast<uint16_t*>(Z_bf16);
  f.rows = rows;
  f.D = D;
  f.tab.ngroups = 1;
  f.tab.in_begin[0] = 0;
  f.tab.in_begin[1] = R;
  f.tab.out_index[0] = 0;
  hipError_t e = launch_fold(f, s);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return FLARE_OK;
}

flare_status encode_impl(flare_dtype dtype, int B, int H, int N, int M, int D, const void* Q,
                         int64_t q_batch_stride, const void* K, const void* V, int R, const int64_t* offsets,
                         const uint8_t* mask, float scale, float* O_part, float* L_part, void* workspace,
                         size_t workspace_bytes, flare_stream_t stream, const MergeOut* mo) {
  flare_status st = check_common(dtype, B, H, N, M, D);
  if (st != FLARE_OK) return st;
  st = check_offsets(N, R, offsets);
  if (st != FLARE_OK) return st;
  if (!std::isfinite(scale)) return fail(FLARE_EINVAL, "scale must be finite");
  if (q_batch_stride < 0) return fail(FLARE_EINVAL, "q_batch_stride must be >= 0");
  if ((int64_t)B * H * M == 0) return FLARE_OK;
  if (!O_part || !L_part) return fail(FLARE_EINVAL, "O_part and L_part must not be NULL");
  if (!Q) return fail(FLARE_EINVAL, "Q must not be NULL");
  if (N > 0 && (!K || !V)) return fail(FLARE_EINVAL, "K and V must not be NULL");
  const EncodePlan plan = plan_encode(dtype, B, H, N, M, D, R, offsets, mask != nullptr);
  if (!plan_fits(plan, R)) return fail(FLARE_EUNSUPPORTED, "too many partitions or chunks (R=%d)", R);
  if (plan.kind != EncKind::Generic) {
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || (q_batch_stride * esize(dtype)) % 16 != 0)
      return fail(FLARE_EINVAL, "Q, K, V and the Q batch stride must be 16-byte aligned");
  }
  if (!aligned16(O_part)) return fail(FLARE_EINVAL, "O_part must be 16-byte aligned");
  if (mo) {
    if (!mo->Z || !mo->L || !mo->counters) return fail(FLARE_EINVAL, "Z, L and counters must not be NULL");
    if (!aligned16(mo->Z)) return fail(FLARE_EINVAL, "Z must be 16-byte aligned");
    if (reinterpret_cast<uintptr_t>(mo->Z_bf16) & 7u) return fail(FLARE_EINVAL, "Z_bf16 must be 8-byte aligned");
    if (reinterpret_cast<uintptr_t>(mo->counters) & 3u) return fail(FLARE_EINVAL, "counters must be 4-byte aligned");
  }
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes)
      return fail(FLARE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", plan.ws_bytes,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(FLARE_EINVAL, "workspace must be 16-byte aligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);

  EncodeArgs a;
  memset(&a, 0, sizeof(a));
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.mask = mask;
  a.O_part = O_part;
  a.L_part = L_part;
  const size_t per = (size_t)B * H * M;
  char* ws = static_cast<char*>(workspace);
  if (plan.mw_bytes) {
    a.mask_words = reinterpret_cast<const uint64_t*>(ws);
    a.mask_words_stride = plan.mw_stride;
  }
  if (plan.nslots) {
    a.ws_O = reinterpret_cast<float*>(ws + plan.mw_bytes);
    a.ws_L = reinterpret_cast<float*>(ws + plan.mw_bytes + plan.o_bytes);
  }
  a.q_bstride = q_batch_stride;
  a.B = B;
  a.H = H;
  a.N = N;
  a.M = M;
  a.D = D;
  a.R = R;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;

  if (plan.mw_bytes) {
    hipError_t e = launch_mask_words(mask, B, N, reinterpret_cast<uint64_t*>(ws), plan.mw_stride, s);
    if (e != hipSuccess) return hip_fail(e, "mask launch");
  }

  // The merge runs inside the matrix-core encoder launch when that one launch
  // holds every chunk (each (batch, head) then has nc workgroups in it).
  const int nc = (int)plan.chunks.size();
  const bool fused = mo && plan.kind == EncKind::Mfma && nc >= 1 && nc <= kMaxChunks && R <= kMaxFuseParts;
  if (fused) {
    a.fz.cnt = mo->counters;
    int nonempty = 0;
    for (int r = 0; r < R; ++r) nonempty += plan.first_chunk[r + 1] > plan.first_chunk[r];
    a.fz.target = nonempty;
    a.fz.Z = mo->Z;
    a.fz.L = mo->L;
    a.fz.Zb = static_cast<uint16_t*>(mo->Z_bf16);
    for (int r = 0; r <= R; ++r) a.fz.pchunk[r] = (int16_t)plan.first_chunk[r];
  }

  // encoder launches over groups of at most kMaxChunks consecutive chunks
  for (int c0 = 0; c0 < nc; c0 += kMaxChunks) {
    const int n = std::min(kMaxChunks, nc - c0);
    a.tab.nchunks = n;
    for (int i = 0; i < n; ++i) {
      a.tab.bnd[i] = plan.chunks[c0 + i].lo;
      a.tab.slot[i] = plan.slot[c0 + i];
    }
    a.tab.bnd[n] = plan.chunks[c0 + n - 1].hi;
    hipError_t e;
    a.order = nullptr;
    if (plan.order_bytes && (int64_t)B * n <= kMaxOrderItems) {
      int32_t* order = reinterpret_cast<int32_t*>(ws + plan.ws_bytes - plan.order_bytes);
      e = launch_heavy_first(a.mask_words, a.mask_words_stride, a.tab, B, H, order, s);
      if (e != hipSuccess) return hip_fail(e, "launch-order launch");
      a.order = order;
    }
    switch (plan.kind) {
      case EncKind::Mfma: e = launch_encode_mfma(a, s); break;
      case EncKind::Q1: e = launch_encode_q1(a, s); break;
      default: e = launch_encode_generic(a, dtype == FLARE_BF16, s); break;
    }
    if (e != hipSuccess) return hip_fail(e, "encode launch");
  }
  if (fused) return FLARE_OK;

  // fold split partitions and write the empty state of empty partitions
  FoldArgs f;
  memset(&f, 0, sizeof(f));
  f.in_O = a.ws_O;
  f.in_L = a.ws_L;
  f.out_O = O_part;
  f.out_L = L_part;
  f.rows = (int64_t)per;
  f.D = D;
  int ng = 0;
  int cursor = 0;   // slots are numbered in partition order, so groups are consecutive
  auto flush = [&]() -> hipError_t {
    if (ng == 0) return hipSuccess;
    f.tab.ngroups = ng;
    hipError_t e = launch_fold(f, s);
    ng = 0;
    return e;
  };
  for (int r = 0; r < R; ++r) {
    const int n = plan.first_chunk[r + 1] - plan.first_chunk[r];
    if (n == 1) continue;   // written directly by the encoder
    if (ng == 0) f.tab.in_begin[0] = cursor;
    f.tab.out_index[ng] = r;
    cursor += n;            // n == 0: an empty group writes (0, -inf)
    f.tab.in_begin[ng + 1] = cursor;
    if (++ng == kMaxGroups) {
      hipError_t e = flush();
      if (e != hipSuccess) return hip_fail(e, "fold launch");
    }
  }
  hipError_t e = flush();
  if (e != hipSuccess) return hip_fail(e, "fold launch");
  if (mo) return merge_states(R, (int64_t)per, D, O_part, L_part, mo->Z, mo->L, mo->Z_bf16, s);
  return FLARE_OK;
}

// ------------------------------------------------- fixed scratch (no allocation)
// flare_encode_noalloc takes its workspace from this array instead of a caller
// buffer.  Each device holds its own copy for the life of the process.  Host
// code never passes the array's name to a kernel (on the host it only stands in
// for the symbol): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current.
constexpr size_t kScratchBytes = FLARE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first
// call on that device).
flare_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FLARE_EUNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || !aligned16(p)) return fail(FLARE_EHIP, "scratch address %p unusable", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FLARE_OK;
}

// ------------------------------------------------- second stream (backward)
// Where the key/value kernel cannot also hold the query-gradient accumulators
// (256 latent rows at head dim 128), the two backward kernels read the same
// inputs and write disjoint outputs, and the first is bound by HBM while the
// second is bound by the matrix cores: the query-gradient kernel runs on a
// second stream of the same device (default priority, not blocking on the null
// stream), ordered after the caller's stream by one event and joined back to it
// by another, so its workgroups fill the CUs that the memory-bound kernel
// leaves.  One such stream per device, created on first use.
std::mutex g_aux_mu;
hipStream_t g_aux[kMaxDevices] = {};

flare_status aux_stream_for(hipStream_t s, hipStream_t* out) {
  int dev = -1;
  hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "device of the stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(FLARE_EUNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_aux_mu);
  if (!g_aux[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    hipStream_t st = nullptr;
    e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) return hip_fail(e, "second stream");
    g_aux[dev] = st;
  }
  *out = g_aux[dev];
  return FLARE_OK;
}

}  // namespace

extern "C" {

flare_status flare_encode_noalloc(flare_dtype dtype, int B, int H, int N, int M, int D, const void* Q,
                                  int64_t q_batch_stride, const void* K, const void* V, int R,
                                  const int64_t* offsets, const uint8_t* mask, float scale, float* O_part,
                                  float* L_part, flare_stream_t stream) {
  // arguments flare_encode would reject are reported by it, unchanged
  size_t need = 0;
  if (check_common(dtype, B, H, N, M, D) == FLARE_OK && check_offsets(N, R, offsets) == FLARE_OK) {
    need = plan_encode(dtype, B, H, N, M, D, R, offsets, mask != nullptr).ws_bytes;
    if (need > kScratchBytes)
      return fail(FLARE_EWORKSPACE,
                  "flare_encode_noalloc: these arguments need %zu bytes of scratch, above its fixed %zu bytes "
                  "(call flare_encode with a workspace instead)",
                  need, kScratchBytes);
  }
  void* ws = nullptr;
  if (need > 0) {
    const flare_status st = scratch_of_current_device(&ws);
    if (st != FLARE_OK) return st;
  }
  return encode_impl(dtype, B, H, N, M, D, Q, q_batch_stride, K, V, R, offsets, mask, scale, O_part, L_part, ws,
                     need > 0 ? kScratchBytes : 0, stream, nullptr);
}

flare_status flare_encode(flare_dtype dtype, int B, int H, int N, int M, int D, const void* Q,
                          int64_t q_batch_stride, const void* K, const void* V, int R,
                          const int64_t* offsets, const uint8_t* mask, float scale, float* O_part,
                          float* L_part, void* workspace, size_t workspace_bytes, flare_stream_t stream) {
  return encode_impl(dtype, B, H, N, M, D, Q, q_batch_stride, K, V, R, offsets, mask, scale, O_part, L_part,
                     workspace, workspace_bytes, stream, nullptr);
}

flare_status flare_encode_merge(flare_dtype dtype, int B, int H, int N, int M, int D, const void* Q,
                                int64_t q_batch_stride, const void* K, const void* V, int R,
                                const int64_t* offsets, const uint8_t* mask, float scale, float* O_part,
                                float* L_part, float* Z, float* L, void* Z_bf16, uint32_t* counters,
                                void* workspace, size_t workspace_bytes, flare_stream_t stream) {
  const MergeOut mo{counters, Z, L, Z_bf16};
  return encode_impl(dtype, B, H, N, M, D, Q, q_batch_stride, K, V, R, offsets, mask, scale, O_part, L_part,
                     workspace, workspace_bytes, stream, &mo);
}

flare_status lse_merge(int R, int64_t rows, int D, const float* O_part, const float* L_part, float* Z,
                       float* L, void* Z_bf16, flare_stream_t stream) {
  if (R < 1) return fail(FLARE_EINVAL, "R=%d; need R >= 1", R);
  if (rows < 0) return fail(FLARE_EINVAL, "rows must be >= 0");
  if (D % 4 != 0 || D < 4 || D > 256) return fail(FLARE_EUNSUPPORTED, "D=%d unsupported", D);
  if (R > 65535) return fail(FLARE_EUNSUPPORTED, "R=%d exceeds 65535 states", R);
  if (rows == 0) return FLARE_OK;
  if (!O_part || !L_part || !Z || !L) return fail(FLARE_EINVAL, "NULL pointer argument");
  if (!aligned16(O_part) || !aligned16(Z)) return fail(FLARE_EINVAL, "O_part and Z must be 16-byte aligned");
  if (Z_bf16 && (reinterpret_cast<uintptr_t>(Z_bf16) & 7u)) return fail(FLARE_EINVAL, "Z_bf16 must be 8-byte aligned");
  return merge_states(R, rows, D, O_part, L_part, Z, L, Z_bf16, static_cast<hipStream_t>(stream));
}

flare_status flare_decode(flare_dtype dtype, int B, int H, int N, int M, int D, const void* Xq,
                          const void* Klat, int64_t klat_batch_stride, const float* Z,
                          const uint8_t* token_mask, float scale, void* Y, flare_stream_t stream) {
  flare_status st = check_common(dtype, B, H, N, M, D);
  if (st != FLARE_OK) return st;
  if (M > 256) return fail(FLARE_EUNSUPPORTED, "decode supports M <= 256 (M=%d)", M);
  if (!std::isfinite(scale)) return fail(FLARE_EINVAL, "scale must be finite");
  if (klat_batch_stride < 0) return fail(FLARE_EINVAL, "klat_batch_stride must be >= 0");
  if ((int64_t)B * H * N == 0) return FLARE_OK;
  if (M == 0) return fail(FLARE_EINVAL, "decode needs M >= 1 latents");
  if (!Xq || !Klat || !Z || !Y) return fail(FLARE_EINVAL, "NULL pointer argument");
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.Xq = Xq;
  a.Klat = Klat;
  a.Z = Z;
  a.token_mask = token_mask;
  a.Y = Y;
  a.klat_bstride = klat_batch_stride;
  a.B = B;
  a.H = H;
  a.N = N;
  a.M = M;
  a.D = D;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == FLARE_BF16 && decode_mfma_supported(M, D)) {
    if (!aligned16(Xq) || !aligned16(Klat) || !aligned16(Y) || (klat_batch_stride * 2) % 16 != 0)
      return fail(FLARE_EINVAL, "Xq, Klat, Y and the Klat batch stride must be 16-byte aligned");
    // One workgroup fills a CU (its LDS holds the staged latents and the
    // waves' rings); aim for about two rounds of workgroups over the chip so
    // the staging is amortised over thousands of tokens.
    const int round = 32 * decode_waves(D);
    const int64_t per_slice = std::max<int64_t>(1, 512 / std::max<int64_t>(1, (int64_t)B * H));
    int tpb = (int)std::min<int64_t>(8192, (N + per_slice - 1) / per_slice);
    tpb = std::min(8192, std::max(round, round_up(tpb, round)));
    a.tokens_per_block = tpb;
    e = launch_decode_mfma(a, s);
  } else {
    e = launch_decode_generic(a, dtype == FLARE_BF16, s);
  }
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return FLARE_OK;
}

}  // extern "C"

namespace {
// Backward plan: the row term c, the mask's validity words and one slot of
// partial query gradients per token chunk (matrix-core path).
struct BwdPlan {
  bool mfma = false;
  std::vector<int32_t> bnd;   // chunk boundaries over [0, N)
  size_t c_bytes = 0, mw_bytes = 0, dq_bytes = 0, order_bytes = 0, ws_bytes = 0;
  int64_t mw_stride = 0;
};

BwdPlan plan_bwd(flare_dtype dt, int B, int H, int N, int M, int D, bool masked) {
  BwdPlan p;
  p.mfma = dt == FLARE_BF16 && bwd_mfma_supported(M, D) && N > 0;
  p.c_bytes = align256((size_t)B * H * M * sizeof(float));
  if (p.mfma) {
    // as many workgroups as the CUs hold at once (one or two per CU, by the
    // key/value kernel's registers and LDS), chunks of whole tiles
    const int64_t bh = std::max<int64_t>(1, (int64_t)B * H);
    // masked inputs: twice the chunks, launched heaviest first, so that the
    // uneven valid lengths even out over the CUs
    const int64_t slots = 256 * (int64_t)bwd_kv_blocks_per_cu(M, D) * (masked ? 2 : 1);
    int64_t per = std::max<int64_t>(1, (slots + bh - 1) / bh);
    int64_t len = ((N + per - 1) / per + 63) / 64 * 64;
    len = std::max<int64_t>(len, 1024);
    while ((N + len - 1) / len > kMaxChunks) len *= 2;
    for (int64_t t = 0; t < N; t += len) p.bnd.push_back((int32_t)t);
    p.bnd.push_back(N);
    const int nslots = (int)p.bnd.size() - 1;
    p.dq_bytes = align256((size_t)nslots * B * H * M * D * sizeof(float));
    if (masked) {
      p.mw_stride = (N + 63) / 64 + 1;
      p.mw_bytes = align256((size_t)B * p.mw_stride * sizeof(uint64_t));
      if ((int64_t)B * nslots <= kMaxOrderItems) p.order_bytes = align256((size_t)B * H * nslots * sizeof(int32_t));
    }
  }
  p.ws_bytes = p.c_bytes + p.mw_bytes + p.dq_bytes + p.order_bytes;
  return p;
}

// Decode backward plan: per-token statistics (log2-normaliser, delta), the
// mask's validity words and per-chunk partial latent gradients (matrix-core
// path).
struct DecBwdPlan {
  bool mfma = false;
  std::vector<int32_t> bnd;   // latent-side chunk boundaries over [0, N)
  int tokens_per_block = 0;   // token side
  int64_t stats_stride = 0, mw_stride = 0;
  size_t stats_bytes = 0, mw_bytes = 0, part_bytes = 0, ws_bytes = 0;
};

DecBwdPlan plan_decode_bwd(flare_dtype dt, int B, int H, int N, int M, int D, bool masked) {
  DecBwdPlan p;
  p.mfma = dt == FLARE_BF16 && decode_bwd_mfma_supported(M, D) && N > 0;
  p.stats_stride = ((int64_t)N + 63) / 64 * 64;
  p.stats_bytes = align256((size_t)B * H * p.stats_stride * sizeof(float));
  if (p.mfma) {
    const int64_t bh = std::max<int64_t>(1, (int64_t)B * H);
    // token side: whole blocks of (waves x 32) tokens, about two workgroups per CU
    const int round = 32 * decode_bwd_waves(D);
    const int64_t per_slice = std::max<int64_t>(1, 512 / bh);
    int tpb = (int)std::min<int64_t>(8192, (N + per_slice - 1) / per_slice);
    p.tokens_per_block = std::min(8192, std::max(round, round_up(tpb, round)));
    // latent side: about two workgroups per CU, chunks of whole tiles
    int64_t per = std::max<int64_t>(1, (512 + bh - 1) / bh);
    int64_t len = std::max<int64_t>(1024, ((N + per - 1) / per + 63) / 64 * 64);
    while ((N + len - 1) / len > kMaxChunks) len *= 2;
    for (int64_t t = 0; t < N; t += len) p.bnd.push_back((int32_t)t);
    p.bnd.push_back(N);
    const int nslots = (int)p.bnd.size() - 1;
    if (masked) {
      p.mw_stride = (N + 63) / 64 + 1;
      p.mw_bytes = align256((size_t)B * p.mw_stride * sizeof(uint64_t));
    }
    p.part_bytes = align256((size_t)nslots * B * H * 2 * M * D * sizeof(float));
  }
  p.ws_bytes = 2 * p.stats_bytes + p.mw_bytes + p.part_bytes;
  return p;
}
}  // namespace

extern "C" {

size_t flare_encode_bwd_workspace_size(flare_dtype dtype, int B, int H, int N, int M, int D, int R,
                                       const int64_t* offsets, int masked) {
  const std::string saved = g_err;
  if (check_common(dtype, B, H, N, M, D) != FLARE_OK || check_offsets(N, R, offsets) != FLARE_OK) {
    g_err = saved;
    return 0;
  }
  return plan_bwd(dtype, B, H, N, M, D, masked != 0).ws_bytes;
}

flare_status flare_encode_bwd(flare_dtype dtype, int B, int H, int N, int M, int D, const void* Q,
                              int64_t q_batch_stride, const void* K, const void* V, int R,
                              const int64_t* offsets, const uint8_t* mask, float scale, const float* Z,
                              const float* L, const void* dZ, float* dQ, void* dK, void* dV, void* dQ_cast,
                              int flags, void* workspace, size_t workspace_bytes, flare_stream_t stream) {
  flare_status st = check_common(dtype, B, H, N, M, D);
  if (st != FLARE_OK) return st;
  st = check_offsets(N, R, offsets);
  if (st != FLARE_OK) return st;
  if (!std::isfinite(scale)) return fail(FLARE_EINVAL, "scale must be finite");
  if (q_batch_stride < 0) return fail(FLARE_EINVAL, "q_batch_stride must be >= 0");
  if (flags & ~(FLARE_BWD_ACCUMULATE_DQ | FLARE_BWD_ACCUMULATE_DK | FLARE_BWD_ACCUMULATE_DV))
    return fail(FLARE_EINVAL, "unknown flags");
  if ((int64_t)B * H == 0) return FLARE_OK;
  if ((int64_t)M > 0 && (!Q || !Z || !L || !dZ || !dQ)) return fail(FLARE_EINVAL, "NULL pointer argument");
  if (N > 0 && (!K || !V || !dK || !dV)) return fail(FLARE_EINVAL, "NULL pointer argument");
  const BwdPlan plan = plan_bwd(dtype, B, H, N, M, D, mask != nullptr);
  if ((int)plan.bnd.size() - 1 > kMaxChunks) return fail(FLARE_EUNSUPPORTED, "too many backward chunks");
  if (!workspace || workspace_bytes < plan.ws_bytes)
    return fail(FLARE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(FLARE_EINVAL, "workspace must be 16-byte aligned");
  if (plan.mfma) {
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(dZ) || !aligned16(dQ) ||
        !aligned16(dK) || !aligned16(dV) || !aligned16(dQ_cast) ||
        (q_batch_stride * 2) % 16 != 0)
      return fail(FLARE_EINVAL, "Q, K, V, dZ, dQ, dK, dV and the Q batch stride must be 16-byte aligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  BwdArgs a;
  memset(&a, 0, sizeof(a));
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.mask = mask;
  a.Z = Z;
  a.L = L;
  a.dZ = dZ;
  a.c = reinterpret_cast<float*>(ws);
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.q_bstride = q_batch_stride;
  a.B = B;
  a.H = H;
  a.N = N;
  a.M = M;
  a.D = D;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dQ_cast = dQ_cast;
  a.accumulate_dq = (flags & FLARE_BWD_ACCUMULATE_DQ) != 0;
  a.accumulate_dk = (flags & FLARE_BWD_ACCUMULATE_DK) != 0;
  a.accumulate_dv = (flags & FLARE_BWD_ACCUMULATE_DV) != 0;
  const bool bf16 = dtype == FLARE_BF16;
  hipError_t e = launch_bwd_rowdot(dZ, bf16, Z, (int64_t)B * H * M, D, reinterpret_cast<float*>(ws), s);
  if (e != hipSuccess) return hip_fail(e, "backward row-term launch");
  if (!plan.mfma) {
    e = launch_bwd_generic(a, bf16, s);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return FLARE_OK;
  }
  if (plan.mw_bytes) {
    a.mask_words = reinterpret_cast<const uint64_t*>(ws + plan.c_bytes);
    a.mask_words_stride = plan.mw_stride;
    e = launch_mask_words(mask, B, N, reinterpret_cast<uint64_t*>(ws + plan.c_bytes), plan.mw_stride, s);
    if (e != hipSuccess) return hip_fail(e, "mask launch");
  }
  a.ws_dq = reinterpret_cast<float*>(ws + plan.c_bytes + plan.mw_bytes);
  const int nc = (int)plan.bnd.size() - 1;
  a.tab.nchunks = nc;
  for (int i = 0; i <= nc; ++i) a.tab.bnd[i] = plan.bnd[i];
  for (int i = 0; i < nc; ++i) a.tab.slot[i] = (int16_t)i;
  if (plan.order_bytes) {
    int32_t* order = reinterpret_cast<int32_t*>(ws + plan.c_bytes + plan.mw_bytes + plan.dq_bytes);
    e = launch_heavy_first(a.mask_words, a.mask_words_stride, a.tab, B, H, order, s);
    if (e != hipSuccess) return hip_fail(e, "launch-order launch");
    a.order = order;
  }
  // one pass over K, V where the registers allow the fused kernel, else a
  // separate query-gradient pass; both leave per-chunk partials for the reduce
  const bool fuse = bwd_kv_fuses_dq(M, D);
  if (fuse) {
    e = launch_bwd_kv_mfma(a, s);
    if (e != hipSuccess) return hip_fail(e, "key/value-gradient launch");
  } else {
    // the query-gradient kernel on the second stream, alongside the key/value kernel
    hipStream_t aux = nullptr;
    st = aux_stream_for(s, &aux);
    if (st != FLARE_OK) return st;
    hipEvent_t ev[2] = {nullptr, nullptr};
    auto done = [&](hipError_t err, const char* what) -> flare_status {
      for (hipEvent_t x : ev)
        if (x) (void)hipEventDestroy(x);
      return err == hipSuccess ? FLARE_OK : hip_fail(err, what);
    };
    for (hipEvent_t& x : ev)
      if ((e = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess) return done(e, "event");
    if ((e = hipEventRecord(ev[0], s)) != hipSuccess) return done(e, "event record");
    if ((e = hipStreamWaitEvent(aux, ev[0], 0)) != hipSuccess) return done(e, "stream wait");
    if ((e = launch_bwd_dq_mfma(a, aux)) != hipSuccess) return done(e, "query-gradient launch");
    if ((e = hipEventRecord(ev[1], aux)) != hipSuccess) return done(e, "event record");
    if ((e = launch_bwd_kv_mfma(a, s)) != hipSuccess) return done(e, "key/value-gradient launch");
    if ((e = hipStreamWaitEvent(s, ev[1], 0)) != hipSuccess) return done(e, "stream wait");
    st = done(hipSuccess, "");
    if (st != FLARE_OK) return st;
  }
  // partials that already carry s (the fused kernel contracting s dS) are summed as they are
  e = launch_bwd_dq_reduce(a.ws_dq, nc, (int64_t)B * H * M * D, bwd_kv_partials_scaled(M, D) ? 1.f : scale, dQ,
                           a.accumulate_dq != 0, dQ_cast, s);
  if (e != hipSuccess) return hip_fail(e, "query-gradient reduce launch");
  return FLARE_OK;
}


size_t flare_decode_bwd_workspace_size(flare_dtype dtype, int B, int H, int N, int M, int D, int masked) {
  const std::string saved = g_err;
  if (check_common(dtype, B, H, N, M, D) != FLARE_OK || M > 256) {
    g_err = saved;
    return 0;
  }
  return plan_decode_bwd(dtype, B, H, N, M, D, masked != 0).ws_bytes;
}

flare_status flare_decode_bwd(flare_dtype dtype, int B, int H, int N, int M, int D, const void* Xq,
                              const void* Klat, int64_t klat_batch_stride, const float* Z,
                              const uint8_t* token_mask, float scale, const void* dY, void* dXq, float* dKlat,
                              float* dZ, void* dZ_cast, void* workspace, size_t workspace_bytes,
                              flare_stream_t stream) {
  flare_status st = check_common(dtype, B, H, N, M, D);
  if (st != FLARE_OK) return st;
  if (M > 256) return fail(FLARE_EUNSUPPORTED, "decode supports M <= 256 (M=%d)", M);
  if (!std::isfinite(scale)) return fail(FLARE_EINVAL, "scale must be finite");
  if (klat_batch_stride < 0) return fail(FLARE_EINVAL, "klat_batch_stride must be >= 0");
  if ((int64_t)B * H == 0) return FLARE_OK;
  if (M == 0) return fail(FLARE_EINVAL, "decode needs M >= 1 latents");
  if (!Klat || !Z || !dKlat || !dZ) return fail(FLARE_EINVAL, "NULL pointer argument");
  if (N > 0 && (!Xq || !dY || !dXq)) return fail(FLARE_EINVAL, "NULL pointer argument");
  const DecBwdPlan plan = plan_decode_bwd(dtype, B, H, N, M, D, token_mask != nullptr);
  if (!workspace || workspace_bytes < plan.ws_bytes)
    return fail(FLARE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", plan.ws_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(FLARE_EINVAL, "workspace must be 16-byte aligned");
  if (plan.mfma && (!aligned16(Xq) || !aligned16(Klat) || !aligned16(dY) || !aligned16(dXq) ||
                    !aligned16(Z) || !aligned16(dKlat) || !aligned16(dZ) || !aligned16(dZ_cast) ||
                    (klat_batch_stride * 2) % 16 != 0))
    return fail(FLARE_EINVAL, "Xq, Klat, Z, dY and the gradients must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  DecBwdArgs a;
  memset(&a, 0, sizeof(a));
  a.Xq = Xq;
  a.Klat = Klat;
  a.Z = Z;
  a.token_mask = token_mask;
  a.dY = dY;
  a.dXq = dXq;
  a.dKlat = dKlat;
  a.dZ = dZ;
  a.dZ_cast = dZ_cast;
  a.stats_stride = plan.stats_stride;
  a.lse2 = reinterpret_cast<float*>(ws);
  a.delta = reinterpret_cast<float*>(ws + plan.stats_bytes);
  a.klat_bstride = klat_batch_stride;
  a.B = B;
  a.H = H;
  a.N = N;
  a.M = M;
  a.D = D;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  const bool bf16 = dtype == FLARE_BF16;
  hipError_t e;
  if (!plan.mfma) {
    e = launch_decode_bwd_generic(a, bf16, s);
    if (e != hipSuccess) return hip_fail(e, "decode backward launch");
    return FLARE_OK;
  }
  char* p = ws + 2 * plan.stats_bytes;
  if (plan.mw_bytes) {
    a.mask_words = reinterpret_cast<const uint64_t*>(p);
    a.mask_words_stride = plan.mw_stride;
    e = launch_mask_words(token_mask, B, N, reinterpret_cast<uint64_t*>(p), plan.mw_stride, s);
    if (e != hipSuccess) return hip_fail(e, "mask launch");
    p += plan.mw_bytes;
  }
  a.ws_part = reinterpret_cast<float*>(p);
  a.tokens_per_block = plan.tokens_per_block;
  const int nc = (int)plan.bnd.size() - 1;
  a.tab.nchunks = nc;
  for (int i = 0; i <= nc; ++i) a.tab.bnd[i] = plan.bnd[i];
  for (int i = 0; i < nc; ++i) a.tab.slot[i] = (int16_t)i;
  e = launch_decode_bwd_mfma(a, s);
  if (e != hipSuccess) return hip_fail(e, "decode backward launch");
  e = launch_decode_bwd_reduce(a, bf16, s);
  if (e != hipSuccess) return hip_fail(e, "decode backward reduce launch");
  return FLARE_OK;
}

}  // extern "C"
