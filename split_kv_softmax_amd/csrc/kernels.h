// Launch-side interface between the C ABI (capi.hip) and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flare {

// A launch covers up to kMaxChunks token chunks; chunk c of the launch spans
// tokens [bnd[c], bnd[c+1]) of every (batch, head) slice, and lies inside one
// partition.  slot[c] >= 0 sends its state to workspace slot slot[c]; a
// negative slot -(r+1) means the chunk is all of partition r and writes
// O_part[r] / L_part[r] directly.
constexpr int kMaxChunks = 256;

struct ChunkTable {
  int nchunks;
  int32_t bnd[kMaxChunks + 1];
  int16_t slot[kMaxChunks];
};

// Fused merge of an encoder launch.  Partition r owns chunks [pchunk[r],
// pchunk[r+1]) of the chunk table.  A workgroup whose chunk is a whole
// partition adds one to the slice counter cnt[b*H + h] once its state is
// stored; one whose partition is split adds one to the partition counter
// cnt[B*H + (b*H + h)*R + r], and the workgroup that completes that count
// folds the partition's chunk states into O_part / L_part and then adds one
// to the slice counter.  The workgroup that brings the slice counter to
// `target` (the nonempty partitions) writes the empty state of empty
// partitions and merges the R partition states into Z / L (and the bfloat16
// copy Zb when set).  Each completing workgroup puts its counter back to 0.
// cnt == null: no merge.
constexpr int kMaxFuseParts = 256;
struct FuseTable {
  uint32_t* cnt;   // [B*H*(R+1)], 0 on entry
  int target;
  float* Z;        // [B,H,M,D]
  float* L;        // [B,H,M]
  uint16_t* Zb;    // nullable [B,H,M,D]
  int16_t pchunk[kMaxFuseParts + 1];
};

struct EncodeArgs {
  const void* Q;
  const void* K;
  const void* V;
  const uint8_t* mask;
  const uint64_t* mask_words;   // [B, mask_words_stride] validity words (matrix-core path)
  int64_t mask_words_stride;
  float* O_part;   // [R,B,H,M,D]
  float* L_part;   // [R,B,H,M]
  float* ws_O;     // [slots,B,H,M,D]
  float* ws_L;     // [slots,B,H,M]
  int64_t q_bstride;
  int B, H, N, M, D, R;
  float scale;        // s
  float scale_log2;   // s * log2(e)
  ChunkTable tab;
  const int32_t* order;   // launch order of the (b, h, chunk) blocks, heaviest first, or null
  FuseTable fz;
};

// Group g folds input states [in_begin[g], in_begin[g+1]) of `in` into output
// state out_index[g]; an empty group writes the empty state (0, -inf).
constexpr int kMaxGroups = 256;
struct FoldTable {
  int ngroups;
  int32_t in_begin[kMaxGroups + 1];
  int32_t out_index[kMaxGroups];
};

struct FoldArgs {
  const float* in_O;   // [S, rows, D]
  const float* in_L;   // [S, rows]
  float* out_O;        // [G, rows, D]
  float* out_L;        // [G, rows]
  uint16_t* out_bf16;  // nullable [G, rows, D]
  int64_t rows;
  int D;
  FoldTable tab;
};

struct DecodeArgs {
  const void* Xq;
  const void* Klat;
  const float* Z;
  const uint8_t* token_mask;
  void* Y;
  int64_t klat_bstride;
  int B, H, N, M, D;
  float scale_log2;
  int tokens_per_block;   // tokens handled by one workgroup
};

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const uint8_t* mask;
  const uint64_t* mask_words;   // validity words (matrix-core path)
  int64_t mask_words_stride;
  const float* Z;
  const float* L;
  const void* dZ;
  const float* c;               // [B,H,M] rowsum(dZ * Z)
  float* dQ;                    // [B,H,M,D]
  void* dK;                     // [B,H,N,D]
  void* dV;
  float* ws_dq;                 // [chunks,B,H,M,D] partial query gradients (matrix-core path)
  void* dQ_cast;                // [B,H,M,D] dQ also in the input dtype, or null
  int accumulate_dq;            // dQ += instead of dQ =
  int accumulate_dk;            // dK += instead of dK =
  int accumulate_dv;            // dV += instead of dV =
  int64_t q_bstride;
  int B, H, N, M, D;
  float scale;
  float scale_log2;
  ChunkTable tab;               // token chunks (matrix-core path)
  const int32_t* order;         // launch order of the (b, h, chunk) blocks, heaviest first, or null
};

struct DecBwdArgs {
  const void* Xq;               // [B,H,N,D] token queries
  const void* Klat;             // [B|1,H,M,D] latent keys
  const float* Z;               // [B,H,M,D] latent values
  const uint8_t* token_mask;    // [B,N] or null
  const uint64_t* mask_words;   // validity words of token_mask (matrix-core path)
  int64_t mask_words_stride;
  const void* dY;               // [B,H,N,D]
  void* dXq;                    // [B,H,N,D]
  float* dKlat;                 // [B,H,M,D]
  float* dZ;                    // [B,H,M,D]
  void* dZ_cast;                // [B,H,M,D] in the input dtype, or null
  float* lse2;                  // [B*H, stats_stride] per-token log2-normaliser of the scaled scores
  float* delta;                 // [B*H, stats_stride] per-token sum_m A dA
  int64_t stats_stride;         // N rounded up to whole 64-token tiles
  float* ws_part;               // [chunks, B*H, 2, M, D] partial dZ and dKlat/s (matrix-core path)
  int64_t klat_bstride;
  int B, H, N, M, D;
  float scale, scale_log2;
  int tokens_per_block;         // token side (matrix-core path)
  ChunkTable tab;               // latent side chunks (matrix-core path)
};

// Encoder kernels. Return hipSuccess or the launch error.
bool encode_mfma_supported(int M, int D);
int encode_mfma_per_cu(int M, int D, bool masked);   // resident workgroups per CU of the chosen variant
bool encode_ilv_used(int M, int D, bool masked);     // the pipelined encoder serves this shape
hipError_t launch_encode_mfma(const EncodeArgs& a, hipStream_t s);
bool encode_q1_supported(int M, int D);
hipError_t launch_encode_q1(const EncodeArgs& a, hipStream_t s);
hipError_t launch_encode_generic(const EncodeArgs& a, bool bf16, hipStream_t s);
hipError_t launch_mask_words(const uint8_t* mask, int B, int N, uint64_t* words, int64_t stride, hipStream_t s);
// Heavy-first launch order for masked inputs.  Block (b, h, c) of a chunked
// launch is numbered (b*H + h)*nchunks + c; order[i] is the block that the i-th
// launched workgroup runs.  The (batch, chunk) pairs are ranked by their count
// of valid tokens (descending, ties in index order), every head of a pair
// following it, so that the long chunks start first and the short ones fill in.
// At most kMaxOrderItems pairs (B * nchunks); order holds B*H*nchunks entries.
constexpr int kMaxOrderItems = 1024;
hipError_t launch_heavy_first(const uint64_t* mask_words, int64_t mw_stride, const ChunkTable& tab, int B, int H,
                              int32_t* order, hipStream_t s);

hipError_t launch_fold(const FoldArgs& a, hipStream_t s);

hipError_t launch_bwd_rowdot(const void* dZ, bool bf16, const float* Z, int64_t rows, int D, float* c,
                             hipStream_t s);
hipError_t launch_bwd_generic(const BwdArgs& a, bool bf16, hipStream_t s);
bool bwd_mfma_supported(int M, int D);
hipError_t launch_bwd_dq_mfma(const BwdArgs& a, hipStream_t s);
// whether the key/value gradient kernel of this shape also writes the
// query-gradient chunk partials (where the registers allow it); where it does
// not, launch_bwd_dq_mfma runs first
bool bwd_kv_fuses_dq(int M, int D);
// whether the query-gradient chunk partials already carry the scale s (else
// the reduce applies it)
bool bwd_kv_partials_scaled(int M, int D);
// workgroups of the key/value gradient kernel one CU holds at once (its
// registers and LDS), which sizes the token chunks of the backward
int bwd_kv_blocks_per_cu(int M, int D);
hipError_t launch_bwd_kv_mfma(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_dq_reduce(const float* ws, int nslots, int64_t elems, float scale, float* dQ, bool accumulate,
                                void* dQ_cast, hipStream_t s);
hipError_t launch_bwd_kv_generic(const BwdArgs& a, bool bf16, hipStream_t s);

hipError_t launch_decode_bwd_generic(const DecBwdArgs& a, bool bf16, hipStream_t s);
bool decode_bwd_mfma_supported(int M, int D);
int decode_bwd_waves(int D);
hipError_t launch_decode_bwd_mfma(const DecBwdArgs& a, hipStream_t s);
hipError_t launch_decode_bwd_reduce(const DecBwdArgs& a, bool bf16, hipStream_t s);

bool decode_mfma_supported(int M, int D);
int decode_waves(int D);
hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_generic(const DecodeArgs& a, bool bf16, hipStream_t s);

}  // namespace flare
