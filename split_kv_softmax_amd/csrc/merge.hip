// Cross-partition merge of (O_r, L_r) states ("FLARE++: Low-rank attention
// with dynamic attention routing", appendix on context parallelism, eqs.
// 21-23 and the max-stabilised merge paragraph), evaluated as the balanced
// binary tree of "Ring vs. Tree Attention" (two topologies section and the
// semigroup proposition): leaves (m, l, acc) = (L_r, 1, O_r), empty leaves
// (-inf, 0, 0); round k merges state i with state i + 2^k for i = 0 mod 2^(k+1)
// and a state without a partner passes through; one merge takes
// m = max(m1, m2), l = l1 e^(m1-m) + l2 e^(m2-m), acc = acc1 e^(m1-m) + acc2 e^(m2-m).
//
// A thread owns one (row, 4 columns).  Up to 16 states it loads them all at
// once and runs the rounds of the 16-leaf tree on them (absent leaves empty).
// Beyond that it visits the leaves in order keeping one partial state per tree
// level (a binary counter): after leaf i the levels whose bit is set in i are
// merged into it.  Because i is the same for every thread the branches are
// uniform and the level slots stay in registers.  Leftover levels are merged
// from the lowest upwards, which is exactly the round schedule above with its
// pass-through survivors.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace flare {

namespace {
constexpr int kLevels = 16;   // up to 65536 states per group
constexpr int kBatch = 16;    // leaves loaded together (all in flight at once)

struct St {
  float m, l;
  f32x4_t acc;
};

__device__ __forceinline__ St merge_st(const St& x, const St& y) {
  St r;
  r.m = fmaxf(x.m, y.m);
  if (r.m == kNegInf) return St{kNegInf, 0.f, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  const float fx = __expf(x.m - r.m);   // exactly 0 for an empty side
  const float fy = __expf(y.m - r.m);
  r.l = x.l * fx + y.l * fy;
  r.acc = x.acc * fx + y.acc * fy;
  return r;
}
}  // namespace

// Grid-stride over (group, row, 4-column piece); one piece per thread and step.
__global__ __launch_bounds__(256) void fold_kernel(const FoldArgs a) {
  const int D4 = a.D >> 2;
  const int64_t per_group = a.rows * D4;
  const int64_t total = per_group * a.tab.ngroups;
  const int64_t sstride = a.rows * a.D;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < total;
       w += (int64_t)gridDim.x * blockDim.x) {
    const int g = (int)(w / per_group);
    const int64_t e = w - (int64_t)g * per_group;      // (row, piece) within the group
    const int64_t row = e / D4;
    const int64_t off = 4 * e;                          // = row * D + 4 * piece
    const int s0 = a.tab.in_begin[g], s1 = a.tab.in_begin[g + 1];
    const int n = s1 - s0;     // >= 0; a group without states writes the empty state

    St cur{kNegInf, 0.f, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    if (n == 0) {
      // no states: the empty state
    } else if (n <= kBatch) {
      // Up to 16 states: every load issued at once (indices past the group
      // re-read its last state), absent leaves replaced by empty states, and
      // the four rounds of the 16-leaf tree.  Merging a state with an empty
      // one returns it bit for bit (factor exp(0) = 1 on its side, exactly 0
      // on the empty side), so this is the tree with pass-through survivors.
      St t[kBatch];
      float Lb[kBatch];
      f32x4_t Ob[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int64_t s = s0 + (k < n ? k : n - 1);
        Lb[k] = a.in_L[s * a.rows + row];
        Ob[k] = *reinterpret_cast<const f32x4_t*>(a.in_O + s * sstride + off);
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const bool leaf = k < n && Lb[k] != kNegInf;
        t[k].m = leaf ? Lb[k] : kNegInf;
        t[k].l = leaf ? 1.f : 0.f;
        t[k].acc = leaf ? Ob[k] : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int w2 = 1; w2 < kBatch; w2 *= 2)
#pragma unroll
        for (int i = 0; i < kBatch; i += 2 * w2) t[i] = merge_st(t[i], t[i + w2]);
      cur = t[0];
    } else {
      St lv[kLevels];
      for (int i0 = 0; i0 < n; i0 += kBatch) {
        float Lb[kBatch];
        f32x4_t Ob[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int64_t s = s0 + (i0 + k < n ? i0 + k : n - 1);
          Lb[k] = a.in_L[s * a.rows + row];
          Ob[k] = *reinterpret_cast<const f32x4_t*>(a.in_O + s * sstride + off);
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int i = i0 + k;
          if (i < n) {
            St leaf;
            leaf.m = Lb[k];
            leaf.l = (leaf.m == kNegInf) ? 0.f : 1.f;
            leaf.acc = (leaf.m == kNegInf) ? f32x4_t{0.f, 0.f, 0.f, 0.f} : Ob[k];
            // carry: merge the completed left subtrees of equal size into the
            // new leaf; the first level whose bit is clear in i takes the result
            bool carry = true;
#pragma unroll
            for (int lvl = 0; lvl < kLevels; ++lvl) {
              if (carry) {
                if ((i >> lvl) & 1) {
                  leaf = merge_st(lv[lvl], leaf);
                } else {
                  lv[lvl] = leaf;
                  carry = false;
                }
              }
            }
          }
        }
      }
      // collect the levels still occupied (bits of n), lowest first
      bool have = false;
#pragma unroll
      for (int lvl = 0; lvl < kLevels; ++lvl) {
        if ((n >> lvl) & 1) {
          cur = have ? merge_st(lv[lvl], cur) : lv[lvl];
          have = true;
        }
      }
    }
    const int oi = a.tab.out_index[g];
    const bool empty = !(cur.l > 0.f);
    const float inv = empty ? 0.f : 1.f / cur.l;
    f32x4_t z = cur.acc * inv;
    if (empty) z = f32x4_t{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4_t*>(a.out_O + (int64_t)oi * sstride + off) = z;
    if (off % a.D == 0) a.out_L[(int64_t)oi * a.rows + row] = empty ? kNegInf : cur.m + __logf(cur.l);
    if (a.out_bf16) {
      const u32x2_t wv = {pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
      *reinterpret_cast<u32x2_t*>(a.out_bf16 + (int64_t)oi * sstride + off) = wv;
    }
  }
}

hipError_t launch_fold(const FoldArgs& a, hipStream_t s) {
  const int64_t total = a.rows * (a.D / 4) * a.tab.ngroups;
  if (total == 0) return hipSuccess;
  // a few workgroups per CU; each thread walks the pieces grid-stride
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 2048);
  hipLaunchKernelGGL(fold_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace flare
