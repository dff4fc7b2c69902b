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
    // n >= 0; a group without states writes the empty state
    const MState cur = fold_states(a.in_O, a.in_L, s0, s1 - s0, a.rows, row, off, sstride);
    store_state(cur, a.out_O, a.out_L, a.out_bf16, a.tab.out_index[g], a.rows, row, off, sstride, a.D);
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
