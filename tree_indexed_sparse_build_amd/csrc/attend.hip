// tree_attend: exact softmax attention over the keys of the selected leaf
// blocks ("Subquadratic Attention with a Hierarchical Tree-Structured
// Indexer", Abstract: the attention that follows the descent; the NSA /
// InfLLMv2 abstract on the Progressive Sparse Attention related-papers page:
// exact softmax restricted to the tokens of the chosen blocks).
//
// One workgroup per query (or, when few queries would leave most CUs idle,
// `splits` workgroups per query, each on a share of the slots, the last of
// them to finish merging the parts' states): it reads the query's slot
// list, applies the slot rules (repeats count once, negatives are empty,
// out-of-range gives NaN) and runs attend_query.
#include "attend_query.hpp"

namespace tis {
namespace {

template <typename T, int D>
__global__ void __launch_bounds__(kAttendMaxWaves * 64) k_attend(AttendArgs a) {
  __shared__ AttendShared<T, D> sh;
  __shared__ int s_idx[kMaxCandidates];
  __shared__ int s_use[kMaxCandidates];
  __shared__ int s_bad;
  prefetch_kernargs<sizeof(AttendArgs)>();
  const int tid = threadIdx.x;
  // part sp of query qi; the parts of a query are queries apart in the grid,
  // so with a multiple of 8 queries they land on one XCD and share its L2
  const int sp = div_u(static_cast<int>(blockIdx.x), a.queries);
  const int qi = query_of_slot(blockIdx.x - sp * a.queries, a.queries, a.group);
  const int W = a.beam;

  // the query row and the slot list are loaded before anything waits on them
  const uint4 qraw = attend_q_raw<T, D>(a, qi);
  if (tid == 0) s_bad = 0;
  for (int s = tid; s < W; s += blockDim.x) s_idx[s] = a.indices[static_cast<int64_t>(qi) * W + s];
  __syncthreads();
  for (int s = tid; s < W; s += blockDim.x) {
    const int idx = s_idx[s];
    const bool bad = idx >= a.n_blocks;
    // a repeat of an earlier slot counts once: the earlier slots are read
    // without an early exit, so their LDS reads do not wait on each other
    bool seen = false;
    for (int j = 0; j < s; ++j) seen |= s_idx[j] == idx;
    s_use[s] = idx >= 0 && !bad && !seen;
    if (bad) s_bad = 1;
  }
  __syncthreads();
  const int s0 = div_u(sp * W, a.splits);
  const int s1 = div_u((sp + 1) * W, a.splits);
  float *part = a.splits > 1
                    ? a.part + (static_cast<int64_t>(qi) * a.splits + sp) * (D + kPartHeader)
                    : nullptr;
  attend_query<T, D>(a, sh, qi, qraw, s_idx + s0, s_use + s0, s1 - s0, s_bad != 0, part);
  if (a.splits > 1) merge_parts<D>(a, qi);
}

}  // namespace

int attend_waves(int head_dim, Dt dt, int beam, int leaf_block) {
  int rb;
  if (dt == Dt::BF16)
    rb = head_dim == 128 ? AttendGeom<bf16_bits, 128>::RB : AttendGeom<bf16_bits, 64>::RB;
  else
    rb = head_dim == 128 ? AttendGeom<float, 128>::RB : AttendGeom<float, 64>::RB;
  const int64_t units = static_cast<int64_t>(beam) * ((leaf_block + rb - 1) / rb);
  return static_cast<int>(units < kAttendMaxWaves ? units : kAttendMaxWaves);
}

int attend_splits(int64_t queries, int beam, int leaf_block) {
  // A split query pays three dependent memory round trips at its end
  // (the parts' stores, the arrival count, the merge's loads: ~1 us on
  // MI355X).  Measured on decodes of 128 queries with 512 keys each, that is
  // more than the gather on the idle half of the CUs saves; at 64 queries
  // with 1,024 keys it saves 12% of the decode, at 32 with 512 keys 3%.
  if (queries >= 128 || static_cast<int64_t>(beam) * leaf_block < 512) return 1;
  int s = 1;
  while (s * 2 <= beam && queries * s * 2 <= 256) s *= 2;
  return s;
}

size_t attend_workspace(int64_t queries, int head_dim, int splits) {
  if (splits <= 1) return 0;
  return kArriveBytes +
         static_cast<size_t>(queries) * splits * (head_dim + kPartHeader) * sizeof(float);
}

hipError_t launch_attend(Dt dt, int head_dim, const AttendArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.queries) * static_cast<unsigned>(a.splits));
  const int per = (a.beam + a.splits - 1) / a.splits;
  const dim3 block(static_cast<unsigned>(attend_waves(head_dim, dt, per, a.leaf_block) * 64));
  if (dt == Dt::BF16 && head_dim == 128)
    hipLaunchKernelGGL((k_attend<bf16_bits, 128>), grid, block, 0, s, a);
  else if (dt == Dt::BF16 && head_dim == 64)
    hipLaunchKernelGGL((k_attend<bf16_bits, 64>), grid, block, 0, s, a);
  else if (dt == Dt::F32 && head_dim == 128)
    hipLaunchKernelGGL((k_attend<float, 128>), grid, block, 0, s, a);
  else if (dt == Dt::F32 && head_dim == 64)
    hipLaunchKernelGGL((k_attend<float, 64>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tis
