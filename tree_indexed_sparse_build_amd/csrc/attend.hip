// tree_attend: exact softmax attention over the keys of the selected leaf
// blocks ("Subquadratic Attention with a Hierarchical Tree-Structured
// Indexer", Abstract: the final attention after routing; the NSA / InfLLMv2
// abstract on the Progressive Sparse Attention related-papers page: fine
// softmax attention on the selected tokens).
//
// One workgroup per query: it reads the query's slot list, applies the slot
// rules (repeats count once, negatives are empty, out-of-range gives NaN)
// and runs attend_query.  No global workspace, atomics or device-scope
// fences.
#include "attend_query.hpp"

namespace tis {
namespace {

template <typename T, int D>
__global__ void __launch_bounds__(kAttendMaxWaves * 64) k_attend(AttendArgs a) {
  __shared__ AttendShared<T, D> sh;
  __shared__ int s_idx[kMaxCandidates];
  __shared__ int s_use[kMaxCandidates];
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int64_t qi = blockIdx.x;
  const int W = a.beam;

  // the query row and the slot list are loaded before anything waits on them
  // (the launch gives at least min(W, 16) waves, so tid < W covers W <= 1024)
  const uint4 qraw = attend_q_raw<T, D>(a, qi);
  const int my_idx = tid < W ? a.indices[qi * W + tid] : -1;
  if (tid == 0) s_bad = 0;
  if (tid < W) s_idx[tid] = my_idx;
  __syncthreads();
  for (int s = tid; s < W; s += blockDim.x) {
    const int idx = s_idx[s];
    const bool bad = idx >= a.n_blocks;
    bool use = idx >= 0 && !bad;
    for (int j = 0; j < s && use; ++j) use = s_idx[j] != idx;
    s_use[s] = use;
    if (bad) s_bad = 1;
  }
  __syncthreads();
  attend_query<T, D>(a, sh, qi, qraw, s_idx, s_use, W, s_bad != 0);
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

hipError_t launch_attend(Dt dt, int head_dim, const AttendArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.queries));
  const dim3 block(static_cast<unsigned>(attend_waves(head_dim, dt, a.beam, a.leaf_block) * 64));
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
