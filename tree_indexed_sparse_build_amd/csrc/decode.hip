// tree_decode: route then attend for each query in one launch ("Subquadratic
// Attention with a Hierarchical Tree-Structured Indexer", Abstract: routing
// plus final attention is the whole cost of a decode step).
//
// One workgroup of 16 waves per query: route_walk leaves the kept leaves in
// LDS and attend_query gathers them straight away, so the leaf list never
// goes through memory and the step pays for one launch instead of two.  The
// leaves are also written out (ascending) when the caller asks for them.
#include "attend_query.hpp"
#include "route_walk.hpp"

namespace tis {
namespace {

constexpr int kDecodeWaves = 16;

template <typename T, int D>
__global__ void __launch_bounds__(kDecodeWaves * 64) k_decode(RouteArgs ra, AttendArgs aa) {
  __shared__ RouteShared<kDecodeWaves> rsh;
  __shared__ AttendShared<T, D> ash;
  const int64_t qi = blockIdx.x;
  const uint4 qraw = attend_q_raw<T, D>(aa, qi);  // in flight during the walk
  route_walk<T, D, kDecodeWaves>(ra, rsh, qi);
  if (ra.indices) write_ascending<kDecodeWaves * 64>(rsh.front, ra.beam, ra.indices + qi * ra.beam);
  attend_query<T, D>(aa, ash, qi, qraw, rsh.front, nullptr, ra.beam, false);
}

}  // namespace

hipError_t launch_decode(Dt dt, int head_dim, const RouteArgs &ra, const AttendArgs &aa,
                         hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ra.queries));
  const dim3 block(kDecodeWaves * 64);
  if (dt == Dt::BF16 && head_dim == 128)
    hipLaunchKernelGGL((k_decode<bf16_bits, 128>), grid, block, 0, s, ra, aa);
  else if (dt == Dt::BF16 && head_dim == 64)
    hipLaunchKernelGGL((k_decode<bf16_bits, 64>), grid, block, 0, s, ra, aa);
  else if (dt == Dt::F32 && head_dim == 128)
    hipLaunchKernelGGL((k_decode<float, 128>), grid, block, 0, s, ra, aa);
  else if (dt == Dt::F32 && head_dim == 64)
    hipLaunchKernelGGL((k_decode<float, 64>), grid, block, 0, s, ra, aa);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tis
