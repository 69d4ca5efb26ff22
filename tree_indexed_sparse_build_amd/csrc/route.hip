// tree_route: top-down beam traversal ("Subquadratic Attention with a
// Hierarchical Tree-Structured Indexer", Abstract: a query descends the
// summary tree one level at a time and ends with a small set of keys).
//
// One workgroup (8 waves) walks one query through every level in a single
// launch (route_walk); the kept leaves are written in ascending order.
#include "route_walk.hpp"

namespace tis {
namespace {

constexpr int kRouteWaves = 8;

template <typename T, int D, bool CACHE>
__global__ void __launch_bounds__(kRouteWaves * 64) k_route(RouteArgs a) {
  __shared__ RouteShared<kRouteWaves> sh;
  const int qi = query_of_slot(blockIdx.x, a.queries, a.group);
  const int kept = route_walk<T, D, kRouteWaves, kRouteWaves, CACHE>(a, sh, qi);
  int32_t *out = a.indices + static_cast<int64_t>(qi) * a.beam;
  write_ascending<kRouteWaves * 64>(sh.front, kept, out);
  for (int k = kept + static_cast<int>(threadIdx.x); k < a.beam; k += kRouteWaves * 64) out[k] = -1;
}

template <bool CACHE>
hipError_t launch_route_layout(Dt dt, int head_dim, const RouteArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.queries));
  const dim3 block(kRouteWaves * 64);
  if (dt == Dt::BF16 && head_dim == 128)
    hipLaunchKernelGGL((k_route<bf16_bits, 128, CACHE>), grid, block, 0, s, a);
  else if (dt == Dt::BF16 && head_dim == 64)
    hipLaunchKernelGGL((k_route<bf16_bits, 64, CACHE>), grid, block, 0, s, a);
  else if (dt == Dt::F32 && head_dim == 128)
    hipLaunchKernelGGL((k_route<float, 128, CACHE>), grid, block, 0, s, a);
  else if (dt == Dt::F32 && head_dim == 64)
    hipLaunchKernelGGL((k_route<float, 64, CACHE>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(Dt dt, int head_dim, const RouteArgs &a, hipStream_t s) {
  return a.cache ? launch_route_layout<true>(dt, head_dim, a, s)
                 : launch_route_layout<false>(dt, head_dim, a, s);
}

}  // namespace tis
