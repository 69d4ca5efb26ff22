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

template <typename T, typename S, int D, bool CACHE>
__global__ void __launch_bounds__(kRouteWaves * 64) k_route(RouteArgs a) {
  __shared__ RouteShared<kRouteWaves> sh;
  prefetch_kernargs<sizeof(RouteArgs)>();
  const int qi = query_of_slot(blockIdx.x, a.queries, a.group);
  const int kept = route_walk<T, S, D, kRouteWaves, kRouteWaves, CACHE>(a, sh, qi);
  int32_t *out = a.indices + static_cast<int64_t>(qi) * a.beam;
  write_ascending<kRouteWaves * 64>(sh.front, kept, out);
  for (int k = kept + static_cast<int>(threadIdx.x); k < a.beam; k += kRouteWaves * 64) out[k] = -1;
}

template <typename T, typename S, bool CACHE>
hipError_t launch_route_t(int head_dim, const RouteArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.queries));
  const dim3 block(kRouteWaves * 64);
  if (head_dim == 128)
    hipLaunchKernelGGL((k_route<T, S, 128, CACHE>), grid, block, 0, s, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL((k_route<T, S, 64, CACHE>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, typename S>
hipError_t launch_route_ts(int head_dim, const RouteArgs &a, hipStream_t s) {
  return a.cache ? launch_route_t<T, S, true>(head_dim, a, s)
                 : launch_route_t<T, S, false>(head_dim, a, s);
}

}  // namespace

hipError_t launch_route(Dt dt, Dt sdt, int head_dim, const RouteArgs &a, hipStream_t s) {
  if (sdt == Dt::FP8) {  // full tree only
    if (a.cache) return hipErrorInvalidValue;
    return dt == Dt::BF16 ? launch_route_t<bf16_bits, fp8_bits, false>(head_dim, a, s)
                          : launch_route_t<float, fp8_bits, false>(head_dim, a, s);
  }
  if (dt == Dt::BF16)
    return sdt == Dt::BF16 ? launch_route_ts<bf16_bits, bf16_bits>(head_dim, a, s)
                           : launch_route_ts<bf16_bits, float>(head_dim, a, s);
  return sdt == Dt::BF16 ? launch_route_ts<float, bf16_bits>(head_dim, a, s)
                         : launch_route_ts<float, float>(head_dim, a, s);
}

}  // namespace tis
