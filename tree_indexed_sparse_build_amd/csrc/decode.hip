// tree_decode: route then attend for each query in one launch ("Subquadratic
// Attention with a Hierarchical Tree-Structured Indexer", Abstract: a query
// costs its descent through the tree plus the attention at the end).
//
// One workgroup of 16 waves per query: route_walk leaves the kept leaves in
// LDS and attend_query gathers them straight away, so the leaf list never
// goes through memory and the step pays for one launch instead of two.  The
// leaves are also written out (ascending) when the caller asks for them.
// With few queries each query gets `splits` workgroups that all walk the
// tree and each attend over a share of the kept leaves; a small combine
// kernel merges their partial softmax states.
#include "attend_query.hpp"
#include "route_walk.hpp"

namespace tis {
namespace {

constexpr int kDecodeWaves = 16;
constexpr int kDecodeWalkWaves = 8;  // waves that walk the tree (see route_walk)

template <typename T, typename S, int D, bool CACHE>
__global__ void __launch_bounds__(kDecodeWaves * 64) k_decode(RouteArgs ra, AttendArgs aa) {
  __shared__ RouteShared<kDecodeWaves> rsh;
  __shared__ AttendShared<T, D> ash;
  // part sp of query qi (see k_attend: a query's parts share an XCD)
  const int sp = blockIdx.x / aa.queries;
  const int qi = query_of_slot(blockIdx.x - sp * aa.queries, aa.queries, aa.group);
  const uint4 qraw = attend_q_raw<T, D>(aa, qi);  // in flight during the walk
  // every part walks the tree (the repeated summary reads hit the XCD's L2)
  const int kept = route_walk<T, S, D, kDecodeWaves, kDecodeWalkWaves, CACHE>(ra, rsh, qi);
  if (ra.indices && sp == 0) {
    int32_t *out = ra.indices + static_cast<int64_t>(qi) * ra.beam;
    write_ascending<kDecodeWaves * 64>(rsh.front, kept, out);
    for (int k = kept + static_cast<int>(threadIdx.x); k < ra.beam; k += kDecodeWaves * 64)
      out[k] = -1;
  }
  const int s0 = sp * kept / aa.splits;
  const int s1 = (sp + 1) * kept / aa.splits;
  float *part = aa.splits > 1
                    ? aa.part + (static_cast<int64_t>(qi) * aa.splits + sp) * (D + kPartHeader)
                    : nullptr;
  attend_query<T, D, CACHE>(aa, ash, qi, qraw, rsh.front + s0, nullptr, s1 - s0, false, part);
}

template <typename T, typename S, bool CACHE>
hipError_t launch_decode_t(int head_dim, const RouteArgs &ra, const AttendArgs &aa,
                           hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ra.queries) * static_cast<unsigned>(aa.splits));
  const dim3 block(kDecodeWaves * 64);
  if (head_dim == 128)
    hipLaunchKernelGGL((k_decode<T, S, 128, CACHE>), grid, block, 0, s, ra, aa);
  else if (head_dim == 64)
    hipLaunchKernelGGL((k_decode<T, S, 64, CACHE>), grid, block, 0, s, ra, aa);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, typename S>
hipError_t launch_decode_ts(int head_dim, const RouteArgs &ra, const AttendArgs &aa,
                            hipStream_t s) {
  return ra.cache ? launch_decode_t<T, S, true>(head_dim, ra, aa, s)
                  : launch_decode_t<T, S, false>(head_dim, ra, aa, s);
}

}  // namespace

hipError_t launch_decode(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra,
                         const AttendArgs &aa, hipStream_t s) {
  hipError_t e;
  if (sdt == Dt::FP8) {  // full tree only
    if (ra.cache) return hipErrorInvalidValue;
    e = dt == Dt::BF16 ? launch_decode_t<bf16_bits, fp8_bits, false>(head_dim, ra, aa, s)
                       : launch_decode_t<float, fp8_bits, false>(head_dim, ra, aa, s);
  } else if (dt == Dt::BF16) {
    e = sdt == Dt::BF16 ? launch_decode_ts<bf16_bits, bf16_bits>(head_dim, ra, aa, s)
                        : launch_decode_ts<bf16_bits, float>(head_dim, ra, aa, s);
  } else {
    e = sdt == Dt::BF16 ? launch_decode_ts<float, bf16_bits>(head_dim, ra, aa, s)
                        : launch_decode_ts<float, float>(head_dim, ra, aa, s);
  }
  if (e != hipSuccess || aa.splits <= 1) return e;
  return launch_combine(head_dim, aa, s);
}

}  // namespace tis
