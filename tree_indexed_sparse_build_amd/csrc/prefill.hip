// Causal prefill routing: the query at position t routes over the tree of
// the first t + 1 keys and attends over the keys of its kept leaves up to t
// ("Vdev-Ctrl Releases ALHR", Summary: keys read per query averaged over the
// positions of a 1,024-token input; "Subquadratic Attention with a
// Hierarchical Tree-Structured Indexer", Abstract: the tree over the KV cache
// deepens as the context grows).  Position t sees the growing-cache tree at
// n = t + 1: every node to the left of key t is complete and its summary is
// the one a tree over all n keys stores; only the node holding key t at each
// height (the open node) covers fewer keys, and its mean differs per t.
//
//  * k_block_sums + k_sum_up: fp64 key sums in a hierarchy of factor 64
//    (runs of 64, 4096, ... positions), each key read once.
//  * k_prefix_means: for every height h of the tree and every position t,
//    the mean of the keys from the start of t's height-h node up to t (the
//    open node's summary as position t sees it), summed in fp64 and rounded
//    once to the summary type.  One workgroup per (head, height, block of 64
//    positions), a thread per column: it adds up the node's keys that lie
//    before the block from the hierarchy (at most 63 keys, then at most 2 *
//    63 sums a level), then walks the block in key order.
//  * k_prefill: one workgroup per (batch, query head, position), of one
//    wave when a level has at most 32 candidates (beam * b), 2 waves up to
//    64, 4 up to 128, else 8: a prefill query reads few keys, so small workgroups (LDS
//    sized to them) keep more positions in flight on each CU (measured: 8
//    waves 1.5-1.8x the rate of 16).  Wave 0
//    builds the position's level table (depth, existing nodes, first cut, the
//    open rows' offsets) in LDS, a lane per level; the walk reads complete
//    nodes from the
//    cache tree and the open node of each level from the table of partial
//    means; the attention stops at key t.
#include "attend_query.hpp"
#include "route_walk.hpp"

namespace tis {
namespace {

template <typename T> __device__ inline double elem64(const T *p);
template <> __device__ inline double elem64<float>(const float *p) { return *p; }
template <> __device__ inline double elem64<bf16_bits>(const bf16_bits *p) {
  return __uint_as_float(static_cast<uint32_t>(p->v) << 16);
}

// Level 0 of the hierarchy: the sum of each run of 64 keys, in key order.
template <typename T, int D>
__global__ void __launch_bounds__(D) k_block_sums(PrefillArgs a) {
  const int64_t n0 = a.sum_n[0];
  const int64_t head = blockIdx.x / n0;
  const int64_t i = blockIdx.x - head * n0;
  const int c = threadIdx.x;
  const T *kh = static_cast<const T *>(a.K) + head * a.capacity * D + c;
  const int64_t p0 = i * kPrefixRows;
  const int64_t p1 = min(p0 + kPrefixRows, static_cast<int64_t>(a.positions));
  double acc = 0.0;
  for (int64_t t0 = p0; t0 < p1; t0 += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = t0 + u < p1 ? elem64<T>(kh + (t0 + u) * D) : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  a.sums[a.sum_off[0] + (head * n0 + i) * D + c] = acc;
}

// Level k >= 1: the sum of each run of 64 entries of level k - 1, in order.
template <int D>
__global__ void __launch_bounds__(D) k_sum_up(PrefillArgs a, int k) {
  const int64_t n = a.sum_n[k], nb = a.sum_n[k - 1];
  const int64_t head = blockIdx.x / n;
  const int64_t i = blockIdx.x - head * n;
  const int c = threadIdx.x;
  const double *src = a.sums + a.sum_off[k - 1] + head * nb * D + c;
  const int64_t j0 = i * kPrefixRows;
  const int64_t j1 = min(j0 + kPrefixRows, nb);
  double acc = 0.0;
  for (int64_t j = j0; j < j1; j += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = j + u < j1 ? src[(j + u) * D] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  a.sums[a.sum_off[k] + (head * n + i) * D + c] = acc;
}

template <typename T, int D>
__device__ inline double sum_keys(const T *kh, int64_t x, int64_t y) {
  double acc = 0.0;
  for (int64_t t0 = x; t0 < y; t0 += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = t0 + u < y ? elem64<T>(kh + (t0 + u) * D) : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  return acc;
}

// Entries [x, y) of one level's column (stride D), in order.
template <int D>
__device__ inline double sum_entries(const double *lvl, int64_t x, int64_t y) {
  double acc = 0.0;
  for (int64_t j0 = x; j0 < y; j0 += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = j0 + u < y ? lvl[(j0 + u) * D] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  return acc;
}

template <typename T, typename S, int D>
__global__ void __launch_bounds__(D) k_prefix_means(PrefillArgs a) {
  const int64_t nblk = (a.positions + kPrefixRows - 1) / kPrefixRows;
  const int64_t per_head = a.levels * nblk;
  const int64_t head = blockIdx.x / per_head;
  const int64_t rem = blockIdx.x - head * per_head;
  const int h = static_cast<int>(rem / nblk);
  const int64_t p0 = (rem - h * nblk) * kPrefixRows;
  const int64_t p1 = min(p0 + static_cast<int64_t>(kPrefixRows), static_cast<int64_t>(a.positions));
  const int c = threadIdx.x;
  const uint32_t span = static_cast<uint32_t>(a.h_span[h]);
  const T *kh = static_cast<const T *>(a.K) + head * a.capacity * D + c;
  S *pm = static_cast<S *>(a.open_summ);

  // keys of t's node that come before the block: [s0, p0) = up to 63 keys
  // to the first run boundary, then level by level the runs on both ends of
  // what is left, then the middle at the level where it fits
  const int64_t s0 = (p0 / span) * span;
  double acc = 0.0;
  if (s0 < p0) {
    const int64_t a0 = min((s0 + kPrefixRows - 1) / kPrefixRows * kPrefixRows, p0);
    acc += sum_keys<T, D>(kh, s0, a0);
    int64_t x = a0 / kPrefixRows, y = p0 / kPrefixRows;  // level-0 entries [x, y)
    int k = 0;
    for (; k + 1 < a.sum_levels; ++k) {
      const int64_t xu = (x + kPrefixRows - 1) / kPrefixRows * kPrefixRows;
      const int64_t yd = y / kPrefixRows * kPrefixRows;
      if (xu >= yd) break;  // no whole run of the level above in between
      const double *lvl = a.sums + a.sum_off[k] + head * a.sum_n[k] * D + c;
      acc += sum_entries<D>(lvl, x, xu);
      acc += sum_entries<D>(lvl, yd, y);
      x = xu / kPrefixRows;
      y = yd / kPrefixRows;
    }
    acc += sum_entries<D>(a.sums + a.sum_off[k] + head * a.sum_n[k] * D + c, x, y);
  }
  uint32_t held = static_cast<uint32_t>(p0 - s0);  // keys of the node summed so far
  for (int64_t t0 = p0; t0 < p1; t0 += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = t0 + u < p1 ? elem64<T>(kh + (t0 + u) * D) : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t t = t0 + u;
      if (t < p1) {
        if (held == span) {  // t starts a new node
          acc = 0.0;
          held = 0;
        }
        acc += v[u];
        ++held;
        SummaryType<S>::put(pm + ((head * a.positions + t) * a.levels + h) * D + c,
                            acc / static_cast<double>(held));
      }
    }
  }
}

template <typename T, typename S, int D, int NW>
__global__ void __launch_bounds__(NW * 64) k_prefill(RouteArgs ra, AttendArgs aa, PrefillArgs pa) {
  __shared__ RouteShared<NW, NW * 32> rsh;
  __shared__ AttendShared<T, D, NW> ash;
  __shared__ CausalLevels cl;
  const int qi = blockIdx.x;
  const int hrow = qi / pa.positions;          // (batch, query head)
  const int t = qi - hrow * pa.positions;      // position
  const uint4 qraw = attend_q_raw<T, D>(aa, qi);
  if (threadIdx.x < 64) {
    // wave 0 builds the level table, lane j for height j and for level j:
    // every table load at once, then lane exchanges (no serial chain)
    const int lane = threadIdx.x;
    const int bi = hrow / ra.q_heads;
    const int hq = hrow - bi * ra.q_heads;
    const int64_t head = static_cast<int64_t>(bi) * ra.kv_heads + hq / ra.group;
    const uint32_t n = static_cast<uint32_t>(t) + 1u;
    const int levels = pa.levels;
    // a stored height's node span is below 2^31 (it is below the positions)
    const bool hv = lane < levels;
    const uint32_t span = hv ? static_cast<uint32_t>(pa.h_span[lane]) : 0xffffffffu;
    const long long rows = hv ? pa.h_rows[lane] : 0;
    const long long off = hv ? pa.h_off[lane] : 0;
    // depth: the fewest lv >= 1 whose height-lv span covers n (spans grow with h)
    const int lv = 1 + static_cast<int>(__popcll(__ballot(lane >= 1 && hv && span < n)));
    // level l = lane sits at height lv - l
    const bool lev = lane >= 1 && lane <= lv;
    const int h = lev ? lv - lane : 0;
    const uint32_t sp = __shfl(span, h);
    const long long rows_h = __shfl(rows, h);
    const long long off_h = __shfl(off, h);
    const uint32_t ex = lev ? (n + sp - 1u) / sp : 0u;
    // first level below lv with more nodes than the beam, else lv
    const uint64_t cut = __ballot(lev && lane < lv && ex > static_cast<uint32_t>(ra.beam));
    if (lev) {
      cl.exist[lane] = ex;
      cl.rows[lane] = rows_h;
      cl.off[lane] = off_h;
      cl.open_off[lane] = ((head * pa.positions + t) * levels + h) * D;
    }
    if (lane == 0) {
      cl.levels = lv;
      cl.exist[0] = 1;
      cl.exist[lv + 1] = 0;
      cl.first_cut = cut ? __ffsll(static_cast<unsigned long long>(cut)) - 1 : lv;
    }
  }
  __syncthreads();
  const int kept = route_walk<T, S, D, NW, NW, 2, NW * 32>(ra, rsh, qi, &cl, pa.open_summ, hrow);
  if (ra.indices) {
    int32_t *out = ra.indices + static_cast<int64_t>(qi) * ra.beam;
    write_ascending<NW * 64>(rsh.front, kept, out);
    for (int k = kept + static_cast<int>(threadIdx.x); k < ra.beam; k += NW * 64) out[k] = -1;
  }
  attend_query<T, D, true, false, true>(aa, ash, qi, qraw, rsh.front, nullptr, kept, false,
                                        nullptr, 0.0, hrow, static_cast<int64_t>(t) + 1);
}

template <typename T, typename S, int D>
hipError_t launch_prefill_d(const RouteArgs &ra, const AttendArgs &aa, const PrefillArgs &pa,
                            hipStream_t s) {
  const int64_t nblk = (pa.positions + kPrefixRows - 1) / kPrefixRows;
  const dim3 g1(static_cast<unsigned>(pa.heads * pa.levels * nblk));
  const dim3 g2(static_cast<unsigned>(ra.queries));
  hipLaunchKernelGGL((k_block_sums<T, D>), dim3(static_cast<unsigned>(pa.heads * pa.sum_n[0])),
                     dim3(D), 0, s, pa);
  hipError_t e = hipGetLastError();
  for (int k = 1; e == hipSuccess && k < pa.sum_levels; ++k) {
    hipLaunchKernelGGL((k_sum_up<D>), dim3(static_cast<unsigned>(pa.heads * pa.sum_n[k])),
                       dim3(D), 0, s, pa, k);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_prefix_means<T, S, D>), g1, dim3(D), 0, s, pa);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (ra.beam * ra.branching <= 32)
    hipLaunchKernelGGL((k_prefill<T, S, D, 1>), g2, dim3(64), 0, s, ra, aa, pa);
  else if (ra.beam * ra.branching <= 2 * 32)
    hipLaunchKernelGGL((k_prefill<T, S, D, 2>), g2, dim3(2 * 64), 0, s, ra, aa, pa);
  else if (ra.beam * ra.branching <= 4 * 32)
    hipLaunchKernelGGL((k_prefill<T, S, D, 4>), g2, dim3(4 * 64), 0, s, ra, aa, pa);
  else
    hipLaunchKernelGGL((k_prefill<T, S, D, 8>), g2, dim3(8 * 64), 0, s, ra, aa, pa);
  return hipGetLastError();
}

template <typename T, typename S>
hipError_t launch_prefill_ts(int head_dim, const RouteArgs &ra, const AttendArgs &aa,
                             const PrefillArgs &pa, hipStream_t s) {
  if (head_dim == 128) return launch_prefill_d<T, S, 128>(ra, aa, pa, s);
  if (head_dim == 64) return launch_prefill_d<T, S, 64>(ra, aa, pa, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra, const AttendArgs &aa,
                          const PrefillArgs &pa, hipStream_t s) {
  if (dt == Dt::BF16)
    return sdt == Dt::BF16 ? launch_prefill_ts<bf16_bits, bf16_bits>(head_dim, ra, aa, pa, s)
                           : launch_prefill_ts<bf16_bits, float>(head_dim, ra, aa, pa, s);
  return sdt == Dt::BF16 ? launch_prefill_ts<float, bf16_bits>(head_dim, ra, aa, pa, s)
                         : launch_prefill_ts<float, float>(head_dim, ra, aa, pa, s);
}

}  // namespace tis
