// Tree over a growing KV cache: append ("Subquadratic Attention with a
// Hierarchical Tree-Structured Indexer", Abstract: the summary tree lives
// over the KV cache and grows deeper step by step as the context lengthens).
//
// Keys arrive in order, so at every height only the node that holds the
// newest key (the open node) can be partial; every node to its left is
// complete and never changes again.  The state keeps the exact fp64 sum of
// the open node at every height.  An append of keys [n0, n1) adds, leaf by
// leaf, the new keys' column sums to the open sums of all heights; whenever
// a leaf completes a node of height h that node's mean is written and its
// sum restarts from zero; at the end the partial open nodes are written and
// their sums kept.  Every summary is therefore the exact mean of its keys
// rounded once, exactly as a build over the first n1 keys would give.
//
// One workgroup per (batch, KV head): the new keys of a batch of leaves are
// summed in parallel (columns across threads, coalesced rows), then one
// thread per column climbs the heights leaf by leaf.  Decode appends a key
// or a few per step, so the work per launch is tiny and the launch itself is
// the cost; long appends (prefill into an empty tree) stream at one
// workgroup's rate per head.
#include "tis_device.hpp"
#include "tis_internal.hpp"

namespace tis {
namespace {

constexpr int kAppendThreads = 256;
constexpr int kAppendBatch = 16;  // leaves whose sums sit in LDS at once

template <typename T> __device__ inline double key_elem(const T *p);
template <> __device__ inline double key_elem<float>(const float *p) { return *p; }
template <> __device__ inline double key_elem<bf16_bits>(const bf16_bits *p) {
  return __uint_as_float(static_cast<uint32_t>(p->v) << 16);
}

template <typename T, typename S, int D>
__global__ void __launch_bounds__(kAppendThreads) k_cache_append(AppendArgs a) {
  __shared__ double ls[kAppendBatch][D];
  const int64_t head = blockIdx.x;
  const int tid = threadIdx.x;
  const int c = tid % D;
  const int slot = tid / D;
  constexpr int kPar = kAppendThreads / D;  // leaves summed side by side
  const int64_t L = a.leaf_block;
  const int b = a.branching;
  const int H = a.heights;
  const T *kh = static_cast<const T *>(a.K) + head * a.capacity * D + c;
  S *const summ = static_cast<S *>(a.summ);
  double *st = a.state + head * H * D + c;

  // per height h: first summary row of this head, keys under one node
  int64_t base[kMaxLevels];
  uint32_t span[kMaxLevels];
  double open[kMaxLevels];
#pragma unroll
  for (int h = 0; h < kMaxLevels; ++h) {
    base[h] = h < H ? a.block_off[h] + head * a.rows[h] * D : 0;
    span[h] = h < H ? a.span[h] : 1u;
    open[h] = (tid < D && h < H) ? st[h * D] : 0.0;
  }

  const uint32_t n0 = static_cast<uint32_t>(a.n0), n1 = static_cast<uint32_t>(a.n1);
  const uint32_t j0 = n0 / static_cast<uint32_t>(L);
  const uint32_t j1 = (n1 - 1u) / static_cast<uint32_t>(L);
  for (uint32_t jb = j0; jb <= j1; jb += kAppendBatch) {
    const int nb = static_cast<int>(j1 - jb + 1u < kAppendBatch ? j1 - jb + 1u : kAppendBatch);
    // new keys of each leaf of the batch, summed per column in fp64
    for (int s = slot; s < nb; s += kPar) {
      const int64_t j = jb + s;
      const int64_t lo = j * L > a.n0 ? j * L : a.n0;
      const int64_t hi = (j + 1) * L < a.n1 ? (j + 1) * L : a.n1;
      // 8 rows in flight before any is added (a plain loop would wait on
      // every load), then a tail
      double sum = 0.0;
      int64_t t = lo;
      for (; t + 8 <= hi; t += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = key_elem<T>(kh + (t + u) * D);
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
      }
      for (; t < hi; ++t) sum += key_elem<T>(kh + t * D);
      ls[s][c] = sum;
    }
    __syncthreads();
    // climb: every height's open node gains the leaf's new keys; a leaf that
    // completes a node of height h (b^h divides the leaves up to it) closes
    // it: mean written, sum restarted
    if (tid < D) {
      for (int s = 0; s < nb; ++s) {
        const uint32_t j = jb + s;
        const double v = ls[s][c];
        bool closing = (static_cast<int64_t>(j) + 1) * L <= a.n1;  // the leaf is complete
        uint32_t m = j + 1u;  // nodes of height h up to this leaf
#pragma unroll
        for (int h = 0; h < kMaxLevels; ++h) {
          if (h < H) {
            open[h] += v;
            if (closing) {
              SummaryType<S>::put(summ + base[h] + static_cast<int64_t>(m - 1u) * D + c,
                                  open[h] / static_cast<double>(span[h]));
              open[h] = 0.0;
              closing = m % static_cast<uint32_t>(b) == 0u;
              m /= static_cast<uint32_t>(b);
            }
          }
        }
      }
    }
    __syncthreads();
  }
  // the open nodes: write their means over the keys they hold, keep the sums
  if (tid < D) {
#pragma unroll
    for (int h = 0; h < kMaxLevels; ++h) {
      if (h < H) {
        const uint32_t node = n1 / span[h];
        const uint32_t held = n1 - node * span[h];
        if (held > 0u)
          SummaryType<S>::put(summ + base[h] + static_cast<int64_t>(node) * D + c,
                              open[h] / static_cast<double>(held));
        st[h * D] = held > 0u ? open[h] : 0.0;
      }
    }
  }
}

__global__ void __launch_bounds__(256) k_fill_zero(double *p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0;
}

}  // namespace

hipError_t launch_fill_zero(double *p, int64_t elems, hipStream_t s) {
  if (elems <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((elems + 255) / 256));
  hipLaunchKernelGGL(k_fill_zero, grid, dim3(256), 0, s, p, elems);
  return hipGetLastError();
}

namespace {

template <typename T, typename S>
hipError_t launch_cache_append_ts(int head_dim, const AppendArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.heads));
  const dim3 block(kAppendThreads);
  if (head_dim == 128)
    hipLaunchKernelGGL((k_cache_append<T, S, 128>), grid, block, 0, s, a);
  else if (head_dim == 64)
    hipLaunchKernelGGL((k_cache_append<T, S, 64>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_append(Dt dt, Dt sdt, int head_dim, const AppendArgs &a, hipStream_t s) {
  if (dt == Dt::BF16)
    return sdt == Dt::BF16 ? launch_cache_append_ts<bf16_bits, bf16_bits>(head_dim, a, s)
                           : launch_cache_append_ts<bf16_bits, float>(head_dim, a, s);
  return sdt == Dt::BF16 ? launch_cache_append_ts<float, bf16_bits>(head_dim, a, s)
                         : launch_cache_append_ts<float, float>(head_dim, a, s);
}

}  // namespace tis
