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
// Short appends (k_cache_append): one workgroup per (batch, KV head); the
// new keys of a batch of leaves are summed in parallel (columns across
// threads, coalesced rows), then one thread per column climbs the heights
// leaf by leaf.  Decode appends a key or a few per step, so the work per
// launch is tiny and the launch itself is the cost.
//
// Long appends (prefill into a cache) are split into chunks, the nodes of a
// fixed height hc (about 512 or more keys) that hold new keys:
//  * k_append_chunks: one workgroup per (head, chunk) streams the chunk's
//    new rows with 16-byte loads (a wave per leaf, 8 loads in flight a
//    lane), sums every leaf's new keys per column in fp64, then climbs to
//    the chunk's root in LDS (node sum = its children's sums in order).  It
//    writes every summary of heights 0..hc in the chunk: mean = (new-key sum
//    + the old open sum where the node began before the append) / keys
//    held.  It leaves the root's new-key sum for the heights above.
//  * k_append_top: one workgroup per head climbs heights hc+1 .. H-1 from
//    the chunks' sums, a height at a time, a thread per (node, column).
// The new open sums go to the other state buffer, so no chunk reads a sum
// another has already replaced.
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

constexpr int kChunkWaves = 8;
constexpr int kChunkUnroll = 8;  // row loads in flight per lane

template <int M, int LAST, int N>
__device__ inline void row_group_sum(double (&v)[N], int lane) {
  if constexpr (M <= LAST) {
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] = xor_sum<M>(v[e], lane);
    row_group_sum<M * 2, LAST>(v, lane);
  }
}

template <typename T, typename S, int D>
__global__ void __launch_bounds__(kChunkWaves * 64) k_append_chunks(AppendArgs a) {
  constexpr int NT = kChunkWaves * 64;
  constexpr int EL = Vec16<T>::kElems;  // elements per 16-byte load
  constexpr int LPR = D / EL;           // lanes per key row
  constexpr int RPI = 64 / LPR;         // rows per wave-wide load
  // fp64 sums by leaf slot, b^hc rows of D (sized at launch: more chunks of
  // few leaves fit on a CU at once)
  extern __shared__ double ls_dyn[];
  double(*ls)[D] = reinterpret_cast<double(*)[D]>(ls_dyn);
  const int64_t head = blockIdx.x / a.nchunks;
  const int64_t c = a.chunk0 + (static_cast<int64_t>(blockIdx.x) - head * a.nchunks);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int b = a.branching;
  const int hc = a.chunk_height;
  const int64_t L = a.leaf_block;
  const int64_t ck = a.chunk_keys;
  const int64_t cs = c * ck;  // first key of the chunk
  const int64_t lo = a.n0 > cs ? a.n0 : cs;
  const int64_t hi = a.n1 < cs + ck ? a.n1 : cs + ck;
  const int nleaf = static_cast<int>(ck / L);  // b^hc
  const bool last = hi == a.n1;  // holds the open nodes of heights 0..hc after the append
  const T *kh = static_cast<const T *>(a.K) + head * a.capacity * D;
  const double *st = a.state + head * a.heights * D;
  double *sn = a.state_next + head * a.heights * D;
  S *const summ = static_cast<S *>(a.summ);

  // leaves with no new key add nothing to their parents
  for (int i = tid; i < nleaf * D; i += NT) ls[i / D][i % D] = 0.0;
  __syncthreads();

  // leaf sums: a wave per leaf, the leaf's new rows EL columns a lane
  const int cg = lane % LPR;
  const int ro = lane / LPR;
  const int col = cg * EL;
  const int j0 = static_cast<int>((lo - cs) / L);
  const int j1 = static_cast<int>((hi - 1 - cs) / L);
  for (int j = j0 + w; j <= j1; j += kChunkWaves) {
    const int64_t r0 = cs + j * L > lo ? cs + j * L : lo;
    const int64_t r1 = cs + (j + 1) * L < hi ? cs + (j + 1) * L : hi;
    double acc[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[e] = 0.0;
    for (int64_t r = r0; r < r1; r += RPI * kChunkUnroll) {
      uint4 raw[kChunkUnroll];
#pragma unroll
      for (int u = 0; u < kChunkUnroll; ++u) {
        const int64_t row = r + u * RPI + ro;
        raw[u] = row < r1 ? load16(kh + row * D + col) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < kChunkUnroll; ++u) {
        float f[EL];
        Vec16<T>::unpack(raw[u], f);
#pragma unroll
        for (int e = 0; e < EL; ++e) acc[e] += static_cast<double>(f[e]);
      }
    }
    row_group_sum<LPR, 32>(acc, lane);  // over the wave's RPI row groups
    if (ro == 0) {
      const int64_t m = cs / L + j;  // the leaf's index
      const int64_t start = m * L;
      const int64_t held = (start + L < a.n1 ? start + L : a.n1) - start;
      const bool open = last && a.n1 % L != 0 && m == (a.n1 - 1) / L;
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        ls[j][col + e] = acc[e];
        const double sum = acc[e] + (start < a.n0 ? st[col + e] : 0.0);
        SummaryType<S>::put(summ + a.block_off[0] + (head * a.rows[0] + m) * D + col + e,
                            sum / static_cast<double>(held));
        if (open) sn[col + e] = sum;
      }
    }
  }
  __syncthreads();

  // heights 1 .. hc inside the chunk: node k's sum goes to the slot of its
  // first leaf (its children's slots are its own, read before the write)
  int stride = 1;  // leaves under a node of the height below
  for (int h = 1; h <= hc; ++h) {
    const int64_t span = a.span[h];
    const int nn = nleaf / (stride * b);
    for (int i = tid; i < nn * D; i += NT) {
      const int k = i / D;
      const int cl = i - k * D;
      const int base = k * stride * b;
      double sum_new = ls[base][cl];
      for (int ch = 1; ch < b; ++ch) sum_new += ls[base + ch * stride][cl];
      const int64_t m = cs / span + k;
      const int64_t start = m * span;
      if (start < hi && start + span > lo) {  // the node holds new keys
        const int64_t held = (start + span < a.n1 ? start + span : a.n1) - start;
        const double sum = sum_new + (start < a.n0 ? st[h * D + cl] : 0.0);
        SummaryType<S>::put(summ + a.block_off[h] + (head * a.rows[h] + m) * D + cl,
                            sum / static_cast<double>(held));
        if (last && a.n1 % span != 0 && m == (a.n1 - 1) / span) sn[h * D + cl] = sum;
      }
      ls[base][cl] = sum_new;
    }
    stride *= b;
    __syncthreads();
  }
  // where the append ends on a node boundary, the next node starts empty
  if (last) {
    for (int i = tid; i < (hc + 1) * D; i += NT) {
      const int h = i / D;
      if (a.n1 % a.span[h] == 0) sn[i] = 0.0;
    }
  }
  // the chunk root's new-key sum, for the heights above
  if (hc + 1 < a.heights) {
    for (int i = tid; i < D; i += NT)
      a.scratch[(head * a.nchunks + (c - a.chunk0)) * D + i] = ls[0][i];
  }
}

// Heights hc+1 .. H-1 of one head from the chunks' new-key sums, one height
// after another, a thread per (node, column): a node's new-key sum is the
// sum of its children's in order; its summary is (that + the old open sum
// where the node began before the append) / keys held.  A node's sum goes
// to the scratch slot of its first chunk (its first child's slot, read
// before the write by the same thread), so the next height finds it there;
// the barrier between heights orders the slots' writes before their reads.
constexpr int kTopThreads = 1024;

template <typename S, int D>
__global__ void __launch_bounds__(kTopThreads) k_append_top(AppendArgs a) {
  const int64_t head = blockIdx.x;
  const int tid = threadIdx.x;
  const int b = a.branching;
  const int64_t n0 = a.n0, n1 = a.n1;
  const int64_t ck = a.chunk_keys;
  S *const summ = static_cast<S *>(a.summ);
  const double *st = a.state + head * a.heights * D;
  double *sn = a.state_next + head * a.heights * D;
  double *slot = a.scratch + head * a.nchunks * D;  // slot i: chunk chunk0 + i
  for (int h = a.chunk_height + 1; h < a.heights; ++h) {
    const int64_t span = a.span[h];
    const int64_t cspan = a.span[h - 1];  // keys under a child
    const int64_t per_child = cspan / ck;  // chunks under a child
    const int64_t x0 = n0 / span, x1 = (n1 - 1) / span;  // nodes holding new keys
    const int64_t y0 = n0 / cspan, y1 = (n1 - 1) / cspan;  // children holding new keys
    for (int64_t i = tid; i < (x1 - x0 + 1) * D; i += kTopThreads) {
      const int64_t x = x0 + i / D;
      const int cl = static_cast<int>(i % D);
      const int64_t ya = x * b > y0 ? x * b : y0;
      const int64_t yb = x * b + b - 1 < y1 ? x * b + b - 1 : y1;
      // children 8 at a time: their loads all in flight, then added in order
      double s = 0.0;
      for (int64_t yy = ya; yy <= yb; yy += 8) {
        double v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int64_t y = yy + k;
          const int64_t c = y * per_child > a.chunk0 ? y * per_child : a.chunk0;
          v[k] = y <= yb ? slot[(c - a.chunk0) * D + cl] : 0.0;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (yy + k <= yb) s += v[k];
      }
      const int64_t start = x * span;
      const int64_t held = (start + span < n1 ? start + span : n1) - start;
      const double sum = s + (start < n0 ? st[h * D + cl] : 0.0);
      SummaryType<S>::put(summ + a.block_off[h] + (head * a.rows[h] + x) * D + cl,
                          sum / static_cast<double>(held));
      if (x == x1) sn[h * D + cl] = n1 % span != 0 ? sum : 0.0;  // the open node after n1
      const int64_t cx = x * (span / ck) > a.chunk0 ? x * (span / ck) : a.chunk0;
      slot[(cx - a.chunk0) * D + cl] = s;
    }
    __syncthreads();
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

template <typename T, typename S, int D>
hipError_t launch_append_chunked_d(const AppendArgs &a, hipStream_t s) {
  const size_t lds = static_cast<size_t>(a.chunk_keys / a.leaf_block) * D * sizeof(double);
  hipLaunchKernelGGL((k_append_chunks<T, S, D>),
                     dim3(static_cast<unsigned>(a.heads * a.nchunks)), dim3(kChunkWaves * 64),
                     lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.chunk_height + 1 >= a.heights) return e;
  hipLaunchKernelGGL((k_append_top<S, D>), dim3(static_cast<unsigned>(a.heads)),
                     dim3(kTopThreads), 0, s, a);
  return hipGetLastError();
}

template <typename T, typename S>
hipError_t launch_append_chunked_ts(int head_dim, const AppendArgs &a, hipStream_t s) {
  if (head_dim == 128) return launch_append_chunked_d<T, S, 128>(a, s);
  if (head_dim == 64) return launch_append_chunked_d<T, S, 64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_cache_append_chunked(Dt dt, Dt sdt, int head_dim, const AppendArgs &a,
                                       hipStream_t s) {
  if (dt == Dt::BF16)
    return sdt == Dt::BF16 ? launch_append_chunked_ts<bf16_bits, bf16_bits>(head_dim, a, s)
                           : launch_append_chunked_ts<bf16_bits, float>(head_dim, a, s);
  return sdt == Dt::BF16 ? launch_append_chunked_ts<float, bf16_bits>(head_dim, a, s)
                         : launch_append_chunked_ts<float, float>(head_dim, a, s);
}

hipError_t launch_cache_append(Dt dt, Dt sdt, int head_dim, const AppendArgs &a, hipStream_t s) {
  if (dt == Dt::BF16)
    return sdt == Dt::BF16 ? launch_cache_append_ts<bf16_bits, bf16_bits>(head_dim, a, s)
                           : launch_cache_append_ts<bf16_bits, float>(head_dim, a, s);
  return sdt == Dt::BF16 ? launch_cache_append_ts<float, bf16_bits>(head_dim, a, s)
                         : launch_cache_append_ts<float, float>(head_dim, a, s);
}

}  // namespace tis
