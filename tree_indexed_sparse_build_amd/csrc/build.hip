// tree_build: node summaries = mean of the keys under each node, for every
// level ("Subquadratic Attention with a Hierarchical Tree-Structured
// Indexer", Abstract: a tree of recursively compressed key summaries over
// the KV cache).
//
// HBM-bound: K is read exactly once with 16-byte coalesced loads (a wave
// reads whole 1 KB stretches of a leaf block, 16 KB in flight per wave),
// each summary row is written once.  Sums are carried in fp64 in a fixed
// order and rounded once to fp32.  The first kernel finishes every level up
// to the roots of its chunks; when those sit below level 1 a second, small
// kernel climbs the rest from their fp64 sums (a kernel boundary instead of
// device-scope fences between workgroups).
#include "tis_device.hpp"
#include "tis_internal.hpp"

namespace tis {
namespace {

template <int E> __device__ inline void store_mean(float *dst, const double *s, double M) {
  float f[E];
#pragma unroll
  for (int e = 0; e < E; ++e) f[e] = static_cast<float>(s[e] / M);
#pragma unroll
  for (int e = 0; e < E; e += 4)
    *reinterpret_cast<float4 *>(dst + e) = make_float4(f[e], f[e + 1], f[e + 2], f[e + 3]);
}

template <typename T, int D> __global__ void __launch_bounds__(512) k_build(BuildArgs a) {
  using G = RowGeom<T, D>;
  constexpr int E = G::kElemsPerLane;
  constexpr int LPR = G::kLanesPerRow;
  constexpr int R = G::kRowsPerInstr;
  constexpr int U = 16;  // 16-byte loads in flight per lane
  extern __shared__ double lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int b = a.branching;
  const int L = a.leaf_block;
  const int lv = a.levels;
  const int64_t head = blockIdx.x / a.chunks;
  const int64_t chunk = blockIdx.x - head * a.chunks;
  const int col = (lane % LPR) * E;
  const int rsub = lane / LPR;
  const T *kh = static_cast<const T *>(a.K) + head * a.n_keys * D + col;

  // ---- this wave: the b leaves under one node of level lv-1
  const int64_t node1 = chunk * nw + w;
  double pacc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) pacc[e] = 0.0;
  for (int c = 0; c < b; ++c) {
    const int64_t leaf = node1 * b + c;
    const T *kl = kh + leaf * static_cast<int64_t>(L) * D;
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    for (int r0 = 0; r0 < L; r0 += U * R) {
      uint4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = r0 + u * R + rsub;
        v[u] = row < L ? load16(kl + static_cast<int64_t>(row) * D) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float f[E];
        Vec16<T>::unpack(v[u], f);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += static_cast<double>(f[e]);
      }
    }
    // rows of one leaf are spread over the R lane groups of the wave
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = group_sum<LPR, 32>(acc[e], lane);
    if (lane < LPR)
      store_mean<E>(a.summ + a.summ_off[lv] + (head * a.n_at[lv] + leaf) * D + col, acc,
                    static_cast<double>(L));
#pragma unroll
    for (int e = 0; e < E; ++e) pacc[e] += acc[e];
  }

  int lvl = lv - 1;  // level of the wave's node
  if (lvl >= 1 && lane < LPR)
    store_mean<E>(a.summ + a.summ_off[lvl] + (head * a.n_at[lvl] + node1) * D + col, pacc,
                  static_cast<double>(a.n_keys / a.n_at[lvl]));

  // ---- the workgroup's inner levels, from the waves' fp64 sums in LDS
  double *cur = lds;
  double *nxt = lds + nw * D;
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < E; ++e) cur[w * D + col + e] = pacc[e];
  }
  __syncthreads();
  int64_t base = chunk * nw;  // index of cur[0]'s node within its level
  for (int ncur = nw; ncur > 1; ncur /= b) {
    const int nn = ncur / b;
    --lvl;
    base /= b;
    const double M = lvl >= 1 ? static_cast<double>(a.n_keys / a.n_at[lvl]) : 1.0;
    for (int i = tid; i < nn * D; i += blockDim.x) {
      const int n = i / D;
      const int dd = i % D;
      double s = 0.0;
      for (int c = 0; c < b; ++c) s += cur[(n * b + c) * D + dd];
      nxt[n * D + dd] = s;
      if (lvl >= 1)
        a.summ[a.summ_off[lvl] + (head * a.n_at[lvl] + base + n) * D + dd] =
            static_cast<float>(s / M);
    }
    __syncthreads();
    double *t = cur;
    cur = nxt;
    nxt = t;
  }

  // ---- the chunk root: its fp64 sum feeds the levels above (second kernel)
  if (lvl >= 2) {
    double *mine = a.ws_sum + a.ws_off[lvl] + (head * a.n_at[lvl] + base) * D;
    for (int i = tid; i < D; i += blockDim.x) mine[i] = cur[i];
  }
}

// Levels r-1 .. 1 from the fp64 sums of the level-r chunk roots.  One
// workgroup per level-1 node, one thread per column: each thread carries its
// column up through every level of the subtree on its own, so there is no
// barrier; a workgroup's reads of a node row are one coalesced stretch.
template <int D> __global__ void __launch_bounds__(D) k_build_top(BuildArgs a) {
  const int t = threadIdx.x;
  const int b = a.branching;
  const int r = a.root_level;
  const int64_t head = blockIdx.x / b;
  const int64_t n1 = blockIdx.x - head * b;
  for (int l = r - 1; l >= 1; --l) {
    // level l of the subtree holds the b^(l-1) nodes from n1 * b^(l-1) on
    int64_t first = n1;
    int64_t span = 1;
    for (int k = 1; k < l; ++k) {
      first *= b;
      span *= b;
    }
    const double M = static_cast<double>(a.n_keys / a.n_at[l]);
    const double *child = a.ws_sum + a.ws_off[l + 1] + head * a.n_at[l + 1] * D + t;
    for (int64_t n = first; n < first + span; ++n) {
      double s = 0.0;
      for (int c = 0; c < b; ++c) s += child[(n * b + c) * D];
      a.summ[a.summ_off[l] + (head * a.n_at[l] + n) * D + t] = static_cast<float>(s / M);
      if (l >= 2) a.ws_sum[a.ws_off[l] + (head * a.n_at[l] + n) * D + t] = s;
    }
  }
}

}  // namespace

bool plan_build(int64_t heads, int head_dim, int branching, int leaf_block, int levels,
                BuildPlan *p) {
  (void)leaf_block;
  int kg = 0;
  int64_t nw = 1;
  while (kg + 1 <= levels - 1 && nw * branching <= 8) {
    nw *= branching;
    ++kg;
  }
  const int r = levels - 1 - kg;
  int64_t chunks = 1;
  for (int i = 0; i < r; ++i) chunks *= branching;
  if (heads * chunks > 0x7fffffffLL) return false;
  size_t sum = 0;
  int64_t n = 1;
  for (int l = 1; l <= r; ++l) {
    n *= branching;
    if (l >= 2) sum += static_cast<size_t>(heads * n) * head_dim;
  }
  p->root_level = r;
  p->waves = static_cast<int>(nw);
  p->chunks = chunks;
  p->lds_bytes = static_cast<size_t>(2 * nw * head_dim) * sizeof(double);
  p->sum_elems = sum;
  p->workspace_bytes = sum * sizeof(double);
  return true;
}

hipError_t launch_build(Dt dt, int head_dim, int64_t heads, const BuildArgs &a,
                        const BuildPlan &p, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(heads * p.chunks));
  const dim3 block(static_cast<unsigned>(p.waves * 64));
  if (dt == Dt::BF16 && head_dim == 128)
    hipLaunchKernelGGL((k_build<bf16_bits, 128>), grid, block, p.lds_bytes, s, a);
  else if (dt == Dt::BF16 && head_dim == 64)
    hipLaunchKernelGGL((k_build<bf16_bits, 64>), grid, block, p.lds_bytes, s, a);
  else if (dt == Dt::F32 && head_dim == 128)
    hipLaunchKernelGGL((k_build<float, 128>), grid, block, p.lds_bytes, s, a);
  else if (dt == Dt::F32 && head_dim == 64)
    hipLaunchKernelGGL((k_build<float, 64>), grid, block, p.lds_bytes, s, a);
  else
    return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.root_level < 2) return e;
  const dim3 grid2(static_cast<unsigned>(heads * a.branching));
  if (head_dim == 128)
    hipLaunchKernelGGL((k_build_top<128>), grid2, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL((k_build_top<64>), grid2, dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace tis
