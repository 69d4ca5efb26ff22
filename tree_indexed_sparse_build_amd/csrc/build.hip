// tree_build: node summaries = mean of the keys under each node, every level
// in one launch ("Subquadratic Attention with a Hierarchical Tree-Structured
// Indexer", Abstract: a tree of recursively compressed key summaries over
// the KV cache).
//
// HBM-bound: K is read exactly once with 16-byte coalesced loads (a wave
// reads whole 1 KB stretches of a leaf block), each summary row is written
// once.  Sums are carried in fp64 in a fixed order and rounded once to fp32.
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
  constexpr int U = 8;  // 16-byte loads in flight per lane
  extern __shared__ double lds[];
  __shared__ int s_last;

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
    for (int m = LPR; m < 64; m <<= 1) {
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += shfl_xor_f64(acc[e], m);
    }
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

  // ---- levels above the chunk root: the last sibling to arrive climbs
  int r = lvl;
  int64_t node = base;
  while (r >= 2) {
    double *mine = a.ws_sum + a.ws_off[r] + (head * a.n_at[r] + node) * D;
    for (int i = tid; i < D; i += blockDim.x) mine[i] = cur[i];
    __threadfence();
    __syncthreads();
    const int64_t parent = node / b;
    int *ctr = a.ws_cnt + a.cnt_off[r - 1] + head * a.n_at[r - 1] + parent;
    if (tid == 0) {
      const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      const int last = old == b - 1;
      if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const double M = static_cast<double>(a.n_keys / a.n_at[r - 1]);
    const double *sib = a.ws_sum + a.ws_off[r] + (head * a.n_at[r] + parent * b) * D;
    for (int i = tid; i < D; i += blockDim.x) {
      double s = 0.0;
      for (int c = 0; c < b; ++c) s += sib[c * D + i];
      cur[i] = s;
      a.summ[a.summ_off[r - 1] + (head * a.n_at[r - 1] + parent) * D + i] =
          static_cast<float>(s / M);
    }
    __syncthreads();
    // every sibling sum has been read: clear them, so a completed call leaves
    // the workspace all zero whatever geometry used it before
    double *sibw = a.ws_sum + a.ws_off[r] + (head * a.n_at[r] + parent * b) * D;
    for (int i = tid; i < b * D; i += blockDim.x) sibw[i] = 0.0;
    --r;
    node = parent;
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
  size_t cnt = 0, sum = 0;
  int64_t n = 1;
  for (int l = 1; l <= r; ++l) {
    n *= branching;
    if (l <= r - 1) cnt += static_cast<size_t>(heads * n);
    if (l >= 2) sum += static_cast<size_t>(heads * n) * head_dim;
  }
  p->root_level = r;
  p->waves = static_cast<int>(nw);
  p->chunks = chunks;
  p->lds_bytes = static_cast<size_t>(2 * nw * head_dim) * sizeof(double);
  p->cnt_elems = cnt;
  p->sum_elems = sum;
  p->workspace_bytes = align_up(cnt * sizeof(int), 256) + sum * sizeof(double);
  if (p->workspace_bytes < 256) p->workspace_bytes = 256;
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
  return hipGetLastError();
}

}  // namespace tis
