// tree_attend: exact softmax attention over the keys of the selected leaf
// blocks ("Subquadratic Attention with a Hierarchical Tree-Structured
// Indexer", Abstract: the final attention after routing; the NSA / InfLLMv2
// abstract on the Progressive Sparse Attention related-papers page: fine
// softmax attention on the selected tokens).
//
// Gather flash-decode.  One wave per (query, index slot) streams the slot's
// K and V leaf blocks with 16-byte loads (both issued before any math),
// keeps an online softmax (m, l, acc) in fp32 and writes it to the
// workspace; the last wave of the query to arrive merges the partials by
// log-sum-exp into O, so the whole step is one launch.
#include "tis_device.hpp"
#include "tis_internal.hpp"

namespace tis {
namespace {

constexpr int kPartHeader = 4;  // m, l, two pad words: keeps acc 16-byte aligned

template <typename T, int D> __global__ void __launch_bounds__(64) k_attend(AttendArgs a) {
  using G = RowGeom<T, D>;
  constexpr int E = G::kElemsPerLane;
  constexpr int LPR = G::kLanesPerRow;
  constexpr int R = G::kRowsPerInstr;
  constexpr int U = LPR < 16 ? LPR : 16;  // rows-loads per lane per batch
  constexpr int RB = U * R;               // rows per batch
  constexpr int REP = LPR / U;            // lanes sharing one score
  constexpr int PS = D + kPartHeader;
  __shared__ float ps[RB];
  __shared__ int s_last;

  const int lane = threadIdx.x;
  const int W = a.beam;
  const int64_t qi = blockIdx.x / W;
  const int slot = static_cast<int>(blockIdx.x - qi * W);
  const int L = a.leaf_block;
  const int64_t bi = qi / a.q_heads;
  const int hq = static_cast<int>(qi - bi * a.q_heads);
  const int64_t head = bi * a.kv_heads + hq / a.group;
  const int col = (lane % LPR) * E;
  const int rsub = lane / LPR;

  const int32_t *irow = a.indices + qi * W;
  const int idx = irow[slot];
  bool dup = false;
  for (int j0 = 0; j0 < slot; j0 += 64) {
    const int j = j0 + lane;
    dup |= __ballot(j < slot && irow[j] == idx) != 0ull;
  }
  const bool bad = idx >= a.n_blocks;
  const bool empty = idx < 0 || dup;

  float m = -INFINITY;
  float l = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;

  if (!bad && !empty) {
    float q[E];
    Vec16<T>::unpack(load16(static_cast<const T *>(a.Q) + qi * D + col), q);
    const int64_t row0 = head * a.n_keys + static_cast<int64_t>(idx) * L;
    const T *kb = static_cast<const T *>(a.K) + row0 * D + col;
    const T *vb = static_cast<const T *>(a.V) + row0 * D + col;
    for (int r0 = 0; r0 < L; r0 += RB) {
      uint4 kv[U], vv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = r0 + u * R + rsub;
        kv[u] = row < L ? load16(kb + static_cast<int64_t>(row) * D) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = r0 + u * R + rsub;
        vv[u] = row < L ? load16(vb + static_cast<int64_t>(row) * D) : make_uint4(0u, 0u, 0u, 0u);
      }
      float part[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float k[E];
        Vec16<T>::unpack(kv[u], k);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) s = fmaf(q[e], k[e], s);
        part[u] = s;
      }
      // lane now holds the score of row r0 + kk * R + rsub
      const float sc = group_transpose_reduce<U, LPR>(part, lane);
      const int kk = (lane % LPR) / REP;
      const bool valid = r0 + kk * R + rsub < L;
      const float x = valid ? sc * a.scale_log2 : -INFINITY;
      const float mnew = fmaxf(m, wave_max(x));
      const float p = valid ? exp2f(x - mnew) : 0.f;
      const float alpha = exp2f(m - mnew);
      l = l * alpha + wave_sum((lane % REP) == 0 ? p : 0.f);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] *= alpha;
      m = mnew;
      if ((lane % REP) == 0) ps[rsub * U + kk] = p;
      __syncthreads();
      float pr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) pr[u] = ps[rsub * U + u];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float v[E];
        Vec16<T>::unpack(vv[u], v);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(pr[u], v[e], acc[e]);
      }
      __syncthreads();
    }
    // rows were spread over the R lane groups of the wave
#pragma unroll
    for (int mm = LPR; mm < 64; mm <<= 1) {
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += __shfl_xor(acc[e], mm, 64);
    }
  }
  if (bad) l = NAN;

  float *pp = a.part + (qi * W + slot) * PS;
  if (lane == 0) {
    pp[0] = m;
    pp[1] = l;
  }
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < E; e += 4)
      *reinterpret_cast<float4 *>(pp + kPartHeader + col + e) =
          make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
  }

  // ---- the last of the query's W waves merges the partials
  __threadfence();
  __syncthreads();
  if (lane == 0) {
    int *ctr = a.cnt + qi;
    const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == W - 1;
    if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // The merge reads every partial of the query with independent loads,
  // then clears them so the workspace is all zero again when the call ends.
  float *pq = a.part + qi * W * PS;
  float mx = -INFINITY;
  bool anybad = false;
  for (int j = lane; j < W; j += 64) {
    mx = fmaxf(mx, pq[j * PS]);
    anybad |= isnan(pq[j * PS + 1]);
  }
  mx = wave_max(mx);
  anybad = __ballot(anybad) != 0ull;
  constexpr int CPL = D / 64;  // output columns per lane
  float num[CPL], den = 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c) num[c] = 0.f;
  if (mx != -INFINITY) {
    for (int j0 = 0; j0 < W; j0 += 64) {
      // weight of slot j0 + lane, shared with the wave through shuffles
      const int j = j0 + lane;
      const float mj = j < W ? pq[j * PS] : -INFINITY;
      const float wj = exp2f(mj - mx);  // 0 for empty slots
      den += wave_sum(j < W ? wj * pq[j * PS + 1] : 0.f);
      const int n = min(64, W - j0);
      for (int k0 = 0; k0 < n; k0 += 8) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int k = k0 + kk;
          const float wk = __shfl(wj, k & 63, 64);
          if (k < n) {
            const float *row = pq + (j0 + k) * PS + kPartHeader + lane * CPL;
#pragma unroll
            for (int c = 0; c < CPL; ++c) num[c] = fmaf(wk, row[c], num[c]);
          }
        }
      }
    }
  }
  float *o = a.O + qi * D + lane * CPL;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float r = mx == -INFINITY ? 0.f : num[c] / den;
    if (anybad) r = NAN;
    o[c] = r;
  }
  for (int i = lane * 4; i < W * PS; i += 64 * 4)
    *reinterpret_cast<float4 *>(pq + i) = make_float4(0.f, 0.f, 0.f, 0.f);
}

}  // namespace

void plan_attend(int64_t queries, int head_dim, int beam, AttendPlan *p) {
  p->part_elems = static_cast<size_t>(queries) * beam * (head_dim + kPartHeader);
  p->cnt_elems = static_cast<size_t>(queries);
  p->workspace_bytes = align_up(p->cnt_elems * sizeof(int), 256) + p->part_elems * sizeof(float);
}

hipError_t launch_attend(Dt dt, int head_dim, const AttendArgs &a, const AttendPlan &p,
                         hipStream_t s) {
  (void)p;
  const dim3 grid(static_cast<unsigned>(a.queries * a.beam));
  const dim3 block(64);
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
