// tree_attend: exact softmax attention over the keys of the selected leaf
// blocks ("Subquadratic Attention with a Hierarchical Tree-Structured
// Indexer", Abstract: the final attention after routing; the NSA / InfLLMv2
// abstract on the Progressive Sparse Attention related-papers page: fine
// softmax attention on the selected tokens).
//
// Gather flash-decode, one workgroup per query.  The query's work is cut into
// units of RB rows of one selected leaf block; each wave takes units in turn,
// issues the unit's K and V loads together (16 bytes per lane, whole 256-byte
// rows per lane group), and keeps an online softmax (m, l, acc) in fp32.
// The waves' partials meet in LDS and are merged by log-sum-exp, so the
// step needs no global workspace, atomics or device-scope fences.
#include "tis_device.hpp"
#include "tis_internal.hpp"

namespace tis {
namespace {

template <typename T, int D> struct AttendGeom {
  using G = RowGeom<T, D>;
  static constexpr int E = G::kElemsPerLane;
  static constexpr int LPR = G::kLanesPerRow;
  static constexpr int R = G::kRowsPerInstr;
  static constexpr int U = 8;       // K loads (and V loads) per lane per unit
  static constexpr int RB = U * R;  // rows per unit
  static constexpr int REP = LPR / U;
  static_assert(U <= LPR, "a unit's scores must fit one reduction");
};

template <typename T, int D>
__global__ void __launch_bounds__(kAttendMaxWaves * 64) k_attend(AttendArgs a) {
  using AG = AttendGeom<T, D>;
  constexpr int E = AG::E, LPR = AG::LPR, R = AG::R, U = AG::U, RB = AG::RB, REP = AG::REP;
  __shared__ int s_idx[kMaxCandidates];
  __shared__ int s_use[kMaxCandidates];
  __shared__ int s_bad;
  __shared__ float s_p[kAttendMaxWaves][RB];
  __shared__ float s_m[kAttendMaxWaves], s_l[kAttendMaxWaves];
  __shared__ float s_acc[kAttendMaxWaves][D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int64_t qi = blockIdx.x;
  const int W = a.beam;
  const int L = a.leaf_block;
  const int64_t bi = qi / a.q_heads;
  const int hq = static_cast<int>(qi - bi * a.q_heads);
  const int64_t head = bi * a.kv_heads + hq / a.group;
  const int col = (lane % LPR) * E;
  const int rsub = lane / LPR;

  // the query row and the slot list are loaded before anything waits on them
  // (the launch gives at least min(W, 16) waves, so tid < W covers W <= 1024)
  const uint4 qraw = load16(static_cast<const T *>(a.Q) + qi * D + col);
  const int my_idx = tid < W ? a.indices[qi * W + tid] : -1;

  // ---- the query's slots: repeated entries count once, negatives are empty
  if (tid == 0) s_bad = 0;
  if (tid < W) s_idx[tid] = my_idx;
  __syncthreads();
  for (int s = tid; s < W; s += blockDim.x) {
    const int idx = s_idx[s];
    const bool bad = idx >= a.n_blocks;
    bool use = idx >= 0 && !bad;
    for (int j = 0; j < s && use; ++j) use = s_idx[j] != idx;
    s_use[s] = use;
    if (bad) s_bad = 1;
  }
  __syncthreads();

  float q[E];
  Vec16<T>::unpack(qraw, q);
  const T *kh = static_cast<const T *>(a.K) + head * a.n_keys * D + col;
  const T *vh = static_cast<const T *>(a.V) + head * a.n_keys * D + col;
  const int nc = (L + RB - 1) / RB;
  const int units = W * nc;

  float m = -INFINITY, l = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;

  for (int u = w; u < units; u += nw) {
    const int s = u / nc;
    if (!s_use[s]) continue;
    const int r0 = (u - s * nc) * RB;
    const int64_t rowb = static_cast<int64_t>(s_idx[s]) * L + r0;
    uint4 kv[U], vv[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int row = r0 + i * R + rsub;
      kv[i] = row < L ? load16(kh + (rowb + i * R + rsub) * D) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int row = r0 + i * R + rsub;
      vv[i] = row < L ? load16(vh + (rowb + i * R + rsub) * D) : make_uint4(0u, 0u, 0u, 0u);
    }
    float part[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float k[E];
      Vec16<T>::unpack(kv[i], k);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) dot = fmaf(q[e], k[e], dot);
      part[i] = dot;
    }
    // lane holds the score of row r0 + kk * R + rsub
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
    // hand the probabilities to the lanes holding the matching V rows
    if ((lane % REP) == 0) s_p[w][rsub * U + kk] = p;
    __builtin_amdgcn_wave_barrier();
    float pr[U];
#pragma unroll
    for (int i = 0; i < U; ++i) pr[i] = s_p[w][rsub * U + i];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float v[E];
      Vec16<T>::unpack(vv[i], v);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(pr[i], v[e], acc[e]);
    }
  }
  // rows were spread over the R lane groups of the wave
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = group_sum<LPR, 32>(acc[e], lane);
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < E; ++e) s_acc[w][col + e] = acc[e];
  }
  if (lane == 0) {
    s_m[w] = m;
    s_l[w] = l;
  }
  __syncthreads();

  // ---- log-sum-exp merge of the waves' partials, one column per thread
  for (int c = tid; c < D; c += blockDim.x) {
    float mx = -INFINITY;
    for (int j = 0; j < nw; ++j) mx = fmaxf(mx, s_m[j]);
    float r = 0.f;
    if (mx != -INFINITY) {
      float num = 0.f, den = 0.f;
      for (int j = 0; j < nw; ++j) {
        const float wj = exp2f(s_m[j] - mx);  // 0 for waves that saw no key
        den = fmaf(wj, s_l[j], den);
        num = fmaf(wj, s_acc[j][c], num);
      }
      r = num / den;
    }
    if (s_bad) r = NAN;
    a.O[qi * D + c] = r;
  }
}

}  // namespace

int attend_waves(int head_dim, Dt dt, int beam, int leaf_block) {
  int rb;
  if (dt == Dt::BF16)
    rb = head_dim == 128 ? AttendGeom<bf16_bits, 128>::RB : AttendGeom<bf16_bits, 64>::RB;
  else
    rb = head_dim == 128 ? AttendGeom<float, 128>::RB : AttendGeom<float, 64>::RB;
  const int64_t units = static_cast<int64_t>(beam) * ((leaf_block + rb - 1) / rb);
  return static_cast<int>(units < kAttendMaxWaves ? units : kAttendMaxWaves);
}

hipError_t launch_attend(Dt dt, int head_dim, const AttendArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.queries));
  const dim3 block(static_cast<unsigned>(attend_waves(head_dim, dt, a.beam, a.leaf_block) * 64));
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
