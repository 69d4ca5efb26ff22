// tree_route: top-down beam traversal ("Subquadratic Attention with a
// Hierarchical Tree-Structured Indexer", Abstract: queries traverse the tree
// of key summaries from the top down to retrieve a sparse subset of keys).
//
// One workgroup (8 waves) walks one query through every level in a single
// launch.  Levels with no more candidates than the beam keep everything and
// are not scored.  Per scored level: gather the candidate summary rows (half
// a wave per fp32 row of d = 128, 16-byte loads, every row of the level in
// flight at once), dot them with the query in fp64, rank the candidates in
// LDS and put the W best at their rank; their children are the next level's
// candidates.  The kept leaves are written in ascending order.
#include "tis_device.hpp"
#include "tis_internal.hpp"

namespace tis {
namespace {

constexpr int kRouteWaves = 8;
constexpr int kRouteThreads = kRouteWaves * 64;
static_assert(kMaxCandidates <= kRouteThreads / 2, "two or more threads per candidate");

// Ordered key of a candidate: the fp64 score mapped to an unsigned integer
// whose order is the score order, with its `bits` lowest bits replaced by
// (2^bits - 1 - node), bits = enough bits for every node index of the level.
// Larger key = better, and equal scores go to the lower node index.  Scores
// closer than 2^(bits - 52) relative (at most 2^-21 for levels of up to 2^31
// nodes) also fall to the index order; that is far inside the relative cut
// gap of 1e-5 below which a selection counts as a tie.
__device__ inline uint64_t score_key(double s, int node, int bits) {
  s = s + 0.0;  // -0 -> +0
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(s));
  u = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
  const uint64_t mask = (1ull << bits) - 1ull;
  return (u & ~mask) | (mask - static_cast<uint64_t>(node));
}

template <typename T, int D> __device__ inline void load_q(const T *q, int col, double *out);
template <> __device__ inline void load_q<float, 128>(const float *q, int col, double *out) {
  const float4 v = *reinterpret_cast<const float4 *>(q + col);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}
template <> __device__ inline void load_q<float, 64>(const float *q, int col, double *out) {
  load_q<float, 128>(q, col, out);
}
template <> __device__ inline void load_q<bf16_bits, 128>(const bf16_bits *q, int col, double *out) {
  const uint2 v = *reinterpret_cast<const uint2 *>(q + col);
  out[0] = __uint_as_float(v.x << 16);
  out[1] = __uint_as_float(v.x & 0xffff0000u);
  out[2] = __uint_as_float(v.y << 16);
  out[3] = __uint_as_float(v.y & 0xffff0000u);
}
template <> __device__ inline void load_q<bf16_bits, 64>(const bf16_bits *q, int col, double *out) {
  load_q<bf16_bits, 128>(q, col, out);
}

template <typename T, int D> __global__ void __launch_bounds__(kRouteThreads) k_route(RouteArgs a) {
  constexpr int LPR = D / 4;          // lanes per fp32 summary row
  constexpr int RPI = 64 / LPR;       // rows per wave-wide load
  constexpr int U = 8;                // loads in flight per lane
  constexpr int REP = LPR / U;        // lanes sharing one reduced score
  constexpr int ROWS = U * kRouteWaves * RPI;
  __shared__ uint64_t keys[kMaxCandidates];
  __shared__ int pcnt[kRouteThreads];      // partial rank counts, one per thread
  __shared__ int cand[2][kMaxCandidates];  // node id of every candidate, this level / next
  __shared__ int front[kMaxCandidates];    // kept nodes of the level, in rank order

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int64_t qi = blockIdx.x;
  const int64_t bi = qi / a.q_heads;
  const int hq = static_cast<int>(qi - bi * a.q_heads);
  const int64_t head = bi * a.kv_heads + hq / a.group;
  const int b = a.branching;
  const int W = a.beam;
  const int lv = a.levels;
  const int col = (lane % LPR) * 4;
  const int rsub = lane / LPR;

  // Levels whose candidate set is no larger than the beam keep every node,
  // whatever the scores: the walk starts at the first level l0 that cuts,
  // whose candidates are all of its nodes (so its loads need no selection).
  int l0 = 1;
  while (l0 < lv && a.n_at[l0] <= W) ++l0;
  if (a.trace) {
    for (int l = 1; l < l0; ++l) {
      int32_t *tr = a.trace + (qi * lv + (l - 1)) * W;
      for (int k = tid; k < W; k += kRouteThreads) tr[k] = k < a.n_at[l] ? k : -1;
    }
  }

  // the query row is loaded together with the first scored level's summaries
  double q[4];
  load_q<T, D>(static_cast<const T *>(a.Q) + qi * D, col, q);

  int cur = 0;
  int nf = static_cast<int>(a.n_at[l0 - 1]);
  for (int l = l0; l <= lv; ++l) {
    const int C = nf * b;
    const bool all = l == l0;  // candidates are nodes 0..C-1 of level l
    if (C > W) {
      const int bits = 32 - __clz(static_cast<int>(a.n_at[l]) - 1);
      const float *sl = a.summ + a.summ_off[l] + head * a.n_at[l] * D + col;
      for (int base = 0; base < C; base += ROWS) {
        float4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int pos = base + (u * kRouteWaves + w) * RPI + rsub;
          const int node = all ? pos : cand[cur][pos < C ? pos : 0];
          v[u] = pos < C ? *reinterpret_cast<const float4 *>(sl + static_cast<int64_t>(node) * D)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        double part[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          // fp32 x (fp32 or bf16) products are exact in fp64
          double s = q[0] * static_cast<double>(v[u].x);
          s = fma(q[1], static_cast<double>(v[u].y), s);
          s = fma(q[2], static_cast<double>(v[u].z), s);
          s = fma(q[3], static_cast<double>(v[u].w), s);
          part[u] = s;
        }
        const double s = group_transpose_reduce<U, LPR>(part, lane);
        const int k = (lane % LPR) / REP;
        const int pos = base + (k * kRouteWaves + w) * RPI + rsub;
        if ((lane % REP) == 0 && pos < C) keys[pos] = score_key(s, all ? pos : cand[cur][pos], bits);
      }
      __syncthreads();
      // rank of candidate i = number of candidates with a larger key.
      // Threads form `parts` groups of cp (the power of two >= C); group p
      // compares every candidate with one slice of the keys.
      const int lcp = 32 - __clz(C - 1);
      const int lparts = min(9 - lcp, 3);
      const int span = (((C + (1 << lparts) - 1) >> lparts) + 7) & ~7;
      {
        const int i = tid & ((1 << lcp) - 1);
        const int part = tid >> lcp;
        int cnt = 0;
        if (i < C && part < (1 << lparts)) {
          const uint64_t ki = keys[i];
          int j = part * span;
          const int j1 = min(C, j + span);
          for (; j + 8 <= j1; j += 8) {
            uint64_t kj[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) kj[t] = keys[j + t];
#pragma unroll
            for (int t = 0; t < 8; ++t) cnt += kj[t] > ki ? 1 : 0;
          }
          for (; j < j1; ++j) cnt += keys[j] > ki ? 1 : 0;
        }
        pcnt[tid] = cnt;
      }
      __syncthreads();
      // the W best go to front[] at their rank; their children, in the same
      // order, are the next level's candidates
      if (tid < C) {
        int r = 0;
        for (int p = 0; p < (1 << lparts); ++p) r += pcnt[(p << lcp) + tid];
        if (r < W) {
          const int node = all ? tid : cand[cur][tid];
          front[r] = node;
          if (l < lv) {
            for (int c = 0; c < b; ++c) cand[cur ^ 1][r * b + c] = node * b + c;
          }
        }
      }
    } else {
      // no cut: every candidate is kept
      if (tid < C) {
        const int node = all ? tid : cand[cur][tid];
        front[tid] = node;
        if (l < lv) {
          for (int c = 0; c < b; ++c) cand[cur ^ 1][tid * b + c] = node * b + c;
        }
      }
    }
    __syncthreads();
    cur ^= 1;
    nf = C < W ? C : W;
    if (a.trace) {
      // kept nodes of the level in ascending order
      int32_t *tr = a.trace + (qi * lv + (l - 1)) * W;
      for (int k = tid; k < W; k += kRouteThreads) {
        if (k < nf) {
          const int node = front[k];
          int r = 0;
          for (int j = 0; j < nf; ++j) r += front[j] < node ? 1 : 0;
          tr[r] = node;
        } else {
          tr[k] = -1;
        }
      }
    }
  }
  // the kept leaves, ascending
  for (int k = tid; k < W; k += kRouteThreads) {
    const int node = front[k];
    int r = 0;
    for (int j = 0; j < W; ++j) r += front[j] < node ? 1 : 0;
    a.indices[qi * W + r] = node;
  }
}

}  // namespace

hipError_t launch_route(Dt dt, int head_dim, const RouteArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.queries));
  const dim3 block(kRouteThreads);
  if (dt == Dt::BF16 && head_dim == 128)
    hipLaunchKernelGGL((k_route<bf16_bits, 128>), grid, block, 0, s, a);
  else if (dt == Dt::BF16 && head_dim == 64)
    hipLaunchKernelGGL((k_route<bf16_bits, 64>), grid, block, 0, s, a);
  else if (dt == Dt::F32 && head_dim == 128)
    hipLaunchKernelGGL((k_route<float, 128>), grid, block, 0, s, a);
  else if (dt == Dt::F32 && head_dim == 64)
    hipLaunchKernelGGL((k_route<float, 64>), grid, block, 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tis
