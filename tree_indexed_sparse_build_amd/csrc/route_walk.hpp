// One query's walk down the tree ("Subquadratic Attention with a Hierarchical
// Tree-Structured Indexer", Abstract: a query descends the summary tree one
// level at a time and ends with a small set of keys to attend to), as a
// device function shared by the route kernel and the fused decode kernel.
//
// Per scored level: gather the candidate summary rows (half a wave per fp32
// row of d = 128, 16-byte loads, every row of the level in flight at once),
// dot them with the query in fp64, rank the candidates in LDS and put the W
// best at their rank; their children are the next level's candidates.
#pragma once

#include "tis_device.hpp"
#include "tis_internal.hpp"

namespace tis {

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

// Shared memory of one query's walk, for a workgroup of NW waves.
template <int NW> struct RouteShared {
  uint64_t keys[kMaxCandidates];
  int cand[2][kMaxCandidates];     // node id of every candidate, this level / next
  int front[kMaxCandidates];       // kept nodes of the level, in rank order
};

// Writes the n distinct values v[0..n) to out[0..n) in ascending order (each
// value goes to the slot given by how many values are smaller).
template <int NT> __device__ inline void write_ascending(const int *v, int n, int32_t *out) {
  for (int k = threadIdx.x; k < n; k += NT) {
    const int x = v[k];
    int r = 0;
    for (int j = 0; j < n; ++j) r += v[j] < x ? 1 : 0;
    out[r] = x;
  }
}

// Walks query qi down the tree (every wave of the NW-wave workgroup takes
// part).  On return, after a barrier, sh.front[0 .. beam) holds the kept
// leaves in rank order, best first.  Levels whose candidate set is no larger
// than the beam keep every node whatever the scores, so the walk starts at
// the first level l0 that cuts; its candidates are all of its nodes, so its
// loads need no selection and go out together with the query row.
template <typename T, int D, int NW>
__device__ void route_walk(const RouteArgs &a, RouteShared<NW> &sh, int64_t qi) {
  constexpr int NT = NW * 64;
  constexpr int LOG_NT = NW == 16 ? 10 : NW == 8 ? 9 : NW == 4 ? 8 : -1;
  static_assert(LOG_NT > 0, "4, 8 or 16 waves");
  static_assert(kMaxCandidates <= NT / 2, "two or more threads per candidate");
  constexpr int LPR = D / 4;          // lanes per fp32 summary row
  constexpr int RPI = 64 / LPR;       // rows per wave-wide load
  constexpr int U = 8;                // loads in flight per lane
  constexpr int REP = LPR / U;        // lanes sharing one reduced score
  constexpr int ROWS = U * NW * RPI;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int64_t bi = qi / a.q_heads;
  const int hq = static_cast<int>(qi - bi * a.q_heads);
  const int64_t head = bi * a.kv_heads + hq / a.group;
  const int b = a.branching;
  const int W = a.beam;
  const int lv = a.levels;
  const int col = (lane % LPR) * 4;
  const int rsub = lane / LPR;

  int l0 = 1;
  while (l0 < lv && a.n_at[l0] <= W) ++l0;
  if (a.trace) {
    for (int l = 1; l < l0; ++l) {
      int32_t *tr = a.trace + (qi * lv + (l - 1)) * W;
      for (int k = tid; k < W; k += NT) tr[k] = k < a.n_at[l] ? k : -1;
    }
  }

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
          const int pos = base + (u * NW + w) * RPI + rsub;
          const int node = all ? pos : sh.cand[cur][pos < C ? pos : 0];
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
        const int pos = base + (k * NW + w) * RPI + rsub;
        if ((lane % REP) == 0 && pos < C)
          sh.keys[pos] = score_key(s, all ? pos : sh.cand[cur][pos], bits);
      }
      __syncthreads();
      // rank of candidate i = number of candidates with a larger key.  Each
      // candidate has a group of g adjacent lanes (g <= 8); lane p of the
      // group counts over keys p, p+g, p+2g, ... (so the g lanes read g
      // neighbouring keys: no bank conflict, and every group of the wave
      // reads the same addresses), then the group adds its counts with DPP,
      // so the ranks need no further trip through LDS.
      {
        const int lcp = 32 - __clz(C - 1);
        const int lg = min(LOG_NT - lcp, 3);
        const int g = 1 << lg;
        const int i = tid >> lg;
        const int part = tid & (g - 1);
        int cnt = 0;
        if (i < C) {
          const uint64_t ki = sh.keys[i];
          int j = part;
          for (; j + 7 * g < C; j += 8 * g) {
            uint64_t kj[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) kj[t] = sh.keys[j + t * g];
#pragma unroll
            for (int t = 0; t < 8; ++t) cnt += kj[t] > ki ? 1 : 0;
          }
          for (; j < C; j += g) cnt += sh.keys[j] > ki ? 1 : 0;
        }
        // g is uniform: every lane of the wave takes the same branches
        if (g >= 2) cnt = xor_sum<1>(cnt, lane);
        if (g >= 4) cnt = xor_sum<2>(cnt, lane);
        if (g >= 8) cnt = xor_sum<4>(cnt, lane);
        // the W best go to front[] at their rank; their children, in the
        // same order, are the next level's candidates
        if (i < C && part == 0 && cnt < W) {
          const int node = all ? i : sh.cand[cur][i];
          sh.front[cnt] = node;
          if (l < lv) {
            for (int c = 0; c < b; ++c) sh.cand[cur ^ 1][cnt * b + c] = node * b + c;
          }
        }
      }
    } else {
      // no cut: every candidate is kept
      if (tid < C) {
        const int node = all ? tid : sh.cand[cur][tid];
        sh.front[tid] = node;
        if (l < lv) {
          for (int c = 0; c < b; ++c) sh.cand[cur ^ 1][tid * b + c] = node * b + c;
        }
      }
    }
    __syncthreads();
    cur ^= 1;
    nf = C < W ? C : W;
    if (a.trace) {
      int32_t *tr = a.trace + (qi * lv + (l - 1)) * W;
      write_ascending<NT>(sh.front, nf, tr);
      for (int k = nf + tid; k < W; k += NT) tr[k] = -1;
    }
  }
}

}  // namespace tis
