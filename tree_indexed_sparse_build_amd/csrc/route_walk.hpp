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

// Pins a register value where it stands: the empty asm reads and "writes"
// it, so the compiler can neither hoist what uses it above this point nor
// out of a loop.  Used to keep the query's widening (which waits for its
// load) behind the summary loads that should already be in flight.
__device__ inline uint32_t pin(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Raw bits of this lane's 4 query elements (columns col .. col + 3).  They
// stay raw until a level's summary loads are in flight, so the wait for the
// query row overlaps those loads.
template <typename T> struct QRaw;
template <> struct QRaw<float> {
  uint4 r;
  __device__ inline void load(const float *q) { r = *reinterpret_cast<const uint4 *>(q); }
  __device__ inline void widen(double *out) const {
    out[0] = __uint_as_float(pin(r.x));
    out[1] = __uint_as_float(pin(r.y));
    out[2] = __uint_as_float(pin(r.z));
    out[3] = __uint_as_float(pin(r.w));
  }
};
template <> struct QRaw<bf16_bits> {
  uint2 r;
  __device__ inline void load(const bf16_bits *q) { r = *reinterpret_cast<const uint2 *>(q); }
  __device__ inline void widen(double *out) const {
    const uint32_t x = pin(r.x), y = pin(r.y);
    out[0] = __uint_as_float(x << 16);
    out[1] = __uint_as_float(x & 0xffff0000u);
    out[2] = __uint_as_float(y << 16);
    out[3] = __uint_as_float(y & 0xffff0000u);
  }
};

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

// Scores the C candidates of one level: candidate p is node p of the level
// (all) or node cand[p], and its key goes to keys[p].  The nsw waves of the
// workgroup cover UU rows per lane per pass, UU just large enough for C, and
// every load of a pass is issued before any is used: rows past C read
// candidate 0 again (always a valid address) and their scores are dropped,
// so no branch splits the loads.
template <typename T, int D, int UU>
__device__ inline void score_rows(const float *sl, int C, bool all, const int *cand,
                                  uint64_t *keys, int bits, const QRaw<T> &qr, int nsw,
                                  int w, int lane) {
  constexpr int LPR = D / 4;    // lanes per fp32 summary row
  constexpr int RPI = 64 / LPR; // rows per wave-wide load
  constexpr int REP = LPR / UU; // lanes sharing one reduced score
  static_assert(UU >= 1 && UU <= LPR, "rows per lane");
  const int rsub = lane / LPR;
  const int rows = UU * nsw * RPI;
  for (int base = 0; base < C; base += rows) {
    int node[UU];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      const int pos = base + (u * nsw + w) * RPI + rsub;
      const int pc = pos < C ? pos : 0;
      node[u] = all ? pc : cand[pc];
    }
    float4 v[UU];
#pragma unroll
    for (int u = 0; u < UU; ++u)
      v[u] = *reinterpret_cast<const float4 *>(sl + static_cast<int64_t>(node[u]) * D);
    double q[4];
    qr.widen(q);
    double part[UU];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      // fp32 x (fp32 or bf16) products are exact in fp64
      double s = q[0] * static_cast<double>(v[u].x);
      s = fma(q[1], static_cast<double>(v[u].y), s);
      s = fma(q[2], static_cast<double>(v[u].z), s);
      s = fma(q[3], static_cast<double>(v[u].w), s);
      part[u] = s;
    }
    const double s = group_transpose_reduce<UU, LPR>(part, lane);
    const int k = (lane % LPR) / REP;
    const int pos = base + (k * nsw + w) * RPI + rsub;
    if ((lane % REP) == 0 && pos < C) keys[pos] = score_key(s, all ? pos : cand[pos], bits);
  }
}

// Walks query qi down the tree (every wave of the NW-wave workgroup takes
// part).  On return, after a barrier, sh.front[0 .. beam) holds the kept
// leaves in rank order, best first.  Levels whose candidate set is no larger
// than the beam keep every node whatever the scores, so the walk starts at
// the first level that cuts (a.first_cut); its candidates are all of its
// nodes, so its loads need no selection and go out together with the query
// row.
//
// Only the first NRW waves work on the walk; all NW waves pass its barriers.
// A workgroup's waves start one after another (on MI355X the last of 16
// starts about a microsecond after the first), so leaving the late waves out
// of the walk keeps them off its critical path: they only have to reach
// each barrier, and the attention after the walk is where they are needed.
template <typename T, int D, int NW, int NRW>
__device__ void route_walk(const RouteArgs &a, RouteShared<NW> &sh, int qi) {
  constexpr int NT = NW * 64;
  constexpr int LOG_NRT = NRW == 16 ? 10 : NRW == 8 ? 9 : NRW == 4 ? 8 : -1;
  static_assert(LOG_NRT > 0 && NRW <= NW, "4, 8 or 16 walking waves");
  static_assert(kMaxCandidates <= NRW * 64 / 2, "two or more threads per candidate");
  constexpr int LPR = D / 4;          // lanes per fp32 summary row
  constexpr int RPI = 64 / LPR;       // rows per wave-wide load

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int bi = qi / a.q_heads;
  const int hq = qi - bi * a.q_heads;
  const int64_t head = static_cast<int64_t>(bi) * a.kv_heads + hq / a.group;
  const int b = a.branching;
  const int W = a.beam;
  const int lv = a.levels;
  const int l0 = a.first_cut;
  const int col = (lane % LPR) * 4;

  QRaw<T> qr;
  qr.load(static_cast<const T *>(a.Q) + static_cast<int64_t>(qi) * D + col);
  if (a.trace) {
    int n_at_l = 1;
    for (int l = 1; l < l0; ++l) {
      n_at_l *= b;  // levels before l0 have at most beam nodes
      int32_t *tr = a.trace + (static_cast<int64_t>(qi) * lv + (l - 1)) * W;
      for (int k = tid; k < W; k += NT) tr[k] = k < n_at_l ? k : -1;
    }
  }

  // level sizes and offsets follow from b alone (scalar arithmetic, no
  // loads): n_l = b^l, and level l starts after heads * d * (b + ... + b^(l-1))
  const int64_t heads = static_cast<int64_t>(a.queries / a.q_heads) * a.kv_heads;
  int64_t n_l = 1, off = 0;
  for (int l = 1; l < l0; ++l) {
    n_l *= b;
    off += heads * n_l * D;
  }
  int cur = 0;
  int nf = static_cast<int>(n_l);
  for (int l = l0; l <= lv; ++l) {
    n_l *= b;
    const int C = nf * b;
    const bool all = l == l0;  // candidates are nodes 0..C-1 of level l
    if (C > W) {
      const int bits = 32 - __clz(static_cast<int>(n_l) - 1);
      const float *sl = a.summ + off + head * n_l * D + col;
      // the walking waves score, each lane taking `per` rows
      const int per = (C + NRW * RPI - 1) / (NRW * RPI);
      const int *cand = sh.cand[cur];
      if (w < NRW) {
        if (per <= 1)
          score_rows<T, D, 1>(sl, C, all, cand, sh.keys, bits, qr, NRW, w, lane);
        else if (per <= 2)
          score_rows<T, D, 2>(sl, C, all, cand, sh.keys, bits, qr, NRW, w, lane);
        else if (per <= 4)
          score_rows<T, D, 4>(sl, C, all, cand, sh.keys, bits, qr, NRW, w, lane);
        else
          score_rows<T, D, 8>(sl, C, all, cand, sh.keys, bits, qr, NRW, w, lane);
      }
      __syncthreads();
      // rank of candidate i = number of candidates with a larger key.  Each
      // candidate has a group of g adjacent lanes (g <= 8); lane p of the
      // group counts over keys p, p+g, p+2g, ... (so the g lanes read g
      // neighbouring keys: no bank conflict, and every group of the wave
      // reads the same addresses), then the group adds its counts with DPP,
      // so the ranks need no further trip through LDS.
      if (w < NRW) {
        const int lcp = 32 - __clz(C - 1);
        const int lg = min(LOG_NRT - lcp, 3);
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
          const int node = all ? i : cand[i];
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
    off += heads * n_l * D;
    if (a.trace) {
      int32_t *tr = a.trace + (static_cast<int64_t>(qi) * lv + (l - 1)) * W;
      write_ascending<NT>(sh.front, nf, tr);
      for (int k = nf + tid; k < W; k += NT) tr[k] = -1;
    }
  }
}

}  // namespace tis
