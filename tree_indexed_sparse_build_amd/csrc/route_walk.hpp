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

// Raw bits of this lane's E query elements (columns col .. col + E - 1, E
// the summary elements one 16-byte load holds: 4 float32 or 8 bfloat16).
// They stay raw until a level's summary loads are in flight, so the wait for
// the query row overlaps those loads.
template <typename T, int E> struct QRaw;
template <> struct QRaw<float, 4> {
  uint4 r;
  __device__ inline void load(const float *q) { r = *reinterpret_cast<const uint4 *>(q); }
  __device__ inline void widen(double *out) const {
    out[0] = __uint_as_float(pin(r.x));
    out[1] = __uint_as_float(pin(r.y));
    out[2] = __uint_as_float(pin(r.z));
    out[3] = __uint_as_float(pin(r.w));
  }
};
template <> struct QRaw<float, 8> {
  QRaw<float, 4> lo, hi;
  __device__ inline void load(const float *q) {
    lo.load(q);
    hi.load(q + 4);
  }
  __device__ inline void widen(double *out) const {
    lo.widen(out);
    hi.widen(out + 4);
  }
};
template <> struct QRaw<bf16_bits, 4> {
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
template <> struct QRaw<bf16_bits, 8> {
  uint4 r;
  __device__ inline void load(const bf16_bits *q) { r = *reinterpret_cast<const uint4 *>(q); }
  __device__ inline void widen(double *out) const {
    const uint4 p = make_uint4(pin(r.x), pin(r.y), pin(r.z), pin(r.w));
    float f[8];
    Vec16<bf16_bits>::unpack(p, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = f[e];
  }
};

// Shared memory of one query's walk, for a workgroup of NW waves whose
// levels have at most MAXC candidates.
template <int NW, int MAXC = kMaxCandidates> struct RouteShared {
  uint64_t keys[MAXC];
  int cand[2][MAXC];     // node id of every candidate (-1: hole), this level / next
  int front[MAXC];       // kept nodes of the level, in rank order
  int holes[3];          // holes among a level's candidates, slot l mod 3
};

// Level table of one causal-prefill query (position t routes over the tree
// of the first n = t + 1 keys): its depth, first cut level, and per level l
// the nodes that exist, the summary rows per head and block offset of its
// height, and the element offset of its open node's row (the node holding
// key t, whose mean covers keys up to t only) in the table of partial means.
struct CausalLevels {
  int levels, first_cut;
  int64_t exist[kMaxLevels + 2];
  int64_t rows[kMaxLevels + 1];
  int64_t off[kMaxLevels + 1];
  int64_t open_off[kMaxLevels + 1];
};

// Sizes and summary rows of the levels of one (batch, KV head), walked from
// level l0 downwards.  LAYOUT 0: full tree (sizes by scalar arithmetic);
// 1: growing cache (a host table in the arguments); 2: causal prefill (the
// query's own table, in LDS).
template <int LAYOUT> struct LevelCursor {
  int64_t exist;   // nodes of the current level that exist
  int64_t rows;    // summary rows per head in the current level's block
  int64_t off;     // element offset of the current level's block
  int64_t heads;
  int l;           // current level
  int b;
  const RouteArgs *a;
  const CausalLevels *cl;

  __device__ void init(const RouteArgs &ra, const CausalLevels *c, int l0, int d) {
    a = &ra;
    cl = c;
    b = ra.branching;
    l = l0;
    heads = static_cast<int64_t>(div_u(ra.queries, ra.q_heads)) * ra.kv_heads;
    if constexpr (LAYOUT == 0) {
      // full tree: level l has b^l nodes, levels 1 .. l-1 come first
      int64_t n = 1;
      off = 0;
      for (int k = 1; k < l0; ++k) {
        n *= b;
        off += heads * n * d;
      }
      exist = rows = n * b;
    } else if constexpr (LAYOUT == 1) {
      // growing cache: sizes and offsets come from the host (no division)
      exist = ra.lvl_exist[l0];
      rows = ra.lvl_rows[l0];
      off = ra.lvl_off[l0];
    } else {
      exist = cl->exist[l0];
      rows = cl->rows[l0];
      off = cl->off[l0];
    }
  }
  // nodes of the next level down that exist
  __device__ int64_t exist_below() const {
    if constexpr (LAYOUT == 0) return exist * b;
    if constexpr (LAYOUT == 1) return a->lvl_exist[l + 1];
    return cl->exist[l + 1];
  }
  __device__ void down(int d) {
    ++l;
    if constexpr (LAYOUT == 0) {
      off += heads * rows * d;
      rows *= b;
      exist = rows;
    } else if constexpr (LAYOUT == 1) {
      exist = a->lvl_exist[l];
      rows = a->lvl_rows[l];
      off = a->lvl_off[l];
    } else {
      exist = cl->exist[l];
      rows = cl->rows[l];
      off = cl->off[l];
    }
  }
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

// Scores the C candidates of one level: candidate p is node node_of(p) of
// the level (negative: a hole, which reads node 0), whose summary elements
// for this lane's columns start at row_of(node), and emit(p, node, score)
// receives its fp64 dot with the query (once per candidate).  The nsw waves
// of the workgroup cover UU rows per lane per pass, UU just large enough for
// C, and every load of a pass is issued before any is used: rows past C read
// candidate 0 again (always a valid address) and their scores are dropped,
// so no branch splits the loads.  A lane loads 16 bytes of a row: 4 float32
// or 8 bfloat16 summary elements.
struct NoScale {
  __device__ float operator()(int) const { return 1.f; }
};

// The walk's optional side job (see route_walk): none.
struct NoPrep {};

template <typename T, typename S, int D, int UU, bool HOLES, typename NodeOf, typename RowOf,
          typename Emit, typename ScaleOf = NoScale>
__device__ inline void score_rows(RowOf row_of, int C, NodeOf node_of, Emit emit,
                                  const QRaw<T, RowLoad<S>::E> &qr, int nsw, int w, int lane,
                                  ScaleOf scale_of = ScaleOf()) {
  constexpr int E = RowLoad<S>::E;
  constexpr int LPR = D / E;    // lanes per summary row
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
      node[u] = node_of(pos < C ? pos : 0);
    }
    typename RowLoad<S>::Raw v[UU];
    float scl[UU];  // fp8 rows: the row's power-of-two scale
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      const int nd = HOLES && node[u] < 0 ? 0 : node[u];  // a hole reads node 0
      v[u] = RowLoad<S>::load(row_of(nd));
      if constexpr (kIsFp8<S>) scl[u] = scale_of(nd);
    }
    double q[E];
    qr.widen(q);
    double part[UU];
#pragma unroll
    for (int u = 0; u < UU; ++u) {
      // fp32 x (fp32, bf16 or e4m3) products are exact in fp64, and so is
      // the scaling of an fp8 row's partial dot by its power of two
      float f[E];
      RowLoad<S>::unpack(v[u], f);
      double s = q[0] * static_cast<double>(f[0]);
#pragma unroll
      for (int e = 1; e < E; ++e) s = fma(q[e], static_cast<double>(f[e]), s);
      if constexpr (kIsFp8<S>) s *= static_cast<double>(scl[u]);
      part[u] = s;
    }
    const double s = group_transpose_reduce<UU, LPR>(part, lane);
    const int k = (lane % LPR) / REP;
    const int pos = base + (k * nsw + w) * RPI + rsub;
    if ((lane % REP) == 0 && pos < C) emit(pos, node_of(pos), s);
  }
}

// Walks query qi down the tree (every wave of the NW-wave workgroup takes
// part) and returns how many leaves it keeps (beam, or fewer when a growing
// cache has fewer leaves).  On return, after a barrier, sh.front[0 .. that)
// holds the kept leaves in rank order, best first.  Levels whose existing
// nodes number no more than the beam keep them all whatever the scores, so
// the walk starts at the first level l0 that cuts (a.first_cut); its
// candidates are all of its nodes, so its loads need no selection and go out
// together with the query row.  Below l0 the candidates are the children of
// the kept nodes; in a growing cache the last existing node may have fewer
// children, and the missing ones are holes that score below every node.
//
// Only the first NRW waves work on the walk; all NW waves pass its barriers.
// A workgroup's waves start one after another (on MI355X the last of 16
// starts about a microsecond after the first), so leaving the late waves out
// of the walk keeps them off its critical path: they only have to reach
// each barrier, and the attention after the walk is where they are needed.
//
// With a Prep other than NoPrep (growing cache only), the score of the last
// existing node of each level (the open node, whose stored row is not
// current) comes from open_score[l] instead of its row.  The waves that do
// not walk call prep->run(w - NRW, lane) as they start: it must fill
// open_score[l] for l0 < l <= levels and write level l0's key of that node
// into sh.keys before they reach the walk's first barrier (the walking
// waves score the other nodes of level l0 meanwhile).
template <typename T, typename S, int D, int NW, int NRW, int LAYOUT,
          int MAXC = kMaxCandidates, typename Prep = NoPrep, int SMAXC = kMaxCandidates>
__device__ int route_walk(const RouteArgs &a, RouteShared<NW, SMAXC> &sh, int qi,
                          const CausalLevels *cl = nullptr, const void *open_summ = nullptr,
                          int hrow = -1, const Prep *prep = nullptr,
                          const double *open_score = nullptr,
                          unsigned long long *tl = nullptr) {
  constexpr bool CACHE = LAYOUT != 0;  // nodes past the last key may be missing
  constexpr bool OPEN = !__is_same(Prep, NoPrep);
  static_assert(!kIsFp8<S> || LAYOUT == 0, "fp8 summaries: full tree only");
  static_assert(!OPEN || (LAYOUT == 1 && NRW < NW), "open-node scores: growing cache, idle waves");
  constexpr int NT = NW * 64;
  constexpr int LOG_NRT =
      NRW == 16 ? 10 : NRW == 8 ? 9 : NRW == 4 ? 8 : NRW == 2 ? 7 : NRW == 1 ? 6 : -1;
  static_assert(LOG_NRT > 0 && NRW <= NW, "1, 2, 4, 8 or 16 walking waves");
  // MAXC: the most candidates a level of this launch may have (beam * b,
  // checked by the host); the ranking needs two or more threads for each
  static_assert(MAXC <= SMAXC && MAXC <= NRW * 64 / 2, "two or more threads per candidate");
  constexpr int E = RowLoad<S>::E;     // summary elements per lane (one load)
  constexpr int LPR = D / E;           // lanes per summary row
  constexpr int RPI = 64 / LPR;        // rows per wave-wide load

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  // (batch, query head) row of the query: qi itself, or given (prefill)
  const int hr = LAYOUT == 2 ? hrow : qi;
  const int bi = div_u(hr, a.q_heads);
  const int hq = hr - bi * a.q_heads;
  const int64_t head = static_cast<int64_t>(bi) * a.kv_heads + div_u(hq, a.group);
  const int b = a.branching;
  const int W = a.beam;
  const int lv = LAYOUT == 2 ? cl->levels : a.levels;
  const int l0 = LAYOUT == 2 ? cl->first_cut : a.first_cut;
  const int col = (lane % LPR) * E;

  QRaw<T, E> qr;
  qr.load(static_cast<const T *>(a.Q) + static_cast<int64_t>(qi) * D + col);


  if constexpr (OPEN) {
    if (w >= NRW) prep->run(w - NRW, lane);
  }

  LevelCursor<LAYOUT> lc;
  lc.init(a, cl, l0, D);
  if (a.trace) {
    // levels above l0 keep every node that exists
    for (int l = 1; l < l0; ++l) {
      int64_t n = 1;
      for (int k = 0; k < l; ++k) n *= b;
      const int64_t e = LAYOUT == 2 ? cl->exist[l] : CACHE ? a.lvl_exist[l] : n;
      int32_t *tr = a.trace + (static_cast<int64_t>(qi) * lv + (l - 1)) * W;
      for (int k = tid; k < W; k += NT) tr[k] = k < e ? k : -1;
    }
  }
  // slot l mod 3 holds the holes among level l's candidates: level l reads
  // its slot, writes the next one and clears the one after, which no level
  // touches between two barriers of this one
  if (CACHE && tid == 0) sh.holes[0] = sh.holes[1] = sh.holes[2] = 0;

  int cur = 0;
  // kept nodes of the level above l0: all that exist (the root when l0 = 1)
  int nf;
  {
    int64_t n_above = 1;
    if (l0 > 1) {
      if constexpr (LAYOUT == 0) {
        for (int l = 1; l < l0; ++l) n_above *= b;
      } else if constexpr (LAYOUT == 1) {
        n_above = a.lvl_exist[l0 - 1];
      } else {
        n_above = cl->exist[l0 - 1];
      }
    }
    nf = static_cast<int>(n_above);
  }
  for (int l = l0; l <= lv; ++l) {
    const bool all = l == l0;  // candidates are nodes 0..C-1 of level l
    // candidate slots, and how many of them are real nodes
    const int C = all ? static_cast<int>(lc.exist) : nf * b;
    // a full tree has no holes: every child exists
    const int live = (all || !CACHE) ? C : C - sh.holes[l % 3];
    const int keep = live < W ? live : W;
    const int64_t e_below = CACHE && l < lv ? lc.exist_below() : 0;
    int *holes_next = &sh.holes[(l + 1) % 3];
    if (CACHE && tid == 0) sh.holes[(l + 2) % 3] = 0;
    if (live > W) {
      const int bits = 32 - __clz(static_cast<int>(lc.exist) - 1);
      const S *sl = static_cast<const S *>(a.summ) + lc.off + head * lc.rows * D + col;
      // prefill: the open node (the last that exists) covers keys up to the
      // query's position only; its mean comes from the table of partial means
      const S *open_row = LAYOUT == 2 ? static_cast<const S *>(open_summ) + cl->open_off[l] + col
                                      : sl;
      const int64_t last = lc.exist - 1;
      const auto row_of = [&](int nd) {
        return LAYOUT == 2 && nd == last ? open_row : sl + static_cast<int64_t>(nd) * D;
      };
      const float *scl = kIsFp8<S> ? a.scales + lc.off / D + head * lc.rows : nullptr;
      const auto scale_of = [&](int nd) { return scl[nd]; };
      // the walking waves score, each lane taking `per` rows
      const int per = (C + NRW * RPI - 1) / (NRW * RPI);
      const int *cand = sh.cand[cur];
      const auto node_of = [&](int p) { return all ? p : cand[p]; };
      uint64_t *keys = sh.keys;
      const auto emit = [&](int pos, int nd, double s) {
        if constexpr (OPEN) {
          // the open node: prep wrote its key at l0 and its score below
          if (nd == last) {
            if (l != l0) keys[pos] = score_key(open_score[l], nd, bits);
            return;
          }
        }
        // a hole (a child past the end of a growing cache) gets key 0, below
        // every real key, so it is never ranked among the kept
        keys[pos] = CACHE && nd < 0 ? 0ull : score_key(s, nd, bits);
      };
      if (w < NRW) {
        if (per <= 1)
          score_rows<T, S, D, 1, CACHE>(row_of, C, node_of, emit, qr, NRW, w, lane, scale_of);
        else if (per <= 2)
          score_rows<T, S, D, 2, CACHE>(row_of, C, node_of, emit, qr, NRW, w, lane, scale_of);
        else if (per <= 4 || kIsFp8<S>)  // fp8: at most 4 rows a lane (registers), then passes
          score_rows<T, S, D, 4, CACHE>(row_of, C, node_of, emit, qr, NRW, w, lane, scale_of);
        else
          score_rows<T, S, D, 8, CACHE>(row_of, C, node_of, emit, qr, NRW, w, lane, scale_of);
      }
      if (l - l0 < 8) tl_stamp(tl, 8 + 2 * (l - l0));
      __syncthreads();
      // rank of candidate i = number of candidates with a larger key.  Each
      // candidate has a group of g adjacent lanes (g <= 8); lane p of the
      // group counts over keys p, p+g, p+2g, ... (so the g lanes read g
      // neighbouring keys: no bank conflict, and every group of the wave
      // reads the same addresses), then the group adds its counts with DPP,
      // so the ranks need no further trip through LDS.  Holes have key 0 and
      // rank at least `live`, so they are never kept.
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
        if (i < C && part == 0 && cnt < keep) {
          const int node = all ? i : cand[i];
          sh.front[cnt] = node;
          if (l < lv) {
            int missing = 0;
            for (int c = 0; c < b; ++c) {
              const int child = node * b + c;
              const bool exists = !CACHE || child < e_below;
              sh.cand[cur ^ 1][cnt * b + c] = exists ? child : -1;
              missing += exists ? 0 : 1;
            }
            if (CACHE && missing) *holes_next = missing;  // only the last node has holes
          }
        }
      }
    } else {
      // no cut: every real candidate is kept, in slot order
      if (tid < C) {
        const int node = all ? tid : sh.cand[cur][tid];
        if (node >= 0) {
          // slots past the holes move down by their number
          int r = tid;
          if (CACHE && !all && sh.holes[l % 3] && tid > 0) {
            for (int j = 0; j < tid; ++j) r -= sh.cand[cur][j] < 0 ? 1 : 0;
          }
          sh.front[r] = node;
          if (l < lv) {
            int missing = 0;
            for (int c = 0; c < b; ++c) {
              const int child = node * b + c;
              const bool exists = !CACHE || child < e_below;
              sh.cand[cur ^ 1][r * b + c] = exists ? child : -1;
              missing += exists ? 0 : 1;
            }
            if (CACHE && missing) *holes_next = missing;
          }
        }
      }
    }
    __syncthreads();
    if (live > W && l - l0 < 8) tl_stamp(tl, 9 + 2 * (l - l0));
    cur ^= 1;
    nf = keep;
    if (l < lv) lc.down(D);
    if (a.trace) {
      int32_t *tr = a.trace + (static_cast<int64_t>(qi) * lv + (l - 1)) * W;
      write_ascending<NT>(sh.front, nf, tr);
      for (int k = nf + tid; k < W; k += NT) tr[k] = -1;
    }
  }
  return nf;
}

}  // namespace tis
