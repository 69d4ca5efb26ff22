// Threshold retrieval over the summary tree with bounding spheres ("Sparse
// Attention as a Range Searching Problem", Methodologie: every key whose
// score reaches a threshold is retrieved; clusters enclosed by bounding
// spheres are pruned when the sphere cannot reach the threshold, so no such
// key is ever lost; survivors are checked exactly).  The clusters are the
// nodes of the summary tree ("Subquadratic Attention with a Hierarchical
// Tree-Structured Indexer", Abstract), so pruning runs level by level.
//
//  * k_radius: for every key, its squared distance (fp64) to the stored
//    summary of each of its lv ancestors; the largest per node is reduced
//    with 64-bit atomic max on the ordered fp64 bits.  A wave owns a run of
//    consecutive leaves of one head and keeps, per level, the running
//    maximum of the node its leaves are under (one lane per level), so it
//    issues one atomic per node it touches.  K is streamed once in batches
//    of 4 row loads a lane, the next batch in flight while the current one
//    is worked on; a batch's keys are widened to fp64 once and reused for
//    every level, since the pass is bound by its fp64 arithmetic (a
//    subtraction and an FMA per key element and level).  The ancestors'
//    summaries go through LDS; only the nodes that change are reloaded, and
//    the next leaf's own centre is fetched ahead of its rows.
//  * k_radius_quad: the same maxima for leaf blocks of at least 64 keys and
//    trees of up to 8 levels: 4 lanes a key, 4 keys a lane sharing each
//    widened centre value, a running maximum per level reduced across the
//    wave only when the level's node ends.
//  * k_radius_finish: radius = smallest float32 r with r * r >= the maximum
//    (r * r is exact in fp64, so the test is exact).
//  * threshold walk: one workgroup per query; level by level, the children
//    of the survivors are scored (the beam walk's fp64 row dots) and
//    survive when q.c + |q| r >= tau (fp64); survivors are compacted in
//    ascending order by wave ballots.  A level with more than max_nodes
//    survivors ends the walk as an overflow.
//  * the fused decode attends over the surviving leaves, keeping only keys
//    whose fp64 score reaches tau.
#include "attend_query.hpp"
#include "route_walk.hpp"

namespace tis {
namespace {

constexpr int kRadiusWaves = 4;

template <typename T, typename S, int D>
__global__ void __launch_bounds__(kRadiusWaves * 64) k_radius(RadiusArgs a) {
  using AG = AttendGeom<T, D>;  // row geometry of 16-byte K loads
  constexpr int E = AG::E, LPR = AG::LPR, R = AG::R;
  // U row loads a lane per batch, small enough that the batch's keys stay
  // widened to fp64 across the levels (each element is converted once, then
  // costs a subtraction and an FMA per level: the pass is fp64-bound)
  constexpr int U = 4, RB = U * R, REP = LPR / U;
  static_assert(U <= LPR, "a batch's distances must fit one reduction");
  __shared__ float ctr[kRadiusWaves][kMaxLevels + 1][D];  // this leaf's ancestors' centres
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * kRadiusWaves + w;
  const int64_t head = gw / a.waves_per_head;
  if (head >= a.heads) return;  // whole wave: no barrier below spans waves
  const int64_t n_leaves = a.n_at[a.levels];
  const int64_t leaf0 = (gw - head * a.waves_per_head) * a.leaves_per_wave;
  const int64_t leaf1 = min(leaf0 + a.leaves_per_wave, n_leaves);
  const int lv = a.levels;
  const int L = a.leaf_block;
  const int col = (lane % LPR) * E;
  const int rsub = lane / LPR;
  const int kk = (lane % LPR) / REP;
  const T *kh = static_cast<const T *>(a.K) + head * a.n_keys * D + col;
  const S *summ = static_cast<const S *>(a.summ);
  float (*cw)[D] = ctr[w];

  // lane l - 1 keeps level l's node and the running maximum under it
  const int my_level = lane + 1;
  const bool owner = my_level <= lv;
  const int64_t my_span = owner ? a.span[my_level] : 1;
  int64_t my_node = -1;
  double my_max = 0.0;
  auto flush = [&]() {
    if (owner && my_node >= 0)
      atomicMax(a.d2 + a.node_off[my_level] + head * a.n_at[my_level] + my_node,
                static_cast<unsigned long long>(__double_as_longlong(my_max)));
  };

  // centre row of node `anc` of level l, this lane's columns c = lane, lane + 64
  constexpr int CPL = D / 64;  // centre elements per lane
  const auto centre = [&](int l, int64_t anc, float (&f)[CPL]) {
    const S *row = summ + a.summ_off[l] + (head * a.n_at[l] + anc) * D;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = lane + 64 * j;
      if constexpr (sizeof(S) == 4) {
        f[j] = reinterpret_cast<const float *>(row)[c];
      } else {
        f[j] = __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const bf16_bits *>(row)[c].v)
                               << 16);
      }
    }
  };
  // the levels whose node changes at `leaf` flush their maximum and get
  // their new centre (the leaf level's comes from `pre` when given)
  const auto enter = [&](int64_t leaf, const float *pre) {
    const int64_t node = owner ? leaf / my_span : -1;
    if (owner && node != my_node) {
      flush();
      my_node = node;
      my_max = 0.0;
    }
    for (int l = 1; l <= lv; ++l) {
      const int64_t anc = leaf / a.span[l];
      if (l < lv && leaf != leaf0 && anc == (leaf - 1) / a.span[l]) continue;  // same node
      float f[CPL];
      if (l == lv && pre) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) f[j] = pre[j];
      } else {
        centre(l, anc, f);
      }
#pragma unroll
      for (int j = 0; j < CPL; ++j) cw[l][lane + 64 * j] = f[j];
    }
    // LDS accesses of one wave are performed in order: the rows written
    // above are what the lanes read below
    __builtin_amdgcn_wave_barrier();
  };
  // the wave's rows as one stream of batches of RB rows (nb per leaf): the
  // next batch's loads are issued before the current one is worked on, so
  // they are in flight during its fp64 arithmetic
  const int nb = (L + RB - 1) / RB;
  const int64_t total = (leaf1 - leaf0) * nb;
  const auto load_batch = [&](int64_t q, uint4 (&kv)[U]) {
    const int64_t leaf = leaf0 + q / nb;
    const int r0 = static_cast<int>(q % nb) * RB;
    const T *kl = kh + leaf * L * D;
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int row = r0 + i * R + rsub;
      kv[i] = row < L ? load16(kl + static_cast<int64_t>(row) * D) : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  uint4 cur[U], nxt[U];
  if (total > 0) {
    enter(leaf0, nullptr);
    load_batch(0, cur);
  }
  for (int64_t q = 0; q < total; ++q) {
    const int r0 = static_cast<int>(q % nb) * RB;
    const bool next_leaf = q + 1 < total && (q + 1) % nb == 0;
    float pre[CPL];  // the next leaf's own centre, fetched ahead of its rows
    if (next_leaf) centre(lv, leaf0 + (q + 1) / nb, pre);
    if (q + 1 < total) load_batch(q + 1, nxt);
    const bool valid = r0 + kk * R + rsub < L;
    double kd[U][E];  // the batch's keys, widened once
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float k[E];
      Vec16<T>::unpack(cur[i], k);
#pragma unroll
      for (int e = 0; e < E; ++e) kd[i][e] = static_cast<double>(k[e]);
    }
    for (int l = 1; l <= lv; ++l) {
      double c[E];
#pragma unroll
      for (int e = 0; e < E; ++e) c[e] = static_cast<double>(cw[l][col + e]);
      double part[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        double sq = 0.0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const double diff = kd[i][e] - c[e];  // exact: both are float32 values
          sq = fma(diff, diff, sq);
        }
        part[i] = sq;
      }
      // lane holds the squared distance of row r0 + kk * R + rsub
      const double d2 = group_transpose_reduce<U, LPR>(part, lane);
      const double m = wave_max_d(valid ? d2 : 0.0);
      if (lane == l - 1) my_max = fmax(my_max, m);
    }
    if (next_leaf) {
      __builtin_amdgcn_wave_barrier();  // this leaf's centre reads come first
      enter(leaf0 + (q + 1) / nb, pre);
    }
#pragma unroll
    for (int i = 0; i < U; ++i) cur[i] = nxt[i];
  }
  flush();
}

// Smallest float32 r >= 0 with r * r >= D, from the reduced maxima.
// The same maxima for leaf blocks of at least 64 keys and trees of up to 8
// levels: a wave takes 64 keys of one leaf at a time, a lane a quarter of 4
// keys (keys s, s + 16, s + 32, s + 48 of the batch for lane slot s; 64
// contiguous bytes a load round across a key's 4 lanes).  Each centre
// value is widened once and serves the lane's 4 keys, a key's squared
// distance needs only the two in-quad exchanges (DPP, no LDS swizzle), and
// each lane keeps a running maximum per level that is reduced across the
// wave only when that level's node ends.  (k_radius sums a key across 16
// lanes, widens each centre value for every 4 keys and takes a wave
// maximum every 16 keys; measured on the 32K-key GQA workload, its VALU
// and its loads did not overlap.)  Centres and owner lanes as in k_radius.
template <typename T, typename S, int D, int LV>
__global__ void __launch_bounds__(kRadiusWaves * 64) k_radius_quad(RadiusArgs a) {
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int NL = D * ES / 64;  // 16-byte loads a lane per key (a quarter key)
  constexpr int EPL = 16 / ES;     // elements a load
  constexpr int KPL = 4;           // keys a lane
  __shared__ float ctr[kRadiusWaves][LV][D];  // this leaf's ancestors' centres
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int64_t gw = static_cast<int64_t>(blockIdx.x) * kRadiusWaves + w;
  const int64_t head = gw / a.waves_per_head;
  if (head >= a.heads) return;  // whole wave: no barrier below spans waves
  const int64_t n_leaves = a.n_at[LV];
  const int64_t leaf0 = (gw - head * a.waves_per_head) * a.leaves_per_wave;
  const int64_t leaf1 = min(leaf0 + a.leaves_per_wave, n_leaves);
  const int L = a.leaf_block;
  const int ks = lane >> 2;   // this lane's key slot within the batch
  const int part = lane & 3;  // and its quarter: bytes part * 16 + 64 i
  const T *kh = static_cast<const T *>(a.K) + head * a.n_keys * D;
  const S *summ = static_cast<const S *>(a.summ);
  float (*cw)[D] = ctr[w];

  // the centres of `leaf`'s ancestors, this lane's columns lane + 64 j
  // (fetched a leaf ahead, written to LDS when the leaf starts)
  constexpr int CPL = D / 64;
  const auto fetch_centres = [&](int64_t leaf, float (&f)[LV][CPL]) {
#pragma unroll
    for (int l = 1; l <= LV; ++l) {
      const S *row = summ + a.summ_off[l] + (head * a.n_at[l] + leaf / a.span[l]) * D;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = lane + 64 * j;
        if constexpr (sizeof(S) == 4)
          f[l - 1][j] = reinterpret_cast<const float *>(row)[c];
        else
          f[l - 1][j] = __uint_as_float(
              static_cast<uint32_t>(reinterpret_cast<const bf16_bits *>(row)[c].v) << 16);
      }
    }
  };
  const auto enter = [&](const float (&f)[LV][CPL]) {
#pragma unroll
    for (int l = 0; l < LV; ++l)
#pragma unroll
      for (int j = 0; j < CPL; ++j) cw[l][lane + 64 * j] = f[l][j];
    // LDS accesses of one wave are performed in order: the rows written
    // above are what the lanes read below
    __builtin_amdgcn_wave_barrier();
  };
  // the finished nodes' maxima: a wave maximum of the lanes' running
  // maxima, taken by the level's owner lane (l - 1) to the node's slot
  double run[LV];
#pragma unroll
  for (int l = 0; l < LV; ++l) run[l] = 0.0;
  const auto finish = [&](int64_t leaf, bool last) {
#pragma unroll
    for (int l = 1; l <= LV; ++l) {
      const int64_t node = leaf / a.span[l];
      if (!last && node == (leaf + 1) / a.span[l]) continue;  // the node goes on
      const double m = wave_max_d(run[l - 1]);
      if (lane == l - 1)
        atomicMax(a.d2 + a.node_off[l] + head * a.n_at[l] + node,
                  static_cast<unsigned long long>(__double_as_longlong(m)));
      run[l - 1] = 0.0;
    }
  };
  // load round i of the batch at row r0 of `leaf`: 16 bytes of each of the
  // lane's keys (rows past the block read its last row and are masked)
  const auto load_round = [&](int64_t leaf, int r0, int i, uint4 (&kv)[KPL]) {
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const int row = min(r0 + ks + 16 * k, L - 1);
      kv[k] = load16(reinterpret_cast<const unsigned char *>(kh + (leaf * L + row) * D) +
                     part * 16 + i * 64);
    }
  };
  // one stream of load rounds over the wave's leaves, batches and rounds,
  // the next round's loads (and at a leaf's last round the next leaf's
  // centres) in flight while this one computes
  if (leaf0 >= leaf1) return;
  {
    float f[LV][CPL];
    fetch_centres(leaf0, f);
    enter(f);
  }
  int64_t leaf = leaf0;
  int r0 = 0, i = 0;
  uint4 cur[KPL], nxt[KPL];
  float pre[LV][CPL];
  load_round(leaf, r0, i, cur);
  double sq[KPL][LV];
#pragma unroll
  for (int k = 0; k < KPL; ++k)
#pragma unroll
    for (int l = 0; l < LV; ++l) sq[k][l] = 0.0;
  for (;;) {
    // the next round
    int64_t nleaf = leaf;
    int nr0 = r0, ni = i + 1;
    if (ni == NL) {
      ni = 0;
      nr0 += 16 * KPL;
      if (nr0 >= L) {
        nr0 = 0;
        ++nleaf;
      }
    }
    const bool more = nleaf < leaf1;
    if (more) load_round(nleaf, nr0, ni, nxt);
    const bool new_leaf = more && nleaf != leaf;
    if (new_leaf) fetch_centres(nleaf, pre);
    double kd[KPL][EPL];  // this round's elements of the lane's keys, widened
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      float fv[EPL];
      Vec16<T>::unpack(cur[k], fv);
#pragma unroll
      for (int e = 0; e < EPL; ++e) kd[k][e] = static_cast<double>(fv[e]);
    }
#pragma unroll
    for (int l = 0; l < LV; ++l) {
      const float *c = cw[l] + (part * 16 + i * 64) / ES;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const double cd = static_cast<double>(c[e]);
#pragma unroll
        for (int k = 0; k < KPL; ++k) {
          const double diff = kd[k][e] - cd;  // exact: both are float32 values
          sq[k][l] = fma(diff, diff, sq[k][l]);
        }
      }
    }
    if (i == NL - 1) {  // the batch's keys are complete
#pragma unroll
      for (int k = 0; k < KPL; ++k) {
        const bool valid = r0 + ks + 16 * k < L;
#pragma unroll
        for (int l = 0; l < LV; ++l) {
          double d = sq[k][l];
          d += xor_lane<1>(d, lane);
          d += xor_lane<2>(d, lane);  // the key's squared distance, in its 4 lanes
          run[l] = fmax(run[l], valid ? d : 0.0);
          sq[k][l] = 0.0;
        }
      }
    }
    if (!more || new_leaf) {
      finish(leaf, !more);
      if (!more) break;
      __builtin_amdgcn_wave_barrier();  // this leaf's centre reads come first
      enter(pre);
    }
    leaf = nleaf;
    r0 = nr0;
    i = ni;
#pragma unroll
    for (int k = 0; k < KPL; ++k) cur[k] = nxt[k];
  }
}

template <typename T, typename S, int D>
bool launch_radius_quad(const RadiusArgs &a, dim3 grid, hipStream_t s) {
  const dim3 block(kRadiusWaves * 64);
  switch (a.levels) {
    case 1: hipLaunchKernelGGL((k_radius_quad<T, S, D, 1>), grid, block, 0, s, a); return true;
    case 2: hipLaunchKernelGGL((k_radius_quad<T, S, D, 2>), grid, block, 0, s, a); return true;
    case 3: hipLaunchKernelGGL((k_radius_quad<T, S, D, 3>), grid, block, 0, s, a); return true;
    case 4: hipLaunchKernelGGL((k_radius_quad<T, S, D, 4>), grid, block, 0, s, a); return true;
    case 5: hipLaunchKernelGGL((k_radius_quad<T, S, D, 5>), grid, block, 0, s, a); return true;
    case 6: hipLaunchKernelGGL((k_radius_quad<T, S, D, 6>), grid, block, 0, s, a); return true;
    case 7: hipLaunchKernelGGL((k_radius_quad<T, S, D, 7>), grid, block, 0, s, a); return true;
    case 8: hipLaunchKernelGGL((k_radius_quad<T, S, D, 8>), grid, block, 0, s, a); return true;
    default: return false;
  }
}

__global__ void __launch_bounds__(256) k_radius_finish(const unsigned long long *d2,
                                                       float *radii, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const double D = __longlong_as_double(static_cast<long long>(d2[i]));
  float r = static_cast<float>(sqrt(D));
  for (int k = 0; k < 4; ++k)
    if (static_cast<double>(r) * static_cast<double>(r) < D) r = __uint_as_float(__float_as_uint(r) + 1u);
  for (int k = 0; k < 4; ++k) {
    if (r > 0.f) {
      const float dn = __uint_as_float(__float_as_uint(r) - 1u);
      if (static_cast<double>(dn) * static_cast<double>(dn) >= D) r = dn;
    }
  }
  radii[i] = r;
}

// ------------------------------------------------------------------ walk --
template <int NW> struct ThreshShared {
  double sc[NW * 64];            // scores of one chunk of candidates
  int front[2][kMaxSurvivors];   // survivors of the level above / this level
  int wcnt[NW];                  // survivors per wave of a chunk
};

// Walks query qi down the tree with the sphere bound (every wave of the
// NW-wave workgroup takes part; the first NRW score).  Returns the number
// of surviving leaves, or -1 when a level keeps more than max_nodes; the
// survivors are in sh.front[*buf][0 ..), ascending.
template <typename T, typename S, int D, int NW, int NRW>
__device__ int threshold_walk(const RouteArgs &a, const SphereArgs &sa, ThreshShared<NW> &sh,
                              int qi, int *buf) {
  constexpr int NT = NW * 64;
  constexpr int E = Vec16<S>::kElems;
  constexpr int LPR = D / E;
  constexpr int RPI = 64 / LPR;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int bi = qi / a.q_heads;
  const int hq = qi - bi * a.q_heads;
  const int64_t head = static_cast<int64_t>(bi) * a.kv_heads + hq / a.group;
  const int b = a.branching;
  const int lv = a.levels;
  const int col = (lane % LPR) * E;

  QRaw<T, E> qr;
  qr.load(static_cast<const T *>(a.Q) + static_cast<int64_t>(qi) * D + col);
  double qq;
  {
    double qv[E];
    qr.widen(qv);
    qq = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e) qq = fma(qv[e], qv[e], qq);
    qq = group_sum<1, LPR / 2>(qq, lane);
  }
  const double qn = sqrt(qq);
  const double tau = static_cast<double>(sa.tau[qi]);

  LevelCursor<0> lc;
  lc.init(a, nullptr, 1, D);
  if (tid == 0) sh.front[0][0] = 0;  // the root: its children are nodes 0 .. b-1
  __syncthreads();
  int cur = 0, nf = 1;
  for (int l = 1; l <= lv; ++l) {
    const int C = nf * b;
    const S *sl = static_cast<const S *>(a.summ) + lc.off + head * lc.rows * D + col;
    const float *rl = sa.radii + sa.node_off[l] + head * lc.rows;
    const int *fr = sh.front[cur];
    int *nx = sh.front[cur ^ 1];
    double *sc = sh.sc;
    int kept = 0;
    for (int c0 = 0; c0 < C; c0 += NT) {
      const int Cc = min(NT, C - c0);
      const auto node_of = [&](int p) {
        const int g = c0 + p;
        return fr[g / b] * b + g % b;
      };
      int nd = 0;
      float r = 0.f;
      if (tid < Cc) {
        nd = node_of(tid);
        r = rl[nd];
      }
      const auto emit = [&](int pos, int, double s) { sc[pos] = s; };
      const auto row_of = [&](int n) { return sl + static_cast<int64_t>(n) * D; };
      const int per = (Cc + NRW * RPI - 1) / (NRW * RPI);
      if (w < NRW) {
        if (per <= 1)
          score_rows<T, S, D, 1, false>(row_of, Cc, node_of, emit, qr, NRW, w, lane);
        else if (per <= 2)
          score_rows<T, S, D, 2, false>(row_of, Cc, node_of, emit, qr, NRW, w, lane);
        else if (per <= 4)
          score_rows<T, S, D, 4, false>(row_of, Cc, node_of, emit, qr, NRW, w, lane);
        else
          score_rows<T, S, D, 8, false>(row_of, Cc, node_of, emit, qr, NRW, w, lane);
      }
      __syncthreads();
      const bool pass = tid < Cc && sc[tid] + qn * static_cast<double>(r) >= tau;
      const uint64_t m = __ballot(pass);
      if (lane == 0) sh.wcnt[w] = __popcll(m);
      __syncthreads();
      int off = 0, total = 0;
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const int cj = sh.wcnt[j];
        off += j < w ? cj : 0;
        total += cj;
      }
      if (pass) {
        const int pos = kept + off + __popcll(m & ((1ull << lane) - 1ull));
        if (pos < sa.max_nodes) nx[pos] = nd;
      }
      kept += total;
      __syncthreads();
    }
    if (kept > sa.max_nodes) return -1;  // the same on every thread
    nf = kept;
    cur ^= 1;
    if (l < lv) lc.down(D);
  }
  *buf = cur;
  return nf;
}

constexpr int kThreshRouteWaves = 8;

template <typename T, typename S, int D>
__global__ void __launch_bounds__(kThreshRouteWaves * 64)
    k_route_threshold(RouteArgs a, SphereArgs sa) {
  __shared__ ThreshShared<kThreshRouteWaves> sh;
  const int qi = query_of_slot(blockIdx.x, a.queries, a.group);
  int buf = 0;
  const int kept = threshold_walk<T, S, D, kThreshRouteWaves, kThreshRouteWaves>(a, sa, sh, qi,
                                                                                 &buf);
  int32_t *out = a.indices + static_cast<int64_t>(qi) * sa.max_nodes;
  for (int k = threadIdx.x; k < sa.max_nodes; k += kThreshRouteWaves * 64)
    out[k] = k < kept ? sh.front[buf][k] : -1;
  if (threadIdx.x == 0 && sa.counts) sa.counts[qi] = kept;
}

constexpr int kThreshDecodeWaves = 16;
constexpr int kThreshDecodeWalkWaves = 8;

template <typename T, typename S, int D>
__global__ void __launch_bounds__(kThreshDecodeWaves * 64)
    k_decode_threshold(RouteArgs ra, SphereArgs sa, AttendArgs aa) {
  __shared__ ThreshShared<kThreshDecodeWaves> sh;
  __shared__ AttendShared<T, D> ash;
  prefetch_kernargs<sizeof(RouteArgs) + sizeof(SphereArgs) + sizeof(AttendArgs)>();
  const int sp = div_u(static_cast<int>(blockIdx.x), aa.queries);
  const int qi = query_of_slot(blockIdx.x - sp * aa.queries, aa.queries, aa.group);
  const uint4 qraw = attend_q_raw<T, D>(aa, qi);
  int buf = 0;
  const int kept = threshold_walk<T, S, D, kThreshDecodeWaves, kThreshDecodeWalkWaves>(
      ra, sa, sh, qi, &buf);
  if (sp == 0) {
    if (ra.indices) {
      int32_t *out = ra.indices + static_cast<int64_t>(qi) * sa.max_nodes;
      for (int k = threadIdx.x; k < sa.max_nodes; k += kThreshDecodeWaves * 64)
        out[k] = k < kept ? sh.front[buf][k] : -1;
    }
    if (threadIdx.x == 0 && sa.counts) sa.counts[qi] = kept;
  }
  const int n = kept < 0 ? 0 : kept;
  const int s0 = sp * n / aa.splits;
  const int s1 = (sp + 1) * n / aa.splits;
  float *part = aa.splits > 1
                    ? aa.part + (static_cast<int64_t>(qi) * aa.splits + sp) * (D + kPartHeader)
                    : nullptr;
  attend_query<T, D, false, true>(aa, ash, qi, qraw, sh.front[buf] + s0, nullptr, s1 - s0,
                                  kept < 0, part, static_cast<double>(sa.tau[qi]));
  if (aa.splits > 1) merge_parts<D>(aa, qi);
}

// ------------------------------------------------------------- launches --
template <typename T, typename S>
hipError_t launch_radii_ts(int head_dim, const RadiusArgs &a, int64_t waves, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((waves + kRadiusWaves - 1) / kRadiusWaves));
  const dim3 block(kRadiusWaves * 64);
  // leaf blocks of 64 keys or more, up to 8 levels: 4 lanes a key, 4 keys
  // a lane; otherwise 16 lanes a key
  bool quad = false;
  if (head_dim != 128 && head_dim != 64) return hipErrorInvalidValue;
  if (a.leaf_block >= 64)
    quad = head_dim == 128 ? launch_radius_quad<T, S, 128>(a, grid, s)
                           : launch_radius_quad<T, S, 64>(a, grid, s);
  if (!quad) {
    if (head_dim == 128)
      hipLaunchKernelGGL((k_radius<T, S, 128>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((k_radius<T, S, 64>), grid, block, 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2(static_cast<unsigned>((a.total_nodes + 255) / 256));
  hipLaunchKernelGGL(k_radius_finish, g2, dim3(256), 0, s, a.d2, a.radii, a.total_nodes);
  return hipGetLastError();
}

template <typename T, typename S>
hipError_t launch_route_threshold_ts(int head_dim, const RouteArgs &ra, const SphereArgs &sa,
                                     hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ra.queries));
  const dim3 block(kThreshRouteWaves * 64);
  if (head_dim == 128)
    hipLaunchKernelGGL((k_route_threshold<T, S, 128>), grid, block, 0, s, ra, sa);
  else if (head_dim == 64)
    hipLaunchKernelGGL((k_route_threshold<T, S, 64>), grid, block, 0, s, ra, sa);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, typename S>
hipError_t launch_decode_threshold_ts(int head_dim, const RouteArgs &ra, const SphereArgs &sa,
                                      const AttendArgs &aa, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ra.queries) * static_cast<unsigned>(aa.splits));
  const dim3 block(kThreshDecodeWaves * 64);
  if (head_dim == 128)
    hipLaunchKernelGGL((k_decode_threshold<T, S, 128>), grid, block, 0, s, ra, sa, aa);
  else if (head_dim == 64)
    hipLaunchKernelGGL((k_decode_threshold<T, S, 64>), grid, block, 0, s, ra, sa, aa);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_radii(Dt dt, Dt sdt, int head_dim, const RadiusArgs &a, int64_t waves,
                        hipStream_t s) {
  hipError_t e = launch_fill_zero(reinterpret_cast<double *>(a.d2), a.total_nodes, s);
  if (e != hipSuccess) return e;
  if (dt == Dt::BF16)
    return sdt == Dt::BF16 ? launch_radii_ts<bf16_bits, bf16_bits>(head_dim, a, waves, s)
                           : launch_radii_ts<bf16_bits, float>(head_dim, a, waves, s);
  return sdt == Dt::BF16 ? launch_radii_ts<float, bf16_bits>(head_dim, a, waves, s)
                         : launch_radii_ts<float, float>(head_dim, a, waves, s);
}

hipError_t launch_route_threshold(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra,
                                  const SphereArgs &sa, hipStream_t s) {
  if (dt == Dt::BF16)
    return sdt == Dt::BF16 ? launch_route_threshold_ts<bf16_bits, bf16_bits>(head_dim, ra, sa, s)
                           : launch_route_threshold_ts<bf16_bits, float>(head_dim, ra, sa, s);
  return sdt == Dt::BF16 ? launch_route_threshold_ts<float, bf16_bits>(head_dim, ra, sa, s)
                         : launch_route_threshold_ts<float, float>(head_dim, ra, sa, s);
}

hipError_t launch_decode_threshold(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra,
                                   const SphereArgs &sa, const AttendArgs &aa, hipStream_t s) {
  hipError_t e;
  if (dt == Dt::BF16)
    e = sdt == Dt::BF16 ? launch_decode_threshold_ts<bf16_bits, bf16_bits>(head_dim, ra, sa, aa, s)
                        : launch_decode_threshold_ts<bf16_bits, float>(head_dim, ra, sa, aa, s);
  else
    e = sdt == Dt::BF16 ? launch_decode_threshold_ts<float, bf16_bits>(head_dim, ra, sa, aa, s)
                        : launch_decode_threshold_ts<float, float>(head_dim, ra, sa, aa, s);
  return e;
}

}  // namespace tis
