// Causal prefill routing: the query at position t routes over the tree of
// the first t + 1 keys and attends over the keys of its kept leaves up to t
// ("Vdev-Ctrl Releases ALHR", Summary: keys read per query averaged over the
// positions of a 1,024-token input; "Subquadratic Attention with a
// Hierarchical Tree-Structured Indexer", Abstract: the tree over the KV cache
// deepens as the context grows).  Position t sees the growing-cache tree at
// n = t + 1: every node to the left of key t is complete and its summary is
// the one a tree over all n keys stores; only the node holding key t at each
// height (the open node) covers fewer keys, and its mean differs per t.
//
//  * k_block_sums + k_sum_up: fp64 key sums in a hierarchy of factor 64
//    (runs of 64, 4096, ... positions), each key read once.
//  * k_prefix_means: for every height h of the tree and every position t,
//    the mean of the keys from the start of t's height-h node up to t (the
//    open node's summary as position t sees it), summed in fp64 and rounded
//    once to the summary type.  One workgroup per (head, height, block of 64
//    positions), a thread per column: it adds up the node's keys that lie
//    before the block from the hierarchy (at most 63 keys, then at most 2 *
//    63 sums a level), then walks the block in key order.
//  * k_prefill: one workgroup per (batch, query head, position), of one
//    wave when a level has at most 32 candidates (beam * b), 2 waves up to
//    64, 4 up to 128, else 8: a prefill query reads few keys, so small
//    workgroups (LDS sized to them) keep more positions in flight on each CU
//    (measured: 8 waves 1.5-1.8x the rate of 16).  Wave 0 builds the
//    position's level table (depth, existing nodes, first cut, the open
//    rows' offsets) in LDS, a lane per level; the walk reads complete nodes
//    from the cache tree and the open node of each level from the table of
//    partial means.  With leaf blocks of 16 keys or a size that is not a
//    multiple of 16, the same workgroup then attends, stopping at key t;
//    otherwise it only writes the kept leaves, and
//  * k_v_tiles + k_prefill_tiles attend 16 positions of up to 4 query heads
//    at a time on the matrix cores (described below).
#include "attend_query.hpp"
#include "mfma_tile.hpp"
#include "route_walk.hpp"

namespace tis {
namespace {

template <typename T> __device__ inline double elem64(const T *p);
template <> __device__ inline double elem64<float>(const float *p) { return *p; }
template <> __device__ inline double elem64<bf16_bits>(const bf16_bits *p) {
  return __uint_as_float(static_cast<uint32_t>(p->v) << 16);
}

// Level 0 of the hierarchy: the sum of each run of 64 keys, in key order.
template <typename T, int D>
__global__ void __launch_bounds__(D) k_block_sums(PrefillArgs a) {
  const int64_t n0 = a.sum_n[0];
  const int64_t head = blockIdx.x / n0;
  const int64_t i = blockIdx.x - head * n0;
  const int c = threadIdx.x;
  const T *kh = static_cast<const T *>(a.K) + head * a.capacity * D + c;
  const int64_t p0 = i * kPrefixRows;
  const int64_t p1 = min(p0 + kPrefixRows, static_cast<int64_t>(a.positions));
  double acc = 0.0;
  for (int64_t t0 = p0; t0 < p1; t0 += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = t0 + u < p1 ? elem64<T>(kh + (t0 + u) * D) : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  a.sums[a.sum_off[0] + (head * n0 + i) * D + c] = acc;
}

// Level k >= 1: the sum of each run of 64 entries of level k - 1, in order.
template <int D>
__global__ void __launch_bounds__(D) k_sum_up(PrefillArgs a, int k) {
  const int64_t n = a.sum_n[k], nb = a.sum_n[k - 1];
  const int64_t head = blockIdx.x / n;
  const int64_t i = blockIdx.x - head * n;
  const int c = threadIdx.x;
  const double *src = a.sums + a.sum_off[k - 1] + head * nb * D + c;
  const int64_t j0 = i * kPrefixRows;
  const int64_t j1 = min(j0 + kPrefixRows, nb);
  double acc = 0.0;
  for (int64_t j = j0; j < j1; j += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = j + u < j1 ? src[(j + u) * D] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  a.sums[a.sum_off[k] + (head * n + i) * D + c] = acc;
}

template <typename T, int D>
__device__ inline double sum_keys(const T *kh, int64_t x, int64_t y) {
  double acc = 0.0;
  for (int64_t t0 = x; t0 < y; t0 += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = t0 + u < y ? elem64<T>(kh + (t0 + u) * D) : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  return acc;
}

// Entries [x, y) of one level's column (stride D), in order.
template <int D>
__device__ inline double sum_entries(const double *lvl, int64_t x, int64_t y) {
  double acc = 0.0;
  for (int64_t j0 = x; j0 < y; j0 += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = j0 + u < y ? lvl[(j0 + u) * D] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  return acc;
}

template <typename T, typename S, int D>
__global__ void __launch_bounds__(D) k_prefix_means(PrefillArgs a) {
  const int64_t nblk = (a.positions + kPrefixRows - 1) / kPrefixRows;
  const int64_t per_head = a.levels * nblk;
  const int64_t head = blockIdx.x / per_head;
  const int64_t rem = blockIdx.x - head * per_head;
  const int h = static_cast<int>(rem / nblk);
  const int64_t p0 = (rem - h * nblk) * kPrefixRows;
  const int64_t p1 = min(p0 + static_cast<int64_t>(kPrefixRows), static_cast<int64_t>(a.positions));
  const int c = threadIdx.x;
  const uint32_t span = static_cast<uint32_t>(a.h_span[h]);
  const T *kh = static_cast<const T *>(a.K) + head * a.capacity * D + c;
  S *pm = static_cast<S *>(a.open_summ);

  // keys of t's node that come before the block: [s0, p0) = up to 63 keys
  // to the first run boundary, then level by level the runs on both ends of
  // what is left, then the middle at the level where it fits
  const int64_t s0 = (p0 / span) * span;
  double acc = 0.0;
  if (s0 < p0) {
    const int64_t a0 = min((s0 + kPrefixRows - 1) / kPrefixRows * kPrefixRows, p0);
    acc += sum_keys<T, D>(kh, s0, a0);
    int64_t x = a0 / kPrefixRows, y = p0 / kPrefixRows;  // level-0 entries [x, y)
    int k = 0;
    for (; k + 1 < a.sum_levels; ++k) {
      const int64_t xu = (x + kPrefixRows - 1) / kPrefixRows * kPrefixRows;
      const int64_t yd = y / kPrefixRows * kPrefixRows;
      if (xu >= yd) break;  // no whole run of the level above in between
      const double *lvl = a.sums + a.sum_off[k] + head * a.sum_n[k] * D + c;
      acc += sum_entries<D>(lvl, x, xu);
      acc += sum_entries<D>(lvl, yd, y);
      x = xu / kPrefixRows;
      y = yd / kPrefixRows;
    }
    acc += sum_entries<D>(a.sums + a.sum_off[k] + head * a.sum_n[k] * D + c, x, y);
  }
  uint32_t held = static_cast<uint32_t>(p0 - s0);  // keys of the node summed so far
  for (int64_t t0 = p0; t0 < p1; t0 += 8) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = t0 + u < p1 ? elem64<T>(kh + (t0 + u) * D) : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t t = t0 + u;
      if (t < p1) {
        if (held == span) {  // t starts a new node
          acc = 0.0;
          held = 0;
        }
        acc += v[u];
        ++held;
        SummaryType<S>::put(pm + ((head * a.positions + t) * a.levels + h) * D + c,
                            acc / static_cast<double>(held));
      }
    }
  }
}

template <typename T, typename S, int D, int NW, bool ATTEND>
__device__ __forceinline__ void prefill_query(const RouteArgs &ra, const AttendArgs &aa,
                                              const PrefillArgs &pa) {
  __shared__ RouteShared<NW, NW * 32> rsh;
  __shared__ CausalLevels cl;
  const int qi = blockIdx.x;
  const int hrow = qi / pa.positions;          // (batch, query head)
  const int t = qi - hrow * pa.positions;      // position
  const uint4 qraw = attend_q_raw<T, D>(aa, qi);
  if (threadIdx.x < 64) {
    // wave 0 builds the level table, lane j for height j and for level j:
    // every table load at once, then lane exchanges (no serial chain)
    const int lane = threadIdx.x;
    const int bi = hrow / ra.q_heads;
    const int hq = hrow - bi * ra.q_heads;
    const int64_t head = static_cast<int64_t>(bi) * ra.kv_heads + hq / ra.group;
    const uint32_t n = static_cast<uint32_t>(t) + 1u;
    const int levels = pa.levels;
    // a stored height's node span is below 2^31 (it is below the positions)
    const bool hv = lane < levels;
    const uint32_t span = hv ? static_cast<uint32_t>(pa.h_span[lane]) : 0xffffffffu;
    const long long rows = hv ? pa.h_rows[lane] : 0;
    const long long off = hv ? pa.h_off[lane] : 0;
    // depth: the fewest lv >= 1 whose height-lv span covers n (spans grow with h)
    const int lv = 1 + static_cast<int>(__popcll(__ballot(lane >= 1 && hv && span < n)));
    // level l = lane sits at height lv - l
    const bool lev = lane >= 1 && lane <= lv;
    const int h = lev ? lv - lane : 0;
    const uint32_t sp = __shfl(span, h);
    const long long rows_h = __shfl(rows, h);
    const long long off_h = __shfl(off, h);
    const uint32_t ex = lev ? (n + sp - 1u) / sp : 0u;
    // first level below lv with more nodes than the beam, else lv
    const uint64_t cut = __ballot(lev && lane < lv && ex > static_cast<uint32_t>(ra.beam));
    if (lev) {
      cl.exist[lane] = ex;
      cl.rows[lane] = rows_h;
      cl.off[lane] = off_h;
      cl.open_off[lane] = ((head * pa.positions + t) * levels + h) * D;
    }
    if (lane == 0) {
      cl.levels = lv;
      cl.exist[0] = 1;
      cl.exist[lv + 1] = 0;
      cl.first_cut = cut ? __ffsll(static_cast<unsigned long long>(cut)) - 1 : lv;
    }
  }
  __syncthreads();
  const int kept = route_walk<T, S, D, NW, NW, 2, NW * 32>(ra, rsh, qi, &cl, pa.open_summ, hrow);
  if (ra.indices) {
    int32_t *out = ra.indices + static_cast<int64_t>(qi) * ra.beam;
    write_ascending<NW * 64>(rsh.front, kept, out);
    for (int k = kept + static_cast<int>(threadIdx.x); k < ra.beam; k += NW * 64) out[k] = -1;
  }
  if constexpr (ATTEND) {
    __shared__ AttendShared<T, D, NW> ash;
    attend_query<T, D, true, false, true>(aa, ash, qi, qraw, rsh.front, nullptr, kept, false,
                                          nullptr, 0.0, hrow, static_cast<int64_t>(t) + 1);
  }
}

template <typename T, typename S, int D, int NW>
__global__ void __launch_bounds__(NW * 64) k_prefill(RouteArgs ra, AttendArgs aa, PrefillArgs pa) {
  prefill_query<T, S, D, NW, true>(ra, aa, pa);
}

// Routing only (the 16-position attention follows): registers capped for
// 6 waves a SIMD instead of 5, a few spilled (gqa_32k prefill: 2.22 against
// 2.31 ms at 4,096 positions, 47.5 against 48.5 ms at 32,768).
template <typename T, typename S, int D, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(6)))
k_prefill_route(RouteArgs ra, AttendArgs aa, PrefillArgs pa) {
  prefill_query<T, S, D, NW, false>(ra, aa, pa);
}

// ---- block-sparse causal attention on the matrix cores ------------------
// Used when the leaf block is a multiple of 16 keys, after a routing-only
// pass has written every position's kept leaves.  A workgroup takes 16
// consecutive positions of HW query heads that share a KV head (HW = 4, 2
// or 1, dividing the group), a wave per head.  Wave 0 merges the HW * 16
// rows' kept leaves (each list ascending) into one ascending union, each
// leaf with the rows that kept it.  The workgroup then walks the union's
// keys 16 at a time: each key tile of K and of V is loaded once, with
// contiguous 16-byte loads shared by all waves, into LDS (two buffers: the
// next tile loads while this one computes), and every wave reads its
// operands from there:
//   * scores come out transposed, S^T = K Q^T (16 keys x 16 rows, fp32
//     accumulation), so lane l holds row l % 16 and keys 4 (l / 16) + i,
//     i = 0..3, of the key tile: each lane keeps one row's running maximum
//     and a partial sum of that row's weights;
//   * a key counts for a row when the row kept the leaf and the key is not
//     past the row's position;
//   * weights are taken against a reference maximum that moves only when a
//     score passes it by more than 2^8, so the output accumulators are
//     rescaled only then;
//   * the same registers are the A operand of P V (rows x keys), and V is
//     read from a transposed copy, [head][key / 16][d][16], whose 4
//     consecutive keys per lane match the lane's keys.
// bf16 inputs: scores with the 16x16x32 bf16 product, weights split into
// bf16 high and low parts for two 16x16x16 bf16 products with V (fp32
// precision for the weights); fp32 inputs: the 16x16x4 fp32 product for
// both.
// V transposed per tile of 16 keys: vt[head][tile][d][16], zero past the
// positions.  One workgroup of D threads per (head, tile).
template <typename T, int D>
__global__ void __launch_bounds__(D) k_v_tiles(PrefillArgs a) {
  __shared__ T tile[16][D + 1];
  const int64_t tiles = (a.positions + 15) / 16;
  const int64_t head = blockIdx.x / tiles;
  const int64_t tt = blockIdx.x - head * tiles;
  const int c = threadIdx.x;
  const T *vh = static_cast<const T *>(a.V) + head * a.capacity * D;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int64_t key = tt * 16 + k;
    T v{};
    if (key < a.positions) v = vh[key * D + c];
    tile[k][c] = v;
  }
  __syncthreads();
  T *dst = static_cast<T *>(a.vt) + (head * tiles + tt) * D * 16;
  // thread c writes elements c, c + D, ... of the [d][16] block
#pragma unroll
  for (int e = c; e < 16 * D; e += D) dst[e] = tile[e & 15][e >> 4];
}

// Dynamic LDS of k_prefill_tiles, in bytes: the union's length, the rows'
// kept lists (HW * 16 * beam ints), the union (up to HW * 16 * beam leaves,
// each with a 64-bit row mask), then two K tiles (16 rows) and two V tiles
// ([d][16]), rows padded against bank conflicts (K by 16 bytes, V by 4
// elements).
struct TilesLds {
  size_t lists, uni, k, v, total;
  int k_stride;  // bytes per K row in LDS
};
__host__ __device__ inline TilesLds tiles_lds(int hw, int beam, int head_dim, int elem) {
  TilesLds t;
  const size_t rows = static_cast<size_t>(hw) * 16;
  t.lists = 16;
  t.uni = (t.lists + rows * beam * 4 + 15) / 16 * 16;
  t.k = t.uni + rows * beam * 16;
  t.k_stride = head_dim * elem + 16;
  t.v = t.k + 2 * 16 * static_cast<size_t>(t.k_stride);
  t.total = t.v + 2 * static_cast<size_t>(head_dim) * 20 * elem;
  return t;
}
constexpr size_t kTilesMaxLds = 64 * 1024;

struct UnionLeaf {
  int leaf, pad;
  unsigned long long rows;  // bit w * 16 + r: wave w's row r kept the leaf
};

template <typename T, int D, int HW>
__device__ __forceinline__ void prefill_tiles(const AttendArgs &aa, const PrefillArgs &pa) {
  extern __shared__ __align__(16) unsigned char ls_tiles[];
  constexpr int NT = HW * 64;
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int CPR = D * ES / 16;  // 16-byte chunks per K row
  constexpr int VS = TileMath<T, D>::VS;
  const TilesLds lay = tiles_lds(HW, aa.beam, D, ES);
  int *n_union = reinterpret_cast<int *>(ls_tiles);
  int *lists = reinterpret_cast<int *>(ls_tiles + lay.lists);
  UnionLeaf *uni = reinterpret_cast<UnionLeaf *>(ls_tiles + lay.uni);
  unsigned char *ks = ls_tiles + lay.k;
  T *vs = reinterpret_cast<T *>(ls_tiles + lay.v);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int P = pa.positions;
  const int64_t tiles = (P + 15) / 16;
  // workgroups go to the 8 dies in turn: give each die a contiguous run of
  // them, so that the tiles of a KV head meet in one die's L2
  const unsigned bid = (gridDim.x & 7u) == 0u
                           ? (blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3)
                           : blockIdx.x;
  const int64_t hgrp = bid / tiles;  // (batch, group of HW query heads)
  const int t0 = static_cast<int>(bid - hgrp * tiles) * 16;
  const int per_b = aa.q_heads / HW;
  const int bi = static_cast<int>(hgrp / per_b);
  const int hq0 = static_cast<int>(hgrp - static_cast<int64_t>(bi) * per_b) * HW;
  const int64_t head = static_cast<int64_t>(bi) * aa.kv_heads + hq0 / aa.group;
  const int L = aa.leaf_block;
  const int W = aa.beam;
  const int rows = min(16, P - t0);  // rows of this tile that are positions
  const int tmax = t0 + rows - 1;
  // query index of row 0 of wave x: ((bi * Hq + hq0 + x) * P + t0)
  const int64_t qrow0 = (static_cast<int64_t>(bi) * aa.q_heads + hq0) * P + t0;
  const T *kh = static_cast<const T *>(aa.K) + head * aa.key_stride * D;
  const T *vth = static_cast<const T *>(pa.vt) + head * tiles * 16 * D;

  // the rows' kept lists: per head one contiguous block of rows * W
  for (int x = 0; x < HW; ++x) {
    const int32_t *src = aa.indices + (qrow0 + static_cast<int64_t>(x) * P) * W;
    for (int e = tid; e < rows * W; e += NT) lists[x * 16 * W + e] = src[e];
  }
  __syncthreads();
  // wave 0 merges: lane l stands for row l % 16 of wave l / 16
  if (w == 0) {
    const int lr = lane & 15, lw = lane >> 4;
    const bool live = lw < HW && lr < rows;
    const int *mine = lists + (lw * 16 + lr) * W;
    int ptr = 0;
    int nxt = INT_MAX;
    if (live) nxt = mine[0] >= 0 ? mine[0] : INT_MAX;
    int U = 0;
    for (;;) {
      int j = nxt;
      j = min(j, __shfl_xor(j, 1));
      j = min(j, __shfl_xor(j, 2));
      j = min(j, __shfl_xor(j, 4));
      j = min(j, __shfl_xor(j, 8));
      j = min(j, __shfl_xor(j, 16));
      j = min(j, __shfl_xor(j, 32));
      if (j == INT_MAX) break;
      const bool act = nxt == j;
      const unsigned long long m = __ballot(act);
      if (lane == 0) {
        uni[U].leaf = j;
        uni[U].rows = m;
      }
      ++U;
      if (act) {
        ++ptr;
        const int v = ptr < W ? mine[ptr] : -1;
        nxt = v >= 0 ? v : INT_MAX;
      }
    }
    if (lane == 0) *n_union = U;
  }
  __syncthreads();
  const int U = *n_union;

  TileMath<T, D> tm;
  const int tr = t0 + r;  // this lane's row position
  tm.load_q(static_cast<const T *>(aa.Q) + (qrow0 + static_cast<int64_t>(w) * P + r) * D,
            r < rows, g);
  float m = -INFINITY, lsum = 0.f;
  mf_f32x4 o[D / 16];
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) o[nt] = mf_f32x4{0.f, 0.f, 0.f, 0.f};

  // staging of one key tile: K rows kt .. kt + 15 (clamped to the positions)
  // and V's [d][16] block; each thread takes chunks tid, tid + NT, ...  The
  // next tile is in flight in registers while this one computes.  (Tiles
  // further ahead were slower: the compiler then waits for every load in
  // flight before the staging stores into LDS.)
  constexpr int KCH = 16 * CPR;        // 16-byte chunks of a K tile
  constexpr int VCH = 16 * D * ES / 16;  // and of a V tile
  constexpr int KPT = (KCH + NT - 1) / NT;
  constexpr int VPT = (VCH + NT - 1) / NT;
  uint4 kst[KPT], vst[VPT];
  const auto fetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      if (c < KCH) {
        const int row = c / CPR;
        const int64_t key = min(kt + row, P - 1);
        kst[i] = *(reinterpret_cast<const uint4 *>(kh + key * D) + (c - row * CPR));
      }
    }
    const uint4 *vsrc = reinterpret_cast<const uint4 *>(vth + static_cast<int64_t>(kt / 16) * 16 * D);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NT;
      if (c < VCH) vst[i] = vsrc[c];
    }
  };
  const auto stash = [&](int buf) {
    unsigned char *kb = ks + buf * 16 * lay.k_stride;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NT;
      if (c < KCH) {
        const int row = c / CPR;
        *reinterpret_cast<uint4 *>(kb + row * lay.k_stride + (c - row * CPR) * 16) = kst[i];
      }
    }
    // a V row (one dim, 16 keys) is ES chunks; bf16 rows are 40 bytes
    // apart, so their chunks go as two 8-byte halves
    T *vb = vs + buf * D * VS;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NT;
      if (c < VCH) {
        T *dst = vb + (c / ES) * VS + (c % ES) * (16 / ES);
        if constexpr ((VS * ES) % 16 == 0) {
          *reinterpret_cast<uint4 *>(dst) = vst[i];
        } else {
          reinterpret_cast<uint2 *>(dst)[0] = make_uint2(vst[i].x, vst[i].y);
          reinterpret_cast<uint2 *>(dst)[1] = make_uint2(vst[i].z, vst[i].w);
        }
      }
    }
  };

  // key tiles in order: leaf uni[u].leaf, tiles 0, 16, ... of it up to the
  // last row's position
  int u = 0, kt = 0, buf = 0;
  if (U > 0) {
    kt = uni[0].leaf * L;
    fetch(kt);
    stash(0);
  }
  __syncthreads();
  while (u < U) {
    int un = u, ktn = kt + 16;
    if (ktn - uni[u].leaf * L >= L || ktn > tmax) {
      un = u + 1;
      if (un < U) ktn = uni[un].leaf * L;
    }
    if (un < U) fetch(ktn);
    const unsigned wrows = static_cast<unsigned>(uni[u].rows >> (16 * w)) & 0xffffu;
    if (wrows) {
      typename TileMath<T, D>::KReg kr;
      typename TileMath<T, D>::VReg vr;
      TileMath<T, D>::load_k(kr, reinterpret_cast<const T *>(ks + (buf * 16 + r) * lay.k_stride), g);
      TileMath<T, D>::load_v(vr, vs + buf * D * VS, r, g);
      // lane holds S^T[key kt + 4 g + i][row r]
      const mf_f32x4 sc = tm.scores(kr);
      const bool act = (wrows >> r) & 1u;
      const int ahead = tr - kt - 4 * g;  // keys 4 g + i with i <= ahead are not past the row
      float x[4], mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = act && i <= ahead ? sc[i] * aa.scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // the weights are 2^(x - m) for a reference m that moves only when a
      // score passes it by more than 8, so they stay at most 2^8 and the
      // accumulators are rescaled rarely (the normalisation at the end
      // removes m whatever it is)
      const bool move = mx > m + 8.f;
      if (__ballot(move)) {
        const float mnew = move ? mx : m;
        const float alpha = move ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;  // 0 from -inf
        lsum *= alpha;
        m = mnew;
        // output rows 4 g + i take the factor of lane 4 g + i (row 4 g + i)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float ai = __shfl(alpha, 4 * g + i);
#pragma unroll
          for (int nt = 0; nt < D / 16; ++nt) o[nt][i] *= ai;
        }
      }
      // a row with no key yet has m = -inf and only -inf scores
      const float mref = m == -INFINITY ? 0.f : m;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - mref);
      // the normaliser sums the weights as the product used them
      TileMath<T, D>::pv(o, p, vr);
#pragma unroll
      for (int i = 0; i < 4; ++i) lsum += p[i];
    }
    // every wave is done with the other buffer (the barrier before this
    // tile), so the next tile goes there
    if (un < U) stash(buf ^ 1);
    __syncthreads();
    u = un;
    kt = ktn;
    buf ^= 1;
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * g + i;
    const float sc = __shfl(inv, row);
    if (row < rows) {
      float *dst = aa.O + (qrow0 + static_cast<int64_t>(w) * P + row) * D + r;
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) dst[16 * nt] = o[nt][i] * sc;
    }
  }
}

template <typename T, int D, int HW>
__global__ void __launch_bounds__(HW * 64) k_prefill_tiles(AttendArgs aa, PrefillArgs pa) {
  prefill_tiles<T, D, HW>(aa, pa);
}

template <typename T, typename S, int D>
hipError_t launch_prefill_d(const RouteArgs &ra, const AttendArgs &aa, const PrefillArgs &pa,
                            hipStream_t s) {
  const int64_t nblk = (pa.positions + kPrefixRows - 1) / kPrefixRows;
  const dim3 g1(static_cast<unsigned>(pa.heads * pa.levels * nblk));
  const dim3 g2(static_cast<unsigned>(ra.queries));
  hipLaunchKernelGGL((k_block_sums<T, D>), dim3(static_cast<unsigned>(pa.heads * pa.sum_n[0])),
                     dim3(D), 0, s, pa);
  hipError_t e = hipGetLastError();
  for (int k = 1; e == hipSuccess && k < pa.sum_levels; ++k) {
    hipLaunchKernelGGL((k_sum_up<D>), dim3(static_cast<unsigned>(pa.heads * pa.sum_n[k])),
                       dim3(D), 0, s, pa, k);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_prefix_means<T, S, D>), g1, dim3(D), 0, s, pa);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (pa.tiles) {
    // routing only, then the attention of 16 positions at a time
    const int64_t vtiles = (pa.positions + 15) / 16;
    hipLaunchKernelGGL((k_v_tiles<T, D>), dim3(static_cast<unsigned>(pa.heads * vtiles)), dim3(D),
                       0, s, pa);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (ra.beam * ra.branching <= 32)
      hipLaunchKernelGGL((k_prefill_route<T, S, D, 1>), g2, dim3(64), 0, s, ra, aa, pa);
    else if (ra.beam * ra.branching <= 2 * 32)
      hipLaunchKernelGGL((k_prefill_route<T, S, D, 2>), g2, dim3(2 * 64), 0, s, ra, aa, pa);
    else if (ra.beam * ra.branching <= 4 * 32)
      hipLaunchKernelGGL((k_prefill_route<T, S, D, 4>), g2, dim3(4 * 64), 0, s, ra, aa, pa);
    else
      hipLaunchKernelGGL((k_prefill_route<T, S, D, 8>), g2, dim3(8 * 64), 0, s, ra, aa, pa);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t hrows = static_cast<int64_t>(ra.queries) / pa.positions;
    const unsigned grid = static_cast<unsigned>(hrows / pa.tiles * vtiles);
    const size_t lds = tiles_lds(pa.tiles, aa.beam, D, sizeof(T)).total;
    if (pa.tiles == 4)
      hipLaunchKernelGGL((k_prefill_tiles<T, D, 4>), dim3(grid), dim3(4 * 64), lds, s, aa, pa);
    else if (pa.tiles == 2)
      hipLaunchKernelGGL((k_prefill_tiles<T, D, 2>), dim3(grid), dim3(2 * 64), lds, s, aa, pa);
    else
      hipLaunchKernelGGL((k_prefill_tiles<T, D, 1>), dim3(grid), dim3(64), lds, s, aa, pa);
    return hipGetLastError();
  }
  if (ra.beam * ra.branching <= 32)
    hipLaunchKernelGGL((k_prefill<T, S, D, 1>), g2, dim3(64), 0, s, ra, aa, pa);
  else if (ra.beam * ra.branching <= 2 * 32)
    hipLaunchKernelGGL((k_prefill<T, S, D, 2>), g2, dim3(2 * 64), 0, s, ra, aa, pa);
  else if (ra.beam * ra.branching <= 4 * 32)
    hipLaunchKernelGGL((k_prefill<T, S, D, 4>), g2, dim3(4 * 64), 0, s, ra, aa, pa);
  else
    hipLaunchKernelGGL((k_prefill<T, S, D, 8>), g2, dim3(8 * 64), 0, s, ra, aa, pa);
  return hipGetLastError();
}

template <typename T, typename S>
hipError_t launch_prefill_ts(int head_dim, const RouteArgs &ra, const AttendArgs &aa,
                             const PrefillArgs &pa, hipStream_t s) {
  if (head_dim == 128) return launch_prefill_d<T, S, 128>(ra, aa, pa, s);
  if (head_dim == 64) return launch_prefill_d<T, S, 64>(ra, aa, pa, s);
  return hipErrorInvalidValue;
}

}  // namespace

int prefill_tile_heads(int group, int beam, int head_dim, int elem_bytes) {
  for (int hw = 4; hw >= 1; hw /= 2)
    if (group % hw == 0 && tiles_lds(hw, beam, head_dim, elem_bytes).total <= kTilesMaxLds)
      return hw;
  return 0;
}

hipError_t launch_prefill(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra, const AttendArgs &aa,
                          const PrefillArgs &pa, hipStream_t s) {
  if (dt == Dt::BF16)
    return sdt == Dt::BF16 ? launch_prefill_ts<bf16_bits, bf16_bits>(head_dim, ra, aa, pa, s)
                           : launch_prefill_ts<bf16_bits, float>(head_dim, ra, aa, pa, s);
  return sdt == Dt::BF16 ? launch_prefill_ts<float, bf16_bits>(head_dim, ra, aa, pa, s)
                         : launch_prefill_ts<float, float>(head_dim, ra, aa, pa, s);
}

}  // namespace tis
