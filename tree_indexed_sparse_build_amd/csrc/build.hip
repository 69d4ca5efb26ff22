// tree_build: node summaries = mean of the keys under each node, for every
// level ("Subquadratic Attention with a Hierarchical Tree-Structured
// Indexer", Abstract: each node of the index tree holds a compressed summary
// of the cached keys below it, built one level on top of the next).
//
// HBM-bound: K is read exactly once with 16-byte coalesced loads (a wave
// reads whole 1 KB stretches of a leaf block, 16 KB in flight per wave),
// each summary row is written once.  Sums are carried in fp64 in a fixed
// order and rounded once to the summary type (float32 or bfloat16).  A wave
// reduces a subtree of b^kw leaves (a stack of open node sums in registers);
// a workgroup of b^kg waves finishes its chunk's inner levels in LDS.  When
// the chunk roots sit below level 1, their fp64 sums go to the workspace and
// the last chunk of each level-1 subtree to finish climbs the subtree's
// levels above the chunk roots in the same launch (an agent-scope arrival
// count per subtree; the sums travel through device-coherent stores and
// loads, no cache-wide fence).  A level-1 subtree too wide for the
// workgroup's LDS, or more subtrees than the workspace has counters for,
// take one small launch per level instead.  K is read
// exactly once, so its loads carry the streaming (non-temporal) hint:
// measured on MI355X, cold builds run 6-12% faster with it (a K rebuilt back
// to back, partly left in the Infinity Cache by the previous build, runs a
// few percent slower, a regime of repeated benchmarks rather than of use).
// The rows of a workgroup's leaves and wave-level nodes wait in LDS and
// leave in one burst after its last K load (when they fit the budget), so
// the K stream is not broken by a row write every few leaves.
#include "tis_device.hpp"
#include "tis_internal.hpp"

namespace tis {
namespace {

// Mean of a node from its fp64 sum over M keys (rounded once when stored).
// When M is a power of two the product with 1/M is exact, the same value as
// s / M.
__device__ inline double node_mean(const BuildArgs &a, int level, double s) {
  return ((a.pow2_levels >> level) & 1) ? s * a.mean_inv[level] : s / a.mean_div[level];
}

// Transposed reduction of a lane's E column sums over the R = 64 / LPR row
// groups of the wave (lane bits LPR .. 32).  Each step keeps half of the
// remaining columns, so afterwards the lane holds E / R finished columns
// v[0 .. E/R), starting at column rowgroup_offset() of its E-column slice.
template <int E, int LPR, int M, int STEP>
__device__ inline void rowgroup_steps(double (&v)[E], int lane) {
  if constexpr (M >= LPR) {
    constexpr int h = E >> (STEP + 1);
    const bool sel = (lane & M) != 0;
#pragma unroll
    for (int k = 0; k < h; ++k) {
      const double keep = sel ? v[k + h] : v[k];
      const double send = sel ? v[k] : v[k + h];
      v[k] = keep + xor_lane<M>(send, lane);
    }
    rowgroup_steps<E, LPR, M / 2, STEP + 1>(v, lane);
  }
}

template <int E, int LPR> __device__ inline int rowgroup_offset(int lane) {
  int off = 0;
  int h = E / 2;
#pragma unroll
  for (int m = 32; m >= LPR; m >>= 1, h >>= 1) off += (lane & m) ? h : 0;
  return off;
}

// With `through` set (the streaming-load builds of a large K) the summary
// stores carry the device-coherence bit (a relaxed agent-scope atomic store
// is a plain store with that bit): written through rather than left dirty
// in L2.  Measured on MI355X: 1-2% faster on the 0.5-2 GB K builds, 6%
// slower on a K that partly stays in the Infinity Cache, where plain stores
// are used.  Streaming (non-temporal) stores are slower in both cases.
template <int CPL> __device__ inline void store_cols(float *dst, const double *m, bool through) {
  float f[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) f[j] = static_cast<float>(m[j]);
  if (through) {
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      __hip_atomic_store(dst + j, f[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if constexpr (CPL == 2) {
    *reinterpret_cast<float2 *>(dst) = make_float2(f[0], f[1]);
  } else {
    dst[0] = f[0];
  }
}
// bfloat16 summaries: CPL adjacent columns in one 4- or 2-byte store (the
// write-through form only where it is a whole dword)
template <int CPL>
__device__ inline void store_cols(bf16_bits *dst, const double *m, bool through) {
  if constexpr (CPL == 2) {
    const uint32_t v = static_cast<uint32_t>(bf16_from_double(m[0])) |
                       (static_cast<uint32_t>(bf16_from_double(m[1])) << 16);
    uint32_t *p = reinterpret_cast<uint32_t *>(dst);
    if (through)
      __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *p = v;
  } else {
    dst[0].v = bf16_from_double(m[0]);
  }
}

// CPL adjacent finished columns of a row into the LDS staging area.
template <int CPL> __device__ inline void stage_cols(float *dst, const double *m) {
  if constexpr (CPL == 2) {
    *reinterpret_cast<float2 *>(dst) =
        make_float2(static_cast<float>(m[0]), static_cast<float>(m[1]));
  } else {
    dst[0] = static_cast<float>(m[0]);
  }
}
template <int CPL> __device__ inline void stage_cols(bf16_bits *dst, const double *m) {
  if constexpr (CPL == 2) {
    *reinterpret_cast<uint32_t *>(dst) = static_cast<uint32_t>(bf16_from_double(m[0])) |
                                         (static_cast<uint32_t>(bf16_from_double(m[1])) << 16);
  } else {
    dst[0].v = bf16_from_double(m[0]);
  }
}
template <int CPL> __device__ inline void stage_cols(fp8_bits *, const double *) {}

// fp8 rows of nn nodes of level l whose fp64 sums sit in LDS (rows of D),
// the first being node `node0` of the level (head included): one wave a row.
template <int D>
__device__ inline void top_rows_fp8(const BuildArgs &a, fp8_bits *summ, const double *sums,
                                    int nn, int64_t node0, int l) {
  constexpr int C = D / 64;
  const int lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  for (int r = threadIdx.x >> 6; r < nn; r += nw) {
    double m[C];
    int cols[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      cols[j] = lane + 64 * j;
      m[j] = node_mean(a, l, sums[r * D + cols[j]]);
    }
    store_row_fp8<C>(summ + a.summ_off[l] + (node0 + r) * D, a.scales + a.summ_off[l] / D + node0 + r,
                     m, cols, lane);
  }
}

// Levels r-1 .. 1 of the subtree of level-1 node n1 of `head`: the b^(r-2)
// nodes of level r-1 in it sum their children's fp64 sums from the
// workspace (all loads independent; agent-scope loads, since the chunks
// that stored those sums may have run on other XCDs), the levels above are
// summed in LDS (2 b^(r-2) rows of D doubles at `lds`).  Every thread of the
// workgroup takes part.
template <typename S, int D>
__device__ void climb_subtree(const BuildArgs &a, int64_t head, int64_t n1, double *lds) {
  S *const summ = static_cast<S *>(a.summ);
  const int tid = threadIdx.x;
  const int b = a.branching;
  int nn = static_cast<int>(a.top_rows);  // b^(r-2) nodes of level r-1 in the subtree
  int64_t first = n1 * nn;                // their first index within level r-1
  int l = a.root_level - 1;
  double *cur = lds;
  double *nxt = lds + nn * D;
  for (int i = tid; i < nn * D; i += blockDim.x) {
    const int n = i / D;
    const int t = i - n * D;
    const int64_t node = head * a.n_at[l] + first + n;
    const double *child = a.ws_sum + a.ws_off[l + 1] + node * b * D + t;
    // the children's sums, 8 loads in flight at a time, added in child order
    double s = 0.0;
    for (int c0 = 0; c0 < b; c0 += 8) {
      double v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        v[j] = c0 + j < b ? load_coherent(child + static_cast<int64_t>(c0 + j) * D) : 0.0;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (c0 + j < b) s += v[j];
    }
    cur[i] = s;
    if constexpr (!kIsFp8<S>) SummaryType<S>::put(summ + a.summ_off[l] + node * D + t, node_mean(a, l, s));
  }
  __syncthreads();
  if constexpr (kIsFp8<S>) top_rows_fp8<D>(a, summ, cur, nn, head * a.n_at[l] + first, l);
  for (--l; l >= 1; --l) {
    nn /= b;
    first /= b;
    for (int i = tid; i < nn * D; i += blockDim.x) {
      const int n = i / D;
      const int t = i - n * D;
      double s = 0.0;
      for (int c = 0; c < b; ++c) s += cur[(n * b + c) * D + t];
      nxt[i] = s;
      if constexpr (!kIsFp8<S>)
        SummaryType<S>::put(summ + a.summ_off[l] + (head * a.n_at[l] + first + n) * D + t,
                            node_mean(a, l, s));
    }
    __syncthreads();
    if constexpr (kIsFp8<S>) top_rows_fp8<D>(a, summ, nxt, nn, head * a.n_at[l] + first, l);
    double *tmp = cur;
    cur = nxt;
    nxt = tmp;
  }
}

// CLIMB: the last chunk of each level-1 subtree climbs the levels above the
// chunk roots (a compile-time variant, so builds that end at the chunk
// roots run the kernel without that tail)
template <typename T, typename S, int D, bool CLIMB>
__global__ void __launch_bounds__(1024) k_build(BuildArgs a) {
  using G = RowGeom<T, D>;
  constexpr int E = G::kElemsPerLane;
  constexpr int LPR = G::kLanesPerRow;
  constexpr int R = G::kRowsPerInstr;
  constexpr int CPL = E / R;  // finished columns per lane (D / 64)
  constexpr int U = 8;        // 16-byte loads per lane per batch (two batches in flight)
  static_assert(CPL * 64 == D, "one finished column block per lane");
  extern __shared__ double lds[];
  S *const summ = static_cast<S *>(a.summ);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int nw = blockDim.x >> 6;
  const int b = a.branching;
  const int L = a.leaf_block;
  const int lv = a.levels;
  const int kw = a.wave_depth;
  const int64_t head = blockIdx.x / a.chunks;
  const int64_t chunk = blockIdx.x - head * a.chunks;
  const int col = (lane % LPR) * E;
  const int colf = col + rowgroup_offset<E, LPR>(lane);  // this lane's finished columns
  const int rsub = lane / LPR;
  const T *kh = static_cast<const T *>(a.K) + head * a.n_keys * D + col;
  // Staged rows (a.stage, float32 / bfloat16 summaries): the rows of the
  // leaves and register-stack levels of this workgroup's chunk are kept in
  // LDS after the fp64 rows of the inner levels, one block per level (leaves
  // first, then each level up: nw * b^(kw - j) rows for level lv - j), and
  // written out after the last K load, so the K stream is not interrupted by
  // scattered row writes.
  S *const stage = reinterpret_cast<S *>(lds + 2 * nw * D);

  // ---- this wave: the subtree of b^kw leaves under one node of level lv-kw
  const int64_t wnode = chunk * nw + w;
  const int64_t leaf0 = wnode * a.wave_leaves;
  double st[kMaxWaveDepth][CPL];  // running sums of the open node at level lv-k
  int ctr[kMaxWaveDepth];
  int64_t nid[kMaxWaveDepth];     // index of that node within its level
  double root[CPL];
#pragma unroll
  for (int k = 0; k < kMaxWaveDepth; ++k) {
    ctr[k] = 0;
    nid[k] = wnode;
#pragma unroll
    for (int j = 0; j < CPL; ++j) st[k][j] = 0.0;
  }
  for (int k = kMaxWaveDepth - 1; k >= 0; --k) {
    // node of level lv-k-1 that holds the first leaf: wnode * b^(kw-k-1)
    if (k < kw) {
      int64_t n = wnode;
      for (int j = k + 1; j < kw; ++j) n *= b;
      nid[k] = n;
    }
  }
  // staged block of level lv - j (j = 0: the leaves): b^(kw - j) rows per
  // wave, nw * b^(kw - j) in all, blocks in order of j
  auto stage_per = [&](int j) {
    int per = 1;
    for (int i = j; i < kw; ++i) per *= b;
    return per;
  };
  auto stage_base = [&](int j) {
    int rows = 0;
    for (int i = 0; i < j; ++i) rows += stage_per(i) * nw;
    return rows;
  };
  // The wave's leaves are streamed as one sequence of batches of U*R rows
  // (nb batches per leaf).  Loads are double-buffered: the next batch is in
  // flight while the current one is added up and, at a leaf's end, reduced.
  const int nb = (L + U * R - 1) / (U * R);
  int64_t lc = 0;  // leaf / batch of the next load
  int lb = 0;
  int64_t cc = 0;  // leaf / batch being added up
  int cb = 0;
  auto issue = [&](uint4 (&v)[U]) {
    const T *kl = kh + (leaf0 + lc) * static_cast<int64_t>(L) * D;
    const int r0 = lb * U * R;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // rows past the leaf load its last row again (added as zero): every
      // load is issued unconditionally, so the wait before a batch is used
      // counts only the loads issued before it
      const int row = min(r0 + u * R + rsub, L - 1);
      v[u] = load16_stream(kl + static_cast<int64_t>(row) * D);
    }
    if (++lb == nb) {
      lb = 0;
      ++lc;
    }
  };
  double acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0;
  const bool ragged = L % (U * R) != 0;
  auto consume = [&](const uint4 (&v)[U]) {
    const int rc = cb * U * R + rsub;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float f[E];
      Vec16<T>::unpack(v[u], f);
      if (ragged && rc + u * R >= L) {
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] = 0.0f;
      }
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += static_cast<double>(f[e]);
    }
    if (++cb < nb) return;
    // ---- leaf cc complete
    cb = 0;
    const int64_t leaf = leaf0 + cc;
    ++cc;
    rowgroup_steps<E, LPR, 32, 0>(acc, lane);
    {
      double m[CPL];
#pragma unroll
      for (int j = 0; j < CPL; ++j) m[j] = node_mean(a, lv, acc[j]);
      const int64_t node = head * a.n_at[lv] + leaf;
      if constexpr (kIsFp8<S>) {
        int cols[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) cols[j] = colf + j;
        store_row_fp8<CPL>(summ + a.summ_off[lv] + node * D, a.scales + a.summ_off[lv] / D + node,
                           m, cols, lane);
      } else if (a.stage) {
        stage_cols<CPL>(stage + (w * a.wave_leaves + (cc - 1)) * D + colf, m);  // leaf cc - 1
      } else {
        store_cols<CPL>(summ + a.summ_off[lv] + node * D + colf, m, a.through_stores != 0);
      }
    }
    double carry[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) carry[j] = root[j] = acc[j];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    // close every level whose node this leaf completes
#pragma unroll
    for (int k = 0; k < kMaxWaveDepth; ++k) {
      if (k >= kw) break;
#pragma unroll
      for (int j = 0; j < CPL; ++j) st[k][j] += carry[j];
      if (++ctr[k] < b) break;
      const int lvl = lv - k - 1;
      if (lvl >= 1) {
        double m[CPL];
#pragma unroll
        for (int j = 0; j < CPL; ++j) m[j] = node_mean(a, lvl, st[k][j]);
        const int64_t node = head * a.n_at[lvl] + nid[k];
        if constexpr (kIsFp8<S>) {
          int cols[CPL];
#pragma unroll
          for (int j = 0; j < CPL; ++j) cols[j] = colf + j;
          store_row_fp8<CPL>(summ + a.summ_off[lvl] + node * D,
                             a.scales + a.summ_off[lvl] / D + node, m, cols, lane);
        } else if (a.stage) {
          // level lv - (k + 1): the wave's b^(kw-k-1) nodes, the first being
          // wnode * b^(kw-k-1)
          const int per = stage_per(k + 1);
          const int row = stage_base(k + 1) + w * per + static_cast<int>(nid[k] - wnode * per);
          stage_cols<CPL>(stage + static_cast<int64_t>(row) * D + colf, m);
        } else {
          store_cols<CPL>(summ + a.summ_off[lvl] + node * D + colf, m, a.through_stores != 0);
        }
      }
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        carry[j] = root[j] = st[k][j];
        st[k][j] = 0.0;
      }
      ctr[k] = 0;
      ++nid[k];
    }
  };
  // The steady-state loop issues both buffers unconditionally, so the
  // compiler's wait before a batch is used leaves the other batch's loads in
  // flight (a load issued under a condition makes it wait for every load).
  uint4 va[U], vb[U];
  issue(va);
  int64_t left = a.wave_leaves * nb - 1;  // batches still to issue
  while (left >= 2) {
    issue(vb);
    consume(va);
    issue(va);
    consume(vb);
    left -= 2;
  }
  if (left == 1) {
    issue(vb);
    consume(va);
    consume(vb);
  } else {
    consume(va);
  }

  // ---- the workgroup's inner levels, from the waves' fp64 root sums in LDS
  int lvl = lv - kw;  // level of the wave's root
  double *cur = lds;
  double *nxt = lds + nw * D;
#pragma unroll
  for (int j = 0; j < CPL; ++j) cur[w * D + colf + j] = root[j];
  __syncthreads();
  if constexpr (!kIsFp8<S>) {
    if (a.stage) {
      // the staged blocks, each a contiguous run of rows of its level, in
      // 16-byte stores with the non-temporal hint (measured on MI355X: a
      // cold build and decode step of the 32K-key GQA workload 65.2 -> 63.8
      // us, builds of 256K to 1M keys 1-2.5% faster; the same hint on the
      // inner levels' and the climb's stores made the build alone faster
      // but the decode after it slower by as much)
      for (int j = 0; j <= kw; ++j) {
        const int l = lv - j;
        if (l < 1) break;
        const int64_t rows = static_cast<int64_t>(stage_per(j)) * nw;
        const int64_t first = head * a.n_at[l] + chunk * rows;
        const uint4 *src =
            reinterpret_cast<const uint4 *>(stage + static_cast<int64_t>(stage_base(j)) * D);
        uint4 *dst = reinterpret_cast<uint4 *>(summ + a.summ_off[l] + first * D);
        const int64_t n16 = rows * D * static_cast<int64_t>(sizeof(S)) / 16;
        for (int64_t i = tid; i < n16; i += blockDim.x) {
          const uint4 v = src[i];
          __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w},
                                      reinterpret_cast<u32x4_t *>(dst + i));
        }
      }
    }
  }
  int64_t base = chunk * nw;  // index of cur[0]'s node within its level
  for (int ncur = nw; ncur > 1; ncur /= b) {
    const int nn = ncur / b;
    --lvl;
    base /= b;
    for (int i = tid; i < nn * D; i += blockDim.x) {
      const int n = i / D;
      const int dd = i % D;
      double s = 0.0;
      for (int c = 0; c < b; ++c) s += cur[(n * b + c) * D + dd];
      nxt[n * D + dd] = s;
      if constexpr (!kIsFp8<S>) {
        if (lvl >= 1)
          SummaryType<S>::put(summ + a.summ_off[lvl] + (head * a.n_at[lvl] + base + n) * D + dd,
                              node_mean(a, lvl, s));
      }
    }
    __syncthreads();
    if constexpr (kIsFp8<S>) {
      // fp8 rows need their whole row's largest magnitude: one wave a row
      if (lvl >= 1) {
        for (int r = w; r < nn; r += nw) {
          double m[CPL];
          int cols[CPL];
#pragma unroll
          for (int j = 0; j < CPL; ++j) {
            cols[j] = lane + 64 * j;
            m[j] = node_mean(a, lvl, nxt[r * D + cols[j]]);
          }
          const int64_t node = head * a.n_at[lvl] + base + r;
          store_row_fp8<CPL>(summ + a.summ_off[lvl] + node * D,
                             a.scales + a.summ_off[lvl] / D + node, m, cols, lane);
        }
      }
    }
    double *t = cur;
    cur = nxt;
    nxt = t;
  }

  // ---- the chunk root: its fp64 sum feeds the levels above
  if (lvl >= 2) {
    double *mine = a.ws_sum + a.ws_off[lvl] + (head * a.n_at[lvl] + base) * D;
    for (int i = tid; i < D; i += blockDim.x) store_coherent(mine + i, cur[i]);
    if constexpr (CLIMB) {
      // the last chunk of its level-1 subtree to get here climbs the
      // subtree's levels r-1 .. 1 and sets the subtree's counter back to
      // zero; the others are done
      __shared__ int s_last;
      if (tid < D) wait_vector_memory();  // the threads that stored the root's sums
      __syncthreads();
      const int64_t n1 = chunk / a.chunks_per_l1;
      unsigned *cnt = a.arrive + head * b + n1;
      if (tid == 0) {
        const unsigned before = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
        s_last = before == static_cast<unsigned>(a.chunks_per_l1 - 1);
      }
      __syncthreads();
      if (s_last) {
        if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        climb_subtree<S, D>(a, head, n1, lds);  // the LDS rows of this chunk are no longer read
      }
    }
  }
}

// One level l above the chunk roots: node sum = sum of its b children's fp64
// sums (level l+1), one thread per (node, column), every load independent.
// Launched once per level, from r-1 down to 1; the kernel boundary between
// levels orders the writes of one level before the reads of the next.
template <typename S, int D>
__global__ void __launch_bounds__(256) k_build_level(BuildArgs a, int l) {
  const int64_t item = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nodes = a.chunks_at_level[l];  // B*Hkv*n_l
  if (item >= nodes * D) return;
  const int64_t node = item / D;  // (head, node) flattened: head * n_l + n
  const int t = static_cast<int>(item - node * D);
  const int b = a.branching;
  const double *child = a.ws_sum + a.ws_off[l + 1] + node * b * D + t;
  // 8 loads in flight at a time, added in child order
  double s = 0.0;
  for (int c0 = 0; c0 < b; c0 += 8) {
    double v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = c0 + j < b ? child[static_cast<int64_t>(c0 + j) * D] : 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (c0 + j < b) s += v[j];
  }
  SummaryType<S>::put(static_cast<S *>(a.summ) + a.summ_off[l] + node * D + t, node_mean(a, l, s));
  if (l >= 2) a.ws_sum[a.ws_off[l] + node * D + t] = s;
}

// k_build_level for fp8 summaries: one wave per node row (the row's scale
// needs its largest magnitude), 4 rows per workgroup.
template <int D> __global__ void __launch_bounds__(256) k_build_level_fp8(BuildArgs a, int l) {
  constexpr int C = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t node = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (node >= a.chunks_at_level[l]) return;  // whole wave
  const int b = a.branching;
  double m[C];
  int cols[C];
#pragma unroll
  for (int j = 0; j < C; ++j) {
    const int t = lane + 64 * j;
    const double *child = a.ws_sum + a.ws_off[l + 1] + node * b * D + t;
    double s = 0.0;
    for (int c = 0; c < b; ++c) s += child[static_cast<int64_t>(c) * D];
    if (l >= 2) a.ws_sum[a.ws_off[l] + node * D + t] = s;
    cols[j] = t;
    m[j] = node_mean(a, l, s);
  }
  store_row_fp8<C>(static_cast<fp8_bits *>(a.summ) + a.summ_off[l] + node * D,
                   a.scales + a.summ_off[l] / D + node, m, cols, lane);
}

}  // namespace

// Rows of a workgroup's leaves and register-stack levels: nw waves with
// b^kw leaves each, and every level up to the wave roots.
int64_t stage_rows(int64_t nw, int64_t branching, int kw) {
  int64_t rows = 0, per = 1;
  for (int j = 0; j <= kw; ++j, per *= branching) rows += per * nw;
  return rows;
}

bool plan_build(int64_t heads, int head_dim, int branching, int leaf_block, int levels,
                BuildPlan *p) {
  // Choose the wave subtree depth kw (b^kw leaves per wave) and the
  // workgroup depth kg (b^kg <= 16 waves), by tiers measured on MI355X
  // (every plan gives the same summaries, bit for bit): (0) a plan that
  // needs no level above the chunk roots (r <= 1) and has >= 2048 waves;
  // (1) a plan whose waves all run at once (2048 to 4096 waves: the kernel
  // keeps 16 waves a CU on 256 CUs) in >= 512 workgroups, each wave
  // streaming at most 1,024 keys (measured on 262,144-key heads with
  // b = 4: 7% faster than the 8,192 waves of tier 2, run in two rounds);
  // (2) plans with >= 4096 waves and >= 512 workgroups (enough loads in
  // flight on 256 CUs), fewest levels left first; (3) otherwise the most
  // waves.  Within a tier, plans whose wave-level rows fit the LDS staging
  // budget (as float32 rows, so the plan is the same for every summary
  // type) come first: writing those rows in one burst after the last K
  // load, instead of one row at a time between loads, measured 4-10% faster
  // on cold builds.  Ties go to bigger workgroups.
  constexpr int64_t kOneRoundWaves = 256 * 16;
  struct Cand { int kw, kg, r; int64_t waves, wgs; bool stage; int64_t wave_keys; };
  auto ipow = [](int64_t x, int e) {
    int64_t v = 1;
    for (int i = 0; i < e; ++i) v *= x;
    return v;
  };
  auto tier = [](const Cand &c) {
    if (c.r <= 1 && c.waves >= 2048) return 0;
    if (c.waves >= 2048 && c.waves <= kOneRoundWaves && c.wgs >= 512 && c.wave_keys <= 1024)
      return 1;
    if (c.waves >= 4096 && c.wgs >= 512) return 2;
    return 3;
  };
  auto better = [&](const Cand &c, const Cand &o) {
    const int tc = tier(c), to = tier(o);
    if (tc != to) return tc < to;
    if (c.stage != o.stage) return c.stage;
    if (tc == 0) return c.waves > o.waves || (c.waves == o.waves && c.kg > o.kg);
    if (tc == 1 || tc == 2) return c.r < o.r || (c.r == o.r && c.kg > o.kg);
    return c.waves > o.waves || (c.waves == o.waves && c.r < o.r);
  };
  bool have = false;
  Cand best{};
  for (int kw = 0; kw <= kMaxWaveDepth && kw <= levels; ++kw) {
    for (int kg = 0; kw + kg <= levels; ++kg) {
      const int64_t nw = ipow(branching, kg);
      if (nw > 16) break;
      const int r = levels - kw - kg;
      const bool stage = stage_rows(nw, branching, kw) * head_dim * sizeof(float) <= kStageLdsBytes;
      const Cand c{kw, kg, r, heads * ipow(branching, levels - kw), heads * ipow(branching, r),
                   stage, ipow(branching, kw) * leaf_block};
      if (c.wgs > 0x7fffffffLL) continue;
      if (!have || better(c, best)) best = c;
      have = true;
    }
  }
  if (!have) return false;
  const int64_t nw = ipow(branching, best.kg);
  p->wave_depth = best.kw;
  p->root_level = best.r;
  p->waves = static_cast<int>(nw);
  p->chunks = ipow(branching, best.r);
  p->lds_bytes = static_cast<size_t>(2 * nw * head_dim) * sizeof(double);
  size_t sum = 0;
  int64_t n = 1;
  for (int l = 1; l <= best.r; ++l) {
    n *= branching;
    if (l >= 2) sum += static_cast<size_t>(heads * n) * head_dim;
  }
  p->sum_elems = sum;
  p->workspace_bytes = sum > 0 ? kBuildArriveBytes + sum * sizeof(double) : 0;
  return true;
}

namespace {

// Launches of one (input type, summary type, head dim).
template <typename T, typename S, int D>
hipError_t launch_build_t(int64_t heads, const BuildArgs &args, const BuildPlan &p,
                          hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(heads * p.chunks));
  const dim3 block(static_cast<unsigned>(p.waves * 64));
  BuildArgs a = args;
  size_t lds = p.lds_bytes;
  // stage the wave-level rows when they fit the budget (not fp8 rows, whose
  // scale needs the whole row)
  const size_t stage_bytes =
      static_cast<size_t>(stage_rows(p.waves, a.branching, p.wave_depth)) * D * sizeof(S);
  a.stage = !kIsFp8<S> && stage_bytes <= kStageLdsBytes;
  if (a.stage) lds += stage_bytes;
  // chunk roots at level 2 or below: the last chunk of each level-1 subtree
  // climbs it in the same launch when its rows fit the LDS the kernel already
  // has (2 b^(r-2) <= 2 nw rows) and the counters fit the workspace's
  a.fuse_top = p.root_level >= 2 && a.top_rows <= p.waves &&
               heads * a.branching <= kBuildArriveMax;
  if (a.fuse_top)
    hipLaunchKernelGGL((k_build<T, S, D, true>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((k_build<T, S, D, false>), grid, block, lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.root_level < 2 || a.fuse_top) return e;
  // otherwise one small launch per level above the chunk roots
  for (int l = p.root_level - 1; e == hipSuccess && l >= 1; --l) {
    if constexpr (kIsFp8<S>) {
      const dim3 g(static_cast<unsigned>((a.chunks_at_level[l] + 3) / 4));
      hipLaunchKernelGGL((k_build_level_fp8<D>), g, dim3(256), 0, s, a, l);
    } else {
      const int64_t items = a.chunks_at_level[l] * D;
      const dim3 g(static_cast<unsigned>((items + 255) / 256));
      hipLaunchKernelGGL((k_build_level<S, D>), g, dim3(256), 0, s, a, l);
    }
    e = hipGetLastError();
  }
  return e;
}

template <typename T, typename S>
hipError_t launch_build_ts(int head_dim, int64_t heads, const BuildArgs &a, const BuildPlan &p,
                           hipStream_t s) {
  if (head_dim == 128) return launch_build_t<T, S, 128>(heads, a, p, s);
  if (head_dim == 64) return launch_build_t<T, S, 64>(heads, a, p, s);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_build(Dt dt, Dt sdt, int head_dim, int64_t heads, const BuildArgs &a,
                        const BuildPlan &p, hipStream_t s) {
  if (dt == Dt::BF16) {
    if (sdt == Dt::FP8) return launch_build_ts<bf16_bits, fp8_bits>(head_dim, heads, a, p, s);
    return sdt == Dt::BF16 ? launch_build_ts<bf16_bits, bf16_bits>(head_dim, heads, a, p, s)
                           : launch_build_ts<bf16_bits, float>(head_dim, heads, a, p, s);
  }
  if (sdt == Dt::FP8) return launch_build_ts<float, fp8_bits>(head_dim, heads, a, p, s);
  return sdt == Dt::BF16 ? launch_build_ts<float, bf16_bits>(head_dim, heads, a, p, s)
                         : launch_build_ts<float, float>(head_dim, heads, a, p, s);
}

}  // namespace tis
