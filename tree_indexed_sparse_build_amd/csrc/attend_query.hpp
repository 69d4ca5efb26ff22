// Exact softmax attention of one query over a set of leaf blocks, as a
// device function shared by the attend kernel and the fused decode kernel
// ("Subquadratic Attention with a Hierarchical Tree-Structured Indexer",
// Abstract: the attention over the keys a query ends with; the NSA /
// InfLLMv2 abstract on the Progressive Sparse Attention related-papers page:
// exact softmax restricted to the tokens of the chosen blocks).
//
// Gather flash-decode inside one workgroup.  The query's work is cut into
// units of RB rows of one leaf block; each wave takes units in turn, issues
// the unit's K and V loads together (16 bytes per lane, whole 256-byte rows
// per lane group), and keeps an online softmax (m, l, acc) in fp32.  The
// waves' partials meet in LDS and are merged by log-sum-exp.
#pragma once

#include "tis_device.hpp"
#include "tis_internal.hpp"

namespace tis {

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

constexpr int kPartHeader = 4;  // m, l, two pad words: keeps acc 16-byte aligned

// fp32 dot product of the 8 bf16 values of a and of b (16 bytes each, pairs
// in dwords): four dot2 instructions, each adding two bf16 x bf16 products
// (exact in fp32) to the running fp32 sum, with no unpacking of the operands.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline float dot8_bf16(uint4 a, uint4 b) {
  float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x),
                                            __builtin_bit_cast(bf16x2_t, b.x), 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y),
                                      __builtin_bit_cast(bf16x2_t, b.y), s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z),
                                      __builtin_bit_cast(bf16x2_t, b.z), s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w),
                                         __builtin_bit_cast(bf16x2_t, b.w), s, false);
}

// MW: the most waves of the workgroups that use it
template <typename T, int D, int MW = kAttendMaxWaves> struct AttendShared {
  float p[MW][AttendGeom<T, D>::RB];
  float m[MW], l[MW];
  float acc[MW][D];
};

// Element offset, in K and in V, of row 0 of the KV head that query row hr
// reads (the lane's columns are added where it is used).
template <int D> __device__ inline int64_t head_offset(const AttendArgs &a, int hr) {
  const int bi = div_u(hr, a.q_heads);
  const int hq = hr - bi * a.q_heads;
  const int64_t head = static_cast<int64_t>(bi) * a.kv_heads + div_u(hq, a.group);
  return head * a.key_stride * D;
}

// head_offset computed where the caller stands, held there: the empty asm
// takes it as an opaque value, so the compiler cannot move its scalar
// arithmetic (and its argument loads) down to where it is used.  The fused
// decode computes it before its walk, in the shadow of the first level's
// loads, instead of after it, where all 16 waves of the workgroup would
// queue on the CU's one scalar unit for it at once.  Only the offset is held
// opaque: the K and V pointers still come from the kernel's arguments, so
// the compiler keeps the gather's loads global rather than generic (flat)
// ones, which would also count against the LDS wait counter.
template <int D> __device__ inline int64_t head_offset_early(const AttendArgs &a, int hr) {
  int64_t off = head_offset<D>(a, hr);
  asm volatile("" : "+s"(off));
  return off;
}

// This lane's part of the query row in the attend layout (E elements).
template <typename T, int D> __device__ inline uint4 attend_q_raw(const AttendArgs &a, int qi) {
  constexpr int LPR = AttendGeom<T, D>::LPR, E = AttendGeom<T, D>::E;
  const int lane = threadIdx.x & 63;
  return load16(static_cast<const T *>(a.Q) + static_cast<int64_t>(qi) * D + (lane % LPR) * E);
}

// Attention of query qi over the leaf blocks slots[s] (s < nslots) whose
// use[s] is nonzero (use == nullptr: all), every wave of the workgroup
// taking part (RAGGED: the last block of a growing cache may hold fewer
// than L keys; THRESH: only keys whose score q.k, computed in fp64, is at
// least tau take part, and that fp64 score is also the one the softmax
// uses; PREFILL: the query is position t of a causal prefill, its (batch,
// head) row is hrow and its keys end at nk = t + 1).  With part == nullptr
// it writes row qi of O (NaN if `bad`,
// zero if no slot is used); otherwise it writes the workgroup's partial
// softmax state to part: m (log2 units), l (NaN if `bad`), two pad words,
// acc[D], for a later log-sum-exp merge with the query's other parts.
template <typename T, int D, bool RAGGED = false, bool THRESH = false, bool PREFILL = false,
          int MW = kAttendMaxWaves>
__device__ void attend_query(const AttendArgs &a, AttendShared<T, D, MW> &sh, int qi,
                             uint4 qraw, const int *slots, const int *use, int nslots,
                             bool bad, float *part, double tau = 0.0, int hrow = 0,
                             int64_t nk = 0, unsigned long long *tl = nullptr,
                             const int64_t *pre_off = nullptr) {
  using AG = AttendGeom<T, D>;
  constexpr int E = AG::E, LPR = AG::LPR, R = AG::R, U = AG::U, RB = AG::RB, REP = AG::REP;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int L = a.leaf_block;
  const int hr = PREFILL ? hrow : qi;
  const int64_t hoff = pre_off ? *pre_off : head_offset<D>(a, hr);
  const int col = (lane % LPR) * E;
  const int rsub = lane / LPR;
  const int64_t n_keys = PREFILL ? nk : a.n_keys;

  float q[E];
  Vec16<T>::unpack(qraw, q);
  const T *kh = static_cast<const T *>(a.K) + hoff + col;
  const T *vh = static_cast<const T *>(a.V) + hoff + col;
  const int nc = (L + RB - 1) / RB;
  const int units = nslots * nc;

  float m = -INFINITY, l = 0.f;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;

  for (int u = w; u < units; u += nw) {
    const int s = div_u(u, nc);
    if (use && !use[s]) continue;
    const int r0 = (u - s * nc) * RB;
    const int64_t blk0 = static_cast<int64_t>(slots[s]) * L;
    const int64_t rowb = blk0 + r0;
    // keys of the block in use: L, or fewer in the last block of a cache
    const int len = RAGGED ? static_cast<int>(min(static_cast<int64_t>(L), n_keys - blk0)) : L;
    if (RAGGED && r0 >= len) continue;
    uint4 kv[U], vv[U];
    if (u == w) tl_stamp(tl, 2);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int row = r0 + i * R + rsub;
      kv[i] = row < len ? load16(kh + (rowb + i * R + rsub) * D) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int row = r0 + i * R + rsub;
      vv[i] = row < len ? load16(vh + (rowb + i * R + rsub) * D) : make_uint4(0u, 0u, 0u, 0u);
    }
    float sc;
    bool pass = true;
    if constexpr (THRESH) {
      // fp32 x fp32 (or bf16) products are exact in fp64
      double part[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        float k[E];
        Vec16<T>::unpack(kv[i], k);
        double dot = 0.0;
#pragma unroll
        for (int e = 0; e < E; ++e)
          dot = fma(static_cast<double>(q[e]), static_cast<double>(k[e]), dot);
        part[i] = dot;
      }
      const double s64 = group_transpose_reduce<U, LPR>(part, lane);
      pass = s64 >= tau;
      sc = static_cast<float>(s64);
    } else {
      float part[U];
#pragma unroll
      for (int i = 0; i < U; ++i) {
        if constexpr (__is_same(T, bf16_bits)) {
          // bf16 keys and query: the pairs as stored, into gfx950's dot2
          part[i] = dot8_bf16(kv[i], qraw);
        } else {
          float k[E];
          Vec16<T>::unpack(kv[i], k);
          float dot = 0.f;
#pragma unroll
          for (int e = 0; e < E; ++e) dot = fmaf(q[e], k[e], dot);
          part[i] = dot;
        }
      }
      sc = group_transpose_reduce<U, LPR>(part, lane);
    }
    if (u == w) {
      tl_after(tl, sc);
      tl_stamp(tl, 3);
    }
    // lane holds the score of row r0 + kk * R + rsub
    const int kk = (lane % LPR) / REP;
    const bool valid = r0 + kk * R + rsub < len && pass;
    const float x = valid ? sc * a.scale_log2 : -INFINITY;
    const float mnew = fmaxf(m, wave_max(x));
    // hardware 2^x: results below 2^-126 flush to zero, which leaves the
    // weights of everything that contributes at fp32 precision unchanged
    const float p = valid ? __builtin_amdgcn_exp2f(x - mnew) : 0.f;
    // (a threshold can mask every row seen so far: m = mnew = -inf, no rescale)
    const float alpha =
        THRESH && mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
    l = l * alpha + wave_sum((lane % REP) == 0 ? p : 0.f);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] *= alpha;
    m = mnew;
    // hand the probabilities to the lanes holding the matching V rows
    if ((lane % REP) == 0) sh.p[w][rsub * U + kk] = p;
    __builtin_amdgcn_wave_barrier();
    float pr[U];
#pragma unroll
    for (int i = 0; i < U; ++i) pr[i] = sh.p[w][rsub * U + i];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float v[E];
      Vec16<T>::unpack(vv[i], v);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(pr[i], v[e], acc[e]);
    }
    if (u == w) {
      tl_after(tl, acc[0]);
      tl_stamp(tl, 4);
    }
  }
  tl_after(tl, acc[0]);
  tl_stamp(tl, 5);
  // rows were spread over the R lane groups of the wave
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = group_sum<LPR, 32>(acc[e], lane);
  if (lane < LPR) {
#pragma unroll
    for (int e = 0; e < E; ++e) sh.acc[w][col + e] = acc[e];
  }
  if (lane == 0) {
    sh.m[w] = m;
    sh.l[w] = l;
  }
  __syncthreads();
  tl_stamp(tl, 6);

  // ---- log-sum-exp merge of the waves' partials, one column per thread.
  // Every read has a compile-time offset and all are issued before the
  // first is used; slots of waves past nw are never written and are masked
  // (m = -inf, l = acc = 0).
  for (int c = tid; c < D; c += blockDim.x) {
    float mj[MW], lj[MW], aj[MW];
#pragma unroll
    for (int j = 0; j < MW; ++j) {
      mj[j] = sh.m[j];
      lj[j] = sh.l[j];
      aj[j] = sh.acc[j][c];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < MW; ++j) {
      if (j >= nw) {
        mj[j] = -INFINITY;
        lj[j] = 0.f;
        aj[j] = 0.f;
      }
      mx = fmaxf(mx, mj[j]);
    }
    float num = 0.f, den = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int j = 0; j < MW; ++j) {
        const float wj = __builtin_amdgcn_exp2f(mj[j] - mx);  // 0 for waves that saw no key
        den = fmaf(wj, lj[j], den);
        num = fmaf(wj, aj[j], num);
      }
    }
    if (part) {
      // device-coherent stores: the part that merges may run on another XCD
      store_coherent(part + kPartHeader + c, num);
      if (c == 0) {
        store_coherent(part, mx);
        store_coherent(part + 1, bad ? NAN : den);
      }
    } else {
      float r = mx == -INFINITY ? 0.f : num / den;
      if (bad) r = NAN;
      a.O[static_cast<int64_t>(qi) * D + c] = r;
    }
  }
}

// The end of a split query's part, run by every thread of the part's
// workgroup after attend_query has written the part's state: the part that
// arrives last merges the query's `splits` states into row qi of O,
// o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s with M = max_s m_s
// (zero if no part saw a key, NaN if any part is NaN), and sets the query's
// arrival counter back to zero for the next call.
//
// The states travel through device-coherent (agent-scope) stores and loads,
// which bypass the XCDs' private L2 state, so no L2 write-back or invalidate
// is needed (a release fence at agent scope would write back the whole L2;
// measured, that costs more than the split saves).  What orders a part's
// stores before its arrival is the wait for their completion before the
// barrier; the counter is an agent-scope atomic, and the last arriver's
// loads are issued only after it has seen the count.  The merge issues the
// loads of up to 8 parts at once: one memory round trip per 8 parts.
template <int D> __device__ void merge_parts(const AttendArgs &a, int qi) {
  constexpr int PB = 8;  // parts whose loads are in flight together
  __shared__ int s_last;
  const int tid = threadIdx.x;
  if (tid < D) wait_vector_memory();  // the threads that stored the state
  __syncthreads();
  if (tid == 0) {
    const unsigned before = __hip_atomic_fetch_add(a.arrive + qi, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    s_last = before == static_cast<unsigned>(a.splits - 1);
  }
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) __hip_atomic_store(a.arrive + qi, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float *pq = a.part + static_cast<int64_t>(qi) * a.splits * (D + kPartHeader);
  for (int c = tid; c < D; c += blockDim.x) {
    float M = -INFINITY, num = 0.f, den = 0.f;
    bool bad = false;
    for (int s0 = 0; s0 < a.splits; s0 += PB) {
      float m[PB], l[PB], v[PB];
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        // parts past the last re-read the last one and are masked
        const float *ps = pq + min(s0 + j, a.splits - 1) * (D + kPartHeader);
        m[j] = load_coherent(ps);
        l[j] = load_coherent(ps + 1);
        v[j] = load_coherent(ps + kPartHeader + c);
      }
      float mb = M;
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        if (s0 + j >= a.splits) {
          m[j] = -INFINITY;
          l[j] = 0.f;
          v[j] = 0.f;
        }
        bad |= isnan(l[j]);
        mb = fmaxf(mb, m[j]);
      }
      if (mb != -INFINITY) {
        // earlier batches' sums move to the new reference (2^-inf = 0 when
        // there were none)
        const float r = __builtin_amdgcn_exp2f(M - mb);
        num *= r;
        den *= r;
#pragma unroll
        for (int j = 0; j < PB; ++j) {
          const float w = __builtin_amdgcn_exp2f(m[j] - mb);  // 0 for parts that saw no key
          den = fmaf(w, l[j], den);
          num = fmaf(w, v[j], num);
        }
        M = mb;
      }
    }
    const float r = M == -INFINITY ? 0.f : num / den;
    a.O[static_cast<int64_t>(qi) * D + c] = bad ? NAN : r;
  }
}

}  // namespace tis
