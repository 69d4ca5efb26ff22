// tree_decode: route then attend for each query in one launch ("Subquadratic
// Attention with a Hierarchical Tree-Structured Indexer", Abstract: a query
// costs its descent through the tree plus the attention at the end).
//
// One workgroup of 16 waves per query: route_walk leaves the kept leaves in
// LDS and attend_query gathers them straight away, so the leaf list never
// goes through memory and the step pays for one launch instead of two.  The
// leaves are also written out (ascending) when the caller asks for them.
// With few queries each query gets `splits` workgroups that all walk the
// tree and each attend over a share of the kept leaves; the last of them to
// finish merges their partial softmax states.
//
// Fused one-key append + decode over a growing cache (k_decode_append).
// Adding key t = n0 to the tree changes one node per height: the node that
// holds t, whose new sum is the old open sum (zero when t starts the node)
// plus the key; every other node keeps its summary.  So every workgroup can
// decode over the tree of t + 1 keys without waiting for any summary to be
// rewritten: it reads the stored rows of the unchanged nodes, and for the
// node holding t (the last existing node of each level) it computes the new
// mean from the state and the key itself, scored in fp64 while the walk
// scores the first cut level (see OpenNodes).  B * Hkv more workgroups of
// the same launch store the new means and sums; the sums go to the other of
// two state buffers, so no workgroup that still reads the old sums sees the
// new ones.
// The summaries and state it leaves are the ones a separate one-key append
// writes, bit for bit, and the step costs one launch instead of two.
#include "attend_query.hpp"
#include "route_walk.hpp"

namespace tis {
namespace {

constexpr int kDecodeWaves = 16;
constexpr int kDecodeWalkWaves = 8;  // waves that walk the tree (see route_walk)

// After the walk: the kept leaves out (part 0, when asked for), then part
// sp's share of them attended.
template <typename T, int D, bool CACHE>
__device__ inline void decode_attend(const RouteArgs &ra, const AttendArgs &aa,
                                     RouteShared<kDecodeWaves> &rsh, AttendShared<T, D> &ash,
                                     int qi, int sp, uint4 qraw, int kept,
                                     int64_t hoff, unsigned long long *tl = nullptr) {
  if (ra.indices && sp == 0) {
    int32_t *out = ra.indices + static_cast<int64_t>(qi) * ra.beam;
    write_ascending<kDecodeWaves * 64>(rsh.front, kept, out);
    for (int k = kept + static_cast<int>(threadIdx.x); k < ra.beam; k += kDecodeWaves * 64)
      out[k] = -1;
  }
  const int s0 = div_u(sp * kept, aa.splits);
  const int s1 = div_u((sp + 1) * kept, aa.splits);
  float *part = aa.splits > 1
                    ? aa.part + (static_cast<int64_t>(qi) * aa.splits + sp) * (D + kPartHeader)
                    : nullptr;
  attend_query<T, D, CACHE>(aa, ash, qi, qraw, rsh.front + s0, nullptr, s1 - s0, false, part,
                            0.0, 0, 0, tl, &hoff);
  if (aa.splits > 1) merge_parts<D>(aa, qi);
}

template <typename T, typename S, int D, bool CACHE>
__global__ void __launch_bounds__(kDecodeWaves * 64) k_decode(RouteArgs ra, AttendArgs aa) {
  __shared__ RouteShared<kDecodeWaves> rsh;
  __shared__ AttendShared<T, D> ash;
  prefetch_kernargs<sizeof(RouteArgs) + sizeof(AttendArgs)>();
  // part sp of query qi (see k_attend: a query's parts share an XCD)
  const int sp = div_u(static_cast<int>(blockIdx.x), aa.queries);
  const int qi = query_of_slot(blockIdx.x - sp * aa.queries, aa.queries, aa.group);
  const uint4 qraw = attend_q_raw<T, D>(aa, qi);  // in flight during the walk
  const int64_t hoff = head_offset_early<D>(aa, qi);
  // every part walks the tree (the repeated summary reads hit the XCD's L2)
  const int kept = route_walk<T, S, D, kDecodeWaves, kDecodeWalkWaves, CACHE>(ra, rsh, qi);
  decode_attend<T, D, CACHE>(ra, aa, rsh, ash, qi, sp, qraw, kept, hoff);
}

// k_decode with a phase timeline (see tl_stamp): the same walk and gather,
// the same results, plus a wall-clock stamp per wave at each phase.  A
// measurement of where a decode's time goes, not a path of its own.
template <typename T, typename S, int D>
__global__ void __launch_bounds__(kDecodeWaves * 64)
    k_decode_timeline(RouteArgs ra, AttendArgs aa, unsigned long long *tl) {
  __shared__ RouteShared<kDecodeWaves> rsh;
  __shared__ AttendShared<T, D> ash;
  tl_stamp(tl, 0);
  prefetch_kernargs<sizeof(RouteArgs) + sizeof(AttendArgs)>();
  const int sp = div_u(static_cast<int>(blockIdx.x), aa.queries);
  const int qi = query_of_slot(blockIdx.x - sp * aa.queries, aa.queries, aa.group);
  const uint4 qraw = attend_q_raw<T, D>(aa, qi);
  const int64_t hoff = head_offset_early<D>(aa, qi);
  const int kept = route_walk<T, S, D, kDecodeWaves, kDecodeWalkWaves, 0>(
      ra, rsh, qi, nullptr, nullptr, -1, static_cast<const NoPrep *>(nullptr), nullptr, tl);
  tl_stamp(tl, 1);
  decode_attend<T, D, false>(ra, aa, rsh, ash, qi, sp, qraw, kept, hoff, tl);
  __syncthreads();
  tl_stamp(tl, 7);
}

template <typename T> __device__ inline float widen1(const T *p);
template <> __device__ inline float widen1<float>(const float *p) { return *p; }
template <> __device__ inline float widen1<bf16_bits>(const bf16_bits *p) {
  return __uint_as_float(static_cast<uint32_t>(p->v) << 16);
}

// The node holding the new key t at every height of the tree: new sum (old
// open sum + key, in fp64, as a one-key append adds it), new mean rounded
// once to the summary type, and its fp64 score with query qi (as the walk
// scores) into open_score[level]; at the first cut level also its ranking
// key.  Run by the waves that do not walk (one height per row group of
// lanes, 4 columns a lane) while the walking waves score the first cut
// level.
template <typename T, typename S, int D> struct OpenNodes {
  static constexpr int NP = kDecodeWaves - kDecodeWalkWaves;  // waves taking part
  static constexpr int E = 4;
  static constexpr int LPR = D / E;     // lanes per row
  static constexpr int RPI = 64 / LPR;  // rows (heights) per wave
  const RouteArgs &ra;
  const AppendArgs &ap;
  uint64_t *keys;
  double *open_score;
  int64_t head;
  int qi;

  __device__ OpenNodes(const RouteArgs &r, const AppendArgs &a, int q, uint64_t *k, double *os)
      : ra(r), ap(a), keys(k), open_score(os), qi(q) {
    const int bi = div_u(q, ra.q_heads);
    const int hq = q - bi * ra.q_heads;
    head = static_cast<int64_t>(bi) * ra.kv_heads + div_u(hq, ra.group);
  }

  // pw: this wave among the NP; every lane of the wave calls it (the
  // cross-lane sums need their partners, so the loop bound is uniform and
  // whole row groups drop out through `act`)
  __device__ void run(int pw, int lane) const {
    const int col = (lane % LPR) * E;
    const int nh = ra.levels;
    const uint32_t t = static_cast<uint32_t>(ap.n0);
    const T *key = static_cast<const T *>(ap.K) + (head * ap.capacity + t) * D + col;
    const T *qp = static_cast<const T *>(ra.Q) + static_cast<int64_t>(qi) * D + col;
    float kf[E], qf[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      kf[e] = widen1<T>(key + e);
      qf[e] = widen1<T>(qp + e);
    }
    for (int h0 = pw * RPI; h0 < nh; h0 += NP * RPI) {
      const int h = h0 + lane / LPR;
      const bool act = h < nh;
      const int hh = act ? h : 0;
      const uint32_t held = t % ap.span[hh] + 1u;  // keys of t's node up to t
      const double *st = ap.state + (head * ap.heights + hh) * D + col;
      double v[1];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const double sum = st[e] + static_cast<double>(kf[e]);
        // as the walk scores: fp64 products of exact float32 values, summed in fp64
        const double f = SummaryType<S>::value(sum / static_cast<double>(held));
        v[0] = e == 0 ? static_cast<double>(qf[0]) * f : fma(static_cast<double>(qf[e]), f, v[0]);
      }
      const double s = group_transpose_reduce<1, LPR>(v, lane);
      if (act && lane % LPR == 0) {
        const int l = nh - h;
        open_score[l] = s;
        if (l == ra.first_cut) {
          const int last = static_cast<int>(ra.lvl_exist[l]) - 1;
          keys[last] = score_key(s, last, 32 - __clz(last));
        }
      }
    }
  }
};

// The append itself, for (batch, KV head) `head`: at every stored height the
// node holding key t gets the new sum's mean (the summary type), and the new
// sums go to the other state buffer (zero where t completes its node, as the
// next node starts empty).  The same arithmetic as a one-key append.
template <typename T, typename S, int D>
__device__ void append_one(const AppendArgs &ap, int64_t head) {
  const uint32_t t = static_cast<uint32_t>(ap.n0);
  const T *key = static_cast<const T *>(ap.K) + (head * ap.capacity + t) * D;
  S *const summ = static_cast<S *>(ap.summ);
  for (int i = threadIdx.x; i < ap.heights * D; i += kDecodeWaves * 64) {
    const int h = i / D;
    const int c = i - h * D;
    const uint32_t span = ap.span[h];
    const uint32_t held = t % span + 1u;
    const int64_t r = (head * ap.heights + h) * D + c;
    const double sum = ap.state[r] + static_cast<double>(widen1<T>(key + c));
    SummaryType<S>::put(summ + ap.block_off[h] + (head * ap.rows[h] + t / span) * D + c,
                        sum / static_cast<double>(held));
    ap.state_next[r] = held == span ? 0.0 : sum;
  }
}

// Workgroups 0 .. queries * splits - 1 decode (as k_decode); the B * Hkv
// after them append, one (batch, KV head) each.  The appending workgroups
// are short and run on CUs the decode leaves free, and no decode barrier
// waits for their stores.
template <typename T, typename S, int D>
__global__ void __launch_bounds__(kDecodeWaves * 64)
    k_decode_append(RouteArgs ra, AttendArgs aa, AppendArgs ap) {
  __shared__ RouteShared<kDecodeWaves> rsh;
  __shared__ AttendShared<T, D> ash;
  __shared__ double open_score[kMaxLevels + 1];
  prefetch_kernargs<sizeof(RouteArgs) + sizeof(AttendArgs) + sizeof(AppendArgs)>();
  const int nq = aa.queries * aa.splits;
  if (static_cast<int>(blockIdx.x) >= nq) {
    append_one<T, S, D>(ap, static_cast<int64_t>(blockIdx.x) - nq);
    return;
  }
  const int sp = div_u(static_cast<int>(blockIdx.x), aa.queries);
  const int qi = query_of_slot(blockIdx.x - sp * aa.queries, aa.queries, aa.group);
  const uint4 qraw = attend_q_raw<T, D>(aa, qi);
  const int64_t hoff = head_offset_early<D>(aa, qi);
  const OpenNodes<T, S, D> open(ra, ap, qi, rsh.keys, open_score);
  const int kept = route_walk<T, S, D, kDecodeWaves, kDecodeWalkWaves, 1>(
      ra, rsh, qi, nullptr, nullptr, -1, &open, open_score);
  decode_attend<T, D, true>(ra, aa, rsh, ash, qi, sp, qraw, kept, hoff);
}

template <typename T, typename S, bool CACHE>
hipError_t launch_decode_t(int head_dim, const RouteArgs &ra, const AttendArgs &aa,
                           hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ra.queries) * static_cast<unsigned>(aa.splits));
  const dim3 block(kDecodeWaves * 64);
  if (head_dim == 128)
    hipLaunchKernelGGL((k_decode<T, S, 128, CACHE>), grid, block, 0, s, ra, aa);
  else if (head_dim == 64)
    hipLaunchKernelGGL((k_decode<T, S, 64, CACHE>), grid, block, 0, s, ra, aa);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, typename S>
hipError_t launch_decode_ts(int head_dim, const RouteArgs &ra, const AttendArgs &aa,
                            hipStream_t s) {
  return ra.cache ? launch_decode_t<T, S, true>(head_dim, ra, aa, s)
                  : launch_decode_t<T, S, false>(head_dim, ra, aa, s);
}

template <typename T, typename S>
hipError_t launch_decode_append_ts(int head_dim, const RouteArgs &ra, const AttendArgs &aa,
                                   const AppendArgs &ap, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ra.queries) * static_cast<unsigned>(aa.splits) +
                  static_cast<unsigned>(ap.heads));
  const dim3 block(kDecodeWaves * 64);
  if (head_dim == 128)
    hipLaunchKernelGGL((k_decode_append<T, S, 128>), grid, block, 0, s, ra, aa, ap);
  else if (head_dim == 64)
    hipLaunchKernelGGL((k_decode_append<T, S, 64>), grid, block, 0, s, ra, aa, ap);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, typename S>
hipError_t launch_decode_timeline_ts(int head_dim, const RouteArgs &ra, const AttendArgs &aa,
                                     unsigned long long *tl, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(ra.queries) * static_cast<unsigned>(aa.splits));
  const dim3 block(kDecodeWaves * 64);
  if (head_dim == 128)
    hipLaunchKernelGGL((k_decode_timeline<T, S, 128>), grid, block, 0, s, ra, aa, tl);
  else if (head_dim == 64)
    hipLaunchKernelGGL((k_decode_timeline<T, S, 64>), grid, block, 0, s, ra, aa, tl);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_timeline(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra,
                                  const AttendArgs &aa, unsigned long long *tl, hipStream_t s) {
  if (sdt == Dt::FP8 || ra.cache) return hipErrorInvalidValue;  // float32 / bfloat16, full tree
  if (dt == Dt::BF16)
    return sdt == Dt::BF16 ? launch_decode_timeline_ts<bf16_bits, bf16_bits>(head_dim, ra, aa, tl, s)
                           : launch_decode_timeline_ts<bf16_bits, float>(head_dim, ra, aa, tl, s);
  return sdt == Dt::BF16 ? launch_decode_timeline_ts<float, bf16_bits>(head_dim, ra, aa, tl, s)
                         : launch_decode_timeline_ts<float, float>(head_dim, ra, aa, tl, s);
}

hipError_t launch_decode_append(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra,
                                const AttendArgs &aa, const AppendArgs &ap, hipStream_t s) {
  hipError_t e;
  if (sdt == Dt::FP8 || !ra.cache) return hipErrorInvalidValue;
  if (dt == Dt::BF16)
    e = sdt == Dt::BF16 ? launch_decode_append_ts<bf16_bits, bf16_bits>(head_dim, ra, aa, ap, s)
                        : launch_decode_append_ts<bf16_bits, float>(head_dim, ra, aa, ap, s);
  else
    e = sdt == Dt::BF16 ? launch_decode_append_ts<float, bf16_bits>(head_dim, ra, aa, ap, s)
                        : launch_decode_append_ts<float, float>(head_dim, ra, aa, ap, s);
  return e;
}

hipError_t launch_decode(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra,
                         const AttendArgs &aa, hipStream_t s) {
  hipError_t e;
  if (sdt == Dt::FP8) {  // full tree only
    if (ra.cache) return hipErrorInvalidValue;
    e = dt == Dt::BF16 ? launch_decode_t<bf16_bits, fp8_bits, false>(head_dim, ra, aa, s)
                       : launch_decode_t<float, fp8_bits, false>(head_dim, ra, aa, s);
  } else if (dt == Dt::BF16) {
    e = sdt == Dt::BF16 ? launch_decode_ts<bf16_bits, bf16_bits>(head_dim, ra, aa, s)
                        : launch_decode_ts<bf16_bits, float>(head_dim, ra, aa, s);
  } else {
    e = sdt == Dt::BF16 ? launch_decode_ts<float, bf16_bits>(head_dim, ra, aa, s)
                        : launch_decode_ts<float, float>(head_dim, ra, aa, s);
  }
  return e;
}

}  // namespace tis
