// Device-side helpers shared by the kernels of libtis: 16-byte vector access
// to fp32 / bf16 rows, wave64 reductions and the fp64 cross-lane exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tis_internal.hpp"

namespace tis {

// Storage element of a bf16 tensor: its 16-bit pattern.
struct bf16_bits {
  uint16_t v;
};

// Storage element of fp8 summaries: an OCP e4m3 code (1 sign, 4 exponent
// bits with bias 7, 3 fraction bits; largest finite value 448).  A node's
// codes are scaled by a power of two kept beside them (see fp8_scale_exp).
struct fp8_bits {
  uint8_t v;
};

template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int kElems = 4;
  __device__ static inline void unpack(const uint4 &u, float *f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
};
template <> struct Vec16<bf16_bits> {
  static constexpr int kElems = 8;
  // Little-endian: element 2i is the low half of word i.  A bf16 value is the
  // float32 whose upper 16 bits are its pattern, so widening is a shift.
  __device__ static inline void unpack(const uint4 &u, float *f) {
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xffff0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xffff0000u);
    f[4] = __uint_as_float(u.z << 16);
    f[5] = __uint_as_float(u.z & 0xffff0000u);
    f[6] = __uint_as_float(u.w << 16);
    f[7] = __uint_as_float(u.w & 0xffff0000u);
  }
};

// ---- stored summaries --------------------------------------------------
// A summary is the fp64 mean of a node's keys rounded once to its storage
// type: float32 (hardware conversion, round to nearest even) or bfloat16.
// The bfloat16 rounding works on the fp64 bits so that it is one rounding
// (through float32 it would be two, which can differ at a float32 value that
// sits exactly halfway between two bfloat16 values).  In the normal bfloat16
// range, rounding the 52-bit fraction to 7 bits to nearest even is adding
// 2^44 - 1 plus the lowest kept bit and dropping 45 bits; a carry out of the
// fraction steps the exponent, which is the right result, including the step
// past the largest bfloat16 to infinity.  Below 2^-126 the bfloat16 grid is
// the fixed spacing 2^-133: the value is scaled onto it (exactly, a power of
// two) and rounded by rint, which rounds halves to even.
__device__ inline uint16_t bf16_from_double(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(u >> 48) & 0x8000u;
  const uint64_t a = u & 0x7fffffffffffffffull;
  const uint32_t e = static_cast<uint32_t>(a >> 52);  // biased fp64 exponent
  if (e >= 1023u - 126u) {
    const uint64_t r = (a + 0x00000fffffffffffull + ((a >> 45) & 1ull)) >> 45;  // exp | 7 bits
    const uint32_t be = static_cast<uint32_t>(r >> 7);                         // fp64-biased
    if (be >= 1023u + 128u) return static_cast<uint16_t>(sign | 0x7f80u);     // overflow
    return static_cast<uint16_t>(sign | ((be - (1023u - 127u)) << 7) |
                                 static_cast<uint32_t>(r & 0x7fu));
  }
  const double m = __builtin_rint(__longlong_as_double(static_cast<long long>(a)) * 0x1p133);
  return static_cast<uint16_t>(sign | static_cast<uint32_t>(m));  // m <= 128 (128: 2^-126)
}

// e4m3 code -> float (exact): 0 exponent field = subnormal (m * 2^-9).
__device__ inline float e4m3_to_float(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
                      : static_cast<float>(m) * 0x1p-9f;
  return (c & 0x80u) ? -mag : mag;
}

// fp64 -> e4m3, round to nearest even, for |x| <= 448 (the caller's scale
// guarantees it).  From 2^-6 up (normal codes) the 52-bit fraction is
// rounded to 3 bits as for bf16 (add 2^48 - 1 plus the lowest kept bit, drop
// 49 bits; a carry steps the exponent); below, the grid is the fixed spacing
// 2^-9, reached by an exact scaling and rint (halves to even).
__device__ inline uint32_t e4m3_from_double(double x) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(u >> 56) & 0x80u;
  const uint64_t a = u & 0x7fffffffffffffffull;
  if ((a >> 52) >= 1023u - 6u) {
    const uint64_t r = (a + 0x0000ffffffffffffull + ((a >> 49) & 1ull)) >> 49;
    return sign | ((static_cast<uint32_t>(r >> 3) - (1023u - 7u)) << 3) |
           static_cast<uint32_t>(r & 7u);
  }
  const double m = __builtin_rint(__longlong_as_double(static_cast<long long>(a)) * 0x1p9);
  return sign | static_cast<uint32_t>(m);  // m <= 8 (8: 2^-6, the smallest normal)
}

// Scale exponent of an fp8 summary row: the smallest e with amax * 2^-e <=
// 448; 0 for amax = 0; clamped to [-126, 127] (2^e a normal float32).
// With amax = f * 2^k, 0.5 <= f < 1: e = k - 9 if f <= 0.875 (448 = 0.875 *
// 2^9), else k - 8.  f <= 0.875 is the fp64 fraction field <= 0.75 * 2^52.
__device__ inline int fp8_scale_exp(double amax) {
  if (!(amax > 0.0)) return 0;
  const uint64_t a = static_cast<uint64_t>(__double_as_longlong(amax));
  const int k = static_cast<int>(a >> 52) - 1022;
  const bool low = (a & 0x000fffffffffffffull) <= 0x000c000000000000ull;
  int e = low ? k - 9 : k - 8;
  if ((a >> 52) == 0) e = -126;  // a subnormal double: far below any clamp
  return e < -126 ? -126 : e > 127 ? 127 : e;
}

__device__ inline double pow2_double(int e) {
  return __longlong_as_double(static_cast<long long>(static_cast<uint64_t>(e + 1023) << 52));
}

template <typename S> struct SummaryType;
template <> struct SummaryType<float> {
  __device__ static inline float from_mean(double m) { return static_cast<float>(m); }
  __device__ static inline void put(float *p, double m) { *p = static_cast<float>(m); }
  // the stored value, as float32
  __device__ static inline float value(double m) { return static_cast<float>(m); }
};
template <> struct SummaryType<bf16_bits> {
  __device__ static inline bf16_bits from_mean(double m) { return bf16_bits{bf16_from_double(m)}; }
  __device__ static inline void put(bf16_bits *p, double m) { p->v = bf16_from_double(m); }
  __device__ static inline float value(double m) {
    return __uint_as_float(static_cast<uint32_t>(bf16_from_double(m)) << 16);
  }
};

__device__ inline uint4 load16(const void *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

// 16-byte load with the non-temporal (streaming) hint.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ inline uint4 load16_stream(const void *p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// x / d and x % d for x >= 0 and a divisor d >= 1 that is the same for the
// whole wave (a head count, a group size, a split count).  A 32-bit division
// by a runtime value is a chain of some 25 scalar and vector instructions,
// and the scalar ones go through the one scalar unit that all waves of a CU
// share, so a 16-wave workgroup that divides on its critical path waits for
// the whole CU's share of them.  Power-of-two divisors (every geometry of
// the usual workloads) take a shift and a mask instead.
__device__ inline int div_u(int x, int d) {
  return (d & (d - 1)) == 0 ? x >> __builtin_ctz(static_cast<unsigned>(d)) : x / d;
}
__device__ inline int mod_u(int x, int d) {
  return (d & (d - 1)) == 0 ? x & (d - 1) : x % d;
}

// Query served by workgroup slot s (0 <= s < queries).  Workgroups are
// dispatched to the 8 XCDs in turn, so slots s = x (mod 8) share XCD x and
// its L2.  When queries is a multiple of 8 * group, the group queries that
// share a KV head get slots on one XCD, and the reads they have in common
// (the upper tree levels, leaf blocks chosen by several of them) meet in
// that L2 instead of going to HBM once per query.  Any other shape keeps
// the identity.  The map is a bijection either way; only locality depends
// on it.
__device__ inline int query_of_slot(int s, int queries, int group) {
  if (group == 1 || mod_u(queries, 8 * group) != 0) return s;
  const int x = s & 7;
  const int t = s >> 3;
  return (div_u(t, group) * 8 + x) * group + mod_u(t, group);
}

// Row geometry for a wave reading rows of D elements of T, 16 bytes per lane:
// kLanesPerRow lanes cover one row; one wave-wide load covers kRowsPerInstr
// consecutive rows.
template <typename T, int D> struct RowGeom {
  static constexpr int kElemsPerLane = Vec16<T>::kElems;
  static constexpr int kLanesPerRow = D / kElemsPerLane;
  static constexpr int kRowsPerInstr = 64 / kLanesPerRow;
  static_assert(D % kElemsPerLane == 0, "row must be a whole number of 16-byte chunks");
  static_assert(kLanesPerRow <= 64 && 64 % kLanesPerRow == 0, "row must tile a wave");
};

// ---- cross-lane exchange without the LDS crossbar ----------------------
// xor_lane<M>(v, lane): lane l receives v of lane l ^ M.  M = 1, 2: one DPP
// quad permutation; M = 4, 8: two DPP row permutations (xor 4 = xor 3 then
// mirror in 8 lanes, xor 8 = mirror in 16 then mirror in 8); M = 16, 32:
// one permlane swap (gfx950) and a select.
template <int CTRL> __device__ inline uint32_t dpp(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

template <int M> __device__ inline uint32_t xor_lane(uint32_t v, int lane) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane mask");
  if constexpr (M == 1) {
    return dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    return dpp<0x141>(dpp<0x1B>(v));  // quad_perm [3,2,1,0], row_half_mirror
  } else if constexpr (M == 8) {
    return dpp<0x141>(dpp<0x140>(v));  // row_mirror, row_half_mirror
  } else if constexpr (M == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? p[0] : p[1];
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? p[0] : p[1];
  }
}
template <int M> __device__ inline int xor_lane(int v, int lane) {
  return static_cast<int>(xor_lane<M>(static_cast<uint32_t>(v), lane));
}
template <int M> __device__ inline float xor_lane(float v, int lane) {
  return __uint_as_float(xor_lane<M>(__float_as_uint(v), lane));
}
template <int M> __device__ inline double xor_lane(double v, int lane) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = xor_lane<M>(static_cast<uint32_t>(u), lane);
  const uint32_t hi = xor_lane<M>(static_cast<uint32_t>(u >> 32), lane);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// v + (v of lane ^ M), the same on both lanes of each pair.
template <int M, typename F> __device__ inline F xor_sum(F v, int lane) {
  return v + xor_lane<M>(v, lane);
}

// Butterfly reductions over all 64 lanes (every lane gets the result).
__device__ inline float wave_max(float v) {
  const int lane = __lane_id();
  v = fmaxf(v, xor_lane<1>(v, lane));
  v = fmaxf(v, xor_lane<2>(v, lane));
  v = fmaxf(v, xor_lane<4>(v, lane));
  v = fmaxf(v, xor_lane<8>(v, lane));
  v = fmaxf(v, xor_lane<16>(v, lane));
  return fmaxf(v, xor_lane<32>(v, lane));
}

__device__ inline double wave_max_d(double v) {
  const int lane = __lane_id();
  v = fmax(v, xor_lane<1>(v, lane));
  v = fmax(v, xor_lane<2>(v, lane));
  v = fmax(v, xor_lane<4>(v, lane));
  v = fmax(v, xor_lane<8>(v, lane));
  v = fmax(v, xor_lane<16>(v, lane));
  return fmax(v, xor_lane<32>(v, lane));
}

__device__ inline float wave_sum(float v) {
  const int lane = __lane_id();
  v = xor_sum<1>(v, lane);
  v = xor_sum<2>(v, lane);
  v = xor_sum<4>(v, lane);
  v = xor_sum<8>(v, lane);
  v = xor_sum<16>(v, lane);
  return xor_sum<32>(v, lane);
}

// Sum over lane groups: every lane gets the sum over the lanes that differ
// from it only in the bits FIRST, 2*FIRST, ..., LAST.
template <int FIRST, int LAST, typename F> __device__ inline F group_sum(F v, int lane) {
  if constexpr (FIRST <= LAST) {
    v = xor_sum<FIRST>(v, lane);
    return group_sum<FIRST * 2, LAST>(v, lane);
  } else {
    return v;
  }
}

// Transposed reduction over lane groups of LPR consecutive lanes.
// In: every lane holds U partial values v[0..U) (U <= LPR, both powers of 2).
// Out: the lane returns sum over its LPR-lane group of v[k], k = (lane % LPR)
// / (LPR / U); the LPR / U lanes sharing a k all return the same total.
// Each halving step exchanges half of the remaining values, so U values cost
// U - 1 + log2(LPR / U) exchanges instead of U * log2(LPR).
template <int U, int LPR, int STEP, typename F>
__device__ inline void transpose_steps(F (&v)[U], int lane) {
  constexpr int h = U >> (STEP + 1);
  if constexpr (h >= 1) {
    constexpr int m = LPR >> (STEP + 1);
    const bool sel = (lane & m) != 0;
#pragma unroll
    for (int k = 0; k < h; ++k) {
      const F keep = sel ? v[k + h] : v[k];
      const F send = sel ? v[k] : v[k + h];
      v[k] = keep + xor_lane<m>(send, lane);
    }
    transpose_steps<U, LPR, STEP + 1>(v, lane);
  }
}

template <int U, int LPR, typename F> __device__ inline F group_transpose_reduce(F (&v)[U], int lane) {
  static_assert(U >= 1 && U <= LPR, "need U <= LPR");
  transpose_steps<U, LPR, 0>(v, lane);
  return group_sum<1, LPR / U / 2>(v[0], lane);
}

}  // namespace tis

namespace tis {

// A lane's share of a summary row when a walk scores it: E consecutive
// elements from one load (16 bytes of float32 or bf16, 8 bytes of fp8 codes,
// so that fp8 rows keep the bf16 lane layout).
template <typename S> struct RowLoad {
  static constexpr int E = Vec16<S>::kElems;
  using Raw = uint4;
  __device__ static inline Raw load(const S *p) { return load16(p); }
  __device__ static inline void unpack(const Raw &r, float *f) { Vec16<S>::unpack(r, f); }
};
template <> struct RowLoad<fp8_bits> {
  static constexpr int E = 8;
  using Raw = uint2;
  __device__ static inline Raw load(const fp8_bits *p) {
    return *reinterpret_cast<const uint2 *>(p);
  }
  // gfx950's packed conversion decodes OCP e4m3, two codes an instruction
  // (checked against e4m3_to_float for every finite code)
  __device__ static inline void unpack(const Raw &r, float *f) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.x), false);
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.x), true);
    const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.y), false);
    const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(r.y), true);
    f[0] = a[0];
    f[1] = a[1];
    f[2] = b[0];
    f[3] = b[1];
    f[4] = c[0];
    f[5] = c[1];
    f[6] = d[0];
    f[7] = d[1];
  }
};

template <typename S> inline constexpr bool kIsFp8 = false;
template <> inline constexpr bool kIsFp8<fp8_bits> = true;

// Stores one node's fp8 summary row, held by the 64 lanes of a wave (lane
// value j is column cols[j]): the row's power-of-two scale 2^e from its
// largest magnitude, each mean rounded once to e4m3 after an exact scaling by
// 2^-e; lane 0 stores the scale.
template <int C>
__device__ inline void store_row_fp8(fp8_bits *row, float *scale, const double (&m)[C],
                                     const int (&cols)[C], int lane) {
  double amax = 0.0;
#pragma unroll
  for (int j = 0; j < C; ++j) amax = fmax(amax, fabs(m[j]));
  amax = wave_max_d(amax);
  const int e = fp8_scale_exp(amax);
  const double inv = pow2_double(-e);
#pragma unroll
  for (int j = 0; j < C; ++j) row[cols[j]].v = static_cast<uint8_t>(e4m3_from_double(m[j] * inv));
  if (lane == 0) *scale = static_cast<float>(pow2_double(e));
}

// ---- kernel arguments ----------------------------------------------------
// Brings the first BYTES of the launch's argument block into the scalar
// cache with one scalar load per 64-byte line, all issued before any is
// waited for.  The scalar cache starts a launch empty, and the compiler
// fetches arguments where the code first needs them: in the decode kernels
// that was three dependent rounds before the first summary row could be
// requested, each a memory round trip.  Called first thing in a kernel, it
// makes that one round; the compiler's own argument loads then hit.
template <size_t BYTES> __device__ inline void prefetch_kernargs() {
  typedef const __attribute__((address_space(4))) uint32_t kword;
  constexpr int N = static_cast<int>((BYTES + 63) / 64);
  kword *p = (kword *)__builtin_amdgcn_kernarg_segment_ptr();
  uint32_t v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = p[i * 16];
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" ::"s"(v[i]));
}

// ---- phase timeline of the fused decode (measurement only) --------------
// Slot k of wave w of workgroup g is tl[(g * kTimelineWaves + w) *
// kTimelineSlots + k]: the value of the GPU's constant-rate wall clock
// (s_memrealtime) when lane 0 of the wave passed phase k.  Phases: 0 entry;
// 1 walk done; 2 first K load about to issue; 3 first unit's K arrived and
// scored; 4 first unit's V used; 5 the wave's units done; 6 waves' partials
// merged in LDS (barrier passed); 7 end; 8 + 2j scored level j of the walk
// (this wave's rows, before the barrier), 9 + 2j level j ranked (after the
// barrier), j < 8.  Unrecorded slots keep what the caller put there.  With
// tl == nullptr (a constant in every kernel but the timeline one) nothing is
// recorded and the call compiles away.
__device__ inline void tl_stamp(unsigned long long *tl, int slot) {
  if (tl && (threadIdx.x & 63) == 0)
    tl[(static_cast<size_t>(blockIdx.x) * kTimelineWaves + (threadIdx.x >> 6)) * kTimelineSlots +
       slot] = __builtin_amdgcn_s_memrealtime();
}
// Holds back a stamp until v has been computed (so the stamp after a load's
// first use waits for the load).
template <typename V> __device__ inline void tl_after(unsigned long long *tl, const V &v) {
  if (tl) asm volatile("" ::"v"(v));
}

// ---- data handed between workgroups of one launch ----------------------
// Agent-scope (device-coherent) stores and loads: they bypass the XCDs'
// private L2 state, so a workgroup on another XCD reads what was stored
// without an L2 write-back or invalidate (a release or acquire fence at
// agent scope would do both, over the whole L2).  A producer stores with
// store_coherent, waits for the stores to complete (wait_vector_memory) and
// only then counts itself in on an agent-scope atomic; the consumer that
// reads the count issues its load_coherent loads after it.
template <typename F> __device__ inline void store_coherent(F *p, F v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename F> __device__ inline F load_coherent(const F *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0): this wave's vector memory operations, the coherent
// stores included, have completed
__device__ inline void wait_vector_memory() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace tis
