// Device-side helpers shared by the kernels of libtis: 16-byte vector access
// to fp32 / bf16 rows, wave64 reductions and the fp64 cross-lane exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tis {

// Storage element of a bf16 tensor: its 16-bit pattern.
struct bf16_bits {
  uint16_t v;
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

__device__ inline uint4 load16(const void *p) {
  return *reinterpret_cast<const uint4 *>(p);
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

__device__ inline double shfl_xor_f64(double v, int mask) {
  return __shfl_xor(v, mask, 64);
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Transposed reduction over lane groups of LPR consecutive lanes.
// In: every lane holds U partial values v[0..U) (U <= LPR, both powers of 2).
// Out: the lane returns sum over its LPR-lane group of v[k], k = (lane % LPR)
// / (LPR / U); the LPR / U lanes sharing a k all return the same total.
// Each halving step exchanges half of the remaining values, so U values cost
// U - 1 + log2(LPR / U) exchanges instead of U * log2(LPR).
template <int U, int LPR, typename F> __device__ inline F group_transpose_reduce(F (&v)[U], int lane) {
  static_assert(U >= 1 && U <= LPR, "need U <= LPR");
#pragma unroll
  for (int step = 0; (U >> (step + 1)) >= 1; ++step) {
    const int h = U >> (step + 1);
    const int m = LPR >> (step + 1);
    const bool sel = (lane & m) != 0;
#pragma unroll
    for (int k = 0; k < U / 2; ++k) {
      if (k < h) {
        const F keep = sel ? v[k + h] : v[k];
        const F send = sel ? v[k] : v[k + h];
        v[k] = keep + __shfl_xor(send, m, 64);
      }
    }
  }
  F s = v[0];
#pragma unroll
  for (int m = LPR / U / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  return s;
}

}  // namespace tis
