// Operand layouts of the 16x16 matrix-core tiles shared by the kernels that
// attend over key tiles on MFMA (causal prefill, grouped decode attention).
// A tile is 16 keys by 16 query rows:
//   * scores come out transposed, S^T = K Q^T (16 keys x 16 rows, fp32
//     accumulation): lane l holds row l % 16 and keys 4 (l / 16) + i,
//     i = 0..3, so each lane keeps one row's running maximum;
//   * the same registers are the A operand of P V (rows x keys), and V is
//     read from a [d][16] block (LDS, rows VS elements apart), whose 4
//     consecutive keys per lane match the lane's keys; the product lands as
//     O[row 4 (l / 16) + i][dim 16 nt + l % 16].
// bf16 inputs: scores with the 16x16x32 bf16 product (bf16 x bf16 products
// are exact in the fp32 accumulators), weights split into bf16 parts for
// 16x16x16 bf16 products with V; fp32 inputs: the 16x16x4 fp32 product for
// both.
#pragma once

#include "tis_device.hpp"

namespace tis {

typedef short mf_bf16x8 __attribute__((ext_vector_type(8)));
typedef short mf_bf16x4 __attribute__((ext_vector_type(4)));
typedef float mf_f32x4 __attribute__((ext_vector_type(4)));

__device__ inline short bf16_rne(float f) {  // finite f
  const uint32_t u = __float_as_uint(f);
  return static_cast<short>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <typename T, int D> struct TileMath;

template <int D> struct TileMath<bf16_bits, D> {
  // the query rows as the B operand of K Q^T: row r, dims 32 s + 8 g .. + 7
  mf_bf16x8 q[D / 32];
  struct KReg { uint4 v[D / 32]; };
  struct VReg { uint2 v[D / 16]; };
  // elements per V row in LDS: 16 keys and 4 more, so that 16 lanes reading
  // 8 bytes each at rows r = 0..15 start on distinct bank pairs
  static constexpr int VS = 20;
  __device__ void load_q(const bf16_bits *qrow, bool valid, int g) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
      uint4 u = valid ? *reinterpret_cast<const uint4 *>(qrow + 32 * s + 8 * g) : make_uint4(0, 0, 0, 0);
      q[s] = __builtin_bit_cast(mf_bf16x8, u);
    }
  }
  __device__ static void load_k(KReg &k, const bf16_bits *krow, int g) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) k.v[s] = *reinterpret_cast<const uint4 *>(krow + 32 * s + 8 * g);
  }
  // vt points at a key tile's [d][16] block in LDS (rows VS apart): lane
  // column r, key group g
  __device__ static void load_v(VReg &v, const bf16_bits *vt, int r, int g) {
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt)
      v.v[nt] = *reinterpret_cast<const uint2 *>(vt + (16 * nt + r) * VS + 4 * g);
  }
  __device__ mf_f32x4 scores(const KReg &k) const {
    mf_f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8, k.v[s]), q[s], c,
                                                   0, 0, 0);
    return c;
  }
  // o[nt] += P (rows x 16 keys) V (16 keys x dims 16 nt .. + 15).  Each
  // weight p is split into a bf16 high part h (p with its low 16 bits
  // cleared) and a bf16 low part (p - h, which is exact in fp32, rounded to
  // nearest), so h + lo is p to within 2^-16 relative; both products with
  // the bf16 values are exact in the fp32 accumulators.  p is replaced by
  // the weights as used (h + lo), for the normaliser.
  __device__ static void pv(mf_f32x4 *o, float *p, const VReg &v) {
    mf_bf16x4 hi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = __float_as_uint(p[i]);
      const float h = __uint_as_float(u & 0xffff0000u);
      hi[i] = static_cast<short>(u >> 16);
      lo[i] = bf16_rne(p[i] - h);
      p[i] = h + __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(lo[i])) << 16);
    }
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) {
      const mf_bf16x4 vb = __builtin_bit_cast(mf_bf16x4, v.v[nt]);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, vb, o[nt], 0, 0, 0);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, vb, o[nt], 0, 0, 0);
    }
  }
  // The same product with each weight in three bf16 parts: h (the top 16
  // bits), m (the remainder p - h, exact in fp32, rounded to nearest) and
  // l (what m leaves, p - h - m, also exact, rounded), so h + m + l is p to
  // within 2^-24 relative: fp32 weights, as a scalar fp32 product would use
  // them.  p is replaced by h + m + l for the normaliser.
  __device__ static void pv3(mf_f32x4 *o, float *p, const VReg &v) {
    mf_bf16x4 hi, mi, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = __float_as_uint(p[i]);
      const float h = __uint_as_float(u & 0xffff0000u);
      const float r1 = p[i] - h;
      hi[i] = static_cast<short>(u >> 16);
      mi[i] = bf16_rne(r1);
      const float m = __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(mi[i])) << 16);
      const float r2 = r1 - m;
      lo[i] = bf16_rne(r2);
      p[i] = h + (m + __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(lo[i])) << 16));
    }
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) {
      const mf_bf16x4 vb = __builtin_bit_cast(mf_bf16x4, v.v[nt]);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(hi, vb, o[nt], 0, 0, 0);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(mi, vb, o[nt], 0, 0, 0);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(lo, vb, o[nt], 0, 0, 0);
    }
  }
};

template <int D> struct TileMath<float, D> {
  // the query rows: row r, dims 16 s + 4 g .. + 3; product (s, i) pairs
  // lane group g with dim 16 s + 4 g + i in both operands
  float4 q[D / 16];
  struct KReg { float4 v[D / 16]; };
  struct VReg { float4 v[D / 16]; };
  // elements per V row in LDS: 16 keys and 4 more, so that 8 lanes reading
  // 16 bytes each at rows r = 0..7 start on distinct groups of 4 banks
  static constexpr int VS = 20;
  __device__ void load_q(const float *qrow, bool valid, int g) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      q[s] = valid ? *reinterpret_cast<const float4 *>(qrow + 16 * s + 4 * g)
                   : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __device__ static void load_k(KReg &k, const float *krow, int g) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) k.v[s] = *reinterpret_cast<const float4 *>(krow + 16 * s + 4 * g);
  }
  __device__ static void load_v(VReg &v, const float *vt, int r, int g) {
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt)
      v.v[nt] = *reinterpret_cast<const float4 *>(vt + (16 * nt + r) * VS + 4 * g);
  }
  __device__ mf_f32x4 scores(const KReg &k) const {
    mf_f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(k.v[s].x, q[s].x, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(k.v[s].y, q[s].y, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(k.v[s].z, q[s].z, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(k.v[s].w, q[s].w, c, 0, 0, 0);
    }
    return c;
  }
  // product i pairs lane group g with key 4 g + i of the tile (the weights
  // enter in fp32 as they are)
  __device__ static void pv(mf_f32x4 *o, float *p, const VReg &v) {
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) {
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[0], v.v[nt].x, o[nt], 0, 0, 0);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[1], v.v[nt].y, o[nt], 0, 0, 0);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[2], v.v[nt].z, o[nt], 0, 0, 0);
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(p[3], v.v[nt].w, o[nt], 0, 0, 0);
    }
  }
  __device__ static void pv3(mf_f32x4 *o, float *p, const VReg &v) { pv(o, p, v); }
};

}  // namespace tis
