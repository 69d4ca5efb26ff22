// tree_attend_grouped: the attention of tree_attend with the G query heads
// that share a KV head contracted together on the matrix cores ("Subquadratic
// Attention with a Hierarchical Tree-Structured Indexer", Abstract: the
// attention over the keys each query ends with; the NSA / InfLLMv2 abstract
// on the Progressive Sparse Attention related-papers page: exact softmax over
// the tokens of the chosen blocks).  Each head still attends over exactly
// its own blocks; what changes is the order of work: a leaf that several
// heads of a group kept is loaded once for all of them.
//
// The group is one (batch, KV head) and its G query heads, its slot list
// the G x W entries of its heads (head-major).  `splits` workgroups share
// it, part p owning the entries [p n / S, (p + 1) n / S):
//   * the part loads the whole list and, for each entry it owns, finds
//     whether an earlier entry holds the same leaf and which heads hold it
//     (a 64-bit mask); it attends over the leaves whose first entry it owns,
//     for all their heads (slot rules as tree_attend: negatives are empty, a
//     repeat counts once, an entry >= N / L makes that head's row NaN);
//   * each wave takes tiles of 16 keys in turn: 16 keys x 16 heads scores on
//     MFMA (S^T = K Q^T, fp32 accumulation), each head masked to its own
//     leaves, an online softmax per head, and P V on MFMA (bf16: each weight
//     in three bf16 parts, fp32 precision; V goes through a per-wave LDS
//     tile whose rows are read back 4 keys of one dim per lane, the operand
//     order of the product);
//   * the waves' states meet in LDS in one round and are combined by
//     log-sum-exp in wave order; the workgroup writes O, or its partial
//     state when the group is split, and the last part of the group to
//     finish merges the partial states (device-coherent stores and loads,
//     an agent-scope arrival count, as in the split attend).
// More than 16 heads (up to 64) take 2 or 4 row blocks of 16, a wave per
// block per tile.
#include "attend_query.hpp"
#include "mfma_tile.hpp"

namespace tis {
namespace {

template <typename T> struct GroupWaves {
  // bf16 tiles need half the registers and LDS of fp32 ones
  static constexpr int NW = sizeof(T) == 2 ? 8 : 4;
};

// A wave's V tile in LDS, 16 keys in natural layout, rows RS elements apart:
// stored with 8-byte stores, read back as the P V operand (keys 4 g + i of
// dim 16 nt + r per lane).  RS = D + 4 (bf16) or D + 2 (fp32) puts the 4
// key groups of a read 8 banks apart, so the 64 lanes' reads do not collide.
template <typename T, int D> struct VTile;
template <int D> struct VTile<bf16_bits, D> {
  static constexpr int RS = D + 4;
  static constexpr int BYTES = 16 * RS * 2;
  __device__ static void read(typename TileMath<bf16_bits, D>::VReg &v, const unsigned char *blk,
                              int r, int g) {
    const unsigned short *b = reinterpret_cast<const unsigned short *>(blk);
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) {
      const unsigned short *c = b + 4 * g * RS + 16 * nt + r;
      v.v[nt] = make_uint2(static_cast<uint32_t>(c[0]) | (static_cast<uint32_t>(c[RS]) << 16),
                           static_cast<uint32_t>(c[2 * RS]) | (static_cast<uint32_t>(c[3 * RS]) << 16));
    }
  }
};
template <int D> struct VTile<float, D> {
  static constexpr int RS = D + 2;
  static constexpr int BYTES = 16 * RS * 4;
  __device__ static void read(typename TileMath<float, D>::VReg &v, const unsigned char *blk,
                              int r, int g) {
    const float *b = reinterpret_cast<const float *>(blk);
#pragma unroll
    for (int nt = 0; nt < D / 16; ++nt) {
      const float *c = b + 4 * g * RS + 16 * nt + r;
      v.v[nt] = make_float4(c[0], c[RS], c[2 * RS], c[3 * RS]);
    }
  }
};

// 1 if any lane of this lane's aligned group of `tpe` lanes (a power of two
// dividing 64) has `x` set
__device__ inline bool group_any(bool x, int lane, int tpe) {
  const unsigned long long b = __ballot(x);
  const unsigned long long m = tpe >= 64 ? ~0ull : ((1ull << tpe) - 1ull);
  return ((b >> (lane & ~(tpe - 1))) & m) != 0ull;
}

template <typename T, int D, int RBK>
__global__ void __launch_bounds__(GroupWaves<T>::NW * 64) k_attend_group(AttendArgs a) {
  using TM = TileMath<T, D>;
  using VT = VTile<T, D>;
  constexpr int NW = GroupWaves<T>::NW;
  constexpr int NT = NW * 64;
  constexpr int NS = NW / RBK;               // waves per block of 16 heads
  constexpr int ES = static_cast<int>(sizeof(T));
  constexpr int CPR = D * ES / 16;           // 16-byte chunks per row
  constexpr int VPT = 16 * CPR / 64;         // V chunks per lane per tile
  constexpr int EPC = 16 / ES;               // elements per chunk
  constexpr int NR = D / 16 * 4;             // accumulator registers per lane
  constexpr int OBYTES = NW * NR * 64 * 4;   // every wave's accumulators
  constexpr int VBYTES = NW * VT::BYTES;     // every wave's V tile
  // slot entries, padded to whole 4-entry reads of every lane's slice
  __shared__ __align__(16) int s_ent[kGroupMaxEntries + 256];
  // this part's entries: the leaf, if the entry is the leaf's first in the
  // list (else -1), and the heads whose entries hold it
  __shared__ int s_own[kGroupMaxEntries];
  __shared__ unsigned long long s_omask[kGroupMaxEntries];
  __shared__ float s_m[NW][16], s_l[NW][16];
  __shared__ unsigned long long s_bad;
  __shared__ int s_last;
  __shared__ __align__(16) unsigned char s_obuf[OBYTES];
  __shared__ __align__(16) unsigned char s_vbuf[VBYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15;
  const int g = lane >> 4;
  const int rb = w % RBK;  // block of 16 heads
  const int st = w / RBK;  // this wave's place among the block's waves
  const int G = a.group;
  const int W = a.beam;
  const int n = G * W;
  const int L = a.leaf_block;
  const int S = a.splits;
  const int64_t nb = a.n_blocks;
  // the split parts of a group are `groups` apart in the grid, so with a
  // multiple of 8 groups they run on one XCD
  const int groups = a.queries / G;
  const int sp = static_cast<int>(blockIdx.x) / groups;
  const int grp = static_cast<int>(blockIdx.x) - sp * groups;
  const int64_t q0 = static_cast<int64_t>(grp) * G;  // the group's first query row
  const T *kh = static_cast<const T *>(a.K) + static_cast<int64_t>(grp) * a.key_stride * D;
  const T *vh = static_cast<const T *>(a.V) + static_cast<int64_t>(grp) * a.key_stride * D;

  TM tm;
  const int hrow = 16 * rb + r;  // this lane's head in its block
  tm.load_q(static_cast<const T *>(a.Q) + (q0 + min(hrow, G - 1)) * D, hrow < G, g);

  // ---- this part's leaves.  Part sp owns the slot entries [e0, e1) of the
  // group's G x W list (head-major) and attends over the leaves whose first
  // entry in the list is one of them, for every head that kept them: tpe
  // lanes share an entry, each scanning a contiguous slice of the list 4
  // entries at a time (padding: -1, never a leaf).
  const int e0 = n * sp / S;
  const int ne = n * (sp + 1) / S - e0;
  int tpe = 1;
  while (tpe < 64 && tpe * 2 * ne <= NT) tpe *= 2;
  const int n4 = (n + 4 * tpe - 1) / (4 * tpe) * (4 * tpe);
  const int cl = n4 / tpe;
  for (int e = tid; e < n4; e += NT) s_ent[e] = e < n ? a.indices[q0 * W + e] : -1;
  if (tid == 0) s_bad = 0ull;
  __syncthreads();
  for (int e = tid; e < n; e += NT)
    if (s_ent[e] >= nb) atomicOr(&s_bad, 1ull << (e / W));
  const int sub = tid & (tpe - 1);
  for (int base = 0; base < ne; base += NT / tpe) {
    const int e = e0 + base + tid / tpe;
    const int v = e < e0 + ne ? s_ent[e] : -1;
    const bool ok = v >= 0 && v < nb;
    bool dup = false;             // an earlier entry holds v
    unsigned mlo = 0u, mhi = 0u;  // the heads whose entries hold v
    if (ok) {
      const int j0 = sub * cl;
      for (int j = j0; j < j0 + cl; j += 4) {
        const int4 q = *reinterpret_cast<const int4 *>(s_ent + j);
        const int qv[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (qv[k] == v) {
            const int h = (j + k) / W;
            dup |= j + k < e;
            if (h < 32) mlo |= 1u << h; else mhi |= 1u << (h - 32);
          }
        }
      }
    }
    dup = group_any(dup, lane, tpe);
    for (int off = 1; off < tpe; off <<= 1) {
      mlo |= __shfl_xor(mlo, off);
      mhi |= __shfl_xor(mhi, off);
    }
    if (sub == 0 && e < e0 + ne) {
      s_own[e - e0] = ok && !dup ? v : -1;
      s_omask[e - e0] = (static_cast<unsigned long long>(mhi) << 32) | mlo;
    }
  }
  __syncthreads();
  const int tpl = (L + 15) / 16;  // tiles per leaf
  const int T_ = ne * tpl;

  // ---- this wave's tiles
  float m = -INFINITY, lsum = 0.f;
  mf_f32x4 o[D / 16];
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt) o[nt] = mf_f32x4{0.f, 0.f, 0.f, 0.f};
  // the heads of this block that attend over tile t (0: none, or not a
  // first entry)
  const auto rows_of = [&](int t) -> unsigned {
    const int u = t / tpl;
    return s_own[u] >= 0 ? static_cast<unsigned>(s_omask[u] >> (16 * rb)) & 0xffffu : 0u;
  };
  using KReg = typename TM::KReg;
  using VReg = typename TM::VReg;
  // loads of tile t (one with rows: a first entry's leaf)
  const auto fetch = [&](int t, KReg &kr, uint4 *vr) {
    const int u = t / tpl;
    const int kt = (t - u * tpl) * 16;
    const int64_t base = static_cast<int64_t>(s_own[u]) * L;
    TM::load_k(kr, kh + (base + min(kt + r, L - 1)) * D, g);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = lane + 64 * i;
      const int row = c / CPR;
      vr[i] = *reinterpret_cast<const uint4 *>(vh + (base + min(kt + row, L - 1)) * D +
                                                (c - row * CPR) * EPC);
    }
  };
  unsigned char *vblk = s_vbuf + w * VT::BYTES;
  const auto compute = [&](int t, unsigned rows, const KReg &kr, const uint4 *vraw) {
    const int kt = (t - (t / tpl) * tpl) * 16;
    const mf_f32x4 sc = tm.scores(kr);
    // V rows into this wave's tile: chunk c is elements (c % CPR) * EPC ..
    // of key c / CPR
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = lane + 64 * i;
      const int row = c / CPR;
      uint2 *dst = reinterpret_cast<uint2 *>(vblk + (row * VT::RS + (c - row * CPR) * EPC) * ES);
      dst[0] = make_uint2(vraw[i].x, vraw[i].y);
      dst[1] = make_uint2(vraw[i].z, vraw[i].w);
    }
    __builtin_amdgcn_wave_barrier();
    VReg vr;
    VT::read(vr, vblk, r, g);
    const bool act = (rows >> r) & 1u;
    float x[4], mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = act && kt + 4 * g + i < L ? sc[i] * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // weights 2^(x - m) against a reference m that moves only when a score
    // passes it by more than 8 (the factors are applied when it moves; the
    // merges below remove m whatever it is)
    const bool move = mx > m + 8.f;
    if (__ballot(move)) {
      const float mnew = move ? mx : m;
      const float alpha = move ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;  // 0 from -inf
      lsum *= alpha;
      m = mnew;
      // output rows 4 g + i take the factor of head 4 g + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * g + i);
#pragma unroll
        for (int nt = 0; nt < D / 16; ++nt) o[nt][i] *= ai;
      }
    }
    const float mref = m == -INFINITY ? 0.f : m;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - mref);
    TM::pv3(o, p, vr);
#pragma unroll
    for (int i = 0; i < 4; ++i) lsum += p[i];
    __builtin_amdgcn_wave_barrier();
  };

  // tiles t, t + NS, ...: one at a time (measured: issuing the loads of 2
  // or 4 tiles before the first computes was 2-13% slower, warm)
  for (int t = st; t < T_; t += NS) {
    const unsigned rows = rows_of(t);
    if (rows == 0u) continue;
    KReg kr;
    uint4 vr[VPT];
    fetch(t, kr, vr);
    compute(t, rows, kr, vr);
  }

  // ---- the waves' states meet in LDS: per head reference and sum, and
  // the accumulators register by register, lane-major
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  if (g == 0) {
    s_m[w][r] = m;
    s_l[w][r] = lsum;
  }
  float *ob = reinterpret_cast<float *>(s_obuf);
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) ob[(w * NR + nt * 4 + i) * 64 + lane] = o[nt][i];
  __syncthreads();
  // outputs (head h of block b, column c), a thread each in turn: the
  // log-sum-exp combination of the block's waves, in wave order
  for (int oi = tid; oi < RBK * 16 * D; oi += NT) {
    const int hb = oi / D;
    const int c = oi - hb * D;
    const int b = hb >> 4, h = hb & 15;
    const int hq = 16 * b + h;
    if (hq >= G) continue;
    const int reg = (c >> 4) * 4 + (h & 3);
    const int ln = (h >> 2) * 16 + (c & 15);
    float mj[NS], mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      mj[j] = s_m[j * RBK + b][h];
      mx = fmaxf(mx, mj[j]);
    }
    float num = 0.f, den = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const float f = __builtin_amdgcn_exp2f(mj[j] - mx);  // 0 for waves that saw no key
        den = fmaf(f, s_l[j * RBK + b][h], den);
        num = fmaf(f, ob[((j * RBK + b) * NR + reg) * 64 + ln], num);
      }
    }
    const bool bad = (s_bad >> hq) & 1ull;
    if (S == 1) {
      const float v = mx == -INFINITY ? 0.f : num / den;
      a.O[(q0 + hq) * D + c] = bad ? NAN : v;
    } else {
      float *part = a.part + ((static_cast<int64_t>(grp) * S + sp) * G + hq) * (D + kPartHeader);
      store_coherent(part + kPartHeader + c, num);
      if (c == 0) {
        store_coherent(part, mx);
        store_coherent(part + 1, bad ? NAN : den);
      }
    }
  }
  if (S == 1) return;

  // ---- the last workgroup of the group merges the S partial states
  wait_vector_memory();
  __syncthreads();
  if (tid == 0) {
    const unsigned before = __hip_atomic_fetch_add(a.arrive + grp, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
    s_last = before == static_cast<unsigned>(S - 1);
  }
  __syncthreads();
  if (!s_last) return;
  if (tid == 0) __hip_atomic_store(a.arrive + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float *pg = a.part + static_cast<int64_t>(grp) * S * G * (D + kPartHeader);
  const int SG = S * G;  // <= 256: part x = s * G + head
  // the first batch's accumulators (4 outputs x 16 parts a thread) are
  // requested together with the parts' headers
  constexpr int KB = 4, SB = 16;
  float v[KB][SB];
  const auto load_batch = [&](int k0, int s0) {
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        const int oc = min(tid + (k0 + kk) * NT, G * D - 1);
        const int hq = oc / D;
        const int s = min(s0 + j, S - 1);
        v[kk][j] = load_coherent(pg + static_cast<int64_t>(s * G + hq) * (D + kPartHeader) +
                                 kPartHeader + (oc - hq * D));
      }
  };
  load_batch(0, 0);
  float *pm = reinterpret_cast<float *>(s_vbuf);  // reference of part x, then its weight
  float *pl = pm + 256;                            // sum of part x
  float *pden = pl + 256;                          // per head: combined sum (NaN: bad)
  for (int x = tid; x < SG; x += NT) {
    pm[x] = load_coherent(pg + static_cast<int64_t>(x) * (D + kPartHeader));
    pl[x] = load_coherent(pg + static_cast<int64_t>(x) * (D + kPartHeader) + 1);
  }
  __syncthreads();
  for (int hq = tid; hq < G; hq += NT) {
    float mx = -INFINITY;
    bool bad = false;
    for (int s = 0; s < S; ++s) {
      mx = fmaxf(mx, pm[s * G + hq]);
      bad |= isnan(pl[s * G + hq]);
    }
    float den = 0.f;
    for (int s = 0; s < S; ++s) {
      const float f = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pm[s * G + hq] - mx);
      den = fmaf(f, pl[s * G + hq], den);
      pm[s * G + hq] = f;
    }
    pden[hq] = bad ? NAN : (mx == -INFINITY ? -1.f : den);  // -1: no key at all
  }
  __syncthreads();
  const int K2 = (G * D + NT - 1) / NT;  // outputs per thread
  for (int k0 = 0; k0 < K2; k0 += KB) {
    float num[KB] = {};
    for (int s0 = 0; s0 < S; s0 += SB) {
      if (k0 > 0 || s0 > 0) load_batch(k0, s0);
#pragma unroll
      for (int kk = 0; kk < KB; ++kk) {
        const int hq = min(tid + (k0 + kk) * NT, G * D - 1) / D;
#pragma unroll
        for (int j = 0; j < SB; ++j)
          if (s0 + j < S) num[kk] = fmaf(pm[(s0 + j) * G + hq], v[kk][j], num[kk]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      const int oc = tid + (k0 + kk) * NT;
      if (k0 + kk >= K2 || oc >= G * D) continue;
      const int hq = oc / D;
      const float den = pden[hq];
      a.O[(q0 + hq) * D + (oc - hq * D)] = isnan(den) ? NAN : (den < 0.f ? 0.f : num[kk] / den);
    }
  }
}

template <typename T, int D>
hipError_t launch_group_t(const AttendArgs &a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.queries / a.group) * static_cast<unsigned>(a.splits));
  const dim3 block(GroupWaves<T>::NW * 64);
  if (a.group <= 16)
    hipLaunchKernelGGL((k_attend_group<T, D, 1>), grid, block, 0, s, a);
  else if (a.group <= 32)
    hipLaunchKernelGGL((k_attend_group<T, D, 2>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((k_attend_group<T, D, 4>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

int attend_group_splits(int64_t groups, int group, int beam) {
  // up to about one workgroup per CU, no more parts than the group has
  // slots, at most 16 parts (measured on MI355X: each part adds an arrival
  // and a partial state to merge, and 32 parts of 4 heads took 21 us where
  // 16 took 17) and at most 256 partial states for the last part to merge
  if (groups >= kSplitMaxQueries) return 1;
  int s = 1;
  while (s < 16 && groups * s * 2 <= 256 && s * 2 <= group * beam && s * 2 * group <= 256)
    s *= 2;
  return s;
}

size_t attend_group_workspace(int64_t groups, int group, int head_dim, int splits) {
  if (splits <= 1) return 0;
  return kArriveBytes + static_cast<size_t>(groups) * splits * group * (head_dim + kPartHeader) *
                            sizeof(float);
}

hipError_t launch_attend_group(Dt dt, int head_dim, const AttendArgs &a, hipStream_t s) {
  if (a.group < 1 || a.group > kGroupMaxHeads || a.group * a.beam > kGroupMaxEntries)
    return hipErrorInvalidValue;
  if (dt == Dt::BF16 && head_dim == 128) return launch_group_t<bf16_bits, 128>(a, s);
  if (dt == Dt::BF16 && head_dim == 64) return launch_group_t<bf16_bits, 64>(a, s);
  if (dt == Dt::F32 && head_dim == 128) return launch_group_t<float, 128>(a, s);
  if (dt == Dt::F32 && head_dim == 64) return launch_group_t<float, 64>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace tis
