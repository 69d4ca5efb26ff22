// Measurement probes: what the memory system gives the access patterns this
// library relies on, measured on the machine it runs on.  Neither probe is
// part of the method; the benchmark uses them for the ceilings it reports
// beside each kernel's roofline fraction, and the streaming read also empties
// the caches before cold-state timings (it reads, so it leaves no dirty
// lines whose write-back a timed kernel would pay for).
//
//  * k_probe_read: every 16-byte chunk of a buffer read once with one
//    16-byte load per lane, eight loads in flight per lane, over up to
//    65,536 waves: the achievable HBM read rate for the streaming pattern of
//    the build and the gather.
//  * k_probe_chase: one lane follows a chain of dependent 4-byte loads,
//    i = next[i]: the latency of one dependent round trip to wherever the
//    chain's footprint lives (L2, the Infinity Cache or HBM), which bounds a
//    level of the tree walk from below.
#include "tis_device.hpp"
#include "tis_internal.hpp"

namespace tis {
namespace {

constexpr int kProbeThreads = 256;

template <bool NT> __device__ inline uint4 probe_load(const uint4 *p) {
  if constexpr (NT) {
    return load16_stream(p);
  } else {
    return load16(p);
  }
}

// Reads chunks [0, n16).  The XOR of everything read decides whether the
// kernel writes `sink`, so no load can be dropped; the magic value makes the
// write practically never happen.
template <bool NT>
__global__ void __launch_bounds__(kProbeThreads) k_probe_read(const uint4 *p, uint64_t n16,
                                                              uint32_t *sink) {
  constexpr int U = 8;  // loads in flight per lane
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * kProbeThreads;
  uint64_t i = static_cast<uint64_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = probe_load<NT>(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = probe_load<NT>(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// One lane walks `hops` links of the chain from `start`; an index past the
// buffer (a malformed chain) restarts at 0, so no load leaves the buffer.
__global__ void __launch_bounds__(64) k_probe_chase(const uint32_t *next, uint64_t n, uint32_t start,
                                                    int hops, uint32_t *out) {
  if (threadIdx.x != 0) return;
  uint32_t i = start < n ? start : 0u;
  for (int h = 0; h < hops; ++h) {
    i = next[i];
    i = i < n ? i : 0u;
  }
  out[0] = i;
}

}  // namespace

hipError_t launch_probe_read(const void *buf, uint64_t bytes, bool nontemporal, uint32_t *sink,
                             hipStream_t s) {
  const uint64_t n16 = bytes / 16;
  // up to 64 workgroups of 4 waves per CU on 256 CUs (measured best for
  // multi-GiB reads), one per 1,024 chunks for small buffers
  uint64_t blocks = (n16 + 4 * kProbeThreads - 1) / (4 * kProbeThreads);
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  const dim3 grid(static_cast<unsigned>(blocks));
  if (nontemporal)
    hipLaunchKernelGGL((k_probe_read<true>), grid, dim3(kProbeThreads), 0, s,
                       static_cast<const uint4 *>(buf), n16, sink);
  else
    hipLaunchKernelGGL((k_probe_read<false>), grid, dim3(kProbeThreads), 0, s,
                       static_cast<const uint4 *>(buf), n16, sink);
  return hipGetLastError();
}

hipError_t launch_probe_chase(const uint32_t *next, uint64_t n, uint32_t start, int hops,
                              uint32_t *out, hipStream_t s) {
  hipLaunchKernelGGL(k_probe_chase, dim3(1), dim3(64), 0, s, next, n, start, hops, out);
  return hipGetLastError();
}

}  // namespace tis
