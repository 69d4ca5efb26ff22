// Internal declarations shared by the translation units of libtis.
// Kernel argument blocks are passed by value; all offsets are in elements.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tis {

constexpr int kMaxLevels = 16;
constexpr int kMaxCandidates = 256;   // beam * branching scored per level
constexpr int kMaxBranching = 64;
// Phase timeline of the fused decode: slots per wave, waves per workgroup
// (see tl_stamp).
constexpr int kTimelineSlots = 24;
constexpr int kTimelineWaves = 16;

enum class Dt : int { F32 = 0, BF16 = 1, FP8 = 2 };  // FP8: summaries only

// ---------------------------------------------------------------- build --
// Work split.  A wave reduces the b^kw leaves under one node of level lv-kw
// (kw <= kMaxWaveDepth).  A workgroup of nw = b^kg waves owns the subtree of
// one node at level r = lv - kw - kg (a "chunk") and finishes its inner
// levels in LDS.  When r >= 2 the chunk roots leave fp64 sums in the
// workspace and one small kernel per level computes levels r-1 .. 1.
constexpr int kMaxWaveDepth = 3;
constexpr size_t kStageLdsBytes = 64 * 1024;   // LDS budget of the build's staged rows
// A build workspace (when the build needs one) starts with the arrival
// counters of up to kBuildArriveMax level-1 subtrees, at offset 0 whatever
// the geometry; the fp64 node sums follow.
constexpr int64_t kBuildArriveMax = 4096;
constexpr size_t kBuildArriveBytes = kBuildArriveMax * sizeof(unsigned);

struct BuildArgs {
  const void *K;
  void *summ;            // float, bf16 bits or fp8 codes (the summary type)
  float *scales;         // fp8 only: a power-of-two scale per node, level-major
  double *ws_sum;        // fp64 node sums of levels 2..r
  unsigned *arrive;      // [heads * b] chunks of each level-1 subtree done (zero between calls)
  int fuse_top;          // nonzero: the last chunk of each level-1 subtree climbs
                         // its levels r-1 .. 1 (no second kernel)
  int64_t chunks_per_l1; // b^(r-1): chunks under one level-1 node
  int64_t n_keys;        // N
  int64_t chunks;        // b^r chunks per head
  int64_t wave_leaves;   // b^kw
  int branching, leaf_block, levels;
  int root_level;        // r
  int wave_depth;        // kw
  uint32_t pow2_levels;  // bit l set: M_l = N / n_l is a power of two
  int through_stores;    // nonzero: rows written between K loads use device-coherent
                         // stores (K loads always carry the non-temporal hint)
  int stage;             // nonzero: the wave-level summary rows wait in LDS
                         // and leave in one burst after the last K load
  int64_t top_rows;      // b^(r-2): level r-1 nodes under one level-1 node
  int64_t n_at[kMaxLevels + 1];            // b^l
  int64_t chunks_at_level[kMaxLevels + 1]; // B*Hkv*b^l
  int64_t summ_off[kMaxLevels + 1];        // element offset of level l in summ
  int64_t ws_off[kMaxLevels + 1];          // element offset of level l in ws_sum
  double mean_div[kMaxLevels + 1];         // M_l
  double mean_inv[kMaxLevels + 1];         // 1 / M_l when a power of two
};

struct BuildPlan {
  int root_level;        // r
  int wave_depth;        // kw
  int waves;             // nw
  int64_t chunks;        // b^r per head
  size_t lds_bytes;
  size_t sum_elems;
  size_t workspace_bytes;
};

int64_t stage_rows(int64_t nw, int64_t branching, int kw);
bool plan_build(int64_t heads, int head_dim, int branching, int leaf_block, int levels,
                BuildPlan *plan);
// dt: type of K; sdt: type the summaries are stored in
hipError_t launch_build(Dt dt, Dt sdt, int head_dim, int64_t heads, const BuildArgs &a,
                        const BuildPlan &p, hipStream_t s);

// ---------------------------------------------------------------- route --
// The walk reads one of two summary layouts:
//  * full tree (cache == 0): N = b^levels * L, level-major, level l a block
//    [B*Hkv][b^l][d];
//  * growing cache (cache != 0): the tree over the first n_keys of a cache
//    of `capacity` keys per head; height-major (height h = levels - l), height
//    h a block [B*Hkv][ceil(capacity / (L b^h))][d]; node n of level l exists
//    when n * L * b^(levels-l) < n_keys.
struct RouteArgs {
  const void *Q;
  const void *summ;      // float, bf16 bits or fp8 codes (the summary type)
  const float *scales;   // fp8 (full tree only): a scale per node, level-major
  int32_t *indices;
  int32_t *trace;        // may be null
  int queries;           // B * Hq (< 2^31, checked by the host)
  int q_heads, kv_heads, group;
  int branching, levels, beam;
  int first_cut;         // first level with more than beam nodes (levels if none)
  int cache;             // layout (see above)
  int n_keys, leaf_block, capacity;  // growing cache only
  // growing cache, per level l (host-computed): nodes that exist, summary
  // rows per head and element offset of the level's block
  int64_t lvl_exist[kMaxLevels + 2];
  int64_t lvl_rows[kMaxLevels + 1];
  int64_t lvl_off[kMaxLevels + 1];
};

hipError_t launch_route(Dt dt, Dt sdt, int head_dim, const RouteArgs &a, hipStream_t s);

// --------------------------------------------------------------- attend --
// One workgroup per query: its waves split the selected leaf blocks into
// row units, keep online-softmax partials and merge them in LDS.
constexpr int kAttendMaxWaves = 16;

struct AttendArgs {
  const void *Q, *K, *V;
  const int32_t *indices;
  float *O;
  float *part;           // [queries][splits][d + 4] partial states when splits > 1
  unsigned *arrive;      // [queries] parts of each query done so far (zero between calls)
  int splits;            // workgroups per query (1: no split, no workspace)
  int queries;           // B * Hq (< 2^31, checked by the host)
  int64_t n_keys;        // keys in use per head (leaf j holds [jL, min((j+1)L, n_keys)))
  int64_t key_stride;    // rows per head in K and V (n_keys, or a cache's capacity)
  int q_heads, kv_heads, group;
  int leaf_block, beam;
  int64_t n_blocks;      // N / L
  float scale_log2;      // softmax scale * log2(e)
};

int attend_waves(int head_dim, Dt dt, int beam, int leaf_block);
// Workgroups per query: more than one only when few queries would leave most
// CUs idle and each query gathers enough keys to share out.  A split call
// has fewer than kSplitMaxQueries queries.
constexpr int kSplitMaxQueries = 256;
int attend_splits(int64_t queries, int beam, int leaf_block);
// The workspace of a split call: the arrival counters of kSplitMaxQueries
// queries (1 KiB, at offset 0 whatever the geometry, so that one workspace
// serves calls of any shape), then the partial states.
constexpr size_t kArriveBytes = kSplitMaxQueries * sizeof(unsigned);
size_t attend_workspace(int64_t queries, int head_dim, int splits);
hipError_t launch_attend(Dt dt, int head_dim, const AttendArgs &a, hipStream_t s);

// Grouped attend: the G query heads of a KV head together (splits = parts
// per group; a split call has fewer than kSplitMaxQueries groups, whose
// arrival counters sit where the attend's are).
constexpr int kGroupMaxHeads = 64;     // heads per group (one 64-bit mask)
constexpr int kGroupMaxEntries = 512;  // slots per group, G * beam
int attend_group_splits(int64_t groups, int group, int beam);
size_t attend_group_workspace(int64_t groups, int group, int head_dim, int splits);
hipError_t launch_attend_group(Dt dt, int head_dim, const AttendArgs &a, hipStream_t s);

// ---------------------------------------------------------------- decode --
// Route and attend of each query in one workgroup (one launch).
hipError_t launch_decode(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra,
                         const AttendArgs &aa, hipStream_t s);
// The same decode with a per-wave phase timeline in tl (float32 or bfloat16
// summaries over a full tree; see tl_stamp for the layout).
hipError_t launch_decode_timeline(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra,
                                  const AttendArgs &aa, unsigned long long *tl, hipStream_t s);

// ------------------------------------------------------- growing cache --
// Append keys [n0, n1) of a cache of `capacity` keys per head to its tree:
// summaries height-major (height h a block [heads][ceil(capacity / (L
// b^h))][d]), state fp64 [heads][heights][d] open-node sums.
struct AppendArgs {
  const void *K;
  void *summ;            // float or bf16 bits (the summary type)
  double *state;         // the open-node sums before the append
  double *state_next;    // fused append + decode: where the sums after it go
  int64_t heads;         // B * Hkv
  int64_t capacity;
  int64_t n0, n1;        // n1 <= capacity < 2^31
  int leaf_block, branching;
  int heights;           // H: depth of a full cache, stored heights 0 .. H-1
  // per stored height h (host-computed, so the kernel divides nothing wider
  // than 32 bits): element offset of the block, rows per head, keys per node
  int64_t block_off[kMaxLevels];
  uint32_t rows[kMaxLevels];
  uint32_t span[kMaxLevels];   // L b^h: below the capacity (or L itself when H = 1)
  // long appends, split into chunks: the nodes of height chunk_height
  // (chunk_keys = L b^chunk_height keys each) that hold new keys, chunk0 ..
  // chunk0 + nchunks - 1; scratch holds fp64 [heads][nchunks][d], the sum of
  // each chunk's new keys, for the heights above the chunks
  int chunk_height;
  uint32_t chunk_keys;
  int64_t chunk0, nchunks;
  double *scratch;
};

// Chunk height of a cache geometry: the smallest h with L b^h >= 512 keys,
// kept below the cache's depth H and to b^h <= kMaxChunkLeaves leaves.
constexpr int kMaxChunkLeaves = 64;
inline int append_chunk_height(int branching, int leaf_block, int heights) {
  int hc = 0;
  int64_t leaves = 1;
  while (hc + 1 < heights && leaves * branching <= kMaxChunkLeaves &&
         static_cast<int64_t>(leaf_block) * leaves < 512) {
    leaves *= branching;
    ++hc;
  }
  return hc;
}

// Append of one key (n1 = n0 + 1) fused with a decode over the tree of n1
// keys: ra and aa describe the decode at n1, ap the append, with the state
// read from ap.state and written to ap.state_next (two buffers, so that the
// workgroups that read the old sums never see the new ones).
hipError_t launch_decode_append(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra,
                                const AttendArgs &aa, const AppendArgs &ap, hipStream_t s);

// zero `elems` doubles with a kernel (no memset node, so it can sit in a graph)
hipError_t launch_fill_zero(double *p, int64_t elems, hipStream_t s);
hipError_t launch_cache_append(Dt dt, Dt sdt, int head_dim, const AppendArgs &a, hipStream_t s);
// The chunked append: reads the open sums from a.state, writes the new ones
// to a.state_next (two launches when heights remain above the chunks).
hipError_t launch_cache_append_chunked(Dt dt, Dt sdt, int head_dim, const AppendArgs &a,
                                       hipStream_t s);

// ------------------------------------------------------ bounding spheres --
// Radius of every node of a full tree about its stored summary: the largest
// squared key distance, max-reduced in fp64 (as ordered bits, atomically)
// into d2, then rounded up to float32 into radii.  Both are level-major with
// one element per node: level l's block [B*Hkv][b^l] at node_off[l].
struct RadiusArgs {
  const void *K;
  const void *summ;            // float or bf16 bits (the summary type)
  unsigned long long *d2;      // fp64 bits, zeroed before the launch
  float *radii;
  int64_t n_keys;              // N
  int64_t heads;               // B * Hkv
  int64_t leaves_per_wave;
  int64_t waves_per_head;
  int64_t total_nodes;         // B * Hkv * (n_1 + ... + n_lv)
  int branching, leaf_block, levels;
  int64_t n_at[kMaxLevels + 1];      // b^l
  int64_t span[kMaxLevels + 1];      // leaves under a level-l node: b^(lv - l)
  int64_t summ_off[kMaxLevels + 1];  // element offset of level l in summ
  int64_t node_off[kMaxLevels + 1];  // node offset of level l in d2 / radii
};

hipError_t launch_radii(Dt dt, Dt sdt, int head_dim, const RadiusArgs &a, int64_t waves,
                        hipStream_t s);

// Threshold walk and decode: survivors of the sphere bound q.c + |q| r >= tau.
constexpr int kMaxSurvivors = 2048;  // survivors one level may keep
struct SphereArgs {
  const float *radii;          // level-major, as RadiusArgs
  const float *tau;            // [B * Hq]
  int32_t *counts;             // [B * Hq] survivors (-1: overflow), may be null
  int max_nodes;               // survivors a level may keep (<= kMaxSurvivors)
  int64_t node_off[kMaxLevels + 1];
};

hipError_t launch_route_threshold(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra,
                                  const SphereArgs &sa, hipStream_t s);
hipError_t launch_decode_threshold(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra,
                                   const SphereArgs &sa, const AttendArgs &aa, hipStream_t s);

// -------------------------------------------------------- causal prefill --
constexpr int kPrefixRows = 64;    // positions a block (and the sums' factor)
constexpr int kMaxSumLevels = 6;   // 64^6 > 2^31 positions
// levels of the prefix-sum hierarchy over n positions (entries of 64^(k+1)
// positions, for every k with 64^(k+1) < n; at least one)
inline int prefix_sum_levels(int64_t n) {
  int k = 1;
  int64_t c = int64_t{kPrefixRows} * kPrefixRows;
  while (k < kMaxSumLevels && c < n) {
    ++k;
    c *= kPrefixRows;
  }
  return k;
}
// Every position t of a growing cache's first `positions` keys is a query
// over the tree of the first t + 1 keys.  open_summ holds, for every
// (head, position, height < levels), the mean of the keys of t's node up to
// t; complete nodes come from the cache tree's height-major summaries.
struct PrefillArgs {
  const void *K;             // the cache's keys [heads][capacity][d]
  void *open_summ;           // [heads][positions][levels][d], the summary type
  int64_t heads;             // B * Hkv
  int64_t capacity;
  int positions;             // keys in the tree = queries per (batch, head)
  int levels;                // depth of the tree over all positions
  int64_t h_span[kMaxLevels + 1];  // keys under a node of height h: L b^h
  int64_t h_rows[kMaxLevels + 1];  // summary rows per head of height h
  int64_t h_off[kMaxLevels + 1];   // element offset of height h's block
  // fp64 key sums in a hierarchy of factor 64: level k holds, per head, the
  // sums of consecutive runs of 64^(k+1) positions ([heads][sum_n[k]][d] at
  // element sum_off[k] of `sums`), so the keys of any range of positions
  // add up from at most 2 * 63 entries a level
  double *sums;
  int sum_levels;
  int64_t sum_n[kMaxSumLevels];
  int64_t sum_off[kMaxSumLevels];
  // attention 16 positions at a time (leaf blocks of a multiple of 16 keys),
  // `tiles` query heads a workgroup (0: one fused kernel per position): the
  // routing pass writes every position's kept leaves to the attention's
  // indices, V is copied transposed per 16 keys to vt ([heads][ceil(positions
  // / 16)][d][16], the key type)
  int tiles;
  const void *V;
  void *vt;
};

hipError_t launch_prefill(Dt dt, Dt sdt, int head_dim, const RouteArgs &ra, const AttendArgs &aa,
                          const PrefillArgs &pa, hipStream_t s);
// Query heads per workgroup of the 16-position attention (4, 2 or 1,
// dividing the group, within the LDS it may take), 0 if none fits.
int prefill_tile_heads(int group, int beam, int head_dim, int elem_bytes);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// ------------------------------------------------- measurement probes --
hipError_t launch_probe_read(const void *buf, uint64_t bytes, bool nontemporal, uint32_t *sink,
                             hipStream_t s);
hipError_t launch_probe_chase(const uint32_t *next, uint64_t n, uint32_t start, int hops,
                              uint32_t *out, hipStream_t s);

}  // namespace tis
