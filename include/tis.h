/*
 * tis.h -- tree-indexed sparse attention decode on AMD Instinct MI355X (gfx950).
 *
 * The method (ZHA abstract, "Subquadratic Attention with a Hierarchical
 * Tree-Structured Indexer"): an index tree over the KV cache whose nodes hold
 * compressed summaries of the keys below them; each decode query descends it
 * level by level to a small set of keys, and softmax attention runs over that
 * set only.  The tree is static and the keys are routed level by level, as
 * in the ALHR post ("Vdev-Ctrl Releases ALHR", Technical Breakthrough and
 * Core Features).
 *
 * Geometry used by every call
 *   B  batch, Hkv KV heads, Hq query heads (Hq % Hkv == 0, G = Hq / Hkv),
 *   d  head dim (64 or 128), b branching (2..64), L leaf_block (keys per leaf),
 *   lv levels (1..16): branchings below the implicit root, so a head has
 *   b^lv leaves and N = b^lv * L keys.  Level l (1..lv) has n_l = b^l nodes;
 *   node n of level l covers the M_l = N / n_l contiguous keys
 *   [n*M_l, (n+1)*M_l).  The children of node n are n*b .. n*b+b-1.
 *   A query head h reads KV head h / G (contiguous groups).
 *
 * Memory
 *   Every data pointer is a DEVICE pointer (HBM), 16-byte aligned, owned by
 *   the caller.  The library allocates, frees and synchronises nothing; all
 *   work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *   Layouts are dense row-major:
 *     K, V       [B][Hkv][N][d]   element type `dtype`
 *     Q          [B][Hq][d]       element type `dtype`
 *     summaries  float32 or bfloat16 (the tree's summary_dtype), level-major:
 *                for l = 1..lv a block [B][Hkv][n_l][d], block l starting at
 *                element offset d*B*Hkv*(n_1+...+n_{l-1})
 *     indices    int32 [B][Hq][W]
 *     O          float32 [B][Hq][d]
 *
 * Errors
 *   Every argument is checked on the host before anything is enqueued; a call
 *   that returns non-TIS_OK has written nothing.  A launch failure returns
 *   TIS_E_HIP.  Faults inside kernels surface at the caller's next
 *   synchronisation.  tis_last_error() gives a message for the last non-OK
 *   status of the calling thread.  No C++ exception crosses this interface.
 *
 * Workspaces
 *   tis_tree_build, tis_tree_attend, tis_tree_attend_grouped and
 *   tis_tree_decode take a caller-owned
 *   device workspace (16-byte aligned) of at least the size the matching
 *   *_workspace_bytes query returns.  A size of 0 means none is needed and
 *   NULL is accepted.  A workspace starts with arrival counters: the build's
 *   first 16,384 bytes count the finished chunks of each level-1 subtree
 *   (the last chunk of a subtree to finish climbs to level 1), attend's and
 *   decode's first 1,024 bytes count the finished parts of each split query
 *   (few queries, long key sets: the last part to finish merges them), the
 *   grouped attend's those of each split group of query heads.  The
 *   build's fp64 node sums and the split queries' partial softmax states
 *   follow.  Those counter bytes must be zero before a workspace's first
 *   call (allocate it zeroed, or clear it once); every call that completes
 *   leaves them zero, whatever its shape, so one workspace serves any
 *   sequence of calls of its kind.  The rest never matters on entry.  Calls
 *   that share a workspace must be ordered (same stream or synchronised).
 */
#ifndef TIS_H_
#define TIS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tis_status {
  TIS_OK = 0,
  TIS_E_NULL = 1,        /* a required pointer is NULL                        */
  TIS_E_SHAPE = 2,       /* sizes inconsistent (e.g. N != b^lv * L)           */
  TIS_E_DTYPE = 3,       /* unknown element type                              */
  TIS_E_ALIGN = 4,       /* a data pointer is not 16-byte aligned            */
  TIS_E_UNSUPPORTED = 5, /* valid but outside what is compiled (d, b, beam..)  */
  TIS_E_WORKSPACE = 6,   /* workspace missing or smaller than required        */
  TIS_E_HIP = 7          /* the HIP runtime reported an error                 */
} tis_status;

/* Element types.  TIS_FP8_E4M3 is a summary type only (summary_dtype of a
 * tis_tree); inputs are TIS_F32 or TIS_BF16. */
typedef enum tis_dtype { TIS_F32 = 0, TIS_BF16 = 1, TIS_FP8_E4M3 = 2 } tis_dtype;

/* Largest candidate set one level may score: beam * branching <= 256. */
#define TIS_MAX_CANDIDATES 256

/* A built tree: plain descriptor (no hidden state).  The caller sets
 * `summaries` (device, tis_tree_summary_bytes_as() bytes) and
 * `summary_dtype` before tis_tree_build; the build fills in the geometry
 * fields.  Route and decode read summary_dtype from the descriptor.
 *
 * summary_dtype: the type the summaries are stored in.  TIS_F32 (0, also
 *   what a zero-initialised descriptor holds): each node mean rounded once
 *   to float32.  TIS_BF16: rounded once, straight from the fp64 mean, to
 *   bfloat16 (round to nearest, ties to even; not through float32), which
 *   halves the bytes every routing level reads.  TIS_FP8_E4M3: per node, the
 *   smallest power of two 2^e with max_i |mean_i| * 2^-e <= 448 (0 for an
 *   all-zero row; e clamped to [-126, 127]), and each mean * 2^-e rounded
 *   once to OCP e4m3 (round to nearest even, from the fp64 value); a quarter
 *   of the float32 bytes.  Layout: the codes, one byte an element with the
 *   float32 element layout, then (16-byte aligned) one float32 scale 2^e per
 *   node, level-major like the rows.  fp8 summaries serve tis_tree_build,
 *   tis_tree_route and tis_tree_decode; the other calls reject them with
 *   TIS_E_UNSUPPORTED.  The pages fix no precision for the summaries; all
 *   three are the same mean, stored at different widths.  Any other value:
 *   TIS_E_DTYPE. */
typedef struct tis_tree {
  int32_t batch, kv_heads, n_keys, head_dim, branching, leaf_block, levels;
  int32_t summary_dtype;  /* tis_dtype of the stored summaries */
  void *summaries;
} tis_tree;

/* Bytes of a float32 summaries buffer: 4 * d * B * Hkv * (n_1 + ... + n_lv).
 * Returns 0 if the geometry is invalid or the size overflows. */
size_t tis_tree_summary_bytes(int batch, int kv_heads, int head_dim, int branching,
                              int levels);
/* The same for summaries stored as summary_dtype (2 bytes an element for
 * TIS_BF16; for TIS_FP8_E4M3 one byte an element rounded up to 16 bytes plus
 * 4 bytes a node); 0 also for an unknown summary_dtype. */
size_t tis_tree_summary_bytes_as(int batch, int kv_heads, int head_dim, int branching,
                                 int levels, tis_dtype summary_dtype);

/* Bytes of workspace tis_tree_build needs for this geometry; 0 if none or if
 * the geometry is invalid. */
size_t tis_build_workspace_bytes(int batch, int kv_heads, int n_keys, int head_dim,
                                 int branching, int leaf_block, int levels);

/*
 * tis_tree_build -- node summaries for every level (ZHA abstract: each node
 * of the index tree summarizes the cached keys below it; here the summary of
 * a node is the mean of those keys).
 *
 * K        [B][Hkv][N][d] keys, dtype TIS_F32 or TIS_BF16 (read once).
 * tree     in: tree->summaries; out: geometry fields filled in.
 * Each summary is the exact mean of the node's keys (sums accumulated in
 * fp64, in a fixed order), rounded once to tree->summary_dtype.
 * Deterministic.
 * Requires N == b^lv * L, lv >= 1, b >= 2, d in {64,128}.
 */
tis_status tis_tree_build(const void *K, tis_dtype dtype, int batch, int kv_heads,
                          int n_keys, int head_dim, int branching, int leaf_block,
                          int levels, tis_tree *tree, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * tis_tree_route -- top-down beam traversal (ZHA abstract: a query descends
 * the summary tree level by level and ends with a small set of keys).
 *
 * Q        [B][Hq][d], dtype TIS_F32 or TIS_BF16; tree->batch is B.
 * For every query: the candidates of level 1 are the b children of the
 * root; those of level l are all children of the nodes kept at level l-1.
 * A candidate's score is q . summary, computed in fp64 from the stored
 * (float32 or bfloat16) summary.  The kept set is the first min(beam, #candidates) candidates in
 * (score descending, node index ascending) order.
 * indices  out: int32 [B][Hq][beam], the kept leaves in ascending order.
 * trace    optional (NULL to skip): int32 [B][Hq][lv][beam], the kept nodes
 *          of every level in ascending order, padded with -1.
 * Requires 1 <= beam <= b^lv and beam * b <= TIS_MAX_CANDIDATES.
 */
tis_status tis_tree_route(const void *Q, tis_dtype dtype, int q_heads,
                          const tis_tree *tree, int beam, int32_t *indices,
                          int32_t *trace, void *stream);

/* Bytes of workspace tis_tree_attend needs for this geometry (0: none). */
size_t tis_attend_workspace_bytes(int batch, int q_heads, int head_dim, int beam,
                                  int leaf_block);

/*
 * tis_tree_attend -- exact softmax attention over the keys of the selected
 * leaf blocks (ZHA abstract: the attention after the descent; the NSA /
 * InfLLMv2 abstract on the Progressive Sparse Attention related-papers page:
 * exact softmax restricted to the tokens of the chosen blocks).
 *
 * Q [B][Hq][d], K and V [B][Hkv][N][d], all of type `dtype`.
 * indices  int32 [B][Hq][beam] leaf-block numbers, any order.  A negative
 *          entry is an empty slot; a repeated entry counts once; an entry
 *          >= N / L makes that query's output row NaN (never read out of
 *          bounds).  A query whose set is empty gets a zero row.
 * scale    softmax scale; <= 0 selects 1/sqrt(d); NaN or infinite is
 *          rejected (TIS_E_SHAPE).
 * O        out: float32 [B][Hq][d], o = sum_t softmax(scale*q.k_t) v_t over
 *          the union of the selected blocks; fp32 accumulation.
 * workspace, workspace_bytes: see Workspaces (tis_attend_workspace_bytes).
 * Requires N % L == 0 and 1 <= beam <= TIS_MAX_CANDIDATES.
 */
tis_status tis_tree_attend(const void *Q, const void *K, const void *V, tis_dtype dtype,
                           int batch, int q_heads, int kv_heads, int n_keys,
                           int head_dim, int leaf_block, const int32_t *indices,
                           int beam, float scale, float *O, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Bytes of workspace tis_tree_attend_grouped needs for this geometry (0: none). */
size_t tis_attend_grouped_workspace_bytes(int batch, int q_heads, int kv_heads, int head_dim,
                                          int beam);

/*
 * tis_tree_attend_grouped -- tis_tree_attend with the G = q_heads / kv_heads
 * query heads that share a KV head contracted together on the matrix cores
 * (the attention of the ZHA abstract and of the NSA / InfLLMv2 abstract, as
 * for tis_tree_attend; the grouping is an order of work, not a change of
 * what is computed).  Every leaf block kept by any head of a group is read
 * once for the whole group; each head still attends over exactly its own
 * blocks (masked per head).
 *
 * Arguments, layouts, slot rules (negative = empty, repeats count once,
 * >= N / L makes the head's row NaN, an empty set gives a zero row), scale
 * and O exactly as tis_tree_attend; results agree with it to fp32 rounding
 * (weights and sums in fp32, another summation order).
 * workspace, workspace_bytes: see Workspaces
 * (tis_attend_grouped_workspace_bytes; counters in the first 1,024 bytes).
 * Requires N % L == 0, beam >= 1, G <= 64 and G * beam <= 512
 * (TIS_E_UNSUPPORTED otherwise).
 */
tis_status tis_tree_attend_grouped(const void *Q, const void *K, const void *V, tis_dtype dtype,
                                   int batch, int q_heads, int kv_heads, int n_keys,
                                   int head_dim, int leaf_block, const int32_t *indices,
                                   int beam, float scale, float *O, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * tis_tree_decode -- one decode step: tis_tree_route and tis_tree_attend for
 * every query in a single launch (ZHA abstract: a query costs its descent
 * through the tree plus the attention over the keys it ends with).
 *
 * Q [B][Hq][d] and K, V [B][Hkv][N][d] of type `dtype`, matching the tree
 * (B, Hkv, N, d, L as built).  The leaves each query keeps are exactly those
 * tis_tree_route returns; O is the softmax attention over their keys as in
 * tis_tree_attend (summation order may differ in the last fp32 bits).
 * indices  optional (NULL to skip): int32 [B][Hq][beam], the kept leaves in
 *          ascending order.
 * scale    softmax scale; <= 0 selects 1/sqrt(d); NaN or infinite rejected.
 * workspace, workspace_bytes: see Workspaces (tis_decode_workspace_bytes).
 * Requires 1 <= beam <= b^lv and beam * b <= TIS_MAX_CANDIDATES.
 */
tis_status tis_tree_decode(const void *Q, const void *K, const void *V, tis_dtype dtype,
                           int q_heads, const tis_tree *tree, int beam, float scale, float *O,
                           int32_t *indices, void *workspace, size_t workspace_bytes,
                           void *stream);

/* Bytes of workspace tis_tree_decode needs for this geometry (0: none). */
size_t tis_decode_workspace_bytes(int batch, int q_heads, int head_dim, int beam,
                                  int leaf_block);

/* Size of the scratch that tis_tree_decode_noalloc keeps on each GPU. */
#define TIS_NOALLOC_SCRATCH_BYTES (1u << 20)

/*
 * tis_tree_decode_noalloc -- tis_tree_decode for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, checks, kernels and
 * results as tis_tree_decode (bit for bit), without the workspace: the split
 * partial states go to a scratch array of TIS_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on, from its first call there until the
 * process ends.  The call allocates and frees nothing.  The caller still
 * supplies Q, K, V, the tree, O and (optionally) indices.
 *
 * A geometry whose workspace (tis_decode_workspace_bytes) exceeds
 * TIS_NOALLOC_SCRATCH_BYTES is rejected with TIS_E_WORKSPACE before anything
 * is enqueued.  All calls on one GPU share its scratch, whatever their
 * stream: calls that may overlap on one GPU race and give undefined
 * results, so order them (one stream, or synchronise between them).  The
 * scratch is laid out as a workspace (see Workspaces): its arrival counters
 * are zero when the library is loaded and every call leaves them zero; the
 * rest holds what the last call left and no call depends on it.
 * The first call on a device looks up the scratch's address there (no
 * allocation); a failure of that lookup returns TIS_E_HIP.
 */
tis_status tis_tree_decode_noalloc(const void *Q, const void *K, const void *V, tis_dtype dtype,
                                   int q_heads, const tis_tree *tree, int beam, float scale,
                                   float *O, int32_t *indices, void *stream);

/* ------------------------------------------------------------------------
 * Threshold retrieval with bounding spheres
 *
 * The Louver explainer ("Sparse Attention as a Range Searching Problem",
 * Methodologie) retrieves every key whose score q.k reaches a threshold tau,
 * pruning clusters whose bounding sphere cannot reach tau, which never loses
 * such a key.  Here the clusters are the nodes of a built tree:
 *   - centre of a node: its stored summary; radius: the smallest float32 r
 *     with r * r >= the largest squared distance (evaluated in fp64) from
 *     the centre to a key under the node, so every key lies in the sphere;
 *   - a node survives when q.c + |q| r >= tau (fp64; |q| from the fp64 sum of
 *     squares), the largest score any point of its sphere can have;
 *   - level 1 scores the root's children, level l the children of the
 *     level-(l-1) survivors; a level may keep at most max_nodes survivors,
 *     more is an overflow;
 *   - attention: exact softmax over the keys of the surviving leaves whose
 *     fp64 score q.k is >= tau.  As no such key is pruned, this is softmax
 *     over every key of the cache with q.k >= tau.
 * Radii are float32, level-major with one element per node: for l = 1..lv
 * a block [B][Hkv][n_l] starting at node offset B*Hkv*(n_1+...+n_{l-1}).
 * --------------------------------------------------------------------- */

/* Survivors one level may keep (max_nodes). */
#define TIS_MAX_SURVIVORS 2048

/* Bytes of the radii of a tree: 4 * B * Hkv * (n_1 + ... + n_lv) (0 if
 * invalid), and of the workspace tis_tree_radii needs (8 bytes a node). */
size_t tis_tree_radius_bytes(int batch, int kv_heads, int branching, int levels);
size_t tis_radius_workspace_bytes(int batch, int kv_heads, int branching, int levels);

/*
 * tis_tree_radii -- radius of every node of a built tree about its stored
 * summary (either summary type).  K as given to tis_tree_build (read once).
 * radii out: float32, layout above.  workspace: tis_radius_workspace_bytes()
 * bytes, 16-byte aligned (fp64 maxima; contents on entry never matter).
 */
tis_status tis_tree_radii(const void *K, tis_dtype dtype, const tis_tree *tree, float *radii,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * tis_tree_route_threshold -- the surviving leaves of every query.
 * Q [B][Hq][d] of type dtype; radii from tis_tree_radii for this tree;
 * tau float32 [B][Hq] (any value, infinities included).
 * indices out: int32 [B][Hq][max_nodes], the surviving leaves ascending,
 *          padded with -1 (all -1 after an overflow).
 * counts   optional: int32 [B][Hq], the number of surviving leaves, or -1
 *          when some level had more than max_nodes survivors.
 * Requires 1 <= max_nodes <= TIS_MAX_SURVIVORS.
 */
tis_status tis_tree_route_threshold(const void *Q, tis_dtype dtype, int q_heads,
                                    const tis_tree *tree, const float *radii, const float *tau,
                                    int max_nodes, int32_t *indices, int32_t *counts,
                                    void *stream);

/* Bytes of workspace tis_tree_decode_threshold needs (0: none). */
size_t tis_decode_threshold_workspace_bytes(int batch, int q_heads, int head_dim, int max_nodes,
                                            int leaf_block);

/*
 * tis_tree_decode_threshold -- the route above and the attention over the
 * surviving leaves in one launch.  O out: float32 [B][Hq][d], softmax over
 * the keys with fp64 q.k >= tau (a zero row when there is none, NaN after an
 * overflow); scale as for tis_tree_decode.  indices and counts optional, as
 * for tis_tree_route_threshold.
 */
tis_status tis_tree_decode_threshold(const void *Q, const void *K, const void *V, tis_dtype dtype,
                                     int q_heads, const tis_tree *tree, const float *radii,
                                     const float *tau, int max_nodes, float scale, float *O,
                                     int32_t *indices, int32_t *counts, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Measurement probes (no part of the method)
 *
 * The benchmark reports each kernel's roofline fraction beside what the
 * memory system gives the same access pattern on the machine at hand; these
 * two calls measure it.  The caller times them (events around the call).
 * --------------------------------------------------------------------- */

/* Reads every 16-byte chunk of buf[0, bytes) once: 16-byte loads, eight in
 * flight a lane, over up to 16,384 workgroups of 256 threads (the streaming
 * pattern of the build and the gather).  nontemporal != 0 marks the loads as
 * streaming.  Nothing is written except, when the XOR of all the data
 * equals 0x9e3779b9, that value to sink[0] (which keeps the loads live).
 * Reading a buffer larger than the caches also empties them of everything
 * else without leaving dirty lines, which is how the benchmark prepares its
 * cold-cache timings.  buf: device, 16-byte aligned, bytes a positive
 * multiple of 16; sink: device, 4 bytes.  TIS_E_NULL / TIS_E_ALIGN /
 * TIS_E_SHAPE otherwise. */
tis_status tis_probe_read(const void *buf, size_t bytes, int nontemporal, uint32_t *sink,
                          void *stream);

/* One lane follows the chain i = next[i] for `hops` steps from `start` (an
 * index at or past n_elems restarts the chain at 0, so every load stays in
 * the buffer) and writes the last index to out[0].  Timed against hops = 0,
 * it gives the latency of one dependent load to wherever the chain's
 * footprint lives.  next: device uint32 [n_elems], n_elems >= 1; out: device,
 * 4 bytes; 0 <= hops.  TIS_E_NULL / TIS_E_SHAPE otherwise. */
tis_status tis_probe_chase(const uint32_t *next, size_t n_elems, uint32_t start, int hops,
                           uint32_t *out, void *stream);

/* Bytes of the timeline tis_probe_decode_timeline writes for this shape
 * (one 24-slot record per wave of every workgroup; 0 for invalid sizes). */
size_t tis_probe_decode_timeline_bytes(int batch, int q_heads, int beam, int leaf_block);

/* tis_tree_decode (same arguments, same results in O, indices not written)
 * run by an instrumented copy of its kernel that also records where each
 * workgroup's time goes: the descent level by level and the gather that
 * follows it ("Subquadratic Attention with a Hierarchical Tree-Structured
 * Indexer", Abstract: a query's cost is its descent plus the attention at
 * the end).  A measurement, not a path of its own.
 *
 * timeline: device uint64, 8-byte aligned, at least
 * tis_probe_decode_timeline_bytes() bytes, laid out
 * [workgroup][16 waves][24 slots]; workgroup g = part * (batch * q_heads) +
 * slot of a query (a query with several parts has several workgroups).
 * Slot k of a wave receives the GPU's constant-rate wall clock (ticks of
 * hipDeviceAttributeWallClockRate kHz) when the wave's first lane passed
 * phase k: 0 entry; 1 descent done; 2 its first K load about to issue; 3 that
 * unit's keys loaded and scored; 4 its values used; 5 all its units done;
 * 6 the workgroup's partial states merged (barrier passed); 7 end; 8 + 2j
 * its rows of scored level j done, 9 + 2j level j ranked (j < 8, counted
 * from the first level that cuts).  Slots a wave does not pass keep their
 * old contents, so clear the buffer first.  Float32 or bfloat16 summaries
 * (TIS_E_UNSUPPORTED for fp8); TIS_E_NULL without a timeline, TIS_E_ALIGN,
 * TIS_E_WORKSPACE when it is too small; every tis_tree_decode check
 * applies. */
tis_status tis_probe_decode_timeline(const void *Q, const void *K, const void *V,
                                     tis_dtype dtype, int q_heads, const tis_tree *tree, int beam,
                                     float scale, float *O, void *workspace,
                                     size_t workspace_bytes, uint64_t *timeline,
                                     size_t timeline_bytes, void *stream);

/* The GPU's wall-clock rate in kHz (the clock of the decode timeline), or 0
 * if the device cannot be queried. */
int tis_wall_clock_khz(int device);

/* Message for the last non-OK status returned on the calling thread. */
const char *tis_last_error(void);

/* Library version string, e.g. "tis 0.1.0 gfx950". */
const char *tis_version(void);

/* ------------------------------------------------------------------------
 * Tree over a growing KV cache
 *
 * The ZHA abstract describes the index as living over the KV cache and
 * growing deeper step by step as the context lengthens; decode appends keys
 * one step at a time (ALHR post).  These calls keep a tree over the first
 * n_keys rows of a cache that has room for `capacity` keys per head:
 *   - depth: the fewest levels lv >= 1 with b^lv * L >= n_keys, so the tree
 *     gains a level exactly when n_keys first exceeds b^lv * L;
 *   - node n of level l covers keys [n*M_l, (n+1)*M_l) cut at n_keys, with
 *     M_l = b^(lv-l) * L, and exists when that range is not empty (leaf j
 *     holds keys [j*L, min((j+1)*L, n_keys)));
 *   - summary = the exact mean of the keys the node covers, rounded once to
 *     float32 (as for the full tree);
 *   - route: each level scores the existing children of the nodes kept
 *     above and keeps the best min(beam, their number), (score desc, node
 *     index asc); attention runs over the keys of the kept leaves.
 * With n_keys = b^lv * L these are the full-tree definitions exactly.
 *
 * Storage (caller-owned device memory, sized by the two queries below):
 *   K, V       [B][Hkv][capacity][d], element type dtype; rows past n_keys
 *              are never read
 *   summaries  summary_dtype (float32 or bfloat16, as for tis_tree),
 *              height-major so that no level moves when the tree
 *              deepens: for height h = 0 (leaves) .. H-1 a block
 *              [B][Hkv][ceil(capacity / (L*b^h))][d], where H is the depth
 *              of a full cache; level l of a tree of depth lv lives at
 *              height lv - l, node n at row n of its (batch, head) block
 *   state      float64 [2][B][Hkv][H][d], two halves of which state_half
 *              names the one in use: for every height h, the exact sum of
 *              the keys of the node that holds key n_keys (the open node;
 *              zero when n_keys is a multiple of L*b^h).  Appends start from
 *              it, which keeps every summary an exact mean rounded once.
 *              A short tis_cache_tree_append updates the half in use in
 *              place; a long one and tis_cache_tree_append_decode write the
 *              other half and switch to it (their workgroups read the old
 *              sums while others write the new ones).  After the two halves
 *              comes the library's scratch for long appends (a float64 row
 *              of d per (batch, KV head, chunk of the cache)).
 * Summaries are kept for every height up to H-1 whatever the current depth,
 * so a deeper tree finds its upper levels already in place.
 * --------------------------------------------------------------------- */

typedef struct tis_cache_tree {
  int32_t batch, kv_heads, head_dim, branching, leaf_block;
  int32_t capacity;  /* keys per (batch, KV head) the cache has room for     */
  int32_t n_keys;    /* keys in the tree: set by reset (0) and the appends   */
  int32_t levels;    /* depth over n_keys (0 while empty): set by the library */
  int32_t summary_dtype; /* tis_dtype of the stored summaries (as tis_tree)  */
  int32_t state_half; /* half of `state` in use (0 or 1): set by the library */
  void *summaries;   /* tis_cache_tree_summary_bytes_as() bytes              */
  double *state;     /* tis_cache_tree_state_bytes() bytes                   */
} tis_cache_tree;

/* Bytes of the summaries / state buffers of a cache with this geometry
 * (d 64 or 128, b >= 2, L >= 1, capacity >= 1, the full-cache depth H at
 * most 16); 0 if invalid or overflowing. */
size_t tis_cache_tree_summary_bytes(int batch, int kv_heads, int head_dim, int branching,
                                    int leaf_block, int capacity);
/* Summary bytes for summaries stored as summary_dtype (0 if unknown). */
size_t tis_cache_tree_summary_bytes_as(int batch, int kv_heads, int head_dim, int branching,
                                       int leaf_block, int capacity, tis_dtype summary_dtype);
size_t tis_cache_tree_state_bytes(int batch, int kv_heads, int head_dim, int branching,
                                  int leaf_block, int capacity);

/* Empties the tree: n_keys = levels = state_half = 0 and both state
 * halves zeroed (by a kernel on `stream`).  The caller fills in the geometry fields and both pointers
 * first.  Summaries need no clearing: only existing nodes are ever read. */
tis_status tis_cache_tree_reset(tis_cache_tree *tree, void *stream);

/* Adds keys [n_keys, n_keys + n_new) of K (already written to the cache) to
 * the tree, then sets n_keys += n_new and levels to the new depth (host-side
 * fields, updated when the work is enqueued).  Rewrites the summary of every
 * node that gains a key, at every height, and the state; O(n_new * d + H * d
 * * (leaves touched)) work.  Short appends run one workgroup per (batch, KV
 * head); an append of at least one chunk (the nodes of the smallest height
 * with 512 or more keys, at most 64 leaves) runs a workgroup per (head,
 * chunk), then one per head for the heights above the chunks.
 * Requires 0 <= n_new <= capacity - n_keys.  n_new = 0 does nothing. */
tis_status tis_cache_tree_append(const void *K, tis_dtype dtype, int n_new,
                                 tis_cache_tree *tree, void *stream);

/* tis_tree_route over the tree of a cache (n_keys >= 1).  indices [B][Hq]
 * [beam]: the kept leaves ascending, padded with -1 when the tree has fewer
 * than beam leaves; trace (optional) [B][Hq][levels][beam] as for
 * tis_tree_route.  Requires beam >= 1 and beam * b <= TIS_MAX_CANDIDATES. */
tis_status tis_cache_tree_route(const void *Q, tis_dtype dtype, int q_heads,
                                const tis_cache_tree *tree, int beam, int32_t *indices,
                                int32_t *trace, void *stream);

/* tis_tree_decode over the tree of a cache: route and attend in one launch,
 * O [B][Hq][d] float32, indices optional as for tis_cache_tree_route.
 * workspace: tis_decode_workspace_bytes(batch, q_heads, head_dim, beam,
 * leaf_block) bytes, as for tis_tree_decode. */
tis_status tis_cache_tree_decode(const void *Q, const void *K, const void *V, tis_dtype dtype,
                                 int q_heads, const tis_cache_tree *tree, int beam, float scale,
                                 float *O, int32_t *indices, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* One decode step of a growing cache (ZHA Abstract: the tree grows with the
 * context; ALHR Summary: one key arrives per decoded token): adds key n_keys
 * (row n_keys of K and V, already written by the caller, for every batch
 * and KV head) to the tree and decodes Q over the tree of n_keys + 1 keys,
 * in one launch (two when the decode splits its queries).  Results, the
 * summaries and the state left behind are those of
 * tis_cache_tree_append(K, dtype, 1, tree) followed by
 * tis_cache_tree_decode(...), bit for bit; n_keys, levels and state_half are
 * updated when the work is enqueued.  Arguments as for tis_cache_tree_decode;
 * requires n_keys < capacity (TIS_E_SHAPE otherwise, nothing launched).
 * Only the node that holds the new key changes at each height, so every
 * workgroup computes that node's new mean from the state and the key and
 * reads every other node as stored. */
tis_status tis_cache_tree_append_decode(const void *Q, const void *K, const void *V,
                                        tis_dtype dtype, int q_heads, tis_cache_tree *tree,
                                        int beam, float scale, float *O, int32_t *indices,
                                        void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Causal prefill routing
 *
 * The ALHR post (Summary) counts the keys a query reads averaged over the
 * positions of a 1,024-token input: every position is a query over the
 * keys up to it.  Here the query at position t routes over the tree of the
 * first t + 1 keys -- the growing-cache tree at n_keys = t + 1, with its
 * depth, nodes cut at t + 1 and means over the keys they hold -- and attends
 * over the keys of its kept leaf blocks up to t.  The nodes left of key t are
 * the ones a tree over all n_keys keys stores; the node holding key t at
 * each height (partial for t) gets its mean from a table the call computes
 * first.
 * --------------------------------------------------------------------- */

/* Bytes of the workspace tis_causal_prefill needs (0 if invalid), for a
 * tree of n_keys keys, q_heads query heads, the beam and the key type:
 *  - the partial means, B * Hkv * n_keys * depth(n_keys) * d elements of
 *    the summary type;
 *  - fp64 key sums, B * Hkv * d doubles for every run of 64 keys, every run
 *    of 64^2 keys (past 64^2 keys), of 64^3 (past 64^3), and so on: runs of
 *    64^(k+1) are kept while 64^(k+1) < n_keys, and the runs of 64 always;
 *  - when leaf_block is a multiple of 16 and at least 32 (the attention
 *    then takes 16 positions at a time on the matrix cores, if its LDS fits
 *    the beam: beam <= 87 always does), at 256-byte offsets: the
 *    kept leaves, int32 [B][Hq][n_keys][beam], and V transposed per 16 keys,
 *    B * Hkv * ceil(n_keys / 16) * 16 * d elements of the key type. */
size_t tis_causal_prefill_workspace_bytes(int batch, int kv_heads, int q_heads, int head_dim,
                                          int branching, int leaf_block, int n_keys, int beam,
                                          tis_dtype dtype, tis_dtype summary_dtype);

/*
 * tis_causal_prefill -- every position of the first tree->n_keys keys of a
 * cache as a query over its own prefix.
 * tree     a growing-cache tree holding those keys (tis_cache_tree_append),
 *          n_keys >= 1; K, V the cache it was built over.
 * Q        [B][Hq][n_keys][d] of type dtype: the query of every position.
 * O        out: float32 [B][Hq][n_keys][d].
 * indices  optional: int32 [B][Hq][n_keys][beam], each position's kept
 *          leaves ascending, -1 padded where its tree has fewer leaves.
 * workspace: tis_causal_prefill_workspace_bytes() bytes, 16-byte aligned.
 * Requires beam >= 1, beam * b <= TIS_MAX_CANDIDATES and
 * B * Hq * n_keys < 2^31.
 */
tis_status tis_causal_prefill(const void *Q, const void *K, const void *V, tis_dtype dtype,
                              int q_heads, const tis_cache_tree *tree, int beam, float scale,
                              float *O, int32_t *indices, void *workspace, size_t workspace_bytes,
                              void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TIS_H_ */
