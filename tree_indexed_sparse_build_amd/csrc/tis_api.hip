// C-ABI of libtis: argument checks, launch geometry and error mapping.
// Every check runs on the host before anything is enqueued, so a call that
// fails a check touches neither the device nor the HIP runtime.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "tis.h"
#include "tis_internal.hpp"

namespace {

thread_local char g_err[512] = "";

tis_status fail(tis_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// b^e with overflow detection (limit: INT32 range).
bool ipow(int64_t b, int e, int64_t *out) {
  int64_t r = 1;
  for (int i = 0; i < e; ++i) {
    r *= b;
    if (r > 0x7fffffffLL) return false;
  }
  *out = r;
  return true;
}

struct Geometry {
  int64_t n_at[tis::kMaxLevels + 1];
  int64_t summ_off[tis::kMaxLevels + 1];
  int64_t summ_elems;
};

// Checks the tree geometry shared by build and route and fills level sizes.
tis_status check_tree(int batch, int kv_heads, int n_keys, int head_dim, int branching,
                      int leaf_block, int levels, Geometry *g) {
  if (batch < 1 || kv_heads < 1) return fail(TIS_E_SHAPE, "batch and kv_heads must be >= 1");
  if (head_dim != 64 && head_dim != 128)
    return fail(head_dim < 1 ? TIS_E_SHAPE : TIS_E_UNSUPPORTED,
                "head_dim %d: only 64 and 128 are compiled", head_dim);
  if (branching < 2) return fail(TIS_E_SHAPE, "branching %d < 2", branching);
  if (branching > tis::kMaxBranching)
    return fail(TIS_E_UNSUPPORTED, "branching %d > %d", branching, tis::kMaxBranching);
  if (levels < 1) return fail(TIS_E_SHAPE, "levels %d < 1", levels);
  if (levels > tis::kMaxLevels)
    return fail(TIS_E_UNSUPPORTED, "levels %d > %d", levels, tis::kMaxLevels);
  if (leaf_block < 1) return fail(TIS_E_SHAPE, "leaf_block %d < 1", leaf_block);
  int64_t leaves;
  if (!ipow(branching, levels, &leaves) || leaves * leaf_block != static_cast<int64_t>(n_keys))
    return fail(TIS_E_SHAPE, "n_keys %d != branching^levels * leaf_block (%d^%d * %d)", n_keys,
                branching, levels, leaf_block);
  const int64_t heads = static_cast<int64_t>(batch) * kv_heads;
  int64_t off = 0;
  g->n_at[0] = 1;
  g->summ_off[0] = 0;
  for (int l = 1; l <= levels; ++l) {
    g->n_at[l] = g->n_at[l - 1] * branching;
    g->summ_off[l] = off;
    off += heads * g->n_at[l] * head_dim;
  }
  for (int l = levels + 1; l <= tis::kMaxLevels; ++l) g->n_at[l] = g->summ_off[l] = 0;
  g->summ_elems = off;
  return TIS_OK;
}

tis_status check_dtype(tis_dtype dt) {
  if (dt != TIS_F32 && dt != TIS_BF16) return fail(TIS_E_DTYPE, "unknown dtype %d", (int)dt);
  return TIS_OK;
}

// The stored type of a tree's summaries (a field the caller sets).
tis_status check_summary_dtype(const char *who, int32_t sd) {
  if (sd != TIS_F32 && sd != TIS_BF16 && sd != TIS_FP8_E4M3)
    return fail(TIS_E_DTYPE, "%s: unknown summary_dtype %d", who, (int)sd);
  return TIS_OK;
}

// Calls built for float32 and bfloat16 summaries only (fp8 summaries serve
// the full tree's build, route and decode).
tis_status check_summary_dtype_no_fp8(const char *who, int32_t sd) {
  tis_status st = check_summary_dtype(who, sd);
  if (st == TIS_OK && sd == TIS_FP8_E4M3)
    return fail(TIS_E_UNSUPPORTED, "%s: fp8 summaries serve tis_tree_build / route / decode only",
                who);
  return st;
}

tis::Dt to_dt(int32_t d) {
  return d == TIS_BF16 ? tis::Dt::BF16 : d == TIS_FP8_E4M3 ? tis::Dt::FP8 : tis::Dt::F32;
}

size_t summary_elem_bytes(int32_t sd) { return sd == TIS_BF16 ? 2 : sd == TIS_FP8_E4M3 ? 1 : 4; }

// fp8 summaries: the codes (level-major, one byte an element) come first,
// then, 16-byte aligned, one float32 power-of-two scale per node.
size_t fp8_scales_offset(int64_t nodes, int head_dim) {
  return tis::align_up(static_cast<size_t>(nodes) * head_dim, 16);
}

tis_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return TIS_OK;
  return fail(TIS_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Route arguments of a checked tree; queries < 2^31 is checked by the caller.
tis::RouteArgs route_args(const void *Q, const tis_tree *tree, const Geometry &g, int q_heads,
                          int beam, int32_t *indices, int32_t *trace, int64_t queries) {
  tis::RouteArgs a{};
  a.Q = Q;
  a.summ = tree->summaries;
  a.indices = indices;
  a.trace = trace;
  a.queries = static_cast<int>(queries);
  a.q_heads = q_heads;
  a.kv_heads = tree->kv_heads;
  a.group = q_heads / tree->kv_heads;
  a.branching = tree->branching;
  a.levels = tree->levels;
  a.beam = beam;
  a.first_cut = 1;
  while (a.first_cut < tree->levels && g.n_at[a.first_cut] <= beam) ++a.first_cut;
  if (tree->summary_dtype == TIS_FP8_E4M3)
    a.scales = reinterpret_cast<const float *>(
        static_cast<const char *>(tree->summaries) +
        fp8_scales_offset(g.summ_elems / tree->head_dim, tree->head_dim));
  return a;
}

}  // namespace

extern "C" {

size_t tis_tree_summary_bytes(int batch, int kv_heads, int head_dim, int branching, int levels) {
  return tis_tree_summary_bytes_as(batch, kv_heads, head_dim, branching, levels, TIS_F32);
}

size_t tis_tree_summary_bytes_as(int batch, int kv_heads, int head_dim, int branching, int levels,
                                 tis_dtype summary_dtype) {
  if (batch < 1 || kv_heads < 1 || head_dim < 1 || branching < 2 || levels < 1 ||
      levels > tis::kMaxLevels ||
      (summary_dtype != TIS_F32 && summary_dtype != TIS_BF16 && summary_dtype != TIS_FP8_E4M3))
    return 0;
  const size_t es = summary_elem_bytes(summary_dtype);
  int64_t n = 1, total = 0;
  for (int l = 1; l <= levels; ++l) {
    n *= branching;
    if (n > 0x7fffffffLL) return 0;
    total += n;
  }
  const double bytes = 4.0 * head_dim * (double)batch * kv_heads * (double)total;
  if (bytes > 9.0e18) return 0;
  const int64_t nodes = static_cast<int64_t>(batch) * kv_heads * total;
  if (summary_dtype == TIS_FP8_E4M3)
    return fp8_scales_offset(nodes, head_dim) + static_cast<size_t>(nodes) * sizeof(float);
  return es * head_dim * static_cast<size_t>(nodes);
}

size_t tis_build_workspace_bytes(int batch, int kv_heads, int n_keys, int head_dim,
                                 int branching, int leaf_block, int levels) {
  Geometry g;
  char saved[sizeof g_err];
  memcpy(saved, g_err, sizeof saved);
  const tis_status st =
      check_tree(batch, kv_heads, n_keys, head_dim, branching, leaf_block, levels, &g);
  memcpy(g_err, saved, sizeof saved);
  if (st != TIS_OK) return 0;
  tis::BuildPlan p;
  if (!tis::plan_build(static_cast<int64_t>(batch) * kv_heads, head_dim, branching, leaf_block,
                       levels, &p))
    return 0;
  return p.workspace_bytes;
}

tis_status tis_tree_build(const void *K, tis_dtype dtype, int batch, int kv_heads, int n_keys,
                          int head_dim, int branching, int leaf_block, int levels, tis_tree *tree,
                          void *workspace, size_t workspace_bytes, void *stream) {
  if (!K || !tree || !tree->summaries)
    return fail(TIS_E_NULL, "tis_tree_build: K, tree and tree->summaries are required");
  tis_status st = check_dtype(dtype);
  if (st != TIS_OK) return st;
  st = check_summary_dtype("tis_tree_build", tree->summary_dtype);
  if (st != TIS_OK) return st;
  Geometry g;
  st = check_tree(batch, kv_heads, n_keys, head_dim, branching, leaf_block, levels, &g);
  if (st != TIS_OK) return st;
  if (!aligned(K, 16) || !aligned(tree->summaries, 16) || !aligned(workspace, 16))
    return fail(TIS_E_ALIGN, "tis_tree_build: K, summaries and workspace must be 16-byte aligned");
  const int64_t heads = static_cast<int64_t>(batch) * kv_heads;
  tis::BuildPlan p;
  if (!tis::plan_build(heads, head_dim, branching, leaf_block, levels, &p))
    return fail(TIS_E_UNSUPPORTED, "tis_tree_build: grid too large");
  if (p.workspace_bytes > 0 && (!workspace || workspace_bytes < p.workspace_bytes))
    return fail(workspace ? TIS_E_WORKSPACE : TIS_E_NULL,
                "tis_tree_build: workspace of %zu bytes required, %zu given", p.workspace_bytes,
                workspace ? workspace_bytes : (size_t)0);

  tis::BuildArgs a{};
  a.K = K;
  a.summ = tree->summaries;
  if (tree->summary_dtype == TIS_FP8_E4M3)
    a.scales = reinterpret_cast<float *>(static_cast<char *>(tree->summaries) +
                                         fp8_scales_offset(g.summ_elems / head_dim, head_dim));
  // the arrival counters of the level-1 subtrees, then the fp64 node sums
  a.arrive = p.workspace_bytes > 0 ? static_cast<unsigned *>(workspace) : nullptr;
  a.ws_sum = p.workspace_bytes > 0
                 ? reinterpret_cast<double *>(static_cast<char *>(workspace) + tis::kBuildArriveBytes)
                 : nullptr;
  a.n_keys = n_keys;
  a.chunks = p.chunks;
  a.branching = branching;
  a.leaf_block = leaf_block;
  a.levels = levels;
  a.root_level = p.root_level;
  a.wave_depth = p.wave_depth;
  a.through_stores = 1;  // K is streamed once, whatever its size
  a.top_rows = 1;
  for (int l = 2; l < p.root_level; ++l) a.top_rows *= branching;
  a.chunks_per_l1 = 1;
  for (int l = 2; l <= p.root_level; ++l) a.chunks_per_l1 *= branching;
  a.wave_leaves = 1;
  for (int i = 0; i < p.wave_depth; ++i) a.wave_leaves *= branching;
  a.pow2_levels = 0;
  int64_t sum_off = 0;
  for (int l = 0; l <= tis::kMaxLevels; ++l) {
    a.n_at[l] = g.n_at[l];
    a.chunks_at_level[l] = heads * g.n_at[l];
    a.summ_off[l] = g.summ_off[l];
    a.ws_off[l] = 0;
    a.mean_div[l] = a.mean_inv[l] = 1.0;
    if (l >= 1 && l <= levels) {
      const int64_t M = static_cast<int64_t>(n_keys) / g.n_at[l];
      a.mean_div[l] = static_cast<double>(M);
      if ((M & (M - 1)) == 0) {
        a.pow2_levels |= 1u << l;
        a.mean_inv[l] = 1.0 / static_cast<double>(M);
      }
    }
  }
  for (int l = 2; l <= p.root_level; ++l) {
    a.ws_off[l] = sum_off;
    sum_off += heads * g.n_at[l] * head_dim;
  }
  const tis::Dt dt = dtype == TIS_BF16 ? tis::Dt::BF16 : tis::Dt::F32;
  st = hip_status(tis::launch_build(dt, to_dt(tree->summary_dtype), head_dim, heads, a, p,
                                    static_cast<hipStream_t>(stream)),
                  "tis_tree_build launch");
  if (st != TIS_OK) return st;
  tree->batch = batch;
  tree->kv_heads = kv_heads;
  tree->n_keys = n_keys;
  tree->head_dim = head_dim;
  tree->branching = branching;
  tree->leaf_block = leaf_block;
  tree->levels = levels;
  return TIS_OK;
}

tis_status tis_tree_route(const void *Q, tis_dtype dtype, int q_heads, const tis_tree *tree,
                          int beam, int32_t *indices, int32_t *trace, void *stream) {
  if (!Q || !tree || !tree->summaries || !indices)
    return fail(TIS_E_NULL, "tis_tree_route: Q, tree, tree->summaries and indices are required");
  tis_status st = check_dtype(dtype);
  if (st != TIS_OK) return st;
  st = check_summary_dtype("tis_tree_route", tree->summary_dtype);
  if (st != TIS_OK) return st;
  Geometry g;
  st = check_tree(tree->batch, tree->kv_heads, tree->n_keys, tree->head_dim, tree->branching,
                  tree->leaf_block, tree->levels, &g);
  if (st != TIS_OK) return st;
  if (q_heads < 1 || q_heads % tree->kv_heads != 0)
    return fail(TIS_E_SHAPE, "tis_tree_route: q_heads %d is not a positive multiple of kv_heads %d",
                q_heads, tree->kv_heads);
  const int64_t leaves = g.n_at[tree->levels];
  if (beam < 1 || beam > leaves)
    return fail(TIS_E_SHAPE, "tis_tree_route: beam %d outside [1, %lld]", beam, (long long)leaves);
  if (static_cast<int64_t>(beam) * tree->branching > TIS_MAX_CANDIDATES)
    return fail(TIS_E_UNSUPPORTED, "tis_tree_route: beam * branching = %lld > %d",
                (long long)beam * tree->branching, TIS_MAX_CANDIDATES);
  if (!aligned(Q, 16) || !aligned(tree->summaries, 16) || !aligned(indices, 4) ||
      (trace && !aligned(trace, 4)))
    return fail(TIS_E_ALIGN, "tis_tree_route: Q and summaries need 16-byte, indices 4-byte alignment");
  const int64_t queries = static_cast<int64_t>(tree->batch) * q_heads;
  if (queries > 0x7fffffffLL) return fail(TIS_E_UNSUPPORTED, "tis_tree_route: too many queries");

  const tis::RouteArgs a = route_args(Q, tree, g, q_heads, beam, indices, trace, queries);
  const tis::Dt dt = dtype == TIS_BF16 ? tis::Dt::BF16 : tis::Dt::F32;
  return hip_status(tis::launch_route(dt, to_dt(tree->summary_dtype), tree->head_dim, a,
                                     static_cast<hipStream_t>(stream)),
                    "tis_tree_route launch");
}

size_t tis_attend_workspace_bytes(int batch, int q_heads, int head_dim, int beam, int leaf_block) {
  if (batch < 1 || q_heads < 1 || (head_dim != 64 && head_dim != 128) || beam < 1 ||
      leaf_block < 1)
    return 0;
  const int64_t queries = static_cast<int64_t>(batch) * q_heads;
  return tis::attend_workspace(queries, head_dim, tis::attend_splits(queries, beam, leaf_block));
}

size_t tis_decode_workspace_bytes(int batch, int q_heads, int head_dim, int beam, int leaf_block) {
  return tis_attend_workspace_bytes(batch, q_heads, head_dim, beam, leaf_block);
}

// Splits and workspace of an attend or decode call; fails without enqueuing.
static tis_status plan_split(const char *who, int64_t queries, int head_dim, int beam,
                             int leaf_block, void *workspace, size_t workspace_bytes,
                             tis::AttendArgs *a) {
  a->splits = tis::attend_splits(queries, beam, leaf_block);
  a->part = nullptr;
  a->arrive = nullptr;
  const size_t need = tis::attend_workspace(queries, head_dim, a->splits);
  if (need == 0) return TIS_OK;
  if (!workspace)
    return fail(TIS_E_NULL, "%s: a workspace of %zu bytes is required", who, need);
  if (!aligned(workspace, 16))
    return fail(TIS_E_ALIGN, "%s: workspace must be 16-byte aligned", who);
  if (workspace_bytes < need)
    return fail(TIS_E_WORKSPACE, "%s: workspace %zu bytes < %zu required", who, workspace_bytes,
                need);
  a->arrive = static_cast<unsigned *>(workspace);
  a->part = reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + tis::kArriveBytes);
  return TIS_OK;
}

tis_status tis_tree_attend(const void *Q, const void *K, const void *V, tis_dtype dtype, int batch,
                           int q_heads, int kv_heads, int n_keys, int head_dim, int leaf_block,
                           const int32_t *indices, int beam, float scale, float *O,
                           void *workspace, size_t workspace_bytes, void *stream) {
  if (!Q || !K || !V || !indices || !O)
    return fail(TIS_E_NULL, "tis_tree_attend: Q, K, V, indices and O are required");
  tis_status st = check_dtype(dtype);
  if (st != TIS_OK) return st;
  if (batch < 1 || kv_heads < 1 || q_heads < 1 || q_heads % kv_heads != 0)
    return fail(TIS_E_SHAPE, "tis_tree_attend: need batch, kv_heads >= 1 and q_heads a multiple of kv_heads");
  if (head_dim != 64 && head_dim != 128)
    return fail(head_dim < 1 ? TIS_E_SHAPE : TIS_E_UNSUPPORTED,
                "tis_tree_attend: head_dim %d: only 64 and 128 are compiled", head_dim);
  if (leaf_block < 1 || n_keys < 1 || n_keys % leaf_block != 0)
    return fail(TIS_E_SHAPE, "tis_tree_attend: n_keys %d is not a positive multiple of leaf_block %d",
                n_keys, leaf_block);
  if (beam < 1) return fail(TIS_E_SHAPE, "tis_tree_attend: beam %d < 1", beam);
  if (beam > TIS_MAX_CANDIDATES)
    return fail(TIS_E_UNSUPPORTED, "tis_tree_attend: beam %d > %d", beam, TIS_MAX_CANDIDATES);
  if (!(scale == scale) || isinf(scale))
    return fail(TIS_E_SHAPE, "tis_tree_attend: scale must be finite");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
      !aligned(indices, 4))
    return fail(TIS_E_ALIGN, "tis_tree_attend: Q, K, V and O need 16-byte alignment, indices 4-byte");
  const int64_t queries = static_cast<int64_t>(batch) * q_heads;
  if (queries > 0x7fffffffLL) return fail(TIS_E_UNSUPPORTED, "tis_tree_attend: too many queries");

  const double sc = scale > 0.f ? static_cast<double>(scale) : 1.0 / sqrt(static_cast<double>(head_dim));
  tis::AttendArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.indices = indices;
  a.O = O;
  a.queries = static_cast<int>(queries);
  a.n_keys = n_keys;
  a.key_stride = n_keys;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.group = q_heads / kv_heads;
  a.leaf_block = leaf_block;
  a.beam = beam;
  a.n_blocks = n_keys / leaf_block;
  a.scale_log2 = static_cast<float>(sc * 1.4426950408889634);
  st = plan_split("tis_tree_attend", queries, head_dim, beam, leaf_block, workspace,
                  workspace_bytes, &a);
  if (st != TIS_OK) return st;
  const tis::Dt dt = dtype == TIS_BF16 ? tis::Dt::BF16 : tis::Dt::F32;
  return hip_status(tis::launch_attend(dt, head_dim, a, static_cast<hipStream_t>(stream)),
                    "tis_tree_attend launch");
}

size_t tis_attend_grouped_workspace_bytes(int batch, int q_heads, int kv_heads, int head_dim,
                                          int beam) {
  if (batch < 1 || kv_heads < 1 || q_heads < 1 || q_heads % kv_heads != 0 ||
      (head_dim != 64 && head_dim != 128) || beam < 1)
    return 0;
  const int group = q_heads / kv_heads;
  const int64_t groups = static_cast<int64_t>(batch) * kv_heads;
  return tis::attend_group_workspace(groups, group, head_dim,
                                     tis::attend_group_splits(groups, group, beam));
}

tis_status tis_tree_attend_grouped(const void *Q, const void *K, const void *V, tis_dtype dtype,
                                   int batch, int q_heads, int kv_heads, int n_keys,
                                   int head_dim, int leaf_block, const int32_t *indices,
                                   int beam, float scale, float *O, void *workspace,
                                   size_t workspace_bytes, void *stream) {
  const char *who = "tis_tree_attend_grouped";
  if (!Q || !K || !V || !indices || !O)
    return fail(TIS_E_NULL, "%s: Q, K, V, indices and O are required", who);
  tis_status st = check_dtype(dtype);
  if (st != TIS_OK) return st;
  if (batch < 1 || kv_heads < 1 || q_heads < 1 || q_heads % kv_heads != 0)
    return fail(TIS_E_SHAPE, "%s: need batch, kv_heads >= 1 and q_heads a multiple of kv_heads",
                who);
  if (head_dim != 64 && head_dim != 128)
    return fail(head_dim < 1 ? TIS_E_SHAPE : TIS_E_UNSUPPORTED,
                "%s: head_dim %d: only 64 and 128 are compiled", who, head_dim);
  if (leaf_block < 1 || n_keys < 1 || n_keys % leaf_block != 0)
    return fail(TIS_E_SHAPE, "%s: n_keys %d is not a positive multiple of leaf_block %d", who,
                n_keys, leaf_block);
  if (beam < 1) return fail(TIS_E_SHAPE, "%s: beam %d < 1", who, beam);
  const int group = q_heads / kv_heads;
  if (group > tis::kGroupMaxHeads || group * static_cast<int64_t>(beam) > tis::kGroupMaxEntries)
    return fail(TIS_E_UNSUPPORTED, "%s: %d heads per KV head x beam %d: at most %d heads and %d slots per group",
                who, group, beam, tis::kGroupMaxHeads, tis::kGroupMaxEntries);
  if (!(scale == scale) || isinf(scale)) return fail(TIS_E_SHAPE, "%s: scale must be finite", who);
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
      !aligned(indices, 4))
    return fail(TIS_E_ALIGN, "%s: Q, K, V and O need 16-byte alignment, indices 4-byte", who);
  const int64_t queries = static_cast<int64_t>(batch) * q_heads;
  if (queries > 0x7fffffffLL) return fail(TIS_E_UNSUPPORTED, "%s: too many queries", who);

  const double sc = scale > 0.f ? static_cast<double>(scale) : 1.0 / sqrt(static_cast<double>(head_dim));
  tis::AttendArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.indices = indices;
  a.O = O;
  a.queries = static_cast<int>(queries);
  a.n_keys = n_keys;
  a.key_stride = n_keys;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.group = group;
  a.leaf_block = leaf_block;
  a.beam = beam;
  a.n_blocks = n_keys / leaf_block;
  a.scale_log2 = static_cast<float>(sc * 1.4426950408889634);
  const int64_t groups = static_cast<int64_t>(batch) * kv_heads;
  a.splits = tis::attend_group_splits(groups, group, beam);
  const size_t need = tis::attend_group_workspace(groups, group, head_dim, a.splits);
  if (need > 0) {
    if (!workspace) return fail(TIS_E_NULL, "%s: a workspace of %zu bytes is required", who, need);
    if (!aligned(workspace, 16)) return fail(TIS_E_ALIGN, "%s: workspace must be 16-byte aligned", who);
    if (workspace_bytes < need)
      return fail(TIS_E_WORKSPACE, "%s: workspace %zu bytes < %zu required", who, workspace_bytes,
                  need);
    a.arrive = static_cast<unsigned *>(workspace);
    a.part = reinterpret_cast<float *>(static_cast<unsigned char *>(workspace) + tis::kArriveBytes);
  }
  const tis::Dt dt = dtype == TIS_BF16 ? tis::Dt::BF16 : tis::Dt::F32;
  return hip_status(tis::launch_attend_group(dt, head_dim, a, static_cast<hipStream_t>(stream)),
                    "tis_tree_attend_grouped launch");
}

}  // extern "C"

namespace {

// Scratch of tis_tree_decode_noalloc: the split queries' partial softmax
// states, which tis_tree_decode keeps in the caller's workspace.  Every GPU
// the library runs on holds its own copy (part of the code object loaded
// there) until the process ends.  Host code never passes the array's name to
// a kernel: on the host it only stands for the symbol, and the device
// address comes from hipGetSymbolAddress, looked up once per device.
static __device__ __align__(256) unsigned char scratch[TIS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxScratchDevices];

// Device address of `scratch` on the current device.
tis_status scratch_address(const char *who, void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, who);
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(TIS_E_UNSUPPORTED, "%s: device %d is past the %d the library serves", who, dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, who);
    if (!p || !aligned(p, 256))
      return fail(TIS_E_HIP, "%s: no usable address for the library's scratch", who);
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return TIS_OK;
}

// tis_tree_decode, with the split partial states in the caller's workspace
// or (noalloc) in the library's per-device scratch.
tis_status decode_full_tree(const char *who, const void *Q, const void *K, const void *V,
                            tis_dtype dtype, int q_heads, const tis_tree *tree, int beam,
                            float scale, float *O, int32_t *indices, void *workspace,
                            size_t workspace_bytes, bool noalloc, void *stream,
                            unsigned long long *timeline = nullptr,
                            size_t timeline_bytes = 0) {
  if (!Q || !K || !V || !tree || !tree->summaries || !O)
    return fail(TIS_E_NULL, "%s: Q, K, V, tree, tree->summaries and O are required", who);
  tis_status st = check_dtype(dtype);
  if (st != TIS_OK) return st;
  st = check_summary_dtype(who, tree->summary_dtype);
  if (st != TIS_OK) return st;
  Geometry g;
  st = check_tree(tree->batch, tree->kv_heads, tree->n_keys, tree->head_dim, tree->branching,
                  tree->leaf_block, tree->levels, &g);
  if (st != TIS_OK) return st;
  if (q_heads < 1 || q_heads % tree->kv_heads != 0)
    return fail(TIS_E_SHAPE, "%s: q_heads %d is not a positive multiple of kv_heads %d",
                who, q_heads, tree->kv_heads);
  const int64_t leaves = g.n_at[tree->levels];
  if (beam < 1 || beam > leaves)
    return fail(TIS_E_SHAPE, "%s: beam %d outside [1, %lld]", who, beam, (long long)leaves);
  if (static_cast<int64_t>(beam) * tree->branching > TIS_MAX_CANDIDATES)
    return fail(TIS_E_UNSUPPORTED, "%s: beam * branching = %lld > %d", who,
                (long long)beam * tree->branching, TIS_MAX_CANDIDATES);
  if (!(scale == scale) || isinf(scale))
    return fail(TIS_E_SHAPE, "%s: scale must be finite", who);
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
      !aligned(tree->summaries, 16) || (indices && !aligned(indices, 4)))
    return fail(TIS_E_ALIGN, "%s: Q, K, V, O and summaries need 16-byte alignment", who);
  const int64_t queries = static_cast<int64_t>(tree->batch) * q_heads;
  if (queries > 0x7fffffffLL) return fail(TIS_E_UNSUPPORTED, "%s: too many queries", who);

  const tis::RouteArgs ra = route_args(Q, tree, g, q_heads, beam, indices, nullptr, queries);
  const double sc =
      scale > 0.f ? static_cast<double>(scale) : 1.0 / sqrt(static_cast<double>(tree->head_dim));
  tis::AttendArgs aa{};
  aa.Q = Q;
  aa.K = K;
  aa.V = V;
  aa.indices = nullptr;
  aa.O = O;
  aa.queries = static_cast<int>(queries);
  aa.n_keys = tree->n_keys;
  aa.key_stride = tree->n_keys;
  aa.q_heads = q_heads;
  aa.kv_heads = tree->kv_heads;
  aa.group = q_heads / tree->kv_heads;
  aa.leaf_block = tree->leaf_block;
  aa.beam = beam;
  aa.n_blocks = tree->n_keys / tree->leaf_block;
  aa.scale_log2 = static_cast<float>(sc * 1.4426950408889634);
  if (noalloc) {
    const size_t need = tis::attend_workspace(
        queries, tree->head_dim, tis::attend_splits(queries, beam, tree->leaf_block));
    if (need > TIS_NOALLOC_SCRATCH_BYTES)
      return fail(TIS_E_WORKSPACE,
                  "%s: this geometry needs %zu bytes of scratch, more than the %zu the library "
                  "holds; use tis_tree_decode with a workspace",
                  who, need, static_cast<size_t>(TIS_NOALLOC_SCRATCH_BYTES));
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      st = scratch_address(who, &workspace);
      if (st != TIS_OK) return st;
      workspace_bytes = TIS_NOALLOC_SCRATCH_BYTES;
    }
  }
  st = plan_split(who, queries, tree->head_dim, beam, tree->leaf_block, workspace,
                  workspace_bytes, &aa);
  if (st != TIS_OK) return st;
  const tis::Dt dt = dtype == TIS_BF16 ? tis::Dt::BF16 : tis::Dt::F32;
  if (timeline) {
    if (tree->summary_dtype == TIS_FP8_E4M3)
      return fail(TIS_E_UNSUPPORTED, "%s: float32 or bfloat16 summaries only", who);
    const size_t need = static_cast<size_t>(queries) * aa.splits * tis::kTimelineWaves *
                        tis::kTimelineSlots * sizeof(unsigned long long);
    if (!aligned(timeline, 8))
      return fail(TIS_E_ALIGN, "%s: timeline needs 8-byte alignment", who);
    if (timeline_bytes < need)
      return fail(TIS_E_WORKSPACE, "%s: timeline %zu bytes < %zu required", who, timeline_bytes,
                  need);
    return hip_status(tis::launch_decode_timeline(dt, to_dt(tree->summary_dtype), tree->head_dim,
                                                  ra, aa, timeline,
                                                  static_cast<hipStream_t>(stream)),
                      who);
  }
  return hip_status(tis::launch_decode(dt, to_dt(tree->summary_dtype), tree->head_dim, ra, aa,
                                      static_cast<hipStream_t>(stream)),
                    who);
}

}  // namespace

extern "C" {

tis_status tis_tree_decode(const void *Q, const void *K, const void *V, tis_dtype dtype,
                           int q_heads, const tis_tree *tree, int beam, float scale, float *O,
                           int32_t *indices, void *workspace, size_t workspace_bytes,
                           void *stream) {
  return decode_full_tree("tis_tree_decode", Q, K, V, dtype, q_heads, tree, beam, scale, O,
                          indices, workspace, workspace_bytes, false, stream);
}

size_t tis_probe_decode_timeline_bytes(int batch, int q_heads, int beam, int leaf_block) {
  if (batch < 1 || q_heads < 1 || beam < 1 || leaf_block < 1) return 0;
  const int64_t queries = static_cast<int64_t>(batch) * q_heads;
  return static_cast<size_t>(queries) * tis::attend_splits(queries, beam, leaf_block) *
         tis::kTimelineWaves * tis::kTimelineSlots * sizeof(unsigned long long);
}

tis_status tis_probe_decode_timeline(const void *Q, const void *K, const void *V,
                                     tis_dtype dtype, int q_heads, const tis_tree *tree, int beam,
                                     float scale, float *O, void *workspace,
                                     size_t workspace_bytes, uint64_t *timeline,
                                     size_t timeline_bytes, void *stream) {
  if (!timeline)
    return fail(TIS_E_NULL, "tis_probe_decode_timeline: timeline is required");
  return decode_full_tree("tis_probe_decode_timeline", Q, K, V, dtype, q_heads, tree, beam, scale,
                          O, nullptr, workspace, workspace_bytes, false, stream,
                          reinterpret_cast<unsigned long long *>(timeline), timeline_bytes);
}

int tis_wall_clock_khz(int device) {
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, device) != hipSuccess) return 0;
  return v;
}

tis_status tis_tree_decode_noalloc(const void *Q, const void *K, const void *V, tis_dtype dtype,
                                   int q_heads, const tis_tree *tree, int beam, float scale,
                                   float *O, int32_t *indices, void *stream) {
  return decode_full_tree("tis_tree_decode_noalloc", Q, K, V, dtype, q_heads, tree, beam, scale,
                          O, indices, nullptr, 0, true, stream);
}

// ------------------------------------------------------- growing cache --

namespace {

// Fewest levels lv >= 1 with b^lv * L >= n (n >= 1); 0 past kMaxLevels.
int cache_depth(int64_t n, int branching, int leaf_block) {
  int64_t cap = static_cast<int64_t>(branching) * leaf_block;
  for (int lv = 1; lv <= tis::kMaxLevels; ++lv) {
    if (cap >= n) return lv;
    if (cap > (int64_t{1} << 40)) return 0;
    cap *= branching;
  }
  return 0;
}

struct CacheGeometry {
  int heights;          // H
  int64_t heads;
  int64_t summ_elems;   // summary elements
  int64_t state_elems;  // doubles in one state half
  int chunk_height;     // long appends: chunks are the nodes of this height
  int64_t chunk_keys;   // L b^chunk_height
  int64_t scratch_elems;  // doubles after the two halves: a sum per (head, chunk, column)
};

tis_status check_cache(const char *who, int batch, int kv_heads, int head_dim, int branching,
                       int leaf_block, int capacity, CacheGeometry *g) {
  if (batch < 1 || kv_heads < 1)
    return fail(TIS_E_SHAPE, "%s: batch and kv_heads must be >= 1", who);
  if (head_dim != 64 && head_dim != 128)
    return fail(head_dim < 1 ? TIS_E_SHAPE : TIS_E_UNSUPPORTED,
                "%s: head_dim %d: only 64 and 128 are compiled", who, head_dim);
  if (branching < 2) return fail(TIS_E_SHAPE, "%s: branching %d < 2", who, branching);
  if (branching > tis::kMaxBranching)
    return fail(TIS_E_UNSUPPORTED, "%s: branching %d > %d", who, branching, tis::kMaxBranching);
  if (leaf_block < 1) return fail(TIS_E_SHAPE, "%s: leaf_block %d < 1", who, leaf_block);
  if (capacity < 1) return fail(TIS_E_SHAPE, "%s: capacity %d < 1", who, capacity);
  const int H = cache_depth(capacity, branching, leaf_block);
  if (H < 1)
    return fail(TIS_E_UNSUPPORTED, "%s: a full cache would need more than %d levels", who,
                tis::kMaxLevels);
  g->heights = H;
  g->heads = static_cast<int64_t>(batch) * kv_heads;
  int64_t span = leaf_block, elems = 0;
  for (int h = 0; h < H; ++h) {
    elems += g->heads * ((capacity + span - 1) / span) * head_dim;
    span *= branching;
  }
  g->summ_elems = elems;
  g->state_elems = g->heads * H * head_dim;  // one of the two halves
  g->chunk_height = tis::append_chunk_height(branching, leaf_block, H);
  g->chunk_keys = leaf_block;
  for (int h = 0; h < g->chunk_height; ++h) g->chunk_keys *= branching;
  g->scratch_elems = g->heads * ((capacity + g->chunk_keys - 1) / g->chunk_keys) * head_dim;
  return TIS_OK;
}

tis_status check_cache_tree(const char *who, const tis_cache_tree *t, CacheGeometry *g) {
  if (!t || !t->summaries || !t->state)
    return fail(TIS_E_NULL, "%s: tree, tree->summaries and tree->state are required", who);
  tis_status st = check_cache(who, t->batch, t->kv_heads, t->head_dim, t->branching,
                              t->leaf_block, t->capacity, g);
  if (st != TIS_OK) return st;
  st = check_summary_dtype_no_fp8(who, t->summary_dtype);
  if (st != TIS_OK) return st;
  if (!aligned(t->summaries, 16) || !aligned(t->state, 16))
    return fail(TIS_E_ALIGN, "%s: summaries and state need 16-byte alignment", who);
  if (t->state_half != 0 && t->state_half != 1)
    return fail(TIS_E_SHAPE, "%s: state_half %d is neither 0 nor 1", who, t->state_half);
  if (t->n_keys < 0 || t->n_keys > t->capacity)
    return fail(TIS_E_SHAPE, "%s: n_keys %d outside [0, capacity %d]", who, t->n_keys,
                t->capacity);
  const int want = t->n_keys ? cache_depth(t->n_keys, t->branching, t->leaf_block) : 0;
  if (t->levels != want)
    return fail(TIS_E_SHAPE, "%s: levels %d does not match n_keys %d (depth %d)", who, t->levels,
                t->n_keys, want);
  return TIS_OK;
}

// Route arguments over the tree of a cache (n_keys >= 1, checked).
tis::RouteArgs cache_route_args(const void *Q, const tis_cache_tree *t, int q_heads, int beam,
                                int32_t *indices, int32_t *trace, int64_t queries) {
  tis::RouteArgs a{};
  a.Q = Q;
  a.summ = t->summaries;
  a.indices = indices;
  a.trace = trace;
  a.queries = static_cast<int>(queries);
  a.q_heads = q_heads;
  a.kv_heads = t->kv_heads;
  a.group = q_heads / t->kv_heads;
  a.branching = t->branching;
  a.levels = t->levels;
  a.beam = beam;
  a.cache = 1;
  a.n_keys = t->n_keys;
  a.leaf_block = t->leaf_block;
  a.capacity = t->capacity;
  // per level l of the current tree (height levels - l): existing nodes,
  // rows per head and the block's offset in the height-major layout
  const int64_t heads = static_cast<int64_t>(t->batch) * t->kv_heads;
  int64_t span_h[tis::kMaxLevels + 1], hoff[tis::kMaxLevels + 1];
  {
    int64_t span = t->leaf_block, off = 0;
    for (int h = 0; h < t->levels; ++h) {
      span_h[h] = span;
      hoff[h] = off;
      off += heads * ((t->capacity + span - 1) / span) * t->head_dim;
      span *= t->branching;
    }
  }
  for (int l = 0; l <= tis::kMaxLevels + 1; ++l) a.lvl_exist[l] = 0;
  a.lvl_exist[0] = 1;  // the root
  for (int l = 1; l <= t->levels; ++l) {
    const int h = t->levels - l;
    a.lvl_exist[l] = (t->n_keys + span_h[h] - 1) / span_h[h];
    a.lvl_rows[l] = (t->capacity + span_h[h] - 1) / span_h[h];
    a.lvl_off[l] = hoff[h];
  }
  // first level whose existing nodes outnumber the beam
  a.first_cut = 1;
  while (a.first_cut < t->levels && a.lvl_exist[a.first_cut] <= beam) ++a.first_cut;
  return a;
}

tis_status check_cache_query(const char *who, const void *Q, tis_dtype dtype, int q_heads,
                             const tis_cache_tree *t, int beam, CacheGeometry *g,
                             int64_t *queries) {
  tis_status st = check_dtype(dtype);
  if (st != TIS_OK) return st;
  st = check_cache_tree(who, t, g);
  if (st != TIS_OK) return st;
  if (t->n_keys < 1) return fail(TIS_E_SHAPE, "%s: the tree is empty", who);
  if (q_heads < 1 || q_heads % t->kv_heads != 0)
    return fail(TIS_E_SHAPE, "%s: q_heads %d is not a positive multiple of kv_heads %d", who,
                q_heads, t->kv_heads);
  if (beam < 1) return fail(TIS_E_SHAPE, "%s: beam %d < 1", who, beam);
  if (static_cast<int64_t>(beam) * t->branching > TIS_MAX_CANDIDATES)
    return fail(TIS_E_UNSUPPORTED, "%s: beam * branching = %lld > %d", who,
                (long long)beam * t->branching, TIS_MAX_CANDIDATES);
  if (!aligned(Q, 16)) return fail(TIS_E_ALIGN, "%s: Q needs 16-byte alignment", who);
  *queries = static_cast<int64_t>(t->batch) * q_heads;
  if (*queries > 0x7fffffffLL) return fail(TIS_E_UNSUPPORTED, "%s: too many queries", who);
  return TIS_OK;
}

// Append arguments of keys [n_keys, n_keys + n_new) of a checked tree: the
// state in use and the other half, per-height offsets, rows and spans.
tis::AppendArgs cache_append_args(const void *K, const tis_cache_tree *t, const CacheGeometry &g,
                                  int n_new) {
  tis::AppendArgs a{};
  a.K = K;
  a.summ = t->summaries;
  a.state = t->state + (t->state_half ? g.state_elems : 0);
  a.state_next = t->state + (t->state_half ? 0 : g.state_elems);
  a.heads = g.heads;
  a.capacity = t->capacity;
  a.n0 = t->n_keys;
  a.n1 = static_cast<int64_t>(t->n_keys) + n_new;
  a.leaf_block = t->leaf_block;
  a.branching = t->branching;
  a.heights = g.heights;
  int64_t span = t->leaf_block, off = 0;
  for (int h = 0; h < g.heights; ++h) {
    const int64_t rows = (t->capacity + span - 1) / span;
    a.block_off[h] = off;
    a.rows[h] = static_cast<uint32_t>(rows);
    // L b^h < capacity for h < H - 1 by the choice of H, and L b^(H-1)
    // < capacity too unless H = 1 (then it is L): 32 bits always hold it
    a.span[h] = static_cast<uint32_t>(span);
    off += g.heads * rows * t->head_dim;
    span *= t->branching;
  }
  return a;
}

// Attend arguments of a decode over the first n_keys keys of a cache.
tis::AttendArgs cache_attend_args(const void *Q, const void *K, const void *V, float *O,
                                  const tis_cache_tree *t, int q_heads, int beam, float scale,
                                  int64_t queries, int64_t n_keys) {
  const double sc =
      scale > 0.f ? static_cast<double>(scale) : 1.0 / sqrt(static_cast<double>(t->head_dim));
  tis::AttendArgs aa{};
  aa.Q = Q;
  aa.K = K;
  aa.V = V;
  aa.indices = nullptr;
  aa.O = O;
  aa.queries = static_cast<int>(queries);
  aa.n_keys = n_keys;
  aa.key_stride = t->capacity;
  aa.q_heads = q_heads;
  aa.kv_heads = t->kv_heads;
  aa.group = q_heads / t->kv_heads;
  aa.leaf_block = t->leaf_block;
  aa.beam = beam;
  aa.n_blocks = (n_keys + t->leaf_block - 1) / t->leaf_block;
  aa.scale_log2 = static_cast<float>(sc * 1.4426950408889634);
  return aa;
}

}  // namespace

size_t tis_cache_tree_summary_bytes(int batch, int kv_heads, int head_dim, int branching,
                                    int leaf_block, int capacity) {
  return tis_cache_tree_summary_bytes_as(batch, kv_heads, head_dim, branching, leaf_block,
                                         capacity, TIS_F32);
}

size_t tis_cache_tree_summary_bytes_as(int batch, int kv_heads, int head_dim, int branching,
                                       int leaf_block, int capacity, tis_dtype summary_dtype) {
  CacheGeometry g;
  if (summary_dtype != TIS_F32 && summary_dtype != TIS_BF16) return 0;  // no fp8 cache trees
  if (check_cache("tis_cache_tree_summary_bytes", batch, kv_heads, head_dim, branching,
                  leaf_block, capacity, &g) != TIS_OK)
    return 0;
  return static_cast<size_t>(g.summ_elems) * summary_elem_bytes(summary_dtype);
}

size_t tis_cache_tree_state_bytes(int batch, int kv_heads, int head_dim, int branching,
                                  int leaf_block, int capacity) {
  CacheGeometry g;
  if (check_cache("tis_cache_tree_state_bytes", batch, kv_heads, head_dim, branching,
                  leaf_block, capacity, &g) != TIS_OK)
    return 0;
  return static_cast<size_t>(2 * g.state_elems + g.scratch_elems) * sizeof(double);
}

tis_status tis_cache_tree_reset(tis_cache_tree *tree, void *stream) {
  if (!tree || !tree->summaries || !tree->state)
    return fail(TIS_E_NULL, "tis_cache_tree_reset: tree, tree->summaries and tree->state are required");
  CacheGeometry g;
  tis_status st = check_cache("tis_cache_tree_reset", tree->batch, tree->kv_heads,
                              tree->head_dim, tree->branching, tree->leaf_block, tree->capacity,
                              &g);
  if (st != TIS_OK) return st;
  st = check_summary_dtype_no_fp8("tis_cache_tree_reset", tree->summary_dtype);
  if (st != TIS_OK) return st;
  if (!aligned(tree->summaries, 16) || !aligned(tree->state, 16))
    return fail(TIS_E_ALIGN, "tis_cache_tree_reset: summaries and state need 16-byte alignment");
  st = hip_status(tis::launch_fill_zero(tree->state, 2 * g.state_elems,
                                          static_cast<hipStream_t>(stream)),
                  "tis_cache_tree_reset launch");
  if (st != TIS_OK) return st;
  tree->n_keys = 0;
  tree->levels = 0;
  tree->state_half = 0;
  return TIS_OK;
}

tis_status tis_cache_tree_append(const void *K, tis_dtype dtype, int n_new, tis_cache_tree *tree,
                                 void *stream) {
  if (!K) return fail(TIS_E_NULL, "tis_cache_tree_append: K is required");
  tis_status st = check_dtype(dtype);
  if (st != TIS_OK) return st;
  CacheGeometry g;
  st = check_cache_tree("tis_cache_tree_append", tree, &g);
  if (st != TIS_OK) return st;
  if (!aligned(K, 16)) return fail(TIS_E_ALIGN, "tis_cache_tree_append: K needs 16-byte alignment");
  if (n_new < 0 || n_new > tree->capacity - tree->n_keys)
    return fail(TIS_E_SHAPE, "tis_cache_tree_append: n_new %d outside [0, %d] (capacity %d, n_keys %d)",
                n_new, tree->capacity - tree->n_keys, tree->capacity, tree->n_keys);
  if (n_new == 0) return TIS_OK;
  if (g.heads > 0x7fffffffLL)
    return fail(TIS_E_UNSUPPORTED, "tis_cache_tree_append: too many heads");
  tis::AppendArgs a = cache_append_args(K, tree, g, n_new);
  const tis::Dt dt = dtype == TIS_BF16 ? tis::Dt::BF16 : tis::Dt::F32;
  // an append of a chunk's worth of keys or more: chunks in parallel, the
  // new open sums in the other state half; shorter: one workgroup per head,
  // the state updated in place
  const bool chunked = n_new >= g.chunk_keys;
  if (chunked) {
    a.chunk_height = g.chunk_height;
    a.chunk_keys = static_cast<uint32_t>(g.chunk_keys);
    a.chunk0 = a.n0 / g.chunk_keys;
    a.nchunks = (a.n1 - 1) / g.chunk_keys - a.chunk0 + 1;
    a.scratch = tree->state + 2 * g.state_elems;
    if (g.heads * a.nchunks > 0x7fffffffLL)
      return fail(TIS_E_UNSUPPORTED, "tis_cache_tree_append: too many chunks");
    st = hip_status(tis::launch_cache_append_chunked(dt, to_dt(tree->summary_dtype),
                                                     tree->head_dim, a,
                                                     static_cast<hipStream_t>(stream)),
                    "tis_cache_tree_append launch");
  } else {
    st = hip_status(tis::launch_cache_append(dt, to_dt(tree->summary_dtype), tree->head_dim, a,
                                             static_cast<hipStream_t>(stream)),
                    "tis_cache_tree_append launch");
  }
  if (st != TIS_OK) return st;
  if (chunked) tree->state_half ^= 1;
  tree->n_keys += n_new;
  tree->levels = cache_depth(tree->n_keys, tree->branching, tree->leaf_block);
  return TIS_OK;
}

tis_status tis_cache_tree_route(const void *Q, tis_dtype dtype, int q_heads,
                                const tis_cache_tree *tree, int beam, int32_t *indices,
                                int32_t *trace, void *stream) {
  if (!Q || !indices) return fail(TIS_E_NULL, "tis_cache_tree_route: Q and indices are required");
  CacheGeometry g;
  int64_t queries = 0;
  tis_status st = check_cache_query("tis_cache_tree_route", Q, dtype, q_heads, tree, beam, &g,
                                    &queries);
  if (st != TIS_OK) return st;
  if (!aligned(indices, 4) || (trace && !aligned(trace, 4)))
    return fail(TIS_E_ALIGN, "tis_cache_tree_route: indices and trace need 4-byte alignment");
  const tis::RouteArgs a = cache_route_args(Q, tree, q_heads, beam, indices, trace, queries);
  const tis::Dt dt = dtype == TIS_BF16 ? tis::Dt::BF16 : tis::Dt::F32;
  return hip_status(tis::launch_route(dt, to_dt(tree->summary_dtype), tree->head_dim, a,
                                     static_cast<hipStream_t>(stream)),
                    "tis_cache_tree_route launch");
}

tis_status tis_cache_tree_decode(const void *Q, const void *K, const void *V, tis_dtype dtype,
                                 int q_heads, const tis_cache_tree *tree, int beam, float scale,
                                 float *O, int32_t *indices, void *workspace,
                                 size_t workspace_bytes, void *stream) {
  if (!Q || !K || !V || !O)
    return fail(TIS_E_NULL, "tis_cache_tree_decode: Q, K, V and O are required");
  CacheGeometry g;
  int64_t queries = 0;
  tis_status st = check_cache_query("tis_cache_tree_decode", Q, dtype, q_heads, tree, beam, &g,
                                    &queries);
  if (st != TIS_OK) return st;
  if (!(scale == scale) || isinf(scale))
    return fail(TIS_E_SHAPE, "tis_cache_tree_decode: scale must be finite");
  if (!aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || (indices && !aligned(indices, 4)))
    return fail(TIS_E_ALIGN, "tis_cache_tree_decode: K, V and O need 16-byte alignment");
  const tis::RouteArgs ra = cache_route_args(Q, tree, q_heads, beam, indices, nullptr, queries);
  tis::AttendArgs aa =
      cache_attend_args(Q, K, V, O, tree, q_heads, beam, scale, queries, tree->n_keys);
  st = plan_split("tis_cache_tree_decode", queries, tree->head_dim, beam, tree->leaf_block,
                  workspace, workspace_bytes, &aa);
  if (st != TIS_OK) return st;
  const tis::Dt dt = dtype == TIS_BF16 ? tis::Dt::BF16 : tis::Dt::F32;
  return hip_status(tis::launch_decode(dt, to_dt(tree->summary_dtype), tree->head_dim, ra, aa,
                                      static_cast<hipStream_t>(stream)),
                    "tis_cache_tree_decode launch");
}

tis_status tis_cache_tree_append_decode(const void *Q, const void *K, const void *V,
                                        tis_dtype dtype, int q_heads, tis_cache_tree *tree,
                                        int beam, float scale, float *O, int32_t *indices,
                                        void *workspace, size_t workspace_bytes, void *stream) {
  const char *who = "tis_cache_tree_append_decode";
  if (!Q || !K || !V || !O) return fail(TIS_E_NULL, "%s: Q, K, V and O are required", who);
  CacheGeometry g;
  tis_status st = check_cache_tree(who, tree, &g);
  if (st != TIS_OK) return st;
  if (tree->n_keys >= tree->capacity)
    return fail(TIS_E_SHAPE, "%s: the cache is full (capacity %d)", who, tree->capacity);
  // the decode is over the tree with the new key in it
  tis_cache_tree next = *tree;
  next.n_keys = tree->n_keys + 1;
  next.levels = cache_depth(next.n_keys, tree->branching, tree->leaf_block);
  int64_t queries = 0;
  st = check_cache_query(who, Q, dtype, q_heads, &next, beam, &g, &queries);
  if (st != TIS_OK) return st;
  if (!(scale == scale) || isinf(scale)) return fail(TIS_E_SHAPE, "%s: scale must be finite", who);
  if (!aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || (indices && !aligned(indices, 4)))
    return fail(TIS_E_ALIGN, "%s: K, V and O need 16-byte alignment", who);
  if (g.heads > 0x7fffffffLL) return fail(TIS_E_UNSUPPORTED, "%s: too many heads", who);
  const tis::RouteArgs ra = cache_route_args(Q, &next, q_heads, beam, indices, nullptr, queries);
  tis::AttendArgs aa =
      cache_attend_args(Q, K, V, O, &next, q_heads, beam, scale, queries, next.n_keys);
  st = plan_split(who, queries, tree->head_dim, beam, tree->leaf_block, workspace,
                  workspace_bytes, &aa);
  if (st != TIS_OK) return st;
  // one workgroup per query part, then one per (batch, KV head) for the append
  if (queries * aa.splits + g.heads > 0x7fffffffLL)
    return fail(TIS_E_UNSUPPORTED, "%s: too many workgroups", who);
  const tis::AppendArgs ap = cache_append_args(K, tree, g, 1);
  const tis::Dt dt = dtype == TIS_BF16 ? tis::Dt::BF16 : tis::Dt::F32;
  st = hip_status(tis::launch_decode_append(dt, to_dt(tree->summary_dtype), tree->head_dim, ra,
                                            aa, ap, static_cast<hipStream_t>(stream)),
                  "tis_cache_tree_append_decode launch");
  if (st != TIS_OK) return st;
  tree->n_keys = next.n_keys;
  tree->levels = next.levels;
  tree->state_half ^= 1;
  return TIS_OK;
}

// -------------------------------------------------------- causal prefill --

namespace {
// Parts of the causal prefill workspace, byte offsets: the partial means,
// the fp64 run sums, then (leaf blocks of a multiple of 16 keys) the kept
// leaves of every position and V transposed per 16 keys.
struct PrefillLayout {
  size_t sums, indices, vt, total;
  bool tiles;
};

bool prefill_layout(int batch, int kv_heads, int q_heads, int head_dim, int branching,
                    int leaf_block, int n_keys, int beam, tis_dtype dtype,
                    tis_dtype summary_dtype, PrefillLayout *out) {
  if (batch < 1 || kv_heads < 1 || q_heads < 1 || q_heads % kv_heads != 0 ||
      (head_dim != 64 && head_dim != 128) || branching < 2 || branching > tis::kMaxBranching ||
      leaf_block < 1 || n_keys < 1 || beam < 1 || (dtype != TIS_F32 && dtype != TIS_BF16) ||
      (summary_dtype != TIS_F32 && summary_dtype != TIS_BF16))
    return false;
  const int lv = cache_depth(n_keys, branching, leaf_block);
  if (lv < 1) return false;
  const double heads = static_cast<double>(batch) * kv_heads;
  const double rough = heads * n_keys * (lv * head_dim * 4.0 + 2.0 * head_dim * 8.0) +
                       static_cast<double>(batch) * q_heads * n_keys * beam * 4.0 +
                       heads * (n_keys + 16.0) * head_dim * 4.0;
  if (rough > 9.0e18) return false;
  const size_t h = static_cast<size_t>(batch) * kv_heads;
  size_t runs = 0;
  const int kl = tis::prefix_sum_levels(n_keys);
  int64_t run = tis::kPrefixRows;
  for (int k = 0; k < kl; ++k, run *= tis::kPrefixRows)
    runs += static_cast<size_t>((n_keys + run - 1) / run);
  PrefillLayout p{};
  p.sums = h * static_cast<size_t>(n_keys) * lv * head_dim * summary_elem_bytes(summary_dtype);
  p.total = p.sums + h * runs * head_dim * sizeof(double);
  // (16-key leaves: a workgroup would take one key tile per union entry,
  // and the fused kernel is faster there)
  p.tiles = leaf_block % 16 == 0 && leaf_block >= 32 &&
            tis::prefill_tile_heads(q_heads / kv_heads, beam, head_dim,
                                    dtype == TIS_BF16 ? 2 : 4) > 0;
  if (p.tiles) {
    p.indices = tis::align_up(p.total, 256);
    p.vt = tis::align_up(p.indices + static_cast<size_t>(batch) * q_heads * n_keys * beam *
                                         sizeof(int32_t), 256);
    p.total = p.vt + h * static_cast<size_t>((n_keys + 15) / 16) * 16 * head_dim *
                         (dtype == TIS_BF16 ? 2 : 4);
  }
  *out = p;
  return true;
}
}  // namespace

size_t tis_causal_prefill_workspace_bytes(int batch, int kv_heads, int q_heads, int head_dim,
                                          int branching, int leaf_block, int n_keys, int beam,
                                          tis_dtype dtype, tis_dtype summary_dtype) {
  PrefillLayout p;
  if (!prefill_layout(batch, kv_heads, q_heads, head_dim, branching, leaf_block, n_keys, beam,
                      dtype, summary_dtype, &p))
    return 0;
  return p.total;
}

tis_status tis_causal_prefill(const void *Q, const void *K, const void *V, tis_dtype dtype,
                              int q_heads, const tis_cache_tree *tree, int beam, float scale,
                              float *O, int32_t *indices, void *workspace, size_t workspace_bytes,
                              void *stream) {
  if (!Q || !K || !V || !O || !workspace)
    return fail(TIS_E_NULL, "tis_causal_prefill: Q, K, V, O and workspace are required");
  CacheGeometry g;
  int64_t queries = 0;
  tis_status st = check_cache_query("tis_causal_prefill", Q, dtype, q_heads, tree, beam, &g,
                                    &queries);
  if (st != TIS_OK) return st;
  if (!(scale == scale) || isinf(scale))
    return fail(TIS_E_SHAPE, "tis_causal_prefill: scale must be finite");
  const int64_t positions = tree->n_keys;
  const int64_t pq = queries * positions;  // one query per (batch, head, position)
  if (pq > 0x7fffffffLL)
    return fail(TIS_E_UNSUPPORTED, "tis_causal_prefill: %lld queries (batch * q_heads * n_keys) "
                "exceed 2^31 - 1", (long long)pq);
  PrefillLayout lay;
  if (!prefill_layout(tree->batch, tree->kv_heads, q_heads, tree->head_dim, tree->branching,
                      tree->leaf_block, tree->n_keys, beam, dtype,
                      static_cast<tis_dtype>(tree->summary_dtype), &lay))
    return fail(TIS_E_SHAPE, "tis_causal_prefill: invalid geometry");
  const size_t need = lay.total;
  if (workspace_bytes < need)
    return fail(TIS_E_WORKSPACE, "tis_causal_prefill: workspace of %zu bytes required, %zu given",
                need, workspace_bytes);
  if (!aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(workspace, 16) ||
      (indices && !aligned(indices, 4)))
    return fail(TIS_E_ALIGN, "tis_causal_prefill: K, V, O and workspace need 16-byte, indices "
                             "4-byte alignment");
  tis::RouteArgs ra = cache_route_args(Q, tree, q_heads, beam, indices, nullptr, queries);
  ra.queries = static_cast<int>(pq);
  tis::PrefillArgs pa{};
  pa.K = K;
  pa.open_summ = workspace;
  pa.heads = g.heads;
  pa.capacity = tree->capacity;
  pa.positions = tree->n_keys;
  pa.levels = tree->levels;
  {
    pa.sums = reinterpret_cast<double *>(static_cast<char *>(workspace) + lay.sums);
    pa.sum_levels = tis::prefix_sum_levels(tree->n_keys);
    int64_t run = tis::kPrefixRows, off = 0;
    for (int k = 0; k < pa.sum_levels; ++k, run *= tis::kPrefixRows) {
      pa.sum_n[k] = (tree->n_keys + run - 1) / run;
      pa.sum_off[k] = off;
      off += g.heads * pa.sum_n[k] * tree->head_dim;
    }
  }
  {
    int64_t span = tree->leaf_block, off = 0;
    for (int h = 0; h <= tis::kMaxLevels; ++h) {
      pa.h_span[h] = span;
      pa.h_rows[h] = h < g.heights ? (tree->capacity + span - 1) / span : 0;
      pa.h_off[h] = off;
      if (h < g.heights) off += g.heads * pa.h_rows[h] * tree->head_dim;
      if (span <= (int64_t{1} << 40)) span *= tree->branching;
    }
  }
  const double sc =
      scale > 0.f ? static_cast<double>(scale) : 1.0 / sqrt(static_cast<double>(tree->head_dim));
  tis::AttendArgs aa{};
  aa.Q = Q;
  aa.K = K;
  aa.V = V;
  aa.indices = nullptr;
  aa.O = O;
  aa.splits = 1;
  aa.part = nullptr;
  aa.arrive = nullptr;
  aa.queries = static_cast<int>(pq);
  aa.n_keys = tree->n_keys;
  aa.key_stride = tree->capacity;
  aa.q_heads = q_heads;
  aa.kv_heads = tree->kv_heads;
  aa.group = q_heads / tree->kv_heads;
  aa.leaf_block = tree->leaf_block;
  aa.beam = beam;
  aa.n_blocks = (static_cast<int64_t>(tree->n_keys) + tree->leaf_block - 1) / tree->leaf_block;
  aa.scale_log2 = static_cast<float>(sc * 1.4426950408889634);
  if (lay.tiles) {
    // routing writes the kept leaves (to the caller's indices, else the
    // workspace); the attention reads them back 16 positions at a time
    int32_t *kept = indices ? indices
                            : reinterpret_cast<int32_t *>(static_cast<char *>(workspace) +
                                                          lay.indices);
    ra.indices = kept;
    aa.indices = kept;
    pa.tiles = tis::prefill_tile_heads(q_heads / tree->kv_heads, beam, tree->head_dim,
                                       dtype == TIS_BF16 ? 2 : 4);
    pa.V = V;
    pa.vt = static_cast<char *>(workspace) + lay.vt;
  }
  return hip_status(tis::launch_prefill(to_dt(dtype), to_dt(tree->summary_dtype), tree->head_dim,
                                        ra, aa, pa, static_cast<hipStream_t>(stream)),
                    "tis_causal_prefill launch");
}

// ------------------------------------------------------ bounding spheres --

namespace {

int64_t tree_nodes(int batch, int kv_heads, int branching, int levels) {
  if (batch < 1 || kv_heads < 1 || branching < 2 || levels < 1 || levels > tis::kMaxLevels)
    return 0;
  int64_t n = 1, total = 0;
  for (int l = 1; l <= levels; ++l) {
    n *= branching;
    if (n > 0x7fffffffLL) return 0;
    total += n;
  }
  const double nodes = static_cast<double>(batch) * kv_heads * static_cast<double>(total);
  if (nodes > 1.0e17) return 0;
  return static_cast<int64_t>(batch) * kv_heads * total;
}

// Checks shared by the threshold route and decode.
tis_status check_threshold(const char *who, const void *Q, tis_dtype dtype, int q_heads,
                           const tis_tree *tree, const float *radii, const float *tau,
                           int max_nodes, Geometry *g, int64_t *queries) {
  tis_status st = check_dtype(dtype);
  if (st != TIS_OK) return st;
  st = check_summary_dtype_no_fp8(who, tree->summary_dtype);
  if (st != TIS_OK) return st;
  st = check_tree(tree->batch, tree->kv_heads, tree->n_keys, tree->head_dim, tree->branching,
                  tree->leaf_block, tree->levels, g);
  if (st != TIS_OK) return st;
  if (q_heads < 1 || q_heads % tree->kv_heads != 0)
    return fail(TIS_E_SHAPE, "%s: q_heads %d is not a positive multiple of kv_heads %d", who,
                q_heads, tree->kv_heads);
  if (max_nodes < 1) return fail(TIS_E_SHAPE, "%s: max_nodes %d < 1", who, max_nodes);
  if (max_nodes > TIS_MAX_SURVIVORS)
    return fail(TIS_E_UNSUPPORTED, "%s: max_nodes %d > %d", who, max_nodes, TIS_MAX_SURVIVORS);
  if (!aligned(Q, 16) || !aligned(tree->summaries, 16) || !aligned(radii, 4) ||
      !aligned(tau, 4))
    return fail(TIS_E_ALIGN, "%s: Q and summaries need 16-byte, radii and tau 4-byte alignment",
                who);
  *queries = static_cast<int64_t>(tree->batch) * q_heads;
  if (*queries > 0x7fffffffLL) return fail(TIS_E_UNSUPPORTED, "%s: too many queries", who);
  return TIS_OK;
}

tis::SphereArgs sphere_args(const tis_tree *tree, const float *radii, const float *tau,
                            int max_nodes, int32_t *counts) {
  tis::SphereArgs sa{};
  sa.radii = radii;
  sa.tau = tau;
  sa.counts = counts;
  sa.max_nodes = max_nodes;
  const int64_t heads = static_cast<int64_t>(tree->batch) * tree->kv_heads;
  int64_t n = 1, off = 0;
  for (int l = 1; l <= tis::kMaxLevels; ++l) {
    if (l <= tree->levels) {
      n *= tree->branching;
      sa.node_off[l] = off;
      off += heads * n;
    } else {
      sa.node_off[l] = off;
    }
  }
  return sa;
}

}  // namespace

size_t tis_tree_radius_bytes(int batch, int kv_heads, int branching, int levels) {
  return static_cast<size_t>(tree_nodes(batch, kv_heads, branching, levels)) * sizeof(float);
}

size_t tis_radius_workspace_bytes(int batch, int kv_heads, int branching, int levels) {
  return static_cast<size_t>(tree_nodes(batch, kv_heads, branching, levels)) * sizeof(double);
}

tis_status tis_tree_radii(const void *K, tis_dtype dtype, const tis_tree *tree, float *radii,
                          void *workspace, size_t workspace_bytes, void *stream) {
  if (!K || !tree || !tree->summaries || !radii || !workspace)
    return fail(TIS_E_NULL, "tis_tree_radii: K, tree, tree->summaries, radii and workspace are "
                            "required");
  tis_status st = check_dtype(dtype);
  if (st != TIS_OK) return st;
  st = check_summary_dtype_no_fp8("tis_tree_radii", tree->summary_dtype);
  if (st != TIS_OK) return st;
  Geometry g;
  st = check_tree(tree->batch, tree->kv_heads, tree->n_keys, tree->head_dim, tree->branching,
                  tree->leaf_block, tree->levels, &g);
  if (st != TIS_OK) return st;
  const int64_t nodes = tree_nodes(tree->batch, tree->kv_heads, tree->branching, tree->levels);
  if (workspace_bytes < static_cast<size_t>(nodes) * sizeof(double))
    return fail(TIS_E_WORKSPACE, "tis_tree_radii: workspace of %zu bytes required, %zu given",
                static_cast<size_t>(nodes) * sizeof(double), workspace_bytes);
  if (!aligned(K, 16) || !aligned(tree->summaries, 16) || !aligned(radii, 4) ||
      !aligned(workspace, 16))
    return fail(TIS_E_ALIGN, "tis_tree_radii: K, summaries and workspace need 16-byte, radii "
                             "4-byte alignment");
  const int64_t heads = static_cast<int64_t>(tree->batch) * tree->kv_heads;
  const int64_t leaves = g.n_at[tree->levels];
  tis::RadiusArgs a{};
  a.K = K;
  a.summ = tree->summaries;
  a.d2 = static_cast<unsigned long long *>(workspace);
  a.radii = radii;
  a.n_keys = tree->n_keys;
  a.heads = heads;
  // about 4096 waves over the whole tree, each a run of consecutive leaves
  int64_t lpw = heads * leaves / 4096;
  lpw = lpw < 1 ? 1 : lpw > leaves ? leaves : lpw;
  a.leaves_per_wave = lpw;
  a.waves_per_head = (leaves + lpw - 1) / lpw;
  a.total_nodes = nodes;
  a.branching = tree->branching;
  a.leaf_block = tree->leaf_block;
  a.levels = tree->levels;
  int64_t off = 0;
  for (int l = 0; l <= tis::kMaxLevels; ++l) {
    a.n_at[l] = g.n_at[l];
    a.summ_off[l] = g.summ_off[l];
    a.node_off[l] = off;  // level l's block: after the nodes of levels 1 .. l-1
    a.span[l] = 1;
    if (l >= 1 && l <= tree->levels) {
      for (int k = l; k < tree->levels; ++k) a.span[l] *= tree->branching;
      off += heads * g.n_at[l];
    }
  }
  const int64_t waves = heads * a.waves_per_head;
  if (waves / 4 + 1 > 0x7fffffffLL)
    return fail(TIS_E_UNSUPPORTED, "tis_tree_radii: grid too large");
  return hip_status(tis::launch_radii(to_dt(dtype), to_dt(tree->summary_dtype), tree->head_dim,
                                      a, waves, static_cast<hipStream_t>(stream)),
                    "tis_tree_radii launch");
}

tis_status tis_tree_route_threshold(const void *Q, tis_dtype dtype, int q_heads,
                                    const tis_tree *tree, const float *radii, const float *tau,
                                    int max_nodes, int32_t *indices, int32_t *counts,
                                    void *stream) {
  if (!Q || !tree || !tree->summaries || !radii || !tau || !indices)
    return fail(TIS_E_NULL, "tis_tree_route_threshold: Q, tree, tree->summaries, radii, tau and "
                            "indices are required");
  Geometry g;
  int64_t queries = 0;
  tis_status st = check_threshold("tis_tree_route_threshold", Q, dtype, q_heads, tree, radii,
                                  tau, max_nodes, &g, &queries);
  if (st != TIS_OK) return st;
  if (!aligned(indices, 4) || (counts && !aligned(counts, 4)))
    return fail(TIS_E_ALIGN, "tis_tree_route_threshold: indices and counts need 4-byte alignment");
  const tis::RouteArgs ra = route_args(Q, tree, g, q_heads, 1, indices, nullptr, queries);
  const tis::SphereArgs sa = sphere_args(tree, radii, tau, max_nodes, counts);
  return hip_status(tis::launch_route_threshold(to_dt(dtype), to_dt(tree->summary_dtype),
                                                tree->head_dim, ra, sa,
                                                static_cast<hipStream_t>(stream)),
                    "tis_tree_route_threshold launch");
}

size_t tis_decode_threshold_workspace_bytes(int batch, int q_heads, int head_dim, int max_nodes,
                                            int leaf_block) {
  return tis_attend_workspace_bytes(batch, q_heads, head_dim, max_nodes, leaf_block);
}

tis_status tis_tree_decode_threshold(const void *Q, const void *K, const void *V, tis_dtype dtype,
                                     int q_heads, const tis_tree *tree, const float *radii,
                                     const float *tau, int max_nodes, float scale, float *O,
                                     int32_t *indices, int32_t *counts, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  if (!Q || !K || !V || !tree || !tree->summaries || !radii || !tau || !O)
    return fail(TIS_E_NULL, "tis_tree_decode_threshold: Q, K, V, tree, tree->summaries, radii, "
                            "tau and O are required");
  Geometry g;
  int64_t queries = 0;
  tis_status st = check_threshold("tis_tree_decode_threshold", Q, dtype, q_heads, tree, radii,
                                  tau, max_nodes, &g, &queries);
  if (st != TIS_OK) return st;
  if (!(scale == scale) || isinf(scale))
    return fail(TIS_E_SHAPE, "tis_tree_decode_threshold: scale must be finite");
  if (!aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || (indices && !aligned(indices, 4)) ||
      (counts && !aligned(counts, 4)))
    return fail(TIS_E_ALIGN, "tis_tree_decode_threshold: K, V and O need 16-byte, indices and "
                             "counts 4-byte alignment");
  const tis::RouteArgs ra = route_args(Q, tree, g, q_heads, 1, indices, nullptr, queries);
  const tis::SphereArgs sa = sphere_args(tree, radii, tau, max_nodes, counts);
  const double sc =
      scale > 0.f ? static_cast<double>(scale) : 1.0 / sqrt(static_cast<double>(tree->head_dim));
  tis::AttendArgs aa{};
  aa.Q = Q;
  aa.K = K;
  aa.V = V;
  aa.indices = nullptr;
  aa.O = O;
  aa.queries = static_cast<int>(queries);
  aa.n_keys = tree->n_keys;
  aa.key_stride = tree->n_keys;
  aa.q_heads = q_heads;
  aa.kv_heads = tree->kv_heads;
  aa.group = q_heads / tree->kv_heads;
  aa.leaf_block = tree->leaf_block;
  aa.beam = max_nodes;
  aa.n_blocks = tree->n_keys / tree->leaf_block;
  aa.scale_log2 = static_cast<float>(sc * 1.4426950408889634);
  st = plan_split("tis_tree_decode_threshold", queries, tree->head_dim, max_nodes,
                  tree->leaf_block, workspace, workspace_bytes, &aa);
  if (st != TIS_OK) return st;
  return hip_status(tis::launch_decode_threshold(to_dt(dtype), to_dt(tree->summary_dtype),
                                                 tree->head_dim, ra, sa, aa,
                                                 static_cast<hipStream_t>(stream)),
                    "tis_tree_decode_threshold launch");
}

const char *tis_last_error(void) { return g_err; }

const char *tis_version(void) { return "tis 0.1.0 gfx950"; }

// ------------------------------------------------- measurement probes --

tis_status tis_probe_read(const void *buf, size_t bytes, int nontemporal, uint32_t *sink,
                          void *stream) {
  if (!buf || !sink) return fail(TIS_E_NULL, "tis_probe_read: buf and sink are required");
  if (!aligned(buf, 16) || !aligned(sink, 4))
    return fail(TIS_E_ALIGN, "tis_probe_read: buf needs 16-byte alignment, sink 4-byte");
  if (bytes == 0 || bytes % 16 != 0)
    return fail(TIS_E_SHAPE, "tis_probe_read: bytes %zu is not a positive multiple of 16", bytes);
  return hip_status(tis::launch_probe_read(buf, bytes, nontemporal != 0, sink,
                                           static_cast<hipStream_t>(stream)),
                    "tis_probe_read launch");
}

tis_status tis_probe_chase(const uint32_t *next, size_t n_elems, uint32_t start, int hops,
                           uint32_t *out, void *stream) {
  if (!next || !out) return fail(TIS_E_NULL, "tis_probe_chase: next and out are required");
  if (!aligned(next, 4) || !aligned(out, 4))
    return fail(TIS_E_ALIGN, "tis_probe_chase: next and out need 4-byte alignment");
  if (n_elems == 0 || n_elems > 0xffffffffull || hops < 0)
    return fail(TIS_E_SHAPE, "tis_probe_chase: need 1 <= n_elems < 2^32 and hops >= 0");
  return hip_status(tis::launch_probe_chase(next, n_elems, start, hops, out,
                                            static_cast<hipStream_t>(stream)),
                    "tis_probe_chase launch");
}

}  // extern "C"
