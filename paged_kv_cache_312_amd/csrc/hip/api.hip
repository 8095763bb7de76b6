// C ABI of liblbm (include/lbm.h): state machine, planner upload, launches.
//
// The step protocol follows the pages' per-frame pipeline: append (once per
// block), evict, plan once at the first block and run in every block ("How
// the Paged KV Cache Attention Mechanism Enables Long Sequence Inference in
// LingBot-Map", section "Runtime Flow for Frame Processing"; "How FlashInfer's
// Paged KV Cache Attention Outperforms SDPA Fallback in Streaming Inference",
// section "Plan-Run Execution Workflow"), with the deferred-eviction variant in
// which evict (commit) or rollback follows the runs ("How LingBot-Map Uses KV
// Caching for Efficient Streaming Inference", section "Flow-Based Keyframe
// Selection").
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../core/bookkeeping.h"
#include "kernels.h"
#include "lbm.h"

namespace lbm {

int32_t attn_occupancy16();
int32_t attn_occupancy_f32(int32_t head_dim);

int32_t attn_occupancy(int32_t dtype, int32_t head_dim) {
  return dtype == LBM_F32 ? attn_occupancy_f32(head_dim) : attn_occupancy16();
}

int32_t partial_rows(int32_t Tq) { return (Tq + kRowsPerGroup - 1) / kRowsPerGroup * kRowsPerGroup; }

void finish_attn_args(AttnArgs* a, int32_t head_dim, int32_t num_splits, int32_t rows_per_wg,
                      int32_t groups) {
  a->n_tiles = (a->kv_len + kKeysPerTile - 1) / kKeysPerTile;
  a->tiles_per_split = (a->n_tiles + num_splits - 1) / num_splits;
  a->num_splits = (a->n_tiles + a->tiles_per_split - 1) / a->tiles_per_split;
  // query groups: the planner's (16-bit kernel), never fewer than hold the
  // rows nor more than the rows' 32-row halves
  const int32_t q_min = (a->Tq + rows_per_wg - 1) / rows_per_wg;
  a->n_qt = std::min(std::max(groups, q_min), std::max(q_min, (a->Tq + 31) / 32));
  a->rows_pad = partial_rows(a->Tq);
  a->total_items = a->n_qt * a->H * a->num_splits;
  a->items_per_xcd = (a->total_items + 7) / 8;
  a->scale_log2 = float(1.4426950408889634 / std::sqrt(double(head_dim)));
}

static lbm_status kernel_supported(const lbm_config& c) {
  if (c.dtype != LBM_F32 && c.head_dim != 64)
    return fail(LBM_ERR_UNSUPPORTED, "16-bit kernels have head_dim 64 only (got %d)", c.head_dim);
  if (c.dtype == LBM_F32 && c.head_dim != 64 && c.head_dim != 32)
    return fail(LBM_ERR_UNSUPPORTED, "fp32 kernel has head_dim 32 or 64 only (got %d)", c.head_dim);
  return LBM_OK;
}

static lbm_status hip_fail(hipError_t e, const char* what) {
  return fail(LBM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// query rows of one workgroup of the attention kernel for `dtype`
static int32_t kernel_rows_per_wg(int32_t dtype) {
  return dtype == LBM_F32 ? kRowsPerWGf32 : kRowsPerWG16;
}

}  // namespace lbm

using namespace lbm;

struct lbm_cache {
  explicit lbm_cache(const lbm_config& c) : cfg(c), bk(c) {}
  lbm_config cfg;
  Bookkeeping bk;
  std::vector<void*> patch_pools, special_pools;
  char* workspace = nullptr;
  WorkspaceLayout ws;
  int device = 0;
  int32_t num_cu = 256;
  int32_t wg_per_cu = 1;

  // open step
  bool step_open = false;
  int32_t step_nf = 0;
  std::vector<uint8_t> appended;

  // a failed multi-frame graph step left the bookkeeping ahead of the pools:
  // every step call is refused until lbm_cache_reset
  bool poisoned = false;

  // current plan
  bool plan_valid = false;
  uint64_t plan_epoch = 0;
  int32_t plan_q = 0;
  int32_t plan_splits = 0;
  int32_t plan_groups = 0;    // query groups of the plan's launches (0: the fewest)
  int32_t plan_own = 0;       // own rows of a skip-append step planned (0: a normal plan)
  bool plan_fused = false;    // the own rows are the open step's frames (lbm_append_run)
  PlanInfo plan;

  // pinned staging of the table, double-buffered and guarded by events
  int32_t* staging[2] = {nullptr, nullptr};
  hipEvent_t staging_ev[2] = {nullptr, nullptr};
  bool staging_pending[2] = {false, false};
  int staging_next = 0;
  size_t staging_bytes = 0;
};

// A frame step captured as a HIP graph over fixed buffers (see lbm.h).  Two
// instances of the same capture, each copying from its own pinned staging
// buffer, let the host fill one while the other's copy may still be queued.
struct lbm_graph {
  lbm_cache* c = nullptr;
  int32_t nf = 0, nq = 0, ns = 0;
  int32_t groups = 0;  // query groups of the captured launches (0: the fewest)
  size_t bytes = 0;                 // staging = workspace [desc_off, special ids end)
  hipStream_t cap_stream = nullptr;
  hipGraph_t graph[2] = {nullptr, nullptr};
  hipGraphExec_t exec[2] = {nullptr, nullptr};
  char* staging[2] = {nullptr, nullptr};
  hipEvent_t done[2] = {nullptr, nullptr};
  bool pending[2] = {false, false};
  int next = 0;
};

namespace {

lbm_status check_cache(const lbm_cache* c) {
  if (!c) return fail(LBM_ERR_INVALID_ARG, "cache is null");
  return LBM_OK;
}

// check_cache, and the cache not left unusable by a failed step
lbm_status check_live(const lbm_cache* c) {
  if (!c) return fail(LBM_ERR_INVALID_ARG, "cache is null");
  if (c->poisoned) return fail(LBM_ERR_BAD_STATE, "a failed step left the cache unusable; reset it");
  return LBM_OK;
}

lbm_status copy_record(const std::vector<int32_t>& v, int32_t* buf, int64_t cap, int64_t* len) {
  if (!len) return fail(LBM_ERR_INVALID_ARG, "len is null");
  if (cap > 0 && !buf) return fail(LBM_ERR_INVALID_ARG, "buf is null");
  for (int64_t i = 0; i < int64_t(v.size()) && i < cap; ++i) buf[i] = v[size_t(i)];
  *len = int64_t(v.size());
  return LBM_OK;
}

// Row table of the visible set described by (patch ids, special ids) into
// `rowtab`, then the attention launch; both on stream `st`.
// Positions past kv_len (up to the tile boundary of kv_len + own, the own
// rows of a skip-append step included) get position 0's code.
// fused_nf > 0: the plan of lbm_append_run, whose own rows (the last `own`
// positions) get their destinations as codes.
lbm_status launch_rowtab_for(const lbm_config& c, const int32_t* pids, const int32_t* sids,
                             int32_t patch_tokens, int32_t kv_len, int32_t own,
                             uint32_t* rowtab, hipStream_t st, int32_t fused_nf = 0) {
  RowtabArgs r;
  std::memset(&r, 0, sizeof(r));
  r.patch_ids = pids;
  r.special_ids = sids;
  r.rowtab = rowtab;
  r.P = c.patches_per_frame;
  r.SPS = c.special_page_size;
  r.patch_tokens = patch_tokens;
  r.kv_len = kv_len;
  r.n_pos = (kv_len + own + kKeysPerTile - 1) / kKeysPerTile * kKeysPerTile;
  r.row_bytes = int32_t(size_t(c.num_heads) * c.head_dim * dtype_size(c.dtype));
  r.inv_P = 1.0f / float(r.P);
  r.inv_SPS = 1.0f / float(r.SPS);
  if (fused_nf > 0) {
    r.own_rows = own;
    r.own_S = c.special_per_frame;
    r.own_T = c.patches_per_frame + c.special_per_frame;
    r.inv_T = 1.0f / float(r.own_T);
  }
  const hipError_t e = launch_rowtab(r, st);
  if (e != hipSuccess) return hip_fail(e, "row table launch");
  return LBM_OK;
}

AttnArgs base_args(const lbm_config& c, const void* q, void* out, int32_t nq, const void* ppool,
                   const void* spool, const uint32_t* rowtab, char* ws_base,
                   const WorkspaceLayout& ws) {
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q = q;
  a.out = out;
  a.patch_pool = ppool;
  a.special_pool = spool;
  a.rowtab = rowtab;
  a.part_o = reinterpret_cast<float*>(ws_base + ws.part_o_off);
  a.part_ml = reinterpret_cast<float*>(ws_base + ws.part_ml_off);
  a.Tq = nq;
  a.H = c.num_heads;
  const int64_t row_bytes = int64_t(c.num_heads) * c.head_dim * int64_t(dtype_size(c.dtype));
  a.vstride_patch = int32_t(c.patches_per_frame * row_bytes);
  a.vstride_special = int32_t(c.special_page_size * row_bytes);
  a.row_bytes = int32_t(row_bytes);
  return a;
}

// One attention launch over n streams' args (1 <= n <= kMaxBatch; all with
// c's head_dim and dtype, all with or all without own rows), then the merge
// of every stream whose key range is split.
lbm_status launch_attention_batch(const lbm_config& c, AttnArgs* as, int32_t n, int32_t splits,
                                  hipStream_t st, int32_t groups = 0) {
  BatchArgs b;
  std::memset(&b, 0, sizeof(b));
  b.n = n;
  for (int32_t i = 0; i < n; ++i) {
    finish_attn_args(&as[i], c.head_dim, splits, kernel_rows_per_wg(c.dtype), groups);
    b.s[i] = as[i];
    b.item_start[i + 1] = b.item_start[i] + as[i].total_items;
  }
  b.total_items = b.item_start[n];
  b.items_per_xcd = (b.total_items + 7) / 8;
  const bool own = as[0].tr_start < as[0].kv_len;
  hipError_t e = c.dtype == LBM_F32 ? launch_attn_f32(b, c.head_dim, own, st)
                                    : launch_attn16(b, c.head_dim, c.dtype == LBM_F16, own, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  for (int32_t i = 0; i < n; ++i) {
    if (as[i].num_splits > 1) {
      e = launch_merge(as[i], c.head_dim, c.dtype, st);
      if (e != hipSuccess) return hip_fail(e, "merge launch");
    }
  }
  return LBM_OK;
}

lbm_status launch_attention(const lbm_config& c, AttnArgs* a, int32_t splits, hipStream_t st,
                            int32_t groups = 0) {
  return launch_attention_batch(c, a, 1, splits, st, groups);
}

// the planner's query groups are chosen for the 16-bit kernel only
int32_t* groups_out(int32_t dtype, int32_t* g) { return dtype == LBM_F32 ? nullptr : g; }

}  // namespace

// Scratch of lbm_paged_attention_static: the row table and the split partials
// of one call, in device memory that the library never allocates at run time.
// Each GPU holds its own copy from module load until the process ends.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {

// Device address of `scratch` on each device, looked up once per device with
// that device current (the host-side name `scratch` is not a device address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

lbm_status static_scratch(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "current device");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LBM_ERR_UNSUPPORTED, "device %d beyond the %d the static scratch serves", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "static scratch address");
    g_scratch_ptr[dev] = static_cast<char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return LBM_OK;
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// Stateless paged attention with the row table and split partials in `ws`:
// a workspace laid out by workspace_layout(cfg) when ws_bytes is 0, else a
// buffer of ws_bytes bytes laid out here for this call alone (row table, then
// the partials of as many splits as fit).
lbm_status paged_attention_impl(const lbm_config* cfg, const void* q, void* out,
                                int32_t num_q_tokens, const void* patch_pool,
                                const void* special_pool, const int32_t* patch_ids,
                                int32_t n_patch_pages, const int32_t* special_ids,
                                int32_t n_special_tokens, char* ws, size_t ws_bytes,
                                void* hip_stream) {
  if (!cfg) return fail(LBM_ERR_INVALID_ARG, "cfg is null");
  lbm_status st = validate_config(*cfg);
  if (st != LBM_OK) return st;
  if ((st = kernel_supported(*cfg)) != LBM_OK) return st;
  if (!q || !out || !aligned16(q) || !aligned16(out))
    return fail(LBM_ERR_INVALID_ARG, "q/out null or misaligned");
  if ((patch_pool && !aligned16(patch_pool)) || (special_pool && !aligned16(special_pool)))
    return fail(LBM_ERR_INVALID_ARG, "pool not 16-byte aligned");
  if (num_q_tokens < 1 || num_q_tokens > cfg->max_q_tokens)
    return fail(LBM_ERR_INVALID_ARG, "num_q_tokens %d outside 1..%d", num_q_tokens,
                cfg->max_q_tokens);
  if (n_patch_pages < 0 || n_special_tokens < 0)
    return fail(LBM_ERR_INVALID_ARG, "negative table size");
  if (n_patch_pages > 0 && (!patch_pool || !patch_ids))
    return fail(LBM_ERR_INVALID_ARG, "patch pool or ids null");
  if (n_special_tokens > 0 && (!special_pool || !special_ids))
    return fail(LBM_ERR_INVALID_ARG, "special pool or ids null");
  const int64_t kv = int64_t(n_patch_pages) * cfg->patches_per_frame + n_special_tokens;
  if (kv < 1 || kv >= kMaxKvLen) return fail(LBM_ERR_INVALID_ARG, "visible length %lld", (long long)kv);
  const int64_t n_pos = (kv + kKeysPerTile - 1) / kKeysPerTile * kKeysPerTile;
  uint32_t* rowtab = nullptr;
  float* part_ml = nullptr;
  float* part_o = nullptr;
  int32_t cap = 1;
  const WorkspaceLayout wl = workspace_layout(*cfg);
  if (kv > wl.rowtab_len)
    return fail(LBM_ERR_INVALID_ARG, "visible length %lld exceeds the config's %d",
                (long long)kv, wl.rowtab_len);
  if (ws_bytes == 0) {
    rowtab = reinterpret_cast<uint32_t*>(ws + wl.rowtab_off);
    part_ml = reinterpret_cast<float*>(ws + wl.part_ml_off);
    part_o = reinterpret_cast<float*>(ws + wl.part_o_off);
    cap = split_capacity(wl, num_q_tokens);
  } else {
    const size_t tab = align256(size_t(n_pos) * sizeof(uint32_t));
    if (tab > ws_bytes)
      return fail(LBM_ERR_INVALID_ARG,
                  "visible length %lld needs a %zu-byte row table; the static scratch holds %zu",
                  (long long)kv, tab, ws_bytes);
    // one split's (m, l) and O rows; a single split writes no partials
    const size_t rows = size_t(partial_rows(num_q_tokens)) * size_t(cfg->num_heads);
    const size_t ml1 = rows * 2 * sizeof(float), o1 = rows * size_t(cfg->head_dim) * sizeof(float);
    const size_t room = ws_bytes - tab;
    int64_t fit = 0;
    while (fit < kSplitMax && align256(size_t(fit + 1) * ml1) + align256(size_t(fit + 1) * o1) <= room)
      ++fit;
    cap = int32_t(std::max<int64_t>(1, fit));
    rowtab = reinterpret_cast<uint32_t*>(ws);
    part_ml = reinterpret_cast<float*>(ws + tab);
    part_o = reinterpret_cast<float*>(ws + tab + align256(size_t(std::max<int64_t>(fit, 1)) * ml1));
  }
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  st = launch_rowtab_for(*cfg, patch_ids, special_ids, n_patch_pages * cfg->patches_per_frame,
                         int32_t(kv), 0, rowtab, stream);
  if (st != LBM_OK) return st;
  AttnArgs a = base_args(*cfg, q, out, num_q_tokens, patch_pool, special_pool, rowtab, ws,
                         WorkspaceLayout());
  a.part_ml = part_ml;
  a.part_o = part_o;
  a.kv_len = int32_t(kv);
  a.tr_start = a.kv_len;
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  int32_t groups = 0;
  const int32_t ns = choose_splits(num_q_tokens, a.kv_len, cfg->num_heads, ncu,
                                   attn_occupancy(cfg->dtype, cfg->head_dim), cap,
                                   cfg->num_splits, kernel_rows_per_wg(cfg->dtype),
                                   groups_out(cfg->dtype, &groups));
  return launch_attention(*cfg, &a, ns < 1 ? 1 : ns, stream, groups);
}

}  // namespace

extern "C" {

const char* lbm_last_error(void) { return last_error(); }

lbm_status lbm_query_sizes(const lbm_config* cfg, size_t* patch_pool_bytes,
                           size_t* special_pool_bytes, size_t* workspace_bytes) {
  clear_error();
  if (!cfg) return fail(LBM_ERR_INVALID_ARG, "cfg is null");
  lbm_status st = validate_config(*cfg);
  if (st != LBM_OK) return st;
  const size_t row = size_t(cfg->num_heads) * cfg->head_dim * dtype_size(cfg->dtype);
  const size_t pp = size_t(cfg->max_patch_pages) * 2 * cfg->patches_per_frame * row;
  const size_t sp = size_t(cfg->max_special_pages) * 2 * cfg->special_page_size * row;
  const size_t w = workspace_layout(*cfg).total;
  if (patch_pool_bytes) *patch_pool_bytes = pp;
  if (special_pool_bytes) *special_pool_bytes = sp;
  if (workspace_bytes) *workspace_bytes = w;
  return LBM_OK;
}

lbm_status lbm_cache_create(const lbm_config* cfg, void* const* patch_pools,
                            void* const* special_pools, void* workspace, lbm_cache** out) {
  clear_error();
  if (!cfg || !patch_pools || !special_pools || !workspace || !out)
    return fail(LBM_ERR_INVALID_ARG, "null argument");
  lbm_status st = validate_config(*cfg);
  if (st != LBM_OK) return st;
  if ((st = kernel_supported(*cfg)) != LBM_OK) return st;
  for (int32_t b = 0; b < cfg->num_blocks; ++b) {
    if (!patch_pools[b] || !aligned16(patch_pools[b]))
      return fail(LBM_ERR_INVALID_ARG, "patch pool %d null or not 16-byte aligned", b);
    if (cfg->max_special_pages > 0 && (!special_pools[b] || !aligned16(special_pools[b])))
      return fail(LBM_ERR_INVALID_ARG, "special pool %d null or not 16-byte aligned", b);
  }
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(LBM_ERR_INVALID_ARG, "workspace not 256-byte aligned");

  lbm_cache* c = new (std::nothrow) lbm_cache(*cfg);
  if (!c) return fail(LBM_ERR_INVALID_ARG, "out of host memory");
  c->patch_pools.assign(patch_pools, patch_pools + cfg->num_blocks);
  c->special_pools.assign(special_pools, special_pools + cfg->num_blocks);
  c->workspace = static_cast<char*>(workspace);
  c->ws = workspace_layout(*cfg);
  c->appended.assign(size_t(cfg->num_blocks), 0);

  hipError_t e = hipGetDevice(&c->device);
  int ncu = 0;
  if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, c->device);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "device query");
  }
  c->num_cu = ncu > 0 ? ncu : 256;
  c->wg_per_cu = attn_occupancy(cfg->dtype, cfg->head_dim);

  // staging = workspace [desc_off, special ids end): the step descriptor (a
  // graph step's), then the tables
  c->staging_bytes = c->ws.special_ids_off - c->ws.desc_off +
                     sizeof(int32_t) * size_t(std::max(1, cfg->max_special_pages));
  for (int i = 0; i < 2; ++i) {
    e = hipHostMalloc(reinterpret_cast<void**>(&c->staging[i]), c->staging_bytes,
                      hipHostMallocDefault);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&c->staging_ev[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      lbm_cache_destroy(c);
      return hip_fail(e, "staging allocation");
    }
  }
  *out = c;
  return LBM_OK;
}

void lbm_cache_destroy(lbm_cache* c) {
  if (!c) return;
  for (int i = 0; i < 2; ++i) {
    if (c->staging_ev[i]) {
      if (c->staging_pending[i]) (void)hipEventSynchronize(c->staging_ev[i]);
      (void)hipEventDestroy(c->staging_ev[i]);
    }
    if (c->staging[i]) (void)hipHostFree(c->staging[i]);
  }
  delete c;
}

lbm_status lbm_cache_reset(lbm_cache* c) {
  clear_error();
  lbm_status st = check_cache(c);
  if (st != LBM_OK) return st;
  c->bk.reset();
  c->step_open = false;
  c->plan_valid = false;
  c->poisoned = false;
  return LBM_OK;
}

lbm_status lbm_cache_seed_free_lists(lbm_cache* c, const int32_t* patch_order, int32_t n_patch,
                                     const int32_t* special_order, int32_t n_special) {
  clear_error();
  lbm_status st = check_cache(c);
  if (st != LBM_OK) return st;
  st = c->bk.seed_free_lists(patch_order, n_patch, special_order, n_special);
  if (st == LBM_OK) {
    c->step_open = false;
    c->plan_valid = false;
  }
  return st;
}

// The append kernel over block_idx's rows of the open step, into the pages
// block 0's append reserved (the bookkeeping's write map).
static lbm_status launch_block_append(const lbm_cache* c, int32_t block_idx, const void* k,
                                      const void* v, hipStream_t stream) {
  const WriteMap& wm = c->bk.write_map();
  AppendArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k = static_cast<const uint4*>(k);
  a.v = static_cast<const uint4*>(v);
  a.patch_pool = static_cast<uint4*>(c->patch_pools[size_t(block_idx)]);
  a.special_pool = static_cast<uint4*>(c->special_pools[size_t(block_idx)]);
  a.P = c->cfg.patches_per_frame;
  a.S = c->cfg.special_per_frame;
  a.T = a.P + a.S;
  a.SPS = c->cfg.special_page_size;
  a.rc = int32_t(size_t(c->cfg.num_heads) * c->cfg.head_dim * dtype_size(c->cfg.dtype) / 16);
  a.st0 = wm.st0;
  a.sp_first = wm.sp_first;
  for (int32_t f = 0; f < wm.nf; ++f) a.patch_pages[f] = wm.patch_pages[f];
  for (int32_t i = 0; i < wm.n_sp; ++i) a.spages[i] = wm.spages[i];
  const hipError_t e = launch_append(a, wm.nf, stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return LBM_OK;
}

lbm_status lbm_append_frame(lbm_cache* c, int32_t block_idx, const void* k, const void* v,
                            int32_t num_frames, void* hip_stream) {
  clear_error();
  lbm_status st = check_live(c);
  if (st != LBM_OK) return st;
  if (block_idx < 0 || block_idx >= c->cfg.num_blocks)
    return fail(LBM_ERR_INVALID_ARG, "block_idx %d outside 0..%d", block_idx, c->cfg.num_blocks - 1);
  if (!k || !v || !aligned16(k) || !aligned16(v))
    return fail(LBM_ERR_INVALID_ARG, "k/v null or not 16-byte aligned");
  if (num_frames < 1 || num_frames > c->cfg.max_frames_per_step)
    return fail(LBM_ERR_INVALID_ARG, "num_frames %d outside 1..%d", num_frames,
                c->cfg.max_frames_per_step);
  if (block_idx == 0) {
    if (c->step_open) {
      for (int32_t b = 0; b < c->cfg.num_blocks; ++b)
        if (!c->appended[size_t(b)])
          return fail(LBM_ERR_BAD_STATE, "block %d has not appended the previous step", b);
    }
    st = c->bk.reserve(num_frames);
    if (st != LBM_OK) return st;
    c->step_open = true;
    c->step_nf = num_frames;
    std::fill(c->appended.begin(), c->appended.end(), 0);
  } else {
    if (!c->step_open) return fail(LBM_ERR_BAD_STATE, "block %d appends before block 0", block_idx);
    if (c->appended[size_t(block_idx)])
      return fail(LBM_ERR_BAD_STATE, "block %d already appended this step", block_idx);
    if (num_frames != c->step_nf)
      return fail(LBM_ERR_INVALID_ARG, "block %d appends %d frames, block 0 appended %d",
                  block_idx, num_frames, c->step_nf);
  }
  st = launch_block_append(c, block_idx, k, v, static_cast<hipStream_t>(hip_stream));
  if (st != LBM_OK) return st;
  c->appended[size_t(block_idx)] = 1;
  return LBM_OK;
}

lbm_status lbm_evict_frames(lbm_cache* c, int32_t* evicted_ids, int32_t cap, int32_t* n_evicted) {
  clear_error();
  lbm_status st = check_live(c);
  if (st != LBM_OK) return st;
  if (cap > 0 && !evicted_ids) return fail(LBM_ERR_INVALID_ARG, "evicted_ids is null");
  std::vector<int32_t> ev;
  st = c->bk.evict(&ev);
  if (st != LBM_OK) return st;
  for (size_t i = 0; i < ev.size() && int64_t(i) < cap; ++i) evicted_ids[i] = ev[i];
  if (n_evicted) *n_evicted = int32_t(ev.size());
  return LBM_OK;
}

lbm_status lbm_rollback_last_frame(lbm_cache* c) {
  clear_error();
  lbm_status st = check_live(c);
  if (st != LBM_OK) return st;
  st = c->bk.rollback();
  if (st != LBM_OK) return st;
  c->step_open = false;
  return LBM_OK;
}

namespace {

// The plan of a frame step: the visible set of the cache as it stands, plus
// `own` rows of the frame itself on a skip-append step (they follow the
// special stream).  fused_nf > 0: the plan of lbm_append_run for the open
// step of fused_nf frames: the visible set without the step's own rows (its
// patch pages are the last fused_nf visible pages, its specials the last
// fused_nf * S special tokens), then those rows frame by frame at their
// destinations, where each block's append writes them before the block's
// attention reads them.
lbm_status plan_impl(lbm_cache* c, int32_t num_q_tokens, int32_t own, void* hip_stream,
                     int32_t fused_nf = 0) {
  if (num_q_tokens < 1 || num_q_tokens > c->cfg.max_q_tokens)
    return fail(LBM_ERR_INVALID_ARG, "num_q_tokens %d outside 1..%d", num_q_tokens,
                c->cfg.max_q_tokens);
  if (c->bk.empty()) return fail(LBM_ERR_BAD_STATE, "plan on an empty cache");
  PlanInfo p = c->bk.plan_info();
  if (p.kv_len < 1) return fail(LBM_ERR_BAD_STATE, "no visible tokens");
  std::vector<int32_t> pp;
  c->bk.visible_patch_pages(&pp);
  if (fused_nf > 0) {
    const WriteMap& wm = c->bk.write_map();
    const int32_t T = c->cfg.patches_per_frame + c->cfg.special_per_frame;
    bool tail = wm.nf == fused_nf && int32_t(pp.size()) >= fused_nf &&
                p.special_tokens >= fused_nf * c->cfg.special_per_frame;
    for (int32_t f = 0; tail && f < fused_nf; ++f)
      tail = pp[pp.size() - size_t(fused_nf) + size_t(f)] == wm.patch_pages[f];
    if (!tail) return fail(LBM_ERR_BAD_STATE, "the step's frames are not the newest visible ones");
    own = fused_nf * T;
    p.patch_tokens -= fused_nf * c->cfg.patches_per_frame;
    p.kv_len -= own;
  }

  // stage [patch ids | pad | special ids] exactly as laid out in the
  // workspace (the step descriptor before them is the graph step's)
  const int i = c->staging_next;
  if (c->staging_pending[i]) {
    const hipError_t e = hipEventSynchronize(c->staging_ev[i]);
    if (e != hipSuccess) return hip_fail(e, "staging wait");
    c->staging_pending[i] = false;
  }
  char* stg = reinterpret_cast<char*>(c->staging[i]);
  const size_t pp_off = c->ws.patch_ids_off - c->ws.desc_off;
  const size_t sp_off = c->ws.special_ids_off - c->ws.desc_off;
  std::memcpy(stg + pp_off, pp.data(), sizeof(int32_t) * pp.size());
  const std::vector<int32_t>& sp = c->bk.special_pages();
  if (!sp.empty()) std::memcpy(stg + sp_off, sp.data(), sizeof(int32_t) * sp.size());
  const size_t from = pp_off;
  const size_t bytes = sp_off + sizeof(int32_t) * sp.size() - from;
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  hipError_t e = hipMemcpyAsync(c->workspace + c->ws.desc_off + from, stg + from, bytes,
                                hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipEventRecord(c->staging_ev[i], s);
  if (e != hipSuccess) return hip_fail(e, "table upload");
  c->staging_pending[i] = true;
  c->staging_next = i ^ 1;
  lbm_status rs = launch_rowtab_for(
      c->cfg, reinterpret_cast<const int32_t*>(c->workspace + c->ws.patch_ids_off),
      reinterpret_cast<const int32_t*>(c->workspace + c->ws.special_ids_off), p.patch_tokens,
      p.kv_len, own, reinterpret_cast<uint32_t*>(c->workspace + c->ws.rowtab_off), s, fused_nf);
  if (rs != LBM_OK) return rs;

  const int32_t cap = split_capacity(c->ws, num_q_tokens);
  int32_t groups = 0;
  int32_t ns = choose_splits(num_q_tokens, p.kv_len + own, c->cfg.num_heads, c->num_cu,
                             c->wg_per_cu, cap, c->cfg.num_splits,
                             kernel_rows_per_wg(c->cfg.dtype), groups_out(c->cfg.dtype, &groups));
  if (ns < 1) ns = 1;
  c->plan = p;
  c->plan_q = num_q_tokens;
  c->plan_splits = ns;
  c->plan_groups = groups;
  c->plan_own = own;
  c->plan_fused = fused_nf > 0;
  c->plan_epoch = c->bk.epoch();
  c->plan_valid = true;
  return LBM_OK;
}

}  // namespace

lbm_status lbm_plan(lbm_cache* c, int32_t num_q_tokens, void* hip_stream) {
  clear_error();
  lbm_status st = check_live(c);
  if (st != LBM_OK) return st;
  return plan_impl(c, num_q_tokens, 0, hip_stream);
}

lbm_status lbm_plan_transient(lbm_cache* c, int32_t num_q_tokens, int32_t num_own_tokens,
                              void* hip_stream) {
  clear_error();
  lbm_status st = check_live(c);
  if (st != LBM_OK) return st;
  if (num_own_tokens < 1 || num_own_tokens > c->cfg.max_q_tokens)
    return fail(LBM_ERR_INVALID_ARG, "num_own_tokens %d outside 1..%d", num_own_tokens,
                c->cfg.max_q_tokens);
  if (c->step_open) {
    for (int32_t b = 0; b < c->cfg.num_blocks; ++b)
      if (!c->appended[size_t(b)])
        return fail(LBM_ERR_BAD_STATE, "block %d has not appended the open step", b);
  }
  return plan_impl(c, num_q_tokens, num_own_tokens, hip_stream);
}

int32_t lbm_plan_num_splits(const lbm_cache* c) {
  return (c && c->plan_valid) ? c->plan_splits : 0;
}

lbm_status lbm_run(lbm_cache* c, int32_t block_idx, const void* q, void* out,
                   int32_t num_q_tokens, void* hip_stream) {
  clear_error();
  lbm_status st = check_live(c);
  if (st != LBM_OK) return st;
  if (block_idx < 0 || block_idx >= c->cfg.num_blocks)
    return fail(LBM_ERR_INVALID_ARG, "block_idx %d outside 0..%d", block_idx, c->cfg.num_blocks - 1);
  if (!q || !out || !aligned16(q) || !aligned16(out))
    return fail(LBM_ERR_INVALID_ARG, "q/out null or not 16-byte aligned");
  if (!c->plan_valid) return fail(LBM_ERR_BAD_STATE, "run without a plan");
  if (c->plan_epoch != c->bk.epoch())
    return fail(LBM_ERR_BAD_STATE, "plan is stale (append, evict or rollback since)");
  if (num_q_tokens != c->plan_q)
    return fail(LBM_ERR_BAD_STATE, "run with %d queries, plan made for %d", num_q_tokens, c->plan_q);
  if (c->step_open && !c->appended[size_t(block_idx)])
    return fail(LBM_ERR_BAD_STATE, "block %d has not appended the open step", block_idx);
  if (c->plan_own > 0)
    return fail(LBM_ERR_BAD_STATE, "the plan is a skip-append or a fused append plan");
  AttnArgs a = base_args(c->cfg, q, out, num_q_tokens, c->patch_pools[size_t(block_idx)],
                         c->special_pools[size_t(block_idx)],
                         reinterpret_cast<const uint32_t*>(c->workspace + c->ws.rowtab_off),
                         c->workspace, c->ws);
  a.kv_len = c->plan.kv_len;
  a.tr_start = a.kv_len;
  return launch_attention(c->cfg, &a, c->plan_splits, static_cast<hipStream_t>(hip_stream),
                          c->plan_groups);
}

lbm_status lbm_run_transient(lbm_cache* c, int32_t block_idx, const void* q, const void* k,
                             const void* v, void* out, int32_t num_q_tokens, void* hip_stream) {
  clear_error();
  lbm_status st = check_live(c);
  if (st != LBM_OK) return st;
  if (block_idx < 0 || block_idx >= c->cfg.num_blocks)
    return fail(LBM_ERR_INVALID_ARG, "block_idx %d outside 0..%d", block_idx, c->cfg.num_blocks - 1);
  if (!q || !out || !k || !v || !aligned16(q) || !aligned16(out) || !aligned16(k) || !aligned16(v))
    return fail(LBM_ERR_INVALID_ARG, "q/k/v/out null or not 16-byte aligned");
  if (!c->plan_valid) return fail(LBM_ERR_BAD_STATE, "run without a plan");
  if (c->plan_epoch != c->bk.epoch())
    return fail(LBM_ERR_BAD_STATE, "plan is stale (append, evict or rollback since)");
  if (c->plan_own < 1 || c->plan_fused)
    return fail(LBM_ERR_BAD_STATE, "the plan is not a skip-append plan");
  if (num_q_tokens != c->plan_q)
    return fail(LBM_ERR_BAD_STATE, "run with %d queries, plan made for %d", num_q_tokens, c->plan_q);
  AttnArgs a = base_args(c->cfg, q, out, num_q_tokens, c->patch_pools[size_t(block_idx)],
                         c->special_pools[size_t(block_idx)],
                         reinterpret_cast<const uint32_t*>(c->workspace + c->ws.rowtab_off),
                         c->workspace, c->ws);
  a.tr_start = c->plan.kv_len;
  a.kv_len = c->plan.kv_len + c->plan_own;
  a.tk = k;
  a.tv = v;
  return launch_attention(c->cfg, &a, c->plan_splits, static_cast<hipStream_t>(hip_stream),
                          c->plan_groups);
}

lbm_status lbm_append_run(lbm_cache* c, int32_t block_idx, const void* q, const void* k,
                          const void* v, void* out, int32_t num_frames, int32_t num_q_tokens,
                          void* hip_stream) {
  clear_error();
  lbm_status st = check_live(c);
  if (st != LBM_OK) return st;
  if (block_idx < 0 || block_idx >= c->cfg.num_blocks)
    return fail(LBM_ERR_INVALID_ARG, "block_idx %d outside 0..%d", block_idx, c->cfg.num_blocks - 1);
  if (!q || !out || !k || !v || !aligned16(q) || !aligned16(out) || !aligned16(k) || !aligned16(v))
    return fail(LBM_ERR_INVALID_ARG, "q/k/v/out null or not 16-byte aligned");
  if (num_frames < 1 || num_frames > c->cfg.max_frames_per_step)
    return fail(LBM_ERR_INVALID_ARG, "num_frames %d outside 1..%d", num_frames,
                c->cfg.max_frames_per_step);
  if (num_frames > c->cfg.sliding_window)
    return fail(LBM_ERR_INVALID_ARG, "num_frames %d beyond the window of %d frames", num_frames,
                c->cfg.sliding_window);
  if (num_q_tokens < 1 || num_q_tokens > c->cfg.max_q_tokens)
    return fail(LBM_ERR_INVALID_ARG, "num_q_tokens %d outside 1..%d", num_q_tokens,
                c->cfg.max_q_tokens);
  const int32_t T = c->cfg.patches_per_frame + c->cfg.special_per_frame;
  if (int64_t(num_frames) * T > c->cfg.max_q_tokens)
    return fail(LBM_ERR_INVALID_ARG, "%d frames of %d tokens exceed max_q_tokens %d", num_frames,
                T, c->cfg.max_q_tokens);
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (block_idx == 0) {
    if (c->step_open) {
      for (int32_t b = 0; b < c->cfg.num_blocks; ++b)
        if (!c->appended[size_t(b)])
          return fail(LBM_ERR_BAD_STATE, "block %d has not appended the previous step", b);
    }
    const bool was_open = c->step_open;
    const int32_t was_nf = c->step_nf;
    st = c->bk.reserve(num_frames);
    if (st != LBM_OK) return st;
    // the visible set after this step's eviction; eviction itself follows the
    // plan, as in the graph step, so that a refused plan can still be undone
    st = plan_impl(c, num_q_tokens, 0, hip_stream, num_frames);
    if (st != LBM_OK) {
      // as before the call (the previous step, if any, was complete)
      if (num_frames != 1 || c->bk.rollback() != LBM_OK) c->poisoned = true;
      c->step_open = was_open;
      c->step_nf = was_nf;
      return st;
    }
    c->step_open = true;
    c->step_nf = num_frames;
    std::fill(c->appended.begin(), c->appended.end(), 0);
    std::vector<int32_t> evicted;
    st = c->bk.evict(&evicted);
    if (st != LBM_OK) {
      c->poisoned = true;
      return st;
    }
    c->plan_epoch = c->bk.epoch();
  } else {
    if (!c->step_open) return fail(LBM_ERR_BAD_STATE, "block %d appends before block 0", block_idx);
    if (c->appended[size_t(block_idx)])
      return fail(LBM_ERR_BAD_STATE, "block %d already appended this step", block_idx);
    if (num_frames != c->step_nf)
      return fail(LBM_ERR_INVALID_ARG, "block %d appends %d frames, block 0 appended %d",
                  block_idx, num_frames, c->step_nf);
    if (!c->plan_valid || !c->plan_fused || c->plan_epoch != c->bk.epoch())
      return fail(LBM_ERR_BAD_STATE, "the open step was not opened by lbm_append_run");
    if (num_q_tokens != c->plan_q)
      return fail(LBM_ERR_BAD_STATE, "run with %d queries, plan made for %d", num_q_tokens,
                  c->plan_q);
  }
  // The block's rows into the step's pages, then the attention over the
  // visible set and those rows, read back from the pools (the plan's row
  // table holds the rows' destinations at the own positions): two launches
  // back to back, which measured faster than one attention launch that reads
  // the rows from k / v and stores them from the tiles it stages.
  st = launch_block_append(c, block_idx, k, v, s);
  if (st != LBM_OK) return st;
  AttnArgs a = base_args(c->cfg, q, out, num_q_tokens, c->patch_pools[size_t(block_idx)],
                         c->special_pools[size_t(block_idx)],
                         reinterpret_cast<const uint32_t*>(c->workspace + c->ws.rowtab_off),
                         c->workspace, c->ws);
  a.kv_len = c->plan.kv_len + c->plan_own;
  a.tr_start = a.kv_len;
  st = launch_attention(c->cfg, &a, c->plan_splits, s, c->plan_groups);
  if (st != LBM_OK) return st;
  c->appended[size_t(block_idx)] = 1;
  return LBM_OK;
}

lbm_status lbm_run_batch(lbm_cache* const* caches, int32_t n, int32_t block_idx,
                         const void* const* q, void* const* out, void* hip_stream) {
  clear_error();
  if (!caches || !q || !out) return fail(LBM_ERR_INVALID_ARG, "caches/q/out is null");
  if (n < 1 || n > kMaxBatch) return fail(LBM_ERR_INVALID_ARG, "n %d outside 1..%d", n, kMaxBatch);
  AttnArgs as[kMaxBatch];
  int64_t rows = 0;
  int32_t kv_max = 0, cap = kSplitMax;
  const lbm_cache* c0 = caches[0];
  for (int32_t i = 0; i < n; ++i) {
    lbm_cache* c = caches[i];
    lbm_status st = check_live(c);
    if (st != LBM_OK) return st;
    for (int32_t j = 0; j < i; ++j)   // each cache's split partials live in its own workspace
      if (caches[j] == c) return fail(LBM_ERR_INVALID_ARG, "cache %d appears twice", i);
    if (c->cfg.num_heads != c0->cfg.num_heads || c->cfg.head_dim != c0->cfg.head_dim ||
        c->cfg.dtype != c0->cfg.dtype)
      return fail(LBM_ERR_INVALID_ARG, "cache %d: heads, head_dim or dtype differ from cache 0", i);
    if (block_idx < 0 || block_idx >= c->cfg.num_blocks)
      return fail(LBM_ERR_INVALID_ARG, "block_idx %d outside cache %d's 0..%d", block_idx, i,
                  c->cfg.num_blocks - 1);
    if (!q[i] || !out[i] || !aligned16(q[i]) || !aligned16(out[i]))
      return fail(LBM_ERR_INVALID_ARG, "q/out %d null or not 16-byte aligned", i);
    if (!c->plan_valid) return fail(LBM_ERR_BAD_STATE, "cache %d has no plan", i);
    if (c->plan_epoch != c->bk.epoch()) return fail(LBM_ERR_BAD_STATE, "cache %d: stale plan", i);
    if (c->plan_own > 0) return fail(LBM_ERR_BAD_STATE, "cache %d: a skip-append plan", i);
    if (c->step_open && !c->appended[size_t(block_idx)])
      return fail(LBM_ERR_BAD_STATE, "cache %d: block %d has not appended the open step", i,
                  block_idx);
    as[i] = base_args(c->cfg, q[i], out[i], c->plan_q, c->patch_pools[size_t(block_idx)],
                      c->special_pools[size_t(block_idx)],
                      reinterpret_cast<const uint32_t*>(c->workspace + c->ws.rowtab_off),
                      c->workspace, c->ws);
    as[i].kv_len = c->plan.kv_len;
    as[i].tr_start = as[i].kv_len;
    const int32_t rpw = kernel_rows_per_wg(c->cfg.dtype);
    rows += int64_t(c->plan_q + rpw - 1) / rpw * rpw;
    kv_max = std::max(kv_max, c->plan.kv_len);
    cap = std::min(cap, split_capacity(c->ws, c->plan_q));
  }
  // one split count for the whole launch, chosen for the combined work
  int32_t ns = choose_splits(int32_t(std::min<int64_t>(rows, INT32_MAX)), kv_max,
                             c0->cfg.num_heads, c0->num_cu, c0->wg_per_cu, cap,
                             c0->cfg.num_splits, kernel_rows_per_wg(c0->cfg.dtype));
  if (ns < 1) ns = 1;
  return launch_attention_batch(c0->cfg, as, n, ns, static_cast<hipStream_t>(hip_stream));
}

lbm_status lbm_paged_attention(const lbm_config* cfg, const void* q, void* out,
                               int32_t num_q_tokens, const void* patch_pool,
                               const void* special_pool, const int32_t* patch_ids,
                               int32_t n_patch_pages, const int32_t* special_ids,
                               int32_t n_special_tokens, void* workspace, void* hip_stream) {
  clear_error();
  if (!workspace) return fail(LBM_ERR_INVALID_ARG, "workspace is null");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(LBM_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  return paged_attention_impl(cfg, q, out, num_q_tokens, patch_pool, special_pool, patch_ids,
                              n_patch_pages, special_ids, n_special_tokens,
                              static_cast<char*>(workspace), 0, hip_stream);
}

lbm_status lbm_paged_attention_static(const lbm_config* cfg, const void* q, void* out,
                                      int32_t num_q_tokens, const void* patch_pool,
                                      const void* special_pool, const int32_t* patch_ids,
                                      int32_t n_patch_pages, const int32_t* special_ids,
                                      int32_t n_special_tokens, void* hip_stream) {
  clear_error();
  char* base = nullptr;
  lbm_status st = static_scratch(&base);
  if (st != LBM_OK) return st;
  return paged_attention_impl(cfg, q, out, num_q_tokens, patch_pool, special_pool, patch_ids,
                              n_patch_pages, special_ids, n_special_tokens, base,
                              kStaticScratchBytes, hip_stream);
}

lbm_status lbm_get_stats(const lbm_cache* c, lbm_stats* out) {
  clear_error();
  lbm_status st = check_cache(c);
  if (st != LBM_OK) return st;
  if (!out) return fail(LBM_ERR_INVALID_ARG, "out is null");
  *out = c->bk.stats();
  return LBM_OK;
}

lbm_status lbm_dump_state(const lbm_cache* c, int32_t* buf, int64_t cap, int64_t* len) {
  clear_error();
  lbm_status st = check_cache(c);
  if (st != LBM_OK) return st;
  std::vector<int32_t> v;
  c->bk.dump(&v);
  return copy_record(v, buf, cap, len);
}

lbm_status lbm_get_plan(const lbm_cache* c, int32_t* buf, int64_t cap, int64_t* len) {
  clear_error();
  lbm_status st = check_cache(c);
  if (st != LBM_OK) return st;
  std::vector<int32_t> v;
  c->bk.plan_record(&v);
  return copy_record(v, buf, cap, len);
}


namespace {

void graph_release(lbm_graph* g) {
  for (int i = 0; i < 2; ++i) {
    if (g->done[i]) {
      if (g->pending[i]) (void)hipEventSynchronize(g->done[i]);
      (void)hipEventDestroy(g->done[i]);
    }
    if (g->exec[i]) (void)hipGraphExecDestroy(g->exec[i]);
    if (g->graph[i]) (void)hipGraphDestroy(g->graph[i]);
    if (g->staging[i]) (void)hipHostFree(g->staging[i]);
  }
  if (g->cap_stream) (void)hipStreamDestroy(g->cap_stream);
  delete g;
}

// Record one instance of the step on g->cap_stream: the copy of staging[i]
// into the workspace, every block's append, the row table, every block's
// attention (and merge); all per-step values are read from the copied
// StepDesc.
lbm_status graph_capture(lbm_graph* g, int i, const void* const* k, const void* const* v,
                         const void* const* q, void* const* out) {
  lbm_cache* c = g->c;
  const lbm_config& cfg = c->cfg;
  const StepDesc* desc = reinterpret_cast<const StepDesc*>(c->workspace + c->ws.desc_off);
  hipError_t e = hipStreamBeginCapture(g->cap_stream, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) return hip_fail(e, "graph capture begin");
  lbm_status st = LBM_OK;
  e = hipMemcpyAsync(c->workspace + c->ws.desc_off, g->staging[i], g->bytes,
                     hipMemcpyHostToDevice, g->cap_stream);
  if (e != hipSuccess) st = hip_fail(e, "graph table copy");
  for (int32_t b = 0; st == LBM_OK && b < cfg.num_blocks; ++b) {
    AppendArgs a;
    std::memset(&a, 0, sizeof(a));
    a.k = static_cast<const uint4*>(k[b]);
    a.v = static_cast<const uint4*>(v[b]);
    a.patch_pool = static_cast<uint4*>(c->patch_pools[size_t(b)]);
    a.special_pool = static_cast<uint4*>(c->special_pools[size_t(b)]);
    a.P = cfg.patches_per_frame;
    a.S = cfg.special_per_frame;
    a.T = a.P + a.S;
    a.SPS = cfg.special_page_size;
    a.rc = int32_t(size_t(cfg.num_heads) * cfg.head_dim * dtype_size(cfg.dtype) / 16);
    a.desc = desc;
    e = launch_append(a, g->nf, g->cap_stream);
    if (e != hipSuccess) st = hip_fail(e, "graph append");
  }
  if (st == LBM_OK) {
    RowtabArgs r;
    std::memset(&r, 0, sizeof(r));
    r.patch_ids = reinterpret_cast<const int32_t*>(c->workspace + c->ws.patch_ids_off);
    r.special_ids = reinterpret_cast<const int32_t*>(c->workspace + c->ws.special_ids_off);
    r.rowtab = reinterpret_cast<uint32_t*>(c->workspace + c->ws.rowtab_off);
    r.P = cfg.patches_per_frame;
    r.SPS = cfg.special_page_size;
    r.n_pos = c->ws.rowtab_len;
    r.row_bytes = int32_t(size_t(cfg.num_heads) * cfg.head_dim * dtype_size(cfg.dtype));
    r.inv_P = 1.0f / float(r.P);
    r.inv_SPS = 1.0f / float(r.SPS);
    r.desc = desc;
    e = launch_rowtab(r, g->cap_stream);
    if (e != hipSuccess) st = hip_fail(e, "graph row table");
  }
  for (int32_t b = 0; st == LBM_OK && b < cfg.num_blocks; ++b) {
    AttnArgs a = base_args(cfg, q[b], out[b], g->nq, c->patch_pools[size_t(b)],
                           c->special_pools[size_t(b)],
                           reinterpret_cast<const uint32_t*>(c->workspace + c->ws.rowtab_off),
                           c->workspace, c->ws);
    // launch shape for exactly g->ns splits; the kernels take the step's key
    // range from the descriptor
    a.kv_len = g->ns * kKeysPerTile;
    a.tr_start = a.kv_len;
    a.desc = desc;
    st = launch_attention(cfg, &a, g->ns, g->cap_stream, g->groups);
  }
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(g->cap_stream, &graph);
  if (st != LBM_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return st;
  }
  if (e != hipSuccess) return hip_fail(e, "graph capture end");
  g->graph[i] = graph;
  e = hipGraphInstantiate(&g->exec[i], graph, nullptr, nullptr, 0);
  if (e != hipSuccess) return hip_fail(e, "graph instantiate");
  return LBM_OK;
}

}  // namespace

lbm_status lbm_graph_create(lbm_cache* c, int32_t num_frames, const void* const* k,
                            const void* const* v, const void* const* q, void* const* out,
                            lbm_graph** out_graph) {
  clear_error();
  lbm_status st = check_cache(c);
  if (st != LBM_OK) return st;
  if (!out_graph || !k || !v || !q || !out)
    return fail(LBM_ERR_INVALID_ARG, "k/v/q/out or out_graph is null");
  if (num_frames < 1 || num_frames > c->cfg.max_frames_per_step)
    return fail(LBM_ERR_INVALID_ARG, "num_frames %d outside 1..%d", num_frames,
                c->cfg.max_frames_per_step);
  const int32_t T = c->cfg.patches_per_frame + c->cfg.special_per_frame;
  const int32_t nq = num_frames * T;
  if (nq > c->cfg.max_q_tokens)
    return fail(LBM_ERR_INVALID_ARG, "%d query rows exceed max_q_tokens %d", nq,
                c->cfg.max_q_tokens);
  for (int32_t b = 0; b < c->cfg.num_blocks; ++b)
    if (!k[b] || !v[b] || !q[b] || !out[b] || !aligned16(k[b]) || !aligned16(v[b]) ||
        !aligned16(q[b]) || !aligned16(out[b]))
      return fail(LBM_ERR_INVALID_ARG, "block %d: k/v/q/out null or not 16-byte aligned", b);
  lbm_graph* g = new (std::nothrow) lbm_graph();
  if (!g) return fail(LBM_ERR_INVALID_ARG, "out of host memory");
  g->c = c;
  g->nf = num_frames;
  g->nq = nq;
  // split count for the steady state: the full window of patch pages and
  // the special tokens so far
  const int64_t kv_est = int64_t(c->cfg.scale_frames + c->cfg.sliding_window) *
                             c->cfg.patches_per_frame + c->bk.plan_info().special_tokens + nq;
  g->ns = choose_splits(nq, int32_t(std::min<int64_t>(kv_est, kMaxKvLen - 1)), c->cfg.num_heads,
                        c->num_cu, c->wg_per_cu, split_capacity(c->ws, nq), c->cfg.num_splits,
                        kernel_rows_per_wg(c->cfg.dtype), groups_out(c->cfg.dtype, &g->groups));
  if (g->ns < 1) g->ns = 1;
  g->bytes = c->ws.special_ids_off + sizeof(int32_t) * size_t(std::max(1, c->cfg.max_special_pages)) -
             c->ws.desc_off;
  hipError_t e = hipStreamCreateWithFlags(&g->cap_stream, hipStreamNonBlocking);
  for (int i = 0; e == hipSuccess && i < 2; ++i) {
    e = hipHostMalloc(reinterpret_cast<void**>(&g->staging[i]), g->bytes, hipHostMallocDefault);
    if (e == hipSuccess) {
      std::memset(g->staging[i], 0, g->bytes);
      e = hipEventCreateWithFlags(&g->done[i], hipEventDisableTiming);
    }
  }
  if (e != hipSuccess) {
    graph_release(g);
    return hip_fail(e, "graph resources");
  }
  for (int i = 0; i < 2; ++i) {
    st = graph_capture(g, i, k, v, q, out);
    if (st != LBM_OK) {
      graph_release(g);
      return st;
    }
  }
  *out_graph = g;
  return LBM_OK;
}

lbm_status lbm_graph_launch(lbm_graph* g, void* hip_stream) {
  clear_error();
  if (!g) return fail(LBM_ERR_INVALID_ARG, "graph is null");
  lbm_cache* c = g->c;
  if (c->step_open) {
    for (int32_t b = 0; b < c->cfg.num_blocks; ++b)
      if (!c->appended[size_t(b)])
        return fail(LBM_ERR_BAD_STATE, "block %d has not appended the open step", b);
  }
  const int i = g->next;
  if (g->pending[i]) {
    const hipError_t e = hipEventSynchronize(g->done[i]);
    if (e != hipSuccess) return hip_fail(e, "graph staging wait");
    g->pending[i] = false;
  }
  if (c->poisoned) return fail(LBM_ERR_BAD_STATE, "a failed step left the cache unusable; reset it");
  lbm_status st = c->bk.reserve(g->nf);
  if (st != LBM_OK) return st;
  // the visible set after this step's eviction: the latest sliding_window
  // live pages, which the reservation's pages already are (eviction runs
  // only once the launch is enqueued)
  const PlanInfo p = c->bk.plan_info();
  const WriteMap& wm = c->bk.write_map();
  StepDesc d;
  d.kv_len = p.kv_len;
  d.patch_tokens = p.patch_tokens;
  d.n_tiles = (p.kv_len + kKeysPerTile - 1) / kKeysPerTile;
  d.tiles_per_split = (d.n_tiles + g->ns - 1) / g->ns;
  d.st0 = wm.st0;
  d.sp_first = wm.sp_first;
  for (int32_t f = 0; f < wm.nf; ++f) d.patch_pages[f] = wm.patch_pages[f];
  for (int32_t j = 0; j < wm.n_sp; ++j) d.spages[j] = wm.spages[j];
  char* stg = g->staging[i];
  std::memcpy(stg, &d, sizeof(d));
  std::vector<int32_t> pp;
  c->bk.visible_patch_pages(&pp);
  std::memcpy(stg + (c->ws.patch_ids_off - c->ws.desc_off), pp.data(), sizeof(int32_t) * pp.size());
  const std::vector<int32_t>& sp = c->bk.special_pages();
  if (!sp.empty())
    std::memcpy(stg + (c->ws.special_ids_off - c->ws.desc_off), sp.data(),
                sizeof(int32_t) * sp.size());
  hipStream_t s = static_cast<hipStream_t>(hip_stream);
  hipError_t e = hipGraphLaunch(g->exec[i], s);
  if (e != hipSuccess) {
    // nothing of the step was enqueued: undo a one-frame reservation (no
    // evict has run since it); a multi-frame one cannot be undone, so the
    // cache refuses further steps until lbm_cache_reset
    if (g->nf != 1 || c->bk.rollback() != LBM_OK) c->poisoned = true;
    return hip_fail(e, "graph launch");
  }
  std::vector<int32_t> evicted;
  (void)c->bk.evict(&evicted);  // the step is enqueued: commit it
  e = hipEventRecord(g->done[i], s);
  if (e != hipSuccess) {
    // the staging slot can no longer be guarded; the step itself is queued
    c->poisoned = true;
    return hip_fail(e, "graph launch event");
  }
  g->pending[i] = true;
  g->next = i ^ 1;
  // the cache is left as after the call sequence append(all blocks), evict, plan
  c->step_open = true;
  c->step_nf = g->nf;
  std::fill(c->appended.begin(), c->appended.end(), 1);
  c->plan = p;
  c->plan_q = g->nq;
  c->plan_splits = g->ns;
  c->plan_own = 0;
  c->plan_epoch = c->bk.epoch();
  c->plan_valid = true;
  return LBM_OK;
}

int32_t lbm_graph_num_splits(const lbm_graph* g) { return g ? g->ns : 0; }

void lbm_graph_destroy(lbm_graph* g) {
  if (g) graph_release(g);
}

}  // extern "C"
