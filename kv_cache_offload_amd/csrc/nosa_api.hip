// C ABI of libnosa: argument validation, launch geometry, status codes.
//
// Nothing here allocates, frees or synchronises.  Every argument that lives
// on the host is checked before the first launch of a call; the kernels guard
// the values that live in device memory.
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <string>

#include "../../include/nosa.h"
#include "nosa_launch.h"

namespace {
// nosa_debug_expire_step_waits: process-wide, off unless a test turns it on
std::atomic<int> g_expire_step_waits{0};

thread_local std::string g_last_error;

int fail(int code, const char* fn, const char* what) {
  char buf[512];
  snprintf(buf, sizeof buf, "%s: %s", fn, what);
  g_last_error = buf;
  return code;
}

int check_launch(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    char buf[512];
    snprintf(buf, sizeof buf, "launch failed: %s", hipGetErrorString(e));
    return fail(NOSA_ERR_HIP, fn, buf);
  }
  g_last_error.clear();
  return NOSA_OK;
}

// Shape checks common to every call.
int check_dims(const nosa_dims* d, const char* fn) {
  if (!d) return fail(NOSA_ERR_ARG, fn, "dims is NULL");
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->max_blocks < 1)
    return fail(NOSA_ERR_ARG, fn, "batch, head counts and max_blocks must be >= 1");
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(NOSA_ERR_ARG, fn, "n_q_heads must be a multiple of n_kv_heads");
  if (d->n_q_heads / d->n_kv_heads > 16)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "more than 16 query heads per KV head");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "head_dim must be 64 or 128");
  if (d->dtype != NOSA_BF16 && d->dtype != NOSA_F32)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "dtype must be NOSA_BF16 or NOSA_F32");
  if ((int64_t)d->max_blocks * NOSA_BLOCK > INT32_MAX)
    return fail(NOSA_ERR_ARG, fn, "max_blocks * 64 overflows int32 positions");
  return NOSA_OK;
}

constexpr int kMaxSelectBlocks = 4096;  // LDS of the selection stage: 10 bytes per block
constexpr int kMaxPoolSlots = 1024;
constexpr int kMaxFetchK = 64;          // one wavefront holds the selected set
constexpr int kMaxStepK = 256;          // the fused step keeps its lists in LDS

}  // namespace

extern "C" {

// nosa_pool_keys (a block range shared by the batch) and nosa_pool_keys_entries
// (one block per batch entry, named on the device)
static int pool_call(const char* fn, const nosa_dims* dims, const void* kv, int64_t kv_unit_stride,
                     int64_t kv_block_stride, const float* evict_logits, int32_t blk_begin, int32_t blk_end,
                     const int32_t* entry_block, void* k_comp, float* e_sub, float* e_blk, void* stream) {
  if (int rc = check_dims(dims, fn)) return rc;
  if (!kv || !evict_logits || !k_comp || !e_sub || !e_blk)
    return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  if (blk_begin < 0 || blk_end < blk_begin || blk_end > dims->max_blocks)
    return fail(NOSA_ERR_ARG, fn, "need 0 <= blk_begin <= blk_end <= max_blocks");
  if (kv_unit_stride < 0 || kv_block_stride < 0)
    return fail(NOSA_ERR_ARG, fn, "kv strides must be >= 0");
  nosa::LaunchPool a{};
  a.bf16 = dims->dtype == NOSA_BF16;
  a.head_dim = dims->head_dim;
  a.n_units = (int64_t)dims->batch * dims->n_kv_heads;
  a.nb = dims->max_blocks;
  a.blk_begin = blk_begin;
  a.n_blk = blk_end - blk_begin;
  a.entry_block = entry_block;
  a.n_kv_heads = dims->n_kv_heads;
  a.kv = kv;
  a.kv_unit_stride = kv_unit_stride;
  a.kv_block_stride = kv_block_stride;
  a.logits = evict_logits;
  a.k_comp = k_comp;
  a.e_sub = e_sub;
  a.e_blk = e_blk;
  a.stream = (hipStream_t)stream;
  nosa::launch_pool_keys(a);
  return check_launch(fn);
}

int nosa_pool_keys(const nosa_dims* dims, const void* kv, int64_t kv_unit_stride,
                   int64_t kv_block_stride, const float* evict_logits, int32_t blk_begin,
                   int32_t blk_end, void* k_comp, float* e_sub, float* e_blk, void* stream) {
  return pool_call("nosa_pool_keys", dims, kv, kv_unit_stride, kv_block_stride, evict_logits, blk_begin,
                   blk_end, nullptr, k_comp, e_sub, e_blk, stream);
}

int nosa_pool_keys_entries(const nosa_dims* dims, const void* kv, int64_t kv_unit_stride,
                           int64_t kv_block_stride, const float* evict_logits, const int32_t* entry_block,
                           void* k_comp, float* e_sub, float* e_blk, void* stream) {
  static const char* fn = "nosa_pool_keys_entries";
  if (!entry_block) return fail(NOSA_ERR_ARG, fn, "NULL entry_block");
  return pool_call(fn, dims, kv, kv_unit_stride, kv_block_stride, evict_logits, 0, 1, entry_block, k_comp,
                   e_sub, e_blk, stream);
}

// nosa_select_blocks and its variant nosa_select_blocks_fill
static int select_call(const char* fn, bool fill, const nosa_dims* dims, const void* q, int32_t n_query,
                       const int32_t* pos, const void* k_comp, const float* e_blk, int32_t kq, int32_t ke,
                       int32_t* sel, int32_t* n_sel, void* ws, size_t ws_bytes, void* stream,
                       const nosa::LaunchFetch* pool = nullptr) {
  if (int rc = check_dims(dims, fn)) return rc;
  if (n_query < 1) return fail(NOSA_ERR_ARG, fn, "n_query must be >= 1");
  if (kq < 0 || ke < 0) return fail(NOSA_ERR_ARG, fn, "kq and ke must be >= 0");
  if ((int64_t)kq + ke > 65535) return fail(NOSA_ERR_ARG, fn, "kq + ke above 65535");
  if (!q || !pos || !k_comp || !e_blk || !n_sel || !ws || (kq + ke > 0 && !sel))
    return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  if (dims->max_blocks > kMaxSelectBlocks)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "max_blocks above 4096 (256K tokens)");
  if ((int64_t)dims->batch * n_query * dims->n_kv_heads > 65535)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "batch * n_query * n_kv_heads above 65535");
  const size_t need = nosa_workspace_size(dims, NOSA_OP_SELECT, n_query, kq, ke);
  if (ws_bytes < need) return fail(NOSA_ERR_WORKSPACE, fn, "workspace too small");
  nosa::LaunchSelect a{};
  a.bf16 = dims->dtype == NOSA_BF16;
  a.head_dim = dims->head_dim;
  a.batch = dims->batch;
  a.n_query = n_query;
  a.n_q_heads = dims->n_q_heads;
  a.n_kv_heads = dims->n_kv_heads;
  a.nb = dims->max_blocks;
  a.kq = kq;
  a.ke = ke;
  a.fill = fill;
  a.q = q;
  a.pos = pos;
  a.k_comp = k_comp;
  a.e_blk = e_blk;
  a.sel = sel;
  a.n_sel = n_sel;
  a.ws = ws;
  a.pool = pool;
  a.stream = (hipStream_t)stream;
  nosa::launch_select(a);
  return check_launch(fn);
}

int nosa_select_blocks(const nosa_dims* dims, const void* q, int32_t n_query, const int32_t* pos,
                       const void* k_comp, const float* e_blk, int32_t kq, int32_t ke,
                       int32_t* sel, int32_t* n_sel, void* ws, size_t ws_bytes, void* stream) {
  return select_call("nosa_select_blocks", false, dims, q, n_query, pos, k_comp, e_blk, kq, ke, sel, n_sel, ws,
                     ws_bytes, stream);
}

int nosa_select_blocks_fill(const nosa_dims* dims, const void* q, int32_t n_query, const int32_t* pos,
                            const void* k_comp, const float* e_blk, int32_t kq, int32_t ke,
                            int32_t* sel, int32_t* n_sel, void* ws, size_t ws_bytes, void* stream) {
  return select_call("nosa_select_blocks_fill", true, dims, q, n_query, pos, k_comp, e_blk, kq, ke, sel, n_sel, ws,
                     ws_bytes, stream);
}

int nosa_select_blocks_shared(const nosa_dims* dims, const void* q, int32_t n_query, const int32_t* pos,
                              const void* k_comp, const float* e_blk, int32_t kq, int32_t ke,
                              int32_t* sel, int32_t* n_sel, void* ws, size_t ws_bytes, void* stream) {
  static const char* fn = "nosa_select_blocks_shared";
  if (int rc = check_dims(dims, fn)) return rc;
  if (n_query < 1) return fail(NOSA_ERR_ARG, fn, "n_query must be >= 1");
  if (kq < 0 || ke < 0) return fail(NOSA_ERR_ARG, fn, "kq and ke must be >= 0");
  if ((int64_t)kq + ke > 65535) return fail(NOSA_ERR_ARG, fn, "kq + ke above 65535");
  if (!q || !pos || !k_comp || !e_blk || !n_sel || !ws || (kq + ke > 0 && !sel))
    return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  if (dims->dtype != NOSA_BF16) return fail(NOSA_ERR_UNSUPPORTED, fn, "bf16 only");
  const int G = dims->n_q_heads / dims->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "query heads per KV head must be 1, 2, 4 or 8");
  if (dims->max_blocks > kMaxSelectBlocks)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "max_blocks above 4096 (256K tokens)");
  if ((int64_t)dims->batch * n_query * dims->n_kv_heads > 65535)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "batch * n_query * n_kv_heads above 65535");
  const size_t need = nosa_workspace_size(dims, NOSA_OP_SELECT, n_query, kq, ke);
  if (ws_bytes < need) return fail(NOSA_ERR_WORKSPACE, fn, "workspace too small");
  nosa::LaunchSelect a{};
  a.bf16 = true;
  a.head_dim = dims->head_dim;
  a.batch = dims->batch;
  a.n_query = n_query;
  a.n_q_heads = dims->n_q_heads;
  a.n_kv_heads = dims->n_kv_heads;
  a.nb = dims->max_blocks;
  a.kq = kq;
  a.ke = ke;
  a.q = q;
  a.pos = pos;
  a.k_comp = k_comp;
  a.e_blk = e_blk;
  a.sel = sel;
  a.n_sel = n_sel;
  a.ws = ws;
  a.stream = (hipStream_t)stream;
  if (!nosa::launch_select_shared(a)) return fail(NOSA_ERR_UNSUPPORTED, fn, "unsupported shape");
  return check_launch(fn);
}

// nosa_fetch_blocks and its two phases (1: tables, 2: gather): checks the
// arguments and fills the launch descriptor
static int fetch_args(const char* fn, int phases, const nosa_dims* dims, const void* host_kv, void* pool,
                      int32_t pool_slots, int32_t* block_table, int32_t* slot_block, int32_t* slot_last_use,
                      int32_t step, const int32_t* sel, const int32_t* n_sel, int32_t k_cap,
                      const int32_t* insert_block, const void* insert_src, int32_t* phys, int32_t* miss_list,
                      int32_t* n_miss, void* stream, nosa::LaunchFetch& a) {
  if (int rc = check_dims(dims, fn)) return rc;
  if (k_cap < 0 || k_cap > kMaxFetchK)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "k_cap must be in [0, 64]");
  if (pool_slots <= k_cap) return fail(NOSA_ERR_ARG, fn, "pool_slots must exceed k_cap = kq + ke");
  if (pool_slots > kMaxPoolSlots) return fail(NOSA_ERR_UNSUPPORTED, fn, "pool_slots above 1024");
  if (!miss_list || !n_miss) return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  if ((phases & 1) && (!block_table || !slot_block || !slot_last_use || !n_sel || (k_cap > 0 && (!sel || !phys))))
    return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  if ((phases & 2) && (!host_kv || !pool)) return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  if (phases == 3 && insert_block && !insert_src) return fail(NOSA_ERR_ARG, fn, "insert_block needs insert_src");
  if ((int64_t)dims->batch * dims->n_kv_heads > 65535)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "batch * n_kv_heads above 65535");
  a = nosa::LaunchFetch{};
  a.bf16 = dims->dtype == NOSA_BF16;
  a.head_dim = dims->head_dim;
  a.batch = dims->batch;
  a.n_kv_heads = dims->n_kv_heads;
  a.nb = dims->max_blocks;
  a.pool_slots = pool_slots;
  a.k_cap = k_cap;
  a.step = step;
  a.host_kv = host_kv;
  a.pool = pool;
  a.block_table = block_table;
  a.slot_block = slot_block;
  a.slot_last_use = slot_last_use;
  a.sel = sel;
  a.n_sel = n_sel;
  a.insert_block = insert_block;
  a.insert_src = insert_src;
  a.phys = phys;
  a.miss_list = miss_list;
  a.n_miss = n_miss;
  a.phases = phases;
  a.stream = (hipStream_t)stream;
  return NOSA_OK;
}

static int fetch_phases(const char* fn, int phases, const nosa_dims* dims, const void* host_kv, void* pool,
                        int32_t pool_slots, int32_t* block_table, int32_t* slot_block, int32_t* slot_last_use,
                        int32_t step, const int32_t* sel, const int32_t* n_sel, int32_t k_cap,
                        const int32_t* insert_block, const void* insert_src, int32_t* phys, int32_t* miss_list,
                        int32_t* n_miss, void* stream) {
  nosa::LaunchFetch a;
  if (int rc = fetch_args(fn, phases, dims, host_kv, pool, pool_slots, block_table, slot_block, slot_last_use, step,
                          sel, n_sel, k_cap, insert_block, insert_src, phys, miss_list, n_miss, stream, a))
    return rc;
  nosa::launch_fetch(a);
  return check_launch(fn);
}

int nosa_select_update_pool(const nosa_dims* dims, const void* q, const int32_t* pos, const void* k_comp,
                            const float* e_blk, int32_t kq, int32_t ke, int32_t* sel, int32_t* n_sel, void* ws,
                            size_t ws_bytes, int32_t pool_slots, int32_t* block_table, int32_t* slot_block,
                            int32_t* slot_last_use, int32_t step, const int32_t* insert_block, int32_t* phys,
                            int32_t* miss_list, int32_t* n_miss, void* stream) {
  static const char* fn = "nosa_select_update_pool";
  if (kq < 0 || ke < 0) return fail(NOSA_ERR_ARG, fn, "kq and ke must be >= 0");
  if ((int64_t)kq + ke > kMaxFetchK) return fail(NOSA_ERR_UNSUPPORTED, fn, "kq + ke must be <= 64");
  nosa::LaunchFetch f;
  if (int rc = fetch_args(fn, 1, dims, nullptr, nullptr, pool_slots, block_table, slot_block, slot_last_use, step,
                          sel, n_sel, kq + ke, insert_block, nullptr, phys, miss_list, n_miss, stream, f))
    return rc;
  return select_call(fn, false, dims, q, 1, pos, k_comp, e_blk, kq, ke, sel, n_sel, ws, ws_bytes, stream, &f);
}

int nosa_fetch_blocks(const nosa_dims* dims, const void* host_kv, void* pool, int32_t pool_slots,
                      int32_t* block_table, int32_t* slot_block, int32_t* slot_last_use,
                      int32_t step, const int32_t* sel, const int32_t* n_sel, int32_t k_cap,
                      const int32_t* insert_block, const void* insert_src, int32_t* phys,
                      int32_t* miss_list, int32_t* n_miss, void* stream) {
  return fetch_phases("nosa_fetch_blocks", 3, dims, host_kv, pool, pool_slots, block_table, slot_block,
                      slot_last_use, step, sel, n_sel, k_cap, insert_block, insert_src, phys, miss_list, n_miss,
                      stream);
}

int nosa_update_pool(const nosa_dims* dims, int32_t pool_slots, int32_t* block_table, int32_t* slot_block,
                     int32_t* slot_last_use, int32_t step, const int32_t* sel, const int32_t* n_sel,
                     int32_t k_cap, const int32_t* insert_block, int32_t* phys, int32_t* miss_list,
                     int32_t* n_miss, void* stream) {
  return fetch_phases("nosa_update_pool", 1, dims, nullptr, nullptr, pool_slots, block_table, slot_block,
                      slot_last_use, step, sel, n_sel, k_cap, insert_block, nullptr, phys, miss_list, n_miss,
                      stream);
}

int nosa_gather_blocks(const nosa_dims* dims, const void* host_kv, void* pool, int32_t pool_slots, int32_t k_cap,
                       const void* insert_src, const int32_t* miss_list, const int32_t* n_miss, void* stream) {
  return fetch_phases("nosa_gather_blocks", 2, dims, host_kv, pool, pool_slots, nullptr, nullptr, nullptr, 0,
                      nullptr, nullptr, k_cap, nullptr, insert_src, nullptr, const_cast<int32_t*>(miss_list),
                      const_cast<int32_t*>(n_miss), stream);
}

static int sparse_attn(const char* fn, int part, int n_query, const nosa_dims* dims, const void* q, const void* blocks,
                       int32_t blocks_per_head, const int32_t* phys, const int32_t* n_sel, int32_t k_cap,
                       const int32_t* miss_list, const int32_t* n_miss, const void* window_kv,
                       int64_t window_head_stride, int64_t window_block_stride, const int32_t* pos, float scale,
                       void* out, void* ws, size_t ws_bytes, void* stream, const float* bias = nullptr,
                       const void* host_kv = nullptr, const void* insert_src = nullptr) {
  if (int rc = check_dims(dims, fn)) return rc;
  if (k_cap < 0 || k_cap > 512) return fail(NOSA_ERR_UNSUPPORTED, fn, "k_cap must be in [0, 512]");
  if (blocks_per_head < 1 && k_cap > 0) return fail(NOSA_ERR_ARG, fn, "blocks_per_head must be >= 1");
  if (!q || !window_kv || !pos || !out || !n_sel || !ws || (k_cap > 0 && (!blocks || !phys)))
    return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  if (part >= 0 && (!miss_list || !n_miss)) return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  if (part > 2) return fail(NOSA_ERR_ARG, fn, "part must be 0 or 1");
  if (part == 2 && !host_kv) return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  if (window_head_stride < 0 || window_block_stride < 0)
    return fail(NOSA_ERR_ARG, fn, "window strides must be >= 0");
  if (!(scale == scale)) return fail(NOSA_ERR_ARG, fn, "scale is NaN");
  if (n_query < 1) return fail(NOSA_ERR_ARG, fn, "n_query must be >= 1");
  if ((int64_t)dims->batch * n_query * dims->n_kv_heads > 65535)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "batch * n_query * n_kv_heads above 65535");
  const size_t need = nosa_workspace_size(dims, NOSA_OP_ATTN, n_query, k_cap, 0);
  if (ws_bytes < need) return fail(NOSA_ERR_WORKSPACE, fn, "workspace too small");
  nosa::LaunchAttn a{};
  a.bf16 = dims->dtype == NOSA_BF16;
  a.head_dim = dims->head_dim;
  a.batch = dims->batch;
  a.n_q_heads = dims->n_q_heads;
  a.n_kv_heads = dims->n_kv_heads;
  a.nb = dims->max_blocks;
  a.q = q;
  a.blocks = blocks;
  a.blocks_per_head = blocks_per_head;
  a.phys = phys;
  a.n_sel = n_sel;
  a.k_cap = k_cap;
  a.window_kv = window_kv;
  a.window_head_stride = window_head_stride;
  a.window_block_stride = window_block_stride;
  a.pos = pos;
  a.scale = scale;
  a.out = out;
  a.ws = ws;
  a.n_query = n_query;
  a.part = part;
  a.miss_list = miss_list;
  a.n_miss = n_miss;
  a.bias = bias;
  a.host_kv = host_kv;
  a.insert_src = insert_src;
  a.stream = (hipStream_t)stream;
  nosa::launch_attn(a);
  return check_launch(fn);
}

int nosa_sparse_decode_attn(const nosa_dims* dims, const void* q, const void* blocks,
                            int32_t blocks_per_head, const int32_t* phys, const int32_t* n_sel,
                            int32_t k_cap, const void* window_kv, int64_t window_head_stride,
                            int64_t window_block_stride, const int32_t* pos, float scale, void* out,
                            void* ws, size_t ws_bytes, void* stream) {
  return sparse_attn("nosa_sparse_decode_attn", -1, 1, dims, q, blocks, blocks_per_head, phys, n_sel, k_cap,
                     nullptr, nullptr, window_kv, window_head_stride, window_block_stride, pos, scale, out, ws,
                     ws_bytes, stream);
}

int nosa_sparse_decode_attn_bias(const nosa_dims* dims, const void* q, const void* kv, const int32_t* sel,
                                 const int32_t* n_sel, int32_t k_cap, const int32_t* pos, float scale,
                                 const float* evict_logits, void* out, void* ws, size_t ws_bytes, void* stream) {
  static const char* fn = "nosa_sparse_decode_attn_bias";
  if (int rc = check_dims(dims, fn)) return rc;
  if (!evict_logits) return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  // the resident cache, each window read from it
  const int64_t blk = (int64_t)2 * 64 * dims->head_dim;
  return sparse_attn(fn, -1, 1, dims, q, kv, dims->max_blocks, sel, n_sel, k_cap, nullptr, nullptr, kv,
                     dims->max_blocks * blk, blk, pos, scale, out, ws, ws_bytes, stream, evict_logits);
}

int nosa_sparse_decode_attn_pool(const nosa_dims* dims, const void* q, const void* pool, int32_t pool_slots,
                                 const int32_t* phys, const int32_t* n_sel, int32_t k_cap,
                                 const int32_t* miss_list, const int32_t* n_miss, const void* window_kv,
                                 int64_t window_head_stride, int64_t window_block_stride, const int32_t* pos,
                                 float scale, int32_t part, void* out, void* ws, size_t ws_bytes, void* stream) {
  if (part != 0 && part != 1) return fail(NOSA_ERR_ARG, "nosa_sparse_decode_attn_pool", "part must be 0 or 1");
  return sparse_attn("nosa_sparse_decode_attn_pool", part, 1, dims, q, pool, pool_slots, phys, n_sel, k_cap,
                     miss_list, n_miss, window_kv, window_head_stride, window_block_stride, pos, scale, out, ws,
                     ws_bytes, stream);
}

int nosa_sparse_decode_attn_fetch(const nosa_dims* dims, const void* q, const void* host_kv, void* pool,
                                  int32_t pool_slots, const int32_t* phys, const int32_t* n_sel, int32_t k_cap,
                                  const int32_t* miss_list, const int32_t* n_miss, const void* insert_src,
                                  const void* window_kv, int64_t window_head_stride, int64_t window_block_stride,
                                  const int32_t* pos, float scale, void* out, void* ws, size_t ws_bytes,
                                  void* stream) {
  static const char* fn = "nosa_sparse_decode_attn_fetch";
  if (pool_slots < 1) return fail(NOSA_ERR_ARG, fn, "pool_slots must be >= 1");
  if (k_cap > 64) return fail(NOSA_ERR_UNSUPPORTED, fn, "k_cap must be in [0, 64]");
  return sparse_attn(fn, 2, 1, dims, q, pool, pool_slots, phys, n_sel, k_cap, miss_list, n_miss, window_kv,
                     window_head_stride, window_block_stride, pos, scale, out, ws, ws_bytes, stream, nullptr, host_kv,
                     insert_src);
}

int nosa_sparse_chunk_attn(const nosa_dims* dims, const void* q, int32_t n_query, const void* kv,
                           const int32_t* sel, const int32_t* n_sel, int32_t k_cap, const int32_t* pos, float scale,
                           void* out, void* ws, size_t ws_bytes, void* stream) {
  static const char* fn = "nosa_sparse_chunk_attn";
  if (int rc = check_dims(dims, fn)) return rc;
  // every row's window is a block of the cache itself
  const int64_t blk = (int64_t)2 * 64 * dims->head_dim;
  return sparse_attn(fn, -1, n_query, dims, q, kv, dims->max_blocks, sel, n_sel, k_cap,
                     nullptr, nullptr, kv, dims->max_blocks * blk, blk, pos, scale, out, ws, ws_bytes, stream);
}

int nosa_split_qkv(const nosa_dims* dims, const void* qkv, int32_t n_tok, const int32_t* pos, const float* w1,
                   const float* w2, int32_t d_e, void* q_out, void* kv, float* evict_logits, void* stream) {
  static const char* fn = "nosa_split_qkv";
  if (int rc = check_dims(dims, fn)) return rc;
  if (n_tok < 1 || n_tok > 65535) return fail(NOSA_ERR_ARG, fn, "n_tok must be in [1, 65535]");
  if (dims->batch > 65535) return fail(NOSA_ERR_UNSUPPORTED, fn, "batch above 65535");
  if (dims->n_kv_heads > 16) return fail(NOSA_ERR_UNSUPPORTED, fn, "more than 16 KV heads");
  if (d_e < 1 || d_e > 512) return fail(NOSA_ERR_UNSUPPORTED, fn, "d_e must be in [1, 512]");
  if (!qkv || !pos || !w1 || !w2 || !q_out || !kv || !evict_logits) return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  nosa::LaunchQkv a{};
  a.bf16 = dims->dtype == NOSA_BF16;
  a.head_dim = dims->head_dim;
  a.batch = dims->batch;
  a.n_tok = n_tok;
  a.n_q_heads = dims->n_q_heads;
  a.n_kv_heads = dims->n_kv_heads;
  a.nb = dims->max_blocks;
  a.d_e = d_e;
  a.qkv = qkv;
  a.pos = pos;
  a.w1 = w1;
  a.w2 = w2;
  a.q_out = q_out;
  a.kv = kv;
  a.evict_logits = evict_logits;
  a.stream = (hipStream_t)stream;
  nosa::launch_qkv(a);
  return check_launch(fn);
}

}  // extern "C"

namespace nosa {

// Checks every host-side argument of the one-launch step except the
// workspace and fills its launch descriptor (ws left NULL); 0 or a status.
int prepare_step(const char* fn, const nosa_dims* dims, const void* q, const int32_t* pos, const void* k_comp,
                 const float* e_blk, int32_t kq, int32_t ke, const void* kv, float scale, int32_t* sel,
                 int32_t* n_sel, void* out, void* stream, LaunchStep* a) {
  if (int rc = check_dims(dims, fn)) return rc;
  if (kq < 0 || ke < 0) return fail(NOSA_ERR_ARG, fn, "kq and ke must be >= 0");
  if (kq + ke > kMaxStepK) return fail(NOSA_ERR_UNSUPPORTED, fn, "kq + ke above 256");
  if (dims->n_q_heads / dims->n_kv_heads > 8)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "more than 8 query heads per KV head");
  if (dims->max_blocks > kMaxSelectBlocks)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "max_blocks above 4096 (256K tokens)");
  if (!q || !pos || !k_comp || !e_blk || !kv || !n_sel || !out || (kq + ke > 0 && !sel))
    return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  if (!(scale == scale)) return fail(NOSA_ERR_ARG, fn, "scale is NaN");
  if ((int64_t)dims->batch * dims->n_kv_heads > 65535)
    return fail(NOSA_ERR_UNSUPPORTED, fn, "batch * n_kv_heads above 65535");
  *a = LaunchStep{};
  a->bf16 = dims->dtype == NOSA_BF16;
  a->head_dim = dims->head_dim;
  a->batch = dims->batch;
  a->n_q_heads = dims->n_q_heads;
  a->n_kv_heads = dims->n_kv_heads;
  a->nb = dims->max_blocks;
  a->kq = kq;
  a->ke = ke;
  a->q = q;
  a->pos = pos;
  a->k_comp = k_comp;
  a->e_blk = e_blk;
  a->kv = kv;
  a->scale = scale;
  a->sel = sel;
  a->n_sel = n_sel;
  a->out = out;
  a->ws = nullptr;
  a->stream = (hipStream_t)stream;
  a->expire_waits = g_expire_step_waits.load(std::memory_order_relaxed) != 0;
  return NOSA_OK;
}

int report(int code, const char* fn, const char* what) { return fail(code, fn, what); }
int launched(const char* fn) { return check_launch(fn); }

}  // namespace nosa

extern "C" {

int nosa_decode_step(const nosa_dims* dims, const void* q, const int32_t* pos, const void* k_comp,
                     const float* e_blk, int32_t kq, int32_t ke, const void* kv, float scale,
                     int32_t* sel, int32_t* n_sel, void* out, void* ws, size_t ws_bytes, void* stream) {
  static const char* fn = "nosa_decode_step";
  nosa::LaunchStep a;
  if (int rc = nosa::prepare_step(fn, dims, q, pos, k_comp, e_blk, kq, ke, kv, scale, sel, n_sel, out, stream, &a))
    return rc;
  if (!ws) return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  const size_t need = nosa_workspace_size(dims, NOSA_OP_STEP, 1, kq, ke);
  if (ws_bytes < need) return fail(NOSA_ERR_WORKSPACE, fn, "workspace too small");
  a.ws = ws;
  nosa::launch_step(a);
  return check_launch(fn);
}

int nosa_step_timeouts(const nosa_dims* dims, int32_t kq, int32_t ke, const void* ws, int32_t* out,
                       void* stream) {
  static const char* fn = "nosa_step_timeouts";
  if (int rc = check_dims(dims, fn)) return rc;
  if (kq < 0 || ke < 0) return fail(NOSA_ERR_ARG, fn, "kq and ke must be >= 0");
  if (!out) return fail(NOSA_ERR_ARG, fn, "NULL buffer");
  if (!ws) {
    // the static workspace of nosa_decode_step_static on this device
    ws = nosa::static_step_address();
    if (!ws) return fail(NOSA_ERR_ARG, fn, "ws is NULL and nosa_decode_step_static has not run on this device");
  }
  const size_t off = nosa::step_err_offset(dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                                           dims->max_blocks, kq, ke);
  nosa::launch_step_timeouts(ws, off, out, (hipStream_t)stream);
  return check_launch(fn);
}

size_t nosa_workspace_size(const nosa_dims* dims, int32_t op, int32_t n_query, int32_t kq,
                           int32_t ke) {
  if (check_dims(dims, "nosa_workspace_size") != NOSA_OK) return 0;
  if (n_query < 1 || kq < 0 || ke < 0) return 0;
  if (op == NOSA_OP_SELECT)
    return nosa::select_ws_bytes(dims->batch, n_query, dims->n_kv_heads, dims->max_blocks);
  if (op == NOSA_OP_ATTN)
    return nosa::attn_ws_bytes(dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->head_dim, kq + ke, n_query);
  if (op == NOSA_OP_STEP)
    return nosa::step_ws_bytes(dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                               dims->max_blocks, kq, ke);
  return 0;
}

const char* nosa_status_str(int32_t status) {
  switch (status) {
    case NOSA_OK: return "ok";
    case NOSA_ERR_ARG: return "invalid argument";
    case NOSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case NOSA_ERR_HIP: return "HIP runtime error";
    case NOSA_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* nosa_last_error(void) { return g_last_error.c_str(); }

int nosa_debug_expire_step_waits(int32_t on) {
  g_expire_step_waits.store(on ? 1 : 0, std::memory_order_relaxed);
  return NOSA_OK;
}

}  // extern "C"
