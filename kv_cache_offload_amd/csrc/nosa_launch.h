// Internal launch descriptors: the C-ABI layer validates the user's
// arguments, fills one of these and calls the matching launcher.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nosa {

struct LaunchPool {
  bool bf16;
  int head_dim;
  int64_t n_units;  // B * Hkv
  int nb;           // blocks per unit in the cache
  int blk_begin, n_blk;
  const int32_t* entry_block;  // device [B] block per batch entry (n_blk = 1), or null
  int n_kv_heads;
  const void* kv;
  int64_t kv_unit_stride, kv_block_stride;  // elements
  const float* logits;
  void* k_comp;
  float* e_sub;
  float* e_blk;
  hipStream_t stream;
};

struct LaunchFetch {
  bool bf16;
  int head_dim;
  int batch, n_kv_heads, nb, pool_slots, k_cap, step;
  const void* host_kv;
  void* pool;
  int32_t* block_table;
  int32_t* slot_block;
  int32_t* slot_last_use;
  const int32_t* sel;
  const int32_t* n_sel;
  const int32_t* insert_block;
  const void* insert_src;
  int32_t* phys;
  int32_t* miss_list;
  int32_t* n_miss;
  int phases;                  // 1: pool update, 2: gather, 3: both
  hipStream_t stream;
};

struct LaunchSelect {
  bool bf16;
  int head_dim;
  int batch, n_query, n_q_heads, n_kv_heads, nb;
  int kq, ke;
  bool fill;                   // Eq. 7 filled from the candidates left (a variant, off by default)
  const void* q;
  const int32_t* pos;
  const void* k_comp;
  const float* e_blk;
  int32_t* sel;
  int32_t* n_sel;
  void* ws;
  const LaunchFetch* pool;     // the pool update run by the selection's last workgroup, or null
  hipStream_t stream;
};

struct LaunchAttn {
  bool bf16;
  int head_dim;
  int batch, n_q_heads, n_kv_heads, nb;
  const void* q;
  const void* blocks;
  int blocks_per_head;
  const int32_t* phys;
  const int32_t* n_sel;
  int k_cap;
  const void* window_kv;
  int64_t window_head_stride, window_block_stride;
  const int32_t* pos;
  float scale;
  void* out;
  void* ws;
  int n_query;                 // query rows per batch entry (q, pos, phys, out per row)
  int part;                    // -1 whole step; 0 / 1 the two parts of a pool step; 2 a pool step
                               // with the gather folded in
  const int32_t* miss_list;    // parts 0, 1 and 2: the fetch's miss list and counts
  const int32_t* n_miss;
  const float* bias;           // per-token eviction logits added to the attention logits, or NULL
  const void* host_kv;         // part 2: the host cache [B][Hkv][NB][block]
  const void* insert_src;      // part 2: the completed window blocks [B][Hkv][block], or NULL
  hipStream_t stream;
};

struct LaunchQkv {
  bool bf16;
  int head_dim;
  int batch, n_tok, n_q_heads, n_kv_heads, nb, d_e;
  const void* qkv;
  const int32_t* pos;
  const float* w1;
  const float* w2;
  void* q_out;
  void* kv;
  float* evict_logits;
  hipStream_t stream;
};

struct LaunchStep {
  bool bf16;
  int head_dim;
  int batch, n_q_heads, n_kv_heads, nb;
  int kq, ke;
  const void* q;
  const int32_t* pos;
  const void* k_comp;
  const float* e_blk;
  const void* kv;
  float scale;
  int32_t* sel;
  int32_t* n_sel;
  void* out;
  void* ws;
  hipStream_t stream;
  // failure-handling test hook (nosa_debug_expire_step_waits): the score
  // waits of this launch expire
  bool expire_waits;
};

// Geometry of a one-launch step, the key of the library's static workspace.
struct StepKey {
  int batch, n_q_heads, n_kv_heads, head_dim, nb, dtype, kq, ke;
};
constexpr size_t kStaticStepBytes = (size_t)16 << 20;   // the static step workspace per device

// Workspace geometry (bytes), shared by the size query and the launchers.
size_t select_ws_bytes(int batch, int n_query, int n_kv_heads, int nb);
size_t attn_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim, int k_cap, int n_query);
size_t step_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim, int nb, int kq, int ke);
// Byte offset of the timeout counter inside a step workspace.
size_t step_err_offset(int batch, int n_q_heads, int n_kv_heads, int head_dim, int nb, int kq, int ke);
void launch_step_timeouts(const void* ws, size_t off_err, int32_t* out, hipStream_t stream);
// This device's static step workspace, zero-filled on `stream` when first used
// and when the geometry changes; returns 0, or a status with *why set.
int static_step_workspace(const StepKey& key, size_t need, hipStream_t stream, void** ws_out, const char** why);
// Device address of this device's static step workspace (NULL before its first use).
void* static_step_address();
// Dynamic LDS the selection kernel needs for nb candidate blocks.
size_t select_lds_bytes(int nb);

}  // namespace nosa

struct nosa_dims;

namespace nosa {

// The one-launch step's host-side checks (everything but the workspace) and
// its launch descriptor; 0 or a status, with the error text recorded.
int prepare_step(const char* fn, const nosa_dims* dims, const void* q, const int32_t* pos, const void* k_comp,
                 const float* e_blk, int32_t kq, int32_t ke, const void* kv, float scale, int32_t* sel,
                 int32_t* n_sel, void* out, void* stream, LaunchStep* a);
// Record a failure of `fn` (returns code); the status of a call's launches.
int report(int code, const char* fn, const char* what);
int launched(const char* fn);

void launch_pool_keys(const LaunchPool& a);
void launch_select(const LaunchSelect& a);
// chunk-shared selection (bf16; G of 1, 2, 4 or 8); false when unsupported
bool launch_select_shared(const LaunchSelect& a);
void launch_fetch(const LaunchFetch& a);
void launch_attn(const LaunchAttn& a);
void launch_qkv(const LaunchQkv& a);
void launch_step(const LaunchStep& a);

}  // namespace nosa
