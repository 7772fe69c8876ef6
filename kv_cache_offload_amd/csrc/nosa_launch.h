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
  const void* kv;
  int64_t kv_unit_stride, kv_block_stride;  // elements
  const float* logits;
  void* k_comp;
  float* e_sub;
  float* e_blk;
  hipStream_t stream;
};

struct LaunchSelect {
  bool bf16;
  int head_dim;
  int batch, n_query, n_q_heads, n_kv_heads, nb;
  int kq, ke;
  const void* q;
  const int32_t* pos;
  const void* k_comp;
  const float* e_blk;
  int32_t* sel;
  int32_t* n_sel;
  void* ws;
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
  int part;                    // -1 whole step; 0 / 1 the two parts of a pool step
  const int32_t* miss_list;    // parts 0 and 1: the fetch's miss list and counts
  const int32_t* n_miss;
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
};

// Workspace geometry (bytes), shared by the size query and the launchers.
size_t select_ws_bytes(int batch, int n_query, int n_kv_heads, int nb);
size_t attn_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim, int k_cap, int n_query);
size_t step_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim, int nb, int kq, int ke);
// Dynamic LDS the selection kernel needs for nb candidate blocks.
size_t select_lds_bytes(int nb);

void launch_pool_keys(const LaunchPool& a);
void launch_select(const LaunchSelect& a);
// chunk-shared selection (bf16; G of 1, 2, 4 or 8); false when unsupported
bool launch_select_shared(const LaunchSelect& a);
void launch_fetch(const LaunchFetch& a);
void launch_attn(const LaunchAttn& a);
void launch_qkv(const LaunchQkv& a);
void launch_step(const LaunchStep& a);

}  // namespace nosa
