// HBM block pool for NOSA offloading: set difference, slot choice, gather.
//
// NOSI keeps the KV cache in block-sized units on both GPU and CPU and swaps
// out only the blocks not used in the current step (montaan summary,
// "System Optimization (NOSI)" item 2); the blocks to move are found with
// set differences (gist.science summary, "2. Système : NOSI"), and the
// host-to-device transfer reads host memory directly through unified
// virtual addressing (montaan, item 3).
//
// Kernel 1 (one wavefront per (b, h)): the pool update of pool_dev.h.
//
// Kernel 2 (one workgroup per miss): copies the 64-token block from the
// pinned host cache into its pool slot with 16-byte loads through the GPU's
// mapping of host memory; all misses of all (b, h) are in flight together.
#include "nosa_common.h"
#include "nosa_launch.h"
#include "pool_dev.h"

namespace nosa {

constexpr int kGatherThreads = 256;

__global__ void __launch_bounds__(64) pool_update_kernel(
    int n_kv_heads, int nb, int P, int k_cap, int step, int32_t* __restrict__ block_table,
    int32_t* __restrict__ slot_block, int32_t* __restrict__ slot_last_use,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel,
    const int32_t* __restrict__ insert_block, int32_t* __restrict__ phys,
    int32_t* __restrict__ miss_list, int32_t* __restrict__ n_miss) {
  __shared__ PoolLds L;
  const int unit = blockIdx.x;
  const int lane = threadIdx.x;
  const PoolUnit u{nb, P, k_cap, step, block_table + (size_t)unit * nb, slot_block + (size_t)unit * P,
                   slot_last_use + (size_t)unit * P, miss_list + (size_t)unit * (k_cap + 1) * 2,
                   phys + (size_t)unit * k_cap, n_miss + unit};
  // every load that depends on nothing here goes out first (the selection,
  // its size and the inserted block, then the slot tables); the block-table
  // lookups that depend on them follow: two memory round trips before the
  // first decision
  const int n_raw = n_sel[unit];
  const int sel_raw = k_cap > 0 ? sel[(size_t)unit * k_cap + min(lane, k_cap - 1)] : -1;
  const int ins = pool_load(u, insert_block, unit / n_kv_heads, lane, L);
  pool_decide(u, lane, L, sel_raw, n_raw, ins, BlockSync{}, [&](int blk) { return u.bt[blk]; });
}

// One workgroup per (miss entry, unit); entry k_cap is the inserted block.
// The copy goes through u32x4 (nosa_common.h): a native vector stays in
// registers.

__global__ void __launch_bounds__(kGatherThreads) gather_kernel(
    const uint4* __restrict__ host_kv, uint4* __restrict__ pool, const uint4* __restrict__ insert_src,
    int nb, int P, int k_cap, int blk16, const int32_t* __restrict__ miss_list,
    const int32_t* __restrict__ n_miss) {
  const int e = blockIdx.x;
  const int unit = blockIdx.y;
  const int32_t* ml = miss_list + (size_t)unit * (k_cap + 1) * 2;
  const uint4* src;
  int slot;
  if (e < k_cap) {
    if (e >= n_miss[unit]) return;
    const int blk = ml[2 * e];
    slot = ml[2 * e + 1];
    if (blk < 0 || blk >= nb || slot < 0 || slot >= P) return;
    src = host_kv + ((size_t)unit * nb + blk) * blk16;
  } else {
    const int blk = ml[2 * e];
    slot = ml[2 * e + 1];
    if (insert_src == nullptr || blk < 0 || slot < 0 || slot >= P) return;
    src = insert_src + (size_t)unit * blk16;
  }
  const u32x4* src4 = reinterpret_cast<const u32x4*>(src);
  u32x4* dst4 = reinterpret_cast<u32x4*>(pool + ((size_t)unit * P + slot) * blk16);
  // U loads in flight per thread (2: with 4 or 8 the overlapped attention
  // and the link slow each other).  Loads and stores are unguarded, with the
  // same index clamped into the block: an index past the end rewrites the
  // block's last chunk with its own value.  (A guarded store lets the
  // compiler sink each load into its guard, which serialises the loads; the
  // scheduling barrier keeps the scheduler from pairing each store with its
  // load, which does the same.)
  constexpr int U = 2;
  for (int base = 0; base < blk16; base += kGatherThreads * U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src4[min(base + u * kGatherThreads + (int)threadIdx.x, blk16 - 1)];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) dst4[min(base + u * kGatherThreads + (int)threadIdx.x, blk16 - 1)] = v[u];
  }
}

void launch_fetch(const LaunchFetch& a) {
  const int units = a.batch * a.n_kv_heads;
  if (a.phases & 1)
    hipLaunchKernelGGL(pool_update_kernel, dim3(units), dim3(64), 0, a.stream, a.n_kv_heads, a.nb,
                       a.pool_slots, a.k_cap, a.step, a.block_table, a.slot_block, a.slot_last_use,
                       a.sel, a.n_sel, a.insert_block, a.phys, a.miss_list, a.n_miss);
  if (!(a.phases & 2)) return;
  const int esize = a.bf16 ? 2 : 4;
  const int blk16 = 2 * kBlock * a.head_dim * esize / 16;
  hipLaunchKernelGGL(gather_kernel, dim3(a.k_cap + 1, units), dim3(kGatherThreads), 0, a.stream,
                     (const uint4*)a.host_kv, (uint4*)a.pool, (const uint4*)a.insert_src, a.nb,
                     a.pool_slots, a.k_cap, blk16, a.miss_list, a.n_miss);
}

}  // namespace nosa
