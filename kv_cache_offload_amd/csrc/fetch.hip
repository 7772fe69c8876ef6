// HBM block pool for NOSA offloading: set difference, slot choice, gather.
//
// NOSI keeps the KV cache in block-sized units on both GPU and CPU and swaps
// out only the blocks not used in the current step (montaan summary,
// "System Optimization (NOSI)" item 2); the blocks to move are found with
// set differences (gist.science summary, "2. Système : NOSI"), and the
// host-to-device transfer reads host memory directly through unified
// virtual addressing (montaan, item 3).
//
// Kernel 1 (one wavefront per (b, h)): the selected set S arrives sorted, one
// entry per lane.  Membership is a table lookup (block_table), the misses are
// compacted with a ballot, the free slots are listed in ascending order, and
// the LRU victims among the evictable slots (resident, not in S) are found
// one at a time by a wavefront minimum of (last_use, block id) keys held in
// registers.  Miss i takes the i-th free slot, then the victims in order --
// the same outcome as assigning the misses one at a time.  Every table entry
// is written at most once per call.
//
// Kernel 2 (one workgroup per miss): copies the 64-token block from the
// pinned host cache into its pool slot with 16-byte loads through the GPU's
// mapping of host memory; all misses of all (b, h) are in flight together.
#include "nosa_common.h"
#include "nosa_launch.h"

namespace nosa {

constexpr int kMaxSlots = 1024;
constexpr int kGatherThreads = 256;

__device__ __forceinline__ uint64_t lru_key(int last_use, int block) {
  return ((uint64_t)((uint32_t)last_use ^ 0x80000000u) << 32) | (uint32_t)block;
}


// Minimum over the wavefront of a 64-bit key: the high words first, then the
// low words of the lanes holding that high word (two DPP reductions).
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  const uint32_t hi = wave_min_u32((uint32_t)(v >> 32));
  const uint32_t lo = wave_min_u32((uint32_t)(v >> 32) == hi ? (uint32_t)v : 0xffffffffu);
  return ((uint64_t)hi << 32) | lo;
}

__global__ void __launch_bounds__(64) pool_update_kernel(
    int n_kv_heads, int nb, int P, int k_cap, int step, int32_t* __restrict__ block_table,
    int32_t* __restrict__ slot_block, int32_t* __restrict__ slot_last_use,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel,
    const int32_t* __restrict__ insert_block, int32_t* __restrict__ phys,
    int32_t* __restrict__ miss_list, int32_t* __restrict__ n_miss) {
  __shared__ int s_blk[kMaxSlots], s_lu[kMaxSlots], s_free[kMaxSlots], s_vict[kMaxSlots];
  __shared__ uint8_t s_prot[kMaxSlots];
  const int unit = blockIdx.x;
  const int b = unit / n_kv_heads;
  const int lane = threadIdx.x;
  const uint64_t below = (1ull << lane) - 1ull;
  int32_t* bt = block_table + (size_t)unit * nb;
  int32_t* sb = slot_block + (size_t)unit * P;
  int32_t* lu = slot_last_use + (size_t)unit * P;
  int32_t* ml = miss_list + (size_t)unit * (k_cap + 1) * 2;

  // every load that depends on nothing here goes out first (the selection,
  // its size and the inserted block, then the slot tables), and the two
  // block-table lookups that depend on them go out together: two memory
  // round trips before the first decision
  const int n_raw = n_sel[unit];
  const int sel_raw = k_cap > 0 ? sel[(size_t)unit * k_cap + min(lane, k_cap - 1)] : -1;
  int ins = insert_block ? insert_block[b] : -1;
  for (int s = lane; s < P; s += 64) {
    s_blk[s] = sb[s];
    s_lu[s] = lu[s];
    s_prot[s] = 0;
  }

  // this lane's selected block (S arrives ascending; anything else is skipped)
  const int n = n_raw < 0 ? 0 : (n_raw > k_cap ? k_cap : n_raw);
  int blk = (lane < n) ? sel_raw : -1;
  if (blk >= nb) blk = -1;
  int prev_max = blk;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(prev_max, off);
    if (lane >= off) prev_max = max(prev_max, y);
  }
  int before_max = __shfl_up(prev_max, 1);
  if (lane == 0) before_max = -1;
  if (blk <= before_max) blk = -1;  // not strictly ascending: duplicate or out of order
  if (ins >= nb) ins = -1;
  const int bt_blk = blk >= 0 ? bt[blk] : -1;
  const int bt_ins = ins >= 0 ? bt[ins] : -1;
  __syncthreads();                  // the slot tables are in LDS
  int slot = -1;
  if (blk >= 0 && bt_blk >= 0 && bt_blk < P && s_blk[bt_blk] == blk) slot = bt_blk;
  if (slot >= 0) s_prot[slot] = 1;
  __syncthreads();

  // insertion of the block the window just completed
  if (ins >= 0 && bt_ins >= 0 && bt_ins < P && s_blk[bt_ins] == ins) ins = -1;  // already resident
  int ins_slot = -1, ins_old = -1;
  if (ins >= 0) {
    int fs = kMaxSlots;
    for (int s = lane; s < P; s += 64)
      if (s_blk[s] < 0) fs = min(fs, s);
    fs = (int)wave_min_u32((uint32_t)fs);   // slots and kMaxSlots are non-negative
    if (fs < kMaxSlots) {
      ins_slot = fs;
    } else {
      uint64_t best = ~0ull;
      for (int s = lane; s < P; s += 64)
        if (!s_prot[s]) {
          const uint64_t k = lru_key(s_lu[s], s_blk[s]);
          best = k < best ? k : best;
        }
      best = wave_min_u64(best);
      for (int s = lane; s < P; s += 64)
        if (!s_prot[s] && lru_key(s_lu[s], s_blk[s]) == best) ins_slot = s;
      const uint64_t found = __ballot(ins_slot >= 0);
      ins_slot = found ? __shfl(ins_slot, __ffsll((unsigned long long)found) - 1) : -1;
    }
    __syncthreads();
    if (ins_slot >= 0) {
      ins_old = s_blk[ins_slot];
      __syncthreads();
      if (lane == 0) {
        s_blk[ins_slot] = ins;
        s_lu[ins_slot] = step - 1;
      }
      if (blk == ins) {
        slot = ins_slot;
        s_prot[ins_slot] = 1;
      }
    }
  }
  __syncthreads();

  // misses, ascending, and the slots they take
  const bool miss = (blk >= 0) && (slot < 0);
  const uint64_t mmask = __ballot(miss);
  const int m = __popcll(mmask);
  const int rank = __popcll(mmask & below);
  int n_free = 0;
  for (int base = 0; base < P; base += 64) {
    const int s = base + lane;
    const bool fr = (s < P) && (s_blk[s] < 0);
    const uint64_t fm = __ballot(fr);
    if (fr) s_free[n_free + __popcll(fm & below)] = s;
    n_free += __popcll(fm);
  }
  const int need_v = m - n_free;
  if (need_v > 0) {
    // the need_v evictable slots (resident, not in S) in (last_use, block)
    // order: keys in registers (slot lane + 64 i), one wavefront minimum per
    // victim; keys are distinct because resident blocks are
    constexpr int kRegs = kMaxSlots / 64;
    const int n_regs = (P + 63) / 64;
    for (int r = lane; r < need_v; r += 64) s_vict[r] = -1;
    uint64_t key[kRegs];
#pragma unroll
    for (int i = 0; i < kRegs; ++i) {
      const int s = lane + 64 * i;
      key[i] = ~0ull;
      if (i < n_regs && s < P && s_blk[s] >= 0 && !s_prot[s]) key[i] = lru_key(s_lu[s], s_blk[s]);
    }
    for (int r = 0; r < need_v; ++r) {
      uint64_t best = ~0ull;
#pragma unroll
      for (int i = 0; i < kRegs; ++i)
        if (i < n_regs) best = key[i] < best ? key[i] : best;
      best = wave_min_u64(best);
      if (best == ~0ull) break;   // fewer evictable slots than misses (k > P is rejected on the host)
#pragma unroll
      for (int i = 0; i < kRegs; ++i)
        if (i < n_regs && key[i] == best) {
          s_vict[r] = lane + 64 * i;
          key[i] = ~0ull;
        }
    }
  }
  __syncthreads();
  int evicted_ins = 0;
  if (miss) {
    const int ts = (rank < n_free) ? s_free[rank] : s_vict[rank - n_free];   // >= 0: pool_slots > k_cap
    const int old = s_blk[ts];
    if (old >= 0 && old != ins) bt[old] = -1;
    evicted_ins = (ins >= 0 && old == ins);
    s_blk[ts] = blk;
    bt[blk] = ts;
    slot = ts;
    ml[2 * rank] = blk;
    ml[2 * rank + 1] = ts;
  }
  evicted_ins = __ballot(evicted_ins) != 0;
  __syncthreads();

  if (lane == 0 && ins_slot >= 0) {
    if (ins_old >= 0) bt[ins_old] = -1;
    if (!evicted_ins) bt[ins] = ins_slot;
    ml[2 * k_cap] = evicted_ins ? -1 : ins;
    ml[2 * k_cap + 1] = evicted_ins ? -1 : ins_slot;
  } else if (lane == 0) {
    ml[2 * k_cap] = -1;
    ml[2 * k_cap + 1] = -1;
  }
  for (int i = m + lane; i < k_cap; i += 64) {
    ml[2 * i] = -1;
    ml[2 * i + 1] = -1;
  }
  if (lane < k_cap) phys[(size_t)unit * k_cap + lane] = (lane < n) ? slot : -1;
  if (slot >= 0 && lane < n) s_lu[slot] = step;
  __syncthreads();
  for (int s = lane; s < P; s += 64) {
    sb[s] = s_blk[s];
    lu[s] = s_lu[s];
  }
  if (lane == 0) n_miss[unit] = m;
}

// One workgroup per (miss entry, unit); entry k_cap is the inserted block.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // a native vector stays in registers

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
