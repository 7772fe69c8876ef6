// Pool update of one (b, h) unit by one wavefront: set difference, slot
// choice, table writes.  Used by pool_update_kernel (its own launch) and by
// the selection kernel's last workgroup (selection and update in one launch).
//
// NOSI keeps the cache in block units on both sides and moves only the
// blocks the step uses that the GPU does not hold (montaan summary, "System
// Optimization (NOSI)" item 2), found as set differences (gist.science
// summary, "2. Système : NOSI").  The selected set S arrives sorted, one
// entry per lane.  Membership is a table lookup (block_table), the misses are
// compacted with a ballot, the free slots are listed in ascending order, and
// the LRU victims among the evictable slots (resident, not in S) are found
// one at a time by a wavefront minimum of (last_use, block id) keys held in
// registers.  Miss i takes the i-th free slot, then the victims in order --
// the same outcome as assigning the misses one at a time.  Every table entry
// is written at most once per call.
//
// Two phases, so a caller can issue the loads that do not depend on S before
// S exists: pool_load (slot tables into LDS, the inserted block), then
// pool_decide (everything that needs S).  `sync` orders the wavefront's LDS
// accesses between steps: a workgroup barrier when the workgroup is this one
// wavefront, a wavefront-local wait otherwise.
#pragma once
#include "nosa_common.h"

namespace nosa {

constexpr int kMaxSlots = 1024;

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

struct PoolLds {
  int blk[kMaxSlots], lu[kMaxSlots], free_slot[kMaxSlots], vict[kMaxSlots];
  uint8_t prot[kMaxSlots];
};

// One unit's pool: tables (read/written) and outputs.
struct PoolUnit {
  int nb, P, k_cap, step;
  int32_t* bt;        // block_table row [nb]
  int32_t* sb;        // slot_block row [P]
  int32_t* lu;        // slot_last_use row [P]
  int32_t* ml;        // miss_list row [k_cap + 1][2]
  int32_t* phys;      // phys row [k_cap]
  int32_t* n_miss;    // this unit's count
};

// Orders one wavefront's LDS accesses when other wavefronts of the
// workgroup have left: wait for its own LDS operations, and keep the
// compiler from moving memory accesses across.
struct WaveSync {
  __device__ __forceinline__ void operator()() const {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
  }
};
struct BlockSync {
  __device__ __forceinline__ void operator()() const { __syncthreads(); }
};

// Phase 1: the slot tables into LDS.  Returns the block to insert (-1: none).
__device__ __forceinline__ int pool_load(const PoolUnit& u, const int32_t* insert_block, int b, int lane,
                                         PoolLds& L) {
  const int ins = insert_block ? insert_block[b] : -1;
  for (int s = lane; s < u.P; s += 64) {
    L.blk[s] = u.sb[s];
    L.lu[s] = u.lu[s];
    L.prot[s] = 0;
  }
  return ins;
}

// Phase 2: sel_raw is this lane's entry of S (entries past n_raw ignored);
// slot_of(block) gives the block table's entry of a block in [0, nb).
template <class Sync, class SlotOf>
__device__ __forceinline__ void pool_decide(const PoolUnit& u, int lane, PoolLds& L, int sel_raw, int n_raw,
                                            int ins, Sync sync, SlotOf slot_of) {
  const int nb = u.nb, P = u.P, k_cap = u.k_cap, step = u.step;
  int32_t* bt = u.bt;
  int32_t* ml = u.ml;
  const uint64_t below = (1ull << lane) - 1ull;

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
  // the two block-table lookups that depend on S go out together
  const int bt_blk = blk >= 0 ? slot_of(blk) : -1;
  const int bt_ins = ins >= 0 ? slot_of(ins) : -1;
  sync();                           // the slot tables are in LDS
  int slot = -1;
  if (blk >= 0 && bt_blk >= 0 && bt_blk < P && L.blk[bt_blk] == blk) slot = bt_blk;
  if (slot >= 0) L.prot[slot] = 1;
  sync();

  // insertion of the block the window just completed
  if (ins >= 0 && bt_ins >= 0 && bt_ins < P && L.blk[bt_ins] == ins) ins = -1;  // already resident
  int ins_slot = -1, ins_old = -1;
  if (ins >= 0) {
    int fs = kMaxSlots;
    for (int s = lane; s < P; s += 64)
      if (L.blk[s] < 0) fs = min(fs, s);
    fs = (int)wave_min_u32((uint32_t)fs);   // slots and kMaxSlots are non-negative
    if (fs < kMaxSlots) {
      ins_slot = fs;
    } else {
      uint64_t best = ~0ull;
      for (int s = lane; s < P; s += 64)
        if (!L.prot[s]) {
          const uint64_t k = lru_key(L.lu[s], L.blk[s]);
          best = k < best ? k : best;
        }
      best = wave_min_u64(best);
      for (int s = lane; s < P; s += 64)
        if (!L.prot[s] && lru_key(L.lu[s], L.blk[s]) == best) ins_slot = s;
      const uint64_t found = __ballot(ins_slot >= 0);
      ins_slot = found ? __shfl(ins_slot, __ffsll((unsigned long long)found) - 1) : -1;
    }
    sync();
    if (ins_slot >= 0) {
      ins_old = L.blk[ins_slot];
      sync();
      if (lane == 0) {
        L.blk[ins_slot] = ins;
        L.lu[ins_slot] = step - 1;
      }
      if (blk == ins) {
        slot = ins_slot;
        L.prot[ins_slot] = 1;
      }
    }
  }
  sync();

  // misses, ascending, and the slots they take
  const bool miss = (blk >= 0) && (slot < 0);
  const uint64_t mmask = __ballot(miss);
  const int m = __popcll(mmask);
  const int rank = __popcll(mmask & below);
  int n_free = 0;
  for (int base = 0; base < P; base += 64) {
    const int s = base + lane;
    const bool fr = (s < P) && (L.blk[s] < 0);
    const uint64_t fm = __ballot(fr);
    if (fr) L.free_slot[n_free + __popcll(fm & below)] = s;
    n_free += __popcll(fm);
  }
  const int need_v = m - n_free;
  if (need_v > 0) {
    // the need_v evictable slots (resident, not in S) in (last_use, block)
    // order: keys in registers (slot lane + 64 i), one wavefront minimum per
    // victim; keys are distinct because resident blocks are
    constexpr int kRegs = kMaxSlots / 64;
    const int n_regs = (P + 63) / 64;
    for (int r = lane; r < need_v; r += 64) L.vict[r] = -1;
    uint64_t key[kRegs];
#pragma unroll
    for (int i = 0; i < kRegs; ++i) {
      const int s = lane + 64 * i;
      key[i] = ~0ull;
      if (i < n_regs && s < P && L.blk[s] >= 0 && !L.prot[s]) key[i] = lru_key(L.lu[s], L.blk[s]);
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
          L.vict[r] = lane + 64 * i;
          key[i] = ~0ull;
        }
    }
  }
  sync();
  int evicted_ins = 0;
  if (miss) {
    const int ts = (rank < n_free) ? L.free_slot[rank] : L.vict[rank - n_free];   // >= 0: pool_slots > k_cap
    const int old = L.blk[ts];
    if (old >= 0 && old != ins) bt[old] = -1;
    evicted_ins = (ins >= 0 && old == ins);
    L.blk[ts] = blk;
    bt[blk] = ts;
    slot = ts;
    ml[2 * rank] = blk;
    ml[2 * rank + 1] = ts;
  }
  evicted_ins = __ballot(evicted_ins) != 0;
  sync();

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
  if (lane < k_cap) u.phys[lane] = (lane < n) ? slot : -1;
  if (slot >= 0 && lane < n) L.lu[slot] = step;
  sync();
  for (int s = lane; s < P; s += 64) {
    u.sb[s] = L.blk[s];
    u.lu[s] = L.lu[s];
  }
  if (lane == 0) *u.n_miss = m;
}

}  // namespace nosa
