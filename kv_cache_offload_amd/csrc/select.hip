// Block selection for NOSA decode: query-aware top-kq U query-agnostic top-ke.
//
// Eq. 7 of NOSA (montaan summary, "Key Design Components" item 4) picks up to
// k blocks: kq by the query's block scores, ke by the eviction-head scores.
// Both rank pre-exponential scores (ED-DMA, gist.science summary), so no exp
// or softmax appears here.  The block score is the max over the block's four
// sub-block scores qsum . kbar (two-stage pooling, same summary).
//
// Grid = (splits, query rows x KV heads), 1024 threads per workgroup.
//  * The scan of a (row, KV head) is split over workgroups of ~128 blocks;
//    each publishes its block scores with coherent stores and the workgroup
//    that draws the last ticket selects.  With a single split the scores
//    never leave LDS.
//  * Scan (select_dev.h): bf16 takes 16-row tiles of the compressed keys as
//    the A operand of v_mfma_f32_16x16x32_bf16 with the G query heads as B,
//    sums the heads by DPP and takes a block's max over its four rows in one
//    lane group; fp32 dots each row with the summed query (FMAs, DPP sums).
//  * Selection: each half of the workgroup (one per budget) bins its scores
//    into 256 equal value bins between their min and max, finds the bin
//    holding the k-th best, takes every block above it and ranks the few
//    blocks inside it exactly by (score desc, id asc).  The union is then
//    written in ascending order with one prefix sum.
#include "nosa_common.h"
#include "nosa_launch.h"
#include "select_dev.h"
#include "pool_dev.h"

namespace nosa {

constexpr int kSelThreads = 1024;
constexpr int kMaxSelectBlocks = 4096;  // nb limit of the selection (256K tokens)
constexpr int kMaxPoolK = 64;           // kq + ke limit of the pool update
constexpr int kHalf = kSelThreads / 2;

size_t select_ws_bytes(int batch, int n_query, int n_kv_heads, int nb) {
  const size_t rows = (size_t)batch * n_query * n_kv_heads;
  // tickets, scores per row and block, and (chunk-shared selection) 16
  // partial sums of the query heads, up to 128 fp32 dimensions, per unit
  return rows * kTicketBytes + align256(rows * (size_t)nb * sizeof(float)) +
         align256((size_t)16 * batch * n_kv_heads * 128 * sizeof(float));
}

size_t select_lds_bytes(int nb) {
  // two key arrays (4 B per block), two boundary lists (2 B), two flag arrays (1 B)
  return align256((size_t)nb * 4) * 2 + align256((size_t)nb * 2) * 2 + align256((size_t)nb) * 2;
}

// Scan splits per row: about 128 blocks per workgroup, at most 16, and no
// more workgroups than CUs in all: a second round of 1024-thread workgroups
// costs more than scanning twice the blocks in one (measured: 32 rows of
// 2048 candidates 34.0 -> 22.5 us, 128 rows of 256 22.5 -> 15.0 us, 16 rows
// of 512 unchanged at 12.5 us).
static int select_splits(int rows, int nb) {
  int s = (nb + 127) / 128;
  s = s < 1 ? 1 : (s > 16 ? 16 : s);
  while (s > 1 && rows * s > 256) --s;
  return s;
}

// The pool update of a decode step (one query row per unit), run by
// wavefront 0 of the workgroup that selects (see pool_dev.h).
struct SelPool {
  int P, step;
  int32_t *block_table, *slot_block, *slot_last_use;
  const int32_t* insert_block;
  int32_t *phys, *miss_list, *n_miss;
};

template <class T, int D, bool POOL>
__global__ void __launch_bounds__(kSelThreads) select_kernel(
    const typename T::storage* __restrict__ q, const int32_t* __restrict__ pos,
    const typename T::storage* __restrict__ k_comp, const float* __restrict__ e_blk, int n_query,
    int n_q_heads, int n_kv_heads, int nb, int kq, int ke, int fill, int32_t* __restrict__ sel,
    int32_t* __restrict__ n_sel, int32_t* __restrict__ ticket, float* __restrict__ score, SelPool pl) {
  const int G = n_q_heads / n_kv_heads;
  const int row = blockIdx.y;             // (b * n_query + r) * Hkv + h
  const int h = row % n_kv_heads;
  const int br = row / n_kv_heads;        // b * n_query + r
  const int b = br / n_query;
  const int64_t unit = (int64_t)b * n_kv_heads + h;
  const int k_cap = kq + ke;
  const int tid = threadIdx.x;
  const int n_split = gridDim.x;

  const int p = pos[br];
  const int c = (p >= 0 && p < nb * kBlock) ? p / kBlock : 0;
  const int bps = (nb + n_split - 1) / n_split;     // blocks per split
  const int blk_lo = min(c, (int)blockIdx.x * bps);
  const int blk_hi = min(c, blk_lo + bps);

  extern __shared__ __align__(16) unsigned char lds[];
  const size_t kb = align256((size_t)nb * 4), lb = align256((size_t)nb * 2);
  uint32_t* key_q = reinterpret_cast<uint32_t*>(lds);
  uint32_t* key_e = reinterpret_cast<uint32_t*>(lds + kb);
  uint16_t* blist_q = reinterpret_cast<uint16_t*>(lds + 2 * kb);
  uint16_t* blist_e = reinterpret_cast<uint16_t*>(lds + 2 * kb + lb);
  uint8_t* flag_q = lds + 2 * kb + 2 * lb;
  uint8_t* flag_e = flag_q + align256((size_t)nb);
  __shared__ int s_hist[2][kBins];
  __shared__ int s_small[2][32];
  __shared__ int s_wsum[kSelThreads / 64];
  float* my_score = score + (size_t)row * nb;
  [[maybe_unused]] PoolLds* pool_lds = nullptr;

  // block eviction scores and cleared flags first, so their loads overlap the scan
  const float* eb = e_blk + (size_t)unit * nb;
  if (n_split == 1 || blockIdx.x == 0) {
    for (int j = tid; j < c; j += kSelThreads) {
      key_e[j] = orderable(eb[j]);
      flag_q[j] = 0;
      flag_e[j] = 0;
    }
  }

  // ---- scan: block scores of blocks [blk_lo, blk_hi)
  if (blk_lo < blk_hi) {
    const typename T::storage* qh = q + ((size_t)br * n_q_heads + (size_t)h * G) * D;
    const typename T::storage* kc = k_comp + (size_t)unit * nb * kSubsPerBlock * D;
    if (n_split == 1)
      scan_block_scores<T, D, kSelThreads>(qh, G, kc, kSubsPerBlock * blk_lo, kSubsPerBlock * blk_hi, tid,
                                          [&](int blk, float s) { key_q[blk] = orderable(s); });
    else
      scan_block_scores<T, D, kSelThreads>(qh, G, kc, kSubsPerBlock * blk_lo, kSubsPerBlock * blk_hi, tid,
                                          [&](int blk, float s) { store_coherent(&my_score[blk], s); });
  }

  if (n_split > 1) {
    // ---- ticket: the last workgroup of this row selects
    __shared__ int s_last;
    wait_stores_done();
    __syncthreads();
    if (tid == 0) {
      const int t = ticket_take(&ticket[(size_t)row * kTicketInts]);
      s_last = (t == n_split - 1);
      if (s_last) ticket_reset(&ticket[(size_t)row * kTicketInts]);
    }
    __syncthreads();
    if (!s_last) return;
    for (int j = tid; j < c; j += kSelThreads) {
      key_q[j] = orderable(load_coherent(&my_score[j]));
      if (blockIdx.x != 0) {  // only split 0 prepared these
        key_e[j] = orderable(eb[j]);
        flag_q[j] = 0;
        flag_e[j] = 0;
      }
    }
  }
  // pool update, phase 1: the slot tables go to LDS (wavefront 0) while the
  // scores above are still arriving, and a block -> slot map of the unit's
  // candidates is cleared (every thread), so the update needs no memory
  // round trip once the set is known
  [[maybe_unused]] PoolUnit pu;
  [[maybe_unused]] int p_ins = -1;
  [[maybe_unused]] int16_t* slot_map = nullptr;
  [[maybe_unused]] int32_t* union_ids = nullptr;
  if constexpr (POOL) {
    __shared__ PoolLds s_pool;
    __shared__ int16_t s_map[kMaxSelectBlocks];
    __shared__ int32_t s_union[kMaxPoolK];
    pu = PoolUnit{nb, pl.P, k_cap, pl.step, pl.block_table + (size_t)unit * nb, pl.slot_block + (size_t)unit * pl.P,
                  pl.slot_last_use + (size_t)unit * pl.P, pl.miss_list + (size_t)unit * (k_cap + 1) * 2,
                  pl.phys + (size_t)unit * k_cap, pl.n_miss + unit};
    if (tid < 64) p_ins = pool_load(pu, pl.insert_block, b, tid, s_pool);
    for (int i = tid; i < nb; i += kSelThreads) s_map[i] = -1;
    pool_lds = &s_pool;
    slot_map = s_map;
    union_ids = s_union;
  }
  __syncthreads();
  const int half = tid / kHalf;
  // the fill variant takes the eviction scores' top ke + nq, trimmed below
  const int ke_top = fill ? min(c, ke + min(kq, c)) : ke;
  select_top<kHalf>(half ? key_e : key_q, c, half ? ke_top : kq, half ? flag_e : flag_q, s_hist[half],
                    s_small[half], half ? blist_e : blist_q, tid % kHalf);
  if (fill) keep_fill<kSelThreads>(key_e, flag_q, flag_e, c, ke, reinterpret_cast<int32_t*>(key_q), s_wsum, tid);

  // ---- union in ascending order
  if constexpr (!POOL) {
    const int total = write_union<kSelThreads>(flag_q, flag_e, c, sel + (size_t)row * k_cap, k_cap, s_wsum, tid);
    if (tid == 0) n_sel[row] = total;
  } else {
    // the union into LDS, then out; pool update, phase 2 (wavefront 0) on it
    const int total = write_union<kSelThreads>(flag_q, flag_e, c, union_ids, k_cap, s_wsum, tid);
    __syncthreads();
    int32_t* sr = sel + (size_t)row * k_cap;
    for (int i = tid; i < k_cap; i += kSelThreads) sr[i] = union_ids[i];
    if (tid == 0) n_sel[row] = total;
    if (tid >= 64) return;
    PoolLds& L = *pool_lds;
    for (int s = tid; s < pu.P; s += 64) {
      const int blk = L.blk[s];
      if (blk >= 0 && blk < nb) slot_map[blk] = (int16_t)s;
    }
    WaveSync{}();
    const int sel_raw = k_cap > 0 ? union_ids[min(tid, k_cap - 1)] : -1;
    pool_decide(pu, tid, L, sel_raw, total, p_ins, WaveSync{}, [&](int blk) { return (int)slot_map[blk]; });
  }
}

// ---------------------------------------------------------------------------
// Many query rows per KV head (a prefill chunk): the compressed keys are
// scanned once per chunk of query rows instead of once per row.
//   mscan_kernel  grid (splits, units, row chunks): a 16-row tile of K-bar
//                 (MFMA operand A, loaded once) times the query heads of
//                 16/G rows at a time (operand B), per-row head sums over G
//                 lanes (DPP, the same tree as the single-row scan, so the
//                 scores are identical), max over the block's four rows;
//                 scores go to the workspace [row][block].
//   mtopk_kernel  one workgroup per row: top-kq of its scores and top-ke of E
//                 over its candidates, union ascending (as select_kernel).
constexpr int kMRows = 8;          // query rows per scan workgroup (at least one MFMA column block)
constexpr int kMThreads = 512;
constexpr int kTopkThreads = 1024;  // top-k workgroups, as select_kernel (512: +1.2 us per call at prefill128k)
__host__ __device__ constexpr int mrows_per_chunk(int G) { return 16 / G > kMRows ? 16 / G : kMRows; }

template <int G>
__device__ __forceinline__ float head_sum(float v) {
  if constexpr (G >= 16) return group_sum<16>(v);
  else if constexpr (G >= 8) return group_sum<8>(v);
  else if constexpr (G >= 4) return group_sum<4>(v);
  else if constexpr (G >= 2) return group_sum<2>(v);
  else return v;
}

template <int D, int G>
__global__ void __launch_bounds__(kMThreads) mscan_kernel(const uint16_t* __restrict__ q, const int32_t* __restrict__ pos,
                                                          const uint16_t* __restrict__ k_comp, int n_query,
                                                          int n_q_heads, int n_kv_heads, int nb, float* __restrict__ score) {
  constexpr int NK = D / 32;
  constexpr int QPB = 16 / G;       // query rows per 16-column MFMA block
  constexpr int RPC = mrows_per_chunk(G);
  constexpr int NCB = RPC / QPB;    // column blocks per chunk
  constexpr int WAVES = kMThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int n_split = gridDim.x;
  const int unit = blockIdx.y;       // b * Hkv + h
  const int b = unit / n_kv_heads, h = unit % n_kv_heads;
  const int r0 = blockIdx.z * RPC;
  // the scan covers blocks below the largest window of the chunk
  int cmax = 0;
  for (int r = r0; r < min(n_query, r0 + RPC); ++r) {
    const int p = pos[(size_t)b * n_query + r];
    const int c = (p >= 0 && p < nb * kBlock) ? p / kBlock : 0;
    cmax = max(cmax, c);
  }
  const int bps = (nb + n_split - 1) / n_split;
  const int blk_lo = min(cmax, (int)blockIdx.x * bps), blk_hi = min(cmax, blk_lo + bps);
  if (blk_lo >= blk_hi) return;
  const int row_lo = kSubsPerBlock * blk_lo, row_hi = kSubsPerBlock * blk_hi;
  const uint16_t* kc = k_comp + (size_t)unit * nb * kSubsPerBlock * D;
  // B operands of the chunk: column block cb, lane column col -> row r0 + cb*QPB + col/G, head col%G
  bf16x8 qf[NCB][NK];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int r = r0 + cb * QPB + col / G;
    const int hd = h * G + col % G;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const uint4 u = r < n_query ? ld16(q + (((size_t)b * n_query + r) * n_q_heads + hd) * D + 32 * s + 8 * grp)
                                  : make_uint4(0, 0, 0, 0);
      qf[cb][s] = __builtin_bit_cast(bf16x8, u);
    }
  }
  const int n_tiles = (row_hi - row_lo + 15) / 16;
  for (int tile = wave; tile < n_tiles; tile += WAVES) {
    const int row = min(row_lo + 16 * tile + col, row_hi - 1);
    uint4 ka[NK];
#pragma unroll
    for (int s = 0; s < NK; ++s) ka[s] = ld16(kc + (size_t)row * D + 32 * s + 8 * grp);
    const int rowb = row_lo + 16 * tile + 4 * grp;   // first row of this lane group's block
    const int blk = rowb / kSubsPerBlock;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NK; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[s]), qf[cb][s], acc, 0, 0, 0);
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, head_sum<G>(acc[i]));
      const int r = r0 + cb * QPB + col / G;
      if (col % G == 0 && r < n_query && rowb < row_hi)
        score[(((size_t)b * n_query + r) * n_kv_heads + h) * nb + blk] = m;
    }
  }
}

template <class T>
__global__ void __launch_bounds__(kTopkThreads) mtopk_kernel(const int32_t* __restrict__ pos, const float* __restrict__ e_blk,
                                                          const float* __restrict__ score, int n_query, int n_kv_heads,
                                                          int nb, int kq, int ke, int fill, int32_t* __restrict__ sel,
                                                          int32_t* __restrict__ n_sel) {
  constexpr int kH = kTopkThreads / 2;
  const int row = blockIdx.x;               // (b * n_query + r) * Hkv + h
  const int h = row % n_kv_heads;
  const int br = row / n_kv_heads;
  const int b = br / n_query;
  const int64_t unit = (int64_t)b * n_kv_heads + h;
  const int tid = threadIdx.x;
  const int k_cap = kq + ke;
  const int p = pos[br];
  const int c = (p >= 0 && p < nb * kBlock) ? p / kBlock : 0;
  extern __shared__ __align__(16) unsigned char lds[];
  const size_t kb = align256((size_t)nb * 4), lb = align256((size_t)nb * 2);
  uint32_t* key_q = reinterpret_cast<uint32_t*>(lds);
  uint32_t* key_e = reinterpret_cast<uint32_t*>(lds + kb);
  uint16_t* blist_q = reinterpret_cast<uint16_t*>(lds + 2 * kb);
  uint16_t* blist_e = reinterpret_cast<uint16_t*>(lds + 2 * kb + lb);
  uint8_t* flag_q = lds + 2 * kb + 2 * lb;
  uint8_t* flag_e = flag_q + align256((size_t)nb);
  __shared__ int s_hist[2][kBins];
  __shared__ int s_small[2][32];
  __shared__ int s_wsum[kTopkThreads / 64];
  const float* sc = score + (size_t)row * nb;
  const float* eb = e_blk + (size_t)unit * nb;
  for (int j = tid; j < c; j += kTopkThreads) {
    key_q[j] = orderable(sc[j]);
    key_e[j] = orderable(eb[j]);
    flag_q[j] = 0;
    flag_e[j] = 0;
  }
  __syncthreads();
  const int half = tid / kH;
  const int ke_top = fill ? min(c, ke + min(kq, c)) : ke;
  select_top<kH>(half ? key_e : key_q, c, half ? ke_top : kq, half ? flag_e : flag_q, s_hist[half], s_small[half],
                 half ? blist_e : blist_q, tid % kH);
  if (fill) keep_fill<kTopkThreads>(key_e, flag_q, flag_e, c, ke, reinterpret_cast<int32_t*>(key_q), s_wsum, tid);
  const int total = write_union<kTopkThreads>(flag_q, flag_e, c, sel + (size_t)row * k_cap, k_cap, s_wsum, tid);
  if (tid == 0) n_sel[row] = total;
}

template <int D>
static bool launch_multi(const LaunchSelect& a) {
  const int G = a.n_q_heads / a.n_kv_heads;
  const int rows = a.batch * a.n_query * a.n_kv_heads;
  const int units = a.batch * a.n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  const int chunks = (a.n_query + mrows_per_chunk(G) - 1) / mrows_per_chunk(G);
  int splits = (a.nb + 127) / 128;
  splits = splits < 1 ? 1 : (splits > 32 ? 32 : splits);
  char* ws = (char*)a.ws;
  float* score = (float*)(ws + (size_t)rows * kTicketBytes);
  const dim3 grid(splits, units, chunks);
  const uint16_t* q = (const uint16_t*)a.q;
  const uint16_t* kc = (const uint16_t*)a.k_comp;
  switch (G) {
    case 1: hipLaunchKernelGGL((mscan_kernel<D, 1>), grid, dim3(kMThreads), 0, a.stream, q, a.pos, kc, a.n_query, a.n_q_heads, a.n_kv_heads, a.nb, score); break;
    case 2: hipLaunchKernelGGL((mscan_kernel<D, 2>), grid, dim3(kMThreads), 0, a.stream, q, a.pos, kc, a.n_query, a.n_q_heads, a.n_kv_heads, a.nb, score); break;
    case 4: hipLaunchKernelGGL((mscan_kernel<D, 4>), grid, dim3(kMThreads), 0, a.stream, q, a.pos, kc, a.n_query, a.n_q_heads, a.n_kv_heads, a.nb, score); break;
    case 8: hipLaunchKernelGGL((mscan_kernel<D, 8>), grid, dim3(kMThreads), 0, a.stream, q, a.pos, kc, a.n_query, a.n_q_heads, a.n_kv_heads, a.nb, score); break;
    default: return false;
  }
  hipLaunchKernelGGL((mtopk_kernel<Bf16>), dim3(rows), dim3(kTopkThreads), select_lds_bytes(a.nb), a.stream, a.pos,
                     a.e_blk, score, a.n_query, a.n_kv_heads, a.nb, a.kq, a.ke, a.fill ? 1 : 0, a.sel, a.n_sel);
  return true;
}

// ---------------------------------------------------------------------------
// Chunk-shared selection: one selection for all n_query rows of a unit,
// scored with the sum of every row's G query heads.
//   qsum_kernel         grid (kQsumParts, units): part z sums, in fp32, its
//                       share of the unit's n_query*G query heads (each
//                       thread 8 dimensions of every 32nd head of the share,
//                       in head order, then the thread sums added in order);
//   shared_scan_kernel  grid (splits, units): adds the kQsumParts partial
//                       sums in order, then each 16-lane group (8 for D = 64)
//                       dots one sub-block row of K-bar with the summed query
//                       (fp32 FMAs, DPP sum); a block's score is the max of
//                       its four rows;
//   mtopk_shared_kernel one workgroup per unit: top-kq / top-ke over the
//                       first row's candidates, the union written to every row.
constexpr int kQsumThreads = 512;
constexpr int kQsumParts = 16;                     // workgroups per unit summing the chunk's query heads

template <int D>
__global__ void __launch_bounds__(kQsumThreads) qsum_kernel(const uint16_t* __restrict__ q, int n_query, int n_q_heads,
                                                            int n_kv_heads, float* __restrict__ qsum) {
  constexpr int CPR = D / 8;                       // 16-byte chunks per head
  constexpr int SLOTS = kQsumThreads / CPR;        // heads summed side by side
  __shared__ float s_part[SLOTS][D];
  const int z = blockIdx.x, unit = blockIdx.y, b = unit / n_kv_heads, h = unit % n_kv_heads;
  const int G = n_q_heads / n_kv_heads, n_heads = n_query * G;
  const int per = (n_heads + kQsumParts - 1) / kQsumParts;
  const int i_lo = z * per, i_hi = min(n_heads, i_lo + per);
  const int ch = threadIdx.x % CPR, slot = threadIdx.x / CPR;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int i = i_lo + slot; i < i_hi; i += SLOTS) {   // head i: row i / G, head h*G + i % G
    const int r = i / G, g = i % G;
    float v[8];
    unpack16(ld16(q + (((size_t)b * n_query + r) * n_q_heads + h * G + g) * D + 8 * ch), v, Bf16{});
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += v[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_part[slot][8 * ch + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float t = 0.f;
    for (int k = 0; k < SLOTS; ++k) t += s_part[k][threadIdx.x];
    qsum[((size_t)z * gridDim.y + unit) * D + threadIdx.x] = t;
  }
}

template <int D>
__global__ void __launch_bounds__(kMThreads) shared_scan_kernel(const int32_t* __restrict__ pos,
                                                                const uint16_t* __restrict__ k_comp,
                                                                const float* __restrict__ qsum, int n_query,
                                                                int n_kv_heads, int nb, float* __restrict__ score) {
  constexpr int LPR = D / 8;                       // lanes per sub-block row, 8 dimensions each
  constexpr int BPW = 64 / (LPR * kSubsPerBlock);  // blocks per wavefront load (1 or 2)
  constexpr int WAVES = kMThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int unit = blockIdx.y, b = unit / n_kv_heads;
  const int p = pos[(size_t)b * n_query];          // the first row's window bounds the candidates
  const int c = (p >= 0 && p < nb * kBlock) ? p / kBlock : 0;
  const int bps = (nb + gridDim.x - 1) / gridDim.x;
  const int blk_lo = min(c, (int)blockIdx.x * bps), blk_hi = min(c, blk_lo + bps);
  if (blk_lo >= blk_hi) return;
  const int ch = lane % LPR, rw = lane / LPR;      // dimensions 8ch.. of row rw of a load
  float qv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  {
    float4 x[kQsumParts][2];
#pragma unroll
    for (int z = 0; z < kQsumParts; ++z) {
      const float* src = qsum + ((size_t)z * gridDim.y + unit) * D + 8 * ch;
      x[z][0] = *reinterpret_cast<const float4*>(src);
      x[z][1] = *reinterpret_cast<const float4*>(src + 4);
    }
#pragma unroll
    for (int z = 0; z < kQsumParts; ++z) {         // the parts in order
      qv[0] += x[z][0].x; qv[1] += x[z][0].y; qv[2] += x[z][0].z; qv[3] += x[z][0].w;
      qv[4] += x[z][1].x; qv[5] += x[z][1].y; qv[6] += x[z][1].z; qv[7] += x[z][1].w;
    }
  }
  const uint16_t* kc = k_comp + (size_t)unit * nb * kSubsPerBlock * D;
  constexpr int U = 4;                             // loads in flight per lane
  constexpr int STEP = WAVES * BPW;
  for (int jb = blk_lo + wave * BPW; jb < blk_hi; jb += STEP * U) {      // uniform over the wavefront
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {                  // rows clamped, results past blk_hi dropped
      const int row = min(kSubsPerBlock * (jb + u * STEP) + rw, kSubsPerBlock * blk_hi - 1);
      raw[u] = ld16(kc + (size_t)row * D + 8 * ch);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j0 = jb + u * STEP;
      float v[8];
      unpack16(raw[u], v, Bf16{});
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(qv[e], v[e], d);
      d = group_sum<LPR>(d);                       // the row's score in every lane of its group
#pragma unroll
      for (int bi = 0; bi < BPW; ++bi) {
        float m = lane_value(d, 4 * bi * LPR);
#pragma unroll
        for (int i = 1; i < kSubsPerBlock; ++i) m = fmaxf(m, lane_value(d, (4 * bi + i) * LPR));
        if (lane == 0 && j0 + bi < blk_hi) score[(size_t)unit * nb + j0 + bi] = m;
      }
    }
  }
}

// One workgroup per unit (b, h): the shared selection of all n_query rows.
__global__ void __launch_bounds__(kTopkThreads) mtopk_shared_kernel(const int32_t* __restrict__ pos,
                                                                 const float* __restrict__ e_blk,
                                                                 const float* __restrict__ score, int n_query,
                                                                 int n_kv_heads, int nb, int kq, int ke,
                                                                 int32_t* __restrict__ sel, int32_t* __restrict__ n_sel) {
  constexpr int kH = kTopkThreads / 2;
  const int unit = blockIdx.x;              // b * Hkv + h
  const int b = unit / n_kv_heads, h = unit % n_kv_heads;
  const int tid = threadIdx.x;
  const int k_cap = kq + ke;
  const int p = pos[(size_t)b * n_query];
  const int c = (p >= 0 && p < nb * kBlock) ? p / kBlock : 0;
  extern __shared__ __align__(16) unsigned char lds[];
  const size_t kb = align256((size_t)nb * 4), lb = align256((size_t)nb * 2);
  uint32_t* key_q = reinterpret_cast<uint32_t*>(lds);
  uint32_t* key_e = reinterpret_cast<uint32_t*>(lds + kb);
  uint16_t* blist_q = reinterpret_cast<uint16_t*>(lds + 2 * kb);
  uint16_t* blist_e = reinterpret_cast<uint16_t*>(lds + 2 * kb + lb);
  uint8_t* flag_q = lds + 2 * kb + 2 * lb;
  uint8_t* flag_e = flag_q + align256((size_t)nb);
  __shared__ int s_hist[2][kBins];
  __shared__ int s_small[2][32];
  __shared__ int s_wsum[kTopkThreads / 64];
  const float* sc = score + (size_t)unit * nb;
  const float* eb = e_blk + (size_t)unit * nb;
  for (int j = tid; j < c; j += kTopkThreads) {
    key_q[j] = orderable(sc[j]);
    key_e[j] = orderable(eb[j]);
    flag_q[j] = 0;
    flag_e[j] = 0;
  }
  __syncthreads();
  const int half = tid / kH;
  select_top<kH>(half ? key_e : key_q, c, half ? ke : kq, half ? flag_e : flag_q, s_hist[half], s_small[half],
                 half ? blist_e : blist_q, tid % kH);
  // the union goes to LDS first, over the dead score keys (write_union
  // writes only after its own barrier, when every top-k pass is done; it has
  // at most min(k_cap, c) <= nb members)
  int32_t* s_list = reinterpret_cast<int32_t*>(key_q);
  const int total = write_union<kTopkThreads>(flag_q, flag_e, c, s_list, min(k_cap, nb), s_wsum, tid);
  __syncthreads();
  for (int i = tid; i < n_query * k_cap; i += kTopkThreads) {
    const int r = i / k_cap, k = i % k_cap;
    sel[(((size_t)b * n_query + r) * n_kv_heads + h) * k_cap + k] = k < total ? s_list[k] : -1;
  }
  for (int r = tid; r < n_query; r += kTopkThreads) n_sel[((size_t)b * n_query + r) * n_kv_heads + h] = total;
}

template <int D>
static void launch_shared(const LaunchSelect& a) {
  const int units = a.batch * a.n_kv_heads;
  const size_t rows = (size_t)a.batch * a.n_query * a.n_kv_heads;
  char* ws = (char*)a.ws;
  float* score = (float*)(ws + (size_t)rows * kTicketBytes);
  float* qs = (float*)(ws + (size_t)rows * kTicketBytes + align256(rows * (size_t)a.nb * sizeof(float)));
  const uint16_t* q = (const uint16_t*)a.q;
  hipLaunchKernelGGL((qsum_kernel<D>), dim3(kQsumParts, units), dim3(kQsumThreads), 0, a.stream, q, a.n_query,
                     a.n_q_heads, a.n_kv_heads, qs);
  // about 4 blocks per wavefront, at most 512 workgroups in all
  int splits = (a.nb + 31) / 32;
  const int cap = 512 / units > 1 ? 512 / units : 1;
  splits = splits < 1 ? 1 : (splits > cap ? cap : splits);
  hipLaunchKernelGGL((shared_scan_kernel<D>), dim3(splits, units), dim3(kMThreads), 0, a.stream, a.pos,
                     (const uint16_t*)a.k_comp, qs, a.n_query, a.n_kv_heads, a.nb, score);
  hipLaunchKernelGGL(mtopk_shared_kernel, dim3(units), dim3(kTopkThreads), select_lds_bytes(a.nb), a.stream, a.pos,
                     a.e_blk, score, a.n_query, a.n_kv_heads, a.nb, a.kq, a.ke, a.sel, a.n_sel);
}

bool launch_select_shared(const LaunchSelect& a) {
  const int G = a.n_q_heads / a.n_kv_heads;
  if (!a.bf16 || (G != 1 && G != 2 && G != 4 && G != 8)) return false;
  if (a.head_dim == 128) launch_shared<128>(a); else launch_shared<64>(a);
  return true;
}

template <class T, int D>
static void launch(const LaunchSelect& a) {
  const int rows = a.batch * a.n_query * a.n_kv_heads;
  const int splits = select_splits(rows, a.nb);
  char* ws = (char*)a.ws;
  int32_t* ticket = (int32_t*)ws;
  float* score = (float*)(ws + (size_t)rows * kTicketBytes);
  const dim3 grid(splits, rows);
  if (a.pool) {
    const LaunchFetch& f = *a.pool;
    const SelPool pl{f.pool_slots, f.step, f.block_table, f.slot_block, f.slot_last_use, f.insert_block, f.phys,
                     f.miss_list, f.n_miss};
    hipLaunchKernelGGL((select_kernel<T, D, true>), grid, dim3(kSelThreads), select_lds_bytes(a.nb), a.stream,
                       (const typename T::storage*)a.q, a.pos, (const typename T::storage*)a.k_comp, a.e_blk,
                       a.n_query, a.n_q_heads, a.n_kv_heads, a.nb, a.kq, a.ke, a.fill ? 1 : 0, a.sel, a.n_sel,
                       ticket, score, pl);
  } else {
    hipLaunchKernelGGL((select_kernel<T, D, false>), grid, dim3(kSelThreads), select_lds_bytes(a.nb), a.stream,
                       (const typename T::storage*)a.q, a.pos, (const typename T::storage*)a.k_comp, a.e_blk,
                       a.n_query, a.n_q_heads, a.n_kv_heads, a.nb, a.kq, a.ke, a.fill ? 1 : 0, a.sel, a.n_sel,
                       ticket, score, SelPool{});
  }
}

void launch_select(const LaunchSelect& a) {
  if (a.bf16 && a.n_query >= kMRows && !a.pool) {
    const bool done = a.head_dim == 128 ? launch_multi<128>(a) : launch_multi<64>(a);
    if (done) return;
  }
  if (a.bf16) {
    if (a.head_dim == 128) launch<Bf16, 128>(a); else launch<Bf16, 64>(a);
  } else {
    if (a.head_dim == 128) launch<F32, 128>(a); else launch<F32, 64>(a);
  }
}

}  // namespace nosa
