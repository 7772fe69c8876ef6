// Split-K block-sparse decode attention for NOSA.
//
// Exact attention over the selected 64-token blocks plus the current window
// block (the second stage of NOSA's two-stage attention, NOSA-1B release
// post, "工程实现亮点").  Grid = (units, splits), a unit being one query row
// of one KV head; each workgroup has WAVES wavefronts and each wavefront
// attends whole 64-token blocks.  Prefill chunks in bf16 with 4 or 8 query
// heads per KV head use chunk_attn_kernel below instead, which packs 16/G
// rows into the MFMA columns.
//
// Per block and wavefront, the G query heads of the KV head form the 16
// columns of a 16x16 MFMA tile (G <= 16, spare columns hold zeros):
//   S^T (64 tokens x 16 heads) = K (64 x D) . Q^T (D x 16)   4 tiles
//   O^T (D x 16 heads)        += V^T (D x 64) . P^T (64 x 16)
// bf16 uses v_mfma_f32_16x16x32_bf16, fp32 uses v_mfma_f32_16x16x4_f32.
// Blocks are stored in MFMA fragment order (nosa_common.h): every operand
// fragment is one contiguous 1 KiB wavefront load straight from HBM into
// registers, and a block's 32 KiB (D=128 bf16) is read exactly once.  The
// token order of the S tiles is permuted so that each lane's softmax weights
// are exactly the P^T operand it needs for the V product, with no data
// exchange.
//
// Each wavefront keeps its block's max / sum per head (exp2 with the scale
// folded in) and its unnormalised output in registers; the wavefronts of a
// workgroup merge through LDS, workgroups through a fp32 workspace written
// with coherent stores; the last workgroup of a (b, h) (atomic ticket)
// merges the splits, normalises and stores the output.
#include "nosa_common.h"
#include "nosa_launch.h"
#include "attn_dev.h"

namespace nosa {

// One block per wavefront and 8 wavefronts per workgroup (4 when the GQA
// group needs all 16 MFMA columns, to keep the LDS merge buffer within
// 64 KiB).  Fewer, fuller workgroups beat more, smaller ones here: every
// split adds a partial to write, a ticket and a share of the final merge.
static inline int attn_waves(int G) { return G <= 8 ? 8 : 4; }
static inline int attn_splits(int k_cap, int G) { return (k_cap + 1 + attn_waves(G) - 1) / attn_waves(G); }

// Packed prefill-chunk attention (see chunk_attn_kernel): NR = 16 / G rows
// per unit for G = 4 or 8 (bf16), 0 when the rows are not packed.
constexpr int kChunkWaves = 8;
static inline int chunk_rows(int G) { return (G == 4 || G == 8) ? 16 / G : 0; }
constexpr int kChunkMaxShare = 2048;                        // union entries per workgroup (nb <= 4096, >= 2 splits)
struct ChunkGeometry {
  size_t units, splits, off_ml, off_o, total;
};
static ChunkGeometry chunk_geometry(int batch, int n_kv_heads, int head_dim, int n_query, int NR) {
  ChunkGeometry g{};
  g.units = (size_t)batch * ((n_query + NR - 1) / NR) * n_kv_heads;
  // splits per unit: about one workgroup per CU in all, at least 2, at most 8
  const size_t s = (256 + g.units - 1) / g.units;
  g.splits = s < 2 ? 2 : (s > 8 ? 8 : s);
  size_t o = g.units * kTicketBytes;                        // tickets
  g.off_ml = o; o += align256(g.units * g.splits * 16 * 2 * sizeof(float));
  g.off_o = o; o += align256(g.units * g.splits * 16 * (size_t)head_dim * sizeof(float));
  g.total = o;
  return g;
}

size_t attn_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim, int k_cap, int n_query) {
  const size_t units = (size_t)batch * n_query * n_kv_heads;
  const size_t G = n_q_heads / n_kv_heads;
  const size_t splits = 2 * attn_splits(k_cap, (int)G);   // both parts of a pool step
  size_t need = units * kTicketBytes + align256(units * splits * G * 2 * sizeof(float)) +
                align256(units * splits * G * head_dim * sizeof(float));
  const int NR = chunk_rows((int)G);
  if (n_query > 1 && NR > 0) {
    const size_t packed = chunk_geometry(batch, n_kv_heads, head_dim, n_query, NR).total;
    need = need > packed ? need : packed;
  }
  return need;
}

// Whether a pool slot is being filled by this step's fetch (a miss, or the
// block the window just completed): its contents are not there until the
// gather is done.
__device__ __forceinline__ bool slot_fetched(int slot, const int32_t* ml, int n_miss, int k_cap) {
  if (slot == ml[2 * k_cap + 1]) return true;
  for (int i = 0; i < n_miss; ++i)
    if (ml[2 * i + 1] == slot) return true;
  return false;
}

// Where the block in a pool slot being filled this step comes from: the host
// cache block of its miss (>= 0), the block the window just completed (-2),
// or nowhere: the slot is resident (-1).
__device__ __forceinline__ int fetch_source(int slot, const int32_t* ml, int n_miss, int k_cap, int nb) {
  if (slot == ml[2 * k_cap + 1] && ml[2 * k_cap] >= 0) return -2;
  for (int i = 0; i < n_miss; ++i)
    if (ml[2 * i + 1] == slot) {
      const int blk = ml[2 * i];
      return (blk >= 0 && blk < nb) ? blk : -1;
    }
  return -1;
}

// PART -1: the whole attention (splits merged by the last workgroup).
// PART 0: a pool step's entries already resident plus the window, while the
//         fetch's gather runs; partials only (slots 0 .. S-1).
// PART 1: the same split of the entries, the fetched ones only (slots S ..
//         2S-1); the last workgroup of the unit merges all 2S partials.
// PART 2: a pool step with the gather folded in: a fetched entry's block is
//         read from the host cache (or the completed window block), written
//         to its pool slot from the registers and attended; entry n_sel + 1
//         copies the completed block when the set does not hold it.  Splits
//         merged by the last workgroup, as in PART -1.
template <class T, int D, int WAVES, int GMAX, int PART>
__global__ void __launch_bounds__(64 * WAVES) attn_kernel(
    const typename T::storage* __restrict__ q, const typename T::storage* __restrict__ blocks,
    int blocks_per_head, const int32_t* __restrict__ phys, const int32_t* __restrict__ n_sel,
    int k_cap, const typename T::storage* __restrict__ window_kv, int64_t win_head_stride,
    int64_t win_block_stride, const int32_t* __restrict__ pos, float scale_log2, int n_q_heads,
    int n_kv_heads, int nb, typename T::storage* __restrict__ out, int32_t* __restrict__ ticket,
    float* __restrict__ part_ml, float* __restrict__ part_o, const int32_t* __restrict__ miss_list,
    const int32_t* __restrict__ n_miss_p, int n_split_main, int n_query, const float* __restrict__ bias,
    const typename T::storage* __restrict__ host_kv, const typename T::storage* __restrict__ insert_src,
    typename T::storage* __restrict__ pool_w) {
  constexpr int ND = D / 16;
  const int G = n_q_heads / n_kv_heads;
  // grid (units, splits): workgroups are dispatched x-fastest, so every
  // unit's first split starts before any unit's second and the light last
  // splits (often just the window) go last
  const int n_split = (PART < 0 || PART == 2) ? (int)gridDim.y : 2 * n_split_main;   // partial slots per unit
  const int split = PART == 1 ? n_split_main + (int)blockIdx.y : (int)blockIdx.y;
  // a unit is one query row of one KV head: unit = (b * n_query + r) * Hkv + h
  // (q, pos, phys / n_sel, out, the ticket and the partials are per unit);
  // the rows of batch entry b share its cache (cache unit b * Hkv + h)
  const int unit = blockIdx.x;
  const int h = unit % n_kv_heads;
  const int br = unit / n_kv_heads;                 // b * n_query + r
  const int b = br / n_query;
  const int cunit = b * n_kv_heads + h;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t blk_elems = (size_t)2 * kBlock * D;

  // the position, the set size and this wavefront's entry go out together
  // (one memory round trip before the block's loads, not three)
  const int e_w = (int)blockIdx.y * WAVES + wave;
  const int p = pos[br];
  const int ns_raw = n_sel[unit];
  const int pb_raw = e_w < k_cap ? phys[(size_t)unit * k_cap + e_w] : -1;
  const bool valid_pos = (p >= 0 && p < nb * kBlock);
  const int c = valid_pos ? p / kBlock : 0;
  int ns = valid_pos ? ns_raw : -1;
  ns = ns < 0 ? -1 : (ns > k_cap ? k_cap : ns);
  const int n_ent = ns + 1;  // selected blocks, then the window (none if pos is invalid)

  // ---- this wavefront's block: entry split*WAVES + wave
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const typename T::storage* q_group = q + ((size_t)br * n_q_heads + (size_t)h * G) * D;
  const int32_t* ml = miss_list + (size_t)unit * (k_cap + 1) * 2;
  int nm = 0;
  if (PART >= 0) {
    nm = n_miss_p[unit];
    nm = nm < 0 ? 0 : (nm > k_cap ? k_cap : nm);
  }
  {
    // entry e of this split: part 0 skips the fetched slots, part 1 takes
    // only those (and no window)
    const int e = e_w;
    const typename T::storage* blk = nullptr;
    [[maybe_unused]] typename T::storage* copy_to = nullptr;   // PART 2: the slot a fetched block fills
    int len = 0, lblk = -1;      // lblk: the block's logical id (its position / 64)
    if (e < ns) {
      const int pb = pb_raw;
      bool take = pb >= 0 && pb < blocks_per_head;
      if ((PART == 0 || PART == 1) && take) take = slot_fetched(pb, ml, nm, k_cap) == (PART == 1);
      if (take) {
        blk = blocks + ((size_t)cunit * blocks_per_head + pb) * blk_elems;
        len = kBlock;
        lblk = pb;
        if constexpr (PART == 2) {
          int src = fetch_source(pb, ml, nm, k_cap, nb);
          if (src == -2 && insert_src == nullptr) src = -1;   // nothing to copy from: the slot as it is
          if (src != -1) {
            copy_to = pool_w + ((size_t)cunit * blocks_per_head + pb) * blk_elems;
            blk = src == -2 ? insert_src + (size_t)cunit * blk_elems : host_kv + ((size_t)cunit * nb + src) * blk_elems;
          }
        }
      }
    } else if (e < n_ent && PART != 1) {
      blk = window_kv + (int64_t)cunit * win_head_stride + (int64_t)c * win_block_stride;
      len = p - c * kBlock + 1;
      lblk = c;
    } else if (PART == 2 && e == n_ent) {
      // the completed block enters its slot whether or not the set holds it
      // (when it does, that entry writes the same bytes too)
      const int ib = ml[2 * k_cap], is = ml[2 * k_cap + 1];
      if (ib >= 0 && is >= 0 && is < blocks_per_head && insert_src != nullptr) {
        blk = insert_src + (size_t)cunit * blk_elems;
        copy_to = pool_w + ((size_t)cunit * blocks_per_head + is) * blk_elems;
        len = 0;       // copied, not attended
      }
    }
    if constexpr (PART == 2) {
      if (blk != nullptr) {
        Frags<T, D> f;
        load_tiles<T, D, 4>(f, blk, 0, lane);
        load_q<T, D>(f, q_group, G, lane);
        if (copy_to != nullptr) store_tiles<T, D, 4>(f, copy_to, 0, lane);
        if (len > 0) attend_frags<T, D, 4>(f, 0, len, scale_log2, lane, m_run, l_run, o);
      }
    } else {
      // the eviction-bias variant (resident cache: phys are block ids < nb)
      const float* bias_blk = (bias != nullptr && blk != nullptr && lblk < nb)
                                  ? bias + ((size_t)cunit * nb + lblk) * kBlock : nullptr;
      if (blk != nullptr) attend_block<T, D>(q_group, G, blk, len, scale_log2, lane, m_run, l_run, o, bias_blk);
    }
  }

  __shared__ AttnLds<D, WAVES, GMAX> L;
  typename T::storage* out_g = out + ((size_t)br * n_q_heads + (size_t)h * G) * D;
  float* pml = part_ml + (size_t)unit * n_split * G * 2;
  float* po = part_o + (size_t)unit * n_split * G * D;
  merge_waves<T, D, WAVES, GMAX>(L, m_run, l_run, o, G, tid, split, n_split, out_g, po, pml);
  if (PART == 0 || n_split == 1) return;

  // ---- the last workgroup of this (b, h) merges the splits
  __shared__ int s_last;
  wait_stores_done();
  __syncthreads();
  if (tid == 0) {
    const int t = ticket_take(&ticket[(size_t)unit * kTicketInts]);
    s_last = (t == (int)gridDim.y - 1);
    if (s_last) ticket_reset(&ticket[(size_t)unit * kTicketInts]);
  }
  __syncthreads();
  if (!s_last) return;
  merge_splits<T, D, WAVES, GMAX>(L, G, tid, n_split, po, pml, out_g);
}

// ---------------------------------------------------------------------------
// Prefill-chunk attention with the rows packed into the MFMA columns (bf16,
// G = 4 or 8): the NR = 16 / G consecutive rows of a unit fill the 16
// columns of the tiles (column = rr * G + head).  The rows of a chunk select
// mostly the same blocks (the same Gamma_e whenever they share a window
// block), so a unit attends the union of its rows' blocks once, every column
// masked to what its own row attends: its selected blocks whole, its window
// block up to its position, nothing else.
//
// Grid (units, S): every workgroup builds the unit's union in LDS (bit rr of
// a block: selected by row rr; bit NR + rr: the window of row rr; the marked
// blocks ranked in ascending order) and takes the S-th share of it; its
// wavefronts walk their entries, folding each block into a running
// partial; the wavefronts merge in LDS, the S workgroups through partials,
// and the last one (ticket) stores every row's heads.
template <int D>
__device__ __forceinline__ void load_q_rows(Frags<Bf16, D>& f, const uint16_t* q, int b, int r0, int n_query,
                                            int n_q_heads, int h, int G, int lane) {
  const int col = lane & 15, grp = lane >> 4, r = r0 + col / G;
  const uint16_t* src = q + (((size_t)b * n_query + r) * n_q_heads + (size_t)h * G + col % G) * D;
#pragma unroll
  for (int s = 0; s < Frags<Bf16, D>::NK; ++s)
    f.q[s] = as_bf16x8(r < n_query ? ld16(src + 32 * s + 8 * grp) : make_uint4(0, 0, 0, 0));
}

template <int D, int NR>
__global__ void __launch_bounds__(64 * kChunkWaves) chunk_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ n_sel, int k_cap, const int32_t* __restrict__ pos, float scale_log2, int n_q_heads,
    int n_kv_heads, int nb, int n_query, uint16_t* __restrict__ out, int32_t* __restrict__ ticket,
    float* __restrict__ part_ml, float* __restrict__ part_o) {
  constexpr int ND = D / 16, WAVES = kChunkWaves, G = 16 / NR, NT = 64 * WAVES;
  // XCD-aware order: workgroups go to the 8 XCDs round-robin in linear
  // order, and the row groups of one KV head attend mostly the same blocks,
  // the same share of them for the same split.  So the linear index picks
  // the (KV head, split) group first: every workgroup of a group lands on
  // the same XCD (with 8 groups; 4 groups: two XCDs), whose L2 then serves
  // the group's re-reads of those blocks.
  const int n_split = gridDim.y;
  const int n_grp = n_kv_heads * n_split;
  const int wid = (int)blockIdx.x + (int)blockIdx.y * (int)gridDim.x;
  const int grp = wid % n_grp, brg = wid / n_grp;
  const int h = grp / n_split, split = grp % n_split;
  const int u = brg * n_kv_heads + h;
  const int n_groups = (n_query + NR - 1) / NR;
  const int b = brg / n_groups, r0 = (brg % n_groups) * NR;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ AttnLds<D, WAVES, 16> L;
  __shared__ int s_ent[kChunkMaxShare];
  __shared__ int s_wsum[WAVES];
  __shared__ int s_share[2];

  // ---- the union (the block marks live in the merge buffer until the merge)
  uint32_t* s_mask = reinterpret_cast<uint32_t*>(&L.o[0][0][0]);
  int rp[NR], rn[NR], rs[NR];                      // each row's position, selection count and entry tid
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) {
    const int r = r0 + rr;
    const size_t row = ((size_t)b * n_query + r) * n_kv_heads + h;
    rp[rr] = r < n_query ? pos[(size_t)b * n_query + r] : -1;
    rn[rr] = r < n_query ? n_sel[row] : 0;
    // the first NT entries go out with the counts, not behind them
    rs[rr] = (r < n_query && tid < k_cap) ? sel[row * k_cap + tid] : -1;
  }
  for (int j = tid; j < nb; j += NT) s_mask[j] = 0u;
  __syncthreads();
#pragma unroll
  for (int rr = 0; rr < NR; ++rr) {
    const int p = rp[rr];
    if (p < 0 || p >= nb * kBlock) continue;       // a row out of range attends nothing
    const size_t row = ((size_t)b * n_query + r0 + rr) * n_kv_heads + h;
    const int ns = rn[rr] < 0 ? 0 : (rn[rr] > k_cap ? k_cap : rn[rr]);
    for (int e = tid; e < ns; e += NT) {
      const int blk = e == tid ? rs[rr] : sel[row * k_cap + e];
      if (blk >= 0 && blk < nb) atomicOr(&s_mask[blk], 1u << rr);
    }
    if (tid == 0) atomicOr(&s_mask[p / kBlock], 1u << (NR + rr));
  }
  __syncthreads();
  {
    // rank the marked blocks (each thread a run of blocks, a wavefront scan
    // and the wavefront totals) and keep this workgroup's share
    const int per = (nb + NT - 1) / NT;
    const int lo = min(nb, tid * per), hi = min(nb, lo + per);
    int cnt = 0;
    for (int j = lo; j < hi; ++j) cnt += s_mask[j] != 0u;
    const int incl = wave_incl_sum(cnt, lane);
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int off = incl - cnt, total = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      if (w < wave) off += s_wsum[w];
      total += s_wsum[w];
    }
    const int sh_lo = (int)((int64_t)total * split / n_split), sh_hi = (int)((int64_t)total * (split + 1) / n_split);
    for (int j = lo; j < hi; ++j) {
      if (s_mask[j] == 0u) continue;
      if (off >= sh_lo && off < sh_hi) s_ent[off - sh_lo] = j | (int)(s_mask[j] << 16);
      ++off;
    }
    if (tid == 0) s_share[0] = sh_hi - sh_lo;
  }
  __syncthreads();
  const int n_share = min(s_share[0], kChunkMaxShare);

  // ---- the share's blocks, one wavefront each in turn
  const int rr = (lane & 15) / G;
  int p = rp[0];                                   // this lane's row's position
#pragma unroll
  for (int k = 1; k < NR; ++k)
    if (rr == k) p = rp[k];
  const bool valid = p >= 0 && p < nb * kBlock;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  Frags<Bf16, D> f;
  load_q_rows<D>(f, q, b, r0, n_query, n_q_heads, h, G, lane);
  const uint16_t* unit_kv = kv + (size_t)(b * n_kv_heads + h) * nb * ((size_t)2 * kBlock * D);
  for (int i = wave; i < n_share; i += WAVES) {
    const int ent = s_ent[i];
    const int blk = ent & 0xffff;
    const uint32_t mask = (uint32_t)ent >> 16;
    int len = 0;                                   // this lane's column: its row's token count
    if (valid) {
      if ((mask >> rr) & 1u) len = kBlock;
      else if ((mask >> (NR + rr)) & 1u) len = p - blk * kBlock + 1;
    }
    load_tiles<Bf16, D, 4>(f, unit_kv + (size_t)blk * ((size_t)2 * kBlock * D), 0, lane);
    float mb, lb;
    f32x4 ob[ND];
    attend_frags<Bf16, D, 4>(f, 0, len, scale_log2, lane, mb, lb, ob);
    combine_partial<ND>(m_run, l_run, o, mb, lb, ob);
  }
  __syncthreads();                                 // the marks are dead: L is the merge buffer again
  float* pml = part_ml + (size_t)u * n_split * 16 * 2;
  float* po = part_o + (size_t)u * n_split * 16 * D;
  merge_waves<Bf16, D, WAVES, 16>(L, m_run, l_run, o, 16, tid, split, n_split, nullptr, po, pml);

  // ---- the last workgroup of the unit merges the S partials
  __shared__ int s_last;
  wait_stores_done();
  __syncthreads();
  if (tid == 0) {
    const int t = ticket_take(&ticket[(size_t)u * kTicketInts]);
    s_last = (t == n_split - 1);
    if (s_last) ticket_reset(&ticket[(size_t)u * kTicketInts]);
  }
  __syncthreads();
  if (!s_last) return;
  constexpr int PER = 16 * D / NT;                 // outputs per thread
  constexpr int kRegSplits = 8;                    // the most splits a launch uses
  float v[PER][kRegSplits];
#pragma unroll
  for (int k = 0; k < PER; ++k)
#pragma unroll
    for (int sp = 0; sp < kRegSplits; ++sp)
      v[k][sp] = sp < n_split ? load_coherent(&po[((size_t)sp * 16 + (tid + k * NT) / D) * D + (tid + k * NT) % D])
                              : 0.f;
  float* fw = &L.o[0][0][0];                       // split weights [split][column]
  float* fl = fw + n_split * 16;
  for (int i = tid; i < n_split * 16; i += NT) {
    fw[i] = load_coherent(&pml[2 * i]);
    fl[i] = load_coherent(&pml[2 * i + 1]);
  }
  __syncthreads();
  if (tid < 16 * kRegSplits) {
    // one 8-lane group per column (lane = split): the maxima and sums by DPP,
    // every split's LDS words read at once
    static_assert(kRegSplits == 8, "one 8-lane group per column");
    const int col = tid >> 3, sp = tid & 7;
    const bool on = sp < n_split;
    const float ms = on ? fw[sp * 16 + col] : -INFINITY;
    const float ls = on ? fl[sp * 16 + col] : 0.f;
    const float M = group_max<8>(ms);
    const float wt = ms == -INFINITY ? 0.f : exp2f(ms - M);
    const float den = group_sum<8>(wt * ls);
    if (on) fw[sp * 16 + col] = wt;
    if (sp == 0) L.den[col] = den;
  }
  __syncthreads();
  const int sp_last = n_split > 0 ? n_split - 1 : 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int idx = tid + k * NT, col = idx / D, d = idx % D, rw = r0 + col / G;
    float num = 0.f;
    // every term, unguarded (reads in bounds; a term past n_split adds 0)
#pragma unroll
    for (int sp = 0; sp < kRegSplits; ++sp)
      num += (sp < n_split ? fw[min(sp, sp_last) * 16 + col] : 0.f) * v[k][sp];
    if (rw >= n_query) continue;
    const float den = L.den[col];
    store_out(&out[(((size_t)b * n_query + rw) * n_q_heads + (size_t)h * G + col % G) * D + d],
              den > 0.f ? num / den : 0.f);
  }
}

template <int D, int NR>
static void launch_chunk(const LaunchAttn& a) {
  const ChunkGeometry g = chunk_geometry(a.batch, a.n_kv_heads, D, a.n_query, NR);
  char* ws = (char*)a.ws;
  int32_t* ticket = (int32_t*)ws;
  float* part_ml = (float*)(ws + g.off_ml);
  float* part_o = (float*)(ws + g.off_o);
  const float scale_log2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((chunk_attn_kernel<D, NR>), dim3((unsigned)g.units, (unsigned)g.splits), dim3(64 * kChunkWaves), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.blocks, a.phys, a.n_sel, a.k_cap, a.pos,
                     scale_log2, a.n_q_heads, a.n_kv_heads, a.nb, a.n_query, (uint16_t*)a.out, ticket, part_ml,
                     part_o);
}

// The packed path needs the chunk layout: bf16, G of 4 or 8, several rows,
// one call over the whole attention, every block (windows included) in one
// resident cache.
static bool chunk_packed(const LaunchAttn& a) {
  const int G = a.n_q_heads / a.n_kv_heads;
  const size_t blk_elems = (size_t)2 * kBlock * a.head_dim;
  return a.bf16 && chunk_rows(G) > 0 && a.n_query > 1 && a.part < 0 && a.blocks == a.window_kv &&
         a.blocks_per_head == a.nb && a.window_block_stride == (int64_t)blk_elems &&
         a.window_head_stride == (int64_t)a.nb * (int64_t)blk_elems;
}

template <class T, int D, int WAVES, int GMAX>
static void launch_w(const LaunchAttn& a) {
  const int units = a.batch * a.n_query * a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int splits = attn_splits(a.k_cap, G);
  // PART 2 has one more entry per unit (the completed block's copy); the
  // partials' layout (2 * splits per unit) has room for it
  const int splits_fetch = (a.k_cap + 2 + WAVES - 1) / WAVES;
  char* ws = (char*)a.ws;
  int32_t* ticket = (int32_t*)ws;
  float* part_ml = (float*)(ws + (size_t)units * kTicketBytes);
  const float scale_log2 = a.scale * 1.4426950408889634f;
  // partial slots are laid out for 2 * splits per unit in every mode
  float* part_o = (float*)((char*)part_ml + align256((size_t)units * 2 * splits * G * 2 * sizeof(float)));
#define NOSA_ATTN_ARGS                                                                                        \
  a.stream, (const typename T::storage*)a.q, (const typename T::storage*)a.blocks, a.blocks_per_head, a.phys, \
      a.n_sel, a.k_cap, (const typename T::storage*)a.window_kv, a.window_head_stride, a.window_block_stride,  \
      a.pos, scale_log2, a.n_q_heads, a.n_kv_heads, a.nb, (typename T::storage*)a.out, ticket, part_ml,        \
      part_o, a.miss_list, a.n_miss, splits, a.n_query, a.bias, (const typename T::storage*)a.host_kv,   \
      (const typename T::storage*)a.insert_src, (typename T::storage*)const_cast<void*>(a.blocks)
  if (a.part < 0)
    hipLaunchKernelGGL((attn_kernel<T, D, WAVES, GMAX, -1>), dim3(units, splits), dim3(64 * WAVES), 0, NOSA_ATTN_ARGS);
  else if (a.part == 2)
    hipLaunchKernelGGL((attn_kernel<T, D, WAVES, GMAX, 2>), dim3(units, splits_fetch), dim3(64 * WAVES), 0,
                       NOSA_ATTN_ARGS);
  else if (a.part == 0)
    hipLaunchKernelGGL((attn_kernel<T, D, WAVES, GMAX, 0>), dim3(units, splits), dim3(64 * WAVES), 0, NOSA_ATTN_ARGS);
  else
    hipLaunchKernelGGL((attn_kernel<T, D, WAVES, GMAX, 1>), dim3(units, splits), dim3(64 * WAVES), 0, NOSA_ATTN_ARGS);
#undef NOSA_ATTN_ARGS
}

template <class T, int D>
static void launch(const LaunchAttn& a) {
  if (a.n_q_heads / a.n_kv_heads <= 8)
    launch_w<T, D, 8, 8>(a);
  else
    launch_w<T, D, 4, 16>(a);
}

void launch_attn(const LaunchAttn& a) {
  if (chunk_packed(a)) {
    const int NR = chunk_rows(a.n_q_heads / a.n_kv_heads);
    if (a.head_dim == 128) {
      if (NR == 2) launch_chunk<128, 2>(a); else launch_chunk<128, 4>(a);
    } else {
      if (NR == 2) launch_chunk<64, 2>(a); else launch_chunk<64, 4>(a);
    }
    return;
  }
  if (a.bf16) {
    if (a.head_dim == 128) launch<Bf16, 128>(a); else launch<Bf16, 64>(a);
  } else {
    if (a.head_dim == 128) launch<F32, 128>(a); else launch<F32, 64>(a);
  }
}

}  // namespace nosa
