// Split-K block-sparse decode attention for NOSA.
//
// Exact attention over the selected 64-token blocks plus the current window
// block (the second stage of NOSA's two-stage attention, NOSA-1B release
// post, "工程实现亮点").  Grid = (splits, B*Hkv); each workgroup has WAVES
// wavefronts and each wavefront attends whole 64-token blocks.
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

size_t attn_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim, int k_cap, int n_query) {
  const size_t units = (size_t)batch * n_query * n_kv_heads;
  const size_t G = n_q_heads / n_kv_heads;
  const size_t splits = 2 * attn_splits(k_cap, (int)G);   // both parts of a pool step
  return align256(units * sizeof(int32_t)) + align256(units * splits * G * 2 * sizeof(float)) +
         align256(units * splits * G * head_dim * sizeof(float));
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

// PART -1: the whole attention (splits merged by the last workgroup).
// PART 0: a pool step's entries already resident plus the window, while the
//         fetch's gather runs; partials only (slots 0 .. S-1).
// PART 1: the same split of the entries, the fetched ones only (slots S ..
//         2S-1); the last workgroup of the unit merges all 2S partials.
template <class T, int D, int WAVES, int GMAX, int PART>
__global__ void __launch_bounds__(64 * WAVES) attn_kernel(
    const typename T::storage* __restrict__ q, const typename T::storage* __restrict__ blocks,
    int blocks_per_head, const int32_t* __restrict__ phys, const int32_t* __restrict__ n_sel,
    int k_cap, const typename T::storage* __restrict__ window_kv, int64_t win_head_stride,
    int64_t win_block_stride, const int32_t* __restrict__ pos, float scale_log2, int n_q_heads,
    int n_kv_heads, int nb, typename T::storage* __restrict__ out, int32_t* __restrict__ ticket,
    float* __restrict__ part_ml, float* __restrict__ part_o, const int32_t* __restrict__ miss_list,
    const int32_t* __restrict__ n_miss_p, int n_split_main, int n_query) {
  constexpr int ND = D / 16;
  const int G = n_q_heads / n_kv_heads;
  // grid (units, splits): workgroups are dispatched x-fastest, so every
  // unit's first split starts before any unit's second and the light last
  // splits (often just the window) go last
  const int n_split = PART < 0 ? (int)gridDim.y : 2 * n_split_main;   // partial slots per unit
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

  const int p = pos[br];
  const bool valid_pos = (p >= 0 && p < nb * kBlock);
  const int c = valid_pos ? p / kBlock : 0;
  int ns = valid_pos ? n_sel[unit] : -1;
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
    const int e = (int)blockIdx.y * WAVES + wave;
    const typename T::storage* blk = nullptr;
    int len = 0;
    if (e < ns) {
      const int pb = phys[(size_t)unit * k_cap + e];
      bool take = pb >= 0 && pb < blocks_per_head;
      if (PART >= 0 && take) take = slot_fetched(pb, ml, nm, k_cap) == (PART == 1);
      if (take) {
        blk = blocks + ((size_t)cunit * blocks_per_head + pb) * blk_elems;
        len = kBlock;
      }
    } else if (e < n_ent && PART != 1) {
      blk = window_kv + (int64_t)cunit * win_head_stride + (int64_t)c * win_block_stride;
      len = p - c * kBlock + 1;
    }
    if (blk != nullptr) attend_block<T, D>(q_group, G, blk, len, scale_log2, lane, m_run, l_run, o);
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
    const int t = ticket_take(&ticket[unit]);
    s_last = (t == (int)gridDim.y - 1);
    if (s_last) ticket_reset(&ticket[unit]);
  }
  __syncthreads();
  if (!s_last) return;
  merge_splits<T, D, WAVES, GMAX>(L, G, tid, n_split, po, pml, out_g);
}

template <class T, int D, int WAVES, int GMAX>
static void launch_w(const LaunchAttn& a) {
  const int units = a.batch * a.n_query * a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int splits = attn_splits(a.k_cap, G);
  char* ws = (char*)a.ws;
  int32_t* ticket = (int32_t*)ws;
  float* part_ml = (float*)(ws + align256((size_t)units * sizeof(int32_t)));
  const float scale_log2 = a.scale * 1.4426950408889634f;
  // partial slots are laid out for 2 * splits per unit in every mode
  float* part_o = (float*)((char*)part_ml + align256((size_t)units * 2 * splits * G * 2 * sizeof(float)));
#define NOSA_ATTN_ARGS                                                                                        \
  a.stream, (const typename T::storage*)a.q, (const typename T::storage*)a.blocks, a.blocks_per_head, a.phys, \
      a.n_sel, a.k_cap, (const typename T::storage*)a.window_kv, a.window_head_stride, a.window_block_stride,  \
      a.pos, scale_log2, a.n_q_heads, a.n_kv_heads, a.nb, (typename T::storage*)a.out, ticket, part_ml,        \
      part_o, a.miss_list, a.n_miss, splits, a.n_query
  if (a.part < 0)
    hipLaunchKernelGGL((attn_kernel<T, D, WAVES, GMAX, -1>), dim3(units, splits), dim3(64 * WAVES), 0, NOSA_ATTN_ARGS);
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
  if (a.bf16) {
    if (a.head_dim == 128) launch<Bf16, 128>(a); else launch<Bf16, 64>(a);
  } else {
    if (a.head_dim == 128) launch<F32, 128>(a); else launch<F32, 64>(a);
  }
}

}  // namespace nosa
