// Compressed keys and block eviction scores (the CIS) for NOSA selection.
//
// Two-stage block pooling per the gist.science summary of NOSA
// ("1. Algorithme : NOSA", block implementation): the keys and the eviction
// logits are mean-pooled over 16-token sub-blocks; the block eviction score
// is the max over the 4 sub-block means of a 64-token block.
//
// Keys sit in the block's MFMA fragment order (nosa_common.h).
#include "nosa_common.h"
#include "nosa_launch.h"

namespace nosa {

// One wavefront per (unit, block).  The block's keys are read as whole 1 KiB
// fragments (every load fully contiguous) and staged in LDS in the same
// order; then each lane owns one 16-byte column chunk of one sub-block and
// adds its 16 tokens serially, in token order, from LDS, so the fp32 sums
// are bit-exact.  The four sub-block logit means are taken by the lanes of
// chunk 0 and their max by lane 0.
// wavefronts per workgroup: 64 KiB of staged keys per workgroup
template <class T, int D>
constexpr int pool_waves() { return 65536 / (kBlock * D * (int)sizeof(typename T::storage)); }

template <class T, int D>
__global__ void __launch_bounds__((64 * pool_waves<T, D>())) pool_keys_kernel(
    const typename T::storage* __restrict__ kv, int64_t kv_unit_stride, int64_t kv_block_stride,
    const float* __restrict__ logits, int64_t n_units, int nb, int blk_begin, int n_blk,
    const int32_t* __restrict__ entry_block, int hkv, typename T::storage* __restrict__ k_comp,
    float* __restrict__ e_sub, float* __restrict__ e_blk) {
  constexpr int EPC = T::kPer16B;              // elements per 16-byte chunk
  constexpr int LPR = D / EPC;                 // chunks per key row
  constexpr int KEY_CHUNKS = kBlock * LPR;     // 16-byte chunks of a block's keys
  constexpr int FRAGS = KEY_CHUNKS / 64;       // 1 KiB fragments
  constexpr bool BF16 = sizeof(typename T::storage) == 2;
  constexpr int kPoolWaves = pool_waves<T, D>();
  __shared__ uint4 s_keys[kPoolWaves][KEY_CHUNKS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t item = (int64_t)blockIdx.x * kPoolWaves + wave;   // (unit, block)
  if (item >= n_units * n_blk) return;
  const int64_t unit = item / n_blk;
  // a block range shared by the batch, or (n_blk = 1) the one block the
  // unit's batch entry names; a whole wavefront leaves together
  int jb = blk_begin + (int)(item % n_blk);
  if (entry_block != nullptr) {
    jb = entry_block[unit / hkv];
    if (jb < 0 || jb >= nb) return;
  }
  const typename T::storage* keys = kv + unit * kv_unit_stride + (int64_t)jb * kv_block_stride;

  // stage the keys: fragment f, lane l -> chunk 64 f + l (contiguous loads,
  // non-temporal: every key is read once)
  uint4* sk = s_keys[wave];
#pragma unroll
  for (int f = 0; f < FRAGS; ++f) sk[64 * f + lane] = ld16_stream(keys + (size_t)(64 * f + lane) * EPC);
  // logits of the block: lane i < 64 reads logit i; sub-block means by lanes
  // of chunk 0 below (read back through a wavefront shuffle of the 64 values)
  const float* lg = logits + ((size_t)unit * nb + jb) * kBlock;
  const float my_logit = lg[lane];
  // this wavefront reads back only what it wrote itself: its LDS writes must
  // be complete (and not reordered past) before the reads below
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  const size_t row0 = (size_t)unit * nb * kSubsPerBlock + (size_t)jb * kSubsPerBlock;
  // each lane: (sub-block, chunk) pairs; LPR*4 pairs per block
  for (int pr = lane; pr < kSubsPerBlock * LPR; pr += 64) {
    const int sb = pr / LPR, ch = pr % LPR;
    float acc[EPC], v[EPC];
    const int e0 = key_chunk_offset<BF16>(kSub * sb, ch, D) / EPC;
    unpack16(sk[e0], acc, T{});
#pragma unroll
    for (int i = 1; i < kSub; ++i) {
      unpack16(sk[key_chunk_offset<BF16>(kSub * sb + i, ch, D) / EPC], v, T{});
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[e] = acc[e] + v[e];
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = acc[e] * 0.0625f;
    st16(k_comp + (row0 + sb) * D + ch * EPC, pack16(acc, T{}));
  }
  // sub-block logit means, in token order, by lanes 0..3; block max by lane 0
  // (every shuffle with all lanes active: a lane reading an inactive lane
  // gets nothing defined)
  float a = __shfl(my_logit, kSub * (lane & 3));
#pragma unroll
  for (int i = 1; i < kSub; ++i) {
    const float v = __shfl(my_logit, kSub * (lane & 3) + i);
    if (lane < kSubsPerBlock) a = a + v;
  }
  if (lane < kSubsPerBlock) {
    a = a * 0.0625f;
    e_sub[row0 + lane] = a;
  }
  const float a0 = __shfl(a, 0), a1 = __shfl(a, 1), a2 = __shfl(a, 2), a3 = __shfl(a, 3);
  if (lane == 0) {
    float best = a0;
    best = a1 > best ? a1 : best;
    best = a2 > best ? a2 : best;
    best = a3 > best ? a3 : best;
    e_blk[(size_t)unit * nb + jb] = best;
  }
}

template <class T, int D>
static void launch(const LaunchPool& a) {
  constexpr int kPoolWaves = pool_waves<T, D>();
  const int64_t items = a.n_units * a.n_blk;
  const int64_t grid = (items + kPoolWaves - 1) / kPoolWaves;
  hipLaunchKernelGGL((pool_keys_kernel<T, D>), dim3((unsigned)grid), dim3(64 * kPoolWaves), 0, a.stream,
                     (const typename T::storage*)a.kv, a.kv_unit_stride, a.kv_block_stride,
                     a.logits, a.n_units, a.nb, a.blk_begin, a.n_blk, a.entry_block, a.n_kv_heads,
                     (typename T::storage*)a.k_comp, a.e_sub, a.e_blk);
}

void launch_pool_keys(const LaunchPool& a) {
  if (a.n_blk <= 0 || a.n_units <= 0) return;
  if (a.bf16) {
    if (a.head_dim == 128) launch<Bf16, 128>(a); else launch<Bf16, 64>(a);
  } else {
    if (a.head_dim == 128) launch<F32, 128>(a); else launch<F32, 64>(a);
  }
}

}  // namespace nosa
