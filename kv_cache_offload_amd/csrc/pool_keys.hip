// Compressed keys and block eviction scores (the CIS) for NOSA selection.
//
// Two-stage block pooling per the gist.science summary of NOSA
// ("1. Algorithme : NOSA", block implementation): the keys and the eviction
// logits are mean-pooled over 16-token sub-blocks; the block eviction score
// is the max over the 4 sub-block means of a 64-token block.
//
// One thread owns one 16-byte column chunk of one sub-block and adds its 16
// tokens serially in token order, so the fp32 sums are bit-exact.  Keys sit
// in the block's MFMA fragment order (nosa_common.h); a wavefront load still
// touches only whole 16-byte chunks of one block's 16 KiB of keys.
#include "nosa_common.h"
#include "nosa_launch.h"

namespace nosa {

template <class T, int D>
__global__ void __launch_bounds__(256) pool_keys_kernel(
    const typename T::storage* __restrict__ kv, int64_t kv_unit_stride, int64_t kv_block_stride,
    const float* __restrict__ logits, int64_t n_units, int nb, int blk_begin, int n_blk,
    typename T::storage* __restrict__ k_comp,
    float* __restrict__ e_sub, float* __restrict__ e_blk) {
  constexpr int EPC = T::kPer16B;   // elements per 16-byte chunk
  constexpr int LPR = D / EPC;      // chunks per key row
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = n_units * n_blk * kSubsPerBlock * LPR;
  if (tid >= total) return;
  const int ch = (int)(tid % LPR);
  int64_t r = tid / LPR;
  const int sb = (int)(r % kSubsPerBlock);
  r /= kSubsPerBlock;
  const int jb = blk_begin + (int)(r % n_blk);
  const int64_t unit = r / n_blk;

  const typename T::storage* keys = kv + unit * kv_unit_stride + (int64_t)jb * kv_block_stride;
  constexpr bool BF16 = sizeof(typename T::storage) == 2;

  uint4 raw[kSub];
#pragma unroll
  for (int i = 0; i < kSub; ++i) raw[i] = ld16(keys + key_chunk_offset<BF16>(kSub * sb + i, ch, D));
  float acc[EPC], v[EPC];
  unpack16(raw[0], acc, T{});
#pragma unroll
  for (int i = 1; i < kSub; ++i) {
    unpack16(raw[i], v, T{});
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = acc[e] + v[e];
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = acc[e] * 0.0625f;
  const size_t srow = (size_t)unit * nb * kSubsPerBlock + (size_t)jb * kSubsPerBlock + sb;
  st16(k_comp + srow * D + ch * EPC, pack16(acc, T{}));

  if (ch == 0 && sb == 0) {
    // eviction logits of this block: 4 sub-block means, then their max
    const float* lg = logits + ((size_t)unit * nb + jb) * kBlock;
    float best = 0.0f;
#pragma unroll
    for (int s = 0; s < kSubsPerBlock; ++s) {
      float a = lg[kSub * s];
#pragma unroll
      for (int i = 1; i < kSub; ++i) a = a + lg[kSub * s + i];
      a = a * 0.0625f;
      e_sub[srow + s] = a;
      best = (s == 0 || a > best) ? a : best;
    }
    e_blk[(size_t)unit * nb + jb] = best;
  }
}

template <class T, int D>
static void launch(const LaunchPool& a) {
  constexpr int LPR = D / T::kPer16B;
  const int64_t total = a.n_units * a.n_blk * kSubsPerBlock * LPR;
  const int threads = 256;
  const int64_t grid = (total + threads - 1) / threads;
  hipLaunchKernelGGL((pool_keys_kernel<T, D>), dim3((unsigned)grid), dim3(threads), 0, a.stream,
                     (const typename T::storage*)a.kv, a.kv_unit_stride, a.kv_block_stride,
                     a.logits, a.n_units, a.nb, a.blk_begin,
                     a.n_blk, (typename T::storage*)a.k_comp, a.e_sub, a.e_blk);
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
