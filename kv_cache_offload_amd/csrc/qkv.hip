// Split of a fused QKV projection's output into the decode path's inputs,
// with the eviction head of Eq. 4 fused in.  NOSI fuses the eviction heads
// with the QKV split into one kernel (montaan summary, "System Optimization
// (NOSI)" item 1); the head scores each KV pair from its value alone,
// s^e_j = softplus(v_j W1) W2 (same summary, "Key Design Components" item 3),
// and those scores are the logits the block pooling averages.
//
// One workgroup per (TT consecutive tokens, batch entry, KV head h); TT = 1
// for a decode step, 16 for a chunk of 16 or more tokens:
//   * query heads h*G .. h*G+G-1 -> q_out, 16-byte copies;
//   * the key -> cache block p/64 in fragment order: each 16-byte chunk of
//     the row is one chunk of a key fragment;
//   * the value -> the same block: a value fragment holds 8 (bf16) or 4
//     (fp32) consecutive tokens of one dimension in 16 bytes, so a run of
//     that many consecutive aligned positions is one 16-byte store per
//     dimension, anything else 2- or 4-byte stores;
//   * s^e = sum_j softplus(v . W1[:, j]) W2[j] with fp32 products and sums:
//     for 16 tokens the products v . W1 are one small matrix product on the
//     matrix cores (v_mfma_f32_16x16x4_f32, values staged in LDS, W1 read
//     into registers), for one token vector FMAs; each wavefront takes 32
//     columns per pass and sums its softplus terms over them (DPP within
//     16-lane rows), and the four wavefront sums are added in order.
// Positions outside [0, NB*64) copy the query only.
#include "nosa_common.h"
#include "nosa_launch.h"

namespace nosa {

__device__ __forceinline__ float softplus_f(float x) {
  // log(1 + e^x) = max(x, 0) + log(1 + e^-|x|), no overflow
  return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}

__device__ __forceinline__ float storage_to_f32(uint16_t b) { return bf16_bits_to_f32(b); }
__device__ __forceinline__ float storage_to_f32(float f) { return f; }
// back to storage: exact, the value came from that type
__device__ __forceinline__ uint16_t f32_to_storage(float f, Bf16) { return (uint16_t)(__float_as_uint(f) >> 16); }
__device__ __forceinline__ float f32_to_storage(float f, F32) { return f; }

// element offset, inside a block's value half, of token tok, dimension d
template <bool BF16>
__device__ __forceinline__ int value_elem_offset(int tok, int d, int D) {
  const int ND = D / 16, u = d >> 4, r = d & 15;
  if constexpr (BF16) {
    const int hh = tok >> 5, g = (tok >> 3) & 3, j = tok & 7;
    return ((hh * ND + u) * 64 + 16 * g + r) * 8 + j;
  } else {
    const int t = tok >> 4, g = (tok >> 2) & 3, j = tok & 3;
    return ((t * ND + u) * 64 + 16 * g + r) * 4 + j;
  }
}

constexpr int kQkvThreads = 256;
constexpr int kQkvWaves = kQkvThreads / 64;
constexpr int kCopyBatch = 8;                        // 16-byte loads in flight per thread
constexpr int kHeadCols = 32;                        // eviction-head columns per wavefront per pass

// TT consecutive tokens of one batch entry per workgroup (TT = 1 for a
// decode step, 16 for a chunk).  Every phase issues its loads before using
// any of them: the copies in batches of kCopyBatch, the W1 operands of the
// first column pass right after the query copy, so they are in flight while
// the key and value rows move.
template <class T, int D, int TT>
__global__ void __launch_bounds__(kQkvThreads) qkv_kernel(const typename T::storage* __restrict__ qkv, int n_tok,
                                                          const int32_t* __restrict__ pos, const float* __restrict__ w1,
                                                          const float* __restrict__ w2, int d_e, int n_q_heads,
                                                          int n_kv_heads, int nb, typename T::storage* __restrict__ q_out,
                                                          typename T::storage* __restrict__ kv,
                                                          float* __restrict__ evict_logits) {
  using S = typename T::storage;
  constexpr int EPC = T::kPer16B;                    // elements (and value-fragment tokens) per 16 bytes
  constexpr int CPR = D / EPC;                       // 16-byte chunks per head row
  constexpr bool BF16 = sizeof(S) == 2;
  constexpr int NKS = D / 4;                         // k-steps of v_mfma_f32_16x16x4_f32 over the dimensions
  constexpr int NVG = (TT + EPC - 1) / EPC;          // value-fragment token groups per dimension
  constexpr int DS = TT == 1 ? D : D + 4;            // staged row stride (padded: conflict-free A reads)
  constexpr int DH = D / 2;                          // dimensions per half-wavefront (one token)
  static_assert(TT == 1 || TT == 16, "one token, or one MFMA row tile of tokens");
  __shared__ __align__(16) float s_v[TT * DS];       // [token][d], fp32
  __shared__ float s_part[kQkvWaves][16];
  __shared__ int s_pos[TT];
  const int t0 = blockIdx.x * TT, b = blockIdx.y, h = blockIdx.z;
  const int nt = min(TT, n_tok - t0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;          // MFMA lane coordinates
  const int G = n_q_heads / n_kv_heads;
  const size_t row_elems = (size_t)(n_q_heads + 2 * n_kv_heads) * D;
  const S* rows = qkv + ((size_t)b * n_tok + t0) * row_elems;
  const int cap = nb * kBlock;

  // W1 operands of this wavefront's kHeadCols columns in pass cg, in
  // registers.  16 tokens (matrix cores): lane (lg, lr) holds, for its two
  // 16-column tiles t, W1[lg NKS + s][col(t, lr)] for every k-step s (lane
  // group lg owns dimensions [lg NKS, lg NKS + NKS)).  One token (vector
  // FMAs): lane l holds W1[hf DH + i][col] for its column col = l % 32 and
  // half hf = l / 32 of the dimensions.  Columns past d_e read the last
  // column; their terms are multiplied by a zero W2 below.
  const float* w1h = w1 + (size_t)h * D * d_e;
  const float* w2h = w2 + (size_t)h * d_e;
  constexpr int NB1 = TT == 1 ? DH : 2 * NKS;
  float bw[NB1], w2r[2];                             // W1 operands; W2 of the lane's column(s), zero past d_e
  auto load_b = [&](int cg) {
    if constexpr (TT == 1) {
      const int c = cg + kHeadCols * wave + (lane & 31), col = min(c, d_e - 1);
      const float* src = w1h + (size_t)(lane >> 5) * DH * d_e + col;
#pragma unroll
      for (int i = 0; i < DH; ++i) bw[i] = src[(size_t)i * d_e];
      const float w2v = w2h[col];
      w2r[0] = (lane < 32 && c < d_e) ? w2v : 0.f;
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int c = cg + kHeadCols * wave + 16 * t + lr, col = min(c, d_e - 1);
        const float* src = w1h + (size_t)lg * NKS * d_e + col;
#pragma unroll
        for (int k = 0; k < NKS; ++k) bw[t * NKS + k] = src[(size_t)k * d_e];
        const float w2v = w2h[col];
        w2r[t] = c < d_e ? w2v : 0.f;
      }
    }
  };

  // key and value rows, 16-byte chunks, each with its token's position
  // (read from global memory, so nothing waits on it first), requested
  // before anything else: nothing they feed depends on the query copy
  constexpr int KV_CHUNKS = 2 * TT * CPR, KVN = (KV_CHUNKS + kQkvThreads - 1) / kQkvThreads;
  const int32_t* pos_t = pos + (size_t)b * n_tok + t0;
  auto valid = [&](int i, int p) { return i < nt && p >= 0 && p < cap; };
  uint4 kvr[KVN];
  int kvp[KVN];
  const int p_own = pos_t[min(tid, nt - 1)];
#pragma unroll
  for (int u = 0; u < KVN; ++u) {                  // unconditional loads (token clamped), zero if skipped
    const int e = min(tid + u * kQkvThreads, KV_CHUNKS - 1);
    const int isv = e >= TT * CPR, f = isv ? e - TT * CPR : e, i = f / CPR, ch = f % CPR;
    kvr[u] = reinterpret_cast<const uint4*>(rows + min(i, nt - 1) * row_elems + (size_t)(n_q_heads + isv * n_kv_heads + h) * D)[ch];
    kvp[u] = pos_t[min(i, nt - 1)];
  }
  // the query heads of this KV head, 16-byte copies.  No branch: indexes
  // past the end are clamped to the last chunk, which those lanes then
  // store again with the same value (a guarded store would pull its load
  // into the guard and serialise the batch).
  {
    const int per = G * CPR, total = nt * per;
    for (int e0 = tid; e0 < total; e0 += kQkvThreads * kCopyBatch) {
      uint4 r[kCopyBatch];
#pragma unroll
      for (int u = 0; u < kCopyBatch; ++u) {
        const int e = min(e0 + u * kQkvThreads, total - 1);
        r[u] = reinterpret_cast<const uint4*>(rows + (e / per) * row_elems + (size_t)h * G * D)[e % per];
      }
#pragma unroll
      for (int u = 0; u < kCopyBatch; ++u) {
        const int e = min(e0 + u * kQkvThreads, total - 1);
        reinterpret_cast<uint4*>(q_out + (((size_t)b * n_tok + t0 + e / per) * n_q_heads + (size_t)h * G) * D)[e % per] = r[u];
      }
    }
  }
  load_b(0);                                         // in flight until the eviction head
  S* unit_kv = kv + ((size_t)b * n_kv_heads + h) * nb * ((size_t)2 * kBlock * D);
  // keys straight to their block, values staged as fp32 [token][d] (zero
  // for skipped tokens); the positions reach LDS for the phases after the
  // barrier
  {
    uint4 r[KVN];
    int pr[KVN];
#pragma unroll
    for (int u = 0; u < KVN; ++u) {
      const int e = min(tid + u * kQkvThreads, KV_CHUNKS - 1);
      const int i = (e >= TT * CPR ? e - TT * CPR : e) / CPR;
      const uint32_t keep = valid(i, kvp[u]) ? ~0u : 0u;   // a mask, not a branch on the load
      r[u] = make_uint4(kvr[u].x & keep, kvr[u].y & keep, kvr[u].z & keep, kvr[u].w & keep);
      pr[u] = valid(i, kvp[u]) ? kvp[u] : -1;
    }
    if (tid < TT) s_pos[tid] = valid(tid, p_own) ? p_own : -1;
#pragma unroll
    for (int u = 0; u < KVN; ++u) {
      const int e = tid + u * kQkvThreads;
      if (e >= KV_CHUNKS) continue;
      const int isv = e >= TT * CPR, f = isv ? e - TT * CPR : e, i = f / CPR, ch = f % CPR;
      if (isv) {
        float v[EPC];
        unpack16(r[u], v, T{});
#pragma unroll
        for (int k = 0; k < EPC; ++k) s_v[i * DS + ch * EPC + k] = v[k];
      } else if (pr[u] >= 0) {
        const int p = pr[u];
        S* blk = unit_kv + (size_t)(p / kBlock) * (2 * kBlock * D);
        *reinterpret_cast<uint4*>(blk + key_chunk_offset<BF16>(p % kBlock, ch, D)) = r[u];
      }
    }
  }
  __syncthreads();
  // values to their blocks.  A value fragment keeps EPC consecutive tokens
  // of one dimension in 16 bytes: a group of EPC tokens at consecutive
  // positions starting on a multiple of EPC is one 16-byte store, any other
  // group is stored element by element.
  for (int e = tid; e < D * NVG; e += kQkvThreads) {
    const int d = e / NVG, i0 = (e % NVG) * EPC;
    int pk[EPC];
    float v[EPC];
#pragma unroll
    for (int k = 0; k < EPC; ++k) {                  // all reads first (indexes clamped), no branches
      const int i = min(i0 + k, TT - 1);
      pk[k] = s_pos[i];
      v[k] = s_v[i * DS + d];
    }
    bool run = (i0 + EPC <= nt) & (pk[0] >= 0) & (pk[0] % EPC == 0);
#pragma unroll
    for (int k = 1; k < EPC; ++k) run &= pk[k] == pk[0] + k;
    if (run) {
      S* blk = unit_kv + (size_t)(pk[0] / kBlock) * (2 * kBlock * D);
      *reinterpret_cast<uint4*>(blk + (size_t)kBlock * D + value_elem_offset<BF16>(pk[0] % kBlock, d, D)) = pack16(v, T{});
    } else {
#pragma unroll
      for (int k = 0; k < EPC; ++k) {
        if (i0 + k >= nt || pk[k] < 0) continue;
        S* blk = unit_kv + (size_t)(pk[k] / kBlock) * (2 * kBlock * D);
        blk[(size_t)kBlock * D + value_elem_offset<BF16>(pk[k] % kBlock, d, D)] = f32_to_storage(v[k], T{});
      }
    }
  }
  if constexpr (TT == 1) {
    // one token: lane l forms v . W1[:, col] over its half of the dimensions
    // with vector FMAs (two chains), the halves meet across lanes l, l ^ 32,
    // and the wavefront sums its columns' softplus terms
    float term = 0.f;
    for (int cg = 0; cg < d_e; cg += kHeadCols * kQkvWaves) {
      if (cg > 0) load_b(cg);
      const float* sv = s_v + (lane >> 5) * DH;
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int i = 0; i < DH; i += 2) {
        a0 = fmaf(sv[i], bw[i], a0);
        a1 = fmaf(sv[i + 1], bw[i + 1], a1);
      }
      const float half = a0 + a1;
      const float hsum = half + __shfl_xor(half, 32);
      term = fmaf(softplus_f(hsum), w2r[0], term);
    }
    const float rs = group_sum<16>(term);            // rows of 16 lanes; the upper two rows hold zeros
    const float tot = rs + lane_value(rs, 16);
    if (lane == 0) s_part[wave][0] = tot;
  } else {
    // 16 tokens on the matrix cores: H[token][col] = sum_d v[token][d]
    // W1[d][col] in fp32 (v_mfma_f32_16x16x4_f32: A = the staged values,
    // rows = tokens; B = W1).  Lane (lg, lr) supplies A = v[lr][lg NKS + s]
    // at k-step s (read once, as 16-byte vectors) and ends a pass with
    // H[4 lg + i][col(t, lr)] in acc[t][i]; it adds softplus(H) W2[col]
    // into term[i].
    float av[NKS];
#pragma unroll
    for (int k = 0; k < NKS; k += 4) {
      const float4 x = *reinterpret_cast<const float4*>(s_v + lr * DS + lg * NKS + k);
      av[k] = x.x; av[k + 1] = x.y; av[k + 2] = x.z; av[k + 3] = x.w;
    }
    float term[4] = {0.f, 0.f, 0.f, 0.f};
    for (int cg = 0; cg < d_e; cg += kHeadCols * kQkvWaves) {
      if (cg > 0) load_b(cg);
      f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[k], bw[k], acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[k], bw[NKS + k], acc[1], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) term[i] = fmaf(softplus_f(acc[t][i]), w2r[t], term[i]);
      }
    }
    // sum over the wavefront's columns (the 16 lanes of a row)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float sum = group_sum<16>(term[i]);
      if (lr == 0) s_part[wave][4 * lg + i] = sum;
    }
  }
  // the wavefront sums are added in wavefront order
  __syncthreads();
  if (tid < nt && s_pos[tid] >= 0) {
    float sc = s_part[0][tid];
#pragma unroll
    for (int w = 1; w < kQkvWaves; ++w) sc += s_part[w][tid];
    evict_logits[((size_t)b * n_kv_heads + h) * ((size_t)cap) + s_pos[tid]] = sc;
  }
}

template <class T, int D, int TT>
static void launch(const LaunchQkv& a) {
  const dim3 grid((a.n_tok + TT - 1) / TT, a.batch, a.n_kv_heads), block(kQkvThreads);
  hipLaunchKernelGGL((qkv_kernel<T, D, TT>), grid, block, 0, a.stream, (const typename T::storage*)a.qkv, a.n_tok,
                     a.pos, a.w1, a.w2, a.d_e, a.n_q_heads, a.n_kv_heads, a.nb, (typename T::storage*)a.q_out,
                     (typename T::storage*)a.kv, a.evict_logits);
}

template <class T>
static void launch_dim(const LaunchQkv& a) {
  const bool chunk = a.n_tok >= 16;
  if (a.head_dim == 128) chunk ? launch<T, 128, 16>(a) : launch<T, 128, 1>(a);
  else chunk ? launch<T, 64, 16>(a) : launch<T, 64, 1>(a);
}

void launch_qkv(const LaunchQkv& a) {
  if (a.bf16) launch_dim<Bf16>(a); else launch_dim<F32>(a);
}

}  // namespace nosa
