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

namespace nosa {

// One block per wavefront and 8 wavefronts per workgroup (4 when the GQA
// group needs all 16 MFMA columns, to keep the LDS merge buffer within
// 64 KiB).  Fewer, fuller workgroups beat more, smaller ones here: every
// split adds a partial to write, a ticket and a share of the final merge.
static inline int attn_waves(int G) { return G <= 8 ? 8 : 4; }
static inline int attn_splits(int k_cap, int G) { return (k_cap + 1 + attn_waves(G) - 1) / attn_waves(G); }

size_t attn_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim, int k_cap) {
  const size_t units = (size_t)batch * n_kv_heads;
  const size_t G = n_q_heads / n_kv_heads;
  const size_t splits = attn_splits(k_cap, (int)G);
  return align256(units * sizeof(int32_t)) + align256(units * splits * G * 2 * sizeof(float)) +
         align256(units * splits * G * head_dim * sizeof(float));
}

// Token of row r of S tile t, chosen so that lane group g (lanes 16g..16g+15)
// ends up holding consecutive tokens for the P^T operand.
template <class T>
__device__ __forceinline__ int tile_token(int t, int r);
template <>
__device__ __forceinline__ int tile_token<Bf16>(int t, int r) {
  return 32 * (t >> 1) + 8 * (r >> 2) + 4 * (t & 1) + (r & 3);
}
template <>
__device__ __forceinline__ int tile_token<F32>(int t, int r) {
  return 16 * t + r;
}

template <class T, int D>
struct Frags;

// bf16: K operand 4 tiles x D/32 k-steps, V operand 2 halves x D/16 d-tiles
template <int D>
struct Frags<Bf16, D> {
  static constexpr int NK = D / 32;
  static constexpr int ND = D / 16;
  bf16x8 q[NK];
  uint4 k[4][NK];
  uint4 v[2][ND];
};
// fp32: K operand 4 tiles x D/16 chunks of 4, V operand 4 tiles x D/16 d-tiles
template <int D>
struct Frags<F32, D> {
  static constexpr int NK = D / 16;
  static constexpr int ND = D / 16;
  float4 q[NK];
  uint4 k[4][NK];
  uint4 v[4][ND];
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

template <class T, int D>
__device__ __forceinline__ void load_q(Frags<T, D>& f, const typename T::storage* qg, int G, int lane) {
  const int col = lane & 15, grp = lane >> 4;
  if constexpr (sizeof(typename T::storage) == 2) {
#pragma unroll
    for (int s = 0; s < Frags<T, D>::NK; ++s) {
      const uint4 u = (col < G) ? ld16(qg + (size_t)col * D + 32 * s + 8 * grp) : make_uint4(0, 0, 0, 0);
      f.q[s] = as_bf16x8(u);
    }
  } else {
#pragma unroll
    for (int s = 0; s < Frags<T, D>::NK; ++s) {
      const uint4 u = (col < G) ? ld16(qg + (size_t)col * D + 16 * s + 4 * grp) : make_uint4(0, 0, 0, 0);
      f.q[s] = make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                           __uint_as_float(u.w));
    }
  }
}

// One block's operands: 32 fully contiguous 1 KiB wavefront loads (see the
// block format in nosa_common.h).
template <class T, int D>
__device__ __forceinline__ void load_block(Frags<T, D>& f, const typename T::storage* blk, int lane) {
  constexpr int EPC = T::kPer16B;
  constexpr int NK = Frags<T, D>::NK, ND = Frags<T, D>::ND;
  const typename T::storage* kp = blk + lane * EPC;
  const typename T::storage* vp = blk + (size_t)kBlock * D + lane * EPC;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int s = 0; s < NK; ++s) f.k[t][s] = ld16(kp + (size_t)(t * NK + s) * 64 * EPC);
  constexpr int NVT = sizeof(f.v) / sizeof(f.v[0]);  // 2 token halves (bf16) or 4 tiles (fp32)
#pragma unroll
  for (int h = 0; h < NVT; ++h)
#pragma unroll
    for (int u = 0; u < ND; ++u) f.v[h][u] = ld16(vp + (size_t)(h * ND + u) * 64 * EPC);
}

// S^T tiles of one block: acc[t][i] = q_col . K[tile_token(t, 4*grp + i)]
template <class T, int D>
__device__ __forceinline__ void block_scores(const Frags<T, D>& f, f32x4 (&acc)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    if constexpr (sizeof(typename T::storage) == 2) {
#pragma unroll
      for (int s = 0; s < Frags<T, D>::NK; ++s)
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.k[t][s]), f.q[s], a, 0, 0, 0);
    } else {
#pragma unroll
      for (int s = 0; s < Frags<T, D>::NK; ++s) {
        const float4 q = f.q[s];
        a = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.k[t][s].x), q.x, a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.k[t][s].y), q.y, a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.k[t][s].z), q.z, a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(f.k[t][s].w), q.w, a, 0, 0, 0);
      }
    }
    acc[t] = a;
  }
}

// O^T += V^T . P^T for one block
template <class T, int D>
__device__ __forceinline__ void block_pv(const Frags<T, D>& f, const float (&p)[4][4], f32x4 (&o)[D / 16]) {
  if constexpr (sizeof(typename T::storage) == 2) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      bf16x8 pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pb[i] = (__bf16)p[2 * h2][i];
        pb[4 + i] = (__bf16)p[2 * h2 + 1][i];
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f.v[h2][dt]), pb, o[dt], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const uint4 v = f.v[t][dt];
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.x), p[t][0], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.y), p[t][1], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.z), p[t][2], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.w), p[t][3], o[dt], 0, 0, 0);
      }
  }
}

template <class T, int D, int WAVES, int GMAX>
__global__ void __launch_bounds__(64 * WAVES) attn_kernel(
    const typename T::storage* __restrict__ q, const typename T::storage* __restrict__ blocks,
    int blocks_per_head, const int32_t* __restrict__ phys, const int32_t* __restrict__ n_sel,
    int k_cap, const typename T::storage* __restrict__ window_kv, int64_t win_head_stride,
    int64_t win_block_stride, const int32_t* __restrict__ pos, float scale_log2, int n_q_heads,
    int n_kv_heads, int nb, typename T::storage* __restrict__ out, int32_t* __restrict__ ticket,
    float* __restrict__ part_ml, float* __restrict__ part_o) {
  constexpr int ND = D / 16;
  constexpr int NT = 64 * WAVES;
  const int G = n_q_heads / n_kv_heads;
  // grid (units, splits): workgroups are dispatched x-fastest, so every
  // unit's first split starts before any unit's second and the light last
  // splits (often just the window) go last
  const int n_split = gridDim.y;
  const int split = blockIdx.y;
  const int unit = blockIdx.x;  // b * Hkv + h
  const int b = unit / n_kv_heads;
  const int h = unit % n_kv_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const size_t blk_elems = (size_t)2 * kBlock * D;

  const int p = pos[b];
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
  const int e = split * WAVES + wave;
  const typename T::storage* blk = nullptr;
  int len = 0;
  if (e < ns) {
    const int pb = phys[(size_t)unit * k_cap + e];
    if (pb >= 0 && pb < blocks_per_head) {
      blk = blocks + ((size_t)unit * blocks_per_head + pb) * blk_elems;
      len = kBlock;
    }
  } else if (e < n_ent) {
    blk = window_kv + (int64_t)unit * win_head_stride + (int64_t)c * win_block_stride;
    len = p - c * kBlock + 1;
  }
  if (blk != nullptr) {
    Frags<T, D> f;
    load_block<T, D>(f, blk, lane);
    load_q<T, D>(f, q + ((size_t)b * n_q_heads + (size_t)h * G) * D, G, lane);
    f32x4 acc[4];
    block_scores<T, D>(f, acc);
    float x[4][4];
    float mb = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tile_token<T>(t, 4 * grp + i);
        x[t][i] = (tok < len) ? acc[t][i] * scale_log2 : -INFINITY;
        mb = fmaxf(mb, x[t][i]);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    float pw[4][4], lb = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pw[t][i] = exp2f(x[t][i] - mb);
        lb += pw[t][i];
      }
    lb += __shfl_xor(lb, 16);
    lb += __shfl_xor(lb, 32);
    m_run = mb;
    l_run = lb;
    block_pv<T, D>(f, pw, o);
  }

  // ---- merge the wavefronts of this workgroup through LDS
  __shared__ float s_o[WAVES][GMAX][D + 4];
  __shared__ float s_m[WAVES][GMAX], s_l[WAVES][GMAX];
  if (col < G) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[wave][col][16 * dt + 4 * grp + i] = o[dt][i];
    if (grp == 0) {
      s_m[wave][col] = m_run;
      s_l[wave][col] = l_run;
    }
  }
  __syncthreads();

  typename T::storage* out_u = out + ((size_t)b * n_q_heads + (size_t)h * G) * D;
  float* pml = part_ml + (size_t)unit * n_split * G * 2;
  float* po = part_o + (size_t)unit * n_split * G * D;
  for (int idx = tid; idx < G * D; idx += NT) {
    const int g = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, s_m[w][g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float wt = (s_m[w][g] == -INFINITY) ? 0.f : exp2f(s_m[w][g] - M);
      num += wt * s_o[w][g][d];
      den += wt * s_l[w][g];
    }
    if (n_split == 1) {
      const float r = den > 0.f ? num / den : 0.f;
      if constexpr (sizeof(typename T::storage) == 2)
        out_u[idx] = (uint16_t)f32_to_bf16_bits(r);
      else
        out_u[idx] = r;
    } else {
      store_coherent(&po[((size_t)split * G + g) * D + d], num);
      if (d == 0) {
        store_coherent(&pml[((size_t)split * G + g) * 2 + 0], M);
        store_coherent(&pml[((size_t)split * G + g) * 2 + 1], den);
      }
    }
  }
  if (n_split == 1) return;

  // ---- the last workgroup of this (b, h) merges the splits
  __shared__ int s_last;
  wait_stores_done();
  __syncthreads();
  if (tid == 0) {
    const int t = ticket_take(&ticket[unit]);
    s_last = (t == n_split - 1);
    if (s_last) ticket_reset(&ticket[unit]);
  }
  __syncthreads();
  if (!s_last) return;

  // every partial this thread needs is loaded in one round trip: the split
  // maxima and sums into LDS (reusing the merge buffer), the numerators into
  // registers; then weights, then the weighted sums
  constexpr int kMaxSplitRegs = 20;
  float* fm = &s_o[0][0][0];
  float* fl = fm + n_split * G;
  __shared__ float s_den[GMAX];
  for (int i = tid; i < n_split * G; i += NT) {
    fm[i] = load_coherent(&pml[2 * i]);
    fl[i] = load_coherent(&pml[2 * i + 1]);
  }
  constexpr int PER = (GMAX * D + NT - 1) / NT;  // outputs per thread
  float v[PER][kMaxSplitRegs];
  const bool in_regs = n_split <= kMaxSplitRegs;
  if (in_regs) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int idx = tid + r * NT;
      const int g = idx / D, d = idx % D;
#pragma unroll
      for (int s = 0; s < kMaxSplitRegs; ++s)
        v[r][s] = (idx < G * D && s < n_split) ? load_coherent(&po[((size_t)s * G + g) * D + d]) : 0.f;
    }
  }
  __syncthreads();
  if (tid < G) {
    float M = -INFINITY;
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, fm[s * G + tid]);
    float den = 0.f;
    for (int s = 0; s < n_split; ++s) {
      const float ms = fm[s * G + tid];
      const float wt = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
      fm[s * G + tid] = wt;
      den += wt * fl[s * G + tid];
    }
    s_den[tid] = den;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int idx = tid + r * NT;
    if (idx >= G * D) break;
    const int g = idx / D, d = idx % D;
    float num = 0.f;
    if (in_regs) {
#pragma unroll
      for (int s = 0; s < kMaxSplitRegs; ++s)
        if (s < n_split) num += fm[s * G + g] * v[r][s];
    } else {
      for (int s = 0; s < n_split; ++s) num += fm[s * G + g] * load_coherent(&po[((size_t)s * G + g) * D + d]);
    }
    const float den = s_den[g];
    const float res = den > 0.f ? num / den : 0.f;
    if constexpr (sizeof(typename T::storage) == 2)
      out_u[idx] = (uint16_t)f32_to_bf16_bits(res);
    else
      out_u[idx] = res;
  }
}

template <class T, int D, int WAVES, int GMAX>
static void launch_w(const LaunchAttn& a) {
  const int units = a.batch * a.n_kv_heads;
  const int G = a.n_q_heads / a.n_kv_heads;
  const int splits = attn_splits(a.k_cap, G);
  char* ws = (char*)a.ws;
  int32_t* ticket = (int32_t*)ws;
  float* part_ml = (float*)(ws + align256((size_t)units * sizeof(int32_t)));
  float* part_o = (float*)((char*)part_ml + align256((size_t)units * splits * G * 2 * sizeof(float)));
  const float scale_log2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((attn_kernel<T, D, WAVES, GMAX>), dim3(units, splits), dim3(64 * WAVES), 0,
                     a.stream, (const typename T::storage*)a.q, (const typename T::storage*)a.blocks,
                     a.blocks_per_head, a.phys, a.n_sel, a.k_cap,
                     (const typename T::storage*)a.window_kv, a.window_head_stride,
                     a.window_block_stride, a.pos, scale_log2, a.n_q_heads, a.n_kv_heads, a.nb,
                     (typename T::storage*)a.out, ticket, part_ml, part_o);
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
