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
//  * Scan: groups of D*esize/16 lanes read one 16-byte chunk each of a row
//    (a wavefront load is 1 KiB of contiguous rows), two rounds of 8 loads
//    per thread in flight; the partial dot products are summed across lanes
//    with DPP and the max over a block's 4 rows is taken on wavefront-uniform
//    lane reads.
//  * Selection: each half of the workgroup (one per budget) bins its scores
//    into 256 equal value bins between their min and max, finds the bin
//    holding the k-th best, takes every block above it and ranks the few
//    blocks inside it exactly by (score desc, id asc).  The union is then
//    written in ascending order with one prefix sum.
#include "nosa_common.h"
#include "nosa_launch.h"

namespace nosa {

constexpr int kSelThreads = 1024;
constexpr int kHalf = kSelThreads / 2;
constexpr int kHalfWaves = kHalf / 64;
constexpr int kBins = 256;
constexpr int kScanUnroll = 8;   // 16-byte loads per thread per round (two rounds in flight)

size_t select_ws_bytes(int batch, int n_query, int n_kv_heads, int nb) {
  const size_t rows = (size_t)batch * n_query * n_kv_heads;
  return align256(rows * sizeof(int32_t)) + align256(rows * (size_t)nb * sizeof(float));
}

size_t select_lds_bytes(int nb) {
  // two key arrays (4 B per block), two boundary lists (2 B), two flag arrays (1 B)
  return align256((size_t)nb * 4) * 2 + align256((size_t)nb * 2) * 2 + align256((size_t)nb) * 2;
}

// Scan splits per row: about 128 blocks per workgroup (measured best at 32K
// context: fewer splits leave the scan's fp32 dot products VALU-bound on too
// few CUs, more add hand-off work), at most 16, and fewer when there are many
// rows to fill the GPU already.
static int select_splits(int rows, int nb) {
  int s = (nb + 127) / 128;
  s = s < 1 ? 1 : (s > 16 ? 16 : s);
  while (s > 1 && rows * s > 2048) --s;
  return s;
}

// Inverse of orderable(): the float a key came from.
__device__ __forceinline__ float key_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Select the k best of keys[0..n) (larger key first, then lower index) and set
// flag[i] = 1 for them.  Run by the kHalf threads `tid` of one half of the
// workgroup; both halves call it together so the barriers match.
//   hist: kBins ints, small: 32 ints, blist: n ids  (all private to the half)
// The bins split [min, max] of the scores evenly in value (fp64 arithmetic:
// the bin of a score never decreases as the score grows), so every block in
// a bin above the threshold bin is selected and only the threshold bin is
// ranked exactly.
__device__ void select_top(const uint32_t* keys, int n, int k, uint8_t* flag, int* hist, int* small,
                           uint16_t* blist, int tid) {
  const int lane = tid & 63, wv = tid >> 6;
  const bool all = k >= n;
  const bool none = k <= 0 || n <= 0;
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = tid; i < n; i += kHalf) {
    const uint32_t u = keys[i];
    lo = min(lo, u);
    hi = max(hi, u);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, off));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, off));
  }
  for (int i = tid; i < kBins; i += kHalf) hist[i] = 0;
  if (lane == 0) {
    small[2 * wv] = (int)lo;
    small[2 * wv + 1] = (int)hi;
  }
  if (tid == 0) small[17] = 0;
  __syncthreads();
  lo = (uint32_t)small[0];
  hi = (uint32_t)small[1];
#pragma unroll
  for (int w = 1; w < kHalfWaves; ++w) {
    lo = min(lo, (uint32_t)small[2 * w]);
    hi = max(hi, (uint32_t)small[2 * w + 1]);
  }
  const double vlo = key_value(lo), vhi = key_value(hi);
  const double scale = vhi > vlo ? (double)kBins / (vhi - vlo) : 0.0;
  auto bin_of = [&](uint32_t u) { return min(kBins - 1, (int)(((double)key_value(u) - vlo) * scale)); };
  if (!none && !all)
    for (int i = tid; i < n; i += kHalf) atomicAdd(&hist[bin_of(keys[i])], 1);
  __syncthreads();
  if (!none && !all && wv == 0) {
    // lane owns bins 255-4*lane .. 252-4*lane (descending)
    int cnt[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { cnt[j] = hist[kBins - 1 - 4 * lane - j]; local += cnt[j]; }
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int run = incl - local;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (run < k && run + cnt[j] >= k) {
        small[16] = kBins - 1 - 4 * lane - j;  // the bin holding the k-th best
        small[18] = k - run;                   // how many of that bin to take
      }
      run += cnt[j];
    }
  }
  __syncthreads();
  const int bstar = small[16];
  const int take = small[18];
  if (!none) {
    for (int i = tid; i < n; i += kHalf) {
      if (all) {
        flag[i] = 1;
        continue;
      }
      const int bi = bin_of(keys[i]);
      if (bi > bstar)
        flag[i] = 1;
      else if (bi == bstar)
        blist[atomicAdd(&small[17], 1)] = (uint16_t)i;
    }
  }
  __syncthreads();
  if (!none && !all) {
    const int m = small[17];
    for (int a = tid; a < m; a += kHalf) {
      const uint32_t ia = blist[a], ua = keys[ia];
      int rank = 0;
#pragma unroll 8
      for (int j = 0; j < m; ++j) {
        const uint32_t ib = blist[j], ub = keys[ib];
        rank += (ub > ua) || (ub == ua && ib < ia);
      }
      if (rank < take) flag[ia] = 1;
    }
  }
  __syncthreads();
}

template <class T, int D>
__global__ void __launch_bounds__(kSelThreads) select_kernel(
    const typename T::storage* __restrict__ q, const int32_t* __restrict__ pos,
    const typename T::storage* __restrict__ k_comp, const float* __restrict__ e_blk, int n_query,
    int n_q_heads, int n_kv_heads, int nb, int kq, int ke, int32_t* __restrict__ sel,
    int32_t* __restrict__ n_sel, int32_t* __restrict__ ticket, float* __restrict__ score) {
  constexpr int EPC = T::kPer16B;
  constexpr int LPR = D / EPC;            // lanes per compressed-key row
  constexpr int RPW = kWave / LPR;        // rows per wavefront load (2, 4 or 8)
  constexpr int WAVES = kSelThreads / kWave;
  constexpr int ROWS_PER_ROUND = WAVES * kScanUnroll * RPW;
  const int G = n_q_heads / n_kv_heads;
  const int row = blockIdx.y;             // (b * n_query + r) * Hkv + h
  const int h = row % n_kv_heads;
  const int br = row / n_kv_heads;        // b * n_query + r
  const int b = br / n_query;
  const int64_t unit = (int64_t)b * n_kv_heads + h;
  const int k_cap = kq + ke;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  float* my_score = score + (size_t)row * nb;

  // block eviction scores and cleared flags first, so their loads overlap the scan
  const float* eb = e_blk + (size_t)unit * nb;
  const bool selector = n_split == 1 || blockIdx.x == 0;
  if (selector) {
    for (int j = tid; j < c; j += kSelThreads) {
      key_e[j] = orderable(eb[j]);
      flag_q[j] = 0;
      flag_e[j] = 0;
    }
  }

  // ---- scan: block scores of blocks [blk_lo, blk_hi)
  if (blk_lo < blk_hi) {
    const int ch = lane % LPR;
    const int row_lo = kSubsPerBlock * blk_lo, row_hi = kSubsPerBlock * blk_hi;
    // the query sum first: all G loads in flight at once, ahead of the key stream
    float qs[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) qs[e] = 0.0f;
    {
      const typename T::storage* qh = q + ((size_t)br * n_q_heads + (size_t)h * G) * D + ch * EPC;
      uint4 qr[16];
#pragma unroll
      for (int g = 0; g < 16; ++g) qr[g] = g < G ? ld16(qh + (size_t)g * D) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        float v[EPC];
        unpack16(qr[g], v, T{});
#pragma unroll
        for (int e = 0; e < EPC; ++e) qs[e] += v[e];
      }
    }
    const typename T::storage* kc = k_comp + (size_t)unit * nb * kSubsPerBlock * D + ch * EPC;
    auto load_round = [&](uint4 (&raw)[kScanUnroll], int r0) {
#pragma unroll
      for (int u = 0; u < kScanUnroll; ++u) {
        const int rr = r0 + (wave * kScanUnroll + u) * RPW + lane / LPR;
        raw[u] = (rr < row_hi) ? ld16(kc + (size_t)rr * D) : make_uint4(0, 0, 0, 0);
      }
    };
    auto score_round = [&](const uint4 (&raw)[kScanUnroll], int r0) {
      float pend = 0.0f;  // first half of a block when a row spans 32 lanes
#pragma unroll
      for (int u = 0; u < kScanUnroll; ++u) {
        const int first = r0 + (wave * kScanUnroll + u) * RPW;  // first row of this load
        float v[EPC];
        unpack16(raw[u], v, T{});
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) s = fmaf(qs[e], v[e], s);
        s = group_sum<(LPR < 16 ? LPR : 16)>(s);
        // row sums sit in lanes 0, 16, 32, 48 (or every 8 lanes); the block
        // maximum is taken on those wavefront-uniform values
        if constexpr (LPR == 16) {
          const float m = fmaxf(fmaxf(lane_value(s, 0), lane_value(s, 16)),
                                fmaxf(lane_value(s, 32), lane_value(s, 48)));
          if (lane == 0 && first < row_hi) {
            if (n_split == 1) key_q[first / kSubsPerBlock] = orderable(m);
            else store_coherent(&my_score[first / kSubsPerBlock], m);
          }
        } else if constexpr (LPR == 8) {
          const float m0 = fmaxf(fmaxf(lane_value(s, 0), lane_value(s, 8)),
                                 fmaxf(lane_value(s, 16), lane_value(s, 24)));
          const float m1 = fmaxf(fmaxf(lane_value(s, 32), lane_value(s, 40)),
                                 fmaxf(lane_value(s, 48), lane_value(s, 56)));
          if (lane < 2 && first + 4 * lane < row_hi) {
            const float m = lane ? m1 : m0;
            const int blk = first / kSubsPerBlock + lane;
            if (n_split == 1) key_q[blk] = orderable(m);
            else store_coherent(&my_score[blk], m);
          }
        } else {  // LPR == 32: two rows per load, a block over two loads
          const float r0s = lane_value(s, 0) + lane_value(s, 16);
          const float r1s = lane_value(s, 32) + lane_value(s, 48);
          const float m = fmaxf(r0s, r1s);
          if ((u & 1) == 0) {
            pend = m;
          } else if (lane == 0 && first < row_hi) {
            const float mb = fmaxf(m, pend);
            if (n_split == 1) key_q[first / kSubsPerBlock] = orderable(mb);
            else store_coherent(&my_score[first / kSubsPerBlock], mb);
          }
        }
      }
    };
    // two rounds of loads in flight: round i+1 streams in while round i is scored
    uint4 ra[kScanUnroll], rb[kScanUnroll];
    load_round(ra, row_lo);
    for (int r0 = row_lo; r0 < row_hi; r0 += 2 * ROWS_PER_ROUND) {
      load_round(rb, r0 + ROWS_PER_ROUND);
      score_round(ra, r0);
      load_round(ra, r0 + 2 * ROWS_PER_ROUND);
      score_round(rb, r0 + ROWS_PER_ROUND);
    }
  }

  if (n_split > 1) {
    // ---- ticket: the last workgroup of this row selects
    __shared__ int s_last;
    wait_stores_done();
    __syncthreads();
    if (tid == 0) {
      const int t = ticket_take(&ticket[row]);
      s_last = (t == n_split - 1);
      if (s_last) ticket_reset(&ticket[row]);
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
  __syncthreads();
  const int half = tid / kHalf;
  select_top(half ? key_e : key_q, c, half ? ke : kq, half ? flag_e : flag_q, s_hist[half],
             s_small[half], half ? blist_e : blist_q, tid % kHalf);

  // ---- union in ascending order: each thread owns a contiguous id range
  __shared__ int s_wsum[WAVES];
  const int per = (c + kSelThreads - 1) / kSelThreads;
  const int lo = tid * per, hi = min(c, lo + per);
  int cnt = 0;
  for (int j = lo; j < hi; ++j) cnt += (flag_q[j] | flag_e[j]) ? 1 : 0;
  int incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int off = incl - cnt, total = 0;
  for (int w = 0; w < WAVES; ++w) {
    if (w < wave) off += s_wsum[w];
    total += s_wsum[w];
  }
  int32_t* out = sel + (size_t)row * k_cap;
  for (int j = lo; j < hi; ++j)
    if (flag_q[j] | flag_e[j]) out[off++] = j;
  for (int i = total + tid; i < k_cap; i += kSelThreads) out[i] = -1;
  if (tid == 0) n_sel[row] = total;
}

template <class T, int D>
static void launch(const LaunchSelect& a) {
  const int rows = a.batch * a.n_query * a.n_kv_heads;
  const int splits = select_splits(rows, a.nb);
  char* ws = (char*)a.ws;
  int32_t* ticket = (int32_t*)ws;
  float* score = (float*)(ws + align256((size_t)rows * sizeof(int32_t)));
  hipLaunchKernelGGL((select_kernel<T, D>), dim3(splits, rows), dim3(kSelThreads),
                     select_lds_bytes(a.nb), a.stream, (const typename T::storage*)a.q, a.pos,
                     (const typename T::storage*)a.k_comp, a.e_blk, a.n_query, a.n_q_heads,
                     a.n_kv_heads, a.nb, a.kq, a.ke, a.sel, a.n_sel, ticket, score);
}

void launch_select(const LaunchSelect& a) {
  if (a.bf16) {
    if (a.head_dim == 128) launch<Bf16, 128>(a); else launch<Bf16, 64>(a);
  } else {
    if (a.head_dim == 128) launch<F32, 128>(a); else launch<F32, 64>(a);
  }
}

}  // namespace nosa
