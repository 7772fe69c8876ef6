// Device building blocks of the NOSA block selection: the compressed-key
// scan (block scores), the exact top-k of a half workgroup, and the
// ascending union.  Used by the stand-alone selection kernel and by the
// fused decode-step kernel.
#pragma once

#include "nosa_common.h"

namespace nosa {

constexpr int kBins = 256;
constexpr int kScanUnroll = 8;   // 16-byte loads per thread per round (two rounds in flight)

// Inverse of orderable(): the float a key came from.
__device__ __forceinline__ float key_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Select the k best of keys[0..n) (larger key first, then lower index) and set
// flag[i] = 1 for them.  Run by the kHalf threads `tid` of one half of the
// workgroup (kHalf <= 1024); both halves call it together so the barriers
// match.  hist: kBins ints, small: 32 ints, blist: n ids (private to the half)
// The bins split [min, max] of the scores evenly in value (fp64 arithmetic:
// the bin of a score never decreases as the score grows), so every block in
// a bin above the threshold bin is selected and only the threshold bin is
// ranked exactly.
template <int kHalf>
__device__ void select_top(const uint32_t* keys, int n, int k, uint8_t* flag, int* hist, int* small,
                           uint16_t* blist, int tid) {
  constexpr int kHalfWaves = kHalf / 64;
  const int lane = tid & 63, wv = tid >> 6;
  const bool all = k >= n;
  const bool none = k <= 0 || n <= 0;
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = tid; i < n; i += kHalf) {
    const uint32_t u = keys[i];
    lo = min(lo, u);
    hi = max(hi, u);
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
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
    const int incl = wave_incl_sum(local, lane);
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


// Scan compressed-key rows [row_lo, row_hi) (whole blocks) of one KV head
// with NT threads; put(blk, score) receives every block score (called by
// one lane per block).  qh: the G query heads of the KV head.
template <class T, int D, int NT, class Put>
__device__ __forceinline__ void scan_block_scores_fma(const typename T::storage* qh, int G,
                                                  const typename T::storage* kc_unit, int row_lo,
                                                  int row_hi, int tid, Put put) {
  constexpr int EPC = T::kPer16B;
  constexpr int LPR = D / EPC;            // lanes per compressed-key row
  constexpr int RPW = kWave / LPR;        // rows per wavefront load (2, 4 or 8)
  constexpr int WAVES = NT / kWave;
  constexpr int ROWS_PER_ROUND = WAVES * kScanUnroll * RPW;
  const int lane = tid & 63, wave = tid >> 6;
  const int ch = lane % LPR;
  const typename T::storage* kc = kc_unit + ch * EPC;
  auto load_round = [&](uint4 (&raw)[kScanUnroll], int r0) {
#pragma unroll
    for (int u = 0; u < kScanUnroll; ++u) {
      const int rr = r0 + (wave * kScanUnroll + u) * RPW + lane / LPR;
      raw[u] = (rr < row_hi) ? ld16(kc + (size_t)rr * D) : make_uint4(0, 0, 0, 0);
    }
  };
  // the first round of keys and the G query rows go out together; the query
  // sum only waits for the query loads
  uint4 ra[kScanUnroll], rb[kScanUnroll];
  load_round(ra, row_lo);
  float qs[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) qs[e] = 0.0f;
  {
    uint4 qr[16];
#pragma unroll
    for (int g = 0; g < 16; ++g) qr[g] = g < G ? ld16(qh + (size_t)g * D + ch * EPC) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      float v[EPC];
      unpack16(qr[g], v, T{});
#pragma unroll
      for (int e = 0; e < EPC; ++e) qs[e] += v[e];
    }
  }
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
        if (lane == 0 && first < row_hi) put(first / kSubsPerBlock, m);
      } else if constexpr (LPR == 8) {
        const float m0 = fmaxf(fmaxf(lane_value(s, 0), lane_value(s, 8)),
                               fmaxf(lane_value(s, 16), lane_value(s, 24)));
        const float m1 = fmaxf(fmaxf(lane_value(s, 32), lane_value(s, 40)),
                               fmaxf(lane_value(s, 48), lane_value(s, 56)));
        if (lane < 2 && first + 4 * lane < row_hi) put(first / kSubsPerBlock + lane, lane ? m1 : m0);
      } else {  // LPR == 32: two rows per load, a block over two loads
        const float r0s = lane_value(s, 0) + lane_value(s, 16);
        const float r1s = lane_value(s, 32) + lane_value(s, 48);
        const float m = fmaxf(r0s, r1s);
        if ((u & 1) == 0)
          pend = m;
        else if (lane == 0 && first < row_hi)
          put(first / kSubsPerBlock, fmaxf(m, pend));
      }
    }
  };
  // two rounds of loads in flight: round i+1 streams in while round i is scored
  for (int r0 = row_lo; r0 < row_hi; r0 += 2 * ROWS_PER_ROUND) {
    load_round(rb, r0 + ROWS_PER_ROUND);
    score_round(ra, r0);
    if (r0 + ROWS_PER_ROUND >= row_hi) break;
    load_round(ra, r0 + 2 * ROWS_PER_ROUND);
    score_round(rb, r0 + ROWS_PER_ROUND);
  }
}

// bf16 scan on MFMA: a 16-row tile of compressed keys times the G query
// heads (16x16x32 products, rows in the A operand, heads in B, fp32
// accumulation), then the per-row sum over the heads (DPP within each
// 16-lane row) and the maximum over the four rows of a block, which the
// accumulator layout puts in one lane group.  Each head's dot product is
// exact-product fp32 accumulation; the head sum is a fixed tree.
// The constructor issues the first round of loads (every load unconditional,
// rows clamped into the range, so a caller can issue more loads behind them
// and the compiler still waits for exactly these); finish() scores them and
// any further rounds.  Requires row_lo < row_hi.
template <int D, int NT>
struct MfmaScan {
  static constexpr int NK = D / 32;      // k-steps of 32 dims
  static constexpr int WAVES = NT / 64;
  // tiles per wavefront per round: two with 8 wavefronts; one with 16, whose
  // 128-VGPR budget two double-buffered tiles overrun (spills)
  static constexpr int TPR = NT >= 1024 ? 1 : 2;
  const uint16_t* kc;
  int row_lo, row_hi, n_tiles, n_rounds, wave, col, grp;
  uint4 ra[TPR][NK];
  bf16x8 qf[NK];

  __device__ __forceinline__ MfmaScan(const uint16_t* qh, int G, const uint16_t* kc_unit, int row_lo_, int row_hi_,
                                      int tid)
      : kc(kc_unit), row_lo(row_lo_), row_hi(row_hi_) {
    const int lane = tid & 63;
    wave = tid >> 6;
    col = lane & 15;
    grp = lane >> 4;
    n_tiles = (row_hi - row_lo + 15) / 16;
    n_rounds = (n_tiles + TPR * WAVES - 1) / (TPR * WAVES);
    load(ra, 0);
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const uint4 u = col < G ? ld16(qh + (size_t)col * D + 32 * s + 8 * grp) : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8, u);
    }
  }
  __device__ __forceinline__ void load(uint4 (&raw)[TPR][NK], int round) const {
#pragma unroll
    for (int t = 0; t < TPR; ++t) {
      const int tile = (round * TPR + t) * WAVES + wave;
      const int row = min(row_lo + 16 * tile + col, row_hi - 1);
#pragma unroll
      for (int s = 0; s < NK; ++s) raw[t][s] = ld16(kc + (size_t)row * D + 32 * s + 8 * grp);
    }
  }
  template <class Put>
  __device__ __forceinline__ void score(const uint4 (&raw)[TPR][NK], int round, Put put) const {
#pragma unroll
    for (int t = 0; t < TPR; ++t) {
      const int tile = (round * TPR + t) * WAVES + wave;
      if (tile >= n_tiles) continue;   // wavefront-uniform
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NK; ++s)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, raw[t][s]), qf[s], acc, 0, 0, 0);
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, group_sum<16>(acc[i]));
      const int row0 = row_lo + 16 * tile + 4 * grp;   // first row of this lane group's block
      if (col == 0 && row0 < row_hi) put(row0 / kSubsPerBlock, m);
    }
  }
  template <class Put>
  __device__ __forceinline__ void finish(Put put) {
    uint4 rb[TPR][NK];
    for (int r = 0; r < n_rounds; r += 2) {
      if (r + 1 < n_rounds) load(rb, r + 1);
      score(ra, r, put);
      if (r + 1 >= n_rounds) break;
      if (r + 2 < n_rounds) load(ra, r + 2);
      score(rb, r + 1, put);
    }
  }
};

template <int D, int NT, class Put>
__device__ __forceinline__ void scan_block_scores_mfma(const uint16_t* qh, int G, const uint16_t* kc_unit,
                                                       int row_lo, int row_hi, int tid, Put put) {
  if (row_lo >= row_hi) return;
  MfmaScan<D, NT> sc(qh, G, kc_unit, row_lo, row_hi, tid);
  sc.finish(put);
}

// Block scores of compressed-key rows [row_lo, row_hi) (whole blocks) of one
// KV head with NT threads: put(blk, score) receives every block score (one
// lane per block).  bf16 keys use the MFMA scan, fp32 keys the FMA scan.
template <class T, int D, int NT, class Put>
__device__ __forceinline__ void scan_block_scores(const typename T::storage* qh, int G,
                                                  const typename T::storage* kc_unit, int row_lo,
                                                  int row_hi, int tid, Put put) {
  if constexpr (sizeof(typename T::storage) == 2)
    scan_block_scores_mfma<D, NT>(qh, G, kc_unit, row_lo, row_hi, tid, put);
  else
    scan_block_scores_fma<T, D, NT>(qh, G, kc_unit, row_lo, row_hi, tid, put);
}

// Write the ids j in [0, c) with pick(j) in ascending order to out[0 ..
// total), pad to k_cap with -1; returns total (in every thread).  wsum:
// NT/64 ints of LDS.
template <int NT, class Pick>
__device__ int write_ids(Pick pick, int c, int32_t* out, int k_cap, int* wsum, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  const int per = (c + NT - 1) / NT;
  const int lo = tid * per, hi = min(c, lo + per);
  int cnt = 0;
  for (int j = lo; j < hi; ++j) cnt += pick(j) ? 1 : 0;
  const int incl = wave_incl_sum(cnt, lane);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int off = incl - cnt, total = 0;
  for (int w = 0; w < NT / 64; ++w) {
    if (w < wave) off += wsum[w];
    total += wsum[w];
  }
  for (int j = lo; j < hi; ++j)
    if (pick(j)) out[off++] = j;
  for (int i = total + tid; i < k_cap; i += NT) out[i] = -1;
  return total;
}

// Eq. 7 read as "fill the remainder from the candidates left" (a variant,
// off by default): given flag_q = Gamma_q and flag_e = the top ke + nq of the
// eviction scores (nq = |Gamma_q|), keep in flag_e only the ke best (key
// desc, id asc) of its members outside Gamma_q.  That is the top-ke of the
// eviction scores over the candidates outside Gamma_q, since at most nq of
// the top ke + nq lie in Gamma_q.  list: scratch of at least ke + nq ints.
template <int NT>
__device__ void keep_fill(const uint32_t* key_e, const uint8_t* flag_q, uint8_t* flag_e, int c, int ke,
                          int32_t* list, int* wsum, int tid) {
  const int n = write_ids<NT>([&](int j) { return flag_e[j] != 0 && flag_q[j] == 0; }, c, list, 0, wsum, tid);
  __syncthreads();
  for (int a = tid; a < n; a += NT) {
    const int ia = list[a];
    const uint32_t ua = key_e[ia];
    int rank = 0;
    for (int b2 = 0; b2 < n; ++b2) {
      const int ib = list[b2];
      const uint32_t ub = key_e[ib];
      rank += (ub > ua) || (ub == ua && ib < ia);
    }
    if (rank >= ke) flag_e[ia] = 0;
  }
  __syncthreads();
}

// The union of two flag arrays, ascending (see write_ids).
template <int NT>
__device__ int write_union(const uint8_t* flag_q, const uint8_t* flag_e, int c, int32_t* out,
                           int k_cap, int* wsum, int tid) {
  return write_ids<NT>([&](int j) { return (flag_q[j] | flag_e[j]) != 0; }, c, out, k_cap, wsum, tid);
}

}  // namespace nosa
