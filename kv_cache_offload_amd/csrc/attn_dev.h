// Device building blocks of the NOSA decode attention: one wavefront
// attends one 64-token block with MFMA; a workgroup merges its wavefronts in
// LDS; the last workgroup of a (b, h) merges the splits.  Used by the
// stand-alone attention kernel and by the fused decode-step kernel.
#pragma once

#include "nosa_common.h"

namespace nosa {

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

template <bool STREAM>
__device__ __forceinline__ uint4 ld16_any(const void* p) {
  if constexpr (STREAM) return ld16_stream(p);
  else return ld16(p);
}

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

// Operands of NTL consecutive 16-token tiles t0 .. t0+NTL-1 of one block
// (NTL = 4: the whole block; NTL = 2: one 32-token half, t0 = 0 or 2): fully
// contiguous 1 KiB wavefront loads (see the block format in nosa_common.h).
// STREAM: non-temporal loads, for blocks no other wavefront of the launch
// reads.
template <class T, int D, int NTL, bool STREAM = false>
__device__ __forceinline__ void load_tiles(Frags<T, D>& f, const typename T::storage* blk, int t0, int lane) {
  constexpr int EPC = T::kPer16B;
  constexpr int NK = Frags<T, D>::NK, ND = Frags<T, D>::ND;
  const typename T::storage* kp = blk + lane * EPC;
  const typename T::storage* vp = blk + (size_t)kBlock * D + lane * EPC;
#pragma unroll
  for (int t = 0; t < NTL; ++t)
#pragma unroll
    for (int s = 0; s < NK; ++s) f.k[t][s] = ld16_any<STREAM>(kp + (size_t)((t0 + t) * NK + s) * 64 * EPC);
  if constexpr (sizeof(typename T::storage) == 2) {
    // V fragments come in 32-token halves
#pragma unroll
    for (int h = 0; h < NTL / 2; ++h)
#pragma unroll
      for (int u = 0; u < ND; ++u) f.v[h][u] = ld16_any<STREAM>(vp + (size_t)((t0 / 2 + h) * ND + u) * 64 * EPC);
  } else {
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
      for (int u = 0; u < ND; ++u) f.v[t][u] = ld16_any<STREAM>(vp + (size_t)((t0 + t) * ND + u) * 64 * EPC);
  }
}

// The operands load_tiles loaded, stored back in the same format to another
// block (a copy of those tiles made on the way through the registers).
template <class T, int D, int NTL>
__device__ __forceinline__ void store_tiles(const Frags<T, D>& f, typename T::storage* blk, int t0, int lane) {
  constexpr int EPC = T::kPer16B;
  constexpr int NK = Frags<T, D>::NK, ND = Frags<T, D>::ND;
  typename T::storage* kp = blk + lane * EPC;
  typename T::storage* vp = blk + (size_t)kBlock * D + lane * EPC;
#pragma unroll
  for (int t = 0; t < NTL; ++t)
#pragma unroll
    for (int s = 0; s < NK; ++s) st16(kp + (size_t)((t0 + t) * NK + s) * 64 * EPC, f.k[t][s]);
  if constexpr (sizeof(typename T::storage) == 2) {
#pragma unroll
    for (int h = 0; h < NTL / 2; ++h)
#pragma unroll
      for (int u = 0; u < ND; ++u) st16(vp + (size_t)((t0 / 2 + h) * ND + u) * 64 * EPC, f.v[h][u]);
  } else {
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
      for (int u = 0; u < ND; ++u) st16(vp + (size_t)((t0 + t) * ND + u) * 64 * EPC, f.v[t][u]);
  }
}

// S^T tiles: acc[t][i] = q_col . K[tile_token(t0 + t, 4*grp + i)]
template <class T, int D, int NTL>
__device__ __forceinline__ void block_scores(const Frags<T, D>& f, f32x4 (&acc)[4]) {
#pragma unroll
  for (int t = 0; t < NTL; ++t) {
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

// O^T += V^T . P^T over the loaded tiles
template <class T, int D, int NTL>
__device__ __forceinline__ void block_pv(const Frags<T, D>& f, const float (&p)[4][4], f32x4 (&o)[D / 16]) {
  if constexpr (sizeof(typename T::storage) == 2) {
#pragma unroll
    for (int h2 = 0; h2 < NTL / 2; ++h2) {
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
    for (int t = 0; t < NTL; ++t)
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

// One wavefront: the unnormalised attention partial of tiles t0 .. t0+NTL-1
// of one block whose operands are in f (load_tiles + load_q), the first
// `len` tokens valid.  m, l are per head (lane column), o holds
// O^T[d = 16*dt + 4*(lane/16) + i][head = lane%16].  bias_blk, when given,
// points at the block's 64 per-token additive logits (natural-log units),
// added to every head's logit of that token (the eviction-bias variant).
template <class T, int D, int NTL>
__device__ __forceinline__ void attend_frags(const Frags<T, D>& f, int t0, int len, float scale_log2, int lane,
                                             float& m_out, float& l_out, f32x4 (&o)[D / 16],
                                             const float* bias_blk = nullptr) {
  const int grp = lane >> 4;
  // the 4 rows of a tile that a lane holds are 4 consecutive tokens
  float4 bias[4];
  if (bias_blk != nullptr) {
#pragma unroll
    for (int t = 0; t < NTL; ++t) bias[t] = *reinterpret_cast<const float4*>(bias_blk + tile_token<T>(t0 + t, 4 * grp));
  }
  f32x4 acc[4];
  block_scores<T, D, NTL>(f, acc);
  float x[4][4];
  float mb = -INFINITY;
#pragma unroll
  for (int t = 0; t < NTL; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tile_token<T>(t0 + t, 4 * grp + i);
      float v = acc[t][i] * scale_log2;
      if (bias_blk != nullptr) {
        const float bv = i == 0 ? bias[t].x : (i == 1 ? bias[t].y : (i == 2 ? bias[t].z : bias[t].w));
        v = fmaf(bv, 1.4426950408889634f, v);      // natural-log units to log2 units
      }
      x[t][i] = (tok < len) ? v : -INFINITY;
      mb = fmaxf(mb, x[t][i]);
    }
  mb = fmaxf(mb, __shfl_xor(mb, 16));
  mb = fmaxf(mb, __shfl_xor(mb, 32));
  // every token masked (the empty half of a short window): an empty partial
  const float mref = mb == -INFINITY ? 0.f : mb;
  float pw[4][4], lb = 0.f;
#pragma unroll
  for (int t = 0; t < NTL; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[t][i] = exp2f(x[t][i] - mref);
      lb += pw[t][i];
    }
  lb += __shfl_xor(lb, 16);
  lb += __shfl_xor(lb, 32);
  m_out = mb;
  l_out = lb;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  block_pv<T, D, NTL>(f, pw, o);
}

template <class T, int D, int NTL, bool STREAM = false>
__device__ __forceinline__ void attend_tiles(const typename T::storage* q_group, int G,
                                             const typename T::storage* blk, int t0, int len,
                                             float scale_log2, int lane, float& m_out,
                                             float& l_out, f32x4 (&o)[D / 16], const float* bias_blk = nullptr) {
  Frags<T, D> f;
  load_tiles<T, D, NTL, STREAM>(f, blk, t0, lane);
  load_q<T, D>(f, q_group, G, lane);
  attend_frags<T, D, NTL>(f, t0, len, scale_log2, lane, m_out, l_out, o, bias_blk);
}

// A whole block (tiles 0..3).
template <class T, int D>
__device__ __forceinline__ void attend_block(const typename T::storage* q_group, int G,
                                             const typename T::storage* blk, int len,
                                             float scale_log2, int lane, float& m_out,
                                             float& l_out, f32x4 (&o)[D / 16], const float* bias_blk = nullptr) {
  attend_tiles<T, D, 4>(q_group, G, blk, 0, len, scale_log2, lane, m_out, l_out, o, bias_blk);
}

template <int D, int WAVES, int GMAX>
struct AttnLds {
  float o[WAVES][GMAX][D + 4];
  float m[WAVES][GMAX];
  float l[WAVES][GMAX];
  float den[GMAX];
};

__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16_bits(v); }
__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }

// Workgroup: merge the WAVES wavefront partials (m_run = -inf for an idle
// wavefront) through LDS.  With a single split the normalised result goes
// to out_g (the G query heads of the KV head); otherwise this split's
// partial (unnormalised sums, max, sum) goes to po / pml with coherent
// stores.
template <class T, int D, int WAVES, int GMAX>
__device__ void merge_waves(AttnLds<D, WAVES, GMAX>& L, float m_run, float l_run,
                            const f32x4 (&o)[D / 16], int G, int tid, int split, int n_split,
                            typename T::storage* out_g, float* po, float* pml) {
  const int lane = tid & 63, wave = tid >> 6, col = lane & 15, grp = lane >> 4;
  constexpr int NT = 64 * WAVES;
  if (col < G) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) L.o[wave][col][16 * dt + 4 * grp + i] = o[dt][i];
    if (grp == 0) {
      L.m[wave][col] = m_run;
      L.l[wave][col] = l_run;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < G * D; idx += NT) {
    const int g = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, L.m[w][g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float wt = (L.m[w][g] == -INFINITY) ? 0.f : exp2f(L.m[w][g] - M);
      num += wt * L.o[w][g][d];
      den += wt * L.l[w][g];
    }
    if (n_split == 1) {
      store_out(&out_g[idx], den > 0.f ? num / den : 0.f);
    } else {
      store_coherent(&po[((size_t)split * G + g) * D + d], num);
      if (d == 0) {
        store_coherent(&pml[((size_t)split * G + g) * 2 + 0], M);
        store_coherent(&pml[((size_t)split * G + g) * 2 + 1], den);
      }
    }
  }
}

// Fold one more unnormalised partial (m_b, l_b, o_b) of the same heads into
// a wavefront's running one (online softmax rescaling).
template <int ND>
__device__ __forceinline__ void combine_partial(float& m_run, float& l_run, f32x4 (&o_run)[ND], float m_b,
                                                float l_b, const f32x4 (&o_b)[ND]) {
  const float M = fmaxf(m_run, m_b);
  if (M == -INFINITY) return;
  const float a = exp2f(m_run - M), b = exp2f(m_b - M);
  l_run = a * l_run + b * l_b;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) o_run[dt][i] = a * o_run[dt][i] + b * o_b[dt][i];
  m_run = M;
}

// ---- merging across the wavefronts and workgroups of one (b, h) unit
// (one-launch step).  A partial is (unnormalised numerators of the G x D
// outputs, per-head max in log2 units, per-head sum).  Thread tid owns the
// outputs tid and tid + NT (head-major), so every flagged store and load
// instruction covers contiguous words; the per-head weights of the pieces
// are computed once, by one lane group per head.

// Maximum over aligned groups of N lanes (N = 8 or 16), every lane of the
// group ends with it.
template <int N>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}

template <int D, int WAVES, int GMAX>
struct MergeLds {
  float o[WAVES][GMAX][D + 4];
  float m[WAVES][GMAX];
  float l[WAVES][GMAX];
  float a[GMAX][16];      // weights of the pieces (wavefronts or records) per head
  float M[GMAX], den[GMAX];
};

// Words of one flagged partial record: GMAX*D numerators (head-major), then
// (max, sum) of each head.
template <int D, int GMAX>
constexpr int part_record_words() { return GMAX * D + 2 * GMAX; }

// Workgroup: the WAVES wavefront partials (m_run = -inf for an idle
// wavefront) -> one partial kept on chip: own[r] = numerator of output
// tid + r * 64 * WAVES, L.M / L.den the heads' max and sum.
template <int D, int WAVES, int GMAX>
__device__ void merge_waves_keep(MergeLds<D, WAVES, GMAX>& L, float m_run, float l_run,
                                 const f32x4 (&o)[D / 16], int G, int tid, float (&own)[2]) {
  static_assert(WAVES == 8, "one 8-lane group per head");
  static_assert(GMAX * D <= 2 * 64 * WAVES, "two outputs per thread");
  const int lane = tid & 63, wave = tid >> 6, col = lane & 15, grp = lane >> 4;
  if (col < G) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<float4*>(&L.o[wave][col][16 * dt + 4 * grp]) =
          make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
    if (grp == 0) {
      L.m[wave][col] = m_run;
      L.l[wave][col] = l_run;
    }
  }
  __syncthreads();
  if (tid < 8 * GMAX) {
    // lane group of 8 = one head, lane = wavefront
    const int g = tid >> 3, w = tid & 7;
    const float mw = g < G ? L.m[w][g] : -INFINITY;
    const float lw = g < G ? L.l[w][g] : 0.f;
    const float M = group_max<8>(mw);
    const float a = mw == -INFINITY ? 0.f : exp2f(mw - M);
    const float den = group_sum<8>(a * lw);
    L.a[g][w] = a;
    if (w == 0) {
      L.M[g] = M;
      L.den[g] = den;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int idx = tid + r * 64 * WAVES, g = idx / D, d = idx % D;
    float n = 0.f;
    if (idx < G * D) {
#pragma unroll
      for (int w = 0; w < WAVES; ++w) n = fmaf(L.a[g][w], L.o[w][g][d], n);
    }
    own[r] = n;
  }
}

// Publish a workgroup's partial (from merge_waves_keep) as flagged words;
// no wait: the merging workgroup polls the words themselves.  A poisoned
// partial carries NaN maxima and sums, which make the merged outputs NaN.
template <int D, int WAVES, int GMAX>
__device__ void publish_part_ll(const MergeLds<D, WAVES, GMAX>& L, int G, int tid, const float (&own)[2],
                                uint64_t* rec, uint32_t flag, bool poison = false) {
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int idx = tid + r * 64 * WAVES;
    if (idx < G * D) ll_store(&rec[idx], own[r], flag);
  }
  if (tid < G) {
    ll_store(&rec[GMAX * D + 2 * tid], poison ? __builtin_nanf("") : L.M[tid], flag);
    ll_store(&rec[GMAX * D + 2 * tid + 1], poison ? __builtin_nanf("") : L.den[tid], flag);
  }
}

// The final merge of a slice of a unit's outputs, by whichever workgroup
// does it (a Q worker, or a merge workgroup): outputs [out_lo, out_lo +
// n_out) (n_out <= 64*WAVES, one per thread) from the unit's n_part flagged records, polled
// until they carry the launch's flag; per-head weights from one 16-lane
// group per head (lane = record); normalised and stored.  Splitting a unit's
// outputs over several such workgroups divides the record bytes each one
// reads.  The first loads of every word go out before get_flag() (which may
// itself wait on memory) is called, so its wait overlaps theirs.  late_flag
// is an LDS word the caller cleared before a barrier that precedes the call.
template <class T, int D, int WAVES, int GMAX, int MAXP, class GetFlag>
__device__ void merge_slice_ll(MergeLds<D, WAVES, GMAX>& L, int G, int tid, int n_part, int out_lo, int n_out,
                               const uint64_t* recs, GetFlag get_flag, int spin_limit, int* err, int* late_flag,
                               typename T::storage* out_g) {
  constexpr int REC = part_record_words<D, GMAX>();
  static_assert(MAXP <= 16, "one 16-lane group per head");
  const int idx = out_lo + tid;
  const bool has = tid < n_out;
  uint64_t w[MAXP];
#pragma unroll
  for (int sp = 0; sp < MAXP; ++sp) w[sp] = (sp < n_part && has) ? ll_load(recs + (size_t)sp * REC + idx) : 0;
  // lanes of the first 16 * GMAX threads also own the (max, sum) words of
  // record sp = tid % 16 for head g = tid / 16
  const int g_ml = tid >> 4, sp_ml = tid & 15;
  const bool has_ml = tid < 16 * GMAX && g_ml < G && sp_ml < n_part;
  const uint64_t* pm = recs + (size_t)sp_ml * REC + GMAX * D + 2 * g_ml;
  uint64_t wm = has_ml ? ll_load(pm) : 0;
  uint64_t wl = has_ml ? ll_load(pm + 1) : 0;
  const uint32_t flag = get_flag();
  bool late = false;   // a wait hit its bound: this workgroup's outputs are NaN
  {
    // one loop for every word this thread waits on, so a record that lands
    // late costs one reload round, not one per word kind
    int it = 0;
    while (true) {
      bool ok = !has_ml || (ll_ok(wm, flag) && ll_ok(wl, flag));
#pragma unroll
      for (int sp = 0; sp < MAXP; ++sp) ok = ok && (!(sp < n_part && has) || ll_ok(w[sp], flag));
      if (ok || it >= spin_limit) {
        if (!ok) {
          atomicAdd(err, 1);
          late = true;
        }
        break;
      }
      __builtin_amdgcn_s_sleep(1);
      if (has_ml && !ll_ok(wm, flag)) wm = ll_load(pm);
      if (has_ml && !ll_ok(wl, flag)) wl = ll_load(pm + 1);
#pragma unroll
      for (int sp = 0; sp < MAXP; ++sp)
        if (sp < n_part && has && !ll_ok(w[sp], flag)) w[sp] = ll_load(recs + (size_t)sp * REC + idx);
      ++it;
    }
  }
  if (tid < 16 * GMAX) {
    const float m = has_ml ? ll_float(wm) : -INFINITY;
    const float l = has_ml ? ll_float(wl) : 0.f;
    const float M = group_max<16>(m);
    const float a = m == -INFINITY ? 0.f : exp2f(m - M);
    const float den = group_sum<16>(a * l);
    // a NaN sum (a poisoned record) keeps the weights NaN
    L.a[g_ml][sp_ml] = (den > 0.f || den != den) ? a / den : 0.f;
  }
  if (late) *late_flag = 1;
  lds_barrier();   // the weights and the flag
  const bool any_late = *late_flag != 0;
  if (has) {
    // every term, with no guard on n_part: a record past n_part has weight 0
    // (the weights above) and payload 0 (w was zeroed), so the 16 weight
    // reads go out together instead of one per branch
    static_assert(MAXP == 16, "the weights above cover 16 records per head");
    const int g = idx / D;
    float n = 0.f;
#pragma unroll
    for (int sp = 0; sp < MAXP; ++sp) n = fmaf(L.a[g][sp], ll_float(w[sp]), n);
    store_out(&out_g[idx], any_late ? __builtin_nanf("") : n);
  }
}

// The last workgroup of a (b, h): merge the n_split partials in one round
// trip (split maxima and sums into LDS, numerators into registers), then
// normalise and store.  Reuses L's merge buffer.
template <class T, int D, int WAVES, int GMAX>
__device__ void merge_splits(AttnLds<D, WAVES, GMAX>& L, int G, int tid, int n_split,
                             const float* po, const float* pml, typename T::storage* out_g) {
  constexpr int NT = 64 * WAVES;
  constexpr int kMaxSplitRegs = 20;
  float* fm = &L.o[0][0][0];
  float* fl = fm + n_split * G;
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
  if (n_split <= 16) {
    // one 16-lane group per head (lane = split): the maxima and sums by DPP,
    // every split's LDS words read at once
    if (tid < 16 * GMAX) {
      const int g = tid >> 4, s = tid & 15;
      const bool on = g < G && s < n_split;
      const float ms = on ? fm[s * G + g] : -INFINITY;
      const float ls = on ? fl[s * G + g] : 0.f;
      const float M = group_max<16>(ms);
      const float wt = ms == -INFINITY ? 0.f : exp2f(ms - M);
      const float den = group_sum<16>(wt * ls);
      if (on) fm[s * G + g] = wt;
      if (g < G && s == 0) L.den[g] = den;
    }
  } else if (tid < G) {
    float M = -INFINITY;
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, fm[s * G + tid]);
    float den = 0.f;
    for (int s = 0; s < n_split; ++s) {
      const float ms = fm[s * G + tid];
      const float wt = (ms == -INFINITY) ? 0.f : exp2f(ms - M);
      fm[s * G + tid] = wt;
      den += wt * fl[s * G + tid];
    }
    L.den[tid] = den;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int idx = tid + r * NT;
    if (idx >= G * D) break;
    const int g = idx / D, d = idx % D;
    float num = 0.f;
    if (in_regs) {
      // every term, unguarded (reads in bounds; a term past n_split adds 0),
      // so the weight reads go out together instead of one per branch
      const int s_last = n_split > 0 ? n_split - 1 : 0;
#pragma unroll
      for (int s = 0; s < kMaxSplitRegs; ++s) {
        const float wt = fm[min(s, s_last) * G + g];
        num += (s < n_split ? wt : 0.f) * v[r][s];
      }
    } else {
      for (int s = 0; s < n_split; ++s)
        num += fm[s * G + g] * load_coherent(&po[((size_t)s * G + g) * D + d]);
    }
    const float den = L.den[g];
    store_out(&out_g[idx], den > 0.f ? num / den : 0.f);
  }
}

}  // namespace nosa
