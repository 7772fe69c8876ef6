// One-launch NOSA decode step (resident cache): block selection and sparse
// attention in a single kernel.
//
// NOSA's query-agnostic selection Gamma_e depends only on the block eviction
// scores, which are fixed once a block is complete (gist.science summary,
// "1. Algorithme : NOSA": the eviction head scores KV pairs independently of
// the query; ED-DMA selects on pre-exponential scores).  So the attention over
// Gamma_e -- three quarters of the step's bytes at kq/k = 1/4 -- does not
// wait for the query-aware scan.  Each (b, KV head) unit gets W + nM
// workgroups:
//   E workers (j < nE)       scan one slice of the unit's compressed keys and
//                            publish the block scores, then attend their
//                            share of Gamma_e (cached per unit in the
//                            workspace, tagged with the window block,
//                            recomputed when the window moves);
//   Q workers (nE <= j < W)  attend the window while the scores arrive, then
//                            each takes top-kq itself (the first one also
//                            writes the union out) and attends its share of
//                            X = Gamma_q \ Gamma_e; then Q worker q combines
//                            all W partials for slice q of the unit's
//                            outputs and stores it;
//   merge workgroups (j >= W) do that final merge instead when the Q workers
//                            are too few for one output per thread (nM = 0
//                            otherwise).
// Work is dealt in 32-token halves of blocks, one per wavefront at a time.
// Every E and Q worker publishes one partial (its wavefronts merged in LDS).
//
// Every hand-off between workgroups goes through flagged 8-byte words
// (payload + launch flag; see nosa_common.h): producers store and move on,
// consumers poll the words.  The flag comes from a per-unit arrival ticket:
// every workgroup of a unit draws one ticket (an atomic add) per launch, the
// launches of one stream draw theirs in order, so ticket / (workgroups per
// unit) is the launch's index whatever the timing -- even a workgroup that
// starts after a merge gave up waiting for it tags its words with its own
// launch's flag.  The workspace never needs resetting between launches.
//
// Workgroup j of unit u has index j * U + u.  Q workers wait on E workers'
// scores and merge workgroups on all the others, workgroups of lower index,
// which the dispatcher has started earlier.  A Q worker's final merge also
// waits on the unit's other Q workers, some of higher index when there are
// two or more, so W >= 3: then the grid stays below 256 + units <= 384
// workgroups (W = ceil(256 / units)), which the MI355X holds all at once (two
// or more of these workgroups fit a CU), and E workers wait on nobody, so
// every wait ends.  The waits are bounded as well: a wait that hits its bound
// is counted in the workspace (nosa_step_timeouts reads the count) and the
// outputs it feeds are written as NaN, never a hang.  Merge workgroups, when
// there are any, come last in the grid, so they occupy CUs only once E
// workers have finished.
#include "nosa_common.h"
#include "nosa_launch.h"
#include "attn_dev.h"
#include "select_dev.h"

namespace nosa {

constexpr int kStepThreads = 512;
constexpr int kStepWaves = kStepThreads / 64;
constexpr int kStepMaxK = 256;        // kq + ke
constexpr int kStepGMax = 8;          // query heads per KV head
constexpr int kSpinLimit = 1 << 18;   // bounded waits: polls of about 1 us, so about 0.3 s
constexpr int kScoreRegs = 8;         // score words polled per thread at once (nb <= 4096)
constexpr int kStepWgsTarget = 256;   // workgroups per launch to aim for: one per CU

struct StepGeometry {
  int units, W, nQ, nE, nM;
  size_t off_arrive, off_err, off_ge, off_score, off_part, total;
};
// Gamma_e cache words per unit: the count, the e_blk address (two words),
// then up to kStepMaxK ids
constexpr int kGeHead = 3;
// Bytes between two units' arrival tickets: one ticket per 256-byte line, so
// the units' atomics do not queue on one line (every workgroup of the launch
// draws one)
constexpr size_t kArriveStride = 256;

static StepGeometry step_geometry(int batch, int n_q_heads, int n_kv_heads, int head_dim, int nb, int kq,
                                  int ke) {
  (void)ke;
  StepGeometry g{};
  g.units = batch * n_kv_heads;
  int W = (kStepWgsTarget + g.units - 1) / g.units;
  W = W < 2 ? 2 : (W > 16 ? 16 : W);
  g.W = W;
  // Q workers: one half block of X per wavefront, at least one E worker left
  int nQ = kq > 0 ? (2 * kq + kStepWaves - 1) / kStepWaves : 0;
  nQ = nQ > W - 1 ? W - 1 : nQ;
  g.nQ = nQ;
  g.nE = W - nQ;
  // the final merge: by the Q workers, one slice of the outputs each, when
  // a slice fits one output per thread; else by merge workgroups of about
  // 256 outputs each, at most 4
  const int GD = (n_q_heads / n_kv_heads) * head_dim;
  if (nQ > 0 && (GD + nQ - 1) / nQ <= kStepThreads)
    g.nM = 0;
  else
    g.nM = GD >= 1024 ? 4 : (GD >= 512 ? 2 : 1);
  const size_t U = g.units;
  const size_t rec = (size_t)kStepGMax * head_dim + 2 * kStepGMax;
  size_t o = 0;
  g.off_arrive = o; o += align256(U * kArriveStride);
  g.off_err = o; o += 256;
  g.off_ge = o; o += align256(U * (kStepMaxK + kGeHead) * 8);
  g.off_score = o; o += align256(U * (size_t)nb * 8);
  g.off_part = o; o += align256(U * (size_t)W * rec * 8);
  g.total = o;
  return g;
}

size_t step_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim, int nb, int kq, int ke) {
  return step_geometry(batch, n_q_heads, n_kv_heads, head_dim, nb, kq, ke).total;
}

size_t step_err_offset(int batch, int n_q_heads, int n_kv_heads, int head_dim, int nb, int kq, int ke) {
  return step_geometry(batch, n_q_heads, n_kv_heads, head_dim, nb, kq, ke).off_err;
}

// Zero, from a vector register the compiler cannot see into.  An atomic on
// an address it can prove uniform is rewritten into one atomic for the
// wavefront plus per-lane offsets, which reads the returned value at once:
// that wait (s_waitcnt vmcnt(0)) also waits for every load the wavefront
// issued before the atomic.  With this offset added to the address the atomic
// keeps its plain form and its result is waited for where it is used.
__device__ __forceinline__ int opaque_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// This launch's flag from one arrival ticket of the unit (thread 0 draws it;
// the caller broadcasts it): launch index + 1, never 0, which is what a word
// nobody has written holds.
__device__ __forceinline__ uint32_t draw_flag(uint64_t* arrive, int wgs_per_unit) {
  const uint64_t t = __hip_atomic_fetch_add(arrive, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (uint32_t)((t / (uint64_t)wgs_per_unit) % 0xFFFFFFFFull) + 1u;
}

template <int D>
static size_t step_lds_bytes(int nb) {
  const size_t a = sizeof(MergeLds<D, kStepWaves, kStepGMax>);
  const size_t s = select_lds_bytes(nb);
  return a > s ? a : s;
}

// Attend half blocks first, first + stride, ... < n_half of the list
// (entry e: half e & 1 of block blk_of(e >> 1), len_of(e >> 1) valid tokens),
// folding them into the wavefront's running partial.  Each half is read by
// one wavefront once per launch, with non-temporal loads: in a decode over
// many layers a block is read again only after the caches have turned over,
// and on cold caches the step runs faster with the hint; a warm repeat of one
// layer's step loses the blocks' cache hits.
template <class T, int D, class BlkOf, class LenOf>
__device__ __forceinline__ void attend_halves(const typename T::storage* q_group, int G,
                                              const typename T::storage* unit_kv, int nb, int first, int stride,
                                              int n_half, BlkOf blk_of, LenOf len_of, float scale_log2, int lane,
                                              float& m_run, float& l_run, f32x4 (&o)[D / 16]) {
  const size_t blk_elems = (size_t)2 * kBlock * D;
  for (int e = first; e < n_half; e += stride) {
    const int blk = blk_of(e >> 1);
    if (blk < 0 || blk >= nb) continue;
    float mb, lb;
    f32x4 ob[D / 16];
    attend_tiles<T, D, 2, true>(q_group, G, unit_kv + (size_t)blk * blk_elems, 2 * (e & 1), len_of(e >> 1),
                          scale_log2, lane, mb, lb, ob);
    combine_partial<D / 16>(m_run, l_run, o, mb, lb, ob);
  }
}

// EXPIRE: the failure-handling test hook (nosa_debug_expire_step_waits): the
// query-aware workers' score waits compare against a flag no launch uses and
// give up after 64 polls, so each expires, is counted and poisons the
// outputs.  A separate instantiation, so the normal kernel carries no trace
// of it.
template <class T, int D, bool EXPIRE>
__global__ void __launch_bounds__(kStepThreads) step_kernel(
    const typename T::storage* __restrict__ q, const int32_t* __restrict__ pos,
    const typename T::storage* __restrict__ k_comp, const float* __restrict__ e_blk,
    const typename T::storage* __restrict__ kv, int n_q_heads, int n_kv_heads, int nb, int kq,
    int ke, float scale_log2, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
    typename T::storage* __restrict__ out, unsigned char* __restrict__ ws, int W, int nQ, int nM,
    size_t off_err, size_t off_ge, size_t off_score, size_t off_part) {
  constexpr uint32_t poll_xor = EXPIRE ? 0x80000000u : 0u;
  constexpr int spin_limit = EXPIRE ? 64 : kSpinLimit;
  constexpr int ND = D / 16;
  constexpr int REC = part_record_words<D, kStepGMax>();
  constexpr int GER = (kStepMaxK + kGeHead + kStepThreads - 1) / kStepThreads;   // cache words per thread
  const int G = n_q_heads / n_kv_heads;
  const int U = gridDim.x / (W + nM);
  const int nE = W - nQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k_cap = kq + ke;

  const int unit = blockIdx.x % U, j = blockIdx.x / U;
  const bool is_q = j >= nE;
  const int b = unit / n_kv_heads, h = unit % n_kv_heads;
  uint64_t* arrive = reinterpret_cast<uint64_t*>(ws + (size_t)unit * kArriveStride);
  int* err = reinterpret_cast<int*>(ws + off_err);
  __shared__ uint32_t s_flag;
  const uint64_t* recs_all = reinterpret_cast<const uint64_t*>(ws + off_part);
  constexpr int REC_ = part_record_words<D, kStepGMax>();

  if (j >= W) {
    // ---------------- merge workgroup m of the unit: a slice of the output
    // from all W records.  Every other workgroup of the unit precedes it in
    // index order.
    extern __shared__ __align__(16) unsigned char lds_m[];
    auto& L = *reinterpret_cast<MergeLds<D, kStepWaves, kStepGMax>*>(lds_m);
    const int m = j - W;
    __shared__ int s_mlate;
    if (tid == 0) {
      s_flag = draw_flag(arrive, W + nM);
      s_mlate = 0;
    }
    __syncthreads();
    const uint32_t flag = s_flag;
    const int GD = G * D, per = (GD + nM - 1) / nM;
    const int lo = min(GD, m * per), n_out = min(per, GD - lo);
    typename T::storage* out_g = out + ((size_t)b * n_q_heads + (size_t)h * G) * D;
    merge_slice_ll<T, D, kStepWaves, kStepGMax, 16>(L, G, tid, W, lo, n_out, recs_all + (size_t)unit * W * REC_,
                                                    [&]() { return flag; }, spin_limit, err, &s_mlate, out_g);
    return;
  }

  uint64_t* score_ll = reinterpret_cast<uint64_t*>(ws + off_score) + (size_t)unit * nb;
  // Gamma_e cache: word 0 = count, words 1, 2 = the e_blk address it was
  // computed from, words 3.. = ids, each tagged with the window block + 1 it
  // was computed for
  uint64_t* ge = reinterpret_cast<uint64_t*>(ws + off_ge) + (size_t)unit * (kStepMaxK + kGeHead);
  const typename T::storage* q_group = q + ((size_t)b * n_q_heads + (size_t)h * G) * D;
  const typename T::storage* unit_kv = kv + (size_t)unit * nb * ((size_t)2 * kBlock * D);
  const float* eb = e_blk + (size_t)unit * nb;

  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int s_hist[kBins];
  __shared__ int s_small[32];
  __shared__ int s_wsum[kStepWaves];
  __shared__ int s_list[kStepMaxK];
  const size_t kb = align256((size_t)nb * 4), lb = align256((size_t)nb * 2);
  uint32_t* key_q = reinterpret_cast<uint32_t*>(lds);
  uint32_t* key_e = reinterpret_cast<uint32_t*>(lds + kb);
  uint16_t* blist = reinterpret_cast<uint16_t*>(lds + 2 * kb);
  uint8_t* flag_q = lds + 2 * kb + 2 * lb;
  uint8_t* flag_e = flag_q + align256((size_t)nb);

  // ---- prologue: the position, the arrival ticket, the Gamma_e cache and
  // (Q workers) the unit's block scores are requested together.  An E worker
  // issues its scan's loads first and these behind them: a wavefront's memory
  // counter is in order, so the wait for the scan's data then never waits
  // for the coherent loads and the ticket, which are used only afterwards.
  int p_raw = 0;
  uint64_t ticket = 0;
  uint64_t gw[GER];
  uint64_t w_sc[kScoreRegs];
  auto prologue = [&]() {
    p_raw = pos[b];
    // (the ticket's result is first needed after the scan)
    if (tid == 0)
      ticket = __hip_atomic_fetch_add(arrive + opaque_zero(), (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int r = 0; r < GER; ++r) {
      const int i = tid + r * kStepThreads;
      gw[r] = i < ke + kGeHead ? ll_load(&ge[i]) : 0;
    }
    if (is_q) {
#pragma unroll
      for (int i = 0; i < kScoreRegs; ++i) {
        const int jj = tid + i * kStepThreads;
        w_sc[i] = jj < nb ? ll_load(&score_ll[jj]) : 0;
      }
    }
  };
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the scan of E worker j covers its slice of all nb blocks (scores of
  // blocks past the window are computed and dropped), so its loads need
  // nothing from the prologue
  const int bps = (nb + nE - 1) / nE;
  const int slice_lo = min(nb, j * bps), slice_hi = min(nb, slice_lo + bps);
  float* s_sc = reinterpret_cast<float*>(lds);
  if (!is_q && kq > 0 && slice_lo < slice_hi) {
    const typename T::storage* kc = k_comp + (size_t)unit * nb * kSubsPerBlock * D;
    auto put = [&](int blk, float sc) { s_sc[blk - slice_lo] = sc; };
    if constexpr (sizeof(typename T::storage) == 2) {
      MfmaScan<D, kStepThreads> scan(q_group, G, kc, kSubsPerBlock * slice_lo, kSubsPerBlock * slice_hi, tid);
      prologue();
      scan.finish(put);
    } else {
      prologue();
      scan_block_scores_fma<T, D, kStepThreads>(q_group, G, kc, kSubsPerBlock * slice_lo, kSubsPerBlock * slice_hi, tid, put);
    }
  } else {
    prologue();
  }
  __shared__ int s_stale;                             // a thread found the Gamma_e cache stale
  __shared__ int s_poison;                            // a score wait of this workgroup expired
  __shared__ int s_late;                              // a record wait of the final merge expired
  if (tid == 0) {
    s_flag = (uint32_t)((ticket / (uint64_t)(W + nM)) % 0xFFFFFFFFull) + 1u;
    s_stale = 0;
    s_poison = 0;
    s_late = 0;
  }

  // ---- now the prologue values
  const bool valid_pos = (p_raw >= 0 && p_raw < nb * kBlock);
  const int c = valid_pos ? p_raw / kBlock : 0;
  const int win_len = valid_pos ? p_raw - c * kBlock + 1 : 0;
  const uint32_t ge_tag = (uint32_t)c + 1u;
  const int ge_cap = min(ke, c);
  const uint64_t eb_addr = (uint64_t)(uintptr_t)e_blk;
  // the cache is current when its count, the e_blk address and every listed
  // id carry this window block's tag
  bool mine = true;
#pragma unroll
  for (int r = 0; r < GER; ++r) {
    const int i = tid + r * kStepThreads;
    if (i >= kGeHead && i < kGeHead + ge_cap) mine = mine && ll_ok(gw[r], ge_tag);
    if (i == 0) mine = mine && ll_ok(gw[r], ge_tag) && (int)(uint32_t)gw[r] == ge_cap;
    if (i == 1) mine = mine && ll_ok(gw[r], ge_tag) && (uint32_t)gw[r] == (uint32_t)eb_addr;
    if (i == 2) mine = mine && ll_ok(gw[r], ge_tag) && (uint32_t)gw[r] == (uint32_t)(eb_addr >> 32);
  }
  if (!is_q && kq > 0) {
    // publish this slice's scores of blocks before the window
    __syncthreads();
    const uint32_t flag = s_flag;
    const int pub_hi = min(slice_hi, c);
    for (int i = tid; i < pub_hi - slice_lo; i += kStepThreads) ll_store(&score_ll[slice_lo + i], s_sc[i], flag);
  } else {
    __syncthreads();                                  // s_stale cleared
  }
  if (!mine) s_stale = 1;
  lds_barrier();                                      // also: s_sc dead
  const bool cache_ok = s_stale == 0;
  // this launch's flag (drawn by thread 0 in the prologue)
  const uint32_t flag = s_flag;

  if (!is_q) {
    // ---------------- E worker: Gamma_e
    int nge;
    if (cache_ok) {
      nge = ge_cap;
#pragma unroll
      for (int r = 0; r < GER; ++r) {
        const int i = tid + r * kStepThreads;
        if (i >= kGeHead && i < kGeHead + ge_cap) s_list[i - kGeHead] = (int)(uint32_t)gw[r];
      }
    } else {
      for (int jj = tid; jj < c; jj += kStepThreads) {
        key_e[jj] = orderable(eb[jj]);
        flag_e[jj] = 0;
      }
      __syncthreads();
      select_top<kStepThreads>(key_e, c, ke, flag_e, s_hist, s_small, blist, tid);
      nge = write_ids<kStepThreads>([&](int jj) { return flag_e[jj] != 0; }, c, s_list, ke, s_wsum, tid);
      if (j == 0) {
        // refresh the cache (every word tagged, so no ordering is needed)
        __syncthreads();
        for (int i = tid; i < nge; i += kStepThreads) ll_store(&ge[kGeHead + i], (uint32_t)s_list[i], ge_tag);
        if (tid == 0) {
          ll_store(&ge[0], (uint32_t)nge, ge_tag);
          ll_store(&ge[1], (uint32_t)eb_addr, ge_tag);
          ll_store(&ge[2], (uint32_t)(eb_addr >> 32), ge_tag);
        }
      }
    }
    __syncthreads();
    if (nQ == 0 && j == 0) {
      // no query-aware budget: the selection output is Gamma_e
      int32_t* su = sel + (size_t)unit * k_cap;
      for (int i = tid; i < k_cap; i += kStepThreads) su[i] = i < nge ? s_list[i] : -1;
      if (tid == 0) n_sel[unit] = nge;
    }
    // Gamma_e halves over the E workers' wavefronts (and the window's two
    // halves when there are no Q workers)
    const int n_half = 2 * nge + (nQ == 0 && valid_pos ? 2 : 0);
    attend_halves<T, D>(q_group, G, unit_kv, nb, j * kStepWaves + wave, nE * kStepWaves, n_half,
                        [&](int i) { return i < nge ? s_list[i] : c; },
                        [&](int i) { return i < nge ? kBlock : win_len; }, scale_log2, lane, m_run, l_run, o);
  } else {
    // ---------------- Q worker
    const int qj = j - nE;
    // Gamma_e membership per candidate (from the cache, or selected here),
    // cleared first behind a barrier: the window's wavefronts reach the
    // later phases well after the others
    for (int jj = tid; jj < c; jj += kStepThreads) {
      flag_e[jj] = 0;
      if (!cache_ok) key_e[jj] = orderable(eb[jj]);
    }
    __syncthreads();
    if (cache_ok) {
#pragma unroll
      for (int r = 0; r < GER; ++r) {
        const int i = tid + r * kStepThreads;
        const int id = (int)(uint32_t)gw[r];
        if (i >= kGeHead && i < kGeHead + ge_cap && id >= 0 && id < c) flag_e[id] = 1;
      }
    } else {
      select_top<kStepThreads>(key_e, c, ke, flag_e, s_hist, s_small, blist, tid);
    }
    // the window's halves first (first Q worker), while the scores arrive
    if (qj == 0 && valid_pos && wave < 2) {
      attend_halves<T, D>(q_group, G, unit_kv, nb, wave, 2, 2, [&](int) { return c; },
                          [&](int) { return win_len; }, scale_log2, lane, m_run, l_run, o);
    }
    uint8_t* bin_q = flag_q;   // per-candidate value bin of the query-aware score
    // the scores (polled together: one reload round per late word, whatever
    // its position) with their range
    {
      int it = 0;
      while (true) {
        bool ok = true;
#pragma unroll
        for (int i = 0; i < kScoreRegs; ++i)
          ok = ok && (tid + i * kStepThreads >= c || ll_ok(w_sc[i], flag ^ poll_xor));
        if (ok || it >= spin_limit) {
          if (!ok) {
            atomicAdd(err, 1);
            s_poison = 1;
          }
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int i = 0; i < kScoreRegs; ++i) {
          const int jj = tid + i * kStepThreads;
          if (jj < c && !ll_ok(w_sc[i], flag ^ poll_xor)) w_sc[i] = ll_load(&score_ll[jj]);
        }
        ++it;
      }
    }
    uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
    for (int i = 0; i < kScoreRegs; ++i) {
      const int jj = tid + i * kStepThreads;
      if (jj < c) {
        const uint32_t k = orderable(ll_float(w_sc[i]));
        key_q[jj] = k;
        kmin = min(kmin, k);
        kmax = max(kmax, k);
      }
    }
    kmin = wave_min_u32(kmin);
    kmax = wave_max_u32(kmax);
    if (lane == 0) {
      s_small[2 * wave] = (int)kmin;
      s_small[2 * wave + 1] = (int)kmax;
    }
    for (int i = tid; i < kBins; i += kStepThreads) s_hist[i] = 0;
    if (tid == 0) s_small[20] = 0;
    __syncthreads();   // keys, ranges, flags
    // Gamma_q = the kq best of c (score desc, id asc): value bins between the
    // scores' min and max (fp64, monotone in the score), the bin holding the
    // kq-th best, and an exact rank inside that bin only
    const bool all_q = kq >= c, none_q = kq <= 0 || c <= 0;
    uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
    for (int w = 0; w < kStepWaves; ++w) {
      lo = min(lo, (uint32_t)s_small[2 * w]);
      hi = max(hi, (uint32_t)s_small[2 * w + 1]);
    }
    const double vlo = key_value(lo), vhi = key_value(hi);
    const double bscale = vhi > vlo ? (double)kBins / (vhi - vlo) : 0.0;
    if (!all_q && !none_q) {
      for (int jj = tid; jj < c; jj += kStepThreads) {
        const int bi = min(kBins - 1, (int)(((double)key_value(key_q[jj]) - vlo) * bscale));
        bin_q[jj] = (uint8_t)bi;
        atomicAdd(&s_hist[bi], 1);
      }
    }
    __syncthreads();
    if (!all_q && !none_q && wave == 0) {
      // lane owns bins 255-4*lane .. 252-4*lane (descending)
      int cnt[4], local = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        cnt[t] = s_hist[kBins - 1 - 4 * lane - t];
        local += cnt[t];
      }
      const int incl = wave_incl_sum(local, lane);
      int run = incl - local;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (run < kq && run + cnt[t] >= kq) {
          s_small[16] = kBins - 1 - 4 * lane - t;   // the bin holding the kq-th best
          s_small[18] = kq - run;                   // how many of that bin to take
        }
        run += cnt[t];
      }
    }
    __syncthreads();
    const int bstar = (all_q || none_q) ? 0 : s_small[16];
    const int take = (all_q || none_q) ? 0 : s_small[18];
    if (!all_q && !none_q)
      for (int jj = tid; jj < c; jj += kStepThreads)
        if (bin_q[jj] == bstar) blist[atomicAdd(&s_small[20], 1)] = (uint16_t)jj;
    __syncthreads();
    const int n_tie = s_small[20];
    auto in_q = [&](int jj) -> bool {
      if (all_q) return true;
      if (none_q) return false;
      const int bi = bin_q[jj];
      if (bi != bstar) return bi > bstar;
      if (n_tie <= take) return true;
      const uint32_t kj = key_q[jj];
      int rank = 0;
      for (int t = 0; t < n_tie; ++t) {
        const int o2 = blist[t];
        const uint32_t ko = key_q[o2];
        rank += (ko > kj) || (ko == kj && o2 < jj);
      }
      return rank < take;
    };
    // X = Gamma_q \ Gamma_e (into LDS) and, from the first Q worker, the union
    // (the call's selection output), both ascending, from one pass over each
    // thread's run of at most kScoreRegs candidates
    int nx;
    {
      const int per = (c + kStepThreads - 1) / kStepThreads;
      const int lo_id = min(c, tid * per), hi_id = min(c, lo_id + per);
      uint32_t mq = 0u, me = 0u;
      for (int jj = lo_id; jj < hi_id; ++jj) {
        if (in_q(jj)) mq |= 1u << (jj - lo_id);
        if (flag_e[jj]) me |= 1u << (jj - lo_id);
      }
      const uint32_t mx = mq & ~me, mu = mq | me;
      const int cx = __builtin_popcount(mx), cu = __builtin_popcount(mu);
      const int ix = wave_incl_sum(cx, lane), iu = wave_incl_sum(cu, lane);
      if (lane == 63) {
        s_wsum[wave] = ix;
        s_small[24 + wave] = iu;
      }
      __syncthreads();
      int ox = ix - cx, ou = iu - cu, tx = 0, tu = 0;
#pragma unroll
      for (int w = 0; w < kStepWaves; ++w) {
        if (w < wave) {
          ox += s_wsum[w];
          ou += s_small[24 + w];
        }
        tx += s_wsum[w];
        tu += s_small[24 + w];
      }
      for (int jj = lo_id; jj < hi_id; ++jj) {
        if (mx & (1u << (jj - lo_id))) s_list[ox++] = jj;
      }
      if (qj == 0) {
        int32_t* su = sel + (size_t)unit * k_cap;
        for (int jj = lo_id; jj < hi_id; ++jj)
          if (mu & (1u << (jj - lo_id))) su[ou++] = jj;
        for (int i = tu + tid; i < k_cap; i += kStepThreads) su[i] = -1;
        if (tid == 0) n_sel[unit] = tu;
      }
      nx = min(tx, kq);
    }
    __syncthreads();
    attend_halves<T, D>(q_group, G, unit_kv, nb, qj * kStepWaves + wave, nQ * kStepWaves, 2 * nx,
                        [&](int i) { return s_list[i]; }, [&](int) { return kBlock; }, scale_log2, lane, m_run,
                        l_run, o);
  }

  // ---------------- the workgroup's partial: wavefronts merged in LDS, published as flagged words
  auto& L = *reinterpret_cast<MergeLds<D, kStepWaves, kStepGMax>*>(lds);
  uint64_t* recs = reinterpret_cast<uint64_t*>(ws + off_part) + (size_t)unit * W * REC;
  float own[2];
  // L reuses the selection arrays' LDS: every read of those came before the
  // last barrier ahead of the attention.  A worker whose score wait timed
  // out poisons its partial, so the unit's outputs come out NaN (the flag
  // was set before several barriers, the merge's own among them).
  merge_waves_keep<D, kStepWaves, kStepGMax>(L, m_run, l_run, o, G, tid, own);
  const bool poison = s_poison != 0;
  publish_part_ll<D, kStepWaves, kStepGMax>(L, G, tid, own, recs + (size_t)j * REC, flag, poison);
  if (nM == 0 && is_q) {
    // ---------------- the final merge: Q worker qj stores slice qj of the
    // unit's outputs from all W records (its own among them)
    const int qj = j - nE;
    const int GD = G * D, per = (GD + nQ - 1) / nQ;
    const int lo = min(GD, qj * per), n_out = min(per, GD - lo);
    lds_barrier();                                    // L's record reads are done
    typename T::storage* out_g = out + ((size_t)b * n_q_heads + (size_t)h * G) * D;
    merge_slice_ll<T, D, kStepWaves, kStepGMax, 16>(L, G, tid, W, lo, n_out, recs, [&]() { return flag; },
                                                    spin_limit, err, &s_late, out_g);
  }
}

template <class T, int D>
static void launch(const LaunchStep& a) {
  const StepGeometry g = step_geometry(a.batch, a.n_q_heads, a.n_kv_heads, D, a.nb, a.kq, a.ke);
  const int wgs = g.units * (g.W + g.nM);
  const float scale_log2 = a.scale * 1.4426950408889634f;
  auto kernel = a.expire_waits ? step_kernel<T, D, true> : step_kernel<T, D, false>;
  hipLaunchKernelGGL(kernel, dim3(wgs), dim3(kStepThreads), step_lds_bytes<D>(a.nb), a.stream,
                     (const typename T::storage*)a.q, a.pos, (const typename T::storage*)a.k_comp,
                     a.e_blk, (const typename T::storage*)a.kv, a.n_q_heads, a.n_kv_heads, a.nb,
                     a.kq, a.ke, scale_log2, a.sel, a.n_sel, (typename T::storage*)a.out,
                     (unsigned char*)a.ws, g.W, g.nQ, g.nM, g.off_err, g.off_ge, g.off_score, g.off_part);
}

void launch_step(const LaunchStep& a) {
  if (a.bf16) {
    if (a.head_dim == 128) launch<Bf16, 128>(a); else launch<Bf16, 64>(a);
  } else {
    if (a.head_dim == 128) launch<F32, 128>(a); else launch<F32, 64>(a);
  }
}

// ---------------------------------------------------------------------------
// The timeout counter of a step workspace, copied out by one thread.
__global__ void copy_counter_kernel(const int* __restrict__ src, int32_t* __restrict__ dst) {
  if (threadIdx.x == 0) *dst = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

void launch_step_timeouts(const void* ws, size_t off_err, int32_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(copy_counter_kernel, dim3(1), dim3(64), 0, stream,
                     reinterpret_cast<const int*>(static_cast<const unsigned char*>(ws) + off_err), out);
}

}  // namespace nosa
