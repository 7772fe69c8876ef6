// One-launch NOSA decode step (resident cache): block selection and sparse
// attention in a single kernel.
//
// NOSA's query-agnostic selection Gamma_e depends only on the block eviction
// scores, which are fixed once a block is complete (gist.science summary,
// "1. Algorithme : NOSA": the eviction head scores KV pairs independently of
// the query; ED-DMA selects on pre-exponential scores).  So the attention over
// Gamma_e and the window -- three quarters of the step's bytes at kq/k = 1/4
// -- does not have to wait for the query-aware scan.  This kernel runs three
// kinds of workgroups at once:
//   R1  compressed-key scan + top-kq (+ top-ke) of one KV head, as in
//       nosa_select_blocks; publishes X = Gamma_q \ Gamma_e and the union;
//   R2  attention over Gamma_e + the window, started immediately (Gamma_e is
//       cached per KV head in the workspace and recomputed when the window
//       moves to a new block);
//   R3  attention over X, started as soon as R1 publishes it.
// The last attention workgroup of a (b, h) merges all partials.
//
// Roles follow the order in which workgroups start (a dynamic id from an
// atomic counter): every R1 workgroup has started before any workgroup that
// waits for one, and R1 waits for nothing, so the R3 spin-waits always end.
// The waits are bounded as well; the last workgroup to finish resets the
// counters and flags for the next launch.
#include "nosa_common.h"
#include "nosa_launch.h"
#include "attn_dev.h"
#include "select_dev.h"

namespace nosa {

constexpr int kStepThreads = 512;
constexpr int kStepWaves = kStepThreads / 64;
constexpr int kStepMaxK = 256;        // kq + ke
constexpr int kSpinLimit = 1 << 22;   // bounded waits (about 0.2 s)

struct StepGeometry {
  int units, S, n2, n3;
  size_t off_ctl, off_sel_ticket, off_attn_ticket, off_xflag, off_xlist, off_ge, off_score, off_ml, off_o, total;
};

static StepGeometry step_geometry(int batch, int n_q_heads, int n_kv_heads, int head_dim, int nb, int kq,
                                  int ke) {
  StepGeometry g{};
  g.units = batch * n_kv_heads;
  const int G = n_q_heads / n_kv_heads;
  g.S = (nb + 127) / 128;
  g.S = g.S < 1 ? 1 : (g.S > 16 ? 16 : g.S);
  g.n2 = (ke + 1 + kStepWaves - 1) / kStepWaves;
  g.n3 = (kq + kStepWaves - 1) / kStepWaves;
  const size_t U = g.units, P = g.n2 + g.n3;
  size_t o = 0;
  g.off_ctl = o; o += 256;
  g.off_sel_ticket = o; o += align256(U * 4);
  g.off_attn_ticket = o; o += align256(U * 4);
  g.off_xflag = o; o += align256(U * 4);
  g.off_xlist = o; o += align256(U * (kq + 1) * 4);
  g.off_ge = o; o += align256(U * (ke + 2) * 4);
  g.off_score = o; o += align256(U * (size_t)nb * 4);
  g.off_ml = o; o += align256(U * P * G * 2 * 4);
  g.off_o = o; o += align256(U * P * G * (size_t)head_dim * 4);
  g.total = o;
  return g;
}

size_t step_ws_bytes(int batch, int n_q_heads, int n_kv_heads, int head_dim, int nb, int kq, int ke) {
  return step_geometry(batch, n_q_heads, n_kv_heads, head_dim, nb, kq, ke).total;
}

template <int D>
static size_t step_lds_bytes(int nb) {
  const size_t a = sizeof(AttnLds<D, kStepWaves, 8>);
  const size_t s = select_lds_bytes(nb);
  return a > s ? a : s;
}

__device__ __forceinline__ void store_coherent_i(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_coherent_i(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <class T, int D>
__global__ void __launch_bounds__(kStepThreads) step_kernel(
    const typename T::storage* __restrict__ q, const int32_t* __restrict__ pos,
    const typename T::storage* __restrict__ k_comp, const float* __restrict__ e_blk,
    const typename T::storage* __restrict__ kv, int n_q_heads, int n_kv_heads, int nb, int kq,
    int ke, float scale_log2, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
    typename T::storage* __restrict__ out, unsigned char* __restrict__ ws, int S, int n2, int n3,
    size_t off_sel_ticket, size_t off_attn_ticket, size_t off_xflag, size_t off_xlist,
    size_t off_ge, size_t off_score, size_t off_ml, size_t off_o) {
  constexpr int ND = D / 16;
  const int G = n_q_heads / n_kv_heads;
  const int U = gridDim.x / (S + n2 + n3);
  const int total_wgs = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k_cap = kq + ke;
  const size_t blk_elems = (size_t)2 * kBlock * D;

  int* ctl = reinterpret_cast<int*>(ws);                 // [0] start order, [1] finished, [2] wait timeouts
  int* sel_ticket = reinterpret_cast<int*>(ws + off_sel_ticket);
  int* attn_ticket = reinterpret_cast<int*>(ws + off_attn_ticket);
  int* xflag = reinterpret_cast<int*>(ws + off_xflag);
  int* xlist_all = reinterpret_cast<int*>(ws + off_xlist);
  int* ge_all = reinterpret_cast<int*>(ws + off_ge);
  float* score_all = reinterpret_cast<float*>(ws + off_score);
  float* ml_all = reinterpret_cast<float*>(ws + off_ml);
  float* o_all = reinterpret_cast<float*>(ws + off_o);

  extern __shared__ __align__(16) unsigned char lds[];
  __shared__ int s_hist[2][kBins];
  __shared__ int s_small[2][32];
  __shared__ int s_wsum[kStepWaves];
  __shared__ int s_list[kStepMaxK];
  __shared__ int s_misc[4];

  if (tid == 0) s_misc[0] = atomicAdd(&ctl[0], 1);
  __syncthreads();
  const int wid = s_misc[0];
  int role, unit, part;
  if (wid >= total_wgs) {
    // the start-order counter was not reset (an earlier launch did not
    // finish): do nothing rather than touch memory for a role that does not
    // exist; the caller re-zeroes the workspace
    role = 0; unit = 0; part = 0;
    if (tid == 0) atomicAdd(&ctl[2], 1);
  } else if (wid < U * S) {
    role = 1; unit = wid % U; part = wid / U;
  } else if (wid < U * (S + n2)) {
    role = 2; unit = (wid - U * S) % U; part = (wid - U * S) / U;
  } else {
    role = 3; unit = (wid - U * (S + n2)) % U; part = (wid - U * (S + n2)) / U;
  }
  const int b = unit / n_kv_heads, h = unit % n_kv_heads;
  const int p = pos[b];
  const bool valid_pos = (p >= 0 && p < nb * kBlock);
  const int c = valid_pos ? p / kBlock : 0;
  const typename T::storage* q_group = q + ((size_t)b * n_q_heads + (size_t)h * G) * D;
  const float* eb = e_blk + (size_t)unit * nb;
  int* xlist = xlist_all + (size_t)unit * (kq + 1);
  int* ge = ge_all + (size_t)unit * (ke + 2);

  const size_t kb = align256((size_t)nb * 4), lb = align256((size_t)nb * 2);
  uint32_t* key_q = reinterpret_cast<uint32_t*>(lds);
  uint32_t* key_e = reinterpret_cast<uint32_t*>(lds + kb);
  uint16_t* blist_q = reinterpret_cast<uint16_t*>(lds + 2 * kb);
  uint16_t* blist_e = reinterpret_cast<uint16_t*>(lds + 2 * kb + lb);
  uint8_t* flag_q = lds + 2 * kb + 2 * lb;
  uint8_t* flag_e = flag_q + align256((size_t)nb);

  if (role == 1) {
    // ---------------- R1: scan, top-k, union, publish X
    float* my_score = score_all + (size_t)unit * nb;
    const int bps = (nb + S - 1) / S;
    const int blk_lo = min(c, part * bps), blk_hi = min(c, blk_lo + bps);
    if (blk_lo < blk_hi) {
      const typename T::storage* kc = k_comp + (size_t)unit * nb * kSubsPerBlock * D;
      scan_block_scores<T, D, kStepThreads>(q_group, G, kc, kSubsPerBlock * blk_lo, kSubsPerBlock * blk_hi, tid,
                                            [&](int blk, float s) { store_coherent(&my_score[blk], s); });
    }
    wait_stores_done();
    __syncthreads();
    if (tid == 0) {
      const int t = ticket_take(&sel_ticket[unit]);
      s_misc[1] = (t == S - 1);
      if (s_misc[1]) ticket_reset(&sel_ticket[unit]);
    }
    __syncthreads();
    if (s_misc[1]) {
      for (int j = tid; j < c; j += kStepThreads) {
        key_q[j] = orderable(load_coherent(&my_score[j]));
        key_e[j] = orderable(eb[j]);
        flag_q[j] = 0;
        flag_e[j] = 0;
      }
      __syncthreads();
      const int half = tid / (kStepThreads / 2);
      select_top<kStepThreads / 2>(half ? key_e : key_q, c, half ? ke : kq, half ? flag_e : flag_q,
                                   s_hist[half], s_small[half], half ? blist_e : blist_q,
                                   tid % (kStepThreads / 2));
      // X = Gamma_q \ Gamma_e first (ascending): the R3 workgroups wait on it
      const int nx = write_ids<kStepThreads>([&](int j) { return flag_q[j] && !flag_e[j]; }, c, s_list,
                                             kq, s_wsum, tid);
      __syncthreads();
      for (int i = tid; i < nx; i += kStepThreads) store_coherent_i(&xlist[1 + i], s_list[i]);
      if (tid == 0) store_coherent_i(&xlist[0], nx);
      wait_stores_done();
      __syncthreads();
      if (tid == 0) store_coherent_i(&xflag[unit], 1);
      // then the union (the call's selection output) and the Gamma_e cache
      const int total = write_union<kStepThreads>(flag_q, flag_e, c, sel + (size_t)unit * k_cap, k_cap, s_wsum, tid);
      if (tid == 0) n_sel[unit] = total;
      if (tid == 0) s_misc[2] = load_coherent_i(&ge[0]);
      __syncthreads();
      if (s_misc[2] != c) {
        const int nge = write_ids<kStepThreads>([&](int j) { return flag_e[j] != 0; }, c, s_list, ke,
                                                s_wsum, tid);
        __syncthreads();
        for (int i = tid; i < nge; i += kStepThreads) store_coherent_i(&ge[2 + i], s_list[i]);
        if (tid == 0) store_coherent_i(&ge[1], nge);
        wait_stores_done();
        __syncthreads();
        if (tid == 0) store_coherent_i(&ge[0], c);
      }
    }
  } else if (role != 0) {
    // ---------------- R2 / R3: attention partials
    int n_ent = 0, nge = 0;
    if (role == 2) {
      // Gamma_e from the cache, or recomputed here when the window moved
      if (tid == 0) s_misc[2] = load_coherent_i(&ge[0]);
      __syncthreads();
      if (s_misc[2] == c) {
        nge = min(max(load_coherent_i(&ge[1]), 0), min(ke, c));
        for (int i = tid; i < nge; i += kStepThreads) s_list[i] = load_coherent_i(&ge[2 + i]);
      } else {
        for (int j = tid; j < c; j += kStepThreads) {
          key_e[j] = orderable(eb[j]);
          flag_e[j] = 0;
        }
        __syncthreads();
        select_top<kStepThreads>(key_e, c, ke, flag_e, s_hist[0], s_small[0], blist_e, tid);
        nge = write_union<kStepThreads>(flag_e, flag_e, c, s_list, ke, s_wsum, tid);
      }
      __syncthreads();
      n_ent = valid_pos ? nge + 1 : 0;   // Gamma_e, then the window
    } else {
      // wait for R1 to publish X (bounded)
      if (tid == 0) {
        int it = 0;
        while (load_coherent_i(&xflag[unit]) == 0 && it < kSpinLimit) {
          __builtin_amdgcn_s_sleep(2);
          ++it;
        }
        if (it == kSpinLimit) atomicAdd(&ctl[2], 1);
        s_misc[3] = it == kSpinLimit ? 0 : min(max(load_coherent_i(&xlist[0]), 0), kq);
      }
      __syncthreads();
      const int nx = s_misc[3];
      for (int i = tid; i < nx; i += kStepThreads) s_list[i] = load_coherent_i(&xlist[1 + i]);
      __syncthreads();
      n_ent = nx;
    }
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int e = part * kStepWaves + wave;
    if (e < n_ent) {
      const typename T::storage* unit_kv = kv + (size_t)unit * nb * blk_elems;
      int blk, len;
      if (role == 2 && e == nge) {
        blk = c;
        len = p - c * kBlock + 1;
      } else {
        blk = s_list[e];
        len = kBlock;
      }
      if (blk >= 0 && blk < nb)
        attend_block<T, D>(q_group, G, unit_kv + (size_t)blk * blk_elems, len, scale_log2, lane, m_run, l_run, o);
    }
    auto& L = *reinterpret_cast<AttnLds<D, kStepWaves, 8>*>(lds);
    const int n_part = n2 + n3;
    const int my_part = role == 2 ? part : n2 + part;
    float* pml = ml_all + (size_t)unit * n_part * G * 2;
    float* po = o_all + (size_t)unit * n_part * G * D;
    typename T::storage* out_g = out + ((size_t)b * n_q_heads + (size_t)h * G) * D;
    // the unit's merger is its attention workgroup that starts last (R3's
    // last part, else R2's): every other one has started before it, so its
    // bounded wait for their partials ends; it keeps its own partial on chip
    const bool merger = n3 > 0 ? (role == 3 && part == n3 - 1) : (role == 2 && part == n2 - 1);
    if (n_part == 1) {
      merge_waves<T, D, kStepWaves, 8>(L, m_run, l_run, o, G, tid, my_part, n_part, out_g, po, pml);
    } else if (!merger) {
      merge_waves<T, D, kStepWaves, 8>(L, m_run, l_run, o, G, tid, my_part, n_part, out_g, po, pml);
      wait_stores_done();
      __syncthreads();
      if (tid == 0) ticket_take(&attn_ticket[unit]);
    } else {
      __shared__ float s_own_m[8], s_own_l[8];
      float own[(8 * D + kStepThreads - 1) / kStepThreads];
      merge_waves_keep<T, D, kStepWaves, 8>(L, m_run, l_run, o, G, tid, own, s_own_m, s_own_l);
      if (tid == 0) {
        int it = 0;
        while (load_coherent_i(&attn_ticket[unit]) < n_part - 1 && it < kSpinLimit) {
          __builtin_amdgcn_s_sleep(1);
          ++it;
        }
        if (it == kSpinLimit) atomicAdd(&ctl[2], 1);
        ticket_reset(&attn_ticket[unit]);
      }
      __syncthreads();
      merge_splits<T, D, kStepWaves, 8>(L, G, tid, n_part, po, pml, out_g, my_part, own, s_own_m, s_own_l);
    }
  }

  // ---- the last workgroup to finish resets the start order and the flags
  wait_stores_done();
  __syncthreads();
  if (tid == 0) s_misc[0] = atomicAdd(&ctl[1], 1);
  __syncthreads();
  if (s_misc[0] == total_wgs - 1) {
    for (int u = tid; u < U; u += kStepThreads) store_coherent_i(&xflag[u], 0);
    if (tid == 0) {
      store_coherent_i(&ctl[0], 0);
      store_coherent_i(&ctl[1], 0);
    }
  }
}

template <class T, int D>
static void launch(const LaunchStep& a) {
  const StepGeometry g = step_geometry(a.batch, a.n_q_heads, a.n_kv_heads, D, a.nb, a.kq, a.ke);
  const int wgs = g.units * (g.S + g.n2 + g.n3);
  const float scale_log2 = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((step_kernel<T, D>), dim3(wgs), dim3(kStepThreads), step_lds_bytes<D>(a.nb), a.stream,
                     (const typename T::storage*)a.q, a.pos, (const typename T::storage*)a.k_comp,
                     a.e_blk, (const typename T::storage*)a.kv, a.n_q_heads, a.n_kv_heads, a.nb,
                     a.kq, a.ke, scale_log2, a.sel, a.n_sel, (typename T::storage*)a.out,
                     (unsigned char*)a.ws, g.S, g.n2, g.n3, g.off_sel_ticket, g.off_attn_ticket,
                     g.off_xflag, g.off_xlist, g.off_ge, g.off_score, g.off_ml, g.off_o);
}

void launch_step(const LaunchStep& a) {
  if (a.bf16) {
    if (a.head_dim == 128) launch<Bf16, 128>(a); else launch<Bf16, 64>(a);
  } else {
    if (a.head_dim == 128) launch<F32, 128>(a); else launch<F32, 64>(a);
  }
}

}  // namespace nosa
