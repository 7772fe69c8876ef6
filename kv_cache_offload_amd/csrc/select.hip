// Block selection for NOSA decode: query-aware top-kq U query-agnostic top-ke.
//
// Eq. 7 of NOSA (montaan summary, "Key Design Components" item 4) picks up to
// k blocks: kq by the query's block scores, ke by the eviction-head scores.
// Both rank pre-exponential scores (ED-DMA, gist.science summary), so no exp
// or softmax appears here.  The block score is the max over the block's four
// sub-block scores qsum . kbar (two-stage pooling, same summary).
//
// One launch per step.  Grid = (scan splits, query rows x KV heads):
//  * every workgroup scans 128 compressed-key rows of one (row, KV head):
//    groups of D*esize/16 lanes read one 16-byte chunk each of a row, so a
//    wavefront load is 1 KiB of contiguous rows; partial dot products are
//    reduced with cross-lane shuffles and the sub-block scores are written to
//    the workspace;
//  * the last workgroup to finish (atomic ticket) max-pools the scores to
//    blocks, runs two radix selections at once (one per budget, one half of
//    the workgroup each), merges the two sets in LDS and writes them in
//    ascending order.  It also resets the ticket for the next call.
#include "nosa_common.h"
#include "nosa_launch.h"

namespace nosa {

constexpr int kSelThreads = 256;
constexpr int kRowsPerWG = 128;  // compressed-key rows (sub-blocks) per scan workgroup

size_t select_ws_bytes(int batch, int n_query, int n_kv_heads, int nb) {
  const size_t rows = (size_t)batch * n_query * n_kv_heads;
  return align256(rows * sizeof(int32_t)) + align256(rows * (size_t)nb * kSubsPerBlock * sizeof(float));
}

size_t select_lds_bytes(int nb) {
  // two key arrays, two flag arrays, two 256-bin histograms, scratch
  return align256((size_t)nb * 4) * 2 + align256((size_t)nb) * 2 + 2 * 256 * 4 + 64 * 4;
}

// Radix selection of the k largest keys among keys[0..n) (ties: lower index
// first); sets flag[i] = 1 for each selected i.  Run by the NT threads
// `tid` of one half-workgroup; both halves call it together so the barriers
// match.  hist: 256 ints; small: 4 ints (both private to the half).
__device__ void radix_topk(const uint32_t* keys, int n, int k, uint8_t* flag, int* hist,
                           int* small, int tid, int NT) {
  const bool active = (k > 0) && (n > 0);
  if (k > n) k = n;
  uint32_t prefix = 0, mask = 0;
  int remaining = k;
  const int lane = tid & 63;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += NT) hist[i] = 0;
    __syncthreads();
    if (active) {
      for (int i = tid; i < n; i += NT) {
        const uint32_t u = keys[i];
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1);
      }
    }
    __syncthreads();
    if (active && tid < 64) {
      // lane owns digits 255-4*lane .. 252-4*lane (descending digit order)
      int c[4], local = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = hist[255 - 4 * lane - j]; local += c[j]; }
      int incl = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      int run = incl - local;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (run < remaining && run + c[j] >= remaining) {
          small[0] = 255 - 4 * lane - j;
          small[1] = run;
        }
        run += c[j];
      }
    }
    __syncthreads();
    if (active) {
      const int d = small[0];
      remaining -= small[1];
      prefix |= (uint32_t)d << shift;
      mask |= 0xFFu << shift;
    }
  }
  // prefix = the k-th largest key; `remaining` of the keys equal to it are taken
  if (active) {
    const int n_eq = hist[prefix & 255u];
    for (int i = tid; i < n; i += NT) {
      const uint32_t u = keys[i];
      if (u > prefix || (u == prefix && n_eq == remaining)) flag[i] = 1;
    }
    if (n_eq > remaining && tid < 64) {
      // ties at the threshold: the lowest indices win, scanned in order
      int left = remaining;
      for (int base = 0; base < n && left > 0; base += 64) {
        const int i = base + lane;
        const bool eq = (i < n) && (keys[i] == prefix);
        const uint64_t m = __ballot(eq);
        const int before = __popcll(m & ((1ull << lane) - 1ull));
        if (eq && before < left) flag[i] = 1;
        left -= __popcll(m);
      }
    }
  }
  __syncthreads();
}

template <class T, int D>
__global__ void __launch_bounds__(kSelThreads) select_kernel(
    const typename T::storage* __restrict__ q, const int32_t* __restrict__ pos,
    const typename T::storage* __restrict__ k_comp, const float* __restrict__ e_blk, int n_query,
    int n_q_heads, int n_kv_heads, int nb, int kq, int ke, int32_t* __restrict__ sel,
    int32_t* __restrict__ n_sel, int32_t* __restrict__ ticket, float* __restrict__ sig) {
  constexpr int EPC = T::kPer16B;
  constexpr int LPR = D / EPC;               // lanes per compressed-key row
  constexpr int RPP = kSelThreads / LPR;     // rows per pass of the workgroup
  constexpr int PASSES = kRowsPerWG / RPP;
  const int G = n_q_heads / n_kv_heads;
  const int row = blockIdx.y;                // (b * n_query + r) * Hkv + h
  const int h = row % n_kv_heads;
  const int br = row / n_kv_heads;           // b * n_query + r
  const int b = br / n_query;
  const int64_t unit = (int64_t)b * n_kv_heads + h;
  const int k_cap = kq + ke;

  const int p = pos[br];
  const int c = (p >= 0 && p < nb * kBlock) ? p / kBlock : 0;
  const int n_rows = c * kSubsPerBlock;
  float* my_sig = sig + (size_t)row * nb * kSubsPerBlock;

  // ---- scan: sub-block scores of this workgroup's rows
  const int tid = threadIdx.x;
  const int ch = tid % LPR;
  const int r0 = blockIdx.x * kRowsPerWG + tid / LPR;
  if ((int)blockIdx.x * kRowsPerWG < n_rows) {
    float qs[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) qs[e] = 0.0f;
    const typename T::storage* qh = q + ((size_t)br * n_q_heads + (size_t)h * G) * D + ch * EPC;
    for (int g = 0; g < G; ++g) {
      float v[EPC];
      unpack16(ld16(qh + (size_t)g * D), v, T{});
#pragma unroll
      for (int e = 0; e < EPC; ++e) qs[e] += v[e];
    }
    const typename T::storage* kc = k_comp + (size_t)unit * nb * kSubsPerBlock * D + ch * EPC;
    uint4 raw[PASSES];
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      const int rr = r0 + i * RPP;
      raw[i] = (rr < n_rows) ? ld16(kc + (size_t)rr * D) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < PASSES; ++i) {
      float v[EPC];
      unpack16(raw[i], v, T{});
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) s = fmaf(qs[e], v[e], s);
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
      const int rr = r0 + i * RPP;
      if (ch == 0 && rr < n_rows) my_sig[rr] = s;
    }
  }

  // ---- ticket: the last workgroup of this row selects
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int t = atomicAdd(&ticket[row], 1);
    s_last = (t == (int)gridDim.x - 1);
    if (s_last) ticket[row] = 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  extern __shared__ __align__(16) unsigned char lds[];
  const size_t keys_bytes = align256((size_t)nb * 4);
  uint32_t* key_q = reinterpret_cast<uint32_t*>(lds);
  uint32_t* key_e = reinterpret_cast<uint32_t*>(lds + keys_bytes);
  uint8_t* flag_q = lds + 2 * keys_bytes;
  uint8_t* flag_e = flag_q + align256((size_t)nb);
  int* hist = reinterpret_cast<int*>(lds + 2 * keys_bytes + 2 * align256((size_t)nb));
  int* small = hist + 2 * 256;

  const float* eb = e_blk + (size_t)unit * nb;
  for (int j = tid; j < c; j += kSelThreads) {
    const float* s4 = my_sig + (size_t)j * kSubsPerBlock;
    float m = s4[0];
#pragma unroll
    for (int i = 1; i < kSubsPerBlock; ++i) m = fmaxf(m, s4[i]);
    key_q[j] = orderable(m);
    key_e[j] = orderable(eb[j]);
    flag_q[j] = 0;
    flag_e[j] = 0;
  }
  __syncthreads();
  const int half = tid / (kSelThreads / 2);
  const int htid = tid % (kSelThreads / 2);
  radix_topk(half ? key_e : key_q, c, half ? ke : kq, half ? flag_e : flag_q, hist + 256 * half,
             small + 2 * half, htid, kSelThreads / 2);

  // ---- union, ascending
  __shared__ int s_wcount[kSelThreads / 64];
  const int lane = tid & 63, wave = tid >> 6;
  int32_t* out = sel + (size_t)row * k_cap;
  int written = 0;
  for (int base = 0; base < c; base += kSelThreads) {
    const int j = base + tid;
    const bool f = (j < c) && (flag_q[j] | flag_e[j]);
    const uint64_t m = __ballot(f);
    if (lane == 0) s_wcount[wave] = __popcll(m);
    __syncthreads();
    int off = written;
    for (int w = 0; w < wave; ++w) off += s_wcount[w];
    if (f) out[off + __popcll(m & ((1ull << lane) - 1ull))] = j;
    int tot = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) tot += s_wcount[w];
    written += tot;
    __syncthreads();
  }
  for (int i = written + tid; i < k_cap; i += kSelThreads) out[i] = -1;
  if (tid == 0) n_sel[row] = written;
}

template <class T, int D>
static void launch(const LaunchSelect& a) {
  const int rows = a.batch * a.n_query * a.n_kv_heads;
  const int n_scan = (a.nb * kSubsPerBlock + kRowsPerWG - 1) / kRowsPerWG;
  char* ws = (char*)a.ws;
  int32_t* ticket = (int32_t*)ws;
  float* sig = (float*)(ws + align256((size_t)rows * sizeof(int32_t)));
  hipLaunchKernelGGL((select_kernel<T, D>), dim3(n_scan, rows), dim3(kSelThreads),
                     select_lds_bytes(a.nb), a.stream, (const typename T::storage*)a.q, a.pos,
                     (const typename T::storage*)a.k_comp, a.e_blk, a.n_query, a.n_q_heads,
                     a.n_kv_heads, a.nb, a.kq, a.ke, a.sel, a.n_sel, ticket, sig);
}

void launch_select(const LaunchSelect& a) {
  if (a.bf16) {
    if (a.head_dim == 128) launch<Bf16, 128>(a); else launch<Bf16, 64>(a);
  } else {
    if (a.head_dim == 128) launch<F32, 128>(a); else launch<F32, 64>(a);
  }
}

}  // namespace nosa
