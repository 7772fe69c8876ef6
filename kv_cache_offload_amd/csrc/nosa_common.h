// Internal helpers shared by the libnosa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nosa {

constexpr int kBlock = 64;   // tokens per KV block
constexpr int kSub = 16;     // tokens per sub-block of the compressed keys
constexpr int kSubsPerBlock = kBlock / kSub;
constexpr int kWave = 64;

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Element types of the cache.  Storage is raw bits; arithmetic is fp32.
struct Bf16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
  static constexpr int kPer16B = 8;  // elements in one 16-byte load
};
struct F32 {
  using storage = float;
  static constexpr int kBytes = 4;
  static constexpr int kPer16B = 4;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16 bits, round to nearest, ties to even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Unpack one 16-byte chunk into fp32 values.
__device__ __forceinline__ void unpack16(const uint4& v, float (&out)[8], Bf16) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(const uint4& v, float (&out)[4], F32) {
  out[0] = __uint_as_float(v.x);
  out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z);
  out[3] = __uint_as_float(v.w);
}

// Pack fp32 values into one 16-byte chunk of the cache type (bf16: nearest-even).
__device__ __forceinline__ uint4 pack16(const float (&in)[8], Bf16) {
  uint4 r;
  r.x = f32_to_bf16_bits(in[0]) | (f32_to_bf16_bits(in[1]) << 16);
  r.y = f32_to_bf16_bits(in[2]) | (f32_to_bf16_bits(in[3]) << 16);
  r.z = f32_to_bf16_bits(in[4]) | (f32_to_bf16_bits(in[5]) << 16);
  r.w = f32_to_bf16_bits(in[6]) | (f32_to_bf16_bits(in[7]) << 16);
  return r;
}
__device__ __forceinline__ uint4 pack16(const float (&in)[4], F32) {
  return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]),
                    __float_as_uint(in[3]));
}

// Order-preserving map of a finite float onto uint32 (larger float -> larger
// key); -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t orderable(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Hand-off of partial results between workgroups of one launch.  The L2
// caches of the XCDs are not coherent with each other; loads and stores at
// agent scope are (gfx950 issues them with sc1), so a workgroup publishes its
// partials with coherent stores, waits until they have completed, and only
// then bumps the ticket; the workgroup that draws the last ticket reads the
// partials with coherent loads.  This needs no L2 write-back or invalidate.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_stores_done() { __builtin_amdgcn_s_waitcnt(0); }
// Workspace tickets (one per unit or row) sit one per 256-byte line, so the
// atomics of different units do not queue on one line.
constexpr size_t kTicketBytes = 256;
constexpr int kTicketInts = (int)(kTicketBytes / sizeof(int));

__device__ __forceinline__ int ticket_take(int* t) {
  return __hip_atomic_fetch_add(t, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ticket_reset(int* t) {
  __hip_atomic_store(t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Flagged words: a 32-bit payload and a 32-bit launch flag in one 8-byte
// word, written and read with single 8-byte coherent accesses (which are
// never torn).  A consumer polls the words themselves until they carry the
// current launch's flag, so a hand-off costs no store wait, no ticket and
// no separate flag load; nothing has to be reset between launches because
// every launch uses a new flag.
__device__ __forceinline__ void ll_store(uint64_t* p, uint32_t payload, uint32_t flag) {
  __hip_atomic_store(p, ((uint64_t)flag << 32) | payload, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void ll_store(uint64_t* p, float payload, uint32_t flag) {
  ll_store(p, __float_as_uint(payload), flag);
}
__device__ __forceinline__ uint64_t ll_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool ll_ok(uint64_t w, uint32_t flag) { return (uint32_t)(w >> 32) == flag; }
__device__ __forceinline__ float ll_float(uint64_t w) { return __uint_as_float((uint32_t)w); }

// ---------------------------------------------------------------------------
// KV block format: MFMA fragment order.
//
// A block holds 64 tokens.  Its first 64*D elements are the keys, its last
// 64*D the values, each stored as a sequence of 1 KiB fragments: fragment f
// holds, for lane l = 0..63, the 16 bytes lane l feeds to one MFMA of the
// decode attention.  A wavefront therefore loads every fragment with one
// fully contiguous 16-byte-per-lane instruction.
//
// bf16 (v_mfma_f32_16x16x32_bf16, 8 elements per lane):
//   key fragment (t, s), t < 4 tiles, s < D/32:   lane l = 16g + r holds
//     K[tile_token(t, r)][32s + 8g .. +7]
//   value fragment (h, u), h < 2, u < D/16:         lane l = 16g + r holds
//     V[32h + 8g .. +7][16u + r]            (8 tokens of one dimension)
//   tile_token(t, r) = 32(t/2) + 8(r/4) + 4(t%2) + r%4
// fp32 (v_mfma_f32_16x16x4_f32, 4 elements per lane per 4 MFMAs):
//   key fragment (t, s), s < D/16:   lane 16g + r holds K[16t + r][16s + 4g .. +3]
//   value fragment (t, u), u < D/16: lane 16g + r holds V[16t + 4g .. +3][16u + r]
// Fragments are numbered t-major (key: t*(D/32 or D/16) + s; value: h or t major).
// ---------------------------------------------------------------------------
__host__ __device__ constexpr int key_frags_per_tile(int D, bool bf16) { return bf16 ? D / 32 : D / 16; }

// Element offset, inside a block, of the 16-byte chunk holding key dims
// [ch*EPC, ch*EPC + EPC) of token `tok` (EPC = 8 for bf16, 4 for fp32).
template <bool BF16>
__device__ __forceinline__ int key_chunk_offset(int tok, int ch, int D) {
  if constexpr (BF16) {
    const int t = 2 * (tok >> 5) + ((tok >> 2) & 1);
    const int r = 4 * ((tok >> 3) & 3) + (tok & 3);
    const int s = ch >> 2, g = ch & 3;
    return ((t * (D / 32) + s) * 64 + 16 * g + r) * 8;
  } else {
    const int t = tok >> 4, r = tok & 15;
    const int s = ch >> 2, g = ch & 3;
    return ((t * (D / 16) + s) * 64 + 16 * g + r) * 4;
  }
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
// The same load with the non-temporal hint, for data a launch reads once and
// the next launch is unlikely to find cached (the KV blocks of a decode
// step): the lines are not kept in the caches at the expense of others.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Cross-lane moves through DPP (a VALU modifier; no LDS round trip).
// 0xB1 = swap with lane^1, 0x4E = lane^2, 0x141 = mirror inside 8 lanes,
// 0x140 = mirror inside 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// Sum over aligned groups of N lanes (N = 1, 2, 4, 8 or 16): every lane of a
// group ends with the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f32<0xB1>(v);
  if constexpr (N >= 4) v += dpp_f32<0x4E>(v);
  if constexpr (N >= 8) v += dpp_f32<0x141>(v);
  if constexpr (N >= 16) v += dpp_f32<0x140>(v);
  return v;
}
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
// Wavefront-wide inclusive prefix sum (all 64 lanes active): Hillis-Steele
// within rows of 16 lanes (row_shr 1, 2, 4, 8; lanes shifted in from outside
// the row add 0), then the row totals added across rows.
__device__ __forceinline__ int wave_incl_sum(int v, int lane) {
  v += dpp_i32<0x111>(v);
  v += dpp_i32<0x112>(v);
  v += dpp_i32<0x114>(v);
  v += dpp_i32<0x118>(v);
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}
// Wavefront-wide min / max of uint32 (all 64 lanes active; result uniform).
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, (uint32_t)dpp_i32<0xB1>((int)v));
  v = min(v, (uint32_t)dpp_i32<0x4E>((int)v));
  v = min(v, (uint32_t)dpp_i32<0x141>((int)v));
  v = min(v, (uint32_t)dpp_i32<0x140>((int)v));
  return min(min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)dpp_i32<0xB1>((int)v));
  v = max(v, (uint32_t)dpp_i32<0x4E>((int)v));
  v = max(v, (uint32_t)dpp_i32<0x141>((int)v));
  v = max(v, (uint32_t)dpp_i32<0x140>((int)v));
  return max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
             max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}
__device__ __forceinline__ void st16(void* p, const uint4& v) { *reinterpret_cast<uint4*>(p) = v; }

// A workgroup barrier that orders LDS only.  __syncthreads() also releases
// global memory, so every wavefront would first wait for its outstanding
// global stores; nothing that follows these barriers needs that.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace nosa
