// nosa_decode_step_static: the one-launch decode step with a workspace the
// library holds itself, for callers that cannot allocate device memory
// (code under graph capture, tight serving loops, harnesses that forbid
// allocation).
//
// The workspace is a file-scope device array of kStaticStepBytes (16 MiB),
// one copy per device, held until the process ends.  Its device address is
// taken once per device with hipGetSymbolAddress on the first call on that
// device; host code uses only that address (the array's name is a host-side
// stand-in, not a device address).  The array is zero-filled on the first
// call on a device and again whenever a call's geometry (dims, kq, ke)
// differs from the previous call's on that device, so no arrival counter,
// flag or cached Gamma_e of another geometry is ever read.  All calls on one
// device share the array: calls that overlap on one device race.
#include <mutex>

#include "../../include/nosa.h"
#include "nosa_common.h"
#include "nosa_launch.h"

namespace nosa {

static __device__ __align__(256) unsigned char scratch[kStaticStepBytes];

namespace {

constexpr int kMaxDevices = 64;

struct StaticSlot {
  void* ptr = nullptr;     // device address of this device's copy of scratch
  bool have_key = false;
  StepKey key{};           // geometry of the previous call on this device
};

std::mutex g_static_mu;
StaticSlot g_static[kMaxDevices];

__global__ void zero_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

bool same_key(const StepKey& a, const StepKey& b) {
  return a.batch == b.batch && a.n_q_heads == b.n_q_heads && a.n_kv_heads == b.n_kv_heads &&
         a.head_dim == b.head_dim && a.nb == b.nb && a.dtype == b.dtype && a.kq == b.kq && a.ke == b.ke;
}

}  // namespace

int static_step_workspace(const StepKey& key, size_t need, hipStream_t stream, void** ws_out, const char** why) {
  *ws_out = nullptr;
  if (need > kStaticStepBytes) {
    *why = "this geometry needs a step workspace larger than the static one (16 MiB)";
    return NOSA_ERR_WORKSPACE;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *why = "hipGetDevice failed or the device index is above 63";
    return NOSA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticSlot& slot = g_static[dev];
  bool first = false;
  if (slot.ptr == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      *why = "hipGetSymbolAddress of the static step workspace failed";
      return NOSA_ERR_HIP;
    }
    slot.ptr = p;
    first = true;
  }
  if (first || !slot.have_key || !same_key(slot.key, key)) {
    // a fill kernel rather than a memset, so the call can be captured in a graph
    const size_t bytes = first ? kStaticStepBytes : align256(need);
    hipLaunchKernelGGL(zero_kernel, dim3(256), dim3(256), 0, stream, static_cast<uint4*>(slot.ptr), bytes / 16);
    slot.key = key;
    slot.have_key = true;
  }
  *ws_out = slot.ptr;
  return NOSA_OK;
}

void* static_step_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_static_mu);
  return g_static[dev].ptr;
}

}  // namespace nosa

extern "C" int nosa_decode_step_static(const nosa_dims* dims, const void* q, const int32_t* pos, const void* k_comp,
                                       const float* e_blk, int32_t kq, int32_t ke, const void* kv, float scale,
                                       int32_t* sel, int32_t* n_sel, void* out, void* stream) {
  static const char* fn = "nosa_decode_step_static";
  nosa::LaunchStep a;
  if (int rc = nosa::prepare_step(fn, dims, q, pos, k_comp, e_blk, kq, ke, kv, scale, sel, n_sel, out, stream, &a))
    return rc;
  const size_t need = nosa::step_ws_bytes(dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                                          dims->max_blocks, kq, ke);
  const nosa::StepKey key{dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                          dims->max_blocks, dims->dtype, kq, ke};
  const char* why = "";
  void* ws = nullptr;
  if (int rc = nosa::static_step_workspace(key, need, a.stream, &ws, &why)) return nosa::report(rc, fn, why);
  a.ws = ws;
  nosa::launch_step(a);
  return nosa::launched(fn);
}
