// Allocation-free form of the fused attention backward: the same kernels as
// mt_op_attn_bwd_rope, with their scratch (the per-row D = rowsum(dO o) and
// the bf16/fp32 copy of dO) in a file-scope device array instead of a
// caller-supplied workspace, for callers that cannot allocate device memory.
//
// The array is one per GPU (each device that loads the library holds its own
// copy until the process ends). Its device address is taken once per device
// with hipGetSymbolAddress, with that device current; host code never passes
// the array's own name to a kernel (on the host that name is a stand-in, not
// a device address). Every call on a GPU uses that GPU's array: calls that
// overlap on one GPU (different streams, or threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "kernels.h"
#include "runtime.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MT_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up once per device).
int scratch_address(void** out) {
  int dev = -1;
  const hipError_t e0 = hipGetDevice(&dev);
  if (e0 != hipSuccess) return mt::set_error(nullptr, MT_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e0));
  if (dev < 0 || dev >= kMaxDevices) return mt::set_error(nullptr, MT_EHIP, "device index out of range");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return mt::set_error(nullptr, MT_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MT_OK;
}

}  // namespace

extern "C" int mt_op_attn_bwd_rope_noalloc(int32_t dtype, const void* qkv, const float* o, const float* dout,
                                           const float* lse, const float* cos, const float* sin, void* dqkv,
                                           int32_t B, int32_t T, int32_t H, int32_t hkv, int32_t hd,
                                           void* stream) {
  if (B < 0 || T < 0 || H < 1 || hd < 1) return mt::set_error(nullptr, MT_EINVAL, "bad attention shape");
  const int64_t need = mt_op_attn_bwd_ws_bytes(dtype, B, T, H, hd);
  if (need > (int64_t)MT_NOALLOC_SCRATCH_BYTES)
    return mt::set_error(nullptr, MT_EINVAL,
                         "mt_op_attn_bwd_rope_noalloc: B*T*H*hd too large: needs " + std::to_string(need) +
                             " bytes of scratch, the maximum is " + std::to_string((int64_t)MT_NOALLOC_SCRATCH_BYTES));
  if ((int64_t)B * T == 0) return MT_OK;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  return mt_op_attn_bwd_rope(dtype, qkv, o, dout, lse, cos, sin, dqkv, ws, B, T, H, hkv, hd, stream);
}
