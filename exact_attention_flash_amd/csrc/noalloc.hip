// The key-split forward without a caller workspace: its partial outputs and
// log-sum-exps go to a fixed device array of this library instead, for callers
// that cannot allocate device memory at the call (code under stream capture,
// serving loops that forbid allocation).
//
// The array is a file-scope __device__ variable: every GPU the library runs on
// holds its own copy, allocated when the code object is loaded on that device and
// kept until the process ends. In host code its name is only a stand-in, not a
// device address: the address is looked up once per device with
// hipGetSymbolAddress (with that device current) and that pointer is what the
// kernels receive.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "flash_attn.h"
#include "fwd_kernel.h"

namespace {

static_assert(FA_SPLITKV_SCRATCH_BYTES % 256 == 0, "scratch size must keep 256-byte alignment");

static __device__ __align__(256) float scratch[FA_SPLITKV_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device. Returns a HIP error code (no allocation is made).
hipError_t scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> hold(g_lock);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int flash_attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                              int64_t B, int64_t H, int64_t N, int64_t d, int causal, float scale,
                                              int num_splits, void* stream, int dtype) {
  if (num_splits < 0) return FA_ERR_ARG;
  // the forward's own checks first, so that argument errors take precedence
  int st = flash_attn_fwd_validate(q, k, v, o, lse, B, H, N, d, causal, scale, stream, dtype);
  if (st != FA_OK) return st;
  if (B == 0 || H == 0 || N == 0) return FA_OK;
  int splits = num_splits;
  if (splits == 0) {
    splits = flash_attn_fwd_splitkv_plan(B, H, N, d, causal, fa::device_cus());
    if (splits < 1) return splits < 0 ? splits : FA_ERR_HIP;
  }
  const int64_t need = flash_attn_fwd_splitkv_workspace_size(B, H, N, d, causal, splits);
  if (need < 0) return static_cast<int>(need);
  if (need > static_cast<int64_t>(FA_SPLITKV_SCRATCH_BYTES)) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    if (scratch_for_current_device(&ws) != hipSuccess) return FA_ERR_HIP;
  }
  // every partial row the merge reads is written by the split pass first: nothing
  // needs clearing between calls
  return flash_attn_fwd_splitkv(q, k, v, o, lse, B, H, N, d, causal, scale, splits, ws,
                                need > 0 ? static_cast<uint64_t>(FA_SPLITKV_SCRATCH_BYTES) : 0u, stream, dtype);
}
