// e2f_noalloc.hip -- e2f_attn_forward for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation): its workspace is the library's own static device array
// `scratch`, one copy per GPU, held until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory, so
// its device address is looked up once per device (hipGetSymbolAddress with
// that device current) and only that address is ever handed to kernels.
// Every call on one GPU shares that GPU's array: calls that overlap on one
// GPU (several streams, several threads) race on it.  The forward needs
// nothing in it cleared: step 1 writes every row it reads, the schedule
// kernels clear their own counts, and the validation flag is reset by a
// kernel before use.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/e2f.h"
#include "e2f_internal.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;   // 64 MiB per GPU
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};   // device address of `scratch` per device, once looked up

// The device address of this device's `scratch`, looked up with that device
// current; nullptr (and the HIP error in *err) on failure.
void* scratch_on(int dev, int* err) {
  std::lock_guard<std::mutex> lk(g_mutex);
  if (g_ptr[dev]) return g_ptr[dev];
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) {
    *err = (int)e;
    return nullptr;
  }
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) {
    *err = (int)e;
    return nullptr;
  }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || ptr == nullptr) {
    *err = e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
    return nullptr;
  }
  g_ptr[dev] = ptr;
  return ptr;
}

}  // namespace

extern "C" {

size_t e2f_attn_noalloc_max_bytes(void) { return kScratchBytes; }

int e2f_attn_forward_noalloc(hipStream_t stream, int64_t N, int K, int lmax, int C, int H,
                             int dtype, const float* pos, const void* h, const int32_t* nbr_idx,
                             const uint8_t* nbr_mask, float scale, float env_cutoff,
                             const float* path_w, void* out, void* out_msg, float* lse,
                             uint32_t flags) {
  const size_t need = e2f_attn_workspace_bytes(N, lmax, C, dtype);
  if (need == 0) return dtype != E2F_F32 && dtype != E2F_BF16 ? E2F_ERR_DTYPE : E2F_ERR_SHAPE;
  if (need > kScratchBytes) return E2F_ERR_WORKSPACE;   // above the static array's size
  if (N == 0)   // argument checks only; nothing is launched
    return e2f_attn_forward(stream, N, K, lmax, C, H, dtype, pos, h, nbr_idx, nbr_mask, scale,
                            env_cutoff, path_w, nullptr, 0, out, out_msg, lse, flags);
  if (const int rt = e2f::runtime_status()) return rt;
  int dev = -1;
  const hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e2f::hip_error_status((int)e);
  if (dev < 0 || dev >= kMaxDevices) return e2f::hip_error_status((int)hipErrorInvalidDevice);
  int err = 0;
  void* ws = scratch_on(dev, &err);
  if (!ws) return e2f::hip_error_status(err);
  // the public forward with the static array as its workspace: every argument check of
  // e2f_attn_forward applies, the array is checked against the inputs and outputs for overlap
  return e2f_attn_forward(stream, N, K, lmax, C, H, dtype, pos, h, nbr_idx, nbr_mask, scale,
                          env_cutoff, path_w, ws, kScratchBytes, out, out_msg, lse, flags);
}

}  // extern "C"
