// fa_noalloc.hip - fa_backward_noalloc: fa_backward with its workspace (the
// fp32 row dot products D_i = sum_t dO_it O_it) in a static device array of
// this library instead of a buffer the caller allocates.
//
// The array lives in device memory of every GPU the library runs on, for the
// life of the process.  Its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and cached; host code uses
// only that address, never the array's name, which in host code is a host
// stand-in and not a device pointer.
//
// Every call on one GPU shares that GPU's array: calls that overlap on one
// GPU (two streams, or two host threads) race on it and must be serialised by
// the caller.  Nothing in the array needs to start at zero: the first of the
// backward's three launches writes every D_i it later reads.

#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"

// One fp32 per query row of the whole batch: B * H * Nq <= 8,388,608 rows
// (for example 8 sequences x 32 heads x 32,768 rows).
static_assert(FA_NOALLOC_SCRATCH_BYTES % 256 == 0, "whole 256-byte blocks");
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, once looked up

// Device address of the current device's copy of `scratch`.
fa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERROR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERROR_UNSUPPORTED;
  std::lock_guard<std::mutex> guard(g_lock);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return FA_ERROR_LAUNCH;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FA_SUCCESS;
}

}  // namespace

extern "C" fa_status fa_backward_noalloc(fa_dtype dtype, int B, int H, int Nq, int Nk, int d,
                                         const void* q, const void* k, const void* v,
                                         const void* o, const void* dout, const float* lse,
                                         const int32_t* seqlens_k, float scale, int causal,
                                         void* dq, void* dk, void* dv, hipStream_t stream) {
  const size_t need = fa_backward_workspace_size(dtype, B, H, Nq, d);
  if (need > kScratchBytes) return FA_ERROR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (need > 0) {
    const fa_status st = scratch_address(&ws);
    if (st != FA_SUCCESS) return st;
  }
  return fa_backward(dtype, B, H, Nq, Nk, d, q, k, v, o, dout, lse, seqlens_k, scale, causal, dq,
                     dk, dv, ws, need, stream);
}
