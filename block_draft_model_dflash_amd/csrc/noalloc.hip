// dflash_top_k_noalloc: the per-row top-k of dflash_top_k with its chunk lists kept in a fixed
// device array of this library instead of caller-provided scratch, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops).
//
// The array lives in the library's code object: each GPU the library runs on holds its own copy
// until the process ends.  Host code must not use the array's name as a device address (on the
// host it names a stand-in); its device address is asked for once per device, with that device
// current, and kept.  Every call on one GPU shares that GPU's copy, so calls that overlap on one
// GPU (two streams, two host threads) race.  Nothing in it must start at zero: the chunk kernel
// writes every entry of a row's lists before the merge reads them.
#include <mutex>

#include "../../include/dflash.h"
#include "common.h"

using namespace dfl;

namespace {
constexpr size_t NOALLOC_TOPK_BYTES = (size_t)1 << 20;  // 1 MiB: DFLASH_TOPK_NOALLOC_BYTES
constexpr int MAX_DEVICES = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[NOALLOC_TOPK_BYTES];

namespace {

std::mutex g_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// The current device's copy of the array (looked up on its first use on that device).
hipError_t device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

int dflash_top_k_noalloc(const float* x, int32_t rows, int32_t width, int32_t ld, int32_t k, float* vals,
                         int32_t* idx, void* stream) {
  size_t need = 0;
  if (!x || !vals || !idx || ld < width || dflash_top_k_scratch_bytes(rows, width, k, &need) != DFLASH_OK)
    return unit_error(DFLASH_EINVAL, "top_k_noalloc: arguments");
  if (need > NOALLOC_TOPK_BYTES)  // rows * ceil(width/4096) * k past the array's 131072 entries
    return unit_error(DFLASH_EINVAL, "top_k_noalloc: rows * ceil(width/4096) * k exceeds 131072");
  void* base = nullptr;
  hipError_t e = device_scratch(&base);
  if (e != hipSuccess) return unit_error(DFLASH_EHIP, "top_k_noalloc: scratch address", e);
  float* pv = (float*)base;
  int* pi = (int*)((unsigned char*)base + need / 2);
  e = launch_top_k(x, rows, width, ld, k, pv, pi, vals, idx, (hipStream_t)stream);
  return e == hipSuccess ? DFLASH_OK : unit_error(DFLASH_EHIP, "top_k_noalloc", e);
}

}  // extern "C"
