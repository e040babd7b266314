// Allocation-free form of moe_dispatch: the tile plan that moe_dispatch reads
// from the caller's workspace (per-(tile, expert) first rows and per-slot
// ranks) is rebuilt from topk_idx in a static device array instead, so the
// call needs no scratch memory from the caller and allocates none itself.
//
// The array exists once per GPU the library runs on, for the life of the
// process.  In host code its name is only a host-side stand-in, so its
// device address is looked up with hipGetSymbolAddress once per device (with
// that device current) and that address, never the name, is what the
// kernels receive.  Every call on one GPU shares the array: calls that
// overlap on one GPU (different streams, or host threads) race on it.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "moe.h"
#include "moe_launch.h"

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the device `stream` belongs to (the
// current device for the null stream).
hipError_t scratch_address(hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return e;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (dev != cur) {
        const hipError_t r = hipSetDevice(cur);
        if (e == hipSuccess) e = r;
      }
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

hipError_t launch_dispatch_noalloc(const void* x, int xdt, int T, int H,
                                   const int32_t* topk_idx, int k, int E,
                                   int pad, const int32_t* counts,
                                   const int32_t* offsets, int pdt, void* rows,
                                   size_t capacity, float* row_scales,
                                   int32_t* row_src, int32_t* tok_row,
                                   hipStream_t s) {
  void* base = nullptr;
  hipError_t e = scratch_address(s, &base);
  if (e != hipSuccess) return e;
  // plan layout in the array: the workspace's tile bases and ranks, then
  // the plan's own counts and offsets (equal to the caller's when those
  // come from the same topk_idx; the dispatch reads the caller's)
  unsigned char* b = (unsigned char*)base;
  const size_t plan = ws_tile_bytes(T, E) + ws_rank_bytes(T, k);
  int32_t* own_counts = (int32_t*)(b + plan);
  int32_t* own_offsets = (int32_t*)(b + plan + align256((size_t)E * 4));
  e = launch_plan(topk_idx, T, k, E, pad, own_counts, own_offsets, b, s);
  if (e != hipSuccess) return e;
  return launch_dispatch(x, xdt, T, H, topk_idx, k, E, counts, offsets, b,
                         pdt, rows, capacity, row_scales, row_src, tok_row, s);
}

}  // namespace moe
