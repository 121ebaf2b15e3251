// The fixed device scratch of the allocation-free entry points: one
// file-scope array that every GPU the library runs on holds for the life of
// the process (kStaticScratchBytes each), used in place of a caller's
// workspace.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address is looked
// up once per device with hipGetSymbolAddress and kept here.
#include <mutex>

#include "kernels.h"

namespace csa {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  void* ptr = nullptr;  // the array's device address on this device
  bool dirty = true;    // zero all of it before the next use
  int64_t rows = -1;    // sizes of the previous call
  int64_t n_cap = -1;
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

}  // namespace

int static_scratch(hipStream_t s, int64_t rows, int64_t n_cap, size_t zero_bytes, void** out) {
  *out = nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch& d = g_dev[dev];
  if (d.ptr == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return -1;
    d.ptr = p;
    d.dirty = true;
  }
  // fill kernels, not memsets, so the call stays capturable
  if (d.dirty) {
    if (launch_clear(d.ptr, kStaticScratchBytes, s) != 0) return -1;
    d.dirty = false;
  } else if ((rows != d.rows || n_cap != d.n_cap) && zero_bytes > 0) {
    // another layout: the zero-state bytes may hold the last call's data
    if (launch_clear(d.ptr, zero_bytes, s) != 0) return -1;
  }
  d.rows = rows;
  d.n_cap = n_cap;
  *out = d.ptr;
  return 0;
}

void static_scratch_mark_dirty() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return;
  std::lock_guard<std::mutex> lock(g_mu);
  g_dev[dev].dirty = true;
}

}  // namespace csa
