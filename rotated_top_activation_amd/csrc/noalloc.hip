// Device-resident workspace for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array below is the workspace of larosa_layer_forward_noalloc: a
// file-scope device array of fixed size that lives, on every GPU the
// library runs on, until the process ends. Host code never uses the array's
// name as an address (in host code it is only a stand-in): on the first
// call on a device, with that device current, hipGetSymbolAddress gives
// that device's own address of it, which is kept per device and used for
// every kernel argument and fill after that.
//
// The layer kernels expect their counters to be zero before a call of a
// given shape and leave them zero after it; a call of another shape finds
// them elsewhere in the workspace. So the array is zero-filled (with a
// kernel, on the caller's stream) on the first call on a device and
// whenever the call's shape differs from the previous call's on that
// device. Every call on a device shares that device's array: calls that
// overlap on one GPU (two streams, or two host threads) race.
#include "launch.hpp"

#include <mutex>

namespace larosa {
namespace {

constexpr size_t kScratchBytes = size_t{16} << 20;  // 16 MiB per device

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
  void *ptr = nullptr;   // this device's address of `scratch`
  bool have_shape = false;
  ScratchShape shape{};  // shape of the last call on this device
};

constexpr int kMaxDevices = 64;
std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

bool same(const ScratchShape &a, const ScratchShape &b) {
  return a.B == b.B && a.d_in == b.d_in && a.d_out == b.d_out && a.k == b.k &&
         a.mode == b.mode && a.act_dt == b.act_dt && a.w_dt == b.w_dt;
}

}  // namespace

size_t scratch_capacity() { return kScratchBytes; }

hipError_t scratch_acquire(const ScratchShape &shape, size_t need, hipStream_t s, void **out) {
  *out = nullptr;
  if (need > kScratchBytes) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceScratch &d = g_dev[dev];
  if (d.ptr == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    d.ptr = p;
  }
  if (!d.have_shape || !same(d.shape, shape)) {
    e = launch_fill_zero(d.ptr, need, s);
    if (e != hipSuccess) return e;
    d.have_shape = true;
    d.shape = shape;
  }
  *out = d.ptr;
  return hipSuccess;
}

}  // namespace larosa
