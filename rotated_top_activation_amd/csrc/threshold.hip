// Magnitude-threshold selection: the contrast to the method's fixed Top-K.
//
// The R-Sparse summary page (研究流程与方法 · R-Sparse框架设计) masks every
// input channel whose magnitude is below a threshold t(s) set by a sparsity
// budget s; the LaRoSA abstract names this kind of magnitude pruning as the
// source of fluctuating sparsity that its fixed K avoids. Here the same keys
// as the Top-K selection are used (fp32 bits with the sign cleared, which
// order like |x|), and a channel is kept iff key >= key(t). The number kept
// therefore varies per token and is written out.
//
// Calibration: t is the keep-th largest magnitude over n calibration entries
// (several tokens' rotated activations). That is an exact radix select over
// all n keys, too many for one workgroup, so each 11/11/9-bit digit pass is
// a grid-wide histogram (LDS per workgroup, added into one global histogram
// with integer atomics, which makes the result independent of order)
// followed by a one-workgroup pick of the digit.
#include "common.hpp"
#include "launch.hpp"
#include "select_core.hpp"

namespace larosa {
namespace {

constexpr int kThreads = 1024;
constexpr int kCalThreads = 256;
constexpr int kCalMaxGrid = 1024;

// Per-token threshold selection; one workgroup per token, thread t owns E
// consecutive channels. idx/val rows have capacity d; count[b] is written.
template <int EMAX>
__global__ __launch_bounds__(kThreads) void threshold_select_kernel(
    const float *__restrict__ x_rot, int d, int E, uint32_t thr_key, int32_t *__restrict__ idx,
    int32_t *__restrict__ count, float *__restrict__ val, float *__restrict__ xs,
    uint32_t *__restrict__ mask) {
  __shared__ uint32_t wave_tot[kThreads / kWave];
  __shared__ uint32_t bitmap[kThreads];  // up to 32768 channels
  __shared__ __align__(16) uint32_t stage[EMAX * kThreads];  // one output row
  __shared__ uint32_t s_total;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const float *xr = x_rot + static_cast<int64_t>(b) * d;
  const int i0 = t * E;
  float v[EMAX];
  uint32_t key[EMAX];
  load_keys4<EMAX>(xr, d, E, key, v);
  if (mask) bitmap[t] = 0u;
  uint32_t n = 0;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) n += !(key[e] & kNoKey) && key[e] >= thr_key;
  const uint32_t incl = block_incl_scan<kThreads>(n, wave_tot);
  const uint32_t pos = incl - n;
  if (t == kThreads - 1) {
    s_total = incl;
    if (count) count[b] = static_cast<int32_t>(incl);
  }
  bool kept[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    kept[e] = !(key[e] & kNoKey) && key[e] >= thr_key;
    if (kept[e] && mask) atomicOr(&bitmap[(i0 + e) >> 5], 1u << ((i0 + e) & 31));
  }
  // Each output row is laid out in LDS and copied out with consecutive lanes
  // on consecutive words (a thread's slots are E consecutive channels).
  const int64_t row = static_cast<int64_t>(b) * d;
  if (xs) {
#pragma unroll
    for (int q = 0; q < EMAX / 4; ++q)
      if (4 * q < E && i0 + 4 * q < d)  // whole quads: E and d are multiples of 4
        *reinterpret_cast<uint4 *>(&stage[i0 + 4 * q]) = make_uint4(
            kept[4 * q] ? __float_as_uint(v[4 * q]) : 0u, kept[4 * q + 1] ? __float_as_uint(v[4 * q + 1]) : 0u,
            kept[4 * q + 2] ? __float_as_uint(v[4 * q + 2]) : 0u, kept[4 * q + 3] ? __float_as_uint(v[4 * q + 3]) : 0u);
    __syncthreads();
    for (int j = t; j < d; j += kThreads) xs[row + j] = __uint_as_float(stage[j]);
  }
  __syncthreads();  // stage is free; s_total is visible
  const int total = static_cast<int>(s_total);
  {
    uint32_t p = pos;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (kept[e]) stage[p++] = static_cast<uint32_t>(i0 + e);
    __syncthreads();
    for (int j = t; j < total; j += kThreads) idx[row + j] = static_cast<int32_t>(stage[j]);
  }
  if (val) {
    __syncthreads();
    uint32_t p = pos;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (kept[e]) stage[p++] = __float_as_uint(v[e]);
    __syncthreads();
    for (int j = t; j < total; j += kThreads) val[row + j] = __uint_as_float(stage[j]);
  }
  if (mask) {
    __syncthreads();
    const int nw = (d + 31) / 32;
    if (t < nw) mask[static_cast<int64_t>(b) * nw + t] = bitmap[t];
  }
}

// Calibration state in the workspace: {prefix, pmask, krem, unused}, then
// the 2048-bin global histogram.
struct CalState {
  uint32_t prefix, pmask, krem, pad;
};

__global__ void calib_init_kernel(CalState *__restrict__ st, uint32_t *__restrict__ hist,
                                  uint32_t keep) {
  for (int i = threadIdx.x; i < 2048; i += blockDim.x) hist[i] = 0u;
  if (threadIdx.x == 0) *st = CalState{0u, 0u, keep, 0u};
}

__global__ __launch_bounds__(kCalThreads) void calib_hist_kernel(
    const float *__restrict__ x, int64_t n, int pass, const CalState *__restrict__ st,
    uint32_t *__restrict__ hist) {
  __shared__ uint32_t h[2048];
  for (int i = threadIdx.x; i < 2048; i += kCalThreads) h[i] = 0u;
  __syncthreads();
  const uint32_t prefix = st->prefix, pmask = st->pmask;
  const int shift = radix_shift(pass);
  const uint32_t dm = radix_dmask(pass);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCalThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCalThreads + threadIdx.x; i < n;
       i += stride) {
    const uint32_t key = __float_as_uint(x[i]) & 0x7FFFFFFFu;
    if ((key & pmask) == prefix) atomicAdd(&h[(key >> shift) & dm], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2048; i += kCalThreads)
    if (h[i]) atomicAdd(&hist[i], h[i]);
}

// Picks this pass's digit from the global histogram, clears the histogram
// for the next pass, and after the last pass writes t.
__global__ __launch_bounds__(kThreads) void calib_pick_kernel(int pass, CalState *__restrict__ st,
                                                              uint32_t *__restrict__ hist,
                                                              float *__restrict__ t_out) {
  __shared__ SelectSmem<kThreads> sm;
  radix_clear<kThreads>(sm);
  __syncthreads();
  for (int i = threadIdx.x; i < 2048; i += kThreads) {
    sm.hist[pad_bin(i)] = hist[i];
    hist[i] = 0u;
  }
  __syncthreads();
  uint32_t prefix = st->prefix, pmask = st->pmask, krem = st->krem;
  radix_resolve<kThreads>(pass, prefix, pmask, krem, sm);
  if (threadIdx.x == 0) {
    *st = CalState{prefix, pmask, krem, 0u};
    if (pass == 2) *t_out = __uint_as_float(prefix);
  }
}

template <int EMAX>
hipError_t launch_thr(const float *x_rot, int B, int d, int E, uint32_t thr_key, int32_t *idx,
                      int32_t *count, float *val, float *xs, uint32_t *mask, hipStream_t s) {
  hipLaunchKernelGGL((threshold_select_kernel<EMAX>), dim3(B), dim3(kThreads), 0, s, x_rot, d,
                     E, thr_key, idx, count, val, xs, mask);
  return hipGetLastError();
}

}  // namespace

uint32_t threshold_key_of(float t) { return __builtin_bit_cast(uint32_t, t) & 0x7FFFFFFFu; }

hipError_t launch_threshold_select(const float *x_rot, int B, int d, uint32_t thr_key,
                                   int32_t *idx, int32_t *count, float *val, float *xs,
                                   uint32_t *mask, hipStream_t s) {
  const int E = slots_per_thread(d, kThreads);
  if (E <= 4) return launch_thr<4>(x_rot, B, d, E, thr_key, idx, count, val, xs, mask, s);
  if (E <= 8) return launch_thr<8>(x_rot, B, d, E, thr_key, idx, count, val, xs, mask, s);
  if (E <= 16) return launch_thr<16>(x_rot, B, d, E, thr_key, idx, count, val, xs, mask, s);
  if (E <= 32) return launch_thr<32>(x_rot, B, d, E, thr_key, idx, count, val, xs, mask, s);
  return hipErrorInvalidValue;
}

size_t calibrate_ws_bytes() { return sizeof(CalState) + 2048 * sizeof(uint32_t); }

hipError_t launch_calibrate(const float *x, int64_t n, uint32_t keep, float *t_out, void *ws,
                            hipStream_t s) {
  auto *st = static_cast<CalState *>(ws);
  auto *hist = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + sizeof(CalState));
  hipLaunchKernelGGL(calib_init_kernel, dim3(1), dim3(256), 0, s, st, hist, keep);
  hipError_t e = hipGetLastError();
  int64_t blocks = (n + kCalThreads * 16 - 1) / (kCalThreads * 16);
  if (blocks > kCalMaxGrid) blocks = kCalMaxGrid;
  if (blocks < 1) blocks = 1;
  for (int pass = 0; pass < 3 && e == hipSuccess; ++pass) {
    hipLaunchKernelGGL(calib_hist_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kCalThreads),
                       0, s, x, n, pass, st, hist);
    e = hipGetLastError();
    if (e != hipSuccess) break;
    hipLaunchKernelGGL(calib_pick_kernel, dim3(1), dim3(kThreads), 0, s, pass, st, hist, t_out);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace larosa
