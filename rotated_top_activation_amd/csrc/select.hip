// Top-K selection, stage 2 of the method (LaRoSA summary page, 方法详解 ·
// 技术框架: keep the K largest-magnitude entries of the rotated activation,
// zero the rest; the abstract's fixed K gives consistent sparsity).
//
// One 1024-thread workgroup per token. Thread t owns the E = ceil(d/1024)
// consecutive channels [t·E, t·E + E) and keeps their values and keys in
// registers. The key of a channel is its fp32 bit pattern with the sign bit
// cleared, which orders like |x|. An exact radix select over the 31 key bits
// (digits of 11, 11 and 9 bits, LDS histograms) finds the K-th largest key
// T and how many channels equal to T are still to be taken; those go to the
// lowest indices. One packed block scan of (count > T, count == T) per thread
// then gives every kept channel its position, so the output indices come out
// ascending without a sort.
//
// Row union for B > 1: each token also writes a d-bit mask of its kept
// channels; a single workgroup ORs the B masks word by word and compacts the
// set bits in index order, and a grid kernel gathers each token's
// coefficient for every union row.
#include "common.hpp"
#include "launch.hpp"

namespace larosa {
namespace {

constexpr int kThreads = 1024;
constexpr int kNumWaves = kThreads / kWave;
constexpr int kBins = 2048;

// Inclusive scan over the 1024 threads of the workgroup (thread order).
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t *wave_tot) {
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  uint32_t x = wave_incl_scan(v, lane);
  if (lane == kWave - 1) wave_tot[w] = x;
  __syncthreads();
  uint32_t off = 0;
  for (int i = 0; i < w; ++i) off += wave_tot[i];
  __syncthreads();  // wave_tot may be rewritten by the next scan
  return x + off;
}

template <int EMAX>
__global__ __launch_bounds__(kThreads) void topk_select_kernel(
    const float *__restrict__ x_rot, int d, int k, int E, int32_t *__restrict__ idx,
    float *__restrict__ val, float *__restrict__ xs, uint32_t *__restrict__ mask) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t wave_tot[kNumWaves];
  __shared__ uint32_t bitmap[kThreads];  // up to 32768 channels
  __shared__ uint32_t s_bin, s_above;

  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const float *xr = x_rot + static_cast<int64_t>(b) * d;
  const int i0 = t * E;

  float v[EMAX];
  uint32_t key[EMAX];  // bit 31 set marks "no channel here"
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const int i = i0 + e;
    if (e < E && i < d) {
      v[e] = xr[i];
      key[e] = __float_as_uint(v[e]) & 0x7FFFFFFFu;
    } else {
      v[e] = 0.f;
      key[e] = 0x80000000u;
    }
  }
  if (mask) bitmap[t] = 0u;

  // Radix select: after the three passes, prefix == T and krem is the number
  // of channels with key == T that still belong to the top K.
  uint32_t prefix = 0u, pmask = 0x80000000u;
  uint32_t krem = static_cast<uint32_t>(k);
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 9 : 0);
    const uint32_t dmask = pass == 2 ? 0x1FFu : 0x7FFu;
    hist[t] = 0u;
    hist[t + kThreads] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if ((key[e] & pmask) == prefix) atomicAdd(&hist[(key[e] >> shift) & dmask], 1u);
    __syncthreads();
    // Thread t looks at the bin pair q = 1023 − t, so thread order runs from
    // the highest bins down and the inclusive scan counts keys at or above.
    const int q = kThreads - 1 - t;
    const uint32_t h_hi = hist[2 * q + 1], h_lo = hist[2 * q];
    const uint32_t pair = h_hi + h_lo;
    const uint32_t incl = block_incl_scan(pair, wave_tot);
    const uint32_t above = incl - pair;  // keys in bins above 2q+1
    if (above < krem && above + h_hi >= krem) {
      s_bin = 2 * q + 1;
      s_above = above;
    } else if (above + h_hi < krem && incl >= krem) {
      s_bin = 2 * q;
      s_above = above + h_hi;
    }
    __syncthreads();
    prefix |= s_bin << shift;
    pmask |= dmask << shift;
    krem -= s_above;
    __syncthreads();  // s_bin / s_above are rewritten by the next pass
  }
  const uint32_t T = prefix;

  // Positions: kept = key > T, plus the first krem channels with key == T.
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    if (key[e] & 0x80000000u) continue;
    gt += key[e] > T;
    eq += key[e] == T;
  }
  const uint32_t packed = (gt << 16) | eq;  // each count <= 32768
  const uint32_t excl = block_incl_scan(packed, wave_tot) - packed;
  uint32_t g = excl >> 16, qe = excl & 0xFFFFu;
  int32_t *idx_b = idx + static_cast<int64_t>(b) * k;
  float *val_b = val + static_cast<int64_t>(b) * k;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    if (key[e] & 0x80000000u) continue;
    const int i = i0 + e;
    bool kept = false;
    uint32_t pos = 0;
    if (key[e] > T) {
      pos = g + (qe < krem ? qe : krem);
      kept = true;
      ++g;
    } else if (key[e] == T) {
      if (qe < krem) {
        pos = g + qe;
        kept = true;
      }
      ++qe;
    }
    if (kept) {
      idx_b[pos] = i;
      val_b[pos] = v[e];
      if (mask) atomicOr(&bitmap[i >> 5], 1u << (i & 31));
    }
    if (xs) xs[static_cast<int64_t>(b) * d + i] = kept ? v[e] : 0.f;
  }
  if (mask) {
    __syncthreads();
    const int nw = (d + 31) / 32;
    if (t < nw) mask[static_cast<int64_t>(b) * nw + t] = bitmap[t];
  }
}

// Union of the B masks: one workgroup, one mask word per thread (d <= 32768).
__global__ __launch_bounds__(kThreads) void union_list_kernel(
    const uint32_t *__restrict__ mask, int B, int d, int32_t *__restrict__ u_idx,
    int32_t *__restrict__ u_count) {
  __shared__ uint32_t wave_tot[kNumWaves];
  const int t = threadIdx.x;
  const int nw = (d + 31) / 32;
  uint32_t word = 0u;
  if (t < nw)
    for (int b = 0; b < B; ++b) word |= mask[static_cast<int64_t>(b) * nw + t];
  const uint32_t c = __popc(word);
  const uint32_t incl = block_incl_scan(c, wave_tot);
  uint32_t pos = incl - c;
  while (word) {
    const int bit = __ffs(word) - 1;
    u_idx[pos++] = t * 32 + bit;
    word &= word - 1u;
  }
  if (t == kThreads - 1) *u_count = static_cast<int32_t>(incl);
}

// coef[j·B + b] = xs[b, u_idx[j]] for j < |U|; rows past |U| get zeros.
__global__ void union_coef_kernel(const int32_t *__restrict__ u_idx,
                                  const int32_t *__restrict__ u_count,
                                  const float *__restrict__ xs, int B, int d,
                                  float *__restrict__ coef) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= static_cast<int64_t>(d) * B) return;
  const int64_t j = e / B;
  const int b = static_cast<int>(e % B);
  const int n = *u_count;
  coef[e] = j < n ? xs[static_cast<int64_t>(b) * d + u_idx[j]] : 0.f;
}

template <int EMAX>
hipError_t launch_sel(const float *x_rot, int B, int d, int k, int E, int32_t *idx,
                      float *val, float *xs, uint32_t *mask, hipStream_t s) {
  hipLaunchKernelGGL((topk_select_kernel<EMAX>), dim3(B), dim3(kThreads), 0, s, x_rot,
                     d, k, E, idx, val, xs, mask);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const float *x_rot, int B, int d, int k, int32_t *idx,
                         float *val, float *xs, uint32_t *mask, hipStream_t s) {
  const int E = (d + kThreads - 1) / kThreads;
  if (E <= 4) return launch_sel<4>(x_rot, B, d, k, E, idx, val, xs, mask, s);
  if (E <= 8) return launch_sel<8>(x_rot, B, d, k, E, idx, val, xs, mask, s);
  if (E <= 16) return launch_sel<16>(x_rot, B, d, k, E, idx, val, xs, mask, s);
  if (E <= 32) return launch_sel<32>(x_rot, B, d, k, E, idx, val, xs, mask, s);
  return hipErrorInvalidValue;
}

hipError_t launch_union(const uint32_t *mask, const float *xs, int B, int d,
                        int32_t *u_idx, int32_t *u_count, float *u_coef,
                        hipStream_t s) {
  hipLaunchKernelGGL(union_list_kernel, dim3(1), dim3(kThreads), 0, s, mask, B, d,
                     u_idx, u_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = static_cast<int64_t>(d) * B;
  hipLaunchKernelGGL(union_coef_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, s, u_idx, u_count, xs, B, d, u_coef);
  return hipGetLastError();
}

}  // namespace larosa
