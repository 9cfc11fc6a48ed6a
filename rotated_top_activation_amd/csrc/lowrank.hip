// Low-rank compensation of the dropped channels (R-Sparse summary page,
// 研究流程与方法 · R-Sparse框架设计: the masked remainder of the input goes
// through a rank-r factorisation A_r·B_r of the weight taken from its SVD,
// and the output is the sparse part plus that low-rank part):
//
//   y = xs·W' + (x_rot − xs)·A_r·B_r
//
// Two kernels here; the product itself is the ordinary gather. The caller
// stores B_r directly below W' (W_ext = [W'; B_r], d_in + r rows), so the
// low-rank term is r more rows of the same product:
//   1. u[b, :] = (x_rot[b, :] − xs[b, :])·A_r, A_r [d_in, r]: split over at
//      most 128 row ranges walked in 32-row chunks (lane j of a wave owns
//      column j of A_r; a wave's eight rows of a chunk are loaded at once),
//      one partial sum per range. A_r is small (d_in·r elements) and is
//      read in full.
//   2. the row list of the product: the kept rows (or the batch's union)
//      followed by rows d_in .. d_in + r − 1, with coefficients xs and u
//      (each entry of u summed from the partials by one wave, in a fixed
//      tree),
//      written in the packed layout of the vector product or the split,
//      transposed layout of the matrix-core product.
// The gather then accumulates both parts in one fp32 sum per output and
// rounds once.
#include "common.hpp"
#include "launch.hpp"

namespace larosa {
namespace {

constexpr int kLrWaves = 4;
constexpr int kLrRowsPerWave = 8;  // loads in flight per lane
constexpr int kLrChunk = kLrWaves * kLrRowsPerWave;
constexpr int kLrMaxSplits = 128;  // partial sums per coefficient

// Rows per split: whole 32-row chunks, at most kLrMaxSplits splits.
int lr_rows_per_split(int d) {
  const int chunks = (d + kLrChunk - 1) / kLrChunk;
  return (chunks + kLrMaxSplits - 1) / kLrMaxSplits * kLrChunk;
}

template <typename WT, int CPL>
__global__ __launch_bounds__(kLrWaves * kWave) void lowrank_proj_kernel(
    const float *__restrict__ x_rot, const float *__restrict__ xs, const WT *__restrict__ a_r,
    int d, int r, int rps, float *__restrict__ part) {
  __shared__ float red[kLrWaves][CPL * kWave];
  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  const int b = blockIdx.y;
  const int split = blockIdx.x;
  const int s0 = split * rps;
  const int s1 = s0 + rps < d ? s0 + rps : d;
  const float *xr = x_rot + static_cast<int64_t>(b) * d;
  const float *xsb = xs + static_cast<int64_t>(b) * d;
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  for (int i0 = s0; i0 < s1; i0 += kLrChunk) {
    // rows i0 + wave + 4·u: every load of the wave's rows issued before use
    float drop[kLrRowsPerWave], av[kLrRowsPerWave][CPL];
#pragma unroll
    for (int u = 0; u < kLrRowsPerWave; ++u) {
      const int i = i0 + wave + kLrWaves * u;
      const bool ok = i < s1;
      drop[u] = ok ? xr[i] - xsb[i] : 0.f;  // x_rot where dropped, exactly 0 where kept
      const WT *row = a_r + static_cast<int64_t>(ok ? i : s0) * r;
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int j = lane + kWave * c;
        av[u][c] = j < r ? Elt<WT>::load(row, j) : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kLrRowsPerWave; ++u)
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = fmaf(drop[u], av[u][c], acc[c]);
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) red[wave][lane + kWave * c] = acc[c];
  __syncthreads();
  for (int j = threadIdx.x; j < r; j += kLrWaves * kWave) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kLrWaves; ++w) s += red[w][j];
    part[(static_cast<int64_t>(b) * gridDim.x + split) * r + j] = s;
  }
}

// Extended row list and coefficients. Base list: `base` (n_dev ? *n_dev :
// n_host entries). rows_ext[j] = base[j] for j < n, d_in + (j − n) for
// j < n + r; *n_ext = n + r. Coefficient of (j, b): xs[b, rows_ext[j]] for
// j < n, u[b, j − n] for the r low-rank rows, zero for j >= n + r. Written
// packed (coef[j·B + b], j < ld) or split and transposed (store_coef_hl,
// ldc = ld). The first `copy_blocks` workgroups write the kept rows and the
// zeros, one entry per thread; the rest give each of the B·r entries of u a
// wave, whose lanes add the projection's partial sums (at most 128) in a
// fixed tree.
__global__ __launch_bounds__(256) void lowrank_list_kernel(
    const int32_t *__restrict__ base, const int32_t *__restrict__ n_dev, int n_host, int d_in,
    int r, const float *__restrict__ xs, const float *__restrict__ part, int splits, int B,
    int64_t ld, int copy_blocks, int32_t *__restrict__ rows_ext, int32_t *__restrict__ n_ext,
    float *__restrict__ coef, uint16_t *__restrict__ coef_hl) {
  const int n = n_dev ? *n_dev : n_host;
  auto put = [&](int64_t j, int b, float c) {
    if (coef_hl) store_coef_hl(coef_hl, ld, b, j, c);
    else coef[j * B + b] = c;
  };
  if (static_cast<int>(blockIdx.x) >= copy_blocks) {
    const int q = (blockIdx.x - copy_blocks) * 4 + wave_id();  // wave-uniform
    if (q >= B * r) return;
    const int b = q / r, jj = q % r;
    const int lane = threadIdx.x % kWave;
    const float *p = part + static_cast<int64_t>(b) * splits * r + jj;
    float v = lane < splits ? p[static_cast<int64_t>(lane) * r] : 0.f;
    if (lane + kWave < splits) v += p[static_cast<int64_t>(lane + kWave) * r];
    const float u = wave_sum(v);
    if (lane == 0) {
      put(n + jj, b, u);
      if (b == 0) rows_ext[n + jj] = d_in + jj;
    }
    return;
  }
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= ld * B) return;
  const int64_t j = coef_hl ? e % ld : e / B;
  const int b = static_cast<int>(coef_hl ? e / ld : e % B);
  if (e == 0) *n_ext = n + r;
  if (j < n) {
    const int row = base[j];
    if (b == 0) rows_ext[j] = row;
    put(j, b, xs[static_cast<int64_t>(b) * d_in + row]);
  } else if (j >= n + r) {
    put(j, b, 0.f);
  }
}

template <typename WT, int CPL>
hipError_t launch_proj(const float *x_rot, const float *xs, const void *a_r, int B, int d, int r,
                       float *part, hipStream_t s) {
  const int rps = lr_rows_per_split(d);
  const int splits = (d + rps - 1) / rps;
  hipLaunchKernelGGL((lowrank_proj_kernel<WT, CPL>), dim3(splits, B), dim3(kLrWaves * kWave), 0,
                     s, x_rot, xs, static_cast<const WT *>(a_r), d, r, rps, part);
  return hipGetLastError();
}

}  // namespace

size_t lowrank_part_bytes(int64_t B, int64_t d, int64_t r) {
  const int rps = lr_rows_per_split(static_cast<int>(d));
  const int64_t splits = (d + rps - 1) / rps;
  return static_cast<size_t>(B) * splits * r * sizeof(float);
}

hipError_t launch_lowrank_proj(const float *x_rot, const float *xs, const void *a_r, int w_dt,
                               int B, int d, int r, float *part, hipStream_t s) {
  hipError_t e;
  const bool f32 = w_dt == kF32;
  if (r <= 64) e = f32 ? launch_proj<float, 1>(x_rot, xs, a_r, B, d, r, part, s)
                       : launch_proj<uint16_t, 1>(x_rot, xs, a_r, B, d, r, part, s);
  else if (r <= 128) e = f32 ? launch_proj<float, 2>(x_rot, xs, a_r, B, d, r, part, s)
                             : launch_proj<uint16_t, 2>(x_rot, xs, a_r, B, d, r, part, s);
  else if (r <= 256) e = f32 ? launch_proj<float, 4>(x_rot, xs, a_r, B, d, r, part, s)
                             : launch_proj<uint16_t, 4>(x_rot, xs, a_r, B, d, r, part, s);
  else return hipErrorInvalidValue;
  return e;
}

hipError_t launch_lowrank_list(const int32_t *base, const int32_t *n_dev, int n_host, int d_in,
                               int r, const float *xs, const float *part, int B, int64_t ld,
                               int32_t *rows_ext, int32_t *n_ext, float *coef, void *coef_hl,
                               hipStream_t s) {
  const int64_t n = ld * B;
  const int rps = lr_rows_per_split(d_in);
  const int splits = (d_in + rps - 1) / rps;  // <= 2 per lane of a wave
  const int copy_blocks = static_cast<int>((n + 255) / 256);
  const int sum_blocks = (B * r + 3) / 4;
  hipLaunchKernelGGL(lowrank_list_kernel, dim3(static_cast<unsigned>(copy_blocks + sum_blocks)),
                     dim3(256), 0, s, base, n_dev, n_host, d_in, r, xs, part, splits, B, ld,
                     copy_blocks, rows_ext, n_ext, coef, static_cast<uint16_t *>(coef_hl));
  return hipGetLastError();
}

}  // namespace larosa
