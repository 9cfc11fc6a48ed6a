// Rotation of the layer input, stage 1 of the method (LaRoSA summary page,
// 方法详解 · 技术框架): x_rot[b, :] = x[b, :]·Q, accumulated in fp32.
//
// The kernel reads the prepared rotation Qt = Qᵀ ([d, q_block], block rows
// transposed), so output channel j is the dot product of x's block segment
// with the contiguous row Qt[j, :]. Each wave owns J consecutive outputs of
// one block and streams their rows with 16-byte loads per lane (1 KB per
// wave per load, J loads in flight per step); the lane sums are folded
// across the wave at the end. No partial sums leave the wave, so the result
// needs no second pass and is the same on every run.
#include "common.hpp"
#include "launch.hpp"

namespace larosa {
namespace {

constexpr int kWavesPerBlock = 4;

// Load V consecutive activations starting at element i as floats.
template <typename XT, int V> struct XLoad;
template <int V> struct XLoad<float, V> {
  __device__ __forceinline__ static void run(const float *x, int64_t i, float *o) {
#pragma unroll
    for (int c = 0; c < V; c += 4) {
      const uint4 q = load16(x + i + c);
      o[c] = __uint_as_float(q.x); o[c + 1] = __uint_as_float(q.y);
      o[c + 2] = __uint_as_float(q.z); o[c + 3] = __uint_as_float(q.w);
    }
  }
};
template <> struct XLoad<uint16_t, 8> {
  __device__ __forceinline__ static void run(const uint16_t *x, int64_t i, float *o) {
    Elt<uint16_t>::unpack(load16(x + i), o);
  }
};
template <> struct XLoad<uint16_t, 4> {
  __device__ __forceinline__ static void run(const uint16_t *x, int64_t i, float *o) {
    const uint2 q = *reinterpret_cast<const uint2 *>(x + i);
    o[0] = bf16_lo(q.x); o[1] = bf16_hi(q.x); o[2] = bf16_lo(q.y); o[3] = bf16_hi(q.y);
  }
};

template <int B, int J, typename XT, typename QT>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void rotate_vec_kernel(
    const XT *__restrict__ x, const QT *__restrict__ qt, float *__restrict__ x_rot,
    int d, int qb) {
  constexpr int V = Elt<QT>::kVec;
  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  const int j0 = (blockIdx.x * kWavesPerBlock + wave) * J;
  if (j0 >= d) return;
  // qb % J == 0 (host-checked), so the J outputs share one block.
  const int64_t xoff = static_cast<int64_t>(j0 / qb) * qb;
  const int chunks = qb / V;

  float acc[J][B];
#pragma unroll
  for (int jj = 0; jj < J; ++jj)
#pragma unroll
    for (int b = 0; b < B; ++b) acc[jj][b] = 0.f;

#pragma unroll 2
  for (int c = lane; c < chunks; c += kWave) {
    uint4 q[J];
#pragma unroll
    for (int jj = 0; jj < J; ++jj)
      q[jj] = load16(qt + static_cast<int64_t>(j0 + jj) * qb + c * V);
    float xf[B][V];
#pragma unroll
    for (int b = 0; b < B; ++b)
      XLoad<XT, V>::run(x, static_cast<int64_t>(b) * d + xoff + c * V, xf[b]);
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      float qf[V];
      Elt<QT>::unpack(q[jj], qf);
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int v = 0; v < V; ++v) acc[jj][b] = fmaf(xf[b][v], qf[v], acc[jj][b]);
    }
  }
#pragma unroll
  for (int jj = 0; jj < J; ++jj)
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const float s = wave_sum(acc[jj][b]);
      if (lane == 0) x_rot[static_cast<int64_t>(b) * d + j0 + jj] = s;
    }
}

// One token, x and Qt of one element type: each wave computes one output
// channel and issues every load of its row (NC 16-byte chunks per lane, the
// matching x chunks alongside) before using any, so a wave's life is about
// one memory round trip plus its share of the transfer.
template <int NC, typename T>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void rotate_row_kernel(
    const T *__restrict__ x, const T *__restrict__ qt, float *__restrict__ x_rot, int d,
    int qb) {
  constexpr int V = Elt<T>::kVec;
  const int lane = threadIdx.x % kWave;
  const int j = blockIdx.x * kWavesPerBlock + wave_id();
  if (j >= d) return;
  const int64_t xoff = static_cast<int64_t>(j / qb) * qb;
  const T *row = qt + static_cast<int64_t>(j) * qb;
  const int chunks = qb / V;
  uint4 xq[NC], q[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + kWave * i;
    const bool ok = c < chunks;
    xq[i] = ok ? load16(x + xoff + c * V) : make_uint4(0, 0, 0, 0);
    q[i] = ok ? load16(row + c * V) : make_uint4(0, 0, 0, 0);
  }
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    float xf[V], qf[V];
    Elt<T>::unpack(xq[i], xf);
    Elt<T>::unpack(q[i], qf);
#pragma unroll
    for (int v = 0; v < V; ++v) acc = fmaf(xf[v], qf[v], acc);
  }
  const float sum = wave_sum(acc);
  if (lane == 0) x_rot[j] = sum;
}

// A few tokens (2 to 8 per group), x and Qt of one element type: one output
// channel per wave, every 16-byte chunk of its Qt row requested at once (NC
// per lane). The workgroup's 8 waves take 8 consecutive channels, which
// share one Q block (q_block is a multiple of 8), so the group's x segments
// of that block are staged once in LDS (NB·q_block elements) while the rows
// are in flight; then each wave reads them from LDS. Qt is read once per group of NB tokens. A token's sum
// runs in the order of the one-token kernel for rows of more than 32 chunks
// (the same lane chunks, the same zero chunks past the row, the same wave
// sum), so there its x_rot does not depend on the batch it came in.
constexpr int kBatchWaves = 8;

template <int NC, int NB, typename T>
__global__ __launch_bounds__(kBatchWaves * kWave) void rotate_rows_batch_kernel(
    const T *__restrict__ x, const T *__restrict__ qt, float *__restrict__ x_rot, int B, int d,
    int qb) {
  constexpr int V = Elt<T>::kVec;
  extern __shared__ __align__(16) unsigned char rot_lds[];
  T *xs = reinterpret_cast<T *>(rot_lds);  // [NB][qb]
  const int t = threadIdx.x;
  const int lane = t % kWave;
  const int j0 = blockIdx.x * kBatchWaves;
  const int j = j0 + wave_id();
  const int b0 = blockIdx.y * NB;
  const int64_t xoff = static_cast<int64_t>(j0 / qb) * qb;
  const int chunks = qb / V;
  uint4 q[NC];
  {
    const T *row = qt + static_cast<int64_t>(j < d ? j : d - 1) * qb;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = lane + kWave * i;
      q[i] = c < chunks ? load16(row + c * V) : make_uint4(0, 0, 0, 0);
    }
  }
  // the group's x segments (tokens past B: the last token's, never stored)
  for (int e = t; e < NB * chunks; e += kBatchWaves * kWave) {
    const int b = e / chunks, c = e % chunks;
    const int bb = b0 + b < B ? b0 + b : B - 1;
    *reinterpret_cast<uint4 *>(xs + b * qb + c * V) =
        load16(x + static_cast<int64_t>(bb) * d + xoff + c * V);
  }
  __syncthreads();
  if (j >= d) return;  // after the only barrier
  float acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + kWave * i;
    const bool ok = c < chunks;
    float qf[V];
    Elt<T>::unpack(q[i], qf);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint4 xq = ok ? *reinterpret_cast<const uint4 *>(xs + b * qb + c * V)
                          : make_uint4(0, 0, 0, 0);
      float xf[V];
      Elt<T>::unpack(xq, xf);
#pragma unroll
      for (int v = 0; v < V; ++v) acc[b] = fmaf(xf[v], qf[v], acc[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const float sum = wave_sum(acc[b]);
    if (lane == 0 && b0 + b < B) x_rot[static_cast<int64_t>(b0 + b) * d + j] = sum;
  }
}

// One token, short rotation blocks (a row of Qt is at most LPR 16-byte
// chunks, LPR <= 32): each wave computes 64 / LPR output channels, LPR lanes
// per channel, so every lane has a chunk to load; the lane groups are summed
// with xor shuffles inside the group (a fixed order).
template <int LPR, typename T>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void rotate_rows_short_kernel(
    const T *__restrict__ x, const T *__restrict__ qt, float *__restrict__ x_rot, int d,
    int qb) {
  constexpr int V = Elt<T>::kVec;
  constexpr int RPW = kWave / LPR;
  const int lane = threadIdx.x % kWave;
  const int j = (blockIdx.x * kWavesPerBlock + wave_id()) * RPW + lane / LPR;
  const int c = lane % LPR;
  const bool ok = j < d && c < qb / V;
  float acc = 0.f;
  if (ok) {
    const int64_t xoff = static_cast<int64_t>(j / qb) * qb;
    float xf[V], qf[V];
    Elt<T>::unpack(load16(x + xoff + c * V), xf);
    Elt<T>::unpack(load16(qt + static_cast<int64_t>(j) * qb + c * V), qf);
#pragma unroll
    for (int v = 0; v < V; ++v) acc = fmaf(xf[v], qf[v], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, kWave);
  if (c == 0 && j < d) x_rot[j] = acc;
}

template <typename T>
bool launch_row(const void *x, const void *qt, float *x_rot, int d, int qb, hipStream_t s) {
  constexpr int V = Elt<T>::kVec;
  const int nc = (qb / V + kWave - 1) / kWave;
  const dim3 grid((d + kWavesPerBlock - 1) / kWavesPerBlock), block(kWavesPerBlock * kWave);
  const auto *xp = static_cast<const T *>(x);
  const auto *qp = static_cast<const T *>(qt);
  const int chunks = qb / V;
  if (chunks <= 32) {
    const int lpr = chunks <= 8 ? 8 : (chunks <= 16 ? 16 : 32);
    const int per_block = kWavesPerBlock * (kWave / lpr);
    const dim3 g((d + per_block - 1) / per_block);
    if (lpr == 8) hipLaunchKernelGGL((rotate_rows_short_kernel<8, T>), g, block, 0, s, xp, qp, x_rot, d, qb);
    else if (lpr == 16) hipLaunchKernelGGL((rotate_rows_short_kernel<16, T>), g, block, 0, s, xp, qp, x_rot, d, qb);
    else hipLaunchKernelGGL((rotate_rows_short_kernel<32, T>), g, block, 0, s, xp, qp, x_rot, d, qb);
    return true;
  }
  if (nc <= 2) hipLaunchKernelGGL((rotate_row_kernel<2, T>), grid, block, 0, s, xp, qp, x_rot, d, qb);
  else if (nc <= 4) hipLaunchKernelGGL((rotate_row_kernel<4, T>), grid, block, 0, s, xp, qp, x_rot, d, qb);
  else if (nc <= 8) hipLaunchKernelGGL((rotate_row_kernel<8, T>), grid, block, 0, s, xp, qp, x_rot, d, qb);
  else if (nc <= 16) hipLaunchKernelGGL((rotate_row_kernel<16, T>), grid, block, 0, s, xp, qp, x_rot, d, qb);
  else return false;
  return true;
}

constexpr size_t kBatchLdsMax = 128 * 1024;  // staged x per workgroup

template <int NC, int NB, typename T>
void launch_batch_k(const T *x, const T *qt, float *x_rot, int B, int d, int qb, hipStream_t s) {
  const dim3 grid((d + kBatchWaves - 1) / kBatchWaves, (B + NB - 1) / NB);
  const size_t lds = static_cast<size_t>(NB) * qb * sizeof(T);
  auto k = rotate_rows_batch_kernel<NC, NB, T>;
  if (lds > 64 * 1024)
    (void)hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  hipLaunchKernelGGL(k, grid, dim3(kBatchWaves * kWave), lds, s, x, qt, x_rot, B, d, qb);
}

template <int NC, typename T>
void launch_batch_nb(const T *x, const T *qt, float *x_rot, int B, int d, int qb, hipStream_t s) {
  // tokens per group: the batch (up to 8), as far as the staged x fits and
  // the row chunks and sums stay in registers (NC·NB <= 32)
  int nb = B <= 2 ? 2 : (B <= 4 ? 4 : 8);
  while (nb > 2 && (static_cast<size_t>(nb) * qb * sizeof(T) > kBatchLdsMax || NC * nb > 32))
    nb /= 2;
  if constexpr (NC * 4 <= 32)
    if (nb == 4) return launch_batch_k<NC, 4, T>(x, qt, x_rot, B, d, qb, s);
  if constexpr (NC * 8 <= 32)
    if (nb == 8) return launch_batch_k<NC, 8, T>(x, qt, x_rot, B, d, qb, s);
  launch_batch_k<NC, 2, T>(x, qt, x_rot, B, d, qb, s);
}

// Tokens in groups of up to 8 (each group reads Qt once); false when the
// form does not apply (a row of more than 512 chunks, a workgroup's 8
// channels spanning two Q blocks, or two tokens' x segments beyond the LDS).
template <typename T>
bool launch_rows_batch(const void *x, const void *qt, float *x_rot, int B, int d, int qb,
                       hipStream_t s) {
  constexpr int V = Elt<T>::kVec;
  const int nc = (qb / V + kWave - 1) / kWave;
  if (qb % kBatchWaves || 2 * static_cast<size_t>(qb) * sizeof(T) > kBatchLdsMax) return false;
  const auto *xp = static_cast<const T *>(x);
  const auto *qp = static_cast<const T *>(qt);
  if (nc <= 2) launch_batch_nb<2, T>(xp, qp, x_rot, B, d, qb, s);
  else if (nc <= 4) launch_batch_nb<4, T>(xp, qp, x_rot, B, d, qb, s);
  else if (nc <= 8) launch_batch_nb<8, T>(xp, qp, x_rot, B, d, qb, s);
  else return false;  // longer rows: the row and two tokens' sums would spill
  return true;
}

template <int B, int J, typename XT, typename QT>
hipError_t launch_t(const void *x, const void *qt, float *x_rot, int d, int qb,
                    hipStream_t s) {
  const int outs_per_block = kWavesPerBlock * J;
  dim3 grid((d + outs_per_block - 1) / outs_per_block);
  hipLaunchKernelGGL((rotate_vec_kernel<B, J, XT, QT>), grid, dim3(kWavesPerBlock * kWave),
                     0, s, static_cast<const XT *>(x), static_cast<const QT *>(qt), x_rot,
                     d, qb);
  return hipGetLastError();
}

template <int B, typename XT, typename QT>
hipError_t launch_j(const void *x, const void *qt, float *x_rot, int d, int qb,
                    hipStream_t s) {
  // Two outputs per wave keeps about eight waves per CU at d = 4096.
  if (qb % 2 == 0) return launch_t<B, 2, XT, QT>(x, qt, x_rot, d, qb, s);
  return launch_t<B, 1, XT, QT>(x, qt, x_rot, d, qb, s);
}

template <int B>
hipError_t launch_b(const void *x, int x_dt, const void *qt, int q_dt, float *x_rot,
                    int d, int qb, hipStream_t s) {
  if (x_dt == kBF16 && q_dt == kBF16) return launch_j<B, uint16_t, uint16_t>(x, qt, x_rot, d, qb, s);
  if (x_dt == kF32 && q_dt == kF32) return launch_j<B, float, float>(x, qt, x_rot, d, qb, s);
  if (x_dt == kF32 && q_dt == kBF16) return launch_j<B, float, uint16_t>(x, qt, x_rot, d, qb, s);
  if (x_dt == kBF16 && q_dt == kF32) return launch_j<B, uint16_t, float>(x, qt, x_rot, d, qb, s);
  return hipErrorInvalidValue;
}

// fp64-accumulating rotation. Each product of two bf16 values, or of two
// fp32 values, is exact in fp64, and the fp64 sum carries a relative error
// near 2^-53·√qb, so rounding it once to fp32 gives the correctly rounded
// x·Q except when that product lies within the fp64 error of an fp32
// rounding midpoint. Index sets taken from this x_rot therefore agree with
// the ones taken from the exact product, not just up to legitimate fp32
// summation-order ties at the K boundary (the method's Top-K, stage 2).
// One wave per output channel and up to NB tokens. For one token this reads
// Qt at about the fp32 form's rate; with more tokens the per-element fp64
// conversions and FMAs (full rate on CDNA4, 16 lanes per clock per SIMD)
// become the bound.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

template <int NC, int NB, typename XT, typename QT>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void rotate_f64_kernel(
    const XT *__restrict__ x, const QT *__restrict__ qt, float *__restrict__ x_rot, int B,
    int d, int qb) {
  constexpr int V = Elt<QT>::kVec;
  const int lane = threadIdx.x % kWave;
  const int j = blockIdx.x * kWavesPerBlock + wave_id();
  if (j >= d) return;
  const int b0 = blockIdx.y * NB;
  const int64_t xoff = static_cast<int64_t>(j / qb) * qb;
  const QT *row = qt + static_cast<int64_t>(j) * qb;
  const int chunks = qb / V;
  const XT *xrow[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int bb = b0 + b < B ? b0 + b : B - 1;  // tokens past B: loaded, not stored
    xrow[b] = x + static_cast<int64_t>(bb) * d + xoff;
  }
  double acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.0;
  // NC·64 chunks of the Qt row in flight at once (the whole row up to
  // q_block = 8192 in bf16); x (shared by every wave of the block, so
  // cache-resident) is read per chunk, one load per token
  for (int seg = 0; seg < chunks; seg += NC * kWave) {
    uint4 q[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = seg + lane + kWave * i;
      q[i] = c < chunks ? load16(row + c * V) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = seg + lane + kWave * i;
      if (c >= chunks) break;
      float qf[V];
      Elt<QT>::unpack(q[i], qf);
      double qd[V];
#pragma unroll
      for (int v = 0; v < V; ++v) qd[v] = static_cast<double>(qf[v]);
      float xf[NB][V];
#pragma unroll
      for (int b = 0; b < NB; ++b) XLoad<XT, V>::run(xrow[b], static_cast<int64_t>(c) * V, xf[b]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int v = 0; v < V; ++v) acc[b] = fma(static_cast<double>(xf[b][v]), qd[v], acc[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const double s = wave_sum_f64(acc[b]);
    if (lane == 0 && b0 + b < B) x_rot[static_cast<int64_t>(b0 + b) * d + j] = static_cast<float>(s);
  }
}

// One token, x and Qt of one element type: every load of the row is issued
// before any is used, as in the fp32 one-token form above.
template <int NC, typename T>
__global__ __launch_bounds__(kWavesPerBlock * kWave) void rotate_row_f64_kernel(
    const T *__restrict__ x, const T *__restrict__ qt, float *__restrict__ x_rot, int d,
    int qb) {
  constexpr int V = Elt<T>::kVec;
  const int lane = threadIdx.x % kWave;
  const int j = blockIdx.x * kWavesPerBlock + wave_id();
  if (j >= d) return;
  const int64_t xoff = static_cast<int64_t>(j / qb) * qb;
  const T *row = qt + static_cast<int64_t>(j) * qb;
  const int chunks = qb / V;
  uint4 xq[NC], q[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + kWave * i;
    const bool ok = c < chunks;
    xq[i] = ok ? load16(x + xoff + c * V) : make_uint4(0, 0, 0, 0);
    q[i] = ok ? load16(row + c * V) : make_uint4(0, 0, 0, 0);
  }
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    float xf[V], qf[V];
    Elt<T>::unpack(xq[i], xf);
    Elt<T>::unpack(q[i], qf);
#pragma unroll
    for (int v = 0; v < V; ++v)
      acc = fma(static_cast<double>(xf[v]), static_cast<double>(qf[v]), acc);
  }
  const double s = wave_sum_f64(acc);
  if (lane == 0) x_rot[j] = static_cast<float>(s);
}

template <typename T>
bool launch_row_f64(const void *x, const void *qt, float *x_rot, int d, int qb, hipStream_t s) {
  constexpr int V = Elt<T>::kVec;
  const int nc = (qb / V + kWave - 1) / kWave;
  const dim3 grid((d + kWavesPerBlock - 1) / kWavesPerBlock), block(kWavesPerBlock * kWave);
  const auto *xp = static_cast<const T *>(x);
  const auto *qp = static_cast<const T *>(qt);
  if (nc <= 2) hipLaunchKernelGGL((rotate_row_f64_kernel<2, T>), grid, block, 0, s, xp, qp, x_rot, d, qb);
  else if (nc <= 4) hipLaunchKernelGGL((rotate_row_f64_kernel<4, T>), grid, block, 0, s, xp, qp, x_rot, d, qb);
  else if (nc <= 8) hipLaunchKernelGGL((rotate_row_f64_kernel<8, T>), grid, block, 0, s, xp, qp, x_rot, d, qb);
  else if (nc <= 16) hipLaunchKernelGGL((rotate_row_f64_kernel<16, T>), grid, block, 0, s, xp, qp, x_rot, d, qb);
  else return false;
  return true;
}

template <int NC, int NB, typename XT, typename QT>
hipError_t launch_f64_t(const void *x, const void *qt, float *x_rot, int B, int d, int qb,
                        hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((d + kWavesPerBlock - 1) / kWavesPerBlock),
                  static_cast<unsigned>((B + NB - 1) / NB));
  hipLaunchKernelGGL((rotate_f64_kernel<NC, NB, XT, QT>), grid, dim3(kWavesPerBlock * kWave), 0,
                     s, static_cast<const XT *>(x), static_cast<const QT *>(qt), x_rot, B, d, qb);
  return hipGetLastError();
}

template <int NB, typename XT, typename QT>
hipError_t launch_f64_nc(const void *x, const void *qt, float *x_rot, int B, int d, int qb,
                         hipStream_t s) {
  const int nc = (qb / Elt<QT>::kVec + kWave - 1) / kWave;
  if (nc <= 2) return launch_f64_t<2, NB, XT, QT>(x, qt, x_rot, B, d, qb, s);
  if (nc <= 4) return launch_f64_t<4, NB, XT, QT>(x, qt, x_rot, B, d, qb, s);
  if (nc <= 8) return launch_f64_t<8, NB, XT, QT>(x, qt, x_rot, B, d, qb, s);
  return launch_f64_t<16, NB, XT, QT>(x, qt, x_rot, B, d, qb, s);  // looped past 16
}

template <typename XT, typename QT>
hipError_t launch_f64_nb(const void *x, const void *qt, float *x_rot, int B, int d, int qb,
                         hipStream_t s) {
  if (B == 1) return launch_f64_nc<1, XT, QT>(x, qt, x_rot, B, d, qb, s);
  if (B == 2) return launch_f64_nc<2, XT, QT>(x, qt, x_rot, B, d, qb, s);
  if (B <= 4) return launch_f64_nc<4, XT, QT>(x, qt, x_rot, B, d, qb, s);
  return launch_f64_nc<8, XT, QT>(x, qt, x_rot, B, d, qb, s);
}

}  // namespace

hipError_t launch_rotate(const void *x, int x_dt, const void *qt, int q_dt,
                         float *x_rot, int B, int d, int qb, hipStream_t s) {
  if (B == 1 && x_dt == q_dt) {
    const bool done = x_dt == kBF16 ? launch_row<uint16_t>(x, qt, x_rot, d, qb, s)
                                    : launch_row<float>(x, qt, x_rot, d, qb, s);
    if (done) return hipGetLastError();
  }
  if (B > 1 && x_dt == q_dt) {
    const bool done = x_dt == kBF16 ? launch_rows_batch<uint16_t>(x, qt, x_rot, B, d, qb, s)
                                    : launch_rows_batch<float>(x, qt, x_rot, B, d, qb, s);
    if (done) return hipGetLastError();
  }
  // Mixed types: tokens four at a time; each group re-reads Qt.
  const int xs = dt_size(x_dt);
  for (int b0 = 0; b0 < B; b0 += 4) {
    const int nb = B - b0 < 4 ? B - b0 : 4;
    const void *xb = static_cast<const char *>(x) + static_cast<int64_t>(b0) * d * xs;
    float *xr = x_rot + static_cast<int64_t>(b0) * d;
    hipError_t e;
    switch (nb) {
      case 1: e = launch_b<1>(xb, x_dt, qt, q_dt, xr, d, qb, s); break;
      case 2: e = launch_b<2>(xb, x_dt, qt, q_dt, xr, d, qb, s); break;
      case 3: e = launch_b<3>(xb, x_dt, qt, q_dt, xr, d, qb, s); break;
      default: e = launch_b<4>(xb, x_dt, qt, q_dt, xr, d, qb, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_rotate_f64(const void *x, int x_dt, const void *qt, int q_dt, float *x_rot,
                             int B, int d, int qb, hipStream_t s) {
  if (B == 1 && x_dt == q_dt) {
    const bool done = x_dt == kBF16 ? launch_row_f64<uint16_t>(x, qt, x_rot, d, qb, s)
                                    : launch_row_f64<float>(x, qt, x_rot, d, qb, s);
    if (done) return hipGetLastError();
  }
  if (x_dt == kBF16 && q_dt == kBF16) return launch_f64_nb<uint16_t, uint16_t>(x, qt, x_rot, B, d, qb, s);
  if (x_dt == kF32 && q_dt == kF32) return launch_f64_nb<float, float>(x, qt, x_rot, B, d, qb, s);
  if (x_dt == kF32 && q_dt == kBF16) return launch_f64_nb<float, uint16_t>(x, qt, x_rot, B, d, qb, s);
  if (x_dt == kBF16 && q_dt == kF32) return launch_f64_nb<uint16_t, float>(x, qt, x_rot, B, d, qb, s);
  return hipErrorInvalidValue;
}

}  // namespace larosa
