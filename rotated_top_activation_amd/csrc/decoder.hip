// Decoder-layer glue around the rotated sparse linears: RMSNorm, rotary
// position embedding, single-query attention over a key/value cache, and the
// residual add. The pages apply the rotated Top-K sparsification to the
// linear layers of a pretrained decoder (LaRoSA summary page, 方法详解 · 技术
// 框架) and give no transformer internals; these follow the LLaMA-style
// layer: RMSNorm with unit gain, rotate-half rotary embedding, softmax
// attention scaled by 1/sqrt(d_head), query head h reading key/value head
// h / (n_heads / n_kv_heads). Arithmetic is fp32 (rotary angles in fp64);
// every output is rounded once to the activation dtype.
#include "common.hpp"
#include "launch.hpp"

namespace larosa {
namespace {

constexpr int kGT = 256;  // threads per workgroup
constexpr int kGW = kGT / kWave;

__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kGW; ++i) s += red[i];
  return s;
}

__device__ __forceinline__ float block_max(float v, float *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) red[w] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < kGW; ++i) m = fmaxf(m, red[i]);
  return m;
}

// out[b, :] = h[b, :] / sqrt(mean(h[b, :]²) + eps); one workgroup per token.
template <typename T>
__global__ __launch_bounds__(kGT) void rmsnorm_kernel(const T *__restrict__ h, T *__restrict__ out,
                                                      int d, float eps) {
  __shared__ float red[kGW];
  const T *row = h + static_cast<int64_t>(blockIdx.x) * d;
  T *orow = out + static_cast<int64_t>(blockIdx.x) * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += kGT) {
    const float v = Elt<T>::load(row, i);
    ss = fmaf(v, v, ss);
  }
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(d) + eps);
  for (int i = threadIdx.x; i < d; i += kGT) Elt<T>::store(orow, i, Elt<T>::load(row, i) * inv);
}

// Rotate-half rotary embedding of the q and k heads of one token row:
// channel i pairs with i + d_head/2, angle pos · theta^(−2i/d_head).
template <typename T>
__global__ __launch_bounds__(kGT) void rope_kernel(const T *__restrict__ qk, int64_t stride,
                                                   T *__restrict__ q_out, T *__restrict__ k_out,
                                                   int B, int n_heads, int n_kv, int dh,
                                                   double pos, double theta) {
  const int half = dh / 2;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_tok = static_cast<int64_t>(n_heads + n_kv) * half;
  if (e >= per_tok * B) return;
  const int b = static_cast<int>(e / per_tok);
  const int r = static_cast<int>(e % per_tok);
  const int head = r / half, i = r % half;
  const T *src = qk + b * stride + static_cast<int64_t>(head) * dh;
  T *dst = head < n_heads ? q_out + (static_cast<int64_t>(b) * n_heads + head) * dh
                          : k_out + (static_cast<int64_t>(b) * n_kv + (head - n_heads)) * dh;
  const double ang = pos * pow(theta, -2.0 * i / dh);
  double sd, cd;
  sincos(ang, &sd, &cd);
  const float s = static_cast<float>(sd), c = static_cast<float>(cd);
  const float a = Elt<T>::load(src, i), bb = Elt<T>::load(src, i + half);
  Elt<T>::store(dst, i, a * c - bb * s);
  Elt<T>::store(dst, i + half, bb * c + a * s);
}

// One workgroup per (query head, token). The cache is [B, n_kv, T, 128];
// the new token's key and value sit at k_new + b·k_stride + kv·128 and
// v_new + b·v_stride + kv·128.
// Single-query attention, one 1024-thread workgroup per (token, head). A key
// or value row (one position's 128 channels) is read by LPR lanes with
// 16-byte loads, so one wave instruction covers 64/LPR rows; the 16 waves
// take interleaved row groups and keep kAttBatch instructions in flight.
// Pass 1 writes the scores of the T cached positions and the new one to LDS;
// then one max and one sum of the exponentials; pass 2 accumulates p·v per
// lane and folds the row slots and the waves.
constexpr int kAT = 1024;
constexpr int kAW = kAT / kWave;
constexpr int kAttBatch = 8;

template <int NW>
__device__ __forceinline__ float block_sum_w(float v, float *red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) s += red[i];
  return s;
}

template <int NW>
__device__ __forceinline__ float block_max_w(float v, float *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (threadIdx.x % kWave == 0) red[w] = v;
  __syncthreads();
  float m = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) m = fmaxf(m, red[i]);
  return m;
}

template <typename T>
__global__ __launch_bounds__(kAT) void decode_attention_kernel(
    const T *__restrict__ q, const T *__restrict__ k_new, int64_t k_stride,
    const T *__restrict__ v_new, int64_t v_stride, const T *__restrict__ kc,
    const T *__restrict__ vc, T *__restrict__ out, int Tlen, int n_heads, int n_kv) {
  constexpr int DH = 128;
  constexpr int V = Elt<T>::kVec;      // channels per 16-byte load
  constexpr int LPR = DH / V;          // lanes per row
  constexpr int RPI = kWave / LPR;     // rows per wave instruction
  constexpr int ROWS = RPI * kAW;      // rows per round of the workgroup
  extern __shared__ float sc[];        // [Tlen + 1] scores, then p
  __shared__ float red[kAW];
  __shared__ float accs[kAW][DH];
  const int h = blockIdx.x, b = blockIdx.y;
  const int g = h / (n_heads / n_kv);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int slot = lane / LPR, c = lane % LPR;
  const T *kbase = kc + (static_cast<int64_t>(b) * n_kv + g) * Tlen * DH;
  const T *vbase = vc + (static_cast<int64_t>(b) * n_kv + g) * Tlen * DH;
  const T *kn = k_new + b * k_stride + static_cast<int64_t>(g) * DH;
  const T *vn = v_new + b * v_stride + static_cast<int64_t>(g) * DH;
  const int n = Tlen + 1;  // positions, the new token last
  auto row_of = [&](const T *base, const T *nw, int t) {
    return t < Tlen ? base + static_cast<int64_t>(t) * DH : nw;
  };
  // this lane's query channels
  float qf[V];
  Elt<T>::unpack(load16(q + (static_cast<int64_t>(b) * n_heads + h) * DH + c * V), qf);
  const float scale = 1.0f / sqrtf(static_cast<float>(DH));

  // pass 1: scores
  float mx = -INFINITY;
  for (int r0 = wave * RPI; r0 < n; r0 += ROWS * kAttBatch) {
    uint4 kq[kAttBatch];
#pragma unroll
    for (int i = 0; i < kAttBatch; ++i) {
      const int t = r0 + i * ROWS + slot;
      kq[i] = t < n ? load16(row_of(kbase, kn, t) + c * V) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kAttBatch; ++i) {
      float kf[V];
      Elt<T>::unpack(kq[i], kf);
      float s = 0.f;
#pragma unroll
      for (int v = 0; v < V; ++v) s = fmaf(qf[v], kf[v], s);
#pragma unroll
      for (int off = LPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, kWave);
      const int t = r0 + i * ROWS + slot;
      if (t < n) {
        s *= scale;
        if (c == 0) sc[t] = s;
        mx = fmaxf(mx, s);
      }
    }
  }
  mx = block_max_w<kAW>(mx, red);  // its barriers also order the sc[] writes
  float sum = 0.f;
  for (int t = threadIdx.x; t < n; t += kAT) {
    const float p = expf(sc[t] - mx);
    sc[t] = p;
    sum += p;
  }
  sum = block_sum_w<kAW>(sum, red);

  // pass 2: Σ p·v, V channels per lane for its row slot
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
  for (int r0 = wave * RPI; r0 < n; r0 += ROWS * kAttBatch) {
    uint4 vq[kAttBatch];
#pragma unroll
    for (int i = 0; i < kAttBatch; ++i) {
      const int t = r0 + i * ROWS + slot;
      vq[i] = t < n ? load16(row_of(vbase, vn, t) + c * V) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kAttBatch; ++i) {
      const int t = r0 + i * ROWS + slot;
      const float p = t < n ? sc[t] : 0.f;
      float vf[V];
      Elt<T>::unpack(vq[i], vf);
#pragma unroll
      for (int v = 0; v < V; ++v) acc[v] = fmaf(p, vf[v], acc[v]);
    }
  }
  // fold the row slots (lanes c, c + LPR, …), then the waves
#pragma unroll
  for (int v = 0; v < V; ++v)
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) acc[v] += __shfl_xor(acc[v], off, kWave);
  if (slot == 0) {
#pragma unroll
    for (int v = 0; v < V; ++v) accs[wave][c * V + v] = acc[v];
  }
  __syncthreads();
  T *orow = out + (static_cast<int64_t>(b) * n_heads + h) * DH;
  for (int i = threadIdx.x; i < DH; i += kAT) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kAW; ++w) s += accs[w][i];
    Elt<T>::store(orow, i, s / sum);
  }
}

// h[i] = h[i] + o[i], rounded to T.
template <typename T>
__global__ __launch_bounds__(kGT) void residual_add_kernel(T *__restrict__ h,
                                                           const T *__restrict__ o, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) Elt<T>::store(h, i, Elt<T>::load(h, i) + Elt<T>::load(o, i));
}

unsigned blocks_for(int64_t n) { return static_cast<unsigned>((n + kGT - 1) / kGT); }

}  // namespace

hipError_t launch_rmsnorm(const void *h, void *out, int64_t B, int64_t d, float eps, int dt,
                          hipStream_t s) {
  if (dt == kF32)
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(static_cast<unsigned>(B)), dim3(kGT), 0, s,
                       static_cast<const float *>(h), static_cast<float *>(out),
                       static_cast<int>(d), eps);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<uint16_t>, dim3(static_cast<unsigned>(B)), dim3(kGT), 0, s,
                       static_cast<const uint16_t *>(h), static_cast<uint16_t *>(out),
                       static_cast<int>(d), eps);
  return hipGetLastError();
}

hipError_t launch_rope(const void *qk, int64_t stride, void *q_out, void *k_out, int64_t B,
                       int64_t n_heads, int64_t n_kv, int64_t dh, int64_t pos, double theta,
                       int dt, hipStream_t s) {
  const int64_t n = B * (n_heads + n_kv) * (dh / 2);
  if (dt == kF32)
    hipLaunchKernelGGL(rope_kernel<float>, dim3(blocks_for(n)), dim3(kGT), 0, s,
                       static_cast<const float *>(qk), stride, static_cast<float *>(q_out),
                       static_cast<float *>(k_out), static_cast<int>(B), static_cast<int>(n_heads),
                       static_cast<int>(n_kv), static_cast<int>(dh), static_cast<double>(pos),
                       theta);
  else
    hipLaunchKernelGGL(rope_kernel<uint16_t>, dim3(blocks_for(n)), dim3(kGT), 0, s,
                       static_cast<const uint16_t *>(qk), stride, static_cast<uint16_t *>(q_out),
                       static_cast<uint16_t *>(k_out), static_cast<int>(B),
                       static_cast<int>(n_heads), static_cast<int>(n_kv), static_cast<int>(dh),
                       static_cast<double>(pos), theta);
  return hipGetLastError();
}

hipError_t launch_decode_attention(const void *q, const void *k_new, int64_t k_stride,
                                   const void *v_new, int64_t v_stride, const void *kc,
                                   const void *vc, void *out, int64_t B, int64_t Tlen,
                                   int64_t n_heads, int64_t n_kv, int dt, hipStream_t s) {
  const size_t lds = (static_cast<size_t>(Tlen) + 1) * sizeof(float);
  dim3 grid(static_cast<unsigned>(n_heads), static_cast<unsigned>(B));
  if (dt == kF32)
    hipLaunchKernelGGL(decode_attention_kernel<float>, grid, dim3(kAT), lds, s,
                       static_cast<const float *>(q), static_cast<const float *>(k_new), k_stride,
                       static_cast<const float *>(v_new), v_stride,
                       static_cast<const float *>(kc), static_cast<const float *>(vc),
                       static_cast<float *>(out), static_cast<int>(Tlen),
                       static_cast<int>(n_heads), static_cast<int>(n_kv));
  else
    hipLaunchKernelGGL(decode_attention_kernel<uint16_t>, grid, dim3(kAT), lds, s,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k_new),
                       k_stride, static_cast<const uint16_t *>(v_new), v_stride,
                       static_cast<const uint16_t *>(kc), static_cast<const uint16_t *>(vc),
                       static_cast<uint16_t *>(out), static_cast<int>(Tlen),
                       static_cast<int>(n_heads), static_cast<int>(n_kv));
  return hipGetLastError();
}

hipError_t launch_residual_add(void *h, const void *o, int64_t n, int dt, hipStream_t s) {
  if (dt == kF32)
    hipLaunchKernelGGL(residual_add_kernel<float>, dim3(blocks_for(n)), dim3(kGT), 0, s,
                       static_cast<float *>(h), static_cast<const float *>(o), n);
  else
    hipLaunchKernelGGL(residual_add_kernel<uint16_t>, dim3(blocks_for(n)), dim3(kGT), 0, s,
                       static_cast<uint16_t *>(h), static_cast<const uint16_t *>(o), n);
  return hipGetLastError();
}

}  // namespace larosa
