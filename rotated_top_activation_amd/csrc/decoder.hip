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

#include <cmath>

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

// The same RMSNorm with 16-byte loads, optionally after the residual add:
// one workgroup per token; thread t owns the 16-byte chunks t, t + 256, ...
// of the row (at most CPT of them), loads every one of them before using
// any, and keeps them in registers for the normalisation, so the row is read
// once. With RESID the row is first h + o rounded to T, written back to h
// (the residual add), and the norm is taken of that rounded sum, exactly as
// a separate add followed by the norm would see it. The sum of squares adds
// a thread's chunks in order, then the block's threads in a fixed tree, so
// the standalone and the fused form give the same bits.
template <typename T, int CPT, bool RESID>
__global__ __launch_bounds__(kGT) void norm_vec_kernel(T *__restrict__ h, const T *__restrict__ o,
                                                       T *__restrict__ out, int d, float eps) {
  constexpr int V = Elt<T>::kVec;
  __shared__ float red[kGW];
  const int64_t base = static_cast<int64_t>(blockIdx.x) * d;
  const int chunks = d / V;
  uint4 hq[CPT], oq[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int j = threadIdx.x + c * kGT;
    const int jc = j < chunks ? j : chunks - 1;
    hq[c] = load16(h + base + static_cast<int64_t>(jc) * V);
    if (RESID) oq[c] = load16(o + base + static_cast<int64_t>(jc) * V);
  }
  float v[CPT][V];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int j = threadIdx.x + c * kGT;
    Elt<T>::unpack(hq[c], v[c]);
    if (RESID) {
      float ov[V];
      Elt<T>::unpack(oq[c], ov);
#pragma unroll
      for (int e = 0; e < V; ++e) v[c][e] = Elt<T>::round(v[c][e] + ov[e]);
    }
    if (j < chunks) {
#pragma unroll
      for (int e = 0; e < V; ++e) ss = fmaf(v[c][e], v[c][e], ss);
      if (RESID) {
#pragma unroll
        for (int e = 0; e < V; ++e) Elt<T>::store(h, base + static_cast<int64_t>(j) * V + e, v[c][e]);
      }
    }
  }
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(d) + eps);
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int j = threadIdx.x + c * kGT;
    if (j < chunks) {
#pragma unroll
      for (int e = 0; e < V; ++e)
        Elt<T>::store(out, base + static_cast<int64_t>(j) * V + e, v[c][e] * inv);
    }
  }
}

// One token: the RMSNorm above (after the residual add with RESID) folded
// into the one-token rotation of the normalised row by a dense Q (q_block
// == d), bf16 only. A 256-thread workgroup first takes the norm exactly as
// norm_vec_kernel does (thread t owns chunks t, t + 256, ...; the same
// rounding of the residual sum, the same order of the sum of squares and the
// same block sum) and lays the normalised row out in LDS as bf16; then each
// of its 4 waves computes one output channel of x_rot as the one-token
// rotation does (lane chunks lane + 64·i, the Qt row requested before the
// norm is taken, the same wave sum). So x_rot, the new residual h_out and the
// normalised row a_out have the bits of larosa_residual_rmsnorm followed by
// larosa_rotate. Workgroup 0 writes h_out and a_out; every workgroup reads h
// and o, so h_out must be another buffer.
constexpr int kNRWaves = kGW;               // one output channel per wave
constexpr int kNRMaxChunks = 8192 / 8;      // d <= 8192 (bf16)

// Eight floats, each already a bf16 value, as one 16-byte chunk.
__device__ __forceinline__ uint4 pack_bf16x8(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e)
    w[e] = static_cast<uint32_t>(f32_to_bf16(f[2 * e])) |
           (static_cast<uint32_t>(f32_to_bf16(f[2 * e + 1])) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int NC, int CPT, bool RESID>
__global__ __launch_bounds__(kGT) void norm_rotate_row_kernel(
    const uint16_t *__restrict__ h, const uint16_t *__restrict__ o, uint16_t *__restrict__ h_out,
    uint16_t *__restrict__ a_out, const uint16_t *__restrict__ qt, float *__restrict__ x_rot,
    int d, float eps) {
  constexpr int V = 8;
  __shared__ float red[kGW];
  __shared__ uint4 arow[kNRMaxChunks];
  const int lane = threadIdx.x % kWave;
  const int j = blockIdx.x * kNRWaves + static_cast<int>(threadIdx.x / kWave);  // < d: d % 4 == 0
  const uint16_t *row = qt + static_cast<int64_t>(j) * d;
  const int chunks = d / V;
  // The residual row first: a wave's loads return in issue order, so the
  // norm (row from L2) then runs while the Qt row is still on its way.
  uint4 hq[CPT], oq[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int jj = threadIdx.x + c * kGT;
    const int jc = jj < chunks ? jj : chunks - 1;
    hq[c] = load16(h + jc * V);
    if (RESID) oq[c] = load16(o + jc * V);
  }
  // keep those loads ahead of the Qt row's (no memory access moves across)
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  // Every lane issues all NC loads (past the row: its last chunk again), so
  // no load sits under a branch and the wait before the norm covers the
  // residual row only.
  uint4 q[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + kWave * i;
    q[i] = load16(row + (c < chunks ? c : chunks - 1) * V);
  }
  // the norm, as norm_vec_kernel takes it
  float v[CPT][V];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int jj = threadIdx.x + c * kGT;
    Elt<uint16_t>::unpack(hq[c], v[c]);
    if (RESID) {
      float ov[V];
      Elt<uint16_t>::unpack(oq[c], ov);
#pragma unroll
      for (int e = 0; e < V; ++e) v[c][e] = Elt<uint16_t>::round(v[c][e] + ov[e]);
    }
    if (jj < chunks) {
#pragma unroll
      for (int e = 0; e < V; ++e) ss = fmaf(v[c][e], v[c][e], ss);
      if (RESID && blockIdx.x == 0 && h_out != nullptr)
        *reinterpret_cast<uint4 *>(h_out + jj * V) = pack_bf16x8(v[c]);
    }
  }
  const float tot = block_sum(ss, red);
  const float inv = 1.0f / sqrtf(tot / static_cast<float>(d) + eps);
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int jj = threadIdx.x + c * kGT;
    if (jj < chunks) {
#pragma unroll
      for (int e = 0; e < V; ++e) v[c][e] = v[c][e] * inv;
      const uint4 a = pack_bf16x8(v[c]);  // rounded once, as the norm kernel stores it
      arow[jj] = a;
      if (blockIdx.x == 0 && a_out != nullptr) *reinterpret_cast<uint4 *>(a_out + jj * V) = a;
    }
  }
  __syncthreads();
  // the one-token rotation of the normalised row
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = lane + kWave * i;
    float af[V], qf[V];
    Elt<uint16_t>::unpack(c < chunks ? arow[c] : make_uint4(0, 0, 0, 0), af);
    Elt<uint16_t>::unpack(c < chunks ? q[i] : make_uint4(0, 0, 0, 0), qf);
#pragma unroll
    for (int e = 0; e < V; ++e) acc = fmaf(af[e], qf[e], acc);
  }
  const float sum = wave_sum(acc);
  if (lane == 0) x_rot[j] = sum;
}

// Rotate-half rotary embedding of the q and k heads of one token row:
// channel i pairs with i + d_head/2, angle pos · theta^(−2i/d_head).
template <typename T>
__global__ __launch_bounds__(kGT) void rope_kernel(const T *__restrict__ qk, int64_t stride,
                                                   T *__restrict__ q_out, T *__restrict__ k_out,
                                                   int B, int n_heads, int n_kv, RopeTable tab) {
  const int dh = tab.dh, half = dh / 2;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_tok = static_cast<int64_t>(n_heads + n_kv) * half;
  if (e >= per_tok * B) return;
  const int b = static_cast<int>(e / per_tok);
  const int r = static_cast<int>(e % per_tok);
  const int head = r / half, i = r % half;
  const T *src = qk + b * stride + static_cast<int64_t>(head) * dh;
  T *dst = head < n_heads ? q_out + (static_cast<int64_t>(b) * n_heads + head) * dh
                          : k_out + (static_cast<int64_t>(b) * n_kv + (head - n_heads)) * dh;
  const float cs = tab.cs[i], sn = tab.sn[i];
  const float a = Elt<T>::load(src, i), bb = Elt<T>::load(src, i + half);
  Elt<T>::store(dst, i, rope_lo(a, bb, cs, sn));
  Elt<T>::store(dst, i + half, rope_hi(a, bb, cs, sn));
}

// The same rotation in place on the first n_rot heads of each token's row
// (row b at qk + b·stride), one thread per pair.
template <typename T>
__global__ __launch_bounds__(kGT) void rope_inplace_kernel(T *__restrict__ qk, int64_t stride,
                                                           int B, int n_rot, RopeTable tab) {
  const int dh = tab.dh, half = dh / 2;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_tok = static_cast<int64_t>(n_rot) * half;
  if (e >= per_tok * B) return;
  const int b = static_cast<int>(e / per_tok);
  const int r = static_cast<int>(e % per_tok);
  const int head = r / half, i = r % half;
  T *row = qk + b * stride + static_cast<int64_t>(head) * dh;
  const float cs = tab.cs[i], sn = tab.sn[i];
  const float a = Elt<T>::load(row, i), bb = Elt<T>::load(row, i + half);
  Elt<T>::store(row, i, rope_lo(a, bb, cs, sn));
  Elt<T>::store(row, i + half, rope_hi(a, bb, cs, sn));
}

// One workgroup per (query head, token). The cache is [B, n_kv, T, 128];
// the new token's key and value sit at k_new + b·k_stride + kv·128 and
// v_new + b·v_stride + kv·128.
// Single-query attention. A key or value row (one position's 128 channels)
// is read by LPR lanes with 16-byte loads, so one wave instruction covers
// 64/LPR rows. The scores go to LDS; then one max and one sum of the
// exponentials; then p·v accumulates per lane and the row slots and the
// waves are folded.

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

// The positions are cut into chunks of kACh, one 256-thread workgroup per
// (token, head, chunk), so a single token still spreads its heads' cache
// reads over the whole chip (32 heads × 33 chunks at T = 2048), and a wave
// issues all its key and value loads before using any (one memory round
// trip per chunk). A chunk
// writes its own maximum score m, Σ exp(s − m) and Σ exp(s − m)·v; a second
// kernel rescales the chunks to the common maximum and adds them in chunk
// order (softmax over the union of the chunks, deterministic).
constexpr int kACT = 256;
constexpr int kACW = kACT / kWave;
constexpr int kACh = 64;  // positions per chunk: every key and value load of a wave in flight at once

template <typename T>
__global__ __launch_bounds__(kACT) void attn_chunk_kernel(
    const T *__restrict__ q, const T *__restrict__ k_new, int64_t k_stride,
    const T *__restrict__ v_new, int64_t v_stride, const T *__restrict__ kc,
    const T *__restrict__ vc, float *__restrict__ part_m, float *__restrict__ part_l,
    float *__restrict__ part_o, int Tlen, int n_heads, int n_kv, int S) {
  constexpr int DH = 128;
  constexpr int V = Elt<T>::kVec;      // channels per 16-byte load
  constexpr int LPR = DH / V;          // lanes per row
  constexpr int RPI = kWave / LPR;     // rows per wave instruction
  constexpr int ROWS = RPI * kACW;     // rows per round of the workgroup
  __shared__ float sc[kACh];           // the chunk's scores, then p
  __shared__ float red[kACW];
  __shared__ float accs[kACW][DH];
  const int h = blockIdx.x / S, ci = blockIdx.x % S, b = blockIdx.y;
  const int g = h / (n_heads / n_kv);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int slot = lane / LPR, c = lane % LPR;
  const T *kbase = kc + (static_cast<int64_t>(b) * n_kv + g) * Tlen * DH;
  const T *vbase = vc + (static_cast<int64_t>(b) * n_kv + g) * Tlen * DH;
  const T *kn = k_new + b * k_stride + static_cast<int64_t>(g) * DH;
  const T *vn = v_new + b * v_stride + static_cast<int64_t>(g) * DH;
  const int n = Tlen + 1;  // positions, the new token last
  const int t0 = ci * kACh;
  const int t1 = t0 + kACh < n ? t0 + kACh : n;  // S = ceil(n / kACh): never empty
  auto row_of = [&](const T *base, const T *nw, int t) {
    return t < Tlen ? base + static_cast<int64_t>(t) * DH : nw;
  };
  float qf[V];
  Elt<T>::unpack(load16(q + (static_cast<int64_t>(b) * n_heads + h) * DH + c * V), qf);
  const float scale = 1.0f / sqrtf(static_cast<float>(DH));

  // every key and value row of this wave's share of the chunk, loaded at once
  constexpr int NI = kACh / ROWS;  // wave instructions per pass (4 bf16, 8 fp32)
  static_assert(NI * ROWS == kACh, "chunk must be whole rounds");
  uint4 kq[NI], vq[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int t = t0 + wave * RPI + i * ROWS + slot;
    const bool ok = t < t1;
    kq[i] = ok ? load16(row_of(kbase, kn, t) + c * V) : make_uint4(0, 0, 0, 0);
    vq[i] = ok ? load16(row_of(vbase, vn, t) + c * V) : make_uint4(0, 0, 0, 0);
  }
  // scores
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float kf[V];
    Elt<T>::unpack(kq[i], kf);
    float sdot = 0.f;
#pragma unroll
    for (int v = 0; v < V; ++v) sdot = fmaf(qf[v], kf[v], sdot);
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) sdot += __shfl_xor(sdot, off, kWave);
    const int t = t0 + wave * RPI + i * ROWS + slot;
    if (t < t1) {
      sdot *= scale;
      if (c == 0) sc[t - t0] = sdot;
      mx = fmaxf(mx, sdot);
    }
  }
  mx = block_max_w<kACW>(mx, red);  // its barriers also order the sc[] writes
  float sum = 0.f;
  for (int t = threadIdx.x; t < t1 - t0; t += kACT) {
    const float p = expf(sc[t] - mx);
    sc[t] = p;
    sum += p;
  }
  sum = block_sum_w<kACW>(sum, red);
  // Σ p·v, V channels per lane for its row slot
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int t = t0 + wave * RPI + i * ROWS + slot;
    const float p = t < t1 ? sc[t - t0] : 0.f;
    float vf[V];
    Elt<T>::unpack(vq[i], vf);
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = fmaf(p, vf[v], acc[v]);
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
  const int64_t pi = (static_cast<int64_t>(b) * n_heads + h) * S + ci;
  for (int i = threadIdx.x; i < DH; i += kACT) {
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kACW; ++w) o += accs[w][i];
    part_o[pi * DH + i] = o;
  }
  if (threadIdx.x == 0) {
    part_m[pi] = mx;
    part_l[pi] = sum;
  }
}

// out[b, h, i] = Σ_c e^{m_c − m}·o_c[i] / Σ_c e^{m_c − m}·l_c, chunks in order.
template <typename T>
__global__ __launch_bounds__(128) void attn_combine_kernel(const float *__restrict__ part_m,
                                                           const float *__restrict__ part_l,
                                                           const float *__restrict__ part_o,
                                                           T *__restrict__ out, int n_heads,
                                                           int S) {
  const int h = blockIdx.x, b = blockIdx.y, i = threadIdx.x;
  const int64_t base = (static_cast<int64_t>(b) * n_heads + h) * S;
  float m = -INFINITY;
#pragma unroll 8
  for (int c = 0; c < S; ++c) m = fmaxf(m, part_m[base + c]);
  float l = 0.f, o = 0.f;
#pragma unroll 8
  for (int c = 0; c < S; ++c) {
    const float w = expf(part_m[base + c] - m);
    l = fmaf(part_l[base + c], w, l);
    o = fmaf(part_o[(base + c) * 128 + i], w, o);
  }
  Elt<T>::store(out, (static_cast<int64_t>(b) * n_heads + h) * 128 + i, o / l);
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

template <typename T, bool RESID>
bool launch_norm_vec(void *h, const void *o, void *out, int64_t B, int64_t d, float eps,
                     hipStream_t s) {
  constexpr int V = Elt<T>::kVec;
  const auto ok16 = [](const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (d % V || !ok16(h) || !ok16(out) || (RESID && !ok16(o))) return false;
  const int64_t per_thread = (d / V + kGT - 1) / kGT;
  const dim3 grid(static_cast<unsigned>(B)), block(kGT);
  T *hp = static_cast<T *>(h);
  const T *op = static_cast<const T *>(o);
  T *outp = static_cast<T *>(out);
  const int di = static_cast<int>(d);
  if (per_thread <= 2) hipLaunchKernelGGL((norm_vec_kernel<T, 2, RESID>), grid, block, 0, s, hp, op, outp, di, eps);
  else if (per_thread <= 4) hipLaunchKernelGGL((norm_vec_kernel<T, 4, RESID>), grid, block, 0, s, hp, op, outp, di, eps);
  else if (per_thread <= 8) hipLaunchKernelGGL((norm_vec_kernel<T, 8, RESID>), grid, block, 0, s, hp, op, outp, di, eps);
  else return false;
  return true;
}

hipError_t launch_residual_rmsnorm(void *h, const void *o, void *out, int64_t B, int64_t d,
                                   float eps, int dt, hipStream_t s) {
  const bool vec = dt == kF32 ? launch_norm_vec<float, true>(h, o, out, B, d, eps, s)
                              : launch_norm_vec<uint16_t, true>(h, o, out, B, d, eps, s);
  if (vec) return hipGetLastError();
  // ragged rows: the two separate steps
  hipError_t e = launch_residual_add(h, o, B * d, dt, s);
  if (e != hipSuccess) return e;
  return launch_rmsnorm(h, out, B, d, eps, dt, s);
}

hipError_t launch_rmsnorm(const void *h, void *out, int64_t B, int64_t d, float eps, int dt,
                          hipStream_t s) {
  // h is only read here (the residual form writes it)
  const bool vec = dt == kF32
                       ? launch_norm_vec<float, false>(const_cast<void *>(h), nullptr, out, B, d, eps, s)
                       : launch_norm_vec<uint16_t, false>(const_cast<void *>(h), nullptr, out, B, d, eps, s);
  if (vec) return hipGetLastError();
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

hipError_t launch_norm_rotate(const void *h, const void *o, void *h_out, void *a_out,
                              const void *qt, float *x_rot, int64_t d, float eps, hipStream_t s) {
  // d % 8 == 0, 256 < d <= 8192 (host-checked): d / 4 whole workgroups
  const int chunks = static_cast<int>(d / 8);
  const int nc = (chunks + kWave - 1) / kWave;
  const int cpt = (chunks + kGT - 1) / kGT;
  if (d % 8 || chunks > kNRMaxChunks || nc > 16) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(d / kNRWaves)), block(kGT);
  const auto *hp = static_cast<const uint16_t *>(h);
  const auto *op = static_cast<const uint16_t *>(o);
  auto *hop = static_cast<uint16_t *>(h_out);
  auto *ap = static_cast<uint16_t *>(a_out);
  const auto *qp = static_cast<const uint16_t *>(qt);
  const int di = static_cast<int>(d);
#define LAROSA_NR(NC, CPT)                                                                         \
  do {                                                                                             \
    if (o)                                                                                         \
      hipLaunchKernelGGL((norm_rotate_row_kernel<NC, CPT, true>), grid, block, 0, s, hp, op, hop,  \
                         ap, qp, x_rot, di, eps);                                                  \
    else                                                                                           \
      hipLaunchKernelGGL((norm_rotate_row_kernel<NC, CPT, false>), grid, block, 0, s, hp, op, hop, \
                         ap, qp, x_rot, di, eps);                                                  \
  } while (0)
  if (nc <= 8 && cpt <= 2) LAROSA_NR(8, 2);
  else LAROSA_NR(16, 4);
#undef LAROSA_NR
  return hipGetLastError();
}

hipError_t launch_rope(const void *qk, int64_t stride, void *q_out, void *k_out, int64_t B,
                       int64_t n_heads, int64_t n_kv, const RopeTable &tab, int dt,
                       hipStream_t s) {
  const int64_t n = B * (n_heads + n_kv) * (tab.dh / 2);
  if (n == 0) return hipSuccess;
  if (dt == kF32)
    hipLaunchKernelGGL(rope_kernel<float>, dim3(blocks_for(n)), dim3(kGT), 0, s,
                       static_cast<const float *>(qk), stride, static_cast<float *>(q_out),
                       static_cast<float *>(k_out), static_cast<int>(B), static_cast<int>(n_heads),
                       static_cast<int>(n_kv), tab);
  else
    hipLaunchKernelGGL(rope_kernel<uint16_t>, dim3(blocks_for(n)), dim3(kGT), 0, s,
                       static_cast<const uint16_t *>(qk), stride, static_cast<uint16_t *>(q_out),
                       static_cast<uint16_t *>(k_out), static_cast<int>(B),
                       static_cast<int>(n_heads), static_cast<int>(n_kv), tab);
  return hipGetLastError();
}

hipError_t launch_rope_inplace(void *qk, int64_t stride, int64_t B, int64_t n_rot,
                               const RopeTable &tab, int dt, hipStream_t s) {
  const int64_t n = B * n_rot * (tab.dh / 2);
  if (n == 0) return hipSuccess;
  if (dt == kF32)
    hipLaunchKernelGGL(rope_inplace_kernel<float>, dim3(blocks_for(n)), dim3(kGT), 0, s,
                       static_cast<float *>(qk), stride, static_cast<int>(B),
                       static_cast<int>(n_rot), tab);
  else
    hipLaunchKernelGGL(rope_inplace_kernel<uint16_t>, dim3(blocks_for(n)), dim3(kGT), 0, s,
                       static_cast<uint16_t *>(qk), stride, static_cast<int>(B),
                       static_cast<int>(n_rot), tab);
  return hipGetLastError();
}

RopeTable rope_table(int64_t dh, double pos, double theta) {
  RopeTable t;
  t.dh = static_cast<int>(dh);
  for (int i = 0; i < kRopeMaxHalf; ++i) {
    const double ang = i < dh / 2 ? pos * std::pow(theta, -2.0 * i / static_cast<double>(dh)) : 0.0;
    t.cs[i] = static_cast<float>(std::cos(ang));
    t.sn[i] = static_cast<float>(std::sin(ang));
  }
  return t;
}

size_t decode_attention_ws_bytes(int64_t B, int64_t Tlen, int64_t n_heads) {
  const int64_t S = (Tlen + 1 + kACh - 1) / kACh;
  return static_cast<size_t>(B) * n_heads * S * (2 + 128) * sizeof(float);
}

hipError_t launch_decode_attention(const void *q, const void *k_new, int64_t k_stride,
                                   const void *v_new, int64_t v_stride, const void *kc,
                                   const void *vc, void *out, int64_t B, int64_t Tlen,
                                   int64_t n_heads, int64_t n_kv, int dt, void *ws,
                                   hipStream_t s) {
  const int S = static_cast<int>((Tlen + 1 + kACh - 1) / kACh);
  const int64_t parts = B * n_heads * S;
  float *pm = static_cast<float *>(ws);
  float *pl = pm + parts;
  float *po = pl + parts;
  const dim3 grid(static_cast<unsigned>(n_heads * S), static_cast<unsigned>(B));
  const dim3 cgrid(static_cast<unsigned>(n_heads), static_cast<unsigned>(B));
  const int T = static_cast<int>(Tlen), H = static_cast<int>(n_heads), K = static_cast<int>(n_kv);
  if (dt == kF32) {
    hipLaunchKernelGGL(attn_chunk_kernel<float>, grid, dim3(kACT), 0, s,
                       static_cast<const float *>(q), static_cast<const float *>(k_new), k_stride,
                       static_cast<const float *>(v_new), v_stride,
                       static_cast<const float *>(kc), static_cast<const float *>(vc), pm, pl, po,
                       T, H, K, S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine_kernel<float>, cgrid, dim3(128), 0, s, pm, pl, po,
                       static_cast<float *>(out), H, S);
  } else {
    hipLaunchKernelGGL(attn_chunk_kernel<uint16_t>, grid, dim3(kACT), 0, s,
                       static_cast<const uint16_t *>(q), static_cast<const uint16_t *>(k_new),
                       k_stride, static_cast<const uint16_t *>(v_new), v_stride,
                       static_cast<const uint16_t *>(kc), static_cast<const uint16_t *>(vc), pm,
                       pl, po, T, H, K, S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_combine_kernel<uint16_t>, cgrid, dim3(128), 0, s, pm, pl, po,
                       static_cast<uint16_t *>(out), H, S);
  }
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
