// Device helpers shared by the HIP kernels of liblarosa (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace larosa {

constexpr int kWave = 64;

// bf16 is carried as its 16-bit pattern. Widening is exact: the pattern is
// the top half of the fp32 pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 → bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// SiLU(g)·u = g / (1 + e^-g) · u in fp32 (one definition for every kernel
// that applies it, so they agree bit for bit).
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Rotary position embedding of one pair (a, b) = (x[i], x[i + dh/2]) of a
// head with the pair's cosine c and sine s: (a·c − b·s, b·c + a·s) in fp32
// with fixed fused multiply-adds (one definition for every kernel that
// applies it).
__device__ __forceinline__ float rope_lo(float a, float b, float c, float s) { return fmaf(-b, s, a * c); }
__device__ __forceinline__ float rope_hi(float a, float b, float c, float s) { return fmaf(a, s, b * c); }

// Element access by type tag: float or uint16_t (bf16).
template <typename T> struct Elt;
template <> struct Elt<float> {
  static constexpr int kVec = 4;  // elements per 16-byte load
  __device__ __forceinline__ static float round(float v) { return v; }
  __device__ __forceinline__ static float load(const float *p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float *p, int64_t i, float v) { p[i] = v; }
  // Unpack one 16-byte chunk into kVec floats.
  __device__ __forceinline__ static void unpack(const uint4 &q, float *o) {
    o[0] = __uint_as_float(q.x); o[1] = __uint_as_float(q.y);
    o[2] = __uint_as_float(q.z); o[3] = __uint_as_float(q.w);
  }
};
template <> struct Elt<uint16_t> {
  static constexpr int kVec = 8;
  // the value after one rounding to this type
  __device__ __forceinline__ static float round(float v) { return bf16_to_f32(f32_to_bf16(v)); }
  __device__ __forceinline__ static float load(const uint16_t *p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t *p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
  __device__ __forceinline__ static void unpack(const uint4 &q, float *o) {
    o[0] = bf16_lo(q.x); o[1] = bf16_hi(q.x); o[2] = bf16_lo(q.y); o[3] = bf16_hi(q.y);
    o[4] = bf16_lo(q.z); o[5] = bf16_hi(q.z); o[6] = bf16_lo(q.w); o[7] = bf16_hi(q.w);
  }
};

// Coefficients of the matrix-core product, stored split: for token b and
// list position k, the bf16 truncation hi of c and lo = bf16(c − hi) sit in
// 16-element groups [b][k / 8] of (8 hi, 8 lo), so one lane's eight
// consecutive positions are one 16-byte hi load and one 16-byte lo load.
// ldc (a multiple of 8) is the padded list length.
__device__ __forceinline__ void store_coef_hl(uint16_t *base, int64_t ldc, int64_t b, int64_t k,
                                              float c) {
  const uint32_t u = __float_as_uint(c) & 0xFFFF0000u;
  const int64_t at = (b * (ldc / 8) + k / 8) * 16 + k % 8;
  base[at] = static_cast<uint16_t>(u >> 16);
  base[at + 8] = f32_to_bf16(c - __uint_as_float(u));
}

__device__ __forceinline__ uint4 load16(const void *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

// Sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Inclusive prefix sum over the lanes of a wave (lane order), with DPP
// lane moves (register to register, no LDS round trip): shifts by 1, 2, 4
// and 8 lanes within each 16-lane row (lanes shifted in from outside the row
// read 0), then the last lane of row 0 added to row 1 and of row 2 to row 3
// (row_bcast:15), then lane 31 added to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
  (void)lane;
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xA, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xC, 0xF, false));
  return v;
}

// Wave index as a value the compiler can keep in a scalar register.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

}  // namespace larosa
