// Block-wide exact Top-K threshold on |x| (device code shared by the
// standalone selection kernel and the fused linear kernel).
//
// Selection rule (LaRoSA summary page, 方法详解 · 技术框架: keep the K
// largest-magnitude entries; ties and order are this library's readings):
// the key of a channel is its fp32 bit pattern with the sign bit cleared,
// which orders like |x|; the kept set is every key above the K-th largest
// key T plus the `krem` lowest-index channels whose key equals T.
//
// Thread t of an NT-thread block owns EMAX register slots; slots without a
// channel carry a key with bit 31 set, which never matches a radix prefix.
// T is found by an exact radix select over the 31 key bits in digits of 11,
// 11 and 9 bits, with a 2048-bin LDS histogram per digit.
#pragma once

#include "common.hpp"

namespace larosa {

constexpr uint32_t kNoKey = 0x80000000u;

// Histogram bin b lives at hist[pad_bin(b)]: one padding word per 32 bins,
// so 64 lanes reading 32 consecutive bins each hit distinct banks.
__device__ __forceinline__ int pad_bin(int b) { return b + (b >> 5); }

template <int NT> struct SelectSmem {
  uint32_t hist[2048 + 64];
  uint32_t wave_tot[NT / kWave];
  uint32_t bin, above, count;
};

// Inclusive scan over the NT threads of the block (thread order).
template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t *wave_tot) {
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  uint32_t x = wave_incl_scan(v, lane);
  if (lane == kWave - 1) wave_tot[w] = x;
  __syncthreads();
  uint32_t off = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) off += i < w ? wave_tot[i] : 0u;
  __syncthreads();  // wave_tot may be rewritten by the next scan
  return x + off;
}

// Suffix search over the 2048 bins in sm.hist, done by wave 0 alone (the
// other waves wait at the closing barrier): the bin holding the krem-th
// largest key and the number of keys in higher bins, left in sm.bin and
// sm.above. Lane l first sums chunk 63 − l (32 bins), so lane order runs
// from the highest chunk down; a wave scan finds the chunk that crosses
// krem, then a second scan over that chunk's bins (highest first) finds the
// bin.
template <int NT>
__device__ __forceinline__ void suffix_search(uint32_t krem, SelectSmem<NT> &sm) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int chunk = 63 - lane;
    uint32_t s = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) s += sm.hist[pad_bin(chunk * 32 + i)];
    const uint32_t incl = wave_incl_scan(s, lane);
    const uint64_t cross = __ballot(incl >= krem);
    const int L = __ffsll(static_cast<unsigned long long>(cross)) - 1;  // krem <= total
    const uint32_t above_chunk = __shfl(incl - s, L, kWave);
    const int c = 63 - L;
    const uint32_t v = lane < 32 ? sm.hist[pad_bin(c * 32 + 31 - lane)] : 0u;
    const uint32_t incl2 = wave_incl_scan(v, lane);
    const uint64_t cross2 = __ballot(lane < 32 && above_chunk + incl2 >= krem);
    const int L2 = __ffsll(static_cast<unsigned long long>(cross2)) - 1;
    if (lane == L2) {
      sm.bin = static_cast<uint32_t>(c * 32 + 31 - lane);
      sm.above = above_chunk + incl2 - v;
      sm.count = v;
    }
  }
  __syncthreads();
}

// Radix digits: pass 0 takes key bits 30..20, pass 1 bits 19..9, pass 2
// bits 8..0 (key bit 31 is the no-key mark).
__host__ __device__ constexpr int radix_shift(int pass) { return pass == 0 ? 20 : (pass == 1 ? 9 : 0); }
__host__ __device__ constexpr uint32_t radix_dmask(int pass) { return pass == 2 ? 0x1FFu : 0x7FFu; }

// A radix pass taken in steps, for callers that hold their keys in another
// layout: radix_clear, then radix_count for every key (both followed by a
// barrier), then radix_resolve, which finds the bin holding the krem-th
// largest key among those matching (prefix, pmask), updates prefix, pmask
// and krem, and returns that bin's count.
template <int NT>
__device__ __forceinline__ void radix_clear(SelectSmem<NT> &sm) {
  for (int i = threadIdx.x; i < 2048 + 64; i += NT) sm.hist[i] = 0u;
}
template <int NT>
__device__ __forceinline__ void radix_count(uint32_t key, int pass, uint32_t prefix, uint32_t pmask,
                                            SelectSmem<NT> &sm) {
  if ((key & pmask) == prefix)
    atomicAdd(&sm.hist[pad_bin(static_cast<int>((key >> radix_shift(pass)) & radix_dmask(pass)))], 1u);
}
template <int NT>
__device__ __forceinline__ uint32_t radix_resolve(int pass, uint32_t &prefix, uint32_t &pmask,
                                                  uint32_t &krem, SelectSmem<NT> &sm) {
  suffix_search<NT>(krem, sm);
  prefix |= sm.bin << radix_shift(pass);
  pmask |= radix_dmask(pass) << radix_shift(pass);
  krem -= sm.above;
  const uint32_t count = sm.count;
  __syncthreads();  // bin / above are rewritten by the next pass
  return count;
}

// Radix passes first_pass..2 over the keys matching (prefix, pmask): finds T
// and krem for the krem-th largest key among them; eq_count is the number of
// keys equal to T (the last digit's bin count).
template <int NT, int EMAX>
__device__ __forceinline__ void radix_threshold_from(const uint32_t (&key)[EMAX], int first_pass,
                                                     uint32_t prefix, uint32_t pmask,
                                                     uint32_t krem, SelectSmem<NT> &sm,
                                                     uint32_t &T, uint32_t &krem_out,
                                                     uint32_t &eq_count) {
  const int t = threadIdx.x;
  uint32_t last_count = 0;
  for (int pass = first_pass; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 9 : 0);
    const uint32_t dmask = pass == 2 ? 0x1FFu : 0x7FFu;
    for (int i = t; i < 2048 + 64; i += NT) sm.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if ((key[e] & pmask) == prefix)
        atomicAdd(&sm.hist[pad_bin(static_cast<int>((key[e] >> shift) & dmask))], 1u);
    __syncthreads();
    suffix_search<NT>(krem, sm);
    prefix |= sm.bin << shift;
    pmask |= dmask << shift;
    krem -= sm.above;
    last_count = sm.count;
    __syncthreads();  // bin / above are rewritten by the next pass
  }
  T = prefix;
  krem_out = krem;
  eq_count = last_count;
}

// Finds T and krem for the top k of the keys held by the block, and the
// number of keys equal to T.
template <int NT, int EMAX>
__device__ __forceinline__ void radix_threshold(const uint32_t (&key)[EMAX], uint32_t k,
                                                SelectSmem<NT> &sm, uint32_t &T,
                                                uint32_t &krem_out, uint32_t &eq_count) {
  radix_threshold_from<NT, EMAX>(key, 0, 0u, kNoKey, k, sm, T, krem_out, eq_count);
}

// Index of the krem-th (1-based) channel, in index order, whose key equals
// T, over slots holding consecutive channels from i0 = t·E. Every thread
// gets the result. Channels with key == T are kept iff their index is at
// most this cut-off.
template <int NT, int EMAX>
__device__ __forceinline__ uint32_t tie_cutoff(const uint32_t (&key)[EMAX], int i0, uint32_t T,
                                               uint32_t krem, SelectSmem<NT> &sm) {
  uint32_t eq = 0;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) eq += key[e] == T;
  const uint32_t incl = block_incl_scan<NT>(eq, sm.wave_tot);
  uint32_t before = incl - eq;
  if (before < krem && incl >= krem) {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (key[e] == T) {
        ++before;
        if (before == krem) sm.bin = static_cast<uint32_t>(i0 + e);
      }
    }
  }
  __syncthreads();
  const uint32_t cut = sm.bin;
  __syncthreads();
  return cut;
}

// Keys of the channels [t·E, t·E + E) of a row (E a multiple of 4, d a
// multiple of 4, row 16-byte aligned), read with 16-byte loads that are all
// issued before any is used. Slots past d get kNoKey; v gets the values.
template <int EMAX>
__device__ __forceinline__ void load_keys4(const float *row, int d, int E, uint32_t (&key)[EMAX],
                                           float (&v)[EMAX]) {
  const int i0 = static_cast<int>(threadIdx.x) * E;
#pragma unroll
  for (int q = 0; q < EMAX / 4; ++q) {
    const int i = i0 + 4 * q < d ? i0 + 4 * q : d - 4;
    const float4 f = *reinterpret_cast<const float4 *>(row + i);
    v[4 * q] = f.x;
    v[4 * q + 1] = f.y;
    v[4 * q + 2] = f.z;
    v[4 * q + 3] = f.w;
  }
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const bool here = e < E && i0 + e < d;
    key[e] = here ? (__float_as_uint(v[e]) & 0x7FFFFFFFu) : kNoKey;
    v[e] = here ? v[e] : 0.f;
  }
}

// Slots per thread for d channels over NT threads: a multiple of 4.
__host__ __device__ constexpr int slots_per_thread(int d, int NT) {
  return (((d + NT - 1) / NT) + 3) / 4 * 4;
}

// Kept flags and ascending output positions of the thread's slots, which
// hold consecutive channels. Slot e is kept iff key > T, or key == T and
// fewer than krem equal keys precede it. Returns the number of kept
// channels owned by lower threads (the position of the first kept slot).
template <int NT, int EMAX>
__device__ __forceinline__ void kept_flags(const uint32_t (&key)[EMAX], uint32_t T, uint32_t krem,
                                           SelectSmem<NT> &sm, bool (&kept)[EMAX],
                                           uint32_t &pos0) {
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    if (key[e] & kNoKey) continue;
    gt += key[e] > T;
    eq += key[e] == T;
  }
  const uint32_t packed = (gt << 16) | eq;  // each count <= 32768
  const uint32_t excl = block_incl_scan<NT>(packed, sm.wave_tot) - packed;
  const uint32_t g0 = excl >> 16;
  uint32_t qe = excl & 0xFFFFu;
  pos0 = g0 + (qe < krem ? qe : krem);
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    bool kp = false;
    if (!(key[e] & kNoKey)) {
      if (key[e] > T) {
        kp = true;
      } else if (key[e] == T) {
        kp = qe < krem;
        ++qe;
      }
    }
    kept[e] = kp;
  }
}

}  // namespace larosa
