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

// Bin counted for slots that hold no channel (never searched).
constexpr int kDummyBin = 2048;

template <int NT> struct SelectSmem {
  uint32_t hist[2048 + 64 + 4];  // 2048 padded bins, then the dummy bin
  uint32_t wave_tot[NT / kWave];
  uint32_t bin, above, count;
};

// Inclusive scan over the NT threads of the block (thread order). With
// trailing_barrier == false the caller must place a barrier before wave_tot
// is written again.
template <int NT>
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, uint32_t *wave_tot,
                                                    bool trailing_barrier = true) {
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  uint32_t x = wave_incl_scan(v, lane);
  if (lane == kWave - 1) wave_tot[w] = x;
  __syncthreads();
  uint32_t off = 0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) off += i < w ? wave_tot[i] : 0u;
  if (trailing_barrier) __syncthreads();  // wave_tot may be rewritten by the next scan
  return x + off;
}

// Suffix search over the 2048 bins in sm.hist by the whole block: the bin
// holding the krem-th largest key and the number of keys in higher bins,
// left in sm.bin and sm.above (sm.count: that bin's count). Thread t owns
// the 2048/NT consecutive bins just below bin 2048 − t·(2048/NT), so thread
// order runs from the highest bin down; one block scan of the per-thread
// sums finds the thread whose bins cross krem (exactly one thread has
// excl < krem <= incl when 1 <= krem <= total), which then walks its own
// bins. Requires 1 <= krem <= the number of counted keys; otherwise the
// result is bin 0 with nothing above it (in range, but meaningless).
template <int NT>
__device__ __forceinline__ void suffix_search(uint32_t krem, SelectSmem<NT> &sm) {
  static_assert(2048 % NT == 0 && NT <= 2048, "block size must divide 2048");
  constexpr int BP = 2048 / NT;
  const int top = 2047 - static_cast<int>(threadIdx.x) * BP;  // highest bin of this thread
  if (threadIdx.x == 0) {  // ordered before the crossing thread's write by the scan's barriers
    sm.bin = 0u;
    sm.above = 0u;
    sm.count = 0u;
  }
  uint32_t h[BP];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < BP; ++i) {
    h[i] = sm.hist[pad_bin(top - i)];
    s += h[i];
  }
  // no trailing barrier: the one closing this function comes first
  const uint32_t incl = block_incl_scan<NT>(s, sm.wave_tot, false);
  uint32_t above = incl - s;
  if (above < krem && incl >= krem) {
#pragma unroll
    for (int i = 0; i < BP; ++i) {
      if (above < krem && above + h[i] >= krem) {
        sm.bin = static_cast<uint32_t>(top - i);
        sm.above = above;
        sm.count = h[i];
      }
      above += h[i];
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
// With clear_hist the histogram is also zeroed (before the closing barrier),
// ready for the next pass's counts.
template <int NT>
__device__ __forceinline__ uint32_t radix_resolve(int pass, uint32_t &prefix, uint32_t &pmask,
                                                  uint32_t &krem, SelectSmem<NT> &sm,
                                                  bool clear_hist = false) {
  suffix_search<NT>(krem, sm);
  prefix |= sm.bin << radix_shift(pass);
  pmask |= radix_dmask(pass) << radix_shift(pass);
  krem -= sm.above;
  const uint32_t count = sm.count;
  if (clear_hist) radix_clear<NT>(sm);
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

// ---- Exact rule from a short candidate list ------------------------------
// After the first digit, only the channels whose first digit equals the
// boundary digit can still be in or out; on typical activations they are a
// few hundred. They are compacted (in index order) into LDS, and the later
// digits and the tie cut-off are resolved on that list with one or two
// entries per thread instead of every slot of every thread.
constexpr int kCandMax = 2048;

struct CandSmem {
  uint32_t key[kCandMax];
  uint32_t idx[kCandMax];
};

// The exact Top-k rule of the keys held by the block (slots [0, E) of each
// thread hold channels i0 + e; other slots and slots past d hold kNoKey):
// channel i with key κ is kept iff κ > T, or κ == T and i <= cut. Requires
// 1 <= k <= the number of channels. Taken in two steps so that a caller can
// act on the first digit (every channel whose first digit is above the
// boundary digit is kept) before the rest is resolved.
struct RuleState {
  uint32_t prefix, pmask, krem, n_cand;
};

// Step 1: the first digit (key bits 30..20) over every slot. The boundary
// digit is st.prefix >> 20; st.n_cand channels share it.
//
// With COPIES > 1 the counts go to COPIES histograms in `copies` (LDS that
// is free during this step, COPIES·kHistStride words, 16-byte aligned; lane
// l counts into copy l % COPIES) and are then summed into sm.hist. Keys
// crowd a few dozen first-digit bins, and an LDS atomic serialises the
// lanes of a wave that hit one word; spread over the copies, those lanes
// mostly hit different words in different banks.
constexpr int kHistWords = 2048 + 64 + 4;  // the words of SelectSmem::hist
constexpr int kHistStride = 2120;          // >= kHistWords, 8 (mod 32): a bin's copies in different banks

// Copies (at most 4) that fit in `words` words of free LDS; 1 counts into
// sm.hist alone.
__host__ __device__ constexpr int hist_copies_for(int words) {
  return words >= 4 * kHistStride ? 4 : (words >= 3 * kHistStride ? 3 : (words >= 2 * kHistStride ? 2 : 1));
}

template <int NT, int EMAX, int COPIES = 1>
__device__ __forceinline__ RuleState rule_first_digit(const uint32_t (&key)[EMAX], int E,
                                                      uint32_t k, SelectSmem<NT> &sm,
                                                      uint32_t *copies = nullptr) {
  static_assert(sizeof(sm.hist) == kHistWords * sizeof(uint32_t), "histogram size");
  static_assert(kHistStride >= kHistWords && kHistStride % 4 == 0, "copy stride");
  uint32_t *hist = sm.hist;
  if constexpr (COPIES > 1) {
    for (int i = threadIdx.x; i < COPIES * kHistStride / 4; i += NT)
      reinterpret_cast<uint4 *>(copies)[i] = make_uint4(0u, 0u, 0u, 0u);
    hist = copies + (threadIdx.x % COPIES) * kHistStride;
  } else {
    radix_clear<NT>(sm);
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    if (e < E) {  // empty slots go to the dummy bin
      const int b = (key[e] & kNoKey) ? kDummyBin : static_cast<int>(key[e] >> radix_shift(0));
      atomicAdd(&hist[pad_bin(b)], 1u);
    }
  }
  __syncthreads();
  if constexpr (COPIES > 1) {
    for (int i = threadIdx.x; i < kHistWords; i += NT) {
      uint32_t s = 0;
#pragma unroll
      for (int c = 0; c < COPIES; ++c) s += copies[c * kHistStride + i];
      sm.hist[i] = s;
    }
    __syncthreads();
  }
  RuleState st{0u, kNoKey, k, 0u};
  // the histogram comes back cleared for rule_finish's second digit
  st.n_cand = radix_resolve<NT>(0, st.prefix, st.pmask, st.krem, sm, true);
  return st;
}

// Step 2: the later digits and the tie cut-off. Every thread gets T and cut.
template <int NT, int EMAX>
__device__ __forceinline__ void rule_finish(const uint32_t (&key)[EMAX], int E, int i0,
                                            RuleState st, SelectSmem<NT> &sm, CandSmem &cs,
                                            uint32_t &T, uint32_t &cut) {
  static_assert(kCandMax % NT == 0, "candidates per thread must be whole");
  constexpr int CPT = kCandMax / NT;
  const int t = threadIdx.x;
  uint32_t prefix = st.prefix, pmask = st.pmask, krem = st.krem;
  const uint32_t n_cand = st.n_cand;
  if (n_cand > static_cast<uint32_t>(kCandMax)) {
    // many equal first digits (tie-heavy data): the later digits on the slots
    uint32_t n_eq;
    radix_threshold_from<NT, EMAX>(key, 1, prefix, pmask, krem, sm, T, krem, n_eq);
    cut = tie_cutoff<NT, EMAX>(key, i0, T, krem, sm);
    return;
  }
  // The second digit straight from the slots (sm.hist arrives cleared from
  // rule_first_digit): no candidate list is needed in the usual case.
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) radix_count<NT>(key[e], 1, prefix, pmask, sm);
  __syncthreads();
  const uint32_t in_bin = radix_resolve<NT>(1, prefix, pmask, krem, sm);
  if (in_bin == 1) {
    // One channel carries the boundary's first two digits (the usual case):
    // its key is T and no other channel has that key, so it is the last one
    // kept (krem == 1) and the third digit and the tie cut-off are not needed.
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (e < E && (key[e] & pmask) == prefix) {
        sm.bin = key[e];
        sm.above = static_cast<uint32_t>(i0 + e);
      }
    }
    __syncthreads();
    T = sm.bin;
    cut = sm.above;
    __syncthreads();
    return;
  }
  // Otherwise the channels with these two digits, compacted in index order
  // (at most n_cand <= kCandMax of them), take the third digit and the cut.
  uint32_t nc = 0;
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) nc += (key[e] & pmask) == prefix;
  uint32_t n2;
  {
    const uint32_t incl = block_incl_scan<NT>(nc, sm.wave_tot);
    uint32_t p = incl - nc;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (e < E && (key[e] & pmask) == prefix) {
        cs.key[p] = key[e];
        cs.idx[p] = static_cast<uint32_t>(i0 + e);
        ++p;
      }
    }
    if (t == NT - 1) sm.count = incl;
  }
  radix_clear<NT>(sm);
  __syncthreads();
  n2 = sm.count;
  for (int j = t; j < static_cast<int>(n2); j += NT) radix_count<NT>(cs.key[j], 2, prefix, pmask, sm);
  __syncthreads();
  radix_resolve<NT>(2, prefix, pmask, krem, sm);
  const uint32_t n_cand2 = n2;
  T = prefix;
  // the krem-th candidate equal to T in index order is the last one kept
  uint32_t eq = 0;
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int j = t * CPT + c;
    eq += j < static_cast<int>(n_cand2) && cs.key[j] == T;
  }
  const uint32_t incl = block_incl_scan<NT>(eq, sm.wave_tot);
  uint32_t before = incl - eq;
  if (before < krem && incl >= krem) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int j = t * CPT + c;
      if (j < static_cast<int>(n_cand2) && cs.key[j] == T) {
        ++before;
        if (before == krem) sm.bin = cs.idx[j];
      }
    }
  }
  __syncthreads();
  cut = sm.bin;
  __syncthreads();
}

// Whether slot e (channel i0 + e) is kept under the rule (T, cut).
template <int EMAX>
__device__ __forceinline__ bool rule_keeps(const uint32_t (&key)[EMAX], int e, int E, int i0,
                                           uint32_t T, uint32_t cut) {
  return e < E && !(key[e] & kNoKey) &&
         (key[e] > T || (key[e] == T && static_cast<uint32_t>(i0 + e) <= cut));
}

}  // namespace larosa
