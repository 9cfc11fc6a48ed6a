// Fused rotated sparse linear for one token (B = 1) in a single persistent
// launch: rotate (stage 1 of the LaRoSA summary page, 方法详解 · 技术框架),
// Top-K select (stage 2), and the product over the kept rows of the folded
// weight (the transfer saving named in the LaRoSA abstract).
//
// The grid is sized from the occupancy of this kernel so that every
// workgroup can be resident at once (an ordinary launch does not guarantee
// it: other work on the GPU can hold CUs, and then the bounded waits below
// give up with a status), and the phases hand over through memory:
//   1. rotate: output channel j is owned by one wave, which writes x_rot[j]
//      with an agent-scope atomic store. Every workgroup takes part.
//   2. select: workgroup 0 is the selector. It waits until every other
//      workgroup has written its arrival slot and tells them so, then
//      copies the magnitude keys of x_rot into LDS and runs an exact radix
//      select over them. After the first digit it already knows
//      the bin B0 (key bits 30..20) holding the K-th largest key: every
//      channel in a higher bin is kept whatever the rest of the select
//      finds. It releases that preliminary rule at once, then finishes the
//      select (the K-th key T, and the index cut-off among channels equal to
//      T, lower index first) and releases the exact rule. Each release is
//      one 64-bit word written into every workgroup's own 128-byte line, so
//      no two workgroups poll the same address. The selector's code runs
//      once per launch on one workgroup, so it is kept short (rolled loops
//      over LDS) to limit cold instruction fetches.
//   3. gather (workgroups 1..G-1): a work unit is (column tile, channel
//      range). A workgroup loads its first unit's slice of x_rot as soon as
//      every rotation is in, and lists on the preliminary rule the channels
//      of the range above bin B0 and those inside it; it streams the first
//      list's rows of W' at once, and appends the kept channels of B0 to the
//      list when the exact rule is in (the first wave to run out of certain
//      rows does that for the workgroup). The last unit of a tile to finish
//      adds the tile's partial sums in split order.
// The bin-B0 rows go last in every unit's accumulation whatever the timing,
// so results do not depend on when the exact rule arrives.
//
// Every hand-over word carries the launch's epoch, a 16-bit number (never 0)
// kept on the device, so a captured graph replays correctly. One 64-bit
// control word holds the previous launch's epoch (high half) and a count of
// workgroups (low half): each workgroup adds 1 once (before any wait) and so
// reads the epoch and the count in one atomic; the last one stores the new
// epoch with a zero count. No workgroup can read the word after that store,
// so every workgroup of a launch has the same epoch even if waits give up.
// A worker arrives by writing the epoch into its own slot, and a release
// counts only with the current epoch, so nothing has to be reset between
// calls. Waits are bounded (the spin limit is a kernel argument): a wait that
// runs past the limit writes LAROSA_ERR_TIMEOUT into the workspace's status
// word and continues with a fallback (an in-bounds but wrong result) instead
// of hanging, and leaves nothing that the next launch could take as its own.
#include "common.hpp"
#include "launch.hpp"
#include "select_core.hpp"

#include <cstddef>
#include <mutex>

namespace larosa {
namespace {

constexpr int kFT = 512;              // threads per workgroup
constexpr int kFW = kFT / kWave;      // waves per workgroup
constexpr int kFRows = 8;             // rows per wave group
constexpr int kFSplitLoads = 32;      // partial sums fetched per round trip
constexpr int kChunks = kFusedMaxD / (4 * kFT);  // 16-byte key chunks per selector thread

// Release words: bits 63..48 the launch's epoch, bits 47..46 the stage.
//   stage 0 (all rotations are in): nothing else
//   stage 1 (preliminary rule):     bits 10..0 = B0
//   stage 2 (exact rule):           bits 45..15 = T, bits 14..0 = cut-off
//                                   (0x7FFF: every channel equal to T;
//                                   d <= 16384, so a real cut-off is lower)
constexpr int kEpochShift = 48;
constexpr int kStageShift = 46;
constexpr uint32_t kCutAll = 0x7FFFu;

__device__ __forceinline__ uint64_t make_word(uint32_t epoch, uint32_t stage, uint64_t payload) {
  return (static_cast<uint64_t>(epoch) << kEpochShift) | (static_cast<uint64_t>(stage) << kStageShift) |
         payload;
}
__device__ __forceinline__ uint32_t word_epoch(uint64_t w) { return static_cast<uint32_t>(w >> kEpochShift); }
__device__ __forceinline__ uint32_t word_stage(uint64_t w) {
  return static_cast<uint32_t>(w >> kStageShift) & 3u;
}

__device__ __forceinline__ void report_timeout(uint32_t *status) {
  __hip_atomic_store(status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct WorkerSmem {
  float red[kFW][kWave * 8];
  int32_t rows[kFusedMaxRowsPerUnit];     // kept rows: certain ones, then bin B0's
  float coef[kFusedMaxRowsPerUnit];
  int32_t crow[kFusedMaxRowsPerUnit];     // channels of bin B0
  float ccoef[kFusedMaxRowsPerUnit];
  uint32_t wave_tot[kFW];
};

struct SelectorSmem {
  SelectSmem<kFT> sel;
  alignas(16) uint32_t key[4];  // d keys (the launch's dynamic LDS extends the array)
};

struct FusedSmem {
  uint32_t ns, nc;          // certain rows / bin-B0 channels of the unit
  uint32_t claim, tail;     // bin-B0 compaction: claimed; done (count + 1)
  uint32_t last;            // this unit is the last of its tile
  uint32_t b0, T, cut, stage;
  uint32_t epoch;           // this launch's epoch
  alignas(16) union {
    SelectorSmem s;
    WorkerSmem w;
  };
};

// LDS bytes of one workgroup: the worker's lists or the selector's
// histogram and keys, whichever is larger.
size_t fused_lds_bytes(int d) {
  const size_t sel = offsetof(FusedSmem, s) + offsetof(SelectorSmem, key) + 4 * static_cast<size_t>(d);
  return sel > sizeof(FusedSmem) ? sel : sizeof(FusedSmem);
}

__device__ __forceinline__ uint32_t lds_load(uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(uint32_t *p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Decodes a release word into sm.
__device__ __forceinline__ void take_word(uint64_t w, FusedSmem &sm) {
  const uint32_t stage = word_stage(w);
  if (stage == 2) {
    const uint32_t T = static_cast<uint32_t>(w >> 15) & 0x7FFFFFFFu;
    const uint32_t c = static_cast<uint32_t>(w) & kCutAll;
    sm.T = T;
    sm.cut = c == kCutAll ? 0xFFFFFFFFu : c;
    sm.b0 = T >> 20;
  } else if (stage == 1) {
    sm.b0 = static_cast<uint32_t>(w) & 0x7FFu;
  }
  lds_store(&sm.stage, stage);
}

// Polls this workgroup's release line until a word of this launch's epoch
// and at least `stage` arrives (bounded); decodes it into sm.
__device__ __forceinline__ void wait_word(uint64_t *line, uint32_t stage, uint32_t epoch,
                                          uint32_t spin_limit, uint32_t *status, FusedSmem &sm) {
  uint32_t spins = 0;
  uint64_t w;
  for (;;) {
    w = __hip_atomic_load(line, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (word_epoch(w) == epoch && word_stage(w) >= stage) break;
    if (spins++ >= spin_limit) {
      report_timeout(status);
      w = make_word(epoch, 2, 0);  // T = 0, cut = 0: keeps every channel of a unit
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  take_word(w, sm);
}

__device__ __forceinline__ void release_all(uint64_t *flags, uint64_t w) {
  for (uint32_t b = 1 + threadIdx.x; b < gridDim.x; b += kFT)
    __hip_atomic_store(&flags[b * 16], w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One radix pass over the selector's LDS keys (rolled loop: 16-byte reads,
// consecutive across the workgroup).
__device__ __forceinline__ uint32_t selector_pass(int pass, const uint32_t *key, int d,
                                                  uint32_t &prefix, uint32_t &pmask,
                                                  uint32_t &krem, SelectSmem<kFT> &sel) {
  radix_clear<kFT>(sel);
  __syncthreads();
#pragma unroll 1
  for (int i = 4 * static_cast<int>(threadIdx.x); i < d; i += 4 * kFT) {
    const uint4 q = *reinterpret_cast<const uint4 *>(key + i);
    radix_count<kFT>(q.x, pass, prefix, pmask, sel);
    radix_count<kFT>(q.y, pass, prefix, pmask, sel);
    radix_count<kFT>(q.z, pass, prefix, pmask, sel);
    radix_count<kFT>(q.w, pass, prefix, pmask, sel);
  }
  __syncthreads();
  return radix_resolve<kFT>(pass, prefix, pmask, krem, sel);
}

// Selector (workgroup 0): waits for the arrivals, selects, releases.
__device__ __forceinline__ void select_and_release(const float *x_rot, int d, int k,
                                                   const uint32_t *arrive, uint64_t *flags,
                                                   int32_t *idx_out, uint32_t epoch,
                                                   uint32_t spin_limit, uint32_t *status,
                                                   FusedSmem &sm) {
  const int t = threadIdx.x;
  const uint32_t G = gridDim.x;
  SelectSmem<kFT> &sel = sm.s.sel;
  uint32_t *key = sm.s.key;
  if (t < kWave) {
    // every worker writes this launch's epoch into its own slot on arrival
    uint32_t spins = 0;
    for (;;) {
      bool in = true;
      for (uint32_t b = 1 + t; b < G; b += kWave)
        in = in && __hip_atomic_load(&arrive[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch;
      if (__all(in)) break;
      if (spins++ >= spin_limit) {
        if (t == 0) report_timeout(status);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  release_all(flags, make_word(epoch, 0, 0));  // stage 0: x_rot is complete
  // the acquire fence makes the workers' x_rot stores visible to ordinary
  // (vector) loads here
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  {
    // keys into LDS: every 16-byte load in flight before any is used
    float4 f[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int i = 4 * (c * kFT + t);
      if (i < d) f[c] = *reinterpret_cast<const float4 *>(x_rot + i);
    }
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int i = 4 * (c * kFT + t);
      if (i < d)
        *reinterpret_cast<uint4 *>(key + i) =
            make_uint4(__float_as_uint(f[c].x) & 0x7FFFFFFFu, __float_as_uint(f[c].y) & 0x7FFFFFFFu,
                       __float_as_uint(f[c].z) & 0x7FFFFFFFu, __float_as_uint(f[c].w) & 0x7FFFFFFFu);
    }
  }

  // first digit: bin B0 of the K-th largest key; release the preliminary rule
  uint32_t prefix = 0, pmask = kNoKey, krem = static_cast<uint32_t>(k);
  selector_pass(0, key, d, prefix, pmask, krem, sel);  // its first barrier covers the key stores
  release_all(flags, make_word(epoch, 1, prefix >> 20));

  // remaining digits: T, and the count of keys equal to T
  uint32_t n_eq = 0;
#pragma unroll 1
  for (int pass = 1; pass < 3; ++pass) n_eq = selector_pass(pass, key, d, prefix, pmask, krem, sel);
  const uint32_t T = prefix;

  // Thread t owns the E consecutive channels [t·E, t·E + E) for the index-
  // order steps below.
  const int E = (d + kFT - 1) / kFT;
  const int i0 = t * E;
  const int i1 = i0 + E < d ? i0 + E : d;
  // index cut-off among the channels equal to T: the krem-th of them
  uint32_t cut = kCutAll;
  if (n_eq != krem) {
    uint32_t eq = 0;
#pragma unroll 1
    for (int i = i0; i < i1; ++i) eq += key[i] == T;
    const uint32_t incl = block_incl_scan<kFT>(eq, sel.wave_tot);
    uint32_t r = incl - eq;
    if (r < krem && incl >= krem) {
#pragma unroll 1
      for (int i = i0; i < i1; ++i)
        if (key[i] == T && ++r == krem) sel.bin = static_cast<uint32_t>(i);
    }
    __syncthreads();
    cut = sel.bin;
  }
  __builtin_amdgcn_s_waitcnt(0);  // earlier words are out first
  release_all(flags, make_word(epoch, 2, (static_cast<uint64_t>(T) << 15) | cut));

  // optional copy of the kept indices, ascending
  if (idx_out) {
    const uint32_t cut32 = cut == kCutAll ? 0xFFFFFFFFu : cut;
    uint32_t n = 0;
#pragma unroll 1
    for (int i = i0; i < i1; ++i)
      n += key[i] > T || (key[i] == T && static_cast<uint32_t>(i) <= cut32);
    uint32_t p = block_incl_scan<kFT>(n, sel.wave_tot) - n;
#pragma unroll 1
    for (int i = i0; i < i1; ++i)
      if (key[i] > T || (key[i] == T && static_cast<uint32_t>(i) <= cut32)) idx_out[p++] = i;
  }
}

// Streams rows[base .. base + kFRows) (clamped to n) of W' into acc.
template <typename T>
__device__ __forceinline__ void gather_group(const T *__restrict__ wf, int64_t d_out, int64_t col,
                                             const int32_t *rows, const float *coef, int base,
                                             int n, float (&acc)[Elt<T>::kVec]) {
  constexpr int V = Elt<T>::kVec;
  int rr[kFRows];
  float c[kFRows];
#pragma unroll
  for (int r = 0; r < kFRows; ++r) {
    const int jl = base + r < n ? base + r : n - 1;
    rr[r] = __builtin_amdgcn_readfirstlane(rows[jl]);
    c[r] = base + r < n ? coef[jl] : 0.f;
  }
  uint4 q[kFRows];
#pragma unroll
  for (int r = 0; r < kFRows; ++r) q[r] = load16(wf + static_cast<int64_t>(rr[r]) * d_out + col);
#pragma unroll
  for (int r = 0; r < kFRows; ++r) {
    float f[V];
    Elt<T>::unpack(q[r], f);
#pragma unroll
    for (int w = 0; w < V; ++w) acc[w] = fmaf(c[r], f[w], acc[w]);
  }
}

template <typename T>
__global__ __launch_bounds__(kFT) void fused_linear_kernel(
    const T *__restrict__ x, const T *__restrict__ qt, const T *__restrict__ wf,
    T *__restrict__ y, int d, int qb, int64_t d_out, int k, float *__restrict__ x_rot,
    uint32_t *__restrict__ arrive, uint64_t *__restrict__ ctl, uint64_t *__restrict__ flags,
    uint32_t *__restrict__ tile_ctr, float *__restrict__ partials,
    int32_t *__restrict__ idx_out, int tiles, int splits, int chans_per_split,
    uint32_t spin_limit, uint32_t *__restrict__ status) {
  constexpr int V = Elt<T>::kVec;
  constexpr int TILE = kWave * V;
  extern __shared__ __align__(16) unsigned char fused_lds[];
  FusedSmem &sm = *reinterpret_cast<FusedSmem *>(fused_lds);
  const int t = threadIdx.x;
  const int lane = t % kWave;
  const int wave = wave_id();
  const uint32_t G = gridDim.x;

  // ---- 1. rotate: x_rot[j] = Σ_i x[blk(j)·qb + i] · Qt[j, i] -------------
  const int chunks = qb / V;
  for (int j = blockIdx.x * kFW + wave; j < d; j += G * kFW) {
    const int64_t xoff = static_cast<int64_t>(j / qb) * qb;
    float acc = 0.f;
#pragma unroll 4
    for (int c = lane; c < chunks; c += kWave) {
      float qf[V], xf[V];
      Elt<T>::unpack(load16(qt + static_cast<int64_t>(j) * qb + c * V), qf);
      Elt<T>::unpack(load16(x + xoff + c * V), xf);
#pragma unroll
      for (int v = 0; v < V; ++v) acc = fmaf(xf[v], qf[v], acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) __hip_atomic_store(x_rot + j, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // this workgroup's x_rot stores have completed
  // this launch's epoch (1 .. 65535) and the workgroup count in one atomic;
  // the last workgroup to count stores the epoch for the next launch
  if (t == 0) {
    const uint64_t old = __hip_atomic_fetch_add(ctl, uint64_t{1}, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t e = static_cast<uint32_t>(old >> 32) % 65535u + 1u;
    sm.epoch = e;
    if (static_cast<uint32_t>(old) == G - 1)
      __hip_atomic_store(ctl, static_cast<uint64_t>(e) << 32, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const uint32_t epoch = sm.epoch;

  // ---- 2. selector ---------------------------------------------------------
  if (blockIdx.x == 0) {
    select_and_release(x_rot, d, k, arrive, flags, idx_out, epoch, spin_limit, status, sm);
    return;
  }

  // ---- arrival; the first unit's slice of x_rot once every rotation is in,
  // then the preliminary (or already the exact) rule ------------------------
  uint64_t *line = &flags[blockIdx.x * 16];
  if (t == 0) {
    __hip_atomic_store(&arrive[blockIdx.x], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_word(line, 0, epoch, spin_limit, status, sm);
  }
  __syncthreads();
  const uint32_t W = G - 1;
  const int units = tiles * splits;
  constexpr int kPer = kFusedMaxRowsPerUnit / kFT;
  float cv[kPer];
  auto load_slice = [&](int u) {
    const int c0 = (u / tiles) * chans_per_split;
    const int c1 = c0 + chans_per_split < d ? c0 + chans_per_split : d;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int i = c0 + t * kPer + m;
      const int ic = i < c1 ? i : c1 - 1;
      cv[m] = __hip_atomic_load(x_rot + ic, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  if (static_cast<int>(blockIdx.x) - 1 < units) load_slice(blockIdx.x - 1);
  if (t == 0 && lds_load(&sm.stage) < 1) wait_word(line, 1, epoch, spin_limit, status, sm);
  __syncthreads();

  // ---- 3. gather over units (column tile, channel range) -----------------
  for (int u = blockIdx.x - 1; u < units; u += W) {
    const int tile = u % tiles, split = u / tiles;
    const int c0 = split * chans_per_split;
    const int c1 = c0 + chans_per_split < d ? c0 + chans_per_split : d;
    const uint32_t b0 = sm.b0;
    if (u != static_cast<int>(blockIdx.x) - 1) load_slice(u);
    // certain rows (bin above B0) and bin-B0 channels of the range, in index
    // order
    uint32_t cls[kPer];  // 2: certain, 1: bin B0, 0: dropped
    uint32_t cnt = 0;    // certain count (low half) and bin-B0 count (high half)
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int i = c0 + t * kPer + m;
      const uint32_t bin = (__float_as_uint(cv[m]) & 0x7FFFFFFFu) >> 20;
      cls[m] = i >= c1 ? 0u : (bin > b0 ? 2u : (bin == b0 ? 1u : 0u));
      cnt += cls[m] == 2u ? 1u : (cls[m] == 1u ? 0x10000u : 0u);
    }
    const uint32_t incl = block_incl_scan<kFT>(cnt, sm.w.wave_tot);
    uint32_t ps = (incl - cnt) & 0xFFFFu, pc = (incl - cnt) >> 16;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int i = c0 + t * kPer + m;
      if (cls[m] == 2u) {
        sm.w.rows[ps] = i;
        sm.w.coef[ps] = cv[m];
        ++ps;
      } else if (cls[m] == 1u) {
        sm.w.crow[pc] = i;
        sm.w.ccoef[pc] = cv[m];
        ++pc;
      }
    }
    if (t == kFT - 1) {
      sm.ns = incl & 0xFFFFu;
      sm.nc = incl >> 16;
      sm.claim = 0;
      sm.tail = 0;
    }
    __syncthreads();
    const int ns = static_cast<int>(sm.ns), nc = static_cast<int>(sm.nc);
    const int64_t col_raw = static_cast<int64_t>(tile) * TILE + lane * V;
    const int64_t col = col_raw < d_out ? col_raw : d_out - V;
    float acc[V];
#pragma unroll
    for (int q = 0; q < V; ++q) acc[q] = 0.f;

    // full groups of certain rows: group g goes to wave g mod kFW
    const int full = ns / kFRows;
    for (int g = wave; g < full; g += kFW)
      gather_group<T>(wf, d_out, col, sm.w.rows, sm.w.coef, g * kFRows, ns, acc);

    // tail: the last partial group of certain rows, then the kept bin-B0
    // channels, appended after them by the first wave to get here
    int n = ns;
    if (nc > 0) {
      uint32_t won = 0;
      if (lane == 0) {
        uint32_t expected = 0;
        won = __hip_atomic_compare_exchange_strong(&sm.claim, &expected, 1u, __ATOMIC_RELAXED,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      won = __shfl(won, 0, kWave);
      if (won) {
        if (lane == 0 && lds_load(&sm.stage) < 2)
          wait_word(line, 2, epoch, spin_limit, status, sm);
        __builtin_amdgcn_wave_barrier();
        const uint32_t Tk = __shfl(lane == 0 ? sm.T : 0u, 0, kWave);
        const uint32_t cut = __shfl(lane == 0 ? sm.cut : 0u, 0, kWave);
        uint32_t m = static_cast<uint32_t>(ns);
        for (int b = 0; b < nc; b += kWave) {
          const int i = b + lane;
          const int ic = i < nc ? i : nc - 1;
          const int32_t row = sm.w.crow[ic];
          const float v = sm.w.ccoef[ic];
          const uint32_t kk = __float_as_uint(v) & 0x7FFFFFFFu;
          const bool kp = i < nc && (kk > Tk || (kk == Tk && static_cast<uint32_t>(row) <= cut));
          const uint64_t mask = __ballot(kp);
          const uint32_t rank = __builtin_amdgcn_mbcnt_hi(
              static_cast<uint32_t>(mask >> 32),
              __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
          if (kp) {
            sm.w.rows[m + rank] = row;
            sm.w.coef[m + rank] = v;
          }
          m += static_cast<uint32_t>(__popcll(mask));
        }
        __builtin_amdgcn_s_waitcnt(0);
        if (lane == 0) lds_store(&sm.tail, m + 1);
      }
      uint32_t tn, spins = 0;
      while ((tn = lds_load(&sm.tail)) == 0u) {
        if (spins++ >= spin_limit) {
          if (lane == 0) report_timeout(status);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      n = tn > 0 ? static_cast<int>(tn - 1) : ns;
    }
    const int ng = (n + kFRows - 1) / kFRows;
    for (int g = full + ((wave - full % kFW) + kFW) % kFW; g < ng; g += kFW)
      gather_group<T>(wf, d_out, col, sm.w.rows, sm.w.coef, g * kFRows, n, acc);

#pragma unroll
    for (int w = 0; w < V; ++w) sm.w.red[wave][lane * V + w] = acc[w];
    __syncthreads();
    const int64_t tile_col0 = static_cast<int64_t>(tile) * TILE;
    for (int e = t; e < TILE; e += kFT) {
      const int64_t cg = tile_col0 + e;
      if (cg >= d_out) continue;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kFW; ++w) s += sm.w.red[w][e];
      if (splits == 1) {
        Elt<T>::store(y, cg, s);
      } else {
        const float old = __hip_atomic_exchange(partials + static_cast<int64_t>(split) * d_out + cg,
                                                s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        (void)old;
      }
    }
    if (splits > 1) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t == 0) {
        const uint32_t prev =
            __hip_atomic_fetch_add(&tile_ctr[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm.last = prev == static_cast<uint32_t>(splits - 1);
      }
      __syncthreads();
      if (sm.last) {
        for (int e = t; e < TILE; e += kFT) {
          const int64_t cg = tile_col0 + e;
          if (cg >= d_out) continue;
          float s = 0.f;
          for (int r0 = 0; r0 < splits; r0 += kFSplitLoads) {
            float pv[kFSplitLoads];
#pragma unroll
            for (int i = 0; i < kFSplitLoads; ++i)
              pv[i] = r0 + i < splits
                          ? __hip_atomic_load(partials + static_cast<int64_t>(r0 + i) * d_out + cg,
                                              __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : 0.f;
#pragma unroll
            for (int i = 0; i < kFSplitLoads; ++i)
              if (r0 + i < splits) s += pv[i];
          }
          Elt<T>::store(y, cg, s);
        }
        if (t == 0)
          __hip_atomic_store(&tile_ctr[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();  // LDS lists and reduction buffer are reused by the next unit
  }
}

// Workgroups of the kernel resident at once on the current device, for a
// given LDS size (cached; a few sizes are in use at a time).
template <typename T>
int resident_blocks(size_t lds) {
  struct Entry {
    int dev;
    size_t lds;
    int n;
  };
  static std::mutex mu;
  static Entry cache[16];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < used; ++i)
    if (cache[i].dev == dev && cache[i].lds == lds) return cache[i].n;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void *>(&fused_linear_kernel<T>), kFT, lds) !=
          hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  const int n = per_cu * cus;
  if (used < 16) cache[used++] = Entry{dev, lds, n};
  return n;
}

template <typename T>
hipError_t launch_t(const FusedArgs &a, hipStream_t s) {
  const size_t lds = fused_lds_bytes(a.d_in);
  int capacity = resident_blocks<T>(lds);
  if (capacity < 2) return hipErrorLaunchFailure;
  if (capacity > kFusedMaxGrid) capacity = kFusedMaxGrid;
  const FusedPlan p = plan_fused(a.d_in, a.d_out, a.k, a.w_dt, capacity);
  char *ws = static_cast<char *>(a.ws);
  uint32_t *arrive = reinterpret_cast<uint32_t *>(ws);
  uint64_t *ctl = reinterpret_cast<uint64_t *>(ws + static_cast<size_t>(kFusedMaxGrid) * 4);
  uint32_t *tile_ctr = reinterpret_cast<uint32_t *>(ws + p.tile_off);
  uint64_t *flags = reinterpret_cast<uint64_t *>(ws + p.flags_off);
  float *x_rot = a.xrot_out ? a.xrot_out : reinterpret_cast<float *>(ws + p.xrot_off);
  float *partials = reinterpret_cast<float *>(ws + p.partial_off);
  hipLaunchKernelGGL((fused_linear_kernel<T>), dim3(p.grid), dim3(kFT), lds, s,
                     static_cast<const T *>(a.x), static_cast<const T *>(a.qt),
                     static_cast<const T *>(a.wf), static_cast<T *>(a.y), a.d_in, a.q_block,
                     a.d_out, a.k, x_rot, arrive, ctl, flags, tile_ctr, partials, a.idx_out,
                     p.tiles, p.splits, p.chans_per_split, a.spin_limit, a.status);
  return hipGetLastError();
}

size_t up256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

FusedPlan plan_fused(int64_t d_in, int64_t d_out, int64_t k, int w_dt, int grid) {
  (void)k;
  FusedPlan p;
  const int V = w_dt == kF32 ? 4 : 8;
  const int64_t tile_cols = static_cast<int64_t>(kWave) * V;
  p.grid = grid;
  p.tiles = static_cast<int>((d_out + tile_cols - 1) / tile_cols);
  // One unit per gathering workgroup (all but the selector) where possible;
  // a unit's channel range must fit its LDS row list.
  int64_t splits = (grid - 1) / p.tiles;
  if (splits < 1) splits = 1;
  const int64_t min_split = (d_in + kFusedMaxRowsPerUnit - 1) / kFusedMaxRowsPerUnit;
  if (splits < min_split) splits = min_split;
  if (splits > d_in) splits = d_in;
  const int64_t cps = (d_in + splits - 1) / splits;
  p.splits = static_cast<int>((d_in + cps - 1) / cps);
  p.chans_per_split = static_cast<int>(cps);
  p.tile_off = up256(static_cast<size_t>(kFusedMaxGrid) * 4 + 8);  // arrival slots, control word
  p.flags_off = p.tile_off + up256(static_cast<size_t>(p.tiles) * 4);
  p.xrot_off = p.flags_off + static_cast<size_t>(kFusedMaxGrid) * 128;
  p.partial_off = p.xrot_off + up256(static_cast<size_t>(d_in) * 4);
  p.bytes = p.partial_off + static_cast<size_t>(p.splits > 1 ? p.splits : 0) * d_out * 4;
  return p;
}

bool fused_supported(int64_t B, int64_t d_in, int act_dt, int w_dt) {
  return B == 1 && d_in <= kFusedMaxD && act_dt == w_dt;
}

hipError_t launch_fused_linear(const FusedArgs &a, hipStream_t s) {
  if (a.w_dt == kBF16) return launch_t<uint16_t>(a, s);
  return launch_t<float>(a, s);
}

}  // namespace larosa
