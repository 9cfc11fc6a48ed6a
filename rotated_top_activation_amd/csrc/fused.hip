// Fused rotated sparse linear for one token (B = 1) in a single persistent
// launch: rotate (stage 1 of the LaRoSA summary page, 方法详解 · 技术框架),
// Top-K select (stage 2), and the product over the kept rows of the folded
// weight (the transfer saving named in the LaRoSA abstract).
//
// Every workgroup of the grid is resident at once (the grid is sized from
// the occupancy of this kernel), and the phases hand over through memory:
//   1. rotate: output channel j is owned by one wave, which writes x_rot[j]
//      with an agent-scope atomic store;
//   2. arrival: hierarchical counters (16 groups, then one) find the last
//      workgroup to finish rotating. That workgroup alone selects: an exact
//      radix select over all of x_rot gives the K-th key T, and a scan gives
//      the index cut-off among channels equal to T (lower index first). It
//      then writes (flag, T, cut-off) as one 64-bit word into every other
//      workgroup's own release line, so no two workgroups poll the same
//      address;
//   3. gather: a work unit is (column tile, channel range). It reads its
//      range of x_rot, keeps channel i iff key > T or (key == T and i <=
//      cut-off), lists those rows in LDS, streams them from W', and the last
//      unit of a tile to finish adds the tile's partial sums in split order.
// All counters and flags return to zero, so the workspace is ready for the
// next call. Waits are bounded: a wait that runs past the limit sets an
// error word in the workspace and continues instead of hanging.
#include "common.hpp"
#include "launch.hpp"
#include "select_core.hpp"

namespace larosa {
namespace {

constexpr int kFT = 512;              // threads per workgroup
constexpr int kFW = kFT / kWave;      // waves per workgroup
constexpr int kFRows = 8;             // rows per wave group
constexpr int kFSplitLoads = 32;      // partial sums fetched per round trip
constexpr int kGroups = 16;           // arrival sub-counters
constexpr uint32_t kSpinLimit = 1u << 22;

// Word offsets inside the synchronisation block (each on its own 128-byte
// line): [0] top arrival count, [32·(1+g)] arrival count of group g, [32·17]
// error word.
constexpr int kErrWord = 32 * (kGroups + 1);

struct FusedSmem {
  SelectSmem<kFT> sel;
  float red[kFW][kWave * 8];
  int32_t rows[kFusedMaxRowsPerUnit];
  float coef[kFusedMaxRowsPerUnit];
  uint32_t T, cut;
  int flag;
};

// Arrival at the grid barrier; true in exactly one workgroup (the last).
__device__ __forceinline__ bool arrive_last(uint32_t *sync, int *s_flag) {
  const uint32_t G = gridDim.x;
  __builtin_amdgcn_s_waitcnt(0);  // this workgroup's stores and atomics have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t g = blockIdx.x % kGroups;
    const uint32_t members = (G - g + kGroups - 1) / kGroups;
    const uint32_t groups = G < kGroups ? G : kGroups;
    bool last = false;
    const uint32_t prev = __hip_atomic_fetch_add(&sync[32 * (1 + g)], 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    if (prev == members - 1) {
      const uint32_t top =
          __hip_atomic_fetch_add(&sync[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = top == groups - 1;
    }
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

template <int EMAX, typename T>
__global__ __launch_bounds__(kFT) void fused_linear_kernel(
    const T *__restrict__ x, const T *__restrict__ qt, const T *__restrict__ wf,
    T *__restrict__ y, int d, int qb, int64_t d_out, int k, float *__restrict__ x_rot,
    uint32_t *__restrict__ sync, uint64_t *__restrict__ flags,
    uint32_t *__restrict__ tile_ctr, float *__restrict__ partials,
    int32_t *__restrict__ idx_out, int tiles, int splits, int chans_per_split) {
  constexpr int V = Elt<T>::kVec;
  constexpr int TILE = kWave * V;
  __shared__ FusedSmem sm;
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

  // ---- 2. arrival; the last workgroup selects and releases the others ----
  if (arrive_last(sync, &sm.flag)) {
    // exact selection over all of x_rot; the acquire fence makes the other
    // workgroups' x_rot stores visible to ordinary (vector) loads here
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const int E = slots_per_thread(d, kFT);
    const int i0 = t * E;
    uint32_t key[EMAX];
    float vv[EMAX];
    load_keys4<EMAX>(x_rot, d, E, key, vv);
    uint32_t T_, krem, n_eq;
    radix_threshold<kFT, EMAX>(key, static_cast<uint32_t>(k), sm.sel, T_, krem, n_eq);
    // channels equal to T are all kept unless there are more than krem
    const uint32_t cut =
        n_eq == krem ? 0xFFFFFFFFu : tie_cutoff<kFT, EMAX>(key, i0, T_, krem, sm.sel);
    // reset the arrival counters: every workgroup has arrived
    if (t <= kGroups)
      __hip_atomic_store(&sync[32 * t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // release: one 64-bit word per workgroup carries the flag bit, T and the
    // cut-off together
    const uint64_t word = (1ull << 63) | (static_cast<uint64_t>(T_) << 32) | cut;
    for (uint32_t b = t; b < G; b += kFT)
      if (b != blockIdx.x)
        __hip_atomic_store(&flags[b * 16], word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t == 0) {
      sm.T = T_;
      sm.cut = cut;
    }
  } else if (t == 0) {
    uint64_t *line = &flags[blockIdx.x * 16];
    uint32_t spins = 0;
    uint64_t word;
    while ((word = __hip_atomic_load(line, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == 0u) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > kSpinLimit) {
        __hip_atomic_store(&sync[kErrWord], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    sm.T = static_cast<uint32_t>(word >> 32) & 0x7FFFFFFFu;
    sm.cut = static_cast<uint32_t>(word);
    __hip_atomic_store(line, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  const uint32_t Tk = sm.T, cut = sm.cut;

  // ---- optional copy of the kept indices (ascending), by workgroup 0 ------
  if (idx_out && blockIdx.x == 0) {
    const int E = (d + kFT - 1) / kFT;
    const int i0 = t * E;
    uint32_t n = 0;
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e;
      if (i >= d) break;
      const uint32_t kk =
          __float_as_uint(__hip_atomic_load(x_rot + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) &
          0x7FFFFFFFu;
      n += kk > Tk || (kk == Tk && static_cast<uint32_t>(i) <= cut);
    }
    uint32_t p = block_incl_scan<kFT>(n, sm.sel.wave_tot) - n;
    for (int e = 0; e < E; ++e) {
      const int i = i0 + e;
      if (i >= d) break;
      const uint32_t kk =
          __float_as_uint(__hip_atomic_load(x_rot + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) &
          0x7FFFFFFFu;
      if (kk > Tk || (kk == Tk && static_cast<uint32_t>(i) <= cut)) idx_out[p++] = i;
    }
  }

  // ---- 3. gather over units (column tile, channel range) -----------------
  const int units = tiles * splits;
  for (int u = blockIdx.x; u < units; u += G) {
    const int tile = u % tiles, split = u / tiles;
    const int c0 = split * chans_per_split;
    const int c1 = c0 + chans_per_split < d ? c0 + chans_per_split : d;
    // kept channels of the range, listed in index order
    constexpr int kPer = kFusedMaxRowsPerUnit / kFT;
    float cv[kPer];
    bool kp[kPer];
    uint32_t n = 0;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int i = c0 + t * kPer + m;
      const int ic = i < c1 ? i : c1 - 1;
      cv[m] = __hip_atomic_load(x_rot + ic, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      const int i = c0 + t * kPer + m;
      const uint32_t kk = __float_as_uint(cv[m]) & 0x7FFFFFFFu;
      kp[m] = i < c1 && (kk > Tk || (kk == Tk && static_cast<uint32_t>(i) <= cut));
      n += kp[m];
    }
    const uint32_t incl = block_incl_scan<kFT>(n, sm.sel.wave_tot);
    uint32_t p = incl - n;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      if (kp[m]) {
        sm.rows[p] = c0 + t * kPer + m;
        sm.coef[p] = cv[m];
        ++p;
      }
    }
    if (t == kFT - 1) sm.flag = static_cast<int>(incl);
    __syncthreads();
    const int nrows = sm.flag;
    const int64_t col_raw = static_cast<int64_t>(tile) * TILE + lane * V;
    const int64_t col = col_raw < d_out ? col_raw : d_out - V;
    float acc[V];
#pragma unroll
    for (int q = 0; q < V; ++q) acc[q] = 0.f;
    for (int base = wave * kFRows; base < nrows; base += kFW * kFRows) {
      int rr[kFRows];
      float c[kFRows];
#pragma unroll
      for (int r = 0; r < kFRows; ++r) {
        const int jl = base + r < nrows ? base + r : nrows - 1;
        rr[r] = __builtin_amdgcn_readfirstlane(sm.rows[jl]);
        c[r] = base + r < nrows ? sm.coef[jl] : 0.f;
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
#pragma unroll
    for (int w = 0; w < V; ++w) sm.red[wave][lane * V + w] = acc[w];
    __syncthreads();
    const int64_t tile_col0 = static_cast<int64_t>(tile) * TILE;
    for (int e = t; e < TILE; e += kFT) {
      const int64_t cg = tile_col0 + e;
      if (cg >= d_out) continue;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kFW; ++w) s += sm.red[w][e];
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
        sm.flag = prev == static_cast<uint32_t>(splits - 1);
      }
      __syncthreads();
      if (sm.flag) {
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

template <int EMAX, typename T>
int resident_blocks() {
  static int cached = -1;
  if (cached < 0) {
    int per_cu = 0, dev = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(&fused_linear_kernel<EMAX, T>), kFT, 0) !=
            hipSuccess ||
        hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 0;
    cached = per_cu * cus;
  }
  return cached;
}

template <int EMAX, typename T>
hipError_t launch_e(const FusedArgs &a, hipStream_t s) {
  int capacity = resident_blocks<EMAX, T>();
  if (capacity <= 0) return hipErrorLaunchFailure;
  if (capacity > kFusedMaxGrid) capacity = kFusedMaxGrid;
  const FusedPlan p = plan_fused(a.d_in, a.d_out, a.k, a.w_dt, capacity);
  char *ws = static_cast<char *>(a.ws);
  uint32_t *sync = reinterpret_cast<uint32_t *>(ws);
  uint32_t *tile_ctr = reinterpret_cast<uint32_t *>(ws + p.tile_off);
  uint64_t *flags = reinterpret_cast<uint64_t *>(ws + p.flags_off);
  float *x_rot = a.xrot_out ? a.xrot_out : reinterpret_cast<float *>(ws + p.xrot_off);
  float *partials = reinterpret_cast<float *>(ws + p.partial_off);
  hipLaunchKernelGGL((fused_linear_kernel<EMAX, T>), dim3(p.grid), dim3(kFT), 0, s,
                     static_cast<const T *>(a.x), static_cast<const T *>(a.qt),
                     static_cast<const T *>(a.wf), static_cast<T *>(a.y), a.d_in, a.q_block,
                     a.d_out, a.k, x_rot, sync, flags, tile_ctr, partials, a.idx_out,
                     p.tiles, p.splits, p.chans_per_split);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const FusedArgs &a, hipStream_t s) {
  const int E = slots_per_thread(a.d_in, kFT);
  if (E <= 8) return launch_e<8, T>(a, s);
  if (E <= 16) return launch_e<16, T>(a, s);
  if (E <= 32) return launch_e<32, T>(a, s);
  return hipErrorInvalidValue;
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
  // One unit per workgroup where possible; a unit's channel range must fit
  // its LDS row list.
  int64_t splits = grid / p.tiles;
  if (splits < 1) splits = 1;
  const int64_t min_split = (d_in + kFusedMaxRowsPerUnit - 1) / kFusedMaxRowsPerUnit;
  if (splits < min_split) splits = min_split;
  if (splits > d_in) splits = d_in;
  const int64_t cps = (d_in + splits - 1) / splits;
  p.splits = static_cast<int>((d_in + cps - 1) / cps);
  p.chans_per_split = static_cast<int>(cps);
  p.tile_off = up256(static_cast<size_t>(32 * (kGroups + 2)) * 4);
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
