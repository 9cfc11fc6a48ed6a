// Selection folded into the product, for one token.
//
// The method's two online stages after the rotation (LaRoSA summary page,
// 方法详解 · 技术框架: keep the K largest-magnitude rotated entries, zero the
// rest; the product then reads only their rows of the folded weight) are one
// launch here. Every workgroup first computes the exact Top-K rule itself
// from the whole rotated vector (16 KB for d = 4096, read from L2): the
// threshold key T and how many channels equal to T are kept (the lowest
// indices). All workgroups reach the same rule, so nothing is broadcast and
// no index list goes through memory; each workgroup builds the list of its
// own kept channels in LDS and starts streaming their rows at once.
//
// Work split: workgroup (tile, split) owns one column tile of 64·V columns
// (V = 8 bf16 or 4 fp32 per 16-byte load) and the kept channels of the
// channel range [split·cps, split·cps + cps). Its 16 waves take interleaved
// groups of eight kept rows, one 16-byte load per lane and row, all eight in
// flight. The waves' sums are combined in LDS; with more than one split the
// partial sums of a tile are added in split order by the tile's
// last-arriving workgroup, as in the standalone product.
//
// The grid is sized to at most one workgroup per CU (256 on MI355X), which
// keeps every workgroup resident for the whole launch.
#include "common.hpp"
#include "launch.hpp"
#include "select_core.hpp"

namespace larosa {
namespace {

constexpr int kSgWaves = 16;
constexpr int kSgThreads = kSgWaves * kWave;
constexpr int kSgRows = 8;        // kept rows per wave group (loads in flight per lane)
constexpr int kSgListMax = 4096;  // channels of one split (LDS row list)
constexpr int kSgMaxSplitLoads = 16;

size_t sg_counter_bytes(int tiles) { return (static_cast<size_t>(tiles) * 4 + 255) / 256 * 256; }

template <typename WT, typename OT, int EMAX>
__global__ __launch_bounds__(kSgThreads) void select_gather_kernel(
    const float *__restrict__ x_rot, int d, int k, int E, int tiles, int splits, int cps,
    const WT *__restrict__ w, int64_t d_out, OT *__restrict__ y, float *__restrict__ partials,
    uint32_t *__restrict__ counters, int32_t *__restrict__ idx_out) {
  constexpr int V = Elt<WT>::kVec;
  constexpr int TILE = kWave * V;
  __shared__ SelectSmem<kSgThreads> sm;
  __shared__ int32_t l_idx[kSgListMax];
  __shared__ float l_val[kSgListMax];
  __shared__ float red[kSgWaves][TILE];
  __shared__ uint32_t s_p0, s_p1;
  __shared__ int s_last;

  const int t = threadIdx.x;
  const int lane = t % kWave;
  const int wave = wave_id();
  const int tile = blockIdx.x % tiles;
  const int split = blockIdx.x / tiles;
  const int c0 = split * cps < d ? split * cps : d;
  const int c1 = c0 + cps < d ? c0 + cps : d;

  // 1. The exact rule over all d channels: T, and krem channels equal to T
  //    kept in index order. kept_flags also gives each thread the number of
  //    kept channels below its first slot.
  float v[EMAX];
  uint32_t key[EMAX];
  load_keys4<EMAX>(x_rot, d, E, key, v);
  uint32_t T, krem, n_eq;
  radix_threshold<kSgThreads, EMAX>(key, static_cast<uint32_t>(k), sm, T, krem, n_eq);
  bool kept[EMAX];
  uint32_t pos;
  kept_flags<kSgThreads, EMAX>(key, T, krem, sm, kept, pos);

  // 2. Positions of this split's first and last kept channel in the global
  //    ascending list, then its kept channels into LDS (and, from tile 0, the
  //    global index list when asked for).
  const int i0 = t * E;
  if (t == 0) {
    if (c0 >= d) s_p0 = static_cast<uint32_t>(k);
    if (c1 >= d) s_p1 = static_cast<uint32_t>(k);
  }
  {
    uint32_t p = pos;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      const int i = i0 + e;
      if (e < E && i < d && i == c0) s_p0 = p;
      if (e < E && i < d && i == c1) s_p1 = p;
      if (kept[e]) ++p;
    }
  }
  __syncthreads();
  const uint32_t p0 = s_p0;
  const int n_list = static_cast<int>(s_p1 - p0);
  {
    uint32_t p = pos;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (!kept[e]) continue;
      const int i = i0 + e;
      if (i >= c0 && i < c1) {
        l_idx[p - p0] = i;
        l_val[p - p0] = v[e];
      }
      if (idx_out && tile == 0 && i >= c0 && i < c1) idx_out[p] = i;
      ++p;
    }
  }
  __syncthreads();

  // 3. Stream the kept rows of this column tile. Lanes past the last column
  //    read a valid column and store nothing.
  const int64_t col_raw = static_cast<int64_t>(tile) * TILE + lane * V;
  const int64_t col = col_raw < d_out ? col_raw : d_out - V;
  float acc[V];
#pragma unroll
  for (int q = 0; q < V; ++q) acc[q] = 0.f;
  for (int base = wave * kSgRows; base < n_list; base += kSgWaves * kSgRows) {
    uint4 q[kSgRows];
    float c[kSgRows];
#pragma unroll
    for (int u = 0; u < kSgRows; ++u) {
      const int j = base + u;  // wave-uniform
      const bool ok = j < n_list;
      const int row = ok ? l_idx[j] : 0;
      c[u] = ok ? l_val[j] : 0.f;
      q[u] = ok ? load16(w + static_cast<int64_t>(row) * d_out + col) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kSgRows; ++u) {
      float f[V];
      Elt<WT>::unpack(q[u], f);
#pragma unroll
      for (int qq = 0; qq < V; ++qq) acc[qq] = fmaf(c[u], f[qq], acc[qq]);
    }
  }

  // 4. Combine the waves; with one split store y, else partial sums.
#pragma unroll
  for (int q = 0; q < V; ++q) red[wave][lane * V + q] = acc[q];
  __syncthreads();
  const int64_t tile_col0 = static_cast<int64_t>(tile) * TILE;
  float *part = partials + static_cast<int64_t>(split) * d_out;
  for (int e = t; e < TILE; e += kSgThreads) {
    const int64_t cg = tile_col0 + e;
    if (cg >= d_out) continue;
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < kSgWaves; ++ww) s += red[ww][e];
    if (splits == 1) {
      Elt<OT>::store(y, cg, s);
    } else {
      // Agent-scope atomic exchange: the value lands at the device-coherent
      // point, like the arrival counter below.
      const float old = __hip_atomic_exchange(part + cg, s, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      (void)old;
    }
  }
  if (splits == 1) return;

  // The tile's last workgroup to arrive adds the partial sums in split
  // order (the result does not depend on arrival order) and resets the
  // tile's counter for the next call.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == static_cast<uint32_t>(splits - 1);
  }
  __syncthreads();
  if (!s_last) return;
  for (int e = t; e < TILE; e += kSgThreads) {
    const int64_t cg = tile_col0 + e;
    if (cg >= d_out) continue;
    const float *p = partials + cg;
    float s = 0.f;
    for (int r0 = 0; r0 < splits; r0 += kSgMaxSplitLoads) {
      float pv[kSgMaxSplitLoads];
#pragma unroll
      for (int i = 0; i < kSgMaxSplitLoads; ++i)
        pv[i] = r0 + i < splits ? __hip_atomic_load(p + (r0 + i) * d_out, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                                : 0.f;
#pragma unroll
      for (int i = 0; i < kSgMaxSplitLoads; ++i)
        if (r0 + i < splits) s += pv[i];
    }
    Elt<OT>::store(y, cg, s);
  }
  if (t == 0)
    __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename WT, typename OT>
hipError_t launch_sg_t(const SelectGatherArgs &a, const SelectGatherPlan &p, hipStream_t s) {
  const int E = slots_per_thread(a.d_in, kSgThreads);
  uint32_t *counters = static_cast<uint32_t *>(a.ws);
  float *partials =
      reinterpret_cast<float *>(static_cast<char *>(a.ws) + sg_counter_bytes(p.tiles));
  const dim3 grid(static_cast<unsigned>(p.tiles * p.splits));
  const auto *w = static_cast<const WT *>(a.w);
  auto *y = static_cast<OT *>(a.y);
#define LAROSA_SG(EM)                                                                       \
  hipLaunchKernelGGL((select_gather_kernel<WT, OT, EM>), grid, dim3(kSgThreads), 0, s,     \
                     a.x_rot, a.d_in, a.k, E, p.tiles, p.splits, p.cps, w, a.d_out, y,      \
                     partials, counters, a.idx_out)
  if (E <= 4) LAROSA_SG(4);
  else if (E <= 8) LAROSA_SG(8);
  else if (E <= 16) LAROSA_SG(16);
  else if (E <= 32) LAROSA_SG(32);
  else return hipErrorInvalidValue;
#undef LAROSA_SG
  return hipGetLastError();
}

}  // namespace

SelectGatherPlan plan_select_gather(int64_t d_in, int64_t d_out, int w_dt) {
  SelectGatherPlan p;
  const int64_t tile_cols = static_cast<int64_t>(kWave) * (w_dt == kF32 ? 4 : 8);
  p.tiles = static_cast<int>((d_out + tile_cols - 1) / tile_cols);
  int64_t splits = 256 / p.tiles;                          // one workgroup per CU
  const int64_t by_list = (d_in + kSgListMax - 1) / kSgListMax;  // LDS list bound
  const int64_t by_size = (d_in + 63) / 64;                // at least 64 channels each
  if (splits > by_size) splits = by_size;
  if (splits < by_list) splits = by_list;
  if (splits < 1) splits = 1;
  const int64_t cps = (d_in + splits - 1) / splits;
  p.cps = static_cast<int>(cps);
  p.splits = static_cast<int>((d_in + cps - 1) / cps);
  return p;
}

size_t select_gather_ws_bytes(int64_t d_in, int64_t d_out, int w_dt) {
  const SelectGatherPlan p = plan_select_gather(d_in, d_out, w_dt);
  if (p.splits <= 1) return 0;
  return sg_counter_bytes(p.tiles) + static_cast<size_t>(p.splits) * d_out * sizeof(float);
}

bool select_gather_supported(int64_t d_in) { return d_in >= 1 && d_in <= 32768; }

hipError_t launch_select_gather(const SelectGatherArgs &a, hipStream_t s) {
  const SelectGatherPlan p = plan_select_gather(a.d_in, a.d_out, a.w_dt);
  if (p.cps > kSgListMax) return hipErrorInvalidValue;
  if (a.w_dt == kBF16 && a.y_dt == kBF16) return launch_sg_t<uint16_t, uint16_t>(a, p, s);
  if (a.w_dt == kBF16 && a.y_dt == kF32) return launch_sg_t<uint16_t, float>(a, p, s);
  if (a.w_dt == kF32 && a.y_dt == kF32) return launch_sg_t<float, float>(a, p, s);
  return hipErrorInvalidValue;
}

}  // namespace larosa
