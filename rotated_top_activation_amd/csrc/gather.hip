// Gather-rows product: y[b, :] = Σ_j coef(j, b) · W[row(j), :].
//
// This is the step where the method saves memory traffic: only the weight
// rows of kept input channels are read (LaRoSA abstract, PMLR 267 page:
// activation sparsity cuts computation and memory transfers). W is
// [d_in, d_out] row-major, so each kept channel is one contiguous row.
//
// Layout of the work (vector path, B <= 8):
//   * a workgroup owns one column tile of 64·V columns (V = 8 bf16 or 4 fp32
//     per 16-byte load) and a contiguous range of the row list;
//   * its waves take interleaved groups of kRows rows; every lane issues
//     one 16-byte load per row, so a wave streams 1 KB of each row and keeps
//     kRows loads in flight;
//   * row index and coefficients are wave-uniform (scalar loads);
//   * the waves' fp32 sums are combined in LDS, then either stored (one
//     split) or written as a partial sum; the last workgroup of a tile to
//     finish adds the partials in split order, so the result does not depend
//     on arrival order and needs no float atomics.
#include "common.hpp"
#include "launch.hpp"

namespace larosa {
namespace {

// Rows per wave group (loads in flight per lane). Four measured faster than
// eight or six: the 7B gate|up product over a given list of 2457 rows takes
// 22.4 µs against 26.7 µs (and the dense product over all 4096 rows 33.7
// against 34.9 µs), one process on one box.
constexpr int kRows = 4;

size_t counter_bytes(int tiles) { return (static_cast<size_t>(tiles) * 4 + 255) / 256 * 256; }
constexpr int kMaxSplitLoads = 16;  // partial sums fetched per round trip

// Largest waves per workgroup for B tokens: the LDS reduction buffer holds
// NW·B·TILE floats (at most 32 KB).
constexpr int max_waves_for(int B) { return B == 1 ? 16 : (B == 2 ? 8 : (B <= 4 ? 4 : 2)); }

template <int B, int NW, typename WT, typename OT, int CMODE>
__global__ __launch_bounds__(NW * 64) void gather_vec_kernel(
    const int32_t *__restrict__ rows, const int32_t *__restrict__ n_rows_dev,
    int64_t max_rows, const void *__restrict__ coef_v,
    int64_t coef_stride, const WT *__restrict__ w, int64_t d_in, int64_t d_out,
    OT *__restrict__ y, float *__restrict__ partials,
    uint32_t *__restrict__ counters, int splits, int rows_per_split) {
  constexpr int V = Elt<WT>::kVec;
  constexpr int TILE = kWave * V;
  __shared__ float red[NW][B][TILE];
  __shared__ int s_last;

  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  // Lanes past the last column read a valid column and store nothing.
  const int64_t col_raw = static_cast<int64_t>(tile) * TILE + lane * V;
  const int64_t col = col_raw < d_out ? col_raw : d_out - V;

  int64_t n = max_rows;
  if (n_rows_dev) {
    int64_t nd = __builtin_amdgcn_readfirstlane(*n_rows_dev);
    n = nd < n ? (nd < 0 ? 0 : nd) : n;
  }
  const int64_t r0 = static_cast<int64_t>(split) * rows_per_split;
  const int64_t r1 = r0 + rows_per_split < n ? r0 + rows_per_split : n;

  float acc[B][V];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int v = 0; v < V; ++v) acc[b][v] = 0.f;

  for (int64_t base = r0 + static_cast<int64_t>(wave) * kRows; base < r1;
       base += static_cast<int64_t>(NW) * kRows) {
    // Index and coefficient loads are unconditional (clamped to the last
    // valid list entry) so they issue back to back; rows past the end of the
    // list or outside [0, d_in) are then masked out.
    int32_t rr[kRows];
    bool ok[kRows];
    float c[kRows][B];
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int64_t jl = base + u < r1 ? base + u : r1 - 1;
      rr[u] = rows ? rows[jl] : static_cast<int32_t>(jl);
    }
#pragma unroll
    for (int u = 0; u < kRows; ++u)
      ok[u] = base + u < r1 && static_cast<uint32_t>(rr[u]) < static_cast<uint64_t>(d_in);
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      const int64_t jl = base + u < r1 ? base + u : r1 - 1;
      const int64_t ri = ok[u] ? rr[u] : 0;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        float cv;
        if (CMODE == kCoefPacked)
          cv = static_cast<const float *>(coef_v)[jl * coef_stride + b];
        else if (CMODE == kCoefActF32)
          cv = static_cast<const float *>(coef_v)[b * coef_stride + ri];
        else
          cv = bf16_to_f32(static_cast<const uint16_t *>(coef_v)[b * coef_stride + ri]);
        c[u][b] = ok[u] ? cv : 0.f;
      }
    }
    uint4 q[kRows];
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      q[u] = make_uint4(0, 0, 0, 0);
      if (ok[u]) q[u] = load16(w + static_cast<int64_t>(rr[u]) * d_out + col);
    }
#pragma unroll
    for (int u = 0; u < kRows; ++u) {
      float f[V];
      Elt<WT>::unpack(q[u], f);
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int v = 0; v < V; ++v) acc[b][v] = fmaf(c[u][b], f[v], acc[b][v]);
    }
  }

  // Combine the waves of this workgroup.
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int v = 0; v < V; ++v) red[wave][b][lane * V + v] = acc[b][v];
  __syncthreads();

  const int64_t tile_col0 = static_cast<int64_t>(tile) * TILE;
  constexpr int ENTRIES = B * TILE;
  float *part = partials + static_cast<int64_t>(split) * B * d_out;
  for (int e = threadIdx.x; e < ENTRIES; e += NW * kWave) {
    const int b = e / TILE, cl = e % TILE;
    const int64_t cg = tile_col0 + cl;
    if (cg >= d_out) continue;
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) s += red[ww][b][cl];
    if (splits == 1) {
      Elt<OT>::store(y, b * d_out + cg, s);
    } else {
      // Written with an agent-scope atomic exchange, so the value lands at
      // the same device-coherent point as the arrival counter below.
      const float old = __hip_atomic_exchange(part + b * d_out + cg, s, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      (void)old;
    }
  }
  if (splits == 1) return;

  // Last workgroup of this tile to arrive adds the partials in split order,
  // so the sum does not depend on arrival order. Every partial write above
  // has completed (waitcnt) before this workgroup's counter increment; the
  // reads below are agent-scope atomic loads, which do not hit stale cache
  // lines. No L2 write-back or invalidate is involved.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&counters[tile], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == static_cast<uint32_t>(splits - 1);
  }
  __syncthreads();
  if (!s_last) return;
  const int64_t stride = static_cast<int64_t>(B) * d_out;
  for (int e = threadIdx.x; e < ENTRIES; e += NW * kWave) {
    const int b = e / TILE, cl = e % TILE;
    const int64_t cg = tile_col0 + cl;
    if (cg >= d_out) continue;
    const float *p = partials + b * d_out + cg;
    float s = 0.f;
    // All loads of a chunk are issued before any is used: one round trip
    // per kMaxSplitLoads splits.
    for (int r0 = 0; r0 < splits; r0 += kMaxSplitLoads) {
      float v[kMaxSplitLoads];
#pragma unroll
      for (int i = 0; i < kMaxSplitLoads; ++i)
        v[i] = r0 + i < splits ? __hip_atomic_load(p + (r0 + i) * stride, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)
                               : 0.f;
#pragma unroll
      for (int i = 0; i < kMaxSplitLoads; ++i)
        if (r0 + i < splits) s += v[i];
    }
    Elt<OT>::store(y, b * d_out + cg, s);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int B, int NW, typename WT, typename OT, int CMODE>
hipError_t launch_nw(const GatherArgs &a, const GatherPlan &p, hipStream_t s) {
  // Token group [b0, b0 + B) of a batch of a.B: coefficients and outputs are
  // offset to the group; the stride between tokens (activation coefficients)
  // or between rows (packed coefficients) is that of the whole batch.
  const int64_t b0 = a.b0;
  const int64_t cstride = a.coef_mode == kCoefPacked ? a.B : a.d_in;
  const char *coef = static_cast<const char *>(a.coef) +
                     (a.coef_mode == kCoefPacked ? b0 * 4
                                                 : b0 * a.d_in * (a.coef_mode == kCoefActF32 ? 4 : 2));
  char *yb = static_cast<char *>(a.y) + b0 * a.d_out * (a.y_dt == kF32 ? 4 : 2);
  // Counters first (their place depends only on the column tiles, so every
  // token group of a batch finds them at zero), partial sums after them.
  uint32_t *counters = static_cast<uint32_t *>(a.ws);
  float *partials = reinterpret_cast<float *>(static_cast<char *>(a.ws) + counter_bytes(p.tiles));
  dim3 grid(p.tiles, p.splits);
  dim3 block(NW * kWave);
  hipLaunchKernelGGL((gather_vec_kernel<B, NW, WT, OT, CMODE>), grid, block, 0, s,
                     a.rows, a.n_rows, a.max_rows, static_cast<const void *>(coef), cstride,
                     static_cast<const WT *>(a.w), a.d_in, a.d_out,
                     reinterpret_cast<OT *>(yb), partials, counters, p.splits,
                     p.rows_per_split);
  return hipGetLastError();
}

template <int B, typename WT, typename OT, int CMODE>
hipError_t launch_t(const GatherArgs &a, const GatherPlan &p, hipStream_t s) {
  constexpr int M = max_waves_for(B);
  if (p.waves >= 16 && M >= 16) return launch_nw<B, (M >= 16 ? 16 : M), WT, OT, CMODE>(a, p, s);
  if (p.waves >= 8 && M >= 8) return launch_nw<B, (M >= 8 ? 8 : M), WT, OT, CMODE>(a, p, s);
  if (p.waves >= 4 && M >= 4) return launch_nw<B, (M >= 4 ? 4 : M), WT, OT, CMODE>(a, p, s);
  return launch_nw<B, M, WT, OT, CMODE>(a, p, s);
}

template <int B>
hipError_t dispatch_types(const GatherArgs &a, const GatherPlan &p, hipStream_t s) {
  if (a.coef_mode == kCoefPacked) {
    if (a.w_dt == kBF16 && a.y_dt == kBF16) return launch_t<B, uint16_t, uint16_t, kCoefPacked>(a, p, s);
    if (a.w_dt == kBF16 && a.y_dt == kF32) return launch_t<B, uint16_t, float, kCoefPacked>(a, p, s);
    if (a.w_dt == kF32 && a.y_dt == kF32) return launch_t<B, float, float, kCoefPacked>(a, p, s);
    return hipErrorInvalidValue;
  }
  if (a.coef_mode == kCoefActBF16 && a.w_dt == kBF16 && a.y_dt == kBF16)
    return launch_t<B, uint16_t, uint16_t, kCoefActBF16>(a, p, s);
  if (a.coef_mode == kCoefActF32 && a.w_dt == kF32 && a.y_dt == kF32)
    return launch_t<B, float, float, kCoefActF32>(a, p, s);
  return hipErrorInvalidValue;
}

}  // namespace

namespace {

GatherPlan plan_with_waves(int waves, int64_t max_rows, int64_t d_out, int w_dt) {
  GatherPlan p;
  p.vec = w_dt == kF32 ? 4 : 8;
  p.waves = waves;
  const int64_t tile_cols = static_cast<int64_t>(kWave) * p.vec;
  p.tiles = static_cast<int>((d_out + tile_cols - 1) / tile_cols);
  // Aim for about 32 waves per CU (256 CUs) while keeping at least two row
  // groups per wave; more splits cost partial-sum traffic and reduction time.
  const int64_t target_wgs = (256 * 32) / waves;
  int64_t splits = (target_wgs + p.tiles - 1) / p.tiles;
  const int64_t unit = static_cast<int64_t>(waves) * kRows;
  int64_t max_splits = max_rows / (2 * unit);
  if (max_splits < 1) max_splits = 1;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int64_t rps = (max_rows + splits - 1) / splits;
  rps = ((rps + unit - 1) / unit) * unit;  // whole row groups per workgroup
  if (rps < 1) rps = 1;
  splits = (max_rows + rps - 1) / rps;
  if (splits < 1) splits = 1;
  p.splits = static_cast<int>(splits);
  p.rows_per_split = static_cast<int>(rps);
  return p;
}

}  // namespace

GatherPlan plan_gather(int B, int64_t max_rows, int64_t d_out, int w_dt) {
  // The widest workgroup that still yields at least 256 workgroups (one per
  // CU); otherwise the narrowest allowed.
  const int m = max_waves_for(B);
  GatherPlan p = plan_with_waves(m, max_rows, d_out, w_dt);
  for (int w = m; w >= 4; w /= 2) {
    p = plan_with_waves(w, max_rows, d_out, w_dt);
    if (static_cast<int64_t>(p.tiles) * p.splits >= 256) break;
  }
  return p;
}

size_t gather_ws_bytes(const GatherPlan &p, int B, int64_t d_out) {
  if (p.splits <= 1) return 0;
  const size_t pbytes = static_cast<size_t>(p.splits) * B * d_out * sizeof(float);
  return counter_bytes(p.tiles) + pbytes;
}

// Most splits any plan_gather(nb, rows, ...) with rows <= max_rows can
// choose. For a fixed wave count the split count is at most
// min(ceil(target / tiles), max(1, rows / (2 · waves · kRows))), which grows
// with rows; but fewer rows can move the choice to narrower workgroups with
// more splits, so every wave count the planner may pick is bounded.
int64_t gather_split_bound(int nb, int64_t max_rows, int64_t d_out, int w_dt) {
  const int m = max_waves_for(nb);
  int64_t bound = 1;
  for (int w = m; w >= (m < 4 ? m : 4); w /= 2) {
    const GatherPlan p = plan_with_waves(w, max_rows, d_out, w_dt);
    const int64_t target_wgs = (256 * 32) / w;
    int64_t by_rows = max_rows / (2 * static_cast<int64_t>(w) * kRows);
    if (by_rows < 1) by_rows = 1;
    const int64_t by_target = (target_wgs + p.tiles - 1) / p.tiles;
    const int64_t sb = by_rows < by_target ? by_rows : by_target;
    if (sb > bound) bound = sb;
  }
  return bound;
}

size_t gather_batch_ws_bytes(int B, int64_t max_rows, int64_t d_out, int w_dt) {
  size_t need = 0;
  for (int nb = 1; nb <= (B < 8 ? B : 8); ++nb) {
    const GatherPlan p = plan_gather(nb, max_rows, d_out, w_dt);
    const int64_t splits = gather_split_bound(nb, max_rows, d_out, w_dt);
    if (splits <= 1) continue;
    const size_t n = counter_bytes(p.tiles) + static_cast<size_t>(splits) * nb * d_out * sizeof(float);
    need = n > need ? n : need;
  }
  return need;
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t s) {
  // Up to eight tokens per launch; larger batches run in groups of eight
  // over the same row list (each group re-reads the rows).
  for (int b0 = 0; b0 < a.B; b0 += 8) {
    GatherArgs g = a;
    g.b0 = b0;
    const int nb = a.B - b0 < 8 ? a.B - b0 : 8;
    const GatherPlan p = plan_gather(nb, a.max_rows, a.d_out, a.w_dt);
    hipError_t e;
    switch (nb) {
      case 1: e = dispatch_types<1>(g, p, s); break;
      case 2: e = dispatch_types<2>(g, p, s); break;
      case 3: e = dispatch_types<3>(g, p, s); break;
      case 4: e = dispatch_types<4>(g, p, s); break;
      case 5: e = dispatch_types<5>(g, p, s); break;
      case 6: e = dispatch_types<6>(g, p, s); break;
      case 7: e = dispatch_types<7>(g, p, s); break;
      default: e = dispatch_types<8>(g, p, s); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace larosa
