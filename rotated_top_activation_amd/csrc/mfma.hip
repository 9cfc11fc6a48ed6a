// Matrix-core (MFMA) forms of the rotation and of the product over kept
// rows, for batches of 16 to 64 tokens in bf16. At these batch sizes the
// fp32 vector forms would either re-read Qᵀ and W' once per small group of
// tokens or run out of FMA throughput; with v_mfma_f32_16x16x32_bf16 every
// weight byte is read once for the whole batch.
//
// Operand layout of v_mfma_f32_16x16x32_bf16 (checked on the device): lane l
// holds row l mod 16 of A (tokens) and column l mod 16 of B (channels or
// output columns), eight consecutive k each starting at k = 8·(l div 16); the
// 16×16 fp32 result has lane l holding rows 4·(l div 16) + i, i < 4, of
// column l mod 16.
//
// Rotation (stage 1 of the LaRoSA summary page, 方法详解 · 技术框架):
// x_rot[b, j] = Σ_i x[b, blk(j)·qb + i] · Qt[j, i]. Both operands are
// contiguous along k (x rows, and rows of the prepared Qt), so each lane
// loads its eight k with one 16-byte load. A wave owns 16 output channels and
// a k-range of their block; k-ranges are summed by a second kernel in a fixed
// order.
//
// Product (the gather of the method's kept rows): y[b, :] = Σ_j c[b, j] ·
// W'[row_j, :]. Rows of W' are contiguous along the output columns, so a
// wave stages 32 rows × 64 columns in its own LDS area and reads the B
// operand back with the gfx950 transpose read (ds_read_b64_tr_b16). The
// fp32 coefficients arrive split into bf16 hi + lo parts (two MFMAs), which
// keeps about 16 significant bits of each coefficient; products and sums
// stay in fp32. Weight rows and coefficients are requested two steps ahead.
#include "common.hpp"
#include "launch.hpp"

namespace larosa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kMK = 32;           // k per MFMA step
constexpr int kMW = 4;            // waves per workgroup (independent units)
constexpr int kMCols = 64;        // output columns per wave in the product
constexpr int kPitch = 80;        // LDS row pitch of a staged W' tile (bf16)

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- rotation --------------------------------------------------------------
// Grid: (d / 16 channel groups, ks k-splits). Part s of x_rot goes to
// out + s·B·d (out = x_rot itself when ks == 1).
template <int MT>
__global__ __launch_bounds__(kMW * kWave) void rotate_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ qt, float *__restrict__ out,
    int B, int d, int qb, int k_per_split) {
  const int lane = threadIdx.x % kWave;
  const int j0 = (blockIdx.x * kMW + wave_id()) * 16;
  if (j0 >= d) return;
  const int blk_off = (j0 / qb) * qb;
  const int kb = blockIdx.y * k_per_split;
  const int ke = kb + k_per_split < qb ? kb + k_per_split : qb;
  const int kl = (lane / 16) * 8;
  const uint16_t *qrow = qt + static_cast<int64_t>(j0 + lane % 16) * qb + kl;
  const uint16_t *xrow[MT];
  bool xok[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int b = m * 16 + lane % 16;
    xok[m] = b < B;
    xrow[m] = x + static_cast<int64_t>(xok[m] ? b : 0) * d + blk_off + kl;
  }
  f32x4 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int U = 4;  // k-steps whose loads are issued together
  for (int k0 = kb; k0 < ke; k0 += U * kMK) {
    uint4 q[U], a[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + u * kMK;
      const bool ok = k < ke;
      q[u] = ok ? load16(qrow + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int m = 0; m < MT; ++m) a[u][m] = ok && xok[m] ? load16(xrow[m] + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = mfma(as_bf16x8(a[u][m]), as_bf16x8(q[u]), acc[m]);
  }
  float *o = out + static_cast<int64_t>(blockIdx.y) * B * d;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = m * 16 + (lane / 16) * 4 + i;
      if (b < B) o[static_cast<int64_t>(b) * d + j0 + lane % 16] = acc[m][i];
    }
}

// ---- product over kept rows ------------------------------------------------
// Grid: (ceil(d_out / 256) column groups of four waves, splits). Split s
// covers list positions [s·rps, s·rps + rps) (rps a multiple of 32). Coefficients
// come split and transposed (store_coef_hl) for list position j (zero past the
// list's end, ldc a multiple of 32 and at least the list length rounded up
// to 32). Split s writes out + s·B·d_out (fp32), or y when there is one split.
template <int MT>
__global__ __launch_bounds__(kMW * kWave) void gather_mfma_kernel(
    const int32_t *__restrict__ rows, const int32_t *__restrict__ n_rows_dev, int max_rows,
    int d_in, const uint16_t *__restrict__ coef_hl, int ldc, const uint16_t *__restrict__ w,
    int64_t d_out, float *__restrict__ out, uint16_t *__restrict__ y, int B, int rps) {
  __shared__ __align__(16) uint16_t tile[kMW][kMK * kPitch];
  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  const int64_t col0 = (static_cast<int64_t>(blockIdx.x) * kMW + wave) * kMCols;
  if (col0 >= d_out) return;  // wave-uniform; no workgroup barriers below
  int n_rows = n_rows_dev ? *n_rows_dev : max_rows;
  n_rows = n_rows < 0 ? 0 : (n_rows > max_rows ? max_rows : n_rows);
  const int r_begin = blockIdx.y * rps;
  const int r_end = r_begin + rps < n_rows ? r_begin + rps : n_rows;
  uint16_t *my = tile[wave];
  // staging: lane l moves 16 bytes of rows (l / 8) + 8·q, columns 8·(l mod 8)
  const int64_t scol_raw = col0 + (lane % 8) * 8;
  const int64_t scol = scol_raw < d_out ? scol_raw : d_out - 8;
  const int srow = lane / 8;
  // transpose reads: source lane s of group g addresses row g·8 + half·4 +
  // s / 4, column 16·ns + 4·(s mod 4)
  const int g = lane / 16, s = lane % 16;
  const int tr_off = (g * 8 + s / 4) * kPitch + 4 * (s % 4);
  // coefficients (split hi/lo, see store_coef_hl): lane l takes token
  // 16·m + l mod 16, list positions k0 + 8·(l div 16) .. + 7, whose hi and
  // lo halves are 16 bytes each at crow[m] + 2·k0
  const uint16_t *crow[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int b = m * 16 + lane % 16;
    crow[m] = coef_hl + (static_cast<int64_t>(b < B ? b : 0) * ldc + g * 8) * 2;
  }
  f32x4 acc[4][MT];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[n][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline: the row indices of step k + 4, and the weight rows
  // and coefficients of step k + 2, are requested while step k is computed
  // (the loop body is unrolled by two so every buffer stays in registers).
  auto fetch_idx = [&](int k0, int (&ix)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = k0 + srow + 8 * q;
      ix[q] = r < r_end ? (rows ? rows[r] : r) : -1;
    }
  };
  auto fetch = [&](int k0, const int (&ix)[4], uint4 (&v)[4], uint4 (&cv)[MT][2]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = ix[q];
      // rows outside [0, d_in) contribute nothing
      v[q] = row >= 0 && row < d_in ? load16(w + static_cast<int64_t>(row) * d_out + scol)
                                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      cv[m][0] = load16(crow[m] + 2 * k0);
      cv[m][1] = load16(crow[m] + 2 * k0 + 8);
    }
  };
  auto step = [&](const uint4 (&v)[4], const uint4 (&cv)[MT][2]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4 *>(my + (srow + 8 * q) * kPitch + (lane % 8) * 8) = v[q];
    bf16x8 ahi[MT], alo[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      ahi[m] = as_bf16x8(cv[m][0]);
      alo[m] = as_bf16x8(cv[m][1]);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS stores are done
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4 *)(my + tr_off + 16 * n));
      const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4 *)(my + tr_off + 4 * kPitch + 16 * n));
      bf16x8 bop;
      __builtin_memcpy(&bop, &lo4, 8);
      __builtin_memcpy(reinterpret_cast<char *>(&bop) + 8, &hi4, 8);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        acc[n][m] = mfma(ahi[m], bop, acc[n][m]);
        acc[n][m] = mfma(alo[m], bop, acc[n][m]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next step's stores
    __builtin_amdgcn_wave_barrier();
  };
  uint4 v0[4], v1[4];
  uint4 c0[MT][2], c1[MT][2];
  int i0[4], i1[4];
  // every fetch is guarded by its step being below r_end, so coefficient
  // reads stay below ldc (a multiple of the step above the list length)
  if (r_begin < r_end) {
    fetch_idx(r_begin, i0);
    fetch(r_begin, i0, v0, c0);
    fetch_idx(r_begin + 2 * kMK, i0);
  }
  if (r_begin + kMK < r_end) {
    fetch_idx(r_begin + kMK, i1);
    fetch(r_begin + kMK, i1, v1, c1);
    fetch_idx(r_begin + 3 * kMK, i1);
  }
  for (int k0 = r_begin; k0 < r_end; k0 += 2 * kMK) {
    step(v0, c0);
    if (k0 + 2 * kMK < r_end) {
      fetch(k0 + 2 * kMK, i0, v0, c0);
      fetch_idx(k0 + 4 * kMK, i0);
    }
    if (k0 + kMK < r_end) {
      step(v1, c1);
      if (k0 + 3 * kMK < r_end) {
        fetch(k0 + 3 * kMK, i1, v1, c1);
        fetch_idx(k0 + 5 * kMK, i1);
      }
    }
  }
  // lane l holds tokens 16·m + 4·(l div 16) + i of column col0 + 16·n + l mod 16
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int64_t col = col0 + 16 * n + lane % 16;
    if (col >= d_out) continue;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = m * 16 + g * 4 + i;
        if (b >= B) continue;
        if (y)
          y[static_cast<int64_t>(b) * d_out + col] = f32_to_bf16(acc[n][m][i]);
        else
          out[(static_cast<int64_t>(blockIdx.y) * B + b) * d_out + col] = acc[n][m][i];
      }
  }
}

// Sums `parts` consecutive [n] fp32 slices in order; writes fp32 or bf16.
template <typename OT>
__global__ void sum_parts_kernel(const float *__restrict__ part, int parts, int64_t n,
                                 OT *__restrict__ dst) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  float4 s = *reinterpret_cast<const float4 *>(part + i);
  for (int p = 1; p < parts; ++p) {
    const float4 v = *reinterpret_cast<const float4 *>(part + static_cast<int64_t>(p) * n + i);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  Elt<OT>::store(dst, i, s.x);
  Elt<OT>::store(dst, i + 1, s.y);
  Elt<OT>::store(dst, i + 2, s.z);
  Elt<OT>::store(dst, i + 3, s.w);
}

// Split coefficients (store_coef_hl) of the bf16 activation x[b, j] for
// j < d_in; zero up to ldc.
__global__ void act_to_coef_t_kernel(const uint16_t *__restrict__ x, int B, int64_t d_in,
                                     int64_t ldc, uint16_t *__restrict__ coef_hl) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= ldc * B) return;
  const int64_t b = e / ldc, j = e % ldc;
  store_coef_hl(coef_hl, ldc, b, j, j < d_in ? bf16_to_f32(x[b * d_in + j]) : 0.f);
}

template <typename OT>
hipError_t sum_parts(const float *part, int parts, int64_t n, OT *dst, hipStream_t s) {
  const int64_t threads = (n + 3) / 4;
  hipLaunchKernelGGL((sum_parts_kernel<OT>), dim3(static_cast<unsigned>((threads + 255) / 256)),
                     dim3(256), 0, s, part, parts, n, dst);
  return hipGetLastError();
}

// Workgroups wanted in flight: about eight waves per CU keep enough loads
// outstanding for HBM at these tile sizes.
constexpr int kTargetWaves = 2048;

}  // namespace

bool mfma_supported(int64_t B, int act_dt, int w_dt) {
  return B >= kMfmaMinB && B <= 64 && act_dt == kBF16 && w_dt == kBF16;
}

int rotate_mfma_splits(int64_t B, int64_t d, int64_t qb) {
  (void)B;
  const int64_t groups = d / 16;
  int64_t ks = (kTargetWaves + groups - 1) / groups;
  const int64_t steps = qb / kMK;
  if (ks > steps) ks = steps;
  if (ks > 8) ks = 8;  // partial sums stay a small fraction of the Qt bytes
  if (ks < 1) ks = 1;
  const int64_t kps = (steps + ks - 1) / ks * kMK;
  return static_cast<int>((qb + kps - 1) / kps);
}

size_t rotate_mfma_ws_bytes(int64_t B, int64_t d, int64_t qb) {
  const int ks = rotate_mfma_splits(B, d, qb);
  return ks > 1 ? static_cast<size_t>(ks) * B * d * 4 : 0;
}

hipError_t launch_rotate_mfma(const void *x, const void *qt, float *x_rot, int B, int d, int qb,
                              void *ws, hipStream_t s) {
  const int ks = ws ? rotate_mfma_splits(B, d, qb) : 1;
  const int steps = qb / kMK;
  const int kps = (steps + ks - 1) / ks * kMK;
  float *out = ks > 1 ? static_cast<float *>(ws) : x_rot;
  const dim3 grid(static_cast<unsigned>((d / 16 + kMW - 1) / kMW), static_cast<unsigned>(ks));
  const int MT = (B + 15) / 16;
  const auto *xp = static_cast<const uint16_t *>(x);
  const auto *qp = static_cast<const uint16_t *>(qt);
  switch (MT) {
    case 1: hipLaunchKernelGGL(rotate_mfma_kernel<1>, grid, dim3(kMW * kWave), 0, s, xp, qp, out, B, d, qb, kps); break;
    case 2: hipLaunchKernelGGL(rotate_mfma_kernel<2>, grid, dim3(kMW * kWave), 0, s, xp, qp, out, B, d, qb, kps); break;
    case 3: hipLaunchKernelGGL(rotate_mfma_kernel<3>, grid, dim3(kMW * kWave), 0, s, xp, qp, out, B, d, qb, kps); break;
    default: hipLaunchKernelGGL(rotate_mfma_kernel<4>, grid, dim3(kMW * kWave), 0, s, xp, qp, out, B, d, qb, kps); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ks == 1) return e;
  return sum_parts<float>(out, ks, static_cast<int64_t>(B) * d, x_rot, s);
}

MfmaGatherPlan plan_gather_mfma(int64_t B, int64_t max_rows, int64_t d_out) {
  (void)B;
  MfmaGatherPlan p;
  p.col_groups = static_cast<int>((d_out + kMCols * kMW - 1) / (kMCols * kMW));
  const int64_t waves = (d_out + kMCols - 1) / kMCols;
  int64_t splits = (kTargetWaves + waves - 1) / waves;
  const int64_t steps = max_rows > 0 ? (max_rows + kMK - 1) / kMK : 1;
  if (splits > steps / 4) splits = steps / 4;  // at least four steps per split
  if (splits > 16) splits = 16;
  if (splits < 1) splits = 1;
  const int64_t rps = (steps + splits - 1) / splits * kMK;
  p.rows_per_split = static_cast<int>(rps);
  p.splits = static_cast<int>((max_rows + rps - 1) / rps);
  if (p.splits < 1) p.splits = 1;
  return p;
}

size_t gather_mfma_ws_bytes(int64_t B, int64_t max_rows, int64_t d_out) {
  const MfmaGatherPlan p = plan_gather_mfma(B, max_rows, d_out);
  return p.splits > 1 ? static_cast<size_t>(p.splits) * B * d_out * 4 : 0;
}

int64_t mfma_coef_ld(int64_t max_rows) { return (max_rows + kMK - 1) / kMK * kMK; }

hipError_t launch_gather_mfma(const int32_t *rows, const int32_t *n_rows, int64_t max_rows,
                              int64_t d_in, const void *coef_hl, int64_t ldc, const void *w,
                              void *y, int B, int64_t d_out, void *ws, hipStream_t s) {
  const MfmaGatherPlan p = plan_gather_mfma(B, max_rows, d_out);
  float *out = static_cast<float *>(ws);
  uint16_t *yy = p.splits == 1 ? static_cast<uint16_t *>(y) : nullptr;
  const dim3 grid(static_cast<unsigned>(p.col_groups), static_cast<unsigned>(p.splits));
  const int MT = (B + 15) / 16;
  const auto *wp = static_cast<const uint16_t *>(w);
  const int mr = static_cast<int>(max_rows), ld = static_cast<int>(ldc);
  const auto *ch = static_cast<const uint16_t *>(coef_hl);
  const int di = static_cast<int>(d_in);
  switch (MT) {
    case 1: hipLaunchKernelGGL(gather_mfma_kernel<1>, grid, dim3(kMW * kWave), 0, s, rows, n_rows, mr, di, ch, ld, wp, d_out, out, yy, B, p.rows_per_split); break;
    case 2: hipLaunchKernelGGL(gather_mfma_kernel<2>, grid, dim3(kMW * kWave), 0, s, rows, n_rows, mr, di, ch, ld, wp, d_out, out, yy, B, p.rows_per_split); break;
    case 3: hipLaunchKernelGGL(gather_mfma_kernel<3>, grid, dim3(kMW * kWave), 0, s, rows, n_rows, mr, di, ch, ld, wp, d_out, out, yy, B, p.rows_per_split); break;
    default: hipLaunchKernelGGL(gather_mfma_kernel<4>, grid, dim3(kMW * kWave), 0, s, rows, n_rows, mr, di, ch, ld, wp, d_out, out, yy, B, p.rows_per_split); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  return sum_parts<uint16_t>(out, p.splits, static_cast<int64_t>(B) * d_out,
                             static_cast<uint16_t *>(y), s);
}

hipError_t launch_act_to_coef_t(const void *x, int B, int64_t d_in, int64_t ldc, void *coefT,
                                hipStream_t s) {
  const int64_t n = ldc * B;
  hipLaunchKernelGGL(act_to_coef_t_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, s, static_cast<const uint16_t *>(x), B, d_in, ldc,
                     static_cast<uint16_t *>(coefT));
  return hipGetLastError();
}

size_t gather_mfma_ws_bound(int64_t B, int64_t d_out) {
  const int64_t waves = (d_out + kMCols - 1) / kMCols;
  int64_t splits = (kTargetWaves + waves - 1) / waves;
  if (splits > 16) splits = 16;
  return splits > 1 ? static_cast<size_t>(splits) * B * d_out * 4 : 0;
}

size_t rotate_mfma_ws_bound(int64_t B, int64_t d) {
  const int64_t groups = d / 16 > 0 ? d / 16 : 1;
  int64_t ks = (kTargetWaves + groups - 1) / groups;
  if (ks > 8) ks = 8;
  return static_cast<size_t>(ks) * B * d * 4;
}

}  // namespace larosa
