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
// stay in fp32. The coefficients of a step are staged once per workgroup in
// LDS; weight rows and coefficients are requested two steps ahead.
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
  // Groups of U k-steps, two groups in flight: the next group's loads are
  // issued before the current one is used (the loop body is unrolled by two
  // so both buffers stay in registers).
  constexpr int U = 2;
  auto load = [&](int k0, uint4 (&q)[U], uint4 (&a)[U][MT]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + u * kMK;
      const bool ok = k < ke;
      q[u] = ok ? load16(qrow + k) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int m = 0; m < MT; ++m) a[u][m] = ok && xok[m] ? load16(xrow[m] + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto use = [&](const uint4 (&q)[U], const uint4 (&a)[U][MT]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = mfma(as_bf16x8(a[u][m]), as_bf16x8(q[u]), acc[m]);
  };
  uint4 q0[U], a0[U][MT], q1[U], a1[U][MT];
  if (kb < ke) load(kb, q0, a0);
  for (int k0 = kb; k0 < ke; k0 += 2 * U * kMK) {
    if (k0 + U * kMK < ke) load(k0 + U * kMK, q1, a1);
    use(q0, a0);
    if (k0 + U * kMK < ke) {
      if (k0 + 2 * U * kMK < ke) load(k0 + 2 * U * kMK, q0, a0);
      use(q1, a1);
    }
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

// The rotation with both operands staged in LDS, for q_block a multiple of
// 64 (a workgroup's 64 channels then lie in one block). Read straight into
// the MFMA layout, a load instruction of the kernel above touches 64 bytes
// of each of 16 Qt rows 16 KB apart; here each wave reads its 16 rows as
// contiguous 256-byte segments (16 lanes per row) into its own LDS tile, the
// workgroup stages the tokens' x chunk once (a quarter per wave), and the
// operands are read back from LDS. Chunks of 128 k; the next chunk's loads
// are issued before the current one is used; one workgroup barrier per
// chunk guards the double-buffered x area.
constexpr int kRC = 128;           // k per staged chunk
constexpr int kRPitch = kRC + 8;   // LDS row pitch (bf16): 272 bytes, no bank conflicts

template <int MT>
__global__ __launch_bounds__(kMW * kWave) void rotate_mfma_staged_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ qt, float *__restrict__ out,
    int B, int d, int qb, int k_per_split) {
  constexpr int TB = MT * 16;
  constexpr int NT = kMW * kWave;
  constexpr int XE = TB * (kRC / 8) / NT;  // staged x chunks of 16 bytes per thread (= MT)
  __shared__ __align__(16) uint16_t xl[2][TB * kRPitch];
  __shared__ __align__(16) uint16_t ql[kMW][16 * kRPitch];
  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  const int jw = (blockIdx.x * kMW + wave) * 16;          // this wave's first channel
  const int jb = blockIdx.x * kMW * 16;                   // the workgroup's (one Qt block)
  // waves past the last channel stage and meet the barriers, store nothing
  const int blk_off = (jb / qb) * qb;
  const int kb = blockIdx.y * k_per_split;
  const int ke = kb + k_per_split < qb ? kb + k_per_split : qb;
  // Qt staging: lane l loads row 4·i + l / 16 of the wave's 16, k 8·(l mod 16)
  const uint16_t *qsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int j = jw + 4 * i + lane / 16;
    j = j < d ? j : d - 1;
    qsrc[i] = qt + static_cast<int64_t>(j) * qb + 8 * (lane % 16);
  }
  const int qdst = (lane / 16) * kRPitch + 8 * (lane % 16);  // + 4·i rows
  // x staging: chunk e = threadIdx.x + NT·i is token e / 16, k 8·(e mod 16)
  const uint16_t *xsrc[XE];
  bool xok[XE];
  int xdst[XE];
#pragma unroll
  for (int i = 0; i < XE; ++i) {
    const int e = static_cast<int>(threadIdx.x) + NT * i;
    const int tok = e / 16;
    xok[i] = tok < B;
    xsrc[i] = x + static_cast<int64_t>(xok[i] ? tok : 0) * d + blk_off + 8 * (e % 16);
    xdst[i] = tok * kRPitch + 8 * (e % 16);
  }
  // operand reads: lane l takes row (token or channel) l mod 16 of a 16-row
  // block, k 8·(l div 16) of the MFMA step
  const int g = lane / 16, s = lane % 16;
  f32x4 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto fetch = [&](int k0, uint4 (&qv)[4], uint4 (&xv)[XE]) {
    const bool qin = k0 + 8 * (lane % 16) < ke;
#pragma unroll
    for (int i = 0; i < 4; ++i) qv[i] = qin ? load16(qsrc[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < XE; ++i) {
      const int e = static_cast<int>(threadIdx.x) + NT * i;
      const bool in = xok[i] && k0 + 8 * (e % 16) < ke;
      xv[i] = in ? load16(xsrc[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  uint16_t *myq = ql[wave];
  auto chunk = [&](int k0, const uint4 (&qv)[4], const uint4 (&xv)[XE], uint16_t *xbuf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4 *>(myq + qdst + 4 * i * kRPitch) = qv[i];
#pragma unroll
    for (int i = 0; i < XE; ++i) *reinterpret_cast<uint4 *>(xbuf + xdst[i]) = xv[i];
    __syncthreads();  // the x chunk is staged (weights in flight are not waited for)
    const int steps = (ke - k0) / kMK < kRC / kMK ? (ke - k0) / kMK : kRC / kMK;
    for (int st = 0; st < steps; ++st) {
      const bf16x8 bq = *reinterpret_cast<const bf16x8 *>(myq + s * kRPitch + st * kMK + 8 * g);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bf16x8 ax =
            *reinterpret_cast<const bf16x8 *>(xbuf + (m * 16 + s) * kRPitch + st * kMK + 8 * g);
        acc[m] = mfma(ax, bq, acc[m]);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // this wave's reads are done before its next stores
    __builtin_amdgcn_wave_barrier();
  };
  uint4 q0[4], x0[XE], q1[4], x1[XE];
  // the workgroup's waves share kb and ke, so they take the same chunks
  if (kb < ke) fetch(kb, q0, x0);
  for (int k0 = kb; k0 < ke; k0 += 2 * kRC) {
    if (k0 + kRC < ke) fetch(k0 + kRC, q1, x1);
    chunk(k0, q0, x0, xl[0]);
    if (k0 + kRC < ke) {
      if (k0 + 2 * kRC < ke) fetch(k0 + 2 * kRC, q0, x0);
      chunk(k0 + kRC, q1, x1, xl[1]);
    }
  }
  if (jw >= d) return;
  float *o = out + static_cast<int64_t>(blockIdx.y) * B * d;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = m * 16 + g * 4 + i;
      if (b < B) o[static_cast<int64_t>(b) * d + jw + s] = acc[m][i];
    }
}

// ---- product over kept rows ------------------------------------------------
// Grid: (ceil(d_out / 256) column groups of four waves, splits). Split s
// covers list positions [s·rps, s·rps + rps) (rps a multiple of 32). Coefficients
// come split and transposed (store_coef_hl) for list position j (zero past the
// list's end, ldc a multiple of 32 and at least the list length rounded up
// to 32). Split s writes out + s·B·d_out (fp32), or y when there is one split.
// Each wave works alone: it loads its own coefficients with its weight rows.
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

// The same product for 49 to 64 tokens. The four waves of a workgroup read
// the same rows (one split) for different columns, so they need the same
// coefficients, which at this batch are twice the weight bytes a wave
// streams: each 32-row step's coefficients (B tokens × 32 positions × hi/lo
// = 128 bytes per token) are staged once per workgroup into LDS
// (double-buffered, one workgroup barrier per step), a quarter per wave.
// With fewer tokens the per-step barrier costs more than the loads it saves.
constexpr int kCPitch = 72;  // staged coefficients: 64 bf16 per token + 8 of padding

template <int MT>
__global__ __launch_bounds__(kMW * kWave) void gather_mfma_shared_kernel(
    const int32_t *__restrict__ rows, const int32_t *__restrict__ n_rows_dev, int max_rows,
    int d_in, const uint16_t *__restrict__ coef_hl, int ldc, const uint16_t *__restrict__ w,
    int64_t d_out, float *__restrict__ out, uint16_t *__restrict__ y, int B, int rps) {
  constexpr int TB = MT * 16;                 // token slots
  constexpr int NT = kMW * kWave;
  constexpr int CE = (TB * 8 + NT - 1) / NT;  // staged 16-byte chunks per thread and step
  __shared__ __align__(16) uint16_t tile[kMW][kMK * kPitch];
  __shared__ __align__(16) uint16_t cst[2][TB * kCPitch];
  const int lane = threadIdx.x % kWave;
  const int wave = wave_id();
  // Waves past the last column still stage coefficients and meet every
  // barrier; their weight loads are clamped to valid columns and they store
  // nothing.
  const int64_t col0 = (static_cast<int64_t>(blockIdx.x) * kMW + wave) * kMCols;
  int n_rows = n_rows_dev ? *n_rows_dev : max_rows;
  n_rows = n_rows < 0 ? 0 : (n_rows > max_rows ? max_rows : n_rows);
  const int r_begin = blockIdx.y * rps;
  const int r_end = r_begin + rps < n_rows ? r_begin + rps : n_rows;
  uint16_t *my = tile[wave];
  // staging of W: lane l moves 16 bytes of rows (l / 8) + 8·q, columns 8·(l mod 8)
  const int64_t scol_raw = col0 + (lane % 8) * 8;
  const int64_t scol = scol_raw < d_out ? scol_raw : d_out - 8;
  const int srow = lane / 8;
  // transpose reads: source lane s of group g addresses row g·8 + half·4 +
  // s / 4, column 16·ns + 4·(s mod 4)
  const int g = lane / 16, s = lane % 16;
  const int tr_off = (g * 8 + s / 4) * kPitch + 4 * (s % 4);
  // staging of coefficients: chunk e = threadIdx.x + NT·i is token e / 8,
  // 16 bytes e mod 8 of that token's 128 bytes for the step (groups of 8
  // positions, hi then lo, as store_coef_hl lays them out); tokens past B
  // stage zeros
  const uint16_t *cptr[CE];
  int coff[CE];
  bool cin[CE], cok[CE];
#pragma unroll
  for (int i = 0; i < CE; ++i) {
    const int e = static_cast<int>(threadIdx.x) + NT * i;
    const int tok = e / 8, ch = e % 8;
    cin[i] = e < TB * 8;
    cok[i] = cin[i] && tok < B;
    cptr[i] = coef_hl + static_cast<int64_t>(cok[i] ? tok : 0) * ldc * 2 + ch * 8;
    coff[i] = tok * kCPitch + ch * 8;
  }
  // A operand of token block m: lane l takes token 16·m + l mod 16, positions
  // 8·(l div 16) .. + 7: hi at that token's 16·(l div 16), lo 8 further
  int aoff[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) aoff[m] = (m * 16 + s) * kCPitch + g * 16;
  f32x4 acc[4][MT];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[n][m] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Software pipeline: the row indices of step k + 4, and the weight rows
  // and coefficient chunks of step k + 2, are requested while step k is
  // computed (the loop body is unrolled by two so every buffer stays in
  // registers).
  auto fetch_idx = [&](int k0, int (&ix)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = k0 + srow + 8 * q;
      ix[q] = r < r_end ? (rows ? rows[r] : r) : -1;
    }
  };
  auto fetch = [&](int k0, const int (&ix)[4], uint4 (&v)[4], uint4 (&cv)[CE]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = ix[q];
      // rows outside [0, d_in) contribute nothing
      v[q] = row >= 0 && row < d_in ? load16(w + static_cast<int64_t>(row) * d_out + scol)
                                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < CE; ++i) cv[i] = cok[i] ? load16(cptr[i] + 2 * k0) : make_uint4(0, 0, 0, 0);
  };
  auto step = [&](const uint4 (&v)[4], const uint4 (&cv)[CE], uint16_t *cbuf) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4 *>(my + (srow + 8 * q) * kPitch + (lane % 8) * 8) = v[q];
#pragma unroll
    for (int i = 0; i < CE; ++i)
      if (cin[i]) *reinterpret_cast<uint4 *>(cbuf + coff[i]) = cv[i];
    // every wave's chunks of this step are in LDS (and every wave has read
    // the buffer's previous contents, two steps ago); weight loads in flight
    // are not waited for
    __syncthreads();
    bf16x8 ahi[MT], alo[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      ahi[m] = *reinterpret_cast<const bf16x8 *>(cbuf + aoff[m]);
      alo[m] = *reinterpret_cast<const bf16x8 *>(cbuf + aoff[m] + 8);
    }
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
  uint4 c0[CE], c1[CE];
  int i0[4], i1[4];
  // every fetch is guarded by its step being below r_end, so coefficient
  // reads stay below ldc (a multiple of the step above the list length);
  // the four waves share r_begin and r_end, so they take the same steps
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
    step(v0, c0, cst[0]);
    if (k0 + 2 * kMK < r_end) {
      fetch(k0 + 2 * kMK, i0, v0, c0);
      fetch_idx(k0 + 4 * kMK, i0);
    }
    if (k0 + kMK < r_end) {
      step(v1, c1, cst[1]);
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
                              void *ws, hipStream_t s, int *parts_out) {
  const int ks = ws ? rotate_mfma_splits(B, d, qb) : 1;
  const bool leave = parts_out != nullptr && ks > 1 && select_takes_parts(d, ks);
  if (parts_out) *parts_out = leave ? ks : 1;
  const int steps = qb / kMK;
  const int kps = (steps + ks - 1) / ks * kMK;
  float *out = ks > 1 ? static_cast<float *>(ws) : x_rot;
  const dim3 grid(static_cast<unsigned>((d / 16 + kMW - 1) / kMW), static_cast<unsigned>(ks));
  const int MT = (B + 15) / 16;
  const auto *xp = static_cast<const uint16_t *>(x);
  const auto *qp = static_cast<const uint16_t *>(qt);
  if (qb % 64 == 0) {
    switch (MT) {
      case 1: hipLaunchKernelGGL(rotate_mfma_staged_kernel<1>, grid, dim3(kMW * kWave), 0, s, xp, qp, out, B, d, qb, kps); break;
      case 2: hipLaunchKernelGGL(rotate_mfma_staged_kernel<2>, grid, dim3(kMW * kWave), 0, s, xp, qp, out, B, d, qb, kps); break;
      case 3: hipLaunchKernelGGL(rotate_mfma_staged_kernel<3>, grid, dim3(kMW * kWave), 0, s, xp, qp, out, B, d, qb, kps); break;
      default: hipLaunchKernelGGL(rotate_mfma_staged_kernel<4>, grid, dim3(kMW * kWave), 0, s, xp, qp, out, B, d, qb, kps); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ks == 1 || leave) return e;
    return sum_parts<float>(out, ks, static_cast<int64_t>(B) * d, x_rot, s);
  }
  switch (MT) {
    case 1: hipLaunchKernelGGL(rotate_mfma_kernel<1>, grid, dim3(kMW * kWave), 0, s, xp, qp, out, B, d, qb, kps); break;
    case 2: hipLaunchKernelGGL(rotate_mfma_kernel<2>, grid, dim3(kMW * kWave), 0, s, xp, qp, out, B, d, qb, kps); break;
    case 3: hipLaunchKernelGGL(rotate_mfma_kernel<3>, grid, dim3(kMW * kWave), 0, s, xp, qp, out, B, d, qb, kps); break;
    default: hipLaunchKernelGGL(rotate_mfma_kernel<4>, grid, dim3(kMW * kWave), 0, s, xp, qp, out, B, d, qb, kps); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ks == 1 || leave) return e;
  return sum_parts<float>(out, ks, static_cast<int64_t>(B) * d, x_rot, s);
}

// Waves of the product kernel for MT token blocks that fit on the chip at
// once: 1024 SIMDs × (512 VGPRs ÷ the kernel's VGPRs, 112 / 156 / 204 / 248
// for MT = 1..4).
int64_t gather_resident_waves(int64_t B) {
  const int mt = static_cast<int>((B + 15) / 16);
  return mt <= 1 ? 4096 : (mt == 2 ? 3072 : 2048);
}

MfmaGatherPlan plan_gather_mfma(int64_t B, int64_t max_rows, int64_t d_out) {
  MfmaGatherPlan p;
  p.col_groups = static_cast<int>((d_out + kMCols * kMW - 1) / (kMCols * kMW));
  const int64_t waves = (d_out + kMCols - 1) / kMCols;
  // as many splits as run in one round of resident waves (a partial second
  // round costs more than the split partial sums save)
  int64_t splits = gather_resident_waves(B) / waves;
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
    default: hipLaunchKernelGGL(gather_mfma_shared_kernel<4>, grid, dim3(kMW * kWave), 0, s, rows, n_rows, mr, di, ch, ld, wp, d_out, out, yy, B, p.rows_per_split); break;
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

// The most split partial sums plan_gather_mfma can ask for at (B, d_out),
// for any row count.
size_t gather_mfma_ws_bound(int64_t B, int64_t d_out) {
  const int64_t waves = (d_out + kMCols - 1) / kMCols;
  int64_t splits = gather_resident_waves(B) / waves;
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
