// Top-K selection, stage 2 of the method (LaRoSA summary page, 方法详解 ·
// 技术框架: keep the K largest-magnitude entries of the rotated activation,
// zero the rest; the abstract's fixed K gives consistent sparsity).
//
// One 1024-thread workgroup per token. Thread t owns the E consecutive
// channels [t·E, t·E + E) (E = ceil(d/1024) rounded up to a multiple of 4,
// read with 16-byte loads) and keeps their values and keys in registers. The key of a channel is its fp32 bit pattern with the sign bit
// cleared, which orders like |x|. An exact radix select over the 31 key bits
// (digits of 11, 11 and 9 bits, LDS histograms) finds the K-th largest key
// T and how many channels equal to T are still to be taken; those go to the
// lowest indices. One packed block scan of (count > T, count == T) per thread
// then gives every kept channel its position, so the output indices come out
// ascending without a sort.
//
// Row union for B > 1: each token also writes a d-bit mask of its kept
// channels; one workgroup ORs the B masks word by word and compacts the set
// bits in index order, and a grid kernel gathers each token's coefficient
// for every union row. In the layer calls the union list is taken by the
// selection launch itself: every token's workgroup writes its mask with
// write-through (agent-scope) stores, waits for them to complete and takes
// an arrival counter; the last to arrive ORs the masks (agent-scope loads,
// which read the device-coherent point) and writes the list, then resets the
// counter. That saves the union launch.
#include "common.hpp"
#include "launch.hpp"
#include "select_core.hpp"

namespace larosa {
namespace {

constexpr int kThreads = 1024;

// Partial sums of the rotation taken per thread at most: kMaxPartLoads
// 16-byte loads (n_parts · EMAX / 4), all in flight at once.
constexpr int kMaxPartLoads = 16;

// The keys of slots [t·E, t·E + E) of row b when x_rot arrives as n_parts
// k-range partial sums (the row's slice p at part_row + p·pstride,
// pstride = B·d): every partial is loaded
// first, then the slices are added in order p = 0, 1, ... (the order of the
// separate sum, so the bits are the same), and the sums are written to
// x_rot.
template <int EMAX>
__device__ __forceinline__ void load_keys_parts(const float *part_row, int64_t pstride,
                                                int n_parts, float *x_rot_row, int d, int E,
                                                uint32_t (&key)[EMAX], float (&v)[EMAX]) {
  constexpr int NQ = EMAX / 4;
  constexpr int MAXP = kMaxPartLoads / NQ;
  const int i0 = static_cast<int>(threadIdx.x) * E;
  float4 g[MAXP][NQ];
#pragma unroll
  for (int p = 0; p < MAXP; ++p)
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int i = i0 + 4 * q < d ? i0 + 4 * q : d - 4;
      g[p][q] = p < n_parts ? *reinterpret_cast<const float4 *>(part_row + p * pstride + i)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    float4 a = g[0][q];
#pragma unroll
    for (int p = 1; p < MAXP; ++p) {
      if (p < n_parts) {
        a.x += g[p][q].x;
        a.y += g[p][q].y;
        a.z += g[p][q].z;
        a.w += g[p][q].w;
      }
    }
    v[4 * q] = a.x;
    v[4 * q + 1] = a.y;
    v[4 * q + 2] = a.z;
    v[4 * q + 3] = a.w;
    // whole 16-byte quads: E and d are multiples of 4
    if (4 * q < E && i0 + 4 * q < d) *reinterpret_cast<float4 *>(x_rot_row + i0 + 4 * q) = a;
  }
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const bool here = e < E && i0 + e < d;
    key[e] = here ? (__float_as_uint(v[e]) & 0x7FFFFFFFu) : kNoKey;
    v[e] = here ? v[e] : 0.f;
  }
}

// OR of word t over the B tokens' masks, C words in flight per round trip.
// Positions past B repeat the last token's word (OR is idempotent), so the
// loads are unconditional and a batch of up to C tokens takes one round trip.
// With COHERENT the loads are agent-scope (the device-coherent point), for
// masks written by other workgroups of the same launch.
template <int C, bool COHERENT = false>
__device__ __forceinline__ uint32_t or_words(const uint32_t *__restrict__ mask, int B, int nw,
                                             int t) {
  uint32_t word = 0u;
  for (int b = 0; b < B; b += C) {
    uint32_t w[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const uint32_t *p = mask + static_cast<int64_t>(b + i < B ? b + i : B - 1) * nw + t;
      if constexpr (COHERENT)
        w[i] = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        w[i] = *p;
    }
#pragma unroll
    for (int i = 0; i < C; ++i) word |= w[i];
  }
  return word;
}

// The union list of the B masks by one workgroup of kThreads (one mask word
// per thread, d <= 32768): the set bits in index order go to u_idx through
// `stage` (at least d words of LDS), the count to *u_count.
template <bool COHERENT>
__device__ __forceinline__ void union_compact(const uint32_t *__restrict__ mask, int B, int d,
                                              int32_t *__restrict__ u_idx,
                                              int32_t *__restrict__ u_count, uint32_t *stage,
                                              uint32_t *wave_tot) {
  const int t = threadIdx.x;
  const int nw = (d + 31) / 32;
  uint32_t word = 0u;
  if (t < nw)
    word = B <= 16 ? or_words<16, COHERENT>(mask, B, nw, t) : or_words<32, COHERENT>(mask, B, nw, t);
  const uint32_t c = __popc(word);
  const uint32_t incl = block_incl_scan<kThreads>(c, wave_tot);
  uint32_t pos = incl - c;
  while (word) {
    const int bit = __ffs(word) - 1;
    stage[pos++] = static_cast<uint32_t>(t * 32 + bit);
    word &= word - 1u;
  }
  // the total: the wave totals left by the scan
  uint32_t total = 0;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) total += wave_tot[i];
  __syncthreads();
  for (int j = t; j < static_cast<int>(total); j += kThreads)
    u_idx[j] = static_cast<int32_t>(stage[j]);
  if (t == kThreads - 1) *u_count = static_cast<int32_t>(incl);
}

// x_rot is either given (n_parts <= 1) or summed here from n_parts partial
// sums (and written).
template <int EMAX>
__global__ __launch_bounds__(kThreads) void topk_select_kernel(
    float *__restrict__ x_rot, int d, int k, int E, int32_t *__restrict__ idx,
    float *__restrict__ val, float *__restrict__ xs, uint32_t *__restrict__ mask,
    const float *__restrict__ parts, int n_parts, UnionTail ut) {
  __shared__ SelectSmem<kThreads> sm;
  __shared__ uint32_t bitmap[kThreads];  // up to 32768 channels
  __shared__ __align__(16) uint32_t stage[EMAX * kThreads];  // one output row

  const int b = blockIdx.x;
  const int t = threadIdx.x;
  float *xr = x_rot + static_cast<int64_t>(b) * d;
  const int i0 = t * E;

  float v[EMAX];
  uint32_t key[EMAX];
  if (n_parts > 1)
    load_keys_parts<EMAX>(parts + static_cast<int64_t>(b) * d, static_cast<int64_t>(gridDim.x) * d,
                          n_parts, xr, d, E, key, v);
  else
    load_keys4<EMAX>(xr, d, E, key, v);
  if (mask) bitmap[t] = 0u;

  // The first digit counts into histogram copies laid out in `stage`, which
  // is free until the outputs; the rest of the rule works on the channels
  // of the boundary digit, listed in the same free words (the one-token
  // product's rule: T and the index cut-off of the keys equal to T).
  static_assert(EMAX * kThreads * sizeof(uint32_t) >= sizeof(CandSmem), "candidates fit in stage");
  constexpr int kCopies = EMAX >= 8 ? hist_copies_for(EMAX * kThreads) : 1;
  const RuleState st =
      rule_first_digit<kThreads, EMAX, kCopies>(key, E, static_cast<uint32_t>(k), sm, stage);
  uint32_t T, cut;
  rule_finish<kThreads, EMAX>(key, E, i0, st, sm, *reinterpret_cast<CandSmem *>(stage), T, cut);
  bool kept[EMAX];
  uint32_t n_kept = 0;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    kept[e] = rule_keeps<EMAX>(key, e, E, i0, T, cut);
    n_kept += kept[e];
  }
  // the position of the thread's first kept channel in the ascending list
  const uint32_t pos = block_incl_scan<kThreads>(n_kept, sm.wave_tot) - n_kept;

  // Outputs go through LDS: a thread's slots are E consecutive channels, so
  // storing them straight to memory would put a wave's 64 lanes 4·E bytes
  // apart (64 partly written lines per store). Each row (xs, then idx, then
  // val) is laid out in `stage` and copied out with consecutive lanes on
  // consecutive words.
  const int64_t row_xs = static_cast<int64_t>(b) * d;
  const int64_t row_k = static_cast<int64_t>(b) * k;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    if (key[e] & kNoKey) continue;
    const int i = i0 + e;
    if (kept[e] && mask) atomicOr(&bitmap[i >> 5], 1u << (i & 31));
  }
  if (xs) {
#pragma unroll
    for (int q = 0; q < EMAX / 4; ++q)
      if (4 * q < E && i0 + 4 * q < d)  // whole quads: E and d are multiples of 4
        *reinterpret_cast<uint4 *>(&stage[i0 + 4 * q]) = make_uint4(
            kept[4 * q] ? __float_as_uint(v[4 * q]) : 0u, kept[4 * q + 1] ? __float_as_uint(v[4 * q + 1]) : 0u,
            kept[4 * q + 2] ? __float_as_uint(v[4 * q + 2]) : 0u, kept[4 * q + 3] ? __float_as_uint(v[4 * q + 3]) : 0u);
    __syncthreads();
    for (int j = t; j < d; j += kThreads) xs[row_xs + j] = __uint_as_float(stage[j]);
    __syncthreads();
  }
  if (idx) {
    uint32_t p = pos;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (!(key[e] & kNoKey) && kept[e]) stage[p++] = static_cast<uint32_t>(i0 + e);
    __syncthreads();
    for (int j = t; j < k; j += kThreads) idx[row_k + j] = static_cast<int32_t>(stage[j]);
    __syncthreads();
  }
  if (val) {
    uint32_t p = pos;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
      if (!(key[e] & kNoKey) && kept[e]) stage[p++] = __float_as_uint(v[e]);
    __syncthreads();
    for (int j = t; j < k; j += kThreads) val[row_k + j] = __uint_as_float(stage[j]);
  }
  if (mask) {
    __syncthreads();
    const int nw = (d + 31) / 32;
    if (t < nw) {
      uint32_t *mp = mask + static_cast<int64_t>(b) * nw + t;
      if (ut.counter)  // read by the last workgroup of this launch
        __hip_atomic_store(mp, bitmap[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        *mp = bitmap[t];
    }
  }
  if (ut.counter == nullptr) return;
  // The union list, by the last token to arrive: every mask store of this
  // workgroup has completed before its arrival is counted.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  __shared__ int s_last;
  if (t == 0)
    s_last = __hip_atomic_fetch_add(ut.counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             static_cast<uint32_t>(gridDim.x - 1);
  __syncthreads();
  if (!s_last) return;
  union_compact<true>(mask, static_cast<int>(gridDim.x), d, ut.u_idx, ut.u_count, stage,
                      sm.wave_tot);
  if (t == 0) __hip_atomic_store(ut.counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Union of the B masks: one workgroup, one mask word per thread (d <= 32768).
__global__ __launch_bounds__(kThreads) void union_list_kernel(
    const uint32_t *__restrict__ mask, int B, int d, int32_t *__restrict__ u_idx,
    int32_t *__restrict__ u_count) {
  __shared__ uint32_t wave_tot[kThreads / kWave];
  __shared__ uint32_t stage[32 * kThreads];  // the list, copied out coalesced
  union_compact<false>(mask, B, d, u_idx, u_count, stage, wave_tot);
}

// coef[j·B + b] = xs[b, u_idx[j]] for j < |U|; rows past |U| get zeros
// (j < d). A workgroup takes 64 consecutive j and every token: it reads
// xs along j (consecutive lanes on consecutive union rows of one token),
// turns the tile in LDS, and writes coef along b.
constexpr int kUcRows = 64;
constexpr int kUcThreads = 256;
__global__ __launch_bounds__(kUcThreads) void union_coef_kernel(
    const int32_t *__restrict__ u_idx, const int32_t *__restrict__ u_count,
    const float *__restrict__ xs, int B, int d, float *__restrict__ coef) {
  __shared__ float tile[kUcRows][kUcRows + 1];  // [j][b] for up to 64 tokens
  const int t = threadIdx.x;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * kUcRows;
  const int n = *u_count;
  const int jj = t % kUcRows;
  const int64_t j = j0 + jj;
  const int row = j < n ? u_idx[j] : 0;
  for (int b0 = 0; b0 < B; b0 += kUcRows) {
    const int nb = B - b0 < kUcRows ? B - b0 : kUcRows;
    for (int bb = t / kUcRows; bb < nb; bb += kUcThreads / kUcRows)
      tile[jj][bb] = j < n ? xs[static_cast<int64_t>(b0 + bb) * d + row] : 0.f;
    __syncthreads();
    for (int e = t; e < kUcRows * nb; e += kUcThreads) {
      const int r = e / nb, bb = e % nb;
      if (j0 + r < d) coef[(j0 + r) * B + b0 + bb] = tile[r][bb];
    }
    __syncthreads();  // the tile is rewritten by the next token group
  }
}

// The union and its split coefficients in one launch, from the B masks: every
// workgroup ORs the masks (one word per thread), counts the set bits with a
// block scan, and so knows the whole union list; it then takes its own
// kUmRows list positions j: u_idx[j], and the coefficients xs[b, u_idx[j]]
// of every token (zero for j in [|U|, ldc)). Workgroup 0 writes |U|. This
// replaces the selection launch's union tail (an arrival counter and the
// last token's OR, three device round trips after the slowest token) plus a
// coefficient launch.
constexpr int kUmRows = 256;
__global__ __launch_bounds__(kThreads) void union_coef_mask_kernel(
    const uint32_t *__restrict__ mask, const float *__restrict__ xs, int B, int d, int64_t ldc,
    uint16_t *__restrict__ coef_hl, int32_t *__restrict__ u_idx, int32_t *__restrict__ u_count) {
  __shared__ uint32_t wave_tot[kThreads / kWave];
  __shared__ int32_t rows[kUmRows];
  const int t = threadIdx.x;
  const int nw = (d + 31) / 32;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * kUmRows;
  uint32_t word = 0u;
  if (t < nw) word = B <= 16 ? or_words<16>(mask, B, nw, t) : or_words<32>(mask, B, nw, t);
  const uint32_t c = __popc(word);
  const uint32_t incl = block_incl_scan<kThreads>(c, wave_tot);
  uint32_t total = 0;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) total += wave_tot[i];
  int64_t pos = incl - c;
  if (pos < j0 + kUmRows && pos + c > j0) {
    while (word) {
      const int bit = __ffs(word) - 1;
      if (pos >= j0 && pos < j0 + kUmRows) rows[pos - j0] = t * 32 + bit;
      ++pos;
      word &= word - 1u;
    }
  }
  __syncthreads();
  const int64_t n = total;
  if (blockIdx.x == 0 && t == 0) *u_count = static_cast<int32_t>(n);
  for (int r = t; r < kUmRows; r += kThreads)
    if (j0 + r < n) u_idx[j0 + r] = rows[r];
  for (int e = t; e < B * kUmRows; e += kThreads) {
    const int b = e / kUmRows, r = e % kUmRows;
    const int64_t j = j0 + r;
    if (j >= ldc) continue;
    store_coef_hl(coef_hl, ldc, b, j, j < n ? xs[static_cast<int64_t>(b) * d + rows[r]] : 0.f);
  }
}

// Split coefficients of coef[j·B + b] for j < rows; zero for j in [rows, ldc).
__global__ void coef_transpose_kernel(const float *__restrict__ coef, int B, int64_t rows,
                                      int64_t ldc, uint16_t *__restrict__ coef_hl) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= ldc * B) return;
  const int b = static_cast<int>(e / ldc);
  const int64_t j = e % ldc;
  store_coef_hl(coef_hl, ldc, b, j, j < rows ? coef[j * B + b] : 0.f);
}

template <int EMAX>
hipError_t launch_sel(float *x_rot, int B, int d, int k, int E, int32_t *idx, float *val,
                      float *xs, uint32_t *mask, const float *parts, int n_parts,
                      const UnionTail &ut, hipStream_t s) {
  if (n_parts > kMaxPartLoads / (EMAX / 4)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((topk_select_kernel<EMAX>), dim3(B), dim3(kThreads), 0, s, x_rot,
                     d, k, E, idx, val, xs, mask, parts, n_parts, ut);
  return hipGetLastError();
}

int select_emax(int d) {
  const int E = slots_per_thread(d, kThreads);
  return E <= 4 ? 4 : (E <= 8 ? 8 : (E <= 16 ? 16 : 32));
}

}  // namespace

bool select_takes_parts(int d, int n_parts) {
  return n_parts >= 1 && n_parts <= kMaxPartLoads / (select_emax(d) / 4);
}

hipError_t launch_select(float *x_rot, int B, int d, int k, int32_t *idx, float *val, float *xs,
                         uint32_t *mask, hipStream_t s, const float *parts, int n_parts,
                         const UnionTail &ut) {
  const int E = slots_per_thread(d, kThreads);
  if (n_parts <= 1) parts = nullptr;
  if (ut.counter != nullptr && (B < 2 || mask == nullptr || ut.u_idx == nullptr ||
                                ut.u_count == nullptr))
    return hipErrorInvalidValue;
  if (E <= 4) return launch_sel<4>(x_rot, B, d, k, E, idx, val, xs, mask, parts, n_parts, ut, s);
  if (E <= 8) return launch_sel<8>(x_rot, B, d, k, E, idx, val, xs, mask, parts, n_parts, ut, s);
  if (E <= 16) return launch_sel<16>(x_rot, B, d, k, E, idx, val, xs, mask, parts, n_parts, ut, s);
  if (E <= 32) return launch_sel<32>(x_rot, B, d, k, E, idx, val, xs, mask, parts, n_parts, ut, s);
  return hipErrorInvalidValue;
}

hipError_t launch_union(const uint32_t *mask, const float *xs, int B, int d,
                        int32_t *u_idx, int32_t *u_count, float *u_coef,
                        hipStream_t s) {
  hipLaunchKernelGGL(union_list_kernel, dim3(1), dim3(kThreads), 0, s, mask, B, d,
                     u_idx, u_count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !u_coef) return e;
  hipLaunchKernelGGL(union_coef_kernel, dim3(static_cast<unsigned>((d + kUcRows - 1) / kUcRows)),
                     dim3(kUcThreads), 0, s, u_idx, u_count, xs, B, d, u_coef);
  return hipGetLastError();
}

hipError_t launch_union_coef(const int32_t *u_idx, const int32_t *u_count, const float *xs, int B,
                             int d, float *u_coef, hipStream_t s) {
  hipLaunchKernelGGL(union_coef_kernel, dim3(static_cast<unsigned>((d + kUcRows - 1) / kUcRows)),
                     dim3(kUcThreads), 0, s, u_idx, u_count, xs, B, d, u_coef);
  return hipGetLastError();
}

hipError_t launch_union_coef_mask(const uint32_t *mask, const float *xs, int B, int d,
                                  int64_t ldc, void *coefT, int32_t *u_idx, int32_t *u_count,
                                  hipStream_t s) {
  if (d > 32 * kThreads || B < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(union_coef_mask_kernel, dim3(static_cast<unsigned>((ldc + kUmRows - 1) / kUmRows)),
                     dim3(kThreads), 0, s, mask, xs, B, d, ldc, static_cast<uint16_t *>(coefT),
                     u_idx, u_count);
  return hipGetLastError();
}

hipError_t launch_coef_transpose(const float *coef, int B, int64_t max_rows, int64_t ldc,
                                 void *coefT, hipStream_t s) {
  const int64_t n = ldc * B;
  hipLaunchKernelGGL(coef_transpose_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, s, coef, B, max_rows, ldc, static_cast<uint16_t *>(coefT));
  return hipGetLastError();
}

}  // namespace larosa
