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
//
// Threshold form (THR): the kept channels are those with |x_rot| >= t (the
// magnitude threshold of the R-Sparse summary page, 研究流程与方法 ·
// R-Sparse框架设计). No rule has to be found: every workgroup compacts its
// split's kept channels at once, and tile 0 also writes how many there are.
#include "common.hpp"
#include "launch.hpp"
#include "select_core.hpp"

namespace larosa {
namespace {

constexpr int kSgWaves = 16;
constexpr int kSgThreads = kSgWaves * kWave;
constexpr int kSgRows = 8;        // kept rows per wave group (loads in flight per lane)
constexpr int kSgListMax = 4096;  // channels of one split (LDS row list)
constexpr int kSgKeysMax = 16384; // channels of the LDS copy of the rotated vector
constexpr int kSgMaxSplitLoads = 32;  // partial sums fetched per round trip

size_t sg_counter_bytes(int tiles) { return (static_cast<size_t>(tiles) * 4 + 255) / 256 * 256; }

template <typename WT, typename OT, int EMAX, bool SWIGLU, bool THR>
__global__ __launch_bounds__(kSgThreads) void select_gather_kernel(
    const float *__restrict__ x_rot, int d, int k, uint32_t thr_key, int E, int tiles,
    int splits, int cps, const WT *__restrict__ w, int64_t d_out, OT *__restrict__ y,
    float *__restrict__ partials, uint32_t *__restrict__ counters,
    int32_t *__restrict__ idx_out, int32_t *__restrict__ count_out) {
  constexpr int V = Elt<WT>::kVec;
  constexpr int TILE = kWave * V;
  constexpr int R = kSgRows;  // loads in flight per lane, list positions per group
  __shared__ SelectSmem<kSgThreads> sm;
  __shared__ CandSmem cs;
  // The row list (indices, then coefficients). Before the list is built the
  // same words hold the first digit's histogram copies.
  // Copies only from 8 key slots per thread: with 4 keys per thread the
  // clear and the sum of the copies cost more than the spread saves.
  constexpr int COPIES = EMAX >= 8 ? 4 : 1;
  constexpr int LIST_WORDS =
      2 * kSgListMax > COPIES * kHistStride ? 2 * kSgListMax : COPIES * kHistStride;
  __shared__ __align__(16) uint32_t lists[LIST_WORDS];
  int32_t *const l_idx = reinterpret_cast<int32_t *>(lists);
  float *const l_val = reinterpret_cast<float *>(lists + kSgListMax);
  // The rotated vector as loaded (fp32 bits, sign included), for the list
  // build; after that the same bytes hold the waves' sums.
  constexpr int KV_WORDS = kSgKeysMax > kSgWaves * TILE ? kSgKeysMax : kSgWaves * TILE;
  __shared__ __align__(16) uint32_t kv[KV_WORDS];
  float(*red)[TILE] = reinterpret_cast<float(*)[TILE]>(kv);
  __shared__ uint32_t s_carry;
  __shared__ int s_last;
  __shared__ float ep[SWIGLU ? TILE : 1];  // the tile's sums, for the SwiGLU epilogue

  const int t = threadIdx.x;
  const int lane = t % kWave;
  const int wave = wave_id();
  const int tile = blockIdx.x % tiles;
  const int split = blockIdx.x / tiles;
  const int c0 = split * cps < d ? split * cps : d;
  const int c1 = c0 + cps < d ? c0 + cps : d;
  const int i0 = t * E;

  // Keys in registers; the signs are kept as one bit per slot (the value of
  // a slot is its key with the sign bit put back), which saves registers.
  uint32_t key[EMAX];
  {
    float v[EMAX];
    load_keys4<EMAX>(x_rot, d, E, key, v);
    // whole 16-byte quads: E and d are multiples of 4
#pragma unroll
    for (int q = 0; q < EMAX / 4; ++q)
      if (4 * q < E && i0 + 4 * q < d)
        *reinterpret_cast<uint4 *>(&kv[i0 + 4 * q]) =
            make_uint4(__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                       __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3]));
  }

  // A chunked ordered compaction over the LDS copy: emit(i, pos) for every
  // channel i of [a, b) with pred(i), pos counting from 0 in index order, one
  // channel per thread and chunk. Returns the count.
  auto compact = [&](int a, int b, auto pred, auto emit) {
    uint32_t carry = 0;
    for (int b0 = a; b0 < b; b0 += kSgThreads) {
      const int i = b0 + t;
      const uint32_t kp = i < b && pred(i);
      const uint32_t incl = block_incl_scan<kSgThreads>(kp, sm.wave_tot);
      if (kp) emit(i, carry + incl - 1);
      if (t == kSgThreads - 1) s_carry = incl;
      __syncthreads();
      carry += s_carry;
      __syncthreads();  // s_carry is rewritten by the next chunk
    }
    return carry;
  };
  auto key_of = [&](int i) { return kv[i] & 0x7FFFFFFFu; };

  // 1. First digit of the rule over all d channels (the same in every
  //    workgroup). A channel whose first digit is above the boundary digit
  //    is kept whatever its later digits. (The threshold form has no rule:
  //    every kept channel is certain.)
  RuleState st{};
  uint32_t digit0 = 0;
  if constexpr (!THR) {
    st = rule_first_digit<kSgThreads, EMAX, COPIES>(key, E, static_cast<uint32_t>(k), sm,
                                                           lists);
    digit0 = st.prefix >> radix_shift(0);
  } else {
    __syncthreads();  // the LDS copy of the vector is complete
  }
  auto certain = [&](int i) {
    if constexpr (THR) return key_of(i) >= thr_key;
    else return (key_of(i) >> radix_shift(0)) > digit0;
  };

  // 2. This split's certain rows, ascending, at the head of the LDS list.
  const int n_cert = static_cast<int>(compact(
      c0, c1, certain,
      [&](int i, uint32_t pos) {
        l_idx[pos] = i;
        l_val[pos] = __uint_as_float(kv[i]);
      }));

  // 3. Start streaming. The row list is read in groups of R positions:
  //    first the certain rows (groups 0 .. CG − 1), then the boundary rows
  //    (the tail, known once the rule is resolved); wave w takes groups w,
  //    w + 16, w + 32, ... This wave's first group of certain rows is
  //    requested now, so the rest of the rule is resolved while it is in
  //    flight. Lanes past the last column read a valid column and store
  //    nothing.
  const int64_t col_raw = static_cast<int64_t>(tile) * TILE + lane * V;
  const int64_t col = col_raw < d_out ? col_raw : d_out - V;
  const int n_cg = (n_cert + R - 1) / R;  // CG
  int n_list = n_cert;
  // A group's list entries are all read first, then its R rows requested
  // back to back. Positions past the group's end (the last group of a
  // segment) repeat the group's last row with coefficient 0: the repeated
  // request hits the same lines as the real one, so it costs no HBM
  // traffic, and no load is conditional.
  auto load_group = [&](int G, uint4(&q)[R], float(&c)[R]) {
    const int lo = G < n_cg ? G * R : n_cert + (G - n_cg) * R;
    const int hi = G < n_cg ? (lo + R < n_cert ? lo + R : n_cert) : (lo + R < n_list ? lo + R : n_list);
    int rows[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int j = lo + u < hi ? lo + u : hi - 1;  // hi > lo for every group read
      rows[u] = l_idx[j];
      const float cv = l_val[j];
      c[u] = lo + u < hi ? cv : 0.f;
    }
#pragma unroll
    for (int u = 0; u < R; ++u) q[u] = load16(w + static_cast<int64_t>(rows[u]) * d_out + col);
  };
  float acc[V];
#pragma unroll
  for (int q = 0; q < V; ++q) acc[q] = 0.f;
  auto consume = [&](const uint4(&q)[R], const float(&c)[R]) {
#pragma unroll
    for (int u = 0; u < R; ++u) {
      float f[V];
      Elt<WT>::unpack(q[u], f);
#pragma unroll
      for (int qq = 0; qq < V; ++qq) acc[qq] = fmaf(c[u], f[qq], acc[qq]);
    }
  };
  uint4 qa[R];
  float ca[R];
  const bool has_a = wave < n_cg;  // the early group
  if (has_a) load_group(wave, qa, ca);

  // 4. The rest of the rule: T, and channels equal to T kept up to `cut`.
  //    Then the first group has (nearly) arrived: it is added up and the
  //    wave's next group of certain rows is requested before the boundary
  //    list is built, so the memory pipe does not run dry meanwhile.
  uint32_t T = 0, cut = 0;
  uint4 qb[R];
  float cb[R];
  bool has_b = false;  // the group requested after the rule
  if constexpr (!THR) {
    rule_finish<kSgThreads, EMAX>(key, E, i0, st, sm, cs, T, cut);
    if (has_a) {
      consume(qa, ca);
      has_b = wave + kSgWaves < n_cg;
      if (has_b) load_group(wave + kSgWaves, qb, cb);
    }
  }
  auto keeps = [&](int i) {
    const uint32_t kk = key_of(i);
    if constexpr (THR) return kk >= thr_key;
    else return kk > T || (kk == T && static_cast<uint32_t>(i) <= cut);
  };

  // 5. The split's kept channels of the boundary digit follow the certain
  //    ones; tile 0 also writes the global ascending index list (parity
  //    checks): the positions of this split's channels follow from the
  //    channels below c1.
  if constexpr (!THR)
    n_list += static_cast<int>(compact(
        c0, c1, [&](int i) { return (key_of(i) >> radix_shift(0)) == digit0 && keeps(i); },
        [&](int i, uint32_t pos) {
          l_idx[n_cert + pos] = i;
          l_val[n_cert + pos] = __uint_as_float(kv[i]);
        }));
  if ((idx_out != nullptr || (THR && count_out != nullptr && c1 == d)) && tile == 0) {
    const uint32_t below = compact(0, c1, keeps, [&](int i, uint32_t pos) {
      if (idx_out != nullptr && i >= c0) idx_out[pos] = i;
    });
    // the last split counts every kept channel
    if (THR && count_out != nullptr && c1 == d && t == 0) *count_out = static_cast<int32_t>(below);
  }
  __syncthreads();  // the vector's LDS copy becomes the waves' sum area

  // 6. Stream the rest of this wave's groups: the one in flight (if any),
  //    then one group of R rows at a time, all R loads in flight.
  const int n_groups = n_cg + (n_list - n_cert + R - 1) / R;
  int G = wave;
  if constexpr (THR) {
    if (has_a) {  // still in flight
      consume(qa, ca);
      G += kSgWaves;
    }
  } else if (has_a) {  // added up after the rule
    G += kSgWaves;
    if (has_b) {
      consume(qb, cb);
      G += kSgWaves;
    }
  }
  for (; G < n_groups; G += kSgWaves) {
    uint4 q[R];
    float c[R];
    load_group(G, q, c);
    consume(q, c);
  }

  // 7. Combine the waves; with one split finish the tile, else partial sums.
#pragma unroll
  for (int q = 0; q < V; ++q) red[wave][lane * V + q] = acc[q];
  __syncthreads();
  const int64_t tile_col0 = static_cast<int64_t>(tile) * TILE;
  // A finished column sum: stored, or staged for the SwiGLU epilogue, which
  // pairs gate column e with up column e + TILE/2 of the tile (rounded to
  // the output type first, as a separate SwiGLU step would see them).
  auto finish = [&](int e, float v) {
    if (SWIGLU) ep[e] = v;
    else Elt<OT>::store(y, tile_col0 + e, v);
  };
  auto epilogue = [&]() {
    if (!SWIGLU) return;
    __syncthreads();
    for (int e = t; e < TILE / 2; e += kSgThreads)
      Elt<OT>::store(y, static_cast<int64_t>(tile) * (TILE / 2) + e,
                     silu_mul(Elt<OT>::round(ep[e]), Elt<OT>::round(ep[TILE / 2 + e])));
  };
  float *part = partials + static_cast<int64_t>(split) * d_out;
  for (int e = t; e < TILE; e += kSgThreads) {
    const int64_t cg = tile_col0 + e;
    if (cg >= d_out) continue;
    float sum = 0.f;
#pragma unroll
    for (int ww = 0; ww < kSgWaves; ++ww) sum += red[ww][e];
    if (splits == 1) {
      finish(e, sum);
    } else {
      // Agent-scope atomic exchange: the value lands at the device-coherent
      // point, like the arrival counter below.
      const float old = __hip_atomic_exchange(part + cg, sum, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
      (void)old;
    }
  }
  if (splits == 1) {
    epilogue();
    return;
  }

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
    float sum = 0.f;
    for (int r0 = 0; r0 < splits; r0 += kSgMaxSplitLoads) {
      float pv[kSgMaxSplitLoads];
#pragma unroll
      for (int i = 0; i < kSgMaxSplitLoads; ++i)
        pv[i] = r0 + i < splits ? __hip_atomic_load(p + (r0 + i) * d_out, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                                : 0.f;
#pragma unroll
      for (int i = 0; i < kSgMaxSplitLoads; ++i)
        if (r0 + i < splits) sum += pv[i];
    }
    finish(e, sum);
  }
  epilogue();
  if (t == 0)
    __hip_atomic_store(&counters[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename WT, typename OT, int EM, bool SW, bool TH>
void launch_sg_k(const SelectGatherArgs &a, const SelectGatherPlan &p, int E, hipStream_t s) {
  uint32_t *counters = static_cast<uint32_t *>(a.ws);
  float *partials =
      reinterpret_cast<float *>(static_cast<char *>(a.ws) + sg_counter_bytes(p.tiles));
  const dim3 grid(static_cast<unsigned>(p.tiles * p.splits)), block(kSgThreads);
  hipLaunchKernelGGL((select_gather_kernel<WT, OT, EM, SW, TH>), grid, block, 0, s, a.x_rot,
                     a.d_in, a.k, a.thr_key, E, p.tiles, p.splits, p.cps,
                     static_cast<const WT *>(a.w), a.d_out, static_cast<OT *>(a.y), partials,
                     counters, a.idx_out, a.count_out);
}

template <typename WT, typename OT, int EM>
void launch_sg_em(const SelectGatherArgs &a, const SelectGatherPlan &p, int E, hipStream_t s) {
  if (a.by_threshold) {
    if (a.swiglu) launch_sg_k<WT, OT, EM, true, true>(a, p, E, s);
    else launch_sg_k<WT, OT, EM, false, true>(a, p, E, s);
  } else {
    if (a.swiglu) launch_sg_k<WT, OT, EM, true, false>(a, p, E, s);
    else launch_sg_k<WT, OT, EM, false, false>(a, p, E, s);
  }
}

template <typename WT, typename OT>
hipError_t launch_sg_t(const SelectGatherArgs &a, const SelectGatherPlan &p, hipStream_t s) {
  const int E = slots_per_thread(a.d_in, kSgThreads);
  if (E <= 4) launch_sg_em<WT, OT, 4>(a, p, E, s);
  else if (E <= 8) launch_sg_em<WT, OT, 8>(a, p, E, s);
  else if (E <= 16) launch_sg_em<WT, OT, 16>(a, p, E, s);
  else return hipErrorInvalidValue;
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

bool select_gather_supported(int64_t d_in) { return d_in >= 1 && d_in <= kSgKeysMax; }

hipError_t launch_select_gather(const SelectGatherArgs &a, hipStream_t s) {
  const SelectGatherPlan p = plan_select_gather(a.d_in, a.d_out, a.w_dt);
  if (p.cps > kSgListMax) return hipErrorInvalidValue;
  if (a.w_dt == kBF16 && a.y_dt == kBF16) return launch_sg_t<uint16_t, uint16_t>(a, p, s);
  if (a.w_dt == kBF16 && a.y_dt == kF32) return launch_sg_t<uint16_t, float>(a, p, s);
  if (a.w_dt == kF32 && a.y_dt == kF32) return launch_sg_t<float, float>(a, p, s);
  return hipErrorInvalidValue;
}

}  // namespace larosa
