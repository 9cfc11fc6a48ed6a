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
// Work split: workgroup (tile, split) owns one column tile of LPR·V columns
// (V = 8 bf16 or 4 fp32 per 16-byte load; LPR lanes per row, 64 or 32) and
// the kept channels of the channel range [split·cps, split·cps + cps). Its
// 16 waves take interleaved groups of 4·(64 / LPR) kept rows: every lane
// holds four 16-byte loads in flight, and one wave load covers 64 / LPR
// rows. The waves' sums are combined in LDS; with more than one split the
// partial sums of a tile are added in split order by the tile's
// last-arriving workgroup, as in the standalone product.
//
// Narrow tiles (LPR = 32: 256 bf16 columns, one 512-byte segment per row)
// serve outputs of at most 12288 columns: 4096 columns then make 16 tiles of
// 16 channel ranges instead of 8 tiles of 32, so a tile's split reduction
// adds 16 partial sums instead of 32 and each workgroup hands over 256 of
// them instead of 512 (11008 → 4096 down product: 20.4 against 21.1 µs;
// 128-column tiles measured 21.7); the 7B q|k|v product (12288 columns)
// takes 48 tiles of 5 ranges instead of 24 of 10 (the 32-layer decoder step
// 4280 against 4306 µs). Wider outputs keep 512-column tiles, which stream
// faster there. With the SwiGLU epilogue a narrow tile takes
// 128 gate and the matching 128 up columns of the interleaved layout, so it
// still finishes whole channels of h.
//
// The grid is sized to at most one workgroup per CU (256 on MI355X), which
// keeps every workgroup resident for the whole launch.
//
// Chained form (CHAIN, the gate|up linear of a one-token MLP): after the
// product the workgroups go on to the down linear's rotation, x_rot2 = h·Q2
// (block-diagonal Q2, blocks of at most 4096), without a second launch and
// without a grid-wide barrier. Each tile's finishing workgroup writes its 256
// channels of h = SiLU(gate)·up with agent-scope atomic stores, waits for
// them to complete and then writes this launch's epoch into the tile's flag
// word. Every workgroup then takes 16 consecutive channels of x_rot2 at a
// time from a work queue, one wave per channel: each wave first requests its
// channels' Q2 rows, which do not depend on h; then one lane per workgroup
// waits (bounded, polling gently) until every tile that covers the channels'
// Q2 blocks carries this epoch, the workgroup copies those blocks of h into
// LDS with agent-scope atomic loads, and the waves take their dot products.
// So the rotation's weight traffic overlaps the product's tail (the
// stragglers and the split reduction) instead of following it. The dot
// products use the one-token rotation kernel's order (lane-strided 16-byte
// chunks, then a wave sum), so x_rot2 has the same bits as that kernel's.
//
// The epoch is kept on the device, so a captured graph replays correctly:
// every workgroup reads the control block's epoch word at its start and uses
// that number + 1 (1 .. 2^31, wrapping). The workgroup that finishes the last
// tile (so every workgroup has arrived, and has read the word) stores the new
// epoch there. The work queue is one of two counters, chosen by the epoch's
// parity; a launch zeroes the other one, which the previous launch used, for
// the next. Flags of earlier launches carry other epochs, and a wait that
// gives up leaves no state ahead of the next launch, so nothing has to be
// reset between calls.
//
// Threshold form (THR): the kept channels are those with |x_rot| >= t (the
// magnitude threshold of the R-Sparse summary page, 研究流程与方法 ·
// R-Sparse框架设计). No rule has to be found: every workgroup compacts its
// split's kept channels at once, and tile 0 also writes how many there are.
#include "common.hpp"
#include "launch.hpp"
#include "select_core.hpp"

#include <type_traits>

namespace larosa {
namespace {

constexpr int kSgWaves = 16;
constexpr int kSgThreads = kSgWaves * kWave;
// Loads in flight per lane (rows per lane and group). Four measured faster
// than eight for both tile widths (7B gate|up 24.8 against 25.2 µs, down
// 17.9 against 18.9 µs at 256-column tiles): a wave's groups are finer, so
// the waves of a workgroup finish closer together.
constexpr int kSgRows = 4;
constexpr int kSgListMax = 4096;  // channels of one split (LDS row list)
constexpr int kSgKeysMax = 16384; // channels of the LDS copy of the rotated vector
constexpr int kSgMaxSplitLoads = 32;  // partial sums fetched per round trip

size_t sg_counter_bytes(int tiles) { return (static_cast<size_t>(tiles) * 4 + 255) / 256 * 256; }

constexpr int kChainChunks = 8;  // 16-byte chunks per lane of a Q2 row: q_block <= 4096

// Epilogue forms of the product.
constexpr int kEpiPlain = 0;  // y stored as summed (or SwiGLU, with SWIGLU)
constexpr int kEpiChain = 1;  // the SwiGLU product chained into the next rotation
constexpr int kEpiRope = 2;   // RoPE on the q and k heads of a q|k|v product

// The RoPE table travels only with the RoPE form (a 1 KB kernel argument).
struct NoRope {};
template <int EPI>
using RopeParam = std::conditional_t<EPI == kEpiRope, RopeArgs, NoRope>;

template <typename WT, typename OT, int EMAX, bool SWIGLU, bool THR, int EPI, int LPR>
__global__ __launch_bounds__(kSgThreads) void select_gather_kernel(
    const float *__restrict__ x_rot, int d, int k, uint32_t thr_key, int E, int tiles,
    int splits, int cps, const WT *__restrict__ w, int64_t d_out, OT *__restrict__ y,
    float *__restrict__ partials, uint32_t *__restrict__ counters,
    int32_t *__restrict__ idx_out, int32_t *__restrict__ count_out, ChainArgs chain,
    RopeParam<EPI> rope) {
  constexpr bool CHAIN = EPI == kEpiChain;
  constexpr bool ROPE = EPI == kEpiRope;
  static_assert(!CHAIN || (SWIGLU && !THR), "the chain follows the SwiGLU product");
  static_assert(!ROPE || (!SWIGLU && !THR), "RoPE follows a plain product");
  static_assert(LPR == kWave || LPR == 32, "lanes per row");
  constexpr int V = Elt<WT>::kVec;
  constexpr int RPW = kWave / LPR;  // rows per wave load
  constexpr int TILE = LPR * V;     // columns per tile
  constexpr int R = kSgRows;        // loads in flight per lane
  constexpr int GP = R * RPW;       // list positions per group
  // SwiGLU tiles: the first half of a tile's columns are gate columns, the
  // second half the matching up columns. In the interleaved layout (blocks of
  // IB = 32·V columns, gate and up alternating) a tile of SEG + SEG columns
  // is segment (tile % TPP) of the interleaved pair (tile / TPP).
  constexpr int SEG = TILE / 2;
  constexpr int IB = 32 * V;
  constexpr int TPP = IB / SEG;
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
  __shared__ float ep[SWIGLU || ROPE ? TILE : 1];  // the tile's sums, for the epilogue

  const int t = threadIdx.x;
  const int lane = t % kWave;
  const int wave = wave_id();
  const int sub = lane / LPR;  // the lane's row slot within a wave load
  // (chain) this launch's epoch from the control block; the first workgroup
  // zeroes the queue counter that the next launch will use
  __shared__ uint32_t s_epoch;
  uint32_t *const ctl32 = reinterpret_cast<uint32_t *>(chain.ctl + 2);  // [epoch word, tiles done]
  if constexpr (CHAIN)
    if (t == 0) {
      const uint32_t e =
          __hip_atomic_load(&ctl32[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 0x7fffffffu;
      s_epoch = e + 1u;
      if (blockIdx.x == 0)
        __hip_atomic_store(&chain.ctl[(e + 2u) & 1u], uint64_t{0}, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  const int tile = blockIdx.x % tiles;
  const int split = blockIdx.x / tiles;
  // global column of the tile's column e
  auto gcol = [&](int e) -> int64_t {
    if constexpr (SWIGLU)
      return static_cast<int64_t>(tile / TPP) * (2 * IB) + (tile % TPP) * SEG + (e / SEG) * IB +
             e % SEG;
    else
      return static_cast<int64_t>(tile) * TILE + e;
  };
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
  //    workgroup): the boundary bin [blo, bhi) of keys (key bits 30..20),
  //    which holds the K-th largest. A channel whose key is at or above bhi
  //    is kept whatever the rest of the rule says. (The threshold form has
  //    no rule: every kept channel is certain.)
  RuleState st{};
  uint32_t blo = 0, bhi = 0;
  if constexpr (!THR) {
    st = rule_first_digit<kSgThreads, EMAX, COPIES>(key, E, static_cast<uint32_t>(k), sm, lists);
    blo = (st.prefix >> radix_shift(0)) << radix_shift(0);
    bhi = blo + (1u << radix_shift(0));
  } else {
    __syncthreads();  // the LDS copy of the vector is complete
  }
  auto certain = [&](int i) {
    if constexpr (THR) return key_of(i) >= thr_key;
    else return key_of(i) >= bhi;
  };

  // 2. This split's certain rows, ascending, at the head of the LDS list.
  const int n_cert = static_cast<int>(compact(
      c0, c1, certain,
      [&](int i, uint32_t pos) {
        l_idx[pos] = i;
        l_val[pos] = __uint_as_float(kv[i]);
      }));

  // 3. Start streaming. The row list is read in groups of GP positions:
  //    first the certain rows (groups 0 .. CG − 1), then the boundary rows
  //    (the tail, known once the rule is resolved); wave w takes groups w,
  //    w + 16, w + 32, ... Within a group, lane slot `sub` takes positions
  //    sub, sub + RPW, ... This wave's first group of certain rows is
  //    requested now, so the rest of the rule is resolved while it is in
  //    flight. Lanes past the last column read a valid column and store
  //    nothing.
  const int64_t col_raw = gcol((lane % LPR) * V);
  const int64_t col = col_raw < d_out ? col_raw : d_out - V;
  const int n_cg = (n_cert + GP - 1) / GP;  // CG
  int n_list = n_cert;
  // A group's list entries are all read first, then the lane's R rows
  // requested back to back. Positions past the group's end (the last group
  // of a segment) repeat the group's last row with coefficient 0: the
  // repeated request hits the same lines as the real one, so it costs no
  // HBM traffic, and no load is conditional.
  auto load_group = [&](int G, uint4(&q)[R], float(&c)[R]) {
    const int lo = G < n_cg ? G * GP : n_cert + (G - n_cg) * GP;
    const int hi = G < n_cg ? (lo + GP < n_cert ? lo + GP : n_cert) : (lo + GP < n_list ? lo + GP : n_list);
    int rows[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int pos = lo + u * RPW + sub;
      const int j = pos < hi ? pos : hi - 1;  // hi > lo for every group read
      rows[u] = l_idx[j];
      const float cv = l_val[j];
      c[u] = pos < hi ? cv : 0.f;
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
        c0, c1, [&](int i) { return key_of(i) >= blo && key_of(i) < bhi && keeps(i); },
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
  const int n_groups = n_cg + (n_list - n_cert + GP - 1) / GP;
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

  // 7. Combine the row slots of each wave (lane butterflies), then the
  //    waves; with one split finish the tile, else partial sums.
  if constexpr (RPW > 1) {
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1)
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] += __shfl_xor(acc[q], off, kWave);
  }
  if (lane < LPR)
#pragma unroll
    for (int q = 0; q < V; ++q) red[wave][lane * V + q] = acc[q];
  __syncthreads();
  const int64_t tile_col0 = static_cast<int64_t>(tile) * TILE;
  // A finished column sum: stored, or staged for the SwiGLU epilogue, which
  // pairs gate column e with up column e + TILE/2 of the tile (rounded to
  // the output type first, as a separate SwiGLU step would see them).
  auto finish = [&](int e, float v) {
    if (SWIGLU || ROPE) ep[e] = v;
    else Elt<OT>::store(y, gcol(e), v);
  };
  auto epilogue = [&]() {
    if constexpr (ROPE) {
      // The tile holds whole heads (dh divides TILE). Each sum is rounded to
      // the output type first, as a separate RoPE step would read it; the
      // table and the arithmetic are larosa_rope's.
      __syncthreads();
      const int dh = rope.tab.dh, half = dh / 2;
      for (int e = t; e < TILE; e += kSgThreads) {
        const int64_t col = tile_col0 + e;
        if (col >= d_out) continue;
        if (col >= rope.rot_cols) {
          Elt<OT>::store(y, col, Elt<OT>::round(ep[e]));
          continue;
        }
        const int j = static_cast<int>(col % dh);
        const int i = j % half;
        const int h0 = e - j;  // the head's first column in the tile
        const float a = Elt<OT>::round(ep[h0 + i]), bb = Elt<OT>::round(ep[h0 + i + half]);
        const float cs = rope.tab.cs[i], sn = rope.tab.sn[i];
        Elt<OT>::store(y, col, j < half ? rope_lo(a, bb, cs, sn) : rope_hi(a, bb, cs, sn));
      }
      return;
    }
    if (!SWIGLU) return;
    __syncthreads();
    if constexpr (CHAIN) {
      // h with agent-scope atomic stores (two bf16 per word), then the tile's
      // flag once every store has completed
      uint32_t *h32 = reinterpret_cast<uint32_t *>(y) + static_cast<int64_t>(tile) * (TILE / 4);
      for (int e = t; e < TILE / 4; e += kSgThreads) {
        const float h0 = silu_mul(Elt<OT>::round(ep[2 * e]), Elt<OT>::round(ep[TILE / 2 + 2 * e]));
        const float h1 =
            silu_mul(Elt<OT>::round(ep[2 * e + 1]), Elt<OT>::round(ep[TILE / 2 + 2 * e + 1]));
        const uint32_t word = static_cast<uint32_t>(f32_to_bf16(h0)) |
                              (static_cast<uint32_t>(f32_to_bf16(h1)) << 16);
        __hip_atomic_store(h32 + e, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t == 0) {
        const uint32_t epoch = s_epoch;
        __hip_atomic_store(&chain.tile_flag[tile], epoch, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        // the last tile finished: every workgroup has read the epoch word
        if (__hip_atomic_fetch_add(&ctl32[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            static_cast<uint32_t>(tiles - 1)) {
          __hip_atomic_store(&ctl32[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&ctl32[0], epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      return;
    }
    for (int e = t; e < TILE / 2; e += kSgThreads)
      Elt<OT>::store(y, static_cast<int64_t>(tile) * (TILE / 2) + e,
                     silu_mul(Elt<OT>::round(ep[e]), Elt<OT>::round(ep[TILE / 2 + e])));
  };
  float *part = partials + static_cast<int64_t>(split) * d_out;
  for (int e = t; e < TILE; e += kSgThreads) {
    const int64_t cg = gcol(e);
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
  } else {
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
    if (s_last) {
      for (int e = t; e < TILE; e += kSgThreads) {
        const int64_t cg = gcol(e);
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
  }
  if constexpr (!CHAIN) return;

  // 8. (chain) x_rot2[j] = h[blk(j)·qb ..]·Qt2[j, :]. Workgroups take chunks
  //    of 16 consecutive channels (one per wave) from the launch's queue as
  //    they finish the product, so the ones that finish early (not a tile's
  //    last split) do most of the rotation. A chunk's Q2 rows are requested
  //    at once, before its block of h is known to be complete; then one lane
  //    waits (bounded) until every product tile of the block has written its
  //    flag, the workgroup copies the block of h into LDS with agent-scope
  //    loads, and the waves take their dot products. The next chunk is
  //    grabbed, and its rows requested, before the current one is summed.
  //    Barriers here are bare s_barrier after an LDS wait, so they do not
  //    wait for the rows in flight.
  const int qb2 = chain.qb;
  const int chunks = qb2 / 8;
  const int n_chunks = (chain.f + kSgWaves - 1) / kSgWaves;
  __shared__ int s_next[2];  // the chunk after the current one, by iteration parity
  __shared__ int s_hblk[2];  // blocks of h staged in LDS: [first, last], -1 when none
  uint64_t *hs = reinterpret_cast<uint64_t *>(kv);  // staged h (two blocks at most)
  const uint64_t *h64 = reinterpret_cast<const uint64_t *>(y);
  auto bar = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS traffic is done
    __builtin_amdgcn_s_barrier();
  };
  const uint32_t epoch = s_epoch;
  uint64_t *const queue = chain.ctl + (epoch & 1u);
  // A grab is issued by thread 0 and its result read one iteration later, so
  // the round trip overlaps a chunk's work.
  auto grab = [&]() {
    return __hip_atomic_fetch_add(queue, uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto chunk_of = [&](uint64_t w) {
    return w < static_cast<uint64_t>(n_chunks) ? static_cast<int>(w) : n_chunks;
  };
  auto load_row = [&](int j, uint4(&q)[kChainChunks]) {
    const uint16_t *row = chain.qt + static_cast<int64_t>(j < chain.f ? j : chain.f - 1) * qb2;
#pragma unroll
    for (int i = 0; i < kChainChunks; ++i) {
      const int cc = lane + kWave * i;
      q[i] = cc < chunks ? load16(row + cc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  uint64_t pending = 0;  // thread 0: the grab in flight
  if (t == 0) {
    s_hblk[0] = -1;
    s_hblk[1] = -1;
    s_next[0] = chunk_of(grab());  // the first chunk (waits once)
    pending = grab();
  }
  bar();  // also: every wave is past the product's last use of LDS
  int cur = s_next[0];
  uint4 rq[kChainChunks], rn[kChainChunks];
  if (cur < n_chunks) load_row(cur * kSgWaves + wave, rq);
  bool gave_up = false;
  int par = 1;
  while (cur < n_chunks) {
    const int jc0 = cur * kSgWaves;
    const int jc1 = jc0 + kSgWaves < chain.f ? jc0 + kSgWaves : chain.f;
    const int b_lo = jc0 / qb2, b_hi = (jc1 - 1) / qb2;
    if (b_lo != s_hblk[0] || b_hi != s_hblk[1]) {
      // wait for every product tile of these blocks, then stage them (the
      // barrier first: no wave still reads the blocks staged before)
      const int hlo = b_lo * qb2, hhi = (b_hi + 1) * qb2;
      const int t_lo = hlo / (TILE / 2), t_hi = (hhi - 1) / (TILE / 2);
      if (wave == 0) {
        uint32_t spins = 0;
        for (;;) {
          bool in = true;
          for (int tt = t_lo + lane; tt <= t_hi; tt += kWave)
            in = in && __hip_atomic_load(&chain.tile_flag[tt], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT) == epoch;
          if (__all(in)) break;
          if (spins++ >= chain.spin_limit) {
            gave_up = true;
            break;
          }
          __builtin_amdgcn_s_sleep(8);
        }
      }
      bar();
      for (int i = t; i < (hhi - hlo) / 4; i += kSgThreads)
        hs[i] = __hip_atomic_load(h64 + hlo / 4 + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (t == 0) {
        s_hblk[0] = b_lo;
        s_hblk[1] = b_hi;
      }
    }
    if (t == 0) s_next[par] = chunk_of(pending);
    bar();  // the staged h, s_hblk and s_next[par] are visible
    const int nxt = s_next[par];
    par ^= 1;
    if (t == 0 && nxt < n_chunks) pending = grab();
    if (nxt < n_chunks) load_row(nxt * kSgWaves + wave, rn);  // in flight during this chunk
    const int j = jc0 + wave;
    if (j < jc1) {
      const uint4 *hb = reinterpret_cast<const uint4 *>(hs) + ((j / qb2) * qb2 - b_lo * qb2) / 8;
      float accr = 0.f;
#pragma unroll
      for (int i = 0; i < kChainChunks; ++i) {
        const int cc = lane + kWave * i;
        const uint4 hx = cc < chunks ? hb[cc] : make_uint4(0, 0, 0, 0);
        float xf[8], qf[8];
        Elt<uint16_t>::unpack(hx, xf);
        Elt<uint16_t>::unpack(rq[i], qf);
#pragma unroll
        for (int v = 0; v < 8; ++v) accr = fmaf(xf[v], qf[v], accr);
      }
      const float sum = wave_sum(accr);
      if (lane == 0) chain.x_rot[j] = sum;
    }
    cur = nxt;
#pragma unroll
    for (int i = 0; i < kChainChunks; ++i) rq[i] = rn[i];
  }
  if (gave_up && lane == 0 && chain.status != nullptr)
    __hip_atomic_store(chain.status, kStatusTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename WT, typename OT, int EM, bool SW, bool TH, int EPI, int LPR>
void launch_sg_l(const SelectGatherArgs &a, const SelectGatherPlan &p, int E, hipStream_t s) {
  uint32_t *counters = static_cast<uint32_t *>(a.ws);
  float *partials =
      reinterpret_cast<float *>(static_cast<char *>(a.ws) + sg_counter_bytes(p.tiles));
  const dim3 grid(static_cast<unsigned>(p.tiles * p.splits)), block(kSgThreads);
  const ChainArgs &chain = a.chain;
  RopeParam<EPI> rope{};
  if constexpr (EPI == kEpiRope) rope = a.rope;
  hipLaunchKernelGGL((select_gather_kernel<WT, OT, EM, SW, TH, EPI, LPR>), grid, block, 0, s, a.x_rot,
                     a.d_in, a.k, a.thr_key, E, p.tiles, p.splits, p.cps,
                     static_cast<const WT *>(a.w), a.d_out, static_cast<OT *>(a.y), partials,
                     counters, a.idx_out, a.count_out, chain, rope);
}

// Narrow tiles exist for bf16 weights only.
template <typename WT, typename OT, int EM, bool SW, bool TH, int EPI>
void launch_sg_k(const SelectGatherArgs &a, const SelectGatherPlan &p, int E, hipStream_t s) {
  if constexpr (sizeof(WT) == 2)
    if (p.lpr == 32) return launch_sg_l<WT, OT, EM, SW, TH, EPI, 32>(a, p, E, s);
  launch_sg_l<WT, OT, EM, SW, TH, EPI, kWave>(a, p, E, s);
}

template <typename WT, typename OT, int EM>
void launch_sg_em(const SelectGatherArgs &a, const SelectGatherPlan &p, int E, hipStream_t s) {
  if (a.by_threshold) {
    if (a.swiglu) launch_sg_k<WT, OT, EM, true, true, kEpiPlain>(a, p, E, s);
    else launch_sg_k<WT, OT, EM, false, true, kEpiPlain>(a, p, E, s);
  } else {
    if constexpr (sizeof(WT) == 2 && sizeof(OT) == 2) {
      if (a.chain.qt != nullptr) {
        launch_sg_k<WT, OT, EM, true, false, kEpiChain>(a, p, E, s);
        return;
      }
      if (a.rope.rot_cols > 0) {
        launch_sg_k<WT, OT, EM, false, false, kEpiRope>(a, p, E, s);
        return;
      }
    }
    if (a.swiglu) launch_sg_k<WT, OT, EM, true, false, kEpiPlain>(a, p, E, s);
    else launch_sg_k<WT, OT, EM, false, false, kEpiPlain>(a, p, E, s);
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
  // narrow tiles (256 columns) for bf16 outputs of at most 12288 columns
  p.lpr = w_dt == kBF16 && d_out <= 12288 ? 32 : kWave;
  const int64_t tile_cols = static_cast<int64_t>(p.lpr) * (w_dt == kF32 ? 4 : 8);
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

bool chain_supported(int64_t q_block, int64_t f) {
  return q_block >= 8 && q_block % 8 == 0 && q_block <= 8 * kWave * kChainChunks && f % q_block == 0;
}

hipError_t launch_select_gather(const SelectGatherArgs &a, hipStream_t s) {
  const SelectGatherPlan p = plan_select_gather(a.d_in, a.d_out, a.w_dt);
  if (p.cps > kSgListMax) return hipErrorInvalidValue;
  if (a.chain.qt != nullptr &&
      (!a.swiglu || a.by_threshold || a.w_dt != kBF16 || a.y_dt != kBF16 ||
       !chain_supported(a.chain.qb, a.chain.f) || a.d_out != 2 * a.chain.f ||
       a.chain.tile_flag == nullptr || a.chain.ctl == nullptr || a.chain.x_rot == nullptr ||
       p.tiles > a.chain.f / 64 + 1))  // the flag words chain_flag_bytes(f) provides
    return hipErrorInvalidValue;
  if (a.rope.rot_cols > 0 &&
      (a.swiglu || a.by_threshold || a.chain.qt != nullptr || a.w_dt != kBF16 ||
       a.y_dt != kBF16 || a.rope.tab.dh < 2 || a.rope.tab.dh % 2 ||
       a.rope.tab.dh > 2 * kRopeMaxHalf || (p.lpr * 8) % a.rope.tab.dh ||
       a.rope.rot_cols % a.rope.tab.dh || a.rope.rot_cols > a.d_out))
    return hipErrorInvalidValue;
  if (a.w_dt == kBF16 && a.y_dt == kBF16) return launch_sg_t<uint16_t, uint16_t>(a, p, s);
  if (a.w_dt == kBF16 && a.y_dt == kF32) return launch_sg_t<uint16_t, float>(a, p, s);
  if (a.w_dt == kF32 && a.y_dt == kF32) return launch_sg_t<float, float>(a, p, s);
  return hipErrorInvalidValue;
}

}  // namespace larosa
