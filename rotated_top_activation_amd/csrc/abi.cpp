// C ABI of liblarosa: argument checks on the host, workspace carving, and
// the step sequence of each call. Every argument is checked before any HIP
// call, so an invalid call enqueues nothing and leaves outputs untouched.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/larosa.h"
#include "launch.hpp"

using namespace larosa;

namespace {

constexpr int64_t kMaxD = 32768;  // select keeps a token's channels in one workgroup
constexpr int64_t kMaxB = 64;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(int dt) { return dt == LAROSA_F32 || dt == LAROSA_BF16; }
int vec_of(int dt) { return dt == LAROSA_F32 ? 4 : 8; }
size_t align256(size_t n) { return (n + 255) / 256 * 256; }

int device_status() {
  static std::once_flag once;
  static int status = LAROSA_OK;
  std::call_once(once, [] {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) status = LAROSA_ERR_NO_DEVICE;
  });
  return status;
}

int launched(hipError_t e) { return e == hipSuccess ? LAROSA_OK : LAROSA_ERR_LAUNCH; }

// The no-throw wall of the C ABI: an exception from the host code of a call
// (std::call_once, std::mutex, allocation inside the runtime) becomes a
// status instead of crossing into C.
template <typename F>
int guard(F &&body) noexcept {
  try {
    return body();
  } catch (...) {
    return LAROSA_ERR_INTERNAL;
  }
}
template <typename F>
size_t guard_size(F &&body) noexcept {
  try {
    return body();
  } catch (...) {
    return 0;
  }
}

hipStream_t stream_of(larosa_stream_t s) { return static_cast<hipStream_t>(s); }

// Workspace carving. Every call that takes a workspace uses the same prefix,
// computed from (B, d_in, d_out) only, so calls of one shape can share one
// workspace in any order:
//   mask   B per-token bit masks of the selection (rewritten by each select)
//   gather the vector product's tile counters (must stay zero between
//          calls) and split partial sums
//   mfma   transposed coefficients and split partial sums of the matrix-core
//          forms (B >= 16, bf16 weights; rewritten by each call)
// larosa_layer_forward then adds its own areas, and the fused kernel's region
// (whose synchronisation words must also stay zero) comes last.
struct Prefix {
  size_t status = 0, mask = 0, gather = 0, flags = 0, mfma_coef = 0, mfma_parts = 0, end = 0;
};

// The first 256 bytes of every layer-call workspace: word 0 holds the
// device-side status (LAROSA_ERR_TIMEOUT from a bounded wait that gave up),
// word 1 the LAROSA_VALIDATE check's flag, word 2 the selection launch's
// arrival counter for the row union (zero between calls).
constexpr size_t kStatusBytes = 256;
UnionTail union_tail(char *status_area, int32_t *u_idx, int32_t *u_count) {
  UnionTail ut;
  ut.counter = reinterpret_cast<uint32_t *>(status_area) + 2;
  ut.u_idx = u_idx;
  ut.u_count = u_count;
  return ut;
}
static_assert(kStatusTimeout == LAROSA_ERR_TIMEOUT, "device status code");

bool mfma_region(int64_t B, int w_dt) { return w_dt == LAROSA_BF16 && B >= kMfmaMinB && B <= kMaxB; }

// rows_bound: the longest row list a product over this workspace takes.
Prefix prefix_for(int64_t B, int64_t d_in, int64_t d_out, int64_t rows_bound, int w_dt) {
  Prefix P;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  P.status = take(kStatusBytes);
  P.mask = take(static_cast<size_t>(B) * mask_words(static_cast<int>(d_in)) * 4);
  size_t g = gather_batch_ws_bytes(static_cast<int>(B), rows_bound, d_out, w_dt);
  if (B == 1) {
    // the one-token product with the selection folded in (same counters)
    const size_t sg = select_gather_ws_bytes(d_in, d_out, w_dt);
    g = sg > g ? sg : g;
  }
  P.gather = take(g);
  // one token: the chained product's tile flags and control block (zero
  // before first use; the chain keeps its epoch and queues there)
  if (B == 1) P.flags = take(chain_flag_bytes(d_out / 2));
  if (mfma_region(B, w_dt)) {
    P.mfma_coef = take(static_cast<size_t>(B) * mfma_coef_ld(rows_bound) * 4);
    size_t parts = rotate_mfma_ws_bound(B, d_in);
    const size_t g = gather_mfma_ws_bound(B, d_out);
    P.mfma_parts = take(parts > g ? parts : g);
  }
  P.end = off;
  return P;
}

struct Layout {
  Prefix p;
  size_t x_rot = 0, idx = 0, val = 0, xs = 0, u_idx = 0, u_cnt = 0, u_coef = 0, fused = 0,
         total = 0;
};

Layout layout_for(int64_t B, int64_t d_in, int64_t d_out, int64_t k, int w_dt) {
  Layout L;
  // The vector product's area covers both the sparse call (max_rows =
  // min(d_in, B·k)) and the dense call (max_rows = d_in): the dense plan has
  // at least as many splits.
  L.p = prefix_for(B, d_in, d_out, d_in, w_dt);
  size_t off = L.p.end;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.x_rot = take(static_cast<size_t>(B) * d_in * 4);
  L.idx = take(static_cast<size_t>(B) * k * 4);
  L.val = take(static_cast<size_t>(B) * k * 4);
  L.xs = take(static_cast<size_t>(B) * d_in * 4);
  L.u_idx = take(static_cast<size_t>(d_in) * 4);
  L.u_cnt = take(4);
  L.u_coef = take(static_cast<size_t>(d_in) * B * 4);
  L.total = off;
  return L;
}

// The fused kernel's region follows the unfused layout, so calls in either
// mode can share one workspace.
Layout layout_with_fused(int64_t B, int64_t d_in, int64_t d_out, int64_t k, int w_dt) {
  Layout L = layout_for(B, d_in, d_out, k, w_dt);
  L.fused = L.total;
  L.total += align256(plan_fused(d_in, d_out, k, w_dt, kFusedMaxGrid).bytes);
  return L;
}

// The low-rank compensated layer: the layer's areas sized for d_in + r rows
// (the product runs over W_ext = [W'; B_r]), then the projection's partial
// sums and the extended row list.
struct LrLayout {
  Layout l;
  size_t part = 0, rows_ext = 0, n_ext = 0, total = 0;
};

LrLayout lowrank_layout(int64_t B, int64_t d_in, int64_t d_out, int64_t k, int64_t r, int w_dt) {
  LrLayout L;
  L.l = layout_for(B, d_in + r, d_out, k, w_dt);
  size_t off = L.l.total;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.part = take(lowrank_part_bytes(B, d_in, r));
  L.rows_ext = take(static_cast<size_t>(d_in + r) * 4);
  L.n_ext = take(4);
  L.total = off;
  return L;
}

constexpr int64_t kMaxRank = 256;

int check_sizes(int64_t B, int64_t d, int64_t k) {
  if (B < 0 || B > kMaxB) return LAROSA_ERR_INVALID_ARG;
  if (d < 1 || d > kMaxD) return LAROSA_ERR_SHAPE;
  if (d % 4) return LAROSA_ERR_ALIGNMENT;
  if (k < 1 || k > d) return LAROSA_ERR_INVALID_ARG;
  return LAROSA_OK;
}

int check_rotation(int64_t d, int64_t qb, int q_dt) {
  if (qb < 1 || qb > d || d % qb) return LAROSA_ERR_SHAPE;
  if (qb % vec_of(q_dt)) return LAROSA_ERR_ALIGNMENT;
  return LAROSA_OK;
}

// The execution mode without the LAROSA_ROTATE_FP64 and LAROSA_VALIDATE
// flags, or -1 when the mode holds any other bit.
int base_mode(int mode) {
  if ((mode & LAROSA_PREROTATED) && (mode & LAROSA_ROTATE_FP64)) return -1;
  const int m = mode & ~(LAROSA_ROTATE_FP64 | LAROSA_VALIDATE | LAROSA_PREROTATED);
  return m == LAROSA_UNFUSED || m == LAROSA_FUSED ? m : -1;
}

bool fp64_rotation(int mode) { return (mode & LAROSA_ROTATE_FP64) != 0; }
bool prerotated(int mode) { return (mode & LAROSA_PREROTATED) != 0; }
bool validating(int mode) { return (mode & LAROSA_VALIDATE) != 0; }

// LAROSA_VALIDATE: flags any NaN or ±inf among the n rotated entries on the
// device, then waits for the stream and reads the flag (status word 1 of
// the workspace).
int check_finite(const float *x_rot, int64_t n, void *ws, hipStream_t s) {
  uint32_t *flag = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + 4);
  hipError_t e = launch_flag_nonfinite(x_rot, n, flag, s);
  uint32_t h = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&h, flag, sizeof(h), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return LAROSA_ERR_LAUNCH;
  return h ? LAROSA_ERR_NONFINITE : LAROSA_OK;
}

// Spin limit of the bounded device-side waits (larosa_set_spin_limit).
std::atomic<uint32_t> g_spin_limit{1u << 22};

}  // namespace

namespace {

// What the selection step keeps: each token's Top-k, or (thr) every
// channel whose magnitude is at least a threshold, with room for d_in per
// token and the number kept written to count_out when it is not NULL.
struct Sel {
  bool thr = false;
  int64_t k = 0;
  uint32_t thr_key = 0;
  int32_t *count_out = nullptr;
};

// The argument checks of a layer call, apart from the workspace. B == 0
// passes (the caller returns LAROSA_OK without work).
int layer_args(const void *x, int act_dtype, const void *Qt, int64_t q_block,
               const void *W_folded, int w_dtype, int64_t B, int64_t d_in, int64_t d_out,
               int64_t k, const void *y, const float *xrot_out, int mode) {
  if (!dtype_ok(act_dtype) || !dtype_ok(w_dtype)) return LAROSA_ERR_DTYPE;
  if (w_dtype == LAROSA_F32 && act_dtype == LAROSA_BF16) return LAROSA_ERR_DTYPE;
  if (int st = check_sizes(B, d_in, k)) return st;
  if (base_mode(mode) < 0) return LAROSA_ERR_INVALID_ARG;
  if (d_out < 1) return LAROSA_ERR_SHAPE;
  if (B == 0) return LAROSA_OK;
  // with LAROSA_PREROTATED x is fp32 x_rot and Qt is not read
  const bool pre = prerotated(mode);
  if (!x || (!Qt && !pre) || !W_folded || !y) return LAROSA_ERR_INVALID_ARG;
  if (pre && xrot_out) return LAROSA_ERR_INVALID_ARG;
  if (int st = check_rotation(d_in, q_block, w_dtype)) return st;
  if (d_in % vec_of(act_dtype) || d_out % vec_of(w_dtype)) return LAROSA_ERR_ALIGNMENT;
  if (!aligned16(x) || !aligned16(Qt) || !aligned16(W_folded) || !aligned16(y))
    return LAROSA_ERR_ALIGNMENT;
  if (xrot_out && !aligned16(xrot_out)) return LAROSA_ERR_ALIGNMENT;
  return LAROSA_OK;
}

int layer_entry(const void *x, int act_dtype, const void *Qt, int64_t q_block,
                const void *W_folded, int w_dtype, int64_t B, int64_t d_in, int64_t d_out,
                const Sel &sel, void *y, int32_t *idx_out, float *xrot_out, int mode, void *ws,
                size_t ws_bytes, larosa_stream_t stream, const RopeArgs *rope = nullptr,
                bool *rope_done = nullptr) {
  // rope: RoPE to fold into the one-token product's epilogue where that
  // product runs (bf16); *rope_done says whether it was.
  const int64_t k = sel.k;
  if (int st = layer_args(x, act_dtype, Qt, q_block, W_folded, w_dtype, B, d_in, d_out, k, y,
                          xrot_out, mode))
    return st;
  if (B == 0) return LAROSA_OK;
  if (!aligned16(ws)) return LAROSA_ERR_ALIGNMENT;
  const bool f64 = fp64_rotation(mode);
  const bool check = validating(mode);
  const bool pre = prerotated(mode);
  const bool fused = base_mode(mode) == LAROSA_FUSED && !f64 && !check && !sel.thr && !pre &&
                     fused_supported(B, d_in, act_dtype, w_dtype);
  const Layout L = fused ? layout_with_fused(B, d_in, d_out, k, w_dtype)
                         : layout_for(B, d_in, d_out, k, w_dtype);
  if (!ws || ws_bytes < L.total) return LAROSA_ERR_WORKSPACE;
  if (int st = device_status()) return st;

  hipStream_t s = stream_of(stream);
  char *base = static_cast<char *>(ws);
  if (fused) {
    FusedArgs f;
    f.x = x;
    f.qt = Qt;
    f.wf = W_folded;
    f.y = y;
    f.w_dt = w_dtype;
    f.d_in = static_cast<int>(d_in);
    f.q_block = static_cast<int>(q_block);
    f.k = static_cast<int>(k);
    f.d_out = d_out;
    f.idx_out = idx_out;
    f.xrot_out = xrot_out;
    f.ws = base + L.fused;
    f.status = reinterpret_cast<uint32_t *>(base + L.p.status);
    f.spin_limit = g_spin_limit.load();
    return launched(launch_fused_linear(f, s));
  }
  float *x_rot = pre        ? const_cast<float *>(static_cast<const float *>(x))
                 : xrot_out ? xrot_out
                            : reinterpret_cast<float *>(base + L.x_rot);
  int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(base + L.idx);
  float *val = reinterpret_cast<float *>(base + L.val);

  // Batches of 16 to 64 tokens in bf16 run the matrix-core forms of the
  // rotation and the product, which read Qt and the union rows once for the
  // whole batch.
  const bool mf = mfma_supported(B, act_dtype, w_dtype);
  // The matrix-core rotation may leave its k-range partial sums for the
  // Top-K selection to add (one launch fewer); x_rot is then written there.
  int n_parts = 1;
  const float *parts = reinterpret_cast<const float *>(base + L.p.mfma_parts);
  hipError_t e =
      pre   ? hipSuccess
      : f64 ? launch_rotate_f64(x, act_dtype, Qt, w_dtype, x_rot, static_cast<int>(B),
                                static_cast<int>(d_in), static_cast<int>(q_block), s)
      : mf && q_block % 32 == 0
          ? launch_rotate_mfma(x, Qt, x_rot, static_cast<int>(B), static_cast<int>(d_in),
                               static_cast<int>(q_block), base + L.p.mfma_parts, s,
                               B > 1 && !sel.thr && !check ? &n_parts : nullptr)
          : launch_rotate(x, act_dtype, Qt, w_dtype, x_rot, static_cast<int>(B),
                          static_cast<int>(d_in), static_cast<int>(q_block), s);
  if (e != hipSuccess) return LAROSA_ERR_LAUNCH;
  // (with the check the rotation sums its own k-range partials, so x_rot
  // is complete here)
  if (check)
    if (int st = check_finite(x_rot, B * d_in, base + L.p.status, s)) return st;

  GatherArgs a;
  a.coef_mode = kCoefPacked;
  a.w = W_folded;
  a.w_dt = w_dtype;
  a.d_in = d_in;
  a.d_out = d_out;
  a.y = y;
  a.y_dt = act_dtype;
  a.B = static_cast<int>(B);
  a.ws = base + L.p.gather;
  if (B == 1 && select_gather_supported(d_in)) {
    // One token: every workgroup of the product computes the exact Top-K rule
    // itself, so selection and product are one launch.
    SelectGatherArgs g;
    g.x_rot = x_rot;
    g.d_in = static_cast<int>(d_in);
    g.k = static_cast<int>(k);
    g.w = W_folded;
    g.w_dt = w_dtype;
    g.d_out = d_out;
    g.y = y;
    g.y_dt = act_dtype;
    g.idx_out = idx_out;
    g.ws = base + L.p.gather;
    g.by_threshold = sel.thr;
    g.thr_key = sel.thr_key;
    g.count_out = sel.count_out;
    const bool fold_rope = rope != nullptr && !sel.thr && act_dtype == LAROSA_BF16 &&
                           w_dtype == LAROSA_BF16;
    if (fold_rope) g.rope = *rope;
    const int st = launched(launch_select_gather(g, s));
    if (st == LAROSA_OK && fold_rope && rope_done) *rope_done = true;
    return st;
  }
  if (B == 1) {
    if (sel.thr) {
      int32_t *cnt = sel.count_out ? sel.count_out : reinterpret_cast<int32_t *>(base + L.u_cnt);
      e = launch_threshold_select(x_rot, 1, static_cast<int>(d_in), sel.thr_key, idx, cnt, val,
                                  nullptr, nullptr, s);
      a.n_rows = cnt;
    } else {
      e = launch_select(x_rot, 1, static_cast<int>(d_in), static_cast<int>(k), idx, val,
                        nullptr, nullptr, s);
      a.n_rows = nullptr;
    }
    if (e != hipSuccess) return LAROSA_ERR_LAUNCH;
    a.rows = idx;
    a.max_rows = k;
    a.coef = val;
  } else {
    float *xs = reinterpret_cast<float *>(base + L.xs);
    uint32_t *mask = reinterpret_cast<uint32_t *>(base + L.p.mask);
    int32_t *u_idx = reinterpret_cast<int32_t *>(base + L.u_idx);
    int32_t *u_cnt = reinterpret_cast<int32_t *>(base + L.u_cnt);
    float *u_coef = reinterpret_cast<float *>(base + L.u_coef);
    if (sel.thr) {
      e = launch_threshold_select(x_rot, static_cast<int>(B), static_cast<int>(d_in),
                                  sel.thr_key, idx, sel.count_out, val, xs, mask, s);
      if (e == hipSuccess && !mf)
        e = launch_union(mask, xs, static_cast<int>(B), static_cast<int>(d_in), u_idx, u_cnt,
                         u_coef, s);
    } else {
      // the union and the product read xs and the masks only: the index
      // list is written when asked for, the values not at all. For the
      // vector product the union list is taken by the selection launch
      // itself; the matrix-core product's coefficient launch takes it from
      // the masks.
      e = launch_select(x_rot, static_cast<int>(B), static_cast<int>(d_in), static_cast<int>(k),
                        idx_out, nullptr, xs, mask, s, parts, n_parts,
                        mf ? UnionTail{} : union_tail(base + L.p.status, u_idx, u_cnt));
      if (e == hipSuccess && !mf)
        e = launch_union_coef(u_idx, u_cnt, xs, static_cast<int>(B), static_cast<int>(d_in),
                              u_coef, s);
    }
    if (e != hipSuccess) return LAROSA_ERR_LAUNCH;
    const int64_t bk = B * k;  // the threshold form's k is d_in
    const int64_t max_rows = bk < d_in ? bk : d_in;
    if (mf) {
      const int64_t ldc = mfma_coef_ld(max_rows);
      void *coefT = base + L.p.mfma_coef;
      e = launch_union_coef_mask(mask, xs, static_cast<int>(B), static_cast<int>(d_in), ldc, coefT,
                                 u_idx, u_cnt, s);
      if (e == hipSuccess)
        e = launch_gather_mfma(u_idx, u_cnt, max_rows, d_in, coefT, ldc, W_folded, y,
                               static_cast<int>(B), d_out, base + L.p.mfma_parts, s);
      return launched(e);
    }
    a.rows = u_idx;
    a.n_rows = u_cnt;
    a.max_rows = max_rows;
    a.coef = u_coef;
  }
  return launched(launch_gather(a, s));
}

int swiglu_entry(const void *x, int act_dtype, const void *Qt, int64_t q_block,
                 const void *W_il, int w_dtype, int64_t B, int64_t d_in, int64_t f,
                 const Sel &sel, void *h, int32_t *idx_out, float *xrot_out, int mode, void *ws,
                 size_t ws_bytes, larosa_stream_t stream) {
  const int64_t k = sel.k;
  if (!dtype_ok(act_dtype) || !dtype_ok(w_dtype)) return LAROSA_ERR_DTYPE;
  if (f < 1 || f % interleave_block(w_dtype)) return LAROSA_ERR_SHAPE;
  if (base_mode(mode) < 0) return LAROSA_ERR_INVALID_ARG;
  const size_t need = larosa_swiglu_workspace_bytes(B, d_in, f, k, mode);
  if (need == 0 && B != 0) {  // invalid sizes: let the layer call name the error
    return layer_entry(x, act_dtype, Qt, q_block, W_il, w_dtype, B, d_in, 2 * f, sel, h, idx_out,
                       xrot_out, mode, ws, ws_bytes, stream);
  }
  if (B == 0) return LAROSA_OK;
  if (!h) return LAROSA_ERR_INVALID_ARG;
  if (!aligned16(h)) return LAROSA_ERR_ALIGNMENT;
  if (!ws || ws_bytes < need) return LAROSA_ERR_WORKSPACE;
  const size_t layer_bytes = larosa_workspace_bytes(B, d_in, 2 * f, k, mode);
  const bool one_launch = (base_mode(mode) == LAROSA_UNFUSED || fp64_rotation(mode) ||
                           validating(mode) || prerotated(mode)) && B == 1 &&
                          select_gather_supported(d_in) &&
                          !(w_dtype == LAROSA_F32 && act_dtype == LAROSA_BF16);
  if (one_launch) {
    // rotation, then the selection, product and SiLU(gate)·up in one launch
    const bool pre = prerotated(mode);
    if (int st = check_sizes(B, d_in, k)) return st;
    if (!x || (!Qt && !pre) || !W_il) return LAROSA_ERR_INVALID_ARG;
    if (pre && xrot_out) return LAROSA_ERR_INVALID_ARG;
    if (int st = check_rotation(d_in, q_block, w_dtype)) return st;
    if (d_in % vec_of(act_dtype)) return LAROSA_ERR_ALIGNMENT;
    if (!aligned16(x) || !aligned16(Qt) || !aligned16(W_il) || !aligned16(ws))
      return LAROSA_ERR_ALIGNMENT;
    if (xrot_out && !aligned16(xrot_out)) return LAROSA_ERR_ALIGNMENT;
    if (int st = device_status()) return st;
    const Layout L = layout_for(B, d_in, 2 * f, k, w_dtype);
    char *base = static_cast<char *>(ws);
    float *x_rot = pre        ? const_cast<float *>(static_cast<const float *>(x))
                   : xrot_out ? xrot_out
                              : reinterpret_cast<float *>(base + L.x_rot);
    hipStream_t s = stream_of(stream);
    const hipError_t er =
        pre ? hipSuccess
        : fp64_rotation(mode)
            ? launch_rotate_f64(x, act_dtype, Qt, w_dtype, x_rot, 1, static_cast<int>(d_in),
                                static_cast<int>(q_block), s)
            : launch_rotate(x, act_dtype, Qt, w_dtype, x_rot, 1, static_cast<int>(d_in),
                            static_cast<int>(q_block), s);
    if (er != hipSuccess) return LAROSA_ERR_LAUNCH;
    if (validating(mode))
      if (int st = check_finite(x_rot, d_in, base + L.p.status, s)) return st;
    SelectGatherArgs g;
    g.x_rot = x_rot;
    g.d_in = static_cast<int>(d_in);
    g.k = static_cast<int>(k);
    g.w = W_il;
    g.w_dt = w_dtype;
    g.d_out = 2 * f;
    g.y = h;
    g.y_dt = act_dtype;
    g.idx_out = idx_out;
    g.ws = base + L.p.gather;
    g.swiglu = true;
    g.by_threshold = sel.thr;
    g.thr_key = sel.thr_key;
    g.count_out = sel.count_out;
    return launched(launch_select_gather(g, s));
  }
  // otherwise the gate|up rows into the workspace, then SiLU(gate)·up
  void *gu = static_cast<char *>(ws) + layer_bytes;
  const int st = layer_entry(x, act_dtype, Qt, q_block, W_il, w_dtype, B, d_in, 2 * f, sel, gu,
                             idx_out, xrot_out, mode, ws, layer_bytes, stream);
  if (st != LAROSA_OK) return st;
  return launched(launch_swiglu_il(gu, h, B, f, interleave_block(w_dtype), act_dtype,
                                   stream_of(stream)));
}

// The MLP workspace: the gate|up call's (SwiGLU) workspace, then the down
// call's.
struct MlpLayout {
  size_t up = 0, down = 0, total = 0;
  size_t up_bytes = 0, down_bytes = 0;
};

MlpLayout mlp_layout(int64_t B, int64_t d, int64_t f, int64_t k1, int64_t k2, int mode) {
  MlpLayout M;
  if (mode & LAROSA_PREROTATED) return M;  // not a flag of the MLP call
  mode &= ~LAROSA_CHAIN;  // the chained form uses the unfused layout
  M.up_bytes = larosa_swiglu_workspace_bytes(B, d, f, k1, mode);
  M.down_bytes = larosa_workspace_bytes(B, f, d, k2, mode);
  if (M.up_bytes == 0 || M.down_bytes == 0) return M;
  // The down region starts at the same offset in every mode (after the
  // larger, one-launch form of the up region), so calls in different modes
  // can share one workspace: each region's areas keep their places.
  const size_t up_fused = larosa_swiglu_workspace_bytes(B, d, f, k1, mode | LAROSA_FUSED);
  if (up_fused > M.up_bytes) M.up_bytes = up_fused;
  M.up = 0;
  M.down = align256(M.up_bytes);
  M.total = M.down + align256(M.down_bytes);
  return M;
}

}  // namespace

extern "C" {

int larosa_abi_version(void) LAROSA_NOEXCEPT { return LAROSA_ABI_VERSION; }

const char *larosa_status_string(int status) LAROSA_NOEXCEPT {
  switch (status) {
    case LAROSA_OK: return "ok";
    case LAROSA_ERR_INVALID_ARG: return "invalid argument";
    case LAROSA_ERR_SHAPE: return "unsupported shape";
    case LAROSA_ERR_ALIGNMENT: return "misaligned pointer or row length";
    case LAROSA_ERR_DTYPE: return "unsupported element type";
    case LAROSA_ERR_WORKSPACE: return "workspace missing or too small";
    case LAROSA_ERR_NO_DEVICE: return "no HIP device";
    case LAROSA_ERR_LAUNCH: return "kernel launch failed";
    case LAROSA_ERR_NONFINITE: return "non-finite rotated input";
    case LAROSA_ERR_TIMEOUT: return "a bounded device-side wait gave up";
    case LAROSA_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

size_t larosa_workspace_bytes(int64_t B, int64_t d_in, int64_t d_out, int64_t k, int mode) LAROSA_NOEXCEPT {
  return guard_size([&]() -> size_t {
  if (check_sizes(B < 1 ? 1 : B, d_in, k) != LAROSA_OK || d_out < 1) return 0;
  if (base_mode(mode) < 0) return 0;
  mode = base_mode(mode);
  // Sized for bf16 weights; fp32 weights have twice the column tiles but the
  // same number of splits at most, and fit in the same bytes or fewer.
  const int64_t b1 = B < 1 ? 1 : B;
  const Layout a = mode == LAROSA_FUSED ? layout_with_fused(b1, d_in, d_out, k, LAROSA_BF16)
                                        : layout_for(b1, d_in, d_out, k, LAROSA_BF16);
  const Layout b = mode == LAROSA_FUSED ? layout_with_fused(b1, d_in, d_out, k, LAROSA_F32)
                                        : layout_for(b1, d_in, d_out, k, LAROSA_F32);
  return a.total > b.total ? a.total : b.total;
  });
}

int larosa_workspace_init(void *ws, size_t bytes, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!ws && bytes) return LAROSA_ERR_INVALID_ARG;
  if (bytes == 0) return LAROSA_OK;
  if (!aligned16(ws)) return LAROSA_ERR_ALIGNMENT;
  if (int st = device_status()) return st;
  return launched(launch_fill_zero(ws, bytes, stream_of(stream)));
  });
}

int larosa_workspace_status(void *ws, int32_t *status_out, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!ws || !status_out) return LAROSA_ERR_INVALID_ARG;
  if (!aligned16(ws) || (reinterpret_cast<uintptr_t>(status_out) & 3u)) return LAROSA_ERR_ALIGNMENT;
  if (int st = device_status()) return st;
  return launched(launch_take_status(static_cast<uint32_t *>(ws), status_out, stream_of(stream)));
  });
}

uint32_t larosa_set_spin_limit(uint32_t limit) LAROSA_NOEXCEPT { return g_spin_limit.exchange(limit); }

int larosa_prepare_rotation(const void *Q, void *Qt, int64_t d, int64_t q_block, int dtype,
                            larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!Q || !Qt) return LAROSA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return LAROSA_ERR_DTYPE;
  if (d < 1) return LAROSA_ERR_SHAPE;
  if (int st = check_rotation(d, q_block, dtype)) return st;
  if (!aligned16(Q) || !aligned16(Qt)) return LAROSA_ERR_ALIGNMENT;
  const size_t bytes = static_cast<size_t>(d) * q_block * dt_size(dtype);
  const char *a = static_cast<const char *>(Q);
  const char *b = static_cast<const char *>(Qt);
  if (a < b + bytes && b < a + bytes) return LAROSA_ERR_INVALID_ARG;
  if (int st = device_status()) return st;
  return launched(launch_transpose_blocks(Q, Qt, d, q_block, dtype, stream_of(stream)));
  });
}

int larosa_fold_weights(const void *Qt, int64_t q_block, const void *W, void *W_folded,
                        int64_t d_in, int64_t d_out, int w_dtype, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!Qt || !W || !W_folded) return LAROSA_ERR_INVALID_ARG;
  if (!dtype_ok(w_dtype)) return LAROSA_ERR_DTYPE;
  if (d_in < 1 || d_out < 1) return LAROSA_ERR_SHAPE;
  if (int st = check_rotation(d_in, q_block, w_dtype)) return st;
  if (d_out % vec_of(w_dtype)) return LAROSA_ERR_ALIGNMENT;
  if (!aligned16(Qt) || !aligned16(W) || !aligned16(W_folded)) return LAROSA_ERR_ALIGNMENT;
  const size_t wb = static_cast<size_t>(d_in) * d_out * dt_size(w_dtype);
  const size_t qbts = static_cast<size_t>(d_in) * q_block * dt_size(w_dtype);
  const char *f = static_cast<const char *>(W_folded);
  const char *w = static_cast<const char *>(W);
  const char *q = static_cast<const char *>(Qt);
  if ((f < w + wb && w < f + wb) || (f < q + qbts && q < f + wb)) return LAROSA_ERR_INVALID_ARG;
  if (int st = device_status()) return st;
  return launched(launch_fold(Qt, q_block, W, W_folded, d_in, d_out, w_dtype, stream_of(stream)));
  });
}

int larosa_rotate(const void *x, int x_dtype, const void *Qt, int64_t q_block, int q_dtype,
                  float *x_rot, int64_t B, int64_t d, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(x_dtype) || !dtype_ok(q_dtype)) return LAROSA_ERR_DTYPE;
  if (int st = check_sizes(B, d, 1)) return st;
  if (B == 0) return LAROSA_OK;
  if (!x || !Qt || !x_rot) return LAROSA_ERR_INVALID_ARG;
  if (int st = check_rotation(d, q_block, q_dtype)) return st;
  if (d % 8 && x_dtype == LAROSA_BF16) return LAROSA_ERR_ALIGNMENT;
  if (!aligned16(x) || !aligned16(Qt) || !aligned16(x_rot)) return LAROSA_ERR_ALIGNMENT;
  if (int st = device_status()) return st;
  // Without a workspace the matrix-core form runs unsplit over each block;
  // up to 4 tokens over blocks of 4096 or more, and up to 8 over blocks of
  // 4096 (which the few-token kernel takes in one pass), the vector forms are
  // faster (d = 4096: 11.0 / 14.4 / 23.7 µs at 2 / 4 / 8 tokens against
  // 26.6 µs).
  const bool vec = (B <= 4 && q_block >= 4096) || (B <= 8 && q_block == 4096);
  if (!vec && mfma_supported(B, x_dtype, q_dtype) && q_block % 32 == 0)
    return launched(launch_rotate_mfma(x, Qt, x_rot, static_cast<int>(B), static_cast<int>(d),
                                       static_cast<int>(q_block), nullptr, stream_of(stream)));
  return launched(launch_rotate(x, x_dtype, Qt, q_dtype, x_rot, static_cast<int>(B),
                                static_cast<int>(d), static_cast<int>(q_block),
                                stream_of(stream)));
  });
}

int larosa_rotate_fp64(const void *x, int x_dtype, const void *Qt, int64_t q_block,
                       int q_dtype, float *x_rot, int64_t B, int64_t d, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(x_dtype) || !dtype_ok(q_dtype)) return LAROSA_ERR_DTYPE;
  if (int st = check_sizes(B, d, 1)) return st;
  if (B == 0) return LAROSA_OK;
  if (!x || !Qt || !x_rot) return LAROSA_ERR_INVALID_ARG;
  if (int st = check_rotation(d, q_block, q_dtype)) return st;
  if (d % 8 && x_dtype == LAROSA_BF16) return LAROSA_ERR_ALIGNMENT;
  if (!aligned16(x) || !aligned16(Qt) || !aligned16(x_rot)) return LAROSA_ERR_ALIGNMENT;
  if (int st = device_status()) return st;
  return launched(launch_rotate_f64(x, x_dtype, Qt, q_dtype, x_rot, static_cast<int>(B),
                                    static_cast<int>(d), static_cast<int>(q_block),
                                    stream_of(stream)));
  });
}

int larosa_topk_select(const float *x_rot, int64_t B, int64_t d, int64_t k, int32_t *idx,
                       float *val, float *xs, int32_t *union_idx, int32_t *union_count,
                       float *union_coef, void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (int st = check_sizes(B, d, k)) return st;
  if (B == 0) return LAROSA_OK;
  if (!x_rot || !idx || !val) return LAROSA_ERR_INVALID_ARG;
  const bool want_union = union_idx != nullptr;
  if (want_union && (!union_count || !union_coef || !xs)) return LAROSA_ERR_INVALID_ARG;
  if (!aligned16(x_rot)) return LAROSA_ERR_ALIGNMENT;
  uint32_t *mask = nullptr;
  if (want_union) {
    const size_t need = kStatusBytes + static_cast<size_t>(B) * mask_words(static_cast<int>(d)) * 4;
    if (!ws || ws_bytes < need) return LAROSA_ERR_WORKSPACE;
    if (!aligned16(ws)) return LAROSA_ERR_ALIGNMENT;
    mask = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + kStatusBytes);
  }
  if (int st = device_status()) return st;
  hipStream_t s = stream_of(stream);
  // x_rot is only read (no partial sums are passed)
  const bool tail = want_union && B > 1;  // the union list taken by the selection launch
  hipError_t e = launch_select(const_cast<float *>(x_rot), static_cast<int>(B),
                               static_cast<int>(d), static_cast<int>(k), idx, val, xs, mask, s,
                               nullptr, 1,
                               tail ? union_tail(static_cast<char *>(ws), union_idx, union_count)
                                    : UnionTail{});
  if (e == hipSuccess && want_union)
    e = tail ? launch_union_coef(union_idx, union_count, xs, static_cast<int>(B),
                                 static_cast<int>(d), union_coef, s)
             : launch_union(mask, xs, static_cast<int>(B), static_cast<int>(d), union_idx,
                            union_count, union_coef, s);
  return launched(e);
  });
}

int larosa_threshold_select(const float *x_rot, int64_t B, int64_t d, float t, int32_t *idx,
                            int32_t *count, float *val, float *xs, int32_t *union_idx,
                            int32_t *union_count, float *union_coef, void *ws, size_t ws_bytes,
                            larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (int st = check_sizes(B, d, 1)) return st;
  if (!(t >= 0.f)) return LAROSA_ERR_INVALID_ARG;  // negative or NaN
  if (B == 0) return LAROSA_OK;
  if (!x_rot || !idx || !count) return LAROSA_ERR_INVALID_ARG;
  const bool want_union = union_idx != nullptr;
  if (want_union && (!union_count || !union_coef || !xs)) return LAROSA_ERR_INVALID_ARG;
  if (!aligned16(x_rot)) return LAROSA_ERR_ALIGNMENT;
  uint32_t *mask = nullptr;
  if (want_union) {
    const size_t need = kStatusBytes + static_cast<size_t>(B) * mask_words(static_cast<int>(d)) * 4;
    if (!ws || ws_bytes < need) return LAROSA_ERR_WORKSPACE;
    if (!aligned16(ws)) return LAROSA_ERR_ALIGNMENT;
    mask = reinterpret_cast<uint32_t *>(static_cast<char *>(ws) + kStatusBytes);
  }
  if (int st = device_status()) return st;
  hipStream_t s = stream_of(stream);
  hipError_t e = launch_threshold_select(x_rot, static_cast<int>(B), static_cast<int>(d),
                                         threshold_key_of(t), idx, count, val, xs, mask, s);
  if (e == hipSuccess && want_union)
    e = launch_union(mask, xs, static_cast<int>(B), static_cast<int>(d), union_idx,
                     union_count, union_coef, s);
  return launched(e);
  });
}

size_t larosa_calibrate_workspace_bytes(void) LAROSA_NOEXCEPT { return calibrate_ws_bytes(); }

int larosa_calibrate_threshold(const float *x_rot, int64_t n, int64_t keep, float *t_out,
                               void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard_size([&]() -> size_t {
  if (n < 1 || n > INT32_MAX) return LAROSA_ERR_SHAPE;
  if (keep < 1 || keep > n) return LAROSA_ERR_INVALID_ARG;
  if (!x_rot || !t_out) return LAROSA_ERR_INVALID_ARG;
  if (!ws || ws_bytes < calibrate_ws_bytes()) return LAROSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LAROSA_ERR_ALIGNMENT;
  if (int st = device_status()) return st;
  return launched(launch_calibrate(x_rot, n, static_cast<uint32_t>(keep), t_out, ws,
                                   stream_of(stream)));
  });
}

size_t larosa_lowrank_workspace_bytes(int64_t B, int64_t d_in, int64_t d_out, int64_t k,
                                      int64_t r) LAROSA_NOEXCEPT {
  return guard_size([&]() -> size_t {
  const int64_t b1 = B < 1 ? 1 : B;
  if (check_sizes(b1, d_in, k) != LAROSA_OK || d_out < 1) return 0;
  if (r < 1 || r > kMaxRank || r > d_in || r > d_out) return 0;
  const size_t a = lowrank_layout(b1, d_in, d_out, k, r, LAROSA_BF16).total;
  const size_t b = lowrank_layout(b1, d_in, d_out, k, r, LAROSA_F32).total;
  return a > b ? a : b;
  });
}

int larosa_lowrank_layer_forward(const void *x, int act_dtype, const void *Qt, int64_t q_block,
                                 const void *W_ext, const void *A_r, int64_t r, int w_dtype,
                                 int64_t B, int64_t d_in, int64_t d_out, int64_t k, void *y,
                                 int32_t *idx_out, float *xrot_out, int mode, void *ws,
                                 size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(act_dtype) || !dtype_ok(w_dtype)) return LAROSA_ERR_DTYPE;
  if (w_dtype == LAROSA_F32 && act_dtype == LAROSA_BF16) return LAROSA_ERR_DTYPE;
  if (int st = check_sizes(B, d_in, k)) return st;
  if (base_mode(mode) < 0 || prerotated(mode)) return LAROSA_ERR_INVALID_ARG;
  if (d_out < 1) return LAROSA_ERR_SHAPE;
  if (r < 1 || r > kMaxRank || r > d_in || r > d_out) return LAROSA_ERR_INVALID_ARG;
  if (B == 0) return LAROSA_OK;
  if (!x || !Qt || !W_ext || !A_r || !y) return LAROSA_ERR_INVALID_ARG;
  if (int st = check_rotation(d_in, q_block, w_dtype)) return st;
  if (d_in % vec_of(act_dtype) || d_out % vec_of(w_dtype)) return LAROSA_ERR_ALIGNMENT;
  if (!aligned16(x) || !aligned16(Qt) || !aligned16(W_ext) || !aligned16(y) || !aligned16(ws))
    return LAROSA_ERR_ALIGNMENT;
  if (xrot_out && !aligned16(xrot_out)) return LAROSA_ERR_ALIGNMENT;
  const LrLayout L = lowrank_layout(B, d_in, d_out, k, r, w_dtype);
  if (!ws || ws_bytes < L.total) return LAROSA_ERR_WORKSPACE;
  if (int st = device_status()) return st;

  hipStream_t s = stream_of(stream);
  char *base = static_cast<char *>(ws);
  float *x_rot = xrot_out ? xrot_out : reinterpret_cast<float *>(base + L.l.x_rot);
  int32_t *idx = idx_out ? idx_out : reinterpret_cast<int32_t *>(base + L.l.idx);
  float *xs = reinterpret_cast<float *>(base + L.l.xs);
  const int Bi = static_cast<int>(B), di = static_cast<int>(d_in), ri = static_cast<int>(r);
  const bool mf = mfma_supported(B, act_dtype, w_dtype);
  int n_parts = 1;  // k-range partial sums left for the selection to add
  const float *parts = reinterpret_cast<const float *>(base + L.l.p.mfma_parts);
  hipError_t e =
      fp64_rotation(mode)
          ? launch_rotate_f64(x, act_dtype, Qt, w_dtype, x_rot, Bi, di, static_cast<int>(q_block), s)
      : mf && q_block % 32 == 0
          ? launch_rotate_mfma(x, Qt, x_rot, Bi, di, static_cast<int>(q_block),
                               base + L.l.p.mfma_parts, s,
                               validating(mode) ? nullptr : &n_parts)
          : launch_rotate(x, act_dtype, Qt, w_dtype, x_rot, Bi, di, static_cast<int>(q_block), s);
  if (e == hipSuccess && validating(mode))
    if (int st = check_finite(x_rot, B * d_in, base + L.l.p.status, s)) return st;
  uint32_t *mask = B > 1 ? reinterpret_cast<uint32_t *>(base + L.l.p.mask) : nullptr;
  if (e == hipSuccess)
    // one token: the kept rows are the product's base list; more: the union is,
    // and the index list is written only when asked for. Coefficients come
    // from xs, so the values are not written.
    e = launch_select(x_rot, Bi, di, static_cast<int>(k), B == 1 ? idx : idx_out, nullptr, xs,
                      mask, s, parts, n_parts,
                      B > 1 ? union_tail(base + L.l.p.status,
                                         reinterpret_cast<int32_t *>(base + L.l.u_idx),
                                         reinterpret_cast<int32_t *>(base + L.l.u_cnt))
                            : UnionTail{});
  // the base row list: the token's kept rows, or the batch's union (taken by
  // the selection launch)
  const int32_t *list = idx;
  const int32_t *n_dev = nullptr;
  int64_t max_rows = k;
  if (e == hipSuccess && B > 1) {
    int32_t *u_idx = reinterpret_cast<int32_t *>(base + L.l.u_idx);
    int32_t *u_cnt = reinterpret_cast<int32_t *>(base + L.l.u_cnt);
    list = u_idx;
    n_dev = u_cnt;
    max_rows = B * k < d_in ? B * k : d_in;
  }
  float *part = reinterpret_cast<float *>(base + L.part);
  if (e == hipSuccess) e = launch_lowrank_proj(x_rot, xs, A_r, w_dtype, Bi, di, ri, part, s);
  if (e != hipSuccess) return LAROSA_ERR_LAUNCH;
  int32_t *rows_ext = reinterpret_cast<int32_t *>(base + L.rows_ext);
  int32_t *n_ext = reinterpret_cast<int32_t *>(base + L.n_ext);
  const int64_t max_ext = max_rows + r;
  if (mf) {
    const int64_t ldc = mfma_coef_ld(max_ext);
    void *coefT = base + L.l.p.mfma_coef;
    e = launch_lowrank_list(list, n_dev, static_cast<int>(k), di, ri, xs, part, Bi, ldc,
                            rows_ext, n_ext, nullptr, coefT, s);
    if (e == hipSuccess)
      e = launch_gather_mfma(rows_ext, n_ext, max_ext, d_in + r, coefT, ldc, W_ext, y, Bi, d_out,
                             base + L.l.p.mfma_parts, s);
    return launched(e);
  }
  float *coef = reinterpret_cast<float *>(base + L.l.u_coef);
  e = launch_lowrank_list(list, n_dev, static_cast<int>(k), di, ri, xs, part, Bi, max_ext,
                          rows_ext, n_ext, coef, nullptr, s);
  if (e != hipSuccess) return LAROSA_ERR_LAUNCH;
  GatherArgs a;
  a.rows = rows_ext;
  a.n_rows = n_ext;
  a.max_rows = max_ext;
  a.coef = coef;
  a.coef_mode = kCoefPacked;
  a.w = W_ext;
  a.w_dt = w_dtype;
  a.d_in = d_in + r;
  a.d_out = d_out;
  a.y = y;
  a.y_dt = act_dtype;
  a.B = Bi;
  a.ws = base + L.l.p.gather;
  return launched(launch_gather(a, s));
  });
}

int larosa_sparse_gemv(const int32_t *rows, const int32_t *n_rows, int64_t max_rows,
                       const float *coef, const void *W_folded, int w_dtype, void *y,
                       int y_dtype, int64_t B, int64_t d_in, int64_t d_out, void *ws,
                       size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(w_dtype) || !dtype_ok(y_dtype)) return LAROSA_ERR_DTYPE;
  if (w_dtype == LAROSA_F32 && y_dtype == LAROSA_BF16) return LAROSA_ERR_DTYPE;
  if (B < 0 || B > kMaxB) return LAROSA_ERR_INVALID_ARG;
  if (d_in < 1 || d_in > kMaxD || d_out < 1) return LAROSA_ERR_SHAPE;
  if (max_rows < 0 || max_rows > INT32_MAX / 2) return LAROSA_ERR_INVALID_ARG;
  if (B == 0) return LAROSA_OK;
  if (!rows || !coef || !W_folded || !y) return LAROSA_ERR_INVALID_ARG;
  if (d_out % vec_of(w_dtype)) return LAROSA_ERR_ALIGNMENT;
  if (!aligned16(W_folded) || !aligned16(y)) return LAROSA_ERR_ALIGNMENT;
  const int64_t mr = max_rows < 1 ? 1 : max_rows;
  const Prefix P = prefix_for(B, d_in, d_out, mr > d_in ? mr : d_in, w_dtype);
  const bool mf = mfma_supported(B, y_dtype, w_dtype);
  if (!ws || ws_bytes < P.end) return LAROSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LAROSA_ERR_ALIGNMENT;
  if (int st = device_status()) return st;
  hipStream_t s = stream_of(stream);
  char *base = static_cast<char *>(ws);
  if (mf) {
    // max_rows == 0 still runs, so y is written (as zeros).
    const int64_t ldc = mfma_coef_ld(mr);
    void *coefT = base + P.mfma_coef;
    hipError_t e = launch_coef_transpose(coef, static_cast<int>(B), max_rows, ldc, coefT, s);
    if (e == hipSuccess)
      e = launch_gather_mfma(rows, n_rows, max_rows, d_in, coefT, ldc, W_folded, y,
                             static_cast<int>(B), d_out, base + P.mfma_parts, s);
    return launched(e);
  }
  GatherArgs a;
  a.rows = rows;
  a.n_rows = n_rows;
  a.max_rows = max_rows;
  a.coef = coef;
  a.coef_mode = kCoefPacked;
  a.w = W_folded;
  a.w_dt = w_dtype;
  a.d_in = d_in;
  a.d_out = d_out;
  a.y = y;
  a.y_dt = y_dtype;
  a.B = static_cast<int>(B);
  a.ws = base + P.gather;
  // max_rows == 0 still runs, so y is written (as zeros).
  return launched(launch_gather(a, s));
  });
}

int larosa_topk_gemv(const float *x_rot, int64_t d_in, int64_t k, const void *W_folded,
                     int w_dtype, void *y, int y_dtype, int64_t d_out, int32_t *idx_out,
                     void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(w_dtype) || !dtype_ok(y_dtype)) return LAROSA_ERR_DTYPE;
  if (w_dtype == LAROSA_F32 && y_dtype == LAROSA_BF16) return LAROSA_ERR_DTYPE;
  if (int st = check_sizes(1, d_in, k)) return st;
  if (!select_gather_supported(d_in)) return LAROSA_ERR_SHAPE;
  if (d_out < 1) return LAROSA_ERR_SHAPE;
  if (!x_rot || !W_folded || !y) return LAROSA_ERR_INVALID_ARG;
  if (d_out % vec_of(w_dtype)) return LAROSA_ERR_ALIGNMENT;
  if (!aligned16(x_rot) || !aligned16(W_folded) || !aligned16(y)) return LAROSA_ERR_ALIGNMENT;
  const Prefix P = prefix_for(1, d_in, d_out, d_in, w_dtype);
  if (!ws || ws_bytes < P.end) return LAROSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LAROSA_ERR_ALIGNMENT;
  if (int st = device_status()) return st;
  SelectGatherArgs g;
  g.x_rot = x_rot;
  g.d_in = static_cast<int>(d_in);
  g.k = static_cast<int>(k);
  g.w = W_folded;
  g.w_dt = w_dtype;
  g.d_out = d_out;
  g.y = y;
  g.y_dt = y_dtype;
  g.idx_out = idx_out;
  g.ws = static_cast<char *>(ws) + P.gather;
  return launched(launch_select_gather(g, stream_of(stream)));
  });
}

int larosa_dense_gemv(const void *x, int act_dtype, const void *W, int w_dtype, void *y,
                      int64_t B, int64_t d_in, int64_t d_out, void *ws, size_t ws_bytes,
                      larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(act_dtype) || !dtype_ok(w_dtype)) return LAROSA_ERR_DTYPE;
  if (act_dtype != w_dtype) return LAROSA_ERR_DTYPE;
  if (B < 0 || B > kMaxB) return LAROSA_ERR_INVALID_ARG;
  if (d_in < 1 || d_in > kMaxD || d_out < 1) return LAROSA_ERR_SHAPE;
  if (B == 0) return LAROSA_OK;
  if (!x || !W || !y) return LAROSA_ERR_INVALID_ARG;
  if (d_out % vec_of(w_dtype)) return LAROSA_ERR_ALIGNMENT;
  if (!aligned16(x) || !aligned16(W) || !aligned16(y)) return LAROSA_ERR_ALIGNMENT;
  const Prefix P = prefix_for(B, d_in, d_out, d_in, w_dtype);
  if (!ws || ws_bytes < P.end) return LAROSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LAROSA_ERR_ALIGNMENT;
  if (int st = device_status()) return st;
  hipStream_t s = stream_of(stream);
  char *base = static_cast<char *>(ws);
  if (mfma_supported(B, act_dtype, w_dtype)) {
    const int64_t ldc = mfma_coef_ld(d_in);
    void *coefT = base + P.mfma_coef;
    hipError_t e = launch_act_to_coef_t(x, static_cast<int>(B), d_in, ldc, coefT, s);
    if (e == hipSuccess)
      e = launch_gather_mfma(nullptr, nullptr, d_in, d_in, coefT, ldc, W, y,
                             static_cast<int>(B), d_out, base + P.mfma_parts, s);
    return launched(e);
  }
  GatherArgs a;
  a.rows = nullptr;
  a.n_rows = nullptr;
  a.max_rows = d_in;
  a.coef = x;
  a.coef_mode = act_dtype == LAROSA_F32 ? kCoefActF32 : kCoefActBF16;
  a.w = W;
  a.w_dt = w_dtype;
  a.d_in = d_in;
  a.d_out = d_out;
  a.y = y;
  a.y_dt = act_dtype;
  a.B = static_cast<int>(B);
  a.ws = base + P.gather;
  return launched(launch_gather(a, s));
  });
}

int larosa_layer_forward(const void *x, int act_dtype, const void *Qt, int64_t q_block,
                         const void *W_folded, int w_dtype, int64_t B, int64_t d_in,
                         int64_t d_out, int64_t k, void *y, int32_t *idx_out, float *xrot_out,
                         int mode, void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  Sel sel;
  sel.k = k;
  return layer_entry(x, act_dtype, Qt, q_block, W_folded, w_dtype, B, d_in, d_out, sel, y,
                     idx_out, xrot_out, mode, ws, ws_bytes, stream);
  });
}

int larosa_layer_forward_noalloc(const void *x, int act_dtype, const void *Qt, int64_t q_block,
                                 const void *W_folded, int w_dtype, int64_t B, int64_t d_in,
                                 int64_t d_out, int64_t k, void *y, int32_t *idx_out,
                                 float *xrot_out, int mode, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  // The one-launch form reports its bounded waits through the workspace,
  // which this caller cannot read: only the unfused steps run here, on x
  // itself (the modes the declaration lists).
  if (base_mode(mode) != LAROSA_UNFUSED || prerotated(mode)) return LAROSA_ERR_INVALID_ARG;
  Sel sel;
  sel.k = k;
  const size_t need = larosa_workspace_bytes(B, d_in, d_out, k, mode);
  if (need == 0 || B == 0)  // invalid sizes or an empty batch: the checks name it
    return layer_entry(x, act_dtype, Qt, q_block, W_folded, w_dtype, B, d_in, d_out, sel, y,
                       idx_out, xrot_out, mode, nullptr, 0, stream);
  // every argument check of the layer call before the scratch is touched
  if (int st = layer_args(x, act_dtype, Qt, q_block, W_folded, w_dtype, B, d_in, d_out, k, y,
                          xrot_out, mode))
    return st;
  if (need > scratch_capacity()) return LAROSA_ERR_WORKSPACE;
  if (int st = device_status()) return st;
  ScratchShape shape{B, d_in, d_out, k, mode, act_dtype, w_dtype};
  void *ws = nullptr;
  if (scratch_acquire(shape, need, stream_of(stream), &ws) != hipSuccess) return LAROSA_ERR_LAUNCH;
  return layer_entry(x, act_dtype, Qt, q_block, W_folded, w_dtype, B, d_in, d_out, sel, y,
                     idx_out, xrot_out, mode, ws, need, stream);
  });
}

int larosa_threshold_layer_forward(const void *x, int act_dtype, const void *Qt,
                                   int64_t q_block, const void *W_folded, int w_dtype, int64_t B,
                                   int64_t d_in, int64_t d_out, float t, void *y,
                                   int32_t *idx_out, int32_t *count_out, float *xrot_out,
                                   int mode, void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!(t >= 0.f)) return LAROSA_ERR_INVALID_ARG;  // negative or NaN
  Sel sel;
  sel.thr = true;
  sel.k = d_in;
  sel.thr_key = threshold_key_of(t);
  sel.count_out = count_out;
  return layer_entry(x, act_dtype, Qt, q_block, W_folded, w_dtype, B, d_in, d_out, sel, y,
                     idx_out, xrot_out, mode, ws, ws_bytes, stream);
  });
}

size_t larosa_swiglu_workspace_bytes(int64_t B, int64_t d_in, int64_t f, int64_t k, int mode) LAROSA_NOEXCEPT {
  return guard_size([&]() -> size_t {
  if (f < 1) return 0;
  const size_t base = larosa_workspace_bytes(B, d_in, 2 * f, k, mode);
  if (base == 0) return 0;
  const int64_t b1 = B < 1 ? 1 : B;
  return base + align256(static_cast<size_t>(b1) * 2 * f * 4);  // the gate|up rows
  });
}

int larosa_interleave_gate_up(const void *W, void *W_il, int64_t d_in, int64_t f, int dtype,
                              larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!W || !W_il) return LAROSA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return LAROSA_ERR_DTYPE;
  if (d_in < 1 || f < 1 || f % interleave_block(dtype)) return LAROSA_ERR_SHAPE;
  if (!aligned16(W) || !aligned16(W_il)) return LAROSA_ERR_ALIGNMENT;
  const size_t bytes = static_cast<size_t>(d_in) * 2 * f * dt_size(dtype);
  const char *a = static_cast<const char *>(W);
  const char *b = static_cast<const char *>(W_il);
  if (a < b + bytes && b < a + bytes) return LAROSA_ERR_INVALID_ARG;
  if (int st = device_status()) return st;
  return launched(launch_interleave(W, W_il, d_in, f, interleave_block(dtype), dtype,
                                    stream_of(stream)));
  });
}

int larosa_swiglu_layer_forward(const void *x, int act_dtype, const void *Qt, int64_t q_block,
                                const void *W_il, int w_dtype, int64_t B, int64_t d_in,
                                int64_t f, int64_t k, void *h, int32_t *idx_out,
                                float *xrot_out, int mode, void *ws, size_t ws_bytes,
                                larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  Sel sel;
  sel.k = k;
  return swiglu_entry(x, act_dtype, Qt, q_block, W_il, w_dtype, B, d_in, f, sel, h, idx_out,
                      xrot_out, mode, ws, ws_bytes, stream);
  });
}

int larosa_threshold_swiglu_layer_forward(const void *x, int act_dtype, const void *Qt,
                                          int64_t q_block, const void *W_il, int w_dtype,
                                          int64_t B, int64_t d_in, int64_t f, float t, void *h,
                                          int32_t *idx_out, int32_t *count_out, float *xrot_out,
                                          int mode, void *ws, size_t ws_bytes,
                                          larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!(t >= 0.f)) return LAROSA_ERR_INVALID_ARG;
  Sel sel;
  sel.thr = true;
  sel.k = d_in;
  sel.thr_key = threshold_key_of(t);
  sel.count_out = count_out;
  return swiglu_entry(x, act_dtype, Qt, q_block, W_il, w_dtype, B, d_in, f, sel, h, idx_out,
                      xrot_out, mode, ws, ws_bytes, stream);
  });
}

int larosa_swiglu(const void *gu, void *h, int64_t B, int64_t f, int dtype,
                  larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(dtype)) return LAROSA_ERR_DTYPE;
  if (B < 0 || B > kMaxB || f < 1) return LAROSA_ERR_INVALID_ARG;
  if (B == 0) return LAROSA_OK;
  if (!gu || !h) return LAROSA_ERR_INVALID_ARG;
  if (f % 8) return LAROSA_ERR_ALIGNMENT;
  if (!aligned16(gu) || !aligned16(h)) return LAROSA_ERR_ALIGNMENT;
  if (int st = device_status()) return st;
  return launched(launch_swiglu(gu, h, B, f, dtype, stream_of(stream)));
  });
}

int larosa_rmsnorm(const void *h, void *out, int64_t B, int64_t d, float eps, int dtype,
                   larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(dtype)) return LAROSA_ERR_DTYPE;
  if (B < 0 || B > kMaxB || d < 1 || !(eps >= 0.f)) return LAROSA_ERR_INVALID_ARG;
  if (B == 0) return LAROSA_OK;
  if (!h || !out) return LAROSA_ERR_INVALID_ARG;
  if (int st = device_status()) return st;
  return launched(launch_rmsnorm(h, out, B, d, eps, dtype, stream_of(stream)));
  });
}

int larosa_rope(const void *qk, int64_t qk_stride, void *q_out, void *k_out, int64_t B,
                int64_t n_heads, int64_t n_kv_heads, int64_t d_head, int64_t pos, float theta,
                int dtype, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(dtype)) return LAROSA_ERR_DTYPE;
  if (B < 0 || B > kMaxB || n_heads < 1 || n_kv_heads < 1 || pos < 0 || !(theta > 0.f))
    return LAROSA_ERR_INVALID_ARG;
  if (d_head < 2 || d_head % 2 || d_head > 2 * kRopeMaxHalf ||
      qk_stride < (n_heads + n_kv_heads) * d_head)
    return LAROSA_ERR_SHAPE;
  if (B == 0) return LAROSA_OK;
  if (!qk || !q_out || !k_out) return LAROSA_ERR_INVALID_ARG;
  if (int st = device_status()) return st;
  return launched(launch_rope(qk, qk_stride, q_out, k_out, B, n_heads, n_kv_heads,
                              rope_table(d_head, static_cast<double>(pos),
                                         static_cast<double>(theta)),
                              dtype, stream_of(stream)));
  });
}

int larosa_qkv_rope_layer_forward(const void *x, int act_dtype, const void *Qt, int64_t q_block,
                                  const void *W_folded, int w_dtype, int64_t B, int64_t d_in,
                                  int64_t k, int64_t n_heads, int64_t n_kv_heads, int64_t d_head,
                                  int64_t pos, float theta, void *y, int32_t *idx_out,
                                  float *xrot_out, int mode, void *ws, size_t ws_bytes,
                                  larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (n_heads < 1 || n_kv_heads < 1 || pos < 0 || !(theta > 0.f) || n_heads > 4096 ||
      n_kv_heads > 4096)
    return LAROSA_ERR_INVALID_ARG;
  if (d_head < 2 || d_head % 2 || d_head > 2 * kRopeMaxHalf) return LAROSA_ERR_SHAPE;
  const int64_t d_out = (n_heads + 2 * n_kv_heads) * d_head;
  RopeArgs r;
  r.rot_cols = static_cast<int>((n_heads + n_kv_heads) * d_head);
  r.tab = rope_table(d_head, static_cast<double>(pos), static_cast<double>(theta));
  // folded only where whole heads fill the one-token product's column tiles
  // (512 columns, or 256 for outputs of at most 12288 columns)
  const SelectGatherPlan sgp = plan_select_gather(d_in, d_out, w_dtype);
  const bool foldable = (static_cast<int64_t>(sgp.lpr) * 8) % d_head == 0;
  Sel sel;
  sel.k = k;
  bool done = false;
  const int st = layer_entry(x, act_dtype, Qt, q_block, W_folded, w_dtype, B, d_in, d_out, sel,
                             y, idx_out, xrot_out, mode, ws, ws_bytes, stream,
                             foldable ? &r : nullptr, &done);
  if (st != LAROSA_OK || done || B == 0) return st;
  return launched(launch_rope_inplace(y, d_out, B, n_heads + n_kv_heads, r.tab, act_dtype,
                                      stream_of(stream)));
  });
}

size_t larosa_decode_attention_workspace_bytes(int64_t B, int64_t T, int64_t n_heads) LAROSA_NOEXCEPT {
  return guard_size([&]() -> size_t {
  if (B < 1 || B > kMaxB || T < 0 || T > 16384 || n_heads < 1) return 0;
  return decode_attention_ws_bytes(B, T, n_heads);
  });
}

int larosa_decode_attention(const void *q, const void *k_new, int64_t k_stride,
                            const void *v_new, int64_t v_stride, const void *k_cache,
                            const void *v_cache, void *out, int64_t B, int64_t T,
                            int64_t n_heads, int64_t n_kv_heads, int64_t d_head, int dtype,
                            void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(dtype)) return LAROSA_ERR_DTYPE;
  if (B < 0 || B > kMaxB || T < 0 || n_heads < 1 || n_kv_heads < 1) return LAROSA_ERR_INVALID_ARG;
  if (d_head != 128 || n_heads % n_kv_heads || T > 16384) return LAROSA_ERR_SHAPE;
  if (k_stride < n_kv_heads * d_head || v_stride < n_kv_heads * d_head) return LAROSA_ERR_SHAPE;
  if ((k_stride * dt_size(dtype)) % 16 || (v_stride * dt_size(dtype)) % 16)
    return LAROSA_ERR_ALIGNMENT;
  if (B == 0) return LAROSA_OK;
  if (!q || !k_new || !v_new || !out || (T > 0 && (!k_cache || !v_cache)))
    return LAROSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) ||
      !aligned16(v_cache) || !aligned16(out) || !aligned16(ws))
    return LAROSA_ERR_ALIGNMENT;
  if (!ws || ws_bytes < decode_attention_ws_bytes(B, T, n_heads)) return LAROSA_ERR_WORKSPACE;
  if (int st = device_status()) return st;
  return launched(launch_decode_attention(q, k_new, k_stride, v_new, v_stride, k_cache, v_cache,
                                          out, B, T, n_heads, n_kv_heads, dtype, ws,
                                          stream_of(stream)));
  });
}

size_t larosa_mlp_workspace_bytes(int64_t B, int64_t d, int64_t f, int64_t k1, int64_t k2,
                                  int mode) LAROSA_NOEXCEPT {
  return guard_size([&]() -> size_t { return mlp_layout(B, d, f, k1, k2, mode).total; });
}

int larosa_mlp_forward(const void *x, int act_dtype, const void *Qt1, int64_t q_block1,
                       const void *W_il, const void *Qt2, int64_t q_block2, const void *W_down,
                       int w_dtype, int64_t B, int64_t d, int64_t f, int64_t k1, int64_t k2,
                       void *h, void *y, int32_t *idx1_out, float *xrot1_out, int32_t *idx2_out,
                       float *xrot2_out, int mode, void *ws, size_t ws_bytes,
                       larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  const bool want_chain = (mode & LAROSA_CHAIN) != 0;
  mode &= ~LAROSA_CHAIN;
  // both linears rotate their own inputs here
  if (prerotated(mode)) return LAROSA_ERR_INVALID_ARG;
  const MlpLayout M = mlp_layout(B, d, f, k1, k2, mode);
  // every argument of both linears first
  if (int st = layer_args(x, act_dtype, Qt1, q_block1, W_il, w_dtype, B, d, 2 * f, k1, h,
                          xrot1_out, mode))
    return st;
  if (int st = layer_args(h, act_dtype, Qt2, q_block2, W_down, w_dtype, B, f, d, k2, y,
                          xrot2_out, mode))
    return st;
  if (f < 1 || f % interleave_block(w_dtype)) return LAROSA_ERR_SHAPE;
  if (B == 0) return LAROSA_OK;
  if (!aligned16(ws)) return LAROSA_ERR_ALIGNMENT;
  if (!ws || M.total == 0 || ws_bytes < M.total) return LAROSA_ERR_WORKSPACE;
  {
    const size_t hb = static_cast<size_t>(B) * f * dt_size(act_dtype);
    const char *hp = static_cast<const char *>(h), *xp = static_cast<const char *>(x);
    const size_t xb = static_cast<size_t>(B) * d * dt_size(act_dtype);
    if (hp < xp + xb && xp < hp + hb) return LAROSA_ERR_INVALID_ARG;  // h must not overlap x
  }
  if (int st = device_status()) return st;
  char *base = static_cast<char *>(ws);
  hipStream_t s = stream_of(stream);
  const bool chain = want_chain && mode == LAROSA_UNFUSED && B == 1 && act_dtype == LAROSA_BF16 &&
                     w_dtype == LAROSA_BF16 && select_gather_supported(d) &&
                     select_gather_supported(f) && chain_supported(q_block2, f);
  if (!chain) {
    // the two layer calls (other batches, modes and types)
    int st = swiglu_entry(x, act_dtype, Qt1, q_block1, W_il, w_dtype, B, d, f, Sel{false, k1},
                          h, idx1_out, xrot1_out, mode, base + M.up, M.up_bytes, stream);
    if (st != LAROSA_OK) return st;
    return layer_entry(h, act_dtype, Qt2, q_block2, W_down, w_dtype, B, f, d, Sel{false, k2}, y,
                       idx2_out, xrot2_out, mode, base + M.down, M.down_bytes, stream);
  }
  // One token: rotate x; the gate|up product with SiLU(gate)·up, chained into
  // the rotation of h; the down product.
  const Layout L1 = layout_for(1, d, 2 * f, k1, w_dtype);
  const Layout L2 = layout_for(1, f, d, k2, w_dtype);
  char *up = base + M.up;
  char *dn = base + M.down;
  float *xr1 = xrot1_out ? xrot1_out : reinterpret_cast<float *>(up + L1.x_rot);
  float *xr2 = xrot2_out ? xrot2_out : reinterpret_cast<float *>(dn + L2.x_rot);
  uint32_t *status = reinterpret_cast<uint32_t *>(up + L1.p.status);
  const uint32_t spin = g_spin_limit.load();
  if (launch_rotate(x, act_dtype, Qt1, w_dtype, xr1, 1, static_cast<int>(d),
                    static_cast<int>(q_block1), s) != hipSuccess)
    return LAROSA_ERR_LAUNCH;
  SelectGatherArgs g;
  g.x_rot = xr1;
  g.d_in = static_cast<int>(d);
  g.k = static_cast<int>(k1);
  g.w = W_il;
  g.w_dt = w_dtype;
  g.d_out = 2 * f;
  g.y = h;
  g.y_dt = act_dtype;
  g.idx_out = idx1_out;
  g.ws = up + L1.p.gather;
  g.swiglu = true;
  g.chain.qt = static_cast<const uint16_t *>(Qt2);
  g.chain.qb = static_cast<int>(q_block2);
  g.chain.f = static_cast<int>(f);
  g.chain.x_rot = xr2;
  g.chain.tile_flag = reinterpret_cast<uint32_t *>(up + L1.p.flags);
  g.chain.ctl = reinterpret_cast<uint64_t *>(up + L1.p.flags + chain_ctl_offset(f));
  g.chain.status = status;
  g.chain.spin_limit = spin;
  if (launch_select_gather(g, s) != hipSuccess) return LAROSA_ERR_LAUNCH;
  SelectGatherArgs g2;
  g2.x_rot = xr2;
  g2.d_in = static_cast<int>(f);
  g2.k = static_cast<int>(k2);
  g2.w = W_down;
  g2.w_dt = w_dtype;
  g2.d_out = d;
  g2.y = y;
  g2.y_dt = act_dtype;
  g2.idx_out = idx2_out;
  g2.ws = dn + L2.p.gather;
  return launched(launch_select_gather(g2, s));
  });
}

int larosa_topk_swiglu_rotate(const float *x_rot, int64_t d_in, int64_t k, const void *W_il,
                              int w_dtype, void *h, int64_t f, const void *Qt2, int64_t q_block2,
                              float *x_rot2, int32_t *idx_out, void *ws, size_t ws_bytes,
                              larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (w_dtype != LAROSA_BF16) return LAROSA_ERR_DTYPE;
  if (int st = check_sizes(1, d_in, k)) return st;
  if (!select_gather_supported(d_in) || !select_gather_supported(f)) return LAROSA_ERR_SHAPE;
  if (f < 1 || f % interleave_block(w_dtype)) return LAROSA_ERR_SHAPE;
  if (!chain_supported(q_block2, f)) return LAROSA_ERR_SHAPE;
  if (!x_rot || !W_il || !h || !Qt2 || !x_rot2) return LAROSA_ERR_INVALID_ARG;
  if (!aligned16(x_rot) || !aligned16(W_il) || !aligned16(h) || !aligned16(Qt2) ||
      !aligned16(x_rot2))
    return LAROSA_ERR_ALIGNMENT;
  const Prefix P = prefix_for(1, d_in, 2 * f, d_in, w_dtype);
  if (!ws || ws_bytes < P.end) return LAROSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LAROSA_ERR_ALIGNMENT;
  if (int st = device_status()) return st;
  char *base = static_cast<char *>(ws);
  SelectGatherArgs g;
  g.x_rot = x_rot;
  g.d_in = static_cast<int>(d_in);
  g.k = static_cast<int>(k);
  g.w = W_il;
  g.w_dt = w_dtype;
  g.d_out = 2 * f;
  g.y = h;
  g.y_dt = LAROSA_BF16;
  g.idx_out = idx_out;
  g.ws = base + P.gather;
  g.swiglu = true;
  g.chain.qt = static_cast<const uint16_t *>(Qt2);
  g.chain.qb = static_cast<int>(q_block2);
  g.chain.f = static_cast<int>(f);
  g.chain.x_rot = x_rot2;
  g.chain.tile_flag = reinterpret_cast<uint32_t *>(base + P.flags);
  g.chain.ctl = reinterpret_cast<uint64_t *>(base + P.flags + chain_ctl_offset(f));
  g.chain.status = reinterpret_cast<uint32_t *>(base + P.status);
  g.chain.spin_limit = g_spin_limit.load();
  return launched(launch_select_gather(g, stream_of(stream)));
  });
}

int larosa_residual_rmsnorm_rotate(const void *h, const void *o, void *h_out, void *a_out,
                                   const void *Qt, int64_t d, float eps, float *x_rot, int dtype,
                                   larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(dtype)) return LAROSA_ERR_DTYPE;
  if (dtype != LAROSA_BF16) return LAROSA_ERR_DTYPE;
  if (d <= 256 || d > 8192 || d % 8) return LAROSA_ERR_SHAPE;
  if (!(eps >= 0.f)) return LAROSA_ERR_INVALID_ARG;
  if (!h || !Qt || !x_rot || (o && !h_out)) return LAROSA_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(Qt) || !aligned16(x_rot) || !aligned16(o) ||
      !aligned16(h_out) || !aligned16(a_out))
    return LAROSA_ERR_ALIGNMENT;
  const size_t bytes = static_cast<size_t>(d) * 2;  // a bf16 row; x_rot is twice that
  auto overlap = [&](const void *p, size_t pn, const void *q, size_t qn) {
    const char *a = static_cast<const char *>(p), *b = static_cast<const char *>(q);
    return a && b && a < b + qn && b < a + pn;
  };
  // the outputs are written while every workgroup still reads h and o
  const void *outs[2] = {o ? h_out : nullptr, a_out};
  for (const void *w : outs)
    if (overlap(w, bytes, h, bytes) || overlap(w, bytes, o, bytes) ||
        overlap(w, bytes, x_rot, 2 * bytes))
      return LAROSA_ERR_INVALID_ARG;
  if (overlap(outs[0], bytes, a_out, bytes) || overlap(x_rot, 2 * bytes, h, bytes) ||
      overlap(x_rot, 2 * bytes, o, bytes))
    return LAROSA_ERR_INVALID_ARG;
  if (int st = device_status()) return st;
  return launched(launch_norm_rotate(h, o, o ? h_out : nullptr, a_out, Qt, x_rot, d, eps,
                                     stream_of(stream)));
  });
}

int larosa_residual_rmsnorm(void *h, const void *o, void *out, int64_t B, int64_t d, float eps,
                            int dtype, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(dtype)) return LAROSA_ERR_DTYPE;
  if (B < 0 || B > kMaxB || d < 1 || !(eps >= 0.f)) return LAROSA_ERR_INVALID_ARG;
  if (B == 0) return LAROSA_OK;
  if (!h || !o || !out) return LAROSA_ERR_INVALID_ARG;
  const size_t bytes = static_cast<size_t>(B) * d * dt_size(dtype);
  const char *hb = static_cast<const char *>(h), *ob = static_cast<const char *>(o),
             *qb = static_cast<const char *>(out);
  if ((qb < hb + bytes && hb < qb + bytes) || (qb < ob + bytes && ob < qb + bytes))
    return LAROSA_ERR_INVALID_ARG;  // out must not overlap h or o
  if (int st = device_status()) return st;
  return launched(launch_residual_rmsnorm(h, o, out, B, d, eps, dtype, stream_of(stream)));
  });
}

int larosa_topk_swiglu_gemv(const float *x_rot, int64_t d_in, int64_t k, const void *W_il,
                            int w_dtype, void *h, int h_dtype, int64_t f, int32_t *idx_out,
                            void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(w_dtype) || !dtype_ok(h_dtype)) return LAROSA_ERR_DTYPE;
  if (w_dtype == LAROSA_F32 && h_dtype == LAROSA_BF16) return LAROSA_ERR_DTYPE;
  if (int st = check_sizes(1, d_in, k)) return st;
  if (!select_gather_supported(d_in)) return LAROSA_ERR_SHAPE;
  if (f < 1 || f % interleave_block(w_dtype)) return LAROSA_ERR_SHAPE;
  if (!x_rot || !W_il || !h) return LAROSA_ERR_INVALID_ARG;
  if (!aligned16(x_rot) || !aligned16(W_il) || !aligned16(h)) return LAROSA_ERR_ALIGNMENT;
  const Prefix P = prefix_for(1, d_in, 2 * f, d_in, w_dtype);
  if (!ws || ws_bytes < P.end) return LAROSA_ERR_WORKSPACE;
  if (!aligned16(ws)) return LAROSA_ERR_ALIGNMENT;
  if (int st = device_status()) return st;
  SelectGatherArgs g;
  g.x_rot = x_rot;
  g.d_in = static_cast<int>(d_in);
  g.k = static_cast<int>(k);
  g.w = W_il;
  g.w_dt = w_dtype;
  g.d_out = 2 * f;
  g.y = h;
  g.y_dt = h_dtype;
  g.idx_out = idx_out;
  g.ws = static_cast<char *>(ws) + P.gather;
  g.swiglu = true;
  return launched(launch_select_gather(g, stream_of(stream)));
  });
}

int larosa_residual_add(void *h, const void *o, int64_t n, int dtype, larosa_stream_t stream) LAROSA_NOEXCEPT {
  return guard([&]() -> int {
  if (!dtype_ok(dtype)) return LAROSA_ERR_DTYPE;
  if (n < 0) return LAROSA_ERR_INVALID_ARG;
  if (n == 0) return LAROSA_OK;
  if (!h || !o) return LAROSA_ERR_INVALID_ARG;
  if (int st = device_status()) return st;
  return launched(launch_residual_add(h, o, n, dtype, stream_of(stream)));
  });
}

}  // extern "C"
