// Host-side launch interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace larosa {

enum Dt { kF32 = 0, kBF16 = 1 };

inline int dt_size(int dt) { return dt == kF32 ? 4 : 2; }

// Status code a bounded device-side wait that gave up writes into the
// status word of its workspace (LAROSA_ERR_TIMEOUT of the C ABI).
constexpr uint32_t kStatusTimeout = 9;

// --- status word and debug checks ---
// *flag = 1 if any of x[0 .. n) is NaN or ±inf, else 0 (flag cleared first).
hipError_t launch_flag_nonfinite(const float *x, int64_t n, uint32_t *flag, hipStream_t s);
// *out = *word; *word = 0 (one thread, stream order).
hipError_t launch_take_status(uint32_t *word, int32_t *out, hipStream_t s);

// --- rotation (dot product per output channel against the prepared Qt) ---
hipError_t launch_rotate(const void *x, int x_dt, const void *qt, int q_dt,
                         float *x_rot, int B, int d, int qb, hipStream_t s);
// --- magnitude-threshold selection and its calibration ---
uint32_t threshold_key_of(float t);  // fp32 bits of t with the sign cleared
// idx/val rows have capacity d; count[b] = kept channels of token b; val,
// xs, count and mask may be NULL.
hipError_t launch_threshold_select(const float *x_rot, int B, int d, uint32_t thr_key,
                                   int32_t *idx, int32_t *count, float *val, float *xs,
                                   uint32_t *mask, hipStream_t s);
size_t calibrate_ws_bytes();
// t_out = the keep-th largest magnitude of x[0 .. n); 1 <= keep <= n < 2^31.
hipError_t launch_calibrate(const float *x, int64_t n, uint32_t keep, float *t_out, void *ws,
                            hipStream_t s);

// --- low-rank compensation of the dropped channels (r <= 256) ---
size_t lowrank_part_bytes(int64_t B, int64_t d, int64_t r);
// Partial sums of u [B, r] = (x_rot − xs)·A_r per row range, into part
// (lowrank_part_bytes).
hipError_t launch_lowrank_proj(const float *x_rot, const float *xs, const void *a_r, int w_dt,
                               int B, int d, int r, float *part, hipStream_t s);
// The kept rows (or union) followed by rows d_in .. d_in + r − 1 of W_ext,
// with their coefficients (u summed from part): packed (coef, ld = list
// capacity) or split and transposed (coef_hl, ld = ldc).
hipError_t launch_lowrank_list(const int32_t *base, const int32_t *n_dev, int n_host, int d_in,
                               int r, const float *xs, const float *part, int B, int64_t ld,
                               int32_t *rows_ext, int32_t *n_ext, float *coef, void *coef_hl,
                               hipStream_t s);

// fp64 accumulation, one rounding to fp32 (any B; one pass per 8 tokens)
hipError_t launch_rotate_f64(const void *x, int x_dt, const void *qt, int q_dt, float *x_rot,
                             int B, int d, int qb, hipStream_t s);

// --- Top-K selection (one workgroup per token) ---
// With n_parts > 1, x_rot arrives as n_parts k-range partial sums of the
// rotation (slice p at parts + p·B·d, added in order p = 0, 1, ...) and is
// written here; select_takes_parts says whether this d allows n_parts.
bool select_takes_parts(int d, int n_parts);
// With counter != NULL (B > 1, masks written) the launch also takes the row
// union: the last workgroup to arrive writes u_idx and *u_count and resets
// the counter (a word that is zero before the call and after it).
struct UnionTail {
  uint32_t *counter = nullptr;
  int32_t *u_idx = nullptr;
  int32_t *u_count = nullptr;
};
hipError_t launch_select(float *x_rot, int B, int d, int k, int32_t *idx, float *val, float *xs,
                         uint32_t *mask, hipStream_t s, const float *parts = nullptr,
                         int n_parts = 1, const UnionTail &ut = UnionTail{});

// --- row union of B > 1 selections (from the per-token bit masks); with
// u_coef == NULL only the list and its count are written ---
hipError_t launch_union(const uint32_t *mask, const float *xs, int B, int d,
                        int32_t *u_idx, int32_t *u_count, float *u_coef,
                        hipStream_t s);
// the coefficients alone, for a list taken by the selection launch
hipError_t launch_union_coef(const int32_t *u_idx, const int32_t *u_count, const float *xs, int B,
                             int d, float *u_coef, hipStream_t s);

inline int mask_words(int d) { return (d + 31) / 32; }

// --- gather-rows product y[b,:] = Σ_j coef(j,b)·W[row(j),:] ---
enum CoefMode { kCoefPacked = 0, kCoefActF32 = 1, kCoefActBF16 = 2 };

struct GatherPlan {
  int vec;             // columns per lane (one 16-byte load)
  int waves;           // waves per workgroup, all on one column tile
  int tiles;           // column tiles of 64·vec columns
  int splits;          // row splits per tile (R); partial sums when R > 1
  int rows_per_split;  // rows of the row list handled by one workgroup
};
GatherPlan plan_gather(int B, int64_t max_rows, int64_t d_out, int w_dt);
// Workspace for the split-row reduction: partial sums, then one counter per
// column tile. Counters must start at zero; the kernel leaves them at zero.
size_t gather_ws_bytes(const GatherPlan &p, int B, int64_t d_out);
// Workspace for a launch_gather call over a batch of B tokens (groups of at
// most eight tokens run one after another and reuse the area).
size_t gather_batch_ws_bytes(int B, int64_t max_rows, int64_t d_out, int w_dt);

struct GatherArgs {
  const int32_t *rows;     // NULL: row j is row j
  const int32_t *n_rows;   // device count, NULL: max_rows
  int64_t max_rows;
  const void *coef;        // packed [max_rows, B] fp32, or activation [B, d_in]
  int coef_mode;
  const void *w;
  int w_dt;
  int64_t d_in, d_out;
  void *y;
  int y_dt;
  int B;                   // tokens in the batch
  int b0 = 0;              // first token of this launch's group (set internally)
  void *ws;                // gather_ws_bytes(plan) bytes
};
hipError_t launch_gather(const GatherArgs &a, hipStream_t s);

// --- selection folded into the product, one token ---
struct SelectGatherPlan {
  int lpr;     // lanes per row: tiles of lpr·V columns (64, or 32 for narrow bf16 outputs)
  int tiles;   // column tiles
  int splits;  // channel ranges per tile (partial sums when > 1)
  int cps;     // channels per range
};
SelectGatherPlan plan_select_gather(int64_t d_in, int64_t d_out, int w_dt);
// Counters (one per column tile, at offset 0, zero between calls) and
// partial sums.
size_t select_gather_ws_bytes(int64_t d_in, int64_t d_out, int w_dt);
bool select_gather_supported(int64_t d_in);
// The chained form (see select_gather.hip): after the SwiGLU product, rotate
// h [f] by the next linear's prepared Q (bf16, blocks of qb) into x_rot.
// tile_flag: one word per product column tile (f / 256 of them); ctl: the
// launch's control block (two queue words, the epoch word and the count of
// finished tiles). Both sit in the workspace, zero-filled before first use;
// the kernel takes its epoch from the control block and advances it.
struct ChainArgs {
  const uint16_t *qt = nullptr;  // NULL: no chain
  int qb = 0;
  int f = 0;
  float *x_rot = nullptr;
  uint32_t *tile_flag = nullptr;
  uint64_t *ctl = nullptr;
  uint32_t *status = nullptr;       // kStatusTimeout when a wait gave up (may be NULL)
  uint32_t spin_limit = 1u << 22;
};
// Bytes of a chained launch's tile flags over f h channels, then its control
// block (24 bytes, 8-byte aligned). One flag per product column tile:
// f / 64 + 1 words cover tiles of 512, 256 or 128 columns.
inline size_t chain_flag_bytes(int64_t f) { return (static_cast<size_t>(f / 64 + 1) * 4 + 7) / 8 * 8 + 24; }
inline size_t chain_ctl_offset(int64_t f) { return chain_flag_bytes(f) - 24; }
bool chain_supported(int64_t q_block, int64_t f);
// The rotary embedding's per-pair cosine and sine at one position, for
// heads of dh <= 2·kRopeMaxHalf channels: angle pos·theta^(-2i/dh) in fp64
// on the host, its cosine and sine rounded to fp32. Every RoPE kernel takes
// the same table (by value), so they agree bit for bit.
constexpr int kRopeMaxHalf = 128;
struct RopeTable {
  int dh = 0;
  float cs[kRopeMaxHalf];
  float sn[kRopeMaxHalf];
};
RopeTable rope_table(int64_t dh, double pos, double theta);  // host
// RoPE folded into a one-token product's epilogue (the q|k|v linear of a
// decoder layer): output columns below rot_cols are heads of tab.dh channels
// (dividing the 512-column tile) rotated with the table, pairing channel i
// with i + dh/2 (the split-half form of larosa_rope); the rest (v) are
// stored as they are.
struct RopeArgs {
  int rot_cols = 0;  // 0: no RoPE
  RopeTable tab;
};
struct SelectGatherArgs {
  const float *x_rot;  // [d_in] fp32
  int d_in, k;
  const void *w;       // [d_in, d_out]
  int w_dt;
  int64_t d_out;
  void *y;             // [d_out]
  int y_dt;
  int32_t *idx_out;    // [k] ascending kept indices, or NULL
  void *ws;
  // swiglu: W's columns are gate|up interleaved in blocks of half a tile and
  // y is h [d_out / 2] = SiLU(gate)·up of the sums rounded to y's type.
  bool swiglu = false;
  // by_threshold: keep the channels whose key (fp32 bits, sign cleared) is
  // >= thr_key instead of the Top-k; idx_out then has capacity d_in and the
  // number kept goes to count_out (either may be NULL).
  bool by_threshold = false;
  uint32_t thr_key = 0;
  int32_t *count_out = nullptr;
  ChainArgs chain;
  RopeArgs rope;
};
hipError_t launch_select_gather(const SelectGatherArgs &a, hipStream_t s);

// --- matrix-core forms for batches of 2..64 tokens in bf16 ---
constexpr int kMfmaMinB = 2;
bool mfma_supported(int64_t B, int act_dt, int w_dt);
// Rotation; qb % 32 == 0. With ws == NULL the k-range is not split (one
// launch, x_rot written directly); otherwise ws holds rotate_mfma_ws_bytes.
// With parts_out, k-range partial sums that the selection can take are
// left in ws unsummed and *parts_out is their count (1: x_rot written).
int rotate_mfma_splits(int64_t B, int64_t d, int64_t qb);
size_t rotate_mfma_ws_bytes(int64_t B, int64_t d, int64_t qb);
hipError_t launch_rotate_mfma(const void *x, const void *qt, float *x_rot, int B, int d, int qb,
                              void *ws, hipStream_t s, int *parts_out = nullptr);
// Product over a row list with coefficients stored split and transposed
// (store_coef_hl in common.hpp; B · ldc · 4 bytes, ldc = mfma_coef_ld(max_rows);
// entries past the list's end must be finite, normally zero). ws holds
// gather_mfma_ws_bytes.
struct MfmaGatherPlan {
  int col_groups;      // workgroups across the columns (256 columns each)
  int splits;          // row splits, summed by a second kernel when > 1
  int rows_per_split;  // a multiple of 32
};
MfmaGatherPlan plan_gather_mfma(int64_t B, int64_t max_rows, int64_t d_out);
size_t gather_mfma_ws_bytes(int64_t B, int64_t max_rows, int64_t d_out);
int64_t mfma_coef_ld(int64_t max_rows);
hipError_t launch_gather_mfma(const int32_t *rows, const int32_t *n_rows, int64_t max_rows,
                              int64_t d_in, const void *coef_hl, int64_t ldc, const void *w,
                              void *y, int B, int64_t d_out, void *ws, hipStream_t s);
// The union of the B masks ([B, ceil(d/32)] words, d <= 32768) as u_idx
// (ascending) and *u_count, and the split coefficients of xs[b, u_idx[j]]
// for j < |U|, zero for j in [|U|, ldc), in one launch.
hipError_t launch_union_coef_mask(const uint32_t *mask, const float *xs, int B, int d,
                                  int64_t ldc, void *coef_hl, int32_t *u_idx, int32_t *u_count,
                                  hipStream_t s);
// Split coefficients of coef[j · B + b] for j < max_rows, zero up to ldc.
hipError_t launch_coef_transpose(const float *coef, int B, int64_t max_rows, int64_t ldc,
                                 void *coef_hl, hipStream_t s);
// Split coefficients of a bf16 activation x [B, d_in], zero up to ldc.
hipError_t launch_act_to_coef_t(const void *x, int B, int64_t d_in, int64_t ldc, void *coef_hl,
                                hipStream_t s);
// Upper bound of gather_mfma_ws_bytes over every row-list length.
size_t gather_mfma_ws_bound(int64_t B, int64_t d_out);
// Upper bound of rotate_mfma_ws_bytes over every block width of d.
size_t rotate_mfma_ws_bound(int64_t B, int64_t d);

// --- fused rotate → select → gather for one token (persistent launch) ---
constexpr int kFusedMaxD = 16384;          // 32 channels per thread of 512
constexpr int kFusedMaxRowsPerUnit = 1024;  // LDS row list of one work unit
constexpr int kFusedMaxGrid = 2048;         // bound used to size the workspace

struct FusedPlan {
  int grid, tiles, splits, chans_per_split;
  // workspace layout: synchronisation words at 0, then these regions
  size_t tile_off, flags_off, xrot_off, partial_off, bytes;
};
FusedPlan plan_fused(int64_t d_in, int64_t d_out, int64_t k, int w_dt, int grid);
bool fused_supported(int64_t B, int64_t d_in, int act_dt, int w_dt);

struct FusedArgs {
  const void *x, *qt, *wf;
  void *y;
  int w_dt;
  int d_in, q_block, k;
  int64_t d_out;
  int32_t *idx_out;   // may be NULL
  float *xrot_out;    // may be NULL (x_rot then lives in the workspace)
  void *ws;           // plan_fused(..., kFusedMaxGrid).bytes, zeroed before first use
  uint32_t *status;   // status word: kStatusTimeout when a bounded wait gave up
  uint32_t spin_limit = 1u << 22;  // polls before a wait gives up
};
hipError_t launch_fused_linear(const FusedArgs &a, hipStream_t s);

// --- device-resident workspace of larosa_layer_forward_noalloc ---
struct ScratchShape {
  int64_t B, d_in, d_out, k;
  int mode, act_dt, w_dt;
};
size_t scratch_capacity();
// This device's scratch address in *out, zero-filled on `s` first when the
// shape differs from the previous call's on this device (need bytes).
// hipErrorInvalidValue when need exceeds scratch_capacity().
hipError_t scratch_acquire(const ScratchShape &shape, size_t need, hipStream_t s, void **out);

// --- offline preparation ---
hipError_t launch_transpose_blocks(const void *q, void *qt, int64_t d, int64_t qb,
                                   int dt, hipStream_t s);
hipError_t launch_fold(const void *qt, int64_t qb, const void *w, void *wf,
                       int64_t d_in, int64_t d_out, int dt, hipStream_t s);

// --- glue ---
hipError_t launch_swiglu(const void *gu, void *h, int64_t B, int64_t f, int dt,
                         hipStream_t s);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s);
// Gate|up columns interleaved in blocks of ib (half a product column tile:
// 256 bf16 or 128 fp32 columns), so one tile holds matching gate and up
// columns.
inline int64_t interleave_block(int w_dt) { return w_dt == kF32 ? 128 : 256; }
hipError_t launch_swiglu_il(const void *gu, void *h, int64_t B, int64_t f, int64_t ib, int dt,
                            hipStream_t s);
hipError_t launch_interleave(const void *w, void *out, int64_t d_in, int64_t f, int64_t ib,
                             int dt, hipStream_t s);

// --- decoder layer around the rotated linears ---
hipError_t launch_rmsnorm(const void *h, void *out, int64_t B, int64_t d, float eps, int dt,
                          hipStream_t s);
hipError_t launch_rope(const void *qk, int64_t stride, void *q_out, void *k_out, int64_t B,
                       int64_t n_heads, int64_t n_kv, const RopeTable &tab, int dt,
                       hipStream_t s);
// RoPE in place on the first n_rot heads of each row (row b at qk + b·stride).
hipError_t launch_rope_inplace(void *qk, int64_t stride, int64_t B, int64_t n_rot,
                               const RopeTable &tab, int dt, hipStream_t s);
// ws: decode_attention_ws_bytes (per-chunk partial results)
size_t decode_attention_ws_bytes(int64_t B, int64_t Tlen, int64_t n_heads);
hipError_t launch_decode_attention(const void *q, const void *k_new, int64_t k_stride,
                                   const void *v_new, int64_t v_stride, const void *kc,
                                   const void *vc, void *out, int64_t B, int64_t Tlen,
                                   int64_t n_heads, int64_t n_kv, int dt, void *ws,
                                   hipStream_t s);
hipError_t launch_residual_add(void *h, const void *o, int64_t n, int dt, hipStream_t s);
// One token, bf16, dense Q (q_block == d <= 8192, d % 8 == 0): x_rot =
// RMSNorm(h [+ o])·Q with the norm folded into the rotation; with o the
// rounded residual sum goes to h_out (another buffer); a_out (optional)
// receives the normalised row.
hipError_t launch_norm_rotate(const void *h, const void *o, void *h_out, void *a_out,
                              const void *qt, float *x_rot, int64_t d, float eps, hipStream_t s);
// h += o (rounded to dt, written back), then out = RMSNorm(h), per token row.
hipError_t launch_residual_rmsnorm(void *h, const void *o, void *out, int64_t B, int64_t d,
                                   float eps, int dt, hipStream_t s);

}  // namespace larosa
