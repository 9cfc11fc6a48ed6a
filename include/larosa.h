/*
 * larosa.h — C ABI of the rotated Top-K sparse linear library (liblarosa.so)
 *
 * The method (LaRoSA; "La RoSA: Enhancing LLM Efficiency via Layerwise
 * Rotated Sparse Activation", abstract on the PMLR 267 proceedings page, and
 * the LaRoSA summary page, 方法详解 · 技术框架 "technical framework"):
 * every linear layer's input activation x is rotated by a layerwise
 * orthogonal matrix Q, then only the K entries of largest magnitude of the
 * rotated vector are kept and the rest set to zero. Because Q·Qᵀ = I, the
 * product (x·Q)·(Qᵀ·W) equals x·W; with Qᵀ folded offline into the weight
 * (W' = Qᵀ·W) the online work is
 *
 *     x_rot = x·Q                       (rotate)
 *     S     = Top-K of |x_rot|          (select; per token)
 *     y     = Σ_{i∈S} x_rot[i]·W'[i,:]  (gather: read only the K rows of W')
 *
 * Conventions for every call below
 *  - Matrices are row-major. W and W' are [d_in, d_out] (the x·W form), so
 *    one input channel owns one contiguous row.
 *  - The rotation argument is always the *prepared* rotation Qt = Qᵀ, packed
 *    block-diagonal: Qt is [d, q_block] row-major, rows c·q_block … (c+1)·
 *    q_block−1 holding block c transposed (q_block == d: one dense block).
 *    larosa_prepare_rotation writes it from Q.
 *  - All tensor pointers are device pointers owned by the caller. The library
 *    allocates no memory and never synchronises the host; each call only
 *    enqueues kernels on `stream` (a hipStream_t; NULL = default stream).
 *  - Every call checks its arguments on the host before any HIP call; on an
 *    error it enqueues nothing and returns the status, leaving outputs as
 *    they were. Nothing is thrown across the ABI.
 *  - Device pointers must be 16-byte aligned. Rows must be whole 16-byte
 *    units: d_out and q_block multiples of 8 (bf16) or 4 (fp32); d a
 *    multiple of 4. Sizes: 1 <= d <= 32768, 1 <= k <= d, B <= 64; B == 0 is
 *    an empty batch and returns LAROSA_OK without work.
 *  - Workspace: calls that take `ws` need at least larosa_workspace_bytes(…)
 *    bytes. The workspace must be zero-filled once before first use
 *    (larosa_workspace_init does it on the device); every call leaves it
 *    ready for the next call of the same shape (B, d_in, d_out, k) on the
 *    same stream. To use it for another shape, zero it again first. Calls
 *    that share one workspace must not run concurrently.
 */
#ifndef LAROSA_H
#define LAROSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LAROSA_ABI_VERSION 9

/* Every entry point is a no-throw C function: exceptions never cross the
 * ABI (a caught one is reported as LAROSA_ERR_INTERNAL). */
#ifdef __cplusplus
#define LAROSA_NOEXCEPT noexcept
#else
#define LAROSA_NOEXCEPT
#endif

typedef void *larosa_stream_t; /* hipStream_t */

/* Element types. */
enum { LAROSA_F32 = 0, LAROSA_BF16 = 1 };

/* Status codes. */
enum {
  LAROSA_OK = 0,
  LAROSA_ERR_INVALID_ARG = 1, /* null pointer, B < 0, k outside [1, d] … */
  LAROSA_ERR_SHAPE = 2,       /* q_block does not divide d, d too large … */
  LAROSA_ERR_ALIGNMENT = 3,   /* pointer not 16-byte aligned, ragged rows */
  LAROSA_ERR_DTYPE = 4,       /* unsupported element type or combination */
  LAROSA_ERR_WORKSPACE = 5,   /* workspace missing or too small */
  LAROSA_ERR_NO_DEVICE = 6,   /* no HIP device visible */
  LAROSA_ERR_LAUNCH = 7,      /* a kernel launch failed */
  LAROSA_ERR_NONFINITE = 8,   /* LAROSA_VALIDATE: the rotated input holds NaN or ±inf */
  LAROSA_ERR_TIMEOUT = 9,     /* a bounded device-side wait gave up (see
                                 larosa_workspace_status) */
  LAROSA_ERR_INTERNAL = 10    /* an unexpected host-side failure (e.g. an
                                 exception) was caught at the ABI */
};

/* Execution modes of larosa_layer_forward. */
enum { LAROSA_UNFUSED = 0, LAROSA_FUSED = 1 };

/* Mode flag, OR-ed into the mode of larosa_layer_forward,
 * larosa_swiglu_layer_forward and their workspace-size calls: the rotation
 * accumulates in fp64 and rounds once to fp32 (larosa_rotate_fp64), so the
 * selected index sets follow the exactly rounded x·Q. With this flag
 * LAROSA_FUSED runs the unfused steps. Any other bit is an invalid mode. */
enum { LAROSA_ROTATE_FP64 = 2 };

/* Debug flag, OR-ed into the mode like LAROSA_ROTATE_FP64: after the
 * rotation the call checks every rotated entry on the device, waits for the
 * stream (the one place the library synchronises the host) and, if any is
 * NaN or ±inf, returns LAROSA_ERR_NONFINITE before the selection runs,
 * leaving y as it was. The Top-K rule orders finite magnitudes and ±inf, and
 * leaves NaN undefined (the oracle rejects it); this mode turns such input
 * into a status. With it, LAROSA_FUSED runs the unfused steps, so that the
 * check happens between the rotation and the selection. Not for graph
 * capture (it waits on the stream). */
enum { LAROSA_VALIDATE = 4 };

/* Mode flag of larosa_mlp_forward and larosa_mlp_workspace_bytes only (any
 * other call takes it as an invalid mode): run the rotation of h inside the
 * gate|up product's launch where that form applies (see larosa_mlp_forward).
 * On MI355X this chained form measures slower than the two launches it
 * replaces, so it is not the default. */
enum { LAROSA_CHAIN = 8 };

/* Mode flag of larosa_layer_forward, larosa_swiglu_layer_forward,
 * larosa_qkv_rope_layer_forward and their workspace-size calls: x already
 * holds the rotated input x_rot = x·Q, fp32 [B, d_in] (for instance from
 * larosa_residual_rmsnorm_rotate), so the rotation step is skipped and Qt
 * is not read (it may be NULL; q_block must still be valid). act_dtype
 * names the element type of y only. The remaining steps (select, union,
 * product and the epilogues) are those of the call without the flag, on
 * the same x_rot, so y has the same bits. xrot_out must be NULL; the flag
 * cannot be combined with LAROSA_ROTATE_FP64, and LAROSA_FUSED with it runs
 * the unfused steps. */
enum { LAROSA_PREROTATED = 16 };

/* LAROSA_ABI_VERSION of the loaded library. */
int larosa_abi_version(void) LAROSA_NOEXCEPT;

/* A static, human-readable name for a status code (never NULL). */
const char *larosa_status_string(int status) LAROSA_NOEXCEPT;

/* Bytes of workspace needed by larosa_layer_forward with these sizes in the
 * given mode. It also covers larosa_topk_select, larosa_topk_gemv, larosa_sparse_gemv and
 * larosa_dense_gemv on the same (B, d_in, d_out, k). Returns 0 for invalid
 * sizes. */
size_t larosa_workspace_bytes(int64_t B, int64_t d_in, int64_t d_out,
                              int64_t k, int mode) LAROSA_NOEXCEPT;

/* Zero-fills `bytes` of workspace with a device kernel (no memset node). */
int larosa_workspace_init(void *ws, size_t bytes, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Device-side status of a workspace. The one-launch (LAROSA_FUSED) kernel
 * waits on other workgroups of its grid; every such wait is bounded, and
 * one that gives up (for instance when the grid is not all resident because
 * other work holds the GPU) records LAROSA_ERR_TIMEOUT in the first word of
 * the workspace, finishes without faulting and leaves the workspace ready
 * for the next call; that call's outputs are then not to be trusted. This
 * call enqueues a copy of the recorded status into *status_out (a device
 * int32: LAROSA_OK or LAROSA_ERR_TIMEOUT) and clears it, in stream order;
 * read status_out after the stream has reached it. ws: a workspace of
 * larosa_workspace_bytes / larosa_swiglu_workspace_bytes size, 16-byte
 * aligned. */
int larosa_workspace_status(void *ws, int32_t *status_out, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Spin limit of the bounded device-side waits above for launches enqueued
 * after this call (process-wide; the default is 1 << 22 polls, far beyond
 * any wait of a resident grid). A limit of 0 makes every such wait give up
 * at once, which exercises the LAROSA_ERR_TIMEOUT path: every kernel still
 * runs to its end and stays within its buffers. Returns the previous limit. */
uint32_t larosa_set_spin_limit(uint32_t limit) LAROSA_NOEXCEPT;

/* Prepared rotation: Qt = Qᵀ block by block. Q is packed [d/q_block,
 * q_block, q_block] (block c of the block-diagonal rotation, row-major);
 * Qt is written as [d, q_block] with Qt[c·q_block + j][i] = Q[c][i][j].
 * Exact (a transpose). Q and Qt must not overlap. dtype: F32 or BF16.
 * The rotation is the method's per-layer orthogonal matrix (LaRoSA summary
 * page, 方法详解 · 关键设计: random or learned). Offline; not on the hot path. */
int larosa_prepare_rotation(const void *Q, void *Qt, int64_t d,
                            int64_t q_block, int dtype,
                            larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Folded weight W' = Qᵀ·W (= Qt·W), formed in fp32 and rounded to nearest
 * even in w_dtype. Qt: prepared rotation [d_in, q_block]; W, W_folded:
 * [d_in, d_out]; all three in w_dtype (F32 or BF16). W_folded must not
 * overlap W or Qt. Offline; not on the hot path. Folding follows from the
 * orthogonality the LaRoSA abstract names: (x·Q)·(Qᵀ·W) = x·W. */
int larosa_fold_weights(const void *Qt, int64_t q_block, const void *W,
                        void *W_folded, int64_t d_in, int64_t d_out,
                        int w_dtype, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Rotation, stage 1 of the method (LaRoSA summary page, 技术框架):
 * x_rot[b, :] = x[b, :]·Q for b < B, accumulated in fp32.
 * x: [B, d] in x_dtype (F32 or BF16); Qt: prepared rotation [d, q_block] in
 * q_dtype (F32 or BF16); x_rot: [B, d] fp32. */
int larosa_rotate(const void *x, int x_dtype, const void *Qt, int64_t q_block,
                  int q_dtype, float *x_rot, int64_t B, int64_t d,
                  larosa_stream_t stream) LAROSA_NOEXCEPT;

/* The same rotation with fp64 accumulation: every product x[b, i]·Q[i, j]
 * of two bf16 or two fp32 values is exact in fp64, the sum is kept in fp64
 * and rounded to nearest even fp32 once. x_rot then equals fp32(x·Q) of the
 * exact product except where that product lies within about 2^-53·√q_block
 * (relative) of an fp32 rounding midpoint, so the Top-K sets taken from it
 * match the exact rotation's (the fixed-K selection of stage 2 depends on
 * the rotated magnitudes only). Arguments, layout and errors as
 * larosa_rotate. Qt is read once per 8 tokens. One token costs about what
 * the fp32 form does (both read Qt once); from a few tokens on, the fp64
 * conversions and FMAs, not HBM, bound it. */
int larosa_rotate_fp64(const void *x, int x_dtype, const void *Qt,
                       int64_t q_block, int q_dtype, float *x_rot, int64_t B,
                       int64_t d, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Top-K selection, stage 2 of the method (LaRoSA summary page, 技术框架;
 * the abstract's fixed-K "consistent model-level sparsity"): for each token
 * b, the k entries of x_rot[b, :] with the largest magnitude. Magnitude is
 * the fp32 value with the sign dropped (−0 equals +0); among equal
 * magnitudes the lower index is kept. NaN inputs give an unspecified but
 * in-bounds selection.
 *   idx  [B, k] int32: kept indices of each token, ascending (required)
 *   val  [B, k] fp32:  x_rot at those indices, unscaled (required)
 *   xs   [B, d] fp32:  x_rot with unkept entries set to 0 (may be NULL
 *                      when B == 1 and no union is asked for)
 * Row union (B > 1, optional: pass union_idx == NULL to skip):
 *   union_idx   [d] int32: ascending union of the tokens' kept indices
 *   union_count [1] int32: its length |U| (written on the device)
 *   union_coef  [d, B] fp32: union_coef[j·B + b] = xs[b, union_idx[j]]
 * When the union is asked for, xs is required, and ws must hold at least
 * larosa_workspace_bytes(B, d, d_out, k, mode) bytes for some valid d_out and
 * mode (a status area and the tokens' bit masks come first in every
 * layout), zero-filled once before first use like any layer workspace: the
 * union list is taken by the selection launch itself (its last workgroup to
 * finish), through an arrival counter in the status area that each call
 * leaves at zero. Without the union ws may be NULL. */
int larosa_topk_select(const float *x_rot, int64_t B, int64_t d, int64_t k,
                       int32_t *idx, float *val, float *xs, int32_t *union_idx,
                       int32_t *union_count, float *union_coef, void *ws,
                       size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Gather product (the saving the LaRoSA abstract names: computation and
 * memory transfers of zeroed channels are skipped):
 *   y[b, :] = Σ_{j < n} coef[j·B + b] · W'[rows[j], :]
 * rows: [max_rows] int32 row indices (entries outside [0, d_in) contribute
 * nothing); n_rows: device int32 holding n (clamped to max_rows), or NULL
 * for n = max_rows; coef: [max_rows, B] fp32; W_folded: [d_in, d_out] in
 * w_dtype; y: [B, d_out] in y_dtype, fp32 accumulation. Only the n listed
 * rows of W' are read. For B == 1 pass (idx, NULL, k, val) from
 * larosa_topk_select; for B > 1 pass (union_idx, union_count, d_in,
 * union_coef). */
int larosa_sparse_gemv(const int32_t *rows, const int32_t *n_rows,
                       int64_t max_rows, const float *coef,
                       const void *W_folded, int w_dtype, void *y,
                       int y_dtype, int64_t B, int64_t d_in, int64_t d_out,
                       void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Selection folded into the product, for one token (LaRoSA summary page,
 * 方法详解 · 技术框架: keep the k largest-magnitude rotated entries, set the
 * rest to zero, so only their rows of the folded weight are read):
 *   y = Σ_{i ∈ S} x_rot[i] · W'[i, :],  S = Top-k of |x_rot| (the rule of
 *   larosa_topk_select: fp32 magnitude, equal magnitudes keep the lower index)
 * x_rot: [d_in] fp32 (one token); W_folded: [d_in, d_out] in w_dtype;
 * y: [d_out] in y_dtype (F32, or BF16 with BF16 weights), fp32 accumulation.
 * idx_out: [k] int32, the kept indices ascending, or NULL. One launch:
 * every workgroup of the product computes the exact rule itself, so no index
 * list goes through memory. d_in <= 16384 (LAROSA_ERR_SHAPE above). ws:
 * workspace of larosa_workspace_bytes(1, d_in, d_out, k, …). */
int larosa_topk_gemv(const float *x_rot, int64_t d_in, int64_t k,
                     const void *W_folded, int w_dtype, void *y, int y_dtype,
                     int64_t d_out, int32_t *idx_out, void *ws, size_t ws_bytes,
                     larosa_stream_t stream) LAROSA_NOEXCEPT;

/* larosa_topk_gemv with SiLU(gate)·up folded in, for one token: the
 * selection and the product over the interleaved folded gate|up weight W_il
 * ([d_in, 2f], see larosa_interleave_gate_up), writing h [f] = SiLU(g)·u of
 * the sums rounded to h_dtype (the step larosa_swiglu_layer_forward runs
 * after its rotation). f a multiple of the interleave block. ws: workspace of
 * larosa_workspace_bytes(1, d_in, 2f, k, …). Other arguments as
 * larosa_topk_gemv. */
int larosa_topk_swiglu_gemv(const float *x_rot, int64_t d_in, int64_t k, const void *W_il,
                            int w_dtype, void *h, int h_dtype, int64_t f, int32_t *idx_out,
                            void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* larosa_topk_swiglu_gemv chained into the next linear's rotation, one
 * launch for one token: h = SiLU(gate)·up as larosa_topk_swiglu_gemv writes
 * it, and x_rot2 [f] fp32 = h·Q2 as larosa_rotate computes it for one token
 * (the same bits for Q2 blocks of 2056 to 4096 channels). Qt2: the down
 * linear's prepared rotation [f, q_block2] in bf16, q_block2 a multiple of 8
 * and at most 4096; bf16 weights and h. The launch's workgroups wait
 * (bounded) for the blocks of h the others write; a wait that gives up
 * records LAROSA_ERR_TIMEOUT for larosa_workspace_status. The step
 * larosa_mlp_forward runs after its first rotation. ws: workspace of
 * larosa_workspace_bytes(1, d_in, 2f, k, …). */
int larosa_topk_swiglu_rotate(const float *x_rot, int64_t d_in, int64_t k, const void *W_il,
                              int w_dtype, void *h, int64_t f, const void *Qt2, int64_t q_block2,
                              float *x_rot2, int32_t *idx_out, void *ws, size_t ws_bytes,
                              larosa_stream_t stream) LAROSA_NOEXCEPT;

/* One rotated sparse linear layer of the method, both online stages of the
 * LaRoSA summary page (方法详解 · 技术框架: stage 1 rotates the layer's input
 * activation with its orthogonal matrix; stage 2 keeps the K entries of
 * largest magnitude and sets the rest to zero) followed by the product that
 * reads only the kept rows of the folded weight (the LaRoSA abstract: the
 * zeroed channels cost neither computation nor memory transfer):
 *   rotate → select → (row union when B > 1) → gather,
 * for every projection that shares the input x. W_folded is the
 * column concatenation of those projections' folded weights
 * ([W'_q | W'_k | W'_v] or [W'_gate | W'_up]), [d_in, d_out] in w_dtype.
 * x: [B, d_in] and y: [B, d_out] in act_dtype; Qt: prepared rotation
 * [d_in, q_block] in w_dtype. idx_out [B, k] and xrot_out [B, d_in] (fp32)
 * are optional copies of the selection and the rotated input (NULL skips
 * them). mode: LAROSA_UNFUSED (one kernel per step) or LAROSA_FUSED (one
 * persistent launch for B == 1; other B fall back to the unfused steps),
 * optionally OR-ed with LAROSA_ROTATE_FP64 and LAROSA_VALIDATE. */
int larosa_layer_forward(const void *x, int act_dtype, const void *Qt,
                         int64_t q_block, const void *W_folded, int w_dtype,
                         int64_t B, int64_t d_in, int64_t d_out, int64_t k,
                         void *y, int32_t *idx_out, float *xrot_out, int mode,
                         void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* larosa_layer_forward for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, whose place takes
 * a 16 MiB device-resident array of the library (one per GPU, held until
 * the process ends). The call itself allocates nothing. Requests needing
 * more than 16 MiB (larosa_workspace_bytes of the sizes) return
 * LAROSA_ERR_WORKSPACE before any work; mode must be LAROSA_UNFUSED,
 * optionally with LAROSA_ROTATE_FP64 or LAROSA_VALIDATE
 * (LAROSA_ERR_INVALID_ARG otherwise, LAROSA_PREROTATED included: the
 * one-launch form reports through a workspace the caller could not read).
 * The array is zero-filled on the
 * first call on a device and again whenever the sizes, mode or types differ
 * from the previous call's on that device (a fill kernel on `stream`).
 * Every call on one GPU shares its array: calls that overlap on one GPU
 * (from two streams or two host threads) race. Other arguments, outputs
 * and errors as larosa_layer_forward. */
int larosa_layer_forward_noalloc(const void *x, int act_dtype, const void *Qt,
                                 int64_t q_block, const void *W_folded, int w_dtype,
                                 int64_t B, int64_t d_in, int64_t d_out, int64_t k,
                                 void *y, int32_t *idx_out, float *xrot_out, int mode,
                                 larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Dense reference product y = x·W over every row of W, with the same
 * streaming and fp32 accumulation as larosa_sparse_gemv. x: [B, d_in] and
 * y: [B, d_out] in act_dtype; W: [d_in, d_out] in w_dtype. The baseline that
 * the sparse product is compared against; not a step of the method. */
int larosa_dense_gemv(const void *x, int act_dtype, const void *W,
                      int w_dtype, void *y, int64_t B, int64_t d_in,
                      int64_t d_out, void *ws, size_t ws_bytes,
                      larosa_stream_t stream) LAROSA_NOEXCEPT;

/* SwiGLU between the two linears of an MLP (LLaMA-style; the method
 * sparsifies the input of the down projection, which is this output):
 *   h[b, i] = SiLU(gu[b, i]) · gu[b, f + i],  SiLU(z) = z / (1 + e^−z)
 * gu: [B, 2f] ([gate | up]); h: [B, f]; both in dtype (F32 or BF16);
 * arithmetic in fp32, rounded to nearest even. f a multiple of 8. */
int larosa_swiglu(const void *gu, void *h, int64_t B, int64_t f, int dtype,
                  larosa_stream_t stream) LAROSA_NOEXCEPT;

/* ---- The gate|up linear of a SwiGLU MLP with SiLU(gate)·up folded in ----
 * The method sparsifies the input of every linear (LaRoSA summary page,
 * 方法详解 · 技术框架); in a SwiGLU MLP the gate and up projections share one
 * input, and their outputs meet only in h = SiLU(gate)·up, which is the
 * input of the down projection. Storing the folded [W'_gate | W'_up] with
 * the two halves' columns interleaved in blocks (256 columns for bf16
 * weights, 128 for fp32) puts matching gate and up columns in every column
 * tile of the product, which can then write h directly. */

/* W_il[r, (i / b)·2b + i mod b] = W[r, i] (gate) and W_il[r, (i / b)·2b + b
 * + i mod b] = W[r, f + i] (up) for the block b above; W: [d_in, 2f] =
 * [gate | up] (folded or not: the permutation acts on columns only). f must
 * be a multiple of b (LAROSA_ERR_SHAPE otherwise); W and W_il must not
 * overlap. Offline; not on the hot path. */
int larosa_interleave_gate_up(const void *W, void *W_il, int64_t d_in, int64_t f, int dtype,
                              larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Workspace for larosa_swiglu_layer_forward: the layer's own
 * (larosa_workspace_bytes(B, d_in, 2f, k, mode)) plus room for the gate|up
 * rows. 0 for invalid sizes. */
size_t larosa_swiglu_workspace_bytes(int64_t B, int64_t d_in, int64_t f, int64_t k, int mode) LAROSA_NOEXCEPT;

/* h[b, i] = SiLU(g[b, i])·u[b, i] with [g | u] = larosa_layer_forward of x
 * over the interleaved folded weight W_il ([d_in, 2f], see above): g and u
 * are rounded to act_dtype first, exactly as larosa_layer_forward followed by
 * larosa_swiglu would see them. h: [B, f] in act_dtype. For one token in
 * LAROSA_UNFUSED mode the selection, product and SwiGLU are one launch
 * after the rotation; other cases run the layer into the workspace and then
 * the SwiGLU step. Other arguments as for larosa_layer_forward; ws: at least
 * larosa_swiglu_workspace_bytes(B, d_in, f, k, mode) bytes, zero-filled once. */
int larosa_swiglu_layer_forward(const void *x, int act_dtype, const void *Qt, int64_t q_block,
                                const void *W_il, int w_dtype, int64_t B, int64_t d_in,
                                int64_t f, int64_t k, void *h, int32_t *idx_out,
                                float *xrot_out, int mode, void *ws, size_t ws_bytes,
                                larosa_stream_t stream) LAROSA_NOEXCEPT;

/* ---- A whole SwiGLU MLP: both rotated sparse linears --------------------
 * Every linear input of the MLP is rotated and Top-K sparsified (LaRoSA
 * summary page, 方法详解 · 技术框架): the gate|up linear reads x, h =
 * SiLU(gate)·up, and the down linear reads h. */

/* Workspace bytes of larosa_mlp_forward (0 for invalid sizes or mode). */
size_t larosa_mlp_workspace_bytes(int64_t B, int64_t d, int64_t f, int64_t k1, int64_t k2,
                                  int mode) LAROSA_NOEXCEPT;

/* h = larosa_swiglu_layer_forward(x; Qt1, W_il, k1) and then
 * y = larosa_layer_forward(h; Qt2, W_down, k2), with the same results as the
 * two calls (bit for bit for Q2 blocks of 2056 to 4096 channels; within the
 * rotation's fp32 error bound otherwise). x: [B, d], h: [B, f], y: [B, d]
 * in act_dtype; W_il: the interleaved folded gate|up weight [d, 2f]; W_down:
 * folded [f, d]; Qt1 [d, q_block1] and Qt2 [f, q_block2] prepared rotations;
 * optional copies of the selections and rotated inputs as for the layer
 * calls (NULL skips). mode: a layer-call mode, optionally OR-ed with
 * LAROSA_CHAIN. With LAROSA_CHAIN, for one token in bf16 with the unfused
 * steps and the fp32 rotation, and Q2 blocks of at most 4096 channels (a
 * multiple of 8), the rotation of h runs inside the gate|up product's
 * launch, overlapping its tail: that launch's workgroups wait (bounded) for
 * the blocks of h written by the others, and a wait that gives up records
 * LAROSA_ERR_TIMEOUT for larosa_workspace_status. Everything else runs the
 * two layer calls. ws: larosa_mlp_workspace_bytes bytes (same mode),
 * zero-filled once; h must not overlap x. */
int larosa_mlp_forward(const void *x, int act_dtype, const void *Qt1, int64_t q_block1,
                       const void *W_il, const void *Qt2, int64_t q_block2, const void *W_down,
                       int w_dtype, int64_t B, int64_t d, int64_t f, int64_t k1, int64_t k2,
                       void *h, void *y, int32_t *idx1_out, float *xrot1_out, int32_t *idx2_out,
                       float *xrot2_out, int mode, void *ws, size_t ws_bytes,
                       larosa_stream_t stream) LAROSA_NOEXCEPT;

/* ---- Magnitude-threshold selection (the contrast to the fixed Top-K) ----
 * The R-Sparse summary page (研究流程与方法 · R-Sparse框架设计) masks every
 * input channel whose magnitude is below a threshold t(s) chosen for a
 * sparsity budget s; the LaRoSA abstract names such magnitude pruning as the
 * source of fluctuating sparsity that its fixed K avoids. These calls run
 * that selection on the rotated activation: channel i of a token is kept iff
 * |x_rot[i]| >= t, compared on the same keys as the Top-K (fp32 bits with the
 * sign cleared, so −0 equals +0 and ±inf rank highest). The number kept
 * varies per token and is written to device memory. t must be a
 * non-negative number (LAROSA_ERR_INVALID_ARG for negative or NaN). */

/* Workspace bytes of larosa_calibrate_threshold (a few KB). */
size_t larosa_calibrate_workspace_bytes(void) LAROSA_NOEXCEPT;

/* *t_out (device fp32) = the keep-th largest magnitude |x_rot[i]| over the
 * n entries x_rot[0 .. n) (e.g. the rotated activations of N calibration
 * tokens, n = N·d). Keeping |x| >= t then keeps keep of those entries, or
 * more when the keep-th magnitude is tied. For a sparsity of p percent use
 * keep = floor(n·(100 − p)/100). Exact radix select on the keys
 * (deterministic). 1 <= keep <= n < 2^31; ws: at least
 * larosa_calibrate_workspace_bytes() bytes, 16-byte aligned, overwritten.
 * Offline: not on the decode path. */
int larosa_calibrate_threshold(const float *x_rot, int64_t n, int64_t keep, float *t_out,
                               void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Per-token threshold selection: for each token b the indices i with
 * |x_rot[b, i]| >= t, ascending, in idx[b·d .. b·d + count[b]) (rows of
 * capacity d; entries past count[b] are not written), their values in val
 * (same layout; may be NULL), count [B] (device), and xs [B, d] (the kept
 * values, zero elsewhere; may be NULL). The union outputs, workspace and
 * errors are as for larosa_topk_select. */
int larosa_threshold_select(const float *x_rot, int64_t B, int64_t d, float t, int32_t *idx,
                            int32_t *count, float *val, float *xs, int32_t *union_idx,
                            int32_t *union_count, float *union_coef, void *ws, size_t ws_bytes,
                            larosa_stream_t stream) LAROSA_NOEXCEPT;

/* larosa_layer_forward with the threshold selection in place of the Top-K:
 * rotate, keep |x_rot| >= t per token, (row union for B > 1), product over
 * the kept rows of W_folded. idx_out ([B, d_in], rows of capacity d_in),
 * count_out ([B] kept channels per token) and xrot_out may be NULL. mode:
 * LAROSA_UNFUSED, optionally with LAROSA_ROTATE_FP64 (LAROSA_FUSED runs the
 * same unfused steps). For one token the selection and the product are one
 * launch after the rotation. ws: larosa_workspace_bytes(B, d_in, d_out,
 * d_in, mode) bytes, zero-filled once. Other arguments and errors as
 * larosa_layer_forward. */
int larosa_threshold_layer_forward(const void *x, int act_dtype, const void *Qt,
                                   int64_t q_block, const void *W_folded, int w_dtype, int64_t B,
                                   int64_t d_in, int64_t d_out, float t, void *y,
                                   int32_t *idx_out, int32_t *count_out, float *xrot_out,
                                   int mode, void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* larosa_swiglu_layer_forward with the threshold selection (see above);
 * ws: larosa_swiglu_workspace_bytes(B, d_in, f, d_in, mode) bytes. */
int larosa_threshold_swiglu_layer_forward(const void *x, int act_dtype, const void *Qt,
                                          int64_t q_block, const void *W_il, int w_dtype,
                                          int64_t B, int64_t d_in, int64_t f, float t, void *h,
                                          int32_t *idx_out, int32_t *count_out, float *xrot_out,
                                          int mode, void *ws, size_t ws_bytes,
                                          larosa_stream_t stream) LAROSA_NOEXCEPT;

/* ---- Low-rank compensation of the dropped channels ---------------------
 * The R-Sparse summary page (研究流程与方法 · R-Sparse框架设计) sends the
 * masked remainder of the input through a rank-r factorisation of the
 * weight taken from its SVD, A_r = U_r·Σ_r^½ and B_r = Σ_r^½·V_rᵀ, and adds
 * that to the sparse output. Applied to the rotated layer (x·W convention,
 * W' = U·Σ·Vᵀ):
 *   y = xs·W' + (x_rot − xs)·A_r·B_r
 * with xs the method's Top-K sparsified rotated input. The factors are
 * inputs prepared offline (any SVD of W'); the caller stores B_r directly
 * below W' as W_ext = [W'; B_r] ([d_in + r, d_out] in w_dtype), so the
 * low-rank term is r more rows of the same product and both parts share one
 * fp32 sum per output, rounded once to act_dtype. The first d_in rows of
 * W_ext are W' itself and serve the other layer calls unchanged. */

/* Workspace bytes of larosa_lowrank_layer_forward; 0 for invalid sizes. */
size_t larosa_lowrank_workspace_bytes(int64_t B, int64_t d_in, int64_t d_out, int64_t k,
                                      int64_t r) LAROSA_NOEXCEPT;

/* Rotate, keep each token's Top-k, then y [B, d_out] = xs·W' + (x_rot −
 * xs)·A_r·B_r. A_r: [d_in, r] in w_dtype (row-major); 1 <= r <= min(256,
 * d_in, d_out) (LAROSA_ERR_INVALID_ARG otherwise). mode: LAROSA_UNFUSED or
 * LAROSA_FUSED (both run the separate steps), optionally with
 * LAROSA_ROTATE_FP64. ws: larosa_lowrank_workspace_bytes(B, d_in, d_out, k,
 * r) bytes, zero-filled once. Other arguments and errors as
 * larosa_layer_forward. */
int larosa_lowrank_layer_forward(const void *x, int act_dtype, const void *Qt, int64_t q_block,
                                 const void *W_ext, const void *A_r, int64_t r, int w_dtype,
                                 int64_t B, int64_t d_in, int64_t d_out, int64_t k, void *y,
                                 int32_t *idx_out, float *xrot_out, int mode, void *ws,
                                 size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* ---- The decoder layer around the rotated linears ----------------------
 * The pages apply the rotated Top-K sparsification to every linear layer of a
 * pretrained decoder (LaRoSA summary page, 方法详解 · 技术框架) and describe no
 * other part of the layer. These calls implement the LLaMA-style layer used
 * by the decoder workloads; they are not steps of the method. fp32 inside,
 * one rounding to dtype (F32 or BF16) per output. */

/* RMSNorm with unit gain: out[b, :] = h[b, :] / sqrt(mean(h[b, :]²) + eps).
 * h, out: [B, d]; they may be the same buffer. */
int larosa_rmsnorm(const void *h, void *out, int64_t B, int64_t d, float eps, int dtype,
                   larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Rotate-half rotary embedding at position pos: for each head, channel i
 * (i < d_head/2) pairs with i + d_head/2 and both turn by
 * pos · theta^(−2i/d_head) (the angle in fp64 on the host, its cosine and
 * sine rounded to fp32; d_head even and at most 256). Row b of qk holds n_heads query heads, then
 * n_kv_heads key heads (d_head channels each) at qk + b·qk_stride; the
 * results go to q_out [B, n_heads·d_head] and k_out [B, n_kv_heads·d_head],
 * which must not overlap qk. */
int larosa_rope(const void *qk, int64_t qk_stride, void *q_out, void *k_out, int64_t B,
                int64_t n_heads, int64_t n_kv_heads, int64_t d_head, int64_t pos, float theta,
                int dtype, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* The q|k|v linear of a decoder layer with the rotary embedding applied:
 * y = larosa_layer_forward(x; Qt, W_folded, k) over d_out = (n_heads +
 * 2·n_kv_heads)·d_head columns (the q heads, then the k heads, then v),
 * after which the q and k heads of every token's row are rotated in place
 * at position pos as larosa_rope computes it (same rounding: each output
 * is rounded to act_dtype before the rotation). The LaRoSA summary page
 * (方法详解 · 技术框架) rotates and sparsifies the input of the attention
 * projections like every other linear; the embedding is the decoder's own
 * step. For one token in bf16 with the one-token product (unfused modes)
 * the rotation runs in that product's epilogue, so no extra launch is made;
 * otherwise a second kernel applies it. y: [B, d_out] in act_dtype. Other
 * arguments, the workspace (larosa_workspace_bytes(B, d_in, d_out, k,
 * mode)) and errors as larosa_layer_forward; LAROSA_ERR_INVALID_ARG for
 * head counts outside 1..4096, pos < 0 or theta <= 0; LAROSA_ERR_SHAPE for
 * a d_head that is odd or above 256. */
int larosa_qkv_rope_layer_forward(const void *x, int act_dtype, const void *Qt, int64_t q_block,
                                  const void *W_folded, int w_dtype, int64_t B, int64_t d_in,
                                  int64_t k, int64_t n_heads, int64_t n_kv_heads, int64_t d_head,
                                  int64_t pos, float theta, void *y, int32_t *idx_out,
                                  float *xrot_out, int mode, void *ws, size_t ws_bytes,
                                  larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Workspace bytes of larosa_decode_attention (per-chunk partial results of
 * 64 positions); 0 for invalid sizes. */
size_t larosa_decode_attention_workspace_bytes(int64_t B, int64_t T, int64_t n_heads) LAROSA_NOEXCEPT;

/* Single-query softmax attention of every query head over its key/value
 * head's T cached positions plus the new token's own key and value:
 *   out[b, h] = Σ_t softmax_t(q[b,h]·k_t / sqrt(d_head)) · v_t,
 * with key/value head h / (n_heads / n_kv_heads). q, out: [B, n_heads·128];
 * the new key and value of token b start at k_new + b·k_stride and
 * v_new + b·v_stride (n_kv_heads·128 channels each); caches are
 * [B, n_kv_heads, T, 128] (head-major). d_head must be 128; T <= 16384.
 * The positions are taken in chunks of 64 whose partial softmax results
 * are combined in chunk order (deterministic) by a second launch; ws: at
 * least larosa_decode_attention_workspace_bytes(B, T, n_heads) bytes,
 * 16-byte aligned, overwritten by each call. */
int larosa_decode_attention(const void *q, const void *k_new, int64_t k_stride,
                            const void *v_new, int64_t v_stride, const void *k_cache,
                            const void *v_cache, void *out, int64_t B, int64_t T,
                            int64_t n_heads, int64_t n_kv_heads, int64_t d_head, int dtype,
                            void *ws, size_t ws_bytes, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* The residual add followed by the next RMSNorm, one launch: for each token
 * row b, h[b, :] = h[b, :] + o[b, :] (rounded to dtype, written back), then
 * out[b, :] = RMSNorm(h[b, :]) as larosa_rmsnorm computes it from the
 * rounded sum (the same bits as larosa_residual_add then larosa_rmsnorm).
 * h, o, out: [B, d]; out must not overlap h or o (h and o may be equal). */
int larosa_residual_rmsnorm(void *h, const void *o, void *out, int64_t B, int64_t d, float eps,
                            int dtype, larosa_stream_t stream) LAROSA_NOEXCEPT;

/* One token: the residual add and RMSNorm folded into the rotation of the
 * normalised row (stage 1 of the method, LaRoSA summary page, 方法详解 ·
 * 技术框架: each linear input is rotated by its layer's Q), in one launch:
 *   v = o ? bf16(h + o) : h;  a = bf16(v / sqrt(mean(v²) + eps));
 *   x_rot = a·Q  (fp32 [d]),
 * with the bits of larosa_residual_rmsnorm (or larosa_rmsnorm when o is
 * NULL) followed by larosa_rotate. With o, the residual sum v is written to
 * h_out, which must not overlap h or o (every workgroup reads h and o whole,
 * so the sum cannot be written in place); a_out, if not NULL, receives a.
 * No output (h_out, a_out, x_rot) may overlap h, o or another output
 * (LAROSA_ERR_INVALID_ARG).
 * Qt: the prepared rotation of a dense Q, [d, d] (q_block == d). bf16 only
 * (LAROSA_ERR_DTYPE otherwise); d a multiple of 8 above 256 and at most
 * 8192 (the sizes whose one-token rotation takes one wave per channel;
 * LAROSA_ERR_SHAPE otherwise); every pointer 16-byte aligned. The decoder glue uses
 * it with LAROSA_PREROTATED layer calls. */
int larosa_residual_rmsnorm_rotate(const void *h, const void *o, void *h_out, void *a_out,
                                   const void *Qt, int64_t d, float eps, float *x_rot, int dtype,
                                   larosa_stream_t stream) LAROSA_NOEXCEPT;

/* Residual add in place: h[i] = h[i] + o[i] for i < n. */
int larosa_residual_add(void *h, const void *o, int64_t n, int dtype, larosa_stream_t stream) LAROSA_NOEXCEPT;

#ifdef __cplusplus
}
#endif

#endif /* LAROSA_H */
