/*
 * qs.h -- C ABI of the Q-Sparse inference hot path for AMD Instinct MI355X
 * (gfx950).  Library: libqs.so.
 *
 * Sources of the operations (cited by page title and section):
 *   [QS-TopK]   Q-Sparse news article (zxwl-tech.com, July 2024), section
 *               "Sparsification with the Top-K function": Y = X . W^T for every
 *               attention/FFN projection; keep the K entries of largest |x|
 *               (K a preset hyperparameter), mask M with X's shape, X (.) M
 *               replaces X in the product; squared-ReLU FFN; activations
 *               quantised before top-K with an epsilon-guarded denominator;
 *               1-bit (ternary) weights with alpha = mean |W|.
 *   [QS-Adv]    Q-Sparse aibase report (aibase.com, pt), section on the
 *               advantages of sparsity: top-K on every linear projection,
 *               I/O as the main inference bottleneck.
 *   [TS-Eq2]    Turbo Sparse summary (blog.csdn.net), Eq. 2: dReLU, ReLU
 *               after both the gate and the up projection.
 *   [TS-Eq3-4]  Turbo Sparse summary, Eq. 3-4: top-k% of the FFN
 *               intermediate by absolute value before W_down.
 *   [TS-Fig]    Turbo Sparse summary, per-layer zero-activation figure
 *               (about 90% of FFN neurons inactive) and its passage on the
 *               MoE model (2 of 8 experts per layer, ~85% of each expert's
 *               neurons inactive, ~3% of the layer's parameters per token).
 *   [QS-STE]    Q-Sparse news article, the back-propagation passage of the
 *               Top-K section: the gradient is computed with respect to the
 *               sparsified tensor and passed unchanged to the tensor before
 *               sparsification (straight-through estimator).
 *   [QS-Block]  Q-Sparse abstract (arXiv 2407.10969 listing page, authors'
 *               English abstract): Block Q-Sparse for batch training and
 *               inference; the same page's Chinese summary (method details,
 *               key-design item 3): activations split into blocks to use the
 *               hardware better.  The rule itself is not on the pages.
 *
 * Readings where the pages are silent (each is part of the contract):
 *   - top-K is per row (token); among equal |x| the lower index wins, so the
 *     selected set is unique; every row gets exactly min(K, D) selected
 *     entries, zero-valued ones included when a row has fewer nonzeros;
 *   - |x| is ordered through its bit pattern: fp32 key = bits & 0x7FFFFFFF,
 *     bf16 key = bits & 0x7FFF, int8 key = |q|; +0 and -0 tie; inputs are
 *     finite (NaN/Inf are outside the contract);
 *   - activation quantiser: gamma = max|x|, s = 127 / (gamma + 1e-5),
 *     q = clamp(rint(x * s), -128, 127), IEEE binary32, round-to-nearest-even
 *     at every step; top-K then runs on |q|;
 *   - ternary weights: alpha = mean |W| over the whole tensor,
 *     t = clamp(rint(W / (alpha + 1e-5)), -1, 1);
 *   - squared ReLU is un-gated: h = relu(u)^2; the FFN intermediate stays
 *     fp32 between the up and the down projection.
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned.  They must point to ordinary
 *     (coarse-grained) device memory of the GPU that runs the stream, as
 *     hipMalloc or torch's CUDA allocator give: outputs and workspaces are
 *     updated with device-scope float and integer atomics, which host-pinned,
 *     managed and fine-grained memory do not support.  The library allocates
 *     no device memory, keeps no pointer after the call returns, and may
 *     access the buffers until the stream reaches the end of the enqueued
 *     work.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous and never synchronise the host.
 *   - Arguments are validated before anything is enqueued; on any error the
 *     call enqueues nothing, leaves every output untouched and returns a
 *     nonzero qs_status; qs_last_error() then describes it.  No C++
 *     exception crosses the ABI.  rows == 0 is a valid no-op.
 *   - Device pointers must be 16-byte aligned.
 *   - Split-K sums: by default a gather whose output is fp32 lets each of
 *     its workgroups add its partial tile into the (zeroed) output with
 *     float atomics, so the fp32 rounding of a sum depends on the order in
 *     which the splits arrive (results stay within the stated error bounds
 *     but may differ in the last bits between runs).  qs_set_deterministic(1)
 *     switches every entry point to fixed-order sums (the last workgroup of
 *     each tile adds the partials in split order): results are then bitwise
 *     deterministic for fixed inputs and shapes.  Integer results are exact
 *     either way.
 *   - A workspace (`ws`, `ws_bytes`) is device memory of at least the size
 *     qs_workspace_bytes() reports for the same op and shape; its contents
 *     are scratch and need no initialisation (qs_gather_linear excepted, see
 *     there).  Two calls that may run at the same time must not share a
 *     workspace.
 */
#ifndef QS_H
#define QS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qs_status {
    QS_OK = 0,
    QS_ERR_INVALID_ARG = 1,   /* null pointer, negative size, K outside [0, D], ... */
    QS_ERR_UNSUPPORTED = 2,   /* valid but not implemented: dtype/layout combo, misalignment */
    QS_ERR_WORKSPACE = 3,     /* ws NULL or ws_bytes below qs_workspace_bytes() */
    QS_ERR_HIP = 4            /* a HIP runtime call failed; qs_last_error() has its text */
} qs_status;

typedef enum qs_dtype {
    QS_F32 = 0,
    QS_BF16 = 1,
    QS_I8 = 2,
    /* (not values: they make every int a valid value of the type, so that an
       out-of-range argument is rejected as QS_ERR_UNSUPPORTED, not undefined) */
    QS_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
    QS_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} qs_dtype;

typedef enum qs_layout {
    QS_LAYOUT_WT = 0,   /* feature-major W^T [d_in, n_out], row j = weights of input feature j */
    QS_LAYOUT_W = 1,    /* neuron-major W [n_out, d_in] (nn.Linear layout) */
    QS_LAYOUT_RANGE_MIN_ = -0x7FFFFFFF - 1,   /* (range only, as for qs_dtype) */
    QS_LAYOUT_RANGE_MAX_ = 0x7FFFFFFF
} qs_layout;

typedef enum qs_act {
    QS_ACT_RELU2 = 0,     /* h = relu(u)^2                       [QS-TopK]  */
    QS_ACT_DRELU = 1,     /* h = relu(x W_gate^T + b_g) * relu(x W_up^T + b_u)   [TS-Eq2] */
    QS_ACT_RELU2_GLU = 2, /* h = relu(x W_gate^T)^2 * (x W_up^T)  [QS-TopK] */
    QS_ACT_RANGE_MIN_ = -0x7FFFFFFF - 1,      /* (range only, as for qs_dtype) */
    QS_ACT_RANGE_MAX_ = 0x7FFFFFFF
} qs_act;

typedef enum qs_op {
    QS_OP_TOPK_MASK = 0,
    QS_OP_SPARSE_LINEAR = 1,
    QS_OP_SPARSE_LINEAR_I8T = 2,
    QS_OP_SPARSE_FFN_RELU2 = 3,
    QS_OP_SPARSE_FFN_DRELU = 4,
    QS_OP_GATHER_LINEAR = 5,
    QS_OP_SPARSE_FFN_RELU2_GLU = 6,
    QS_OP_SPARSE_LINEAR_BACKWARD = 7,
    QS_OP_BLOCK_SPARSE_LINEAR = 8,
    QS_OP_SPARSE_MOE_FFN = 9,    /* rows = tokens * top_k (the (token, expert) pairs) */
    QS_OP_RANGE_MIN_ = -0x7FFFFFFF - 1,       /* (range only, as for qs_dtype) */
    QS_OP_RANGE_MAX_ = 0x7FFFFFFF
} qs_op;

/*
 * qs_topk_mask -- per-row top-K by |x| with ties to the lower index  [QS-TopK]
 *
 *   x       device, [rows, d] row-major, dtype xt (QS_F32, QS_BF16 or QS_I8).
 *   k       0 <= k <= d.
 *   mask    device u8 [rows, d] or NULL: 1 at the selected entries, else 0.
 *   idx     device i32 [rows, k] or NULL: selected indices, ascending.
 *   tau     device u32 [rows] or NULL: key of the K-th largest entry
 *           (0xFFFFFFFF when k == 0).
 *   cutoff  device i32 [rows] or NULL: one past the index of the last
 *           selected entry whose key equals tau (0 when k == 0); entry j is
 *           selected iff key_j > tau or (key_j == tau and j < cutoff).
 *   xs      device fp32 [rows, d] or NULL: the sparsified activation X (.) M
 *           (exact conversion of x at the selected entries, +0 elsewhere).
 *   Limits: d <= 1<<24.
 */
qs_status qs_topk_mask(const void* x, qs_dtype xt, int64_t rows, int64_t d, int64_t k,
                       uint8_t* mask, int32_t* idx, uint32_t* tau, int32_t* cutoff,
                       float* xs, void* stream);

/*
 * qs_sparse_linear -- Y = (X (.) M) . W^T with M the per-row top-K mask of X
 * [QS-TopK], [QS-Adv].
 *
 *   x       device [rows, d_in], dtype xt (QS_F32 or QS_BF16).
 *   k       0 <= k <= d_in.
 *   w       device weights, dtype wt_t (QS_F32 or QS_BF16), layout w_layout:
 *           QS_LAYOUT_WT  W^T [d_in, n_out]: the gather path, which reads only
 *                         the rows of W^T selected by some token of the batch
 *                         (any rows; meant for decode batches).  One bf16
 *                         token with bf16 weights, d_in <= 8192 and n_out <=
 *                         16384 (both multiples of 8) takes one launch with
 *                         fixed-order sums, whatever qs_set_deterministic says;
 *           QS_LAYOUT_W   W [n_out, d_in]: the masked dense MFMA path for large
 *                         token batches; needs xt == wt_t == QS_BF16.
 *   y       device [rows, n_out], dtype yt (QS_F32 or QS_BF16, bf16 rounded
 *           to nearest-even from the fp32 sum).
 *   Arithmetic: fp32 accumulation of the products of the input values.
 *   The products are exact except in one case: with bf16 weights, fp32 x and
 *   tiles of 8 to 16 tokens, the gather runs on the bf16 matrix cores and
 *   carries each selected fp32 activation as the sum of two bf16 numbers
 *   (hi = bf16(x), lo = bf16(x - hi)), a relative error of at most 2^-18 per
 *   activation, inside the fp32 bound 1e-5 * sum |x w|.
 *   Alignment: n_out % 8 == 0 (bf16 weights) or n_out % 4 == 0 (fp32), and
 *   d_in % 8 == 0 for QS_LAYOUT_W.
 */
qs_status qs_sparse_linear(const void* x, qs_dtype xt, int64_t rows, int64_t d_in, int64_t k,
                           const void* w, qs_dtype wt_t, qs_layout w_layout, int64_t n_out,
                           void* y, qs_dtype yt, void* ws, size_t ws_bytes, void* stream);

/*
 * qs_sparse_linear_pitched -- qs_sparse_linear with the row pitch of the
 * weights given  [QS-TopK], [QS-Adv].
 *
 *   ldw     elements from one row of w to the next: the natural pitch (n_out
 *           for QS_LAYOUT_WT, d_in for QS_LAYOUT_W) gives qs_sparse_linear.
 *           Any other pitch needs QS_LAYOUT_WT (every batch size: the gather
 *           paths), ldw >= n_out and a multiple of 8, and W^T (d_in x ldw)
 *           smaller than 1 GiB; QS_ERR_INVALID_ARG or QS_ERR_UNSUPPORTED
 *           otherwise, before anything is enqueued.  The padding columns are
 *           never read.
 *   Why: every workgroup of the gather reads one 128-byte column segment of
 *   each selected row; with a pitch that is a multiple of 512 bytes (the
 *   natural ones of 7B shapes: 8192 and 22016 bytes) those segments sit at
 *   one or two offsets modulo 1 KiB in every row and some tiles' lines pile
 *   onto a subset of the memory channels, so their workgroups finish last.  Rows padded by 64 bf16 (an odd multiple of 128 bytes)
 *   spread every tile over all channels.
 */
qs_status qs_sparse_linear_pitched(const void* x, qs_dtype xt, int64_t rows, int64_t d_in,
                                   int64_t k, const void* w, int64_t ldw, qs_dtype wt_t,
                                   qs_layout w_layout, int64_t n_out, void* y, qs_dtype yt,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * qs_gather_linear -- Y = Xs . W^T for an already sparsified Xs (for example
 * the xs output of qs_topk_mask), reading only the rows of W^T whose input
 * feature is nonzero for some row of Xs  [QS-TopK], [QS-Adv].
 *
 *   xs      device fp32 [rows, d_in].
 *   wt      device W^T [d_in, n_out], dtype wt_t (QS_F32 or QS_BF16), rows ldw
 *           elements apart.
 *   ldw     n_out, or a larger multiple of 8 (padded rows: see
 *           qs_sparse_linear_pitched); QS_ERR_INVALID_ARG otherwise.
 *   y       device [rows, n_out], dtype yt (QS_F32 or QS_BF16).
 *   Arithmetic and alignment as qs_sparse_linear with QS_LAYOUT_WT.
 *   Workspace: sized by qs_workspace_bytes(QS_OP_GATHER_LINEAR, ...); unlike
 *   the other entry points it must be zero-filled once before its first use
 *   (its first 16 KiB hold split-K counters that every call leaves zero), so
 *   that the call is a single kernel launch.
 */
qs_status qs_gather_linear(const float* xs, int64_t rows, int64_t d_in, const void* wt,
                           qs_dtype wt_t, int64_t n_out, int64_t ldw, void* y, qs_dtype yt,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * qs_gather_linear_acc -- Y += Xs . W^T into an fp32 Y, reading the same rows
 * of W^T as qs_gather_linear  [QS-TopK], [QS-Adv].  This is the gather that
 * qs_sparse_linear and qs_sparse_ffn run when their output is fp32 and
 * fixed-order sums are not asked for: every workgroup adds its partial tile
 * into y with float atomics (no handoff between the K-splits), so the
 * rounding of each sum depends on the arrival order of the splits, whatever
 * qs_set_deterministic says.
 *
 *   xs, wt, wt_t, rows, d_in, n_out, ldw: as qs_gather_linear.
 *   y     device fp32 [rows, n_out], read and written.
 *   Workspace: as qs_gather_linear (its counters are not touched).
 *   Limits: as qs_gather_linear; fp32 weights need rows <= 8
 *   (QS_ERR_UNSUPPORTED otherwise).
 */
qs_status qs_gather_linear_acc(const float* xs, int64_t rows, int64_t d_in, const void* wt,
                               qs_dtype wt_t, int64_t n_out, int64_t ldw, float* y, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * qs_topk_gather_linear_acc -- Y += (X (.) M) . W^T into an fp32 Y, with M the
 * per-row top-K mask of X by |x| (ties to the lower index)  [QS-TopK],
 * [TS-Eq3-4]: the selection and the gather in one launch, with no selection
 * output and no sparsified copy of X.  This is the down projection that
 * qs_sparse_ffn runs for one token when neither h nor its index list is
 * asked for.  Every workgroup (one per CU: a 64-column tile and a split of
 * the rows of W^T) finds the top-K descriptor of its row of X itself, keeps
 * the selected nonzero entries of its split and streams their rows of W^T;
 * the workgroups add their sums into y with float atomics, so the rounding
 * of each sum depends on their arrival order.  Meant for one or a few
 * tokens: each row of X gathers its own rows of W^T.
 *
 *   x       device fp32 [rows, d_in] (not sparsified).
 *   k       0 <= k <= d_in.
 *   wt      device bf16 W^T [d_in, n_out], rows ldw elements apart.
 *   ldw     n_out, or a larger multiple of 8 (padded rows: see
 *           qs_sparse_linear_pitched); QS_ERR_INVALID_ARG otherwise.
 *   y       device fp32 [rows, n_out], read and written.
 *   Arithmetic: fp32 products and sums (the fp32 tolerance).
 *   Limits: d_in % 4 == 0, d_in <= 16384, n_out % 8 == 0, rows <= 65535,
 *   W^T (d_in x ldw) smaller than 1 GiB; QS_ERR_UNSUPPORTED otherwise.  No
 *   workspace.
 */
qs_status qs_topk_gather_linear_acc(const float* x, int64_t rows, int64_t d_in, int64_t k,
                                    const void* wt, qs_dtype wt_t, int64_t n_out, int64_t ldw,
                                    float* y, void* stream);

/*
 * qs_set_deterministic -- process-wide choice of the split-K summation (see
 * the conventions above): on != 0 gives fixed-order, bitwise reproducible
 * sums in every entry point; 0 (the default) lets fp32 outputs be summed with
 * float atomics.  Takes effect for calls made after it returns; returns the
 * previous setting.  Not a device call: it cannot fail.
 */
int qs_set_deterministic(int on);

/*
 * qs_sparse_linear_i8t -- quantised Q-Sparse linear  [QS-TopK]
 *
 *   q = absmax int8 quantisation of x per row (see the readings above),
 *   M = top-K of |q| (ties to the lower index),
 *   acc[r,o] = sum_{j in M_r} q[r,j] * t[o,j]   (exact int32),
 *   y[r,o]   = fl32(fl32(acc[r,o]) * fl32(alpha / s_r)).
 *
 *   x          device fp32 [rows, d_in].
 *   wt_packed  device u8 [d_in, n_out/4]: ternary W^T, 2 bits per weight as
 *              two's complement (00 = 0, 01 = +1, 11 = -1); byte c/4 of row j
 *              holds columns c..c+3, column c+i in bits 2i..2i+1 (see
 *              qs_pack_ternary).
 *   alpha      the weight scale (mean |W|, see qs_ternarize).
 *   acc        device i32 [rows, n_out] or NULL.
 *   y          device fp32 [rows, n_out] or NULL.
 *   xq         device i8 [rows, d_in] or NULL: the quantised activations.
 *   xscale     device fp32 [rows] or NULL: s_r.
 *   idx        device i32 [rows, k] or NULL: the selected indices, ascending.
 *   Limits: n_out % 16 == 0; d_in <= 1<<24 (|acc| <= 128 d_in must fit int32).
 */
qs_status qs_sparse_linear_i8t(const float* x, int64_t rows, int64_t d_in, int64_t k,
                               const uint8_t* wt_packed, float alpha, int64_t n_out,
                               int32_t* acc, float* y, int8_t* xq, float* xscale, int32_t* idx,
                               void* ws, size_t ws_bytes, void* stream);

/*
 * qs_sparse_ffn -- sparse FFN: input top-K, up (and gate) projection,
 * activation, optional top-K of the intermediate, gathered down projection.
 *
 *   x        device [rows, d], dtype dt.
 *   act == QS_ACT_RELU2   [QS-TopK], [TS-Eq3-4]
 *       dt QS_F32 or QS_BF16 (weights in the same dtype);
 *       u = (x (.) M1) . W_up^T with M1 = top-k_in of |x|;  h = relu(u)^2;
 *       M2 = top-k_mid of |h| (k_mid < 0: M2 = all of h);
 *       y = (h (.) M2) . W_down^T.
 *       w_gate = NULL; w_up = W_up^T [d, ffn]; w_down_t = W_down^T [ffn, d];
 *       b_gate, b_up must be NULL.
 *   act == QS_ACT_RELU2_GLU   [QS-TopK], [TS-Eq3-4]
 *       The gated reading of the squared ReLU (the article's FFN sentence
 *       names a Hadamard product): dt QS_F32 or QS_BF16 (weights in the same
 *       dtype); xm = x (.) M1, M1 = top-k_in of |x|, feeds both projections;
 *       g = xm . W_gate^T; u = xm . W_up^T; h = fl32(relu(g)^2) * u (fp32);
 *       M2 = top-k_mid of |h| (h can be negative; k_mid < 0: M2 = all of h);
 *       y = (h (.) M2) . W_down^T.
 *       w_gate = W_gate^T [d, ffn]; w_up = W_up^T [d, ffn]; w_down_t =
 *       W_down^T [ffn, d]; b_gate, b_up must be NULL.
 *   act == QS_ACT_DRELU   [TS-Eq2], [TS-Fig]
 *       dt QS_BF16 only;  xm = x (.) M1 (k_in == d: no selection);
 *       g = xm . W_gate^T + b_gate; u = xm . W_up^T + b_up;
 *       h = relu(g) * relu(u); rows of W_up are read only for neurons with
 *       g > 0 for some token of the batch;
 *       M2 = top-k_mid of |h|, or (k_mid < 0) the nonzero entries of h;
 *       y = (h (.) M2) . W_down^T, reading only the rows of W_down^T that
 *       some token selects.
 *       w_gate = W_gate [ffn, d]; w_up = W_up [ffn, d]; w_down_t = W_down^T
 *       [ffn, d]; b_gate, b_up: device fp32 [ffn] or NULL (= 0).
 *   y        device [rows, d], dtype yt (QS_F32 or QS_BF16).
 *   h        device fp32 [rows, ffn] or NULL: the intermediate before M2.
 *   mid_idx  device i32 [rows, ffn] or NULL: for each row the entries of M2,
 *            ascending, in the first mid_cnt[r] slots (the rest is untouched).
 *   mid_cnt  device i32 [rows] or NULL.
 *   Arithmetic: exact products, fp32 accumulation, fp32 intermediate.
 *   Alignment: d % 8 == 0 and ffn % 8 == 0.
 */
qs_status qs_sparse_ffn(const void* x, qs_dtype dt, int64_t rows, int64_t d, int64_t ffn,
                        qs_act act, int64_t k_in, int64_t k_mid,
                        const void* w_gate, const void* w_up, const void* w_down_t,
                        const float* b_gate, const float* b_up,
                        void* y, qs_dtype yt, float* h, int32_t* mid_idx, int32_t* mid_cnt,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * qs_sparse_ffn_pitched -- qs_sparse_ffn with the row pitches of W_up^T (and
 * W_gate^T) and W_down^T given  [QS-TopK], [TS-Eq3-4].
 *
 *   ld_up    elements from one row of w_up (and of w_gate) to the next, at
 *            least the row length (ffn for W_up^T, d for dReLU's W_up), a
 *            multiple of 8.  dReLU needs the natural pitch d (its gate/up
 *            kernels read whole rows); QS_ERR_UNSUPPORTED otherwise.
 *   ld_down  elements from one row of W_down^T to the next, >= d, a multiple
 *            of 8 (every kind).
 *   The natural pitches give qs_sparse_ffn; the others work at every batch
 *   size, each padded matrix smaller than 1 GiB.  Padding columns are never
 *   read.  Rows padded by 64 bf16 keep each column tile's lines off a single
 *   subset of the memory channels (see qs_sparse_linear_pitched).
 */
qs_status qs_sparse_ffn_pitched(const void* x, qs_dtype dt, int64_t rows, int64_t d, int64_t ffn,
                                qs_act act, int64_t k_in, int64_t k_mid, const void* w_gate,
                                const void* w_up, int64_t ld_up, const void* w_down_t,
                                int64_t ld_down, const float* b_gate, const float* b_up,
                                void* y, qs_dtype yt, float* h, int32_t* mid_idx,
                                int32_t* mid_cnt, void* ws, size_t ws_bytes, void* stream);

/*
 * qs_sparse_ffn_static -- qs_sparse_ffn without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.
 *
 *   Arguments, arithmetic, outputs and errors as qs_sparse_ffn.  The
 *   workspace is a file-scope device array of QS_STATIC_SCRATCH_BYTES (32
 *   MiB) in the library, one per GPU, held from the first call on that GPU
 *   until the process ends; the call itself allocates nothing.  A shape
 *   whose qs_sparse_ffn workspace (qs_workspace_bytes) exceeds that size is
 *   rejected with QS_ERR_UNSUPPORTED before anything is enqueued (every
 *   Llama-7B / Mistral-7B shaped FFN of up to 16 tokens fits).
 *   The stream must belong to the current device.  The array keeps the last
 *   call's contents and needs no clearing (every call clears what it uses).
 *   Calls that may overlap on one GPU (other streams, other host threads)
 *   race on the shared array: serialise them.
 */
#define QS_STATIC_SCRATCH_BYTES (32u << 20)
qs_status qs_sparse_ffn_static(const void* x, qs_dtype dt, int64_t rows, int64_t d, int64_t ffn,
                               qs_act act, int64_t k_in, int64_t k_mid,
                               const void* w_gate, const void* w_up, const void* w_down_t,
                               const float* b_gate, const float* b_up,
                               void* y, qs_dtype yt, float* h, int32_t* mid_idx,
                               int32_t* mid_cnt, void* stream);

/*
 * qs_sparse_linear_backward -- gradients of Y = (X (.) M) . W^T for a given
 * dL/dY, the top-K passed by the straight-through estimator  [QS-STE],
 * [QS-TopK]:
 *
 *   dX = dY . W             not masked: the gradient reaching X (.) M is
 *                           copied to X, entries outside the selection too;
 *   dW = dY^T . (X (.) M)   M recomputed from x with the same k (the same
 *                           selection as the forward); feature columns that
 *                           no row selected get exact zeros.
 *
 *   x       device bf16 [rows, d_in]: the forward's input.
 *   k       0 <= k <= d_in, the forward's K.
 *   w       device bf16 weights in layout w_layout (QS_LAYOUT_WT: W^T
 *           [d_in, n_out]; QS_LAYOUT_W: W [n_out, d_in]); may be NULL when
 *           dx is NULL.
 *   dy      device bf16 [rows, n_out].
 *   dx      device [rows, d_in], dtype dxt (QS_F32 or QS_BF16), or NULL.
 *   dw      device, the layout of w (W^T [d_in, n_out] or W [n_out, d_in]),
 *           dtype dwt (QS_F32 or QS_BF16), or NULL; overwritten (rows == 0
 *           writes zeros).
 *   Arithmetic: bf16 products exact in fp32, fp32 accumulation on matrix
 *   cores (v_mfma_f32_32x32x16_bf16), bf16 outputs rounded to nearest-even.
 *   Workspace: qs_workspace_bytes(QS_OP_SPARSE_LINEAR_BACKWARD, rows, d_in,
 *   n_out) (X (.) M in bf16); needed only when dw is given.
 *   Limits: d_in % 8 == 0, n_out % 8 == 0, each operand < 2^30 elements.
 */
qs_status qs_sparse_linear_backward(const void* x, qs_dtype xt, int64_t rows, int64_t d_in,
                                    int64_t k, const void* w, qs_dtype wt_t, qs_layout w_layout,
                                    int64_t n_out, const void* dy, qs_dtype dyt, void* dx,
                                    qs_dtype dxt, void* dw, qs_dtype dwt, void* ws,
                                    size_t ws_bytes, void* stream);

/*
 * qs_block_sparse_linear -- Block Q-Sparse linear Y = (X (.) M) . W^T with M
 * the 2:4 block pattern  [QS-Block], [QS-TopK]
 *
 *   Reading (the pages give no rule): the top-K of [QS-TopK] taken inside
 *   every contiguous block of 4 features of a token, K = 2 per block, ties to
 *   the lower index (bf16 key = bits & 0x7FFF, as qs_topk_mask).  This is the
 *   pattern the structured-sparse matrix cores take, so the product runs on
 *   v_smfmac_f32_32x32x32_bf16 over the kept half of X.
 *
 *   x       device bf16 [rows, d_in].
 *   w       device bf16 W [n_out, d_in] (nn.Linear layout).
 *   y       device [rows, n_out], dtype yt (QS_F32 or QS_BF16, RNE).
 *   mask    device u8 [rows, d_in] or NULL: 1 at the kept entries.
 *   Arithmetic: bf16 products exact in fp32, fp32 accumulation.
 *   Workspace: qs_workspace_bytes(QS_OP_BLOCK_SPARSE_LINEAR, rows, d_in,
 *   n_out) (the packed operand: kept values and 2-bit positions).
 *   Limits: d_in % 32 == 0, n_out % 8 == 0, x and w < 2^30 elements.
 */
qs_status qs_block_sparse_linear(const void* x, qs_dtype xt, int64_t rows, int64_t d_in,
                                 const void* w, qs_dtype wt_t, int64_t n_out, void* y,
                                 qs_dtype yt, uint8_t* mask, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * qs_sparse_moe_ffn -- mixture-of-experts dReLU FFN for decode  [TS-Fig],
 * [TS-Eq2]
 *
 *   Routing (a reading: the pages give no rule): logits = x . W_router^T
 *   (fp32 sums), the top_k logits of each token (ties to the lower expert
 *   index), weights = softmax over the kept logits.  Each chosen expert e
 *   runs the dReLU FFN of qs_sparse_ffn (QS_ACT_DRELU, k_mid < 0): the gate
 *   row of every neuron, the up row only where the gate is positive, the down
 *   projection gathering only the rows of W_down^T where h != 0.  Then
 *   y = sum over the chosen experts of weight_e * y_e (in ascending expert
 *   order).
 *
 *   x          device bf16 [rows, d]; d % 8 == 0, d <= 8192.
 *   w_router   device bf16 [n_experts, d]; 1 <= top_k <= n_experts <= 64.
 *   w_gate     device bf16 [n_experts, ffn, d] (neuron-major per expert).
 *   w_up       device bf16 [n_experts, ffn, d].
 *   w_down_t   device bf16 [n_experts, ffn, d] (W_down^T of each expert).
 *   b_gate, b_up  device fp32 [n_experts, ffn] or NULL.
 *   y          device [rows, d], dtype yt (QS_F32 or QS_BF16).
 *   router_logits  device fp32 [rows, n_experts] or NULL.
 *   experts    device i32 [rows, top_k] or NULL: the chosen experts, ascending.
 *   expert_weights device fp32 [rows, top_k] or NULL: their weights.
 *   h          device fp32 [rows, top_k, ffn] or NULL: each pair's dReLU output.
 *   Arithmetic: fp32 sums of exact bf16 products; fp32 h; ffn % 8 == 0; an
 *   expert matrix < 1 GiB.
 *   Workspace: qs_workspace_bytes(QS_OP_SPARSE_MOE_FFN, rows * top_k, d, ffn).
 */
qs_status qs_sparse_moe_ffn(const void* x, qs_dtype dt, int64_t rows, int64_t d, int64_t ffn,
                            int64_t n_experts, int64_t top_k, const void* w_router,
                            const void* w_gate, const void* w_up, const void* w_down_t,
                            const float* b_gate, const float* b_up, void* y, qs_dtype yt,
                            float* router_logits, int32_t* experts, float* expert_weights,
                            float* h, void* ws, size_t ws_bytes, void* stream);

/*
 * qs_workspace_bytes -- device workspace needed by `op` at this shape.
 *   d = d_in (or the FFN model dimension), n = n_out (or ffn).  The size does
 *   not depend on K, dtypes or layout.  *bytes receives the size (0 for ops
 *   that need none).  Host-only; enqueues nothing.
 */
qs_status qs_workspace_bytes(qs_op op, int64_t rows, int64_t d, int64_t n, size_t* bytes);

/*
 * qs_ternarize -- offline ternary quantisation of a weight matrix  [QS-TopK]
 *   w_host   host fp32 [n_out, d_in] (nn.Linear layout).
 *   t_host   host i8 [n_out, d_in] receives t in {-1, 0, +1}.
 *   alpha    host fp32 receives mean |W|: the exact sum of |w| rounded to
 *            binary64, divided by n_out*d_in in binary64, rounded to binary32.
 *   t = clamp(rint(fl32(w / fl32(alpha + 1e-5))), -1, 1).  Host-only.
 */
qs_status qs_ternarize(const float* w_host, int64_t n_out, int64_t d_in, int8_t* t_host,
                       float* alpha);

/*
 * qs_pack_ternary -- pack t [n_out, d_in] (host, values in {-1,0,1}) into the
 * feature-major 2-bit layout that qs_sparse_linear_i8t reads (host u8
 * [d_in, n_out/4]).  n_out % 4 == 0.  Host-only.
 */
qs_status qs_pack_ternary(const int8_t* t_host, int64_t n_out, int64_t d_in, uint8_t* packed_host);

/* Text of the last error on the calling thread ("" if none); valid until the
 * next qs_* call on this thread. */
const char* qs_last_error(void);

/* Library version string. */
const char* qs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QS_H */
