// Internal declarations shared by the HIP translation units of libqs.so.
// Not part of the public ABI (that is include/qs.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qs {

// ---------------------------------------------------------------- element kinds
enum KeyKind : int {
    KEY_F32 = 0,   // fp32 input, key = bits & 0x7FFFFFFF
    KEY_BF16 = 1,  // bf16 input, key = bits & 0x7FFF
    KEY_I8 = 2,    // int8 input, key = |q|
    KEY_Q8 = 3     // fp32 input quantised in-kernel to int8 (absmax), key = |q|
};

// What the selection kernel writes as the "sparsified activation" X (.) M.
enum XsKind : int {
    XS_NONE = 0,
    XS_F32 = 1,    // float [rows, d]
    XS_BF16 = 2,   // bf16 bits [rows, d]
    XS_I8 = 3      // int8 [rows, d] (masked q)
};

struct TopkArgs {
    const void* x;        // [rows, d]
    int64_t d;
    int64_t k;
    uint8_t* mask;        // [rows, d] or null
    int32_t* idx;         // [rows, idx_stride] or null (first k entries of each row)
    int64_t idx_stride;   // row stride of idx (k unless the caller says otherwise)
    int32_t* count;       // [rows] or null: receives k
    uint32_t* tau;        // [rows] or null
    int32_t* cutoff;      // [rows] or null
    void* xs;             // [rows, d] or null (kind given by xs_kind)
    int8_t* xq;           // KEY_Q8 only: [rows, d] or null
    float* xscale;        // KEY_Q8 only: [rows] or null
    int32_t* zero_ptr;    // block 0 clears zero_ptr[0..n_zero) (split-K counters)
    int n_zero;
    int32_t* zero_rows;   // or null: the workgroup of row r clears
    int64_t zero_row_len; //   zero_rows[r * zero_row_len ..) (zero_row_len % 4 == 0)
    int32_t* zero_rows2;  // or null: cleared the same way (same row length)
    // KEY_F32 only: the row is first mapped elementwise (XF_RELU2: relu(x)^2;
    // XF_RELU2_GLU: relu(x2)^2 * x, x2 of the shape of x), and the mapped
    // values are selected, written to xs and, if h_out is set, to h_out
    // (which may be x itself).  Only rows that the vector kernel takes
    // (topk_xform_supported).
    int xform;
    const float* x2;
    float* h_out;
    // XS_F32 kinds of the vector kernel only (or null): the selected values
    // are also written as the packed A-operand records of the 16-token MFMA
    // gather (bf16 hi parts, and with frag_lo the bf16 lo parts of the
    // remainder; the layout of bfrag_kernel, without its row masks): row r is
    // token r % 16 of token tile r / 16, frag_groups = ceil(d / 32).
    void* frag;
    int64_t frag_groups;
    int frag_lo;
    // 1: any cutoff that gives the same selection will do (a descriptor for
    // a later launch, not an output): when every key equal to tau is
    // selected, cutoff = 0x7FFFFFFF and the tie ranking is skipped.
    int cutoff_any;
};
enum Xform : int { XF_NONE = 0, XF_RELU2 = 1, XF_RELU2_GLU = 2 };
bool topk_xform_supported(int64_t d);

// One workgroup per row.  Returns a HIP error code (hipSuccess = 0).
hipError_t launch_topk(int key_kind, int xs_kind, int64_t rows, const TopkArgs& a,
                       hipStream_t stream);

// ---------------------------------------------------------------- gather GEMV
// The gather kernels address weights through 32-bit buffer offsets.
constexpr int64_t kMaxGatherWeightBytes = int64_t(1) << 30;
enum Epilogue : int { EPI_STORE = 0, EPI_RELU2 = 1, EPI_RELU2_GLU = 2 };

// Launch plan of the gather GEMV: deterministic function of the shape only.
struct GemvPlan {
    int lpr;          // lanes per weight-row segment
    int ept;          // elements per lane (16 bytes of weights)
    int ct;           // columns per tile
    int n_tiles;      // column tiles
    int bt;           // tokens per tile
    int n_tok_tiles;
    int cand;         // candidate input rows per split
    int nsplit;
    size_t partial_floats;  // nsplit * rows * n_out (0 if nsplit == 1)
    size_t prep_bytes;      // compacted-row records of the bf16 MFMA kernel (0 otherwise)
    size_t scratch_floats;  // workspace behind GemvArgs::partial: partials, then prep records
    int n_counters;         // n_tiles * n_tok_tiles
};
// max_bt caps the tokens per tile (1: every row its own tile, e.g. when rows
// use different weight matrices, see GemvArgs::row_expert).
// target_wg > 0: the workgroup count the split-K plan aims for (else the
// default; the plan is still a function of its arguments only).
GemvPlan plan_gemv(int64_t rows, int64_t d_in, int64_t n_out, int w_is_bf16, int max_bt = 16,
                   int64_t target_wg = 0);

struct GemvArgs {
    const float* xs;       // [rows, d_in] fp32, zero where not selected
    int64_t rows, d_in, n_out;
    const void* w;         // W^T [d_in, n_out], fp32 or bf16
    float* partial;        // [scratch_floats]: [nsplit, rows, n_out] partials, prep records
    int32_t* counters;     // [n_counters], zero on entry, left zero on exit
    void* y;               // [rows, n_out]
    int y_bf16;            // output dtype
    int epilogue;          // EPI_STORE, EPI_RELU2 (y is fp32 h) or EPI_RELU2_GLU (y is fp32 h)
    const float* gate;     // EPI_RELU2_GLU: fp32 gate projection [rows, n_out]
    int xs_bf16;           // 1: every xs value is a bf16 number (from bf16 activations)
    const int32_t* row_expert;  // null, or (one token per tile) row r reads the
    int64_t expert_bytes;       //   matrix at w + row_expert[r] * expert_bytes
    // Gated pair (launch_gemv_dual): w2 = W_gate^T of the same shape as w, read
    // at the same selected rows; y = relu(xs . w2)^2 * (xs . w), fp32.  Its
    // split partials go to partial2 ([nsplit, rows, n_out]).
    const void* w2;
    float* partial2;
    // 16-token bf16 tiles: 1 = the packed coefficient records and row masks
    // behind `partial` were written by a previous gather over the same xs
    // (and plan), so the packing launch is skipped; 2 = the records (no
    // masks) were written by the selection launch (xs is not read).
    int frag_ready;
    // 1: y is fp32 and already holds the values to add to; every workgroup
    // adds its partial tile into y (and the dual gather its gate tile into
    // y2) with float atomics, so there is no split handoff and no epilogue
    // (epilogue must be EPI_STORE).  The sum order depends on timing.
    int accumulate;
    float* y2;
    // Accumulate form with one-token tiles only (or null): row r's sums are
    // scaled by row_scale[r] and added into output row row_out[r] (the MoE
    // pairs' routing weights and tokens).
    const float* row_scale;
    const int32_t* row_out;
    // Or null: xs is not sparsified yet; row r's selected entries are those
    // with key > tau_r, or key == tau_r and index < cutoff_r (key = the
    // magnitude bits), with tau = sel_desc[0 .. rows) and cutoff =
    // sel_desc[rows .. 2 rows) (the top-k descriptor of launch_topk), and
    // only they are gathered.
    const uint32_t* sel_desc;
    int64_t sel_k;         // launch_gather_sel: the top-k of h that the workgroups find
    int64_t w_ld;          // elements from one row of w (and w2) to the next (0: n_out)
};
hipError_t launch_gemv(const GemvPlan& p, int w_is_bf16, const GemvArgs& a, hipStream_t stream);
// Both projections of the gated squared ReLU in one gather (tiles of at most
// four tokens, or 16-token tiles of bf16 weights); returns hipErrorNotSupported
// for other plans.  partial2 must not overlap the scratch behind partial.
bool gemv_dual_supported(const GemvPlan& p, int w_is_bf16);
hipError_t launch_gemv_dual(const GemvPlan& p, int w_is_bf16, const GemvArgs& a, hipStream_t stream);
// Plans whose kernel has the accumulate form (all but fp32 16-token tiles).
bool gemv_accumulate_supported(const GemvPlan& p, int w_is_bf16);
// Plans (bf16 weights in 16-token tiles of at least 8 tokens) whose gather
// reads the coefficients best as packed MFMA records written by the selection
// launch (TopkArgs::frag at gemv_records(), frag_ready = 2 here; launch_gemv
// only, not the dual gather).
bool gemv_takes_records(const GemvPlan& p, int w_is_bf16, int64_t rows);
void* gemv_records(const GemvPlan& p, float* partial, int64_t d_in, int64_t* groups);

// ---------------------------------------------------------------- small-batch FFN up projection
// The top-k of each bf16 x row (selected inside every workgroup), then u =
// (x (.) M) . W_up^T (and with w2 the gate's g) over every row that some
// token of the tile selects, no K split (whole 64-column tiles per
// workgroup), then h = relu(u)^2 (relu(g)^2 * u).
struct UpColsArgs {
    const float* xs;         // fp32 [rows, d] sparsified x (0 off the selection), or null:
    const uint16_t* x;       //   bf16 [rows, d], of which every workgroup selects
    int64_t rows, d, ffn, k; //   the top-k of each row itself
    float* zero;             // or null: cleared by the launch (n_zero % 4 == 0)
    int64_t n_zero;
    int32_t* zero_i;         // or null: int32 counters cleared by workgroup 0
    int n_zero_i;
    const uint16_t* w;       // bf16 W_up^T [d, ffn]
    const uint16_t* w2;      // bf16 W_gate^T [d, ffn] (gated form) or null
    float* h;                // fp32 [rows, ffn], or null with hb:
    uint16_t* hb;            //   bf16 [rows, ffn] (nearest-even from the fp32 value)
    float* h2;               // or null: a second copy of h
    int linear;              // 1: h = u, the plain sparse linear (w2 null)
    int64_t w_ld;            // elements from one row of w (and w2) to the next (0: ffn)
};
constexpr int64_t kUpColsMaxD = 16 * 512;
constexpr int64_t kUpColsMaxFfn = 32 * 512;
bool up_cols_supported(int64_t rows, int64_t d, int64_t ffn);
hipError_t launch_up_cols(const UpColsArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- ternary x int8 gather
struct I8tPlan {
    int mfma;        // 1: the int8 matrix-core kernel (token batches); cand = features per split
    int ct, n_tiles, bt, n_tok_tiles, cand, nsplit;
    size_t partial_ints;
    int n_counters;
};
I8tPlan plan_i8t(int64_t rows, int64_t d_in, int64_t n_out);

struct I8tArgs {
    const int8_t* qs;        // [rows, d_in] masked q
    const float* xscale;     // [rows]
    int64_t rows, d_in, n_out;
    const uint8_t* wt;       // [d_in, n_out/4] packed
    float alpha;
    int32_t* partial;        // [nsplit, rows, n_out]
    int32_t* counters;
    int32_t* acc;            // [rows, n_out] or null
    float* y;                // [rows, n_out] or null
    int32_t* acc_sum;        // matrix-core kernel with splits: [rows, n_out], zero on
                             //   entry; the splits add into it (acc itself, or scratch)
};
hipError_t launch_i8t(const I8tPlan& p, const I8tArgs& a, hipStream_t stream);

// The whole quantised linear for 1-4 tokens in one launch: every workgroup
// quantises x, selects the top-k of |q| and sums its output columns over the
// selected rows in exact int32 (no workspace).
struct I8fArgs {
    const float* x;          // fp32 [rows, d_in]
    int64_t rows, d_in, n_out, k;
    const uint8_t* wt;       // [d_in, n_out/4] packed
    float alpha;
    int32_t* acc;            // [rows, n_out] or null
    float* y;                // [rows, n_out] or null
    int8_t* xq;              // [rows, d_in] or null
    float* xscale;           // [rows] or null
    int32_t* idx;            // [rows, k] or null
};
bool i8t_fused_supported(int64_t rows, int64_t d_in, int64_t n_out);
hipError_t launch_i8t_fused(const I8fArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- masked MFMA GEMM
struct MfmaArgs {
    const uint16_t* x;       // bf16 [M, K]: X (.) M
    const uint16_t* w;       // bf16 W [N, K]
    int64_t m, n, k;
    void* y;                 // [M, N]
    int y_bf16;
};
hipError_t launch_masked_gemm(const MfmaArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- bf16 GEMM, either operand layout
// C[M, N] = sum_k A(m, k) B(n, k), fp32 accumulation.  An operand is
// k-contiguous ([M, K] with row pitch lda, K % 8 == 0) or k-major ([K, M]
// with row pitch lda, M % 8 == 0).  Every operand must be < 2^30 elements.
struct GemmArgs {
    const uint16_t* a;
    const uint16_t* b;
    int a_kmajor, b_kmajor;  // (1, 0) is not supported
    int64_t m, n, k, lda, ldb;
    void* c;                 // [M, N] row-major, fp32 or bf16 (RNE)
    int c_bf16;
};
hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream);

// ---------------------------------------------------------------- Block Q-Sparse (2:4)
struct BlockSparseArgs {
    const uint16_t* x;       // bf16 [rows, d], d % 32 == 0
    int64_t rows, d, n;
    const uint16_t* w;       // bf16 W [n, d] (nn.Linear layout), n % 8 == 0
    void* y;                 // [rows, n] fp32 or bf16
    int y_bf16;
    uint8_t* mask;           // [rows, d] or null
    void* ws;                // nm24_packed_bytes(rows, d) bytes: the packed 2:4 operand
};
size_t nm24_packed_bytes(int64_t rows, int64_t d);
hipError_t launch_block_sparse_linear(const BlockSparseArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- dReLU gate/up
struct DreluArgs {
    const uint16_t* x;       // bf16 [rows, d] (already masked if k_in < d)
    int64_t rows, d, ffn;
    const uint16_t* wg;      // [ffn, d]
    const uint16_t* wu;      // [ffn, d]
    const float* bg;         // [ffn] or null
    const float* bu;         // [ffn] or null
    float* h;                // [rows, ffn] fp32
    int32_t* zero_ptr;       // block 0 clears zero_ptr[0..n_zero) (split-K counters)
    int n_zero;
    float* zero_out;         // or null: the launch's workgroups clear zero_out[0..n_zero_out)
    int64_t n_zero_out;      //   (n_zero_out % 4 == 0): the output the down gather adds into
    // Mixture of experts (null for a plain FFN; one-token kernel only): launch
    // row r is the pair (token pair_token[r], expert pair_expert[r]); the
    // expert's matrices start at wg / wu + expert * ffn * d, its biases at
    // bg / bu + expert * ffn, and h row r is the pair's.
    const int32_t* pair_token;
    const int32_t* pair_expert;
    int64_t pairs;
    // Pairs grouped by expert (launch_drelu_grouped): expert e owns the
    // grp_count[e] pair indices at grp_pairs[e * pairs ..], whose tokens are
    // at grp_tok[e * pairs ..].
    const int32_t* grp_count;
    const int32_t* grp_pairs;
    const int32_t* grp_tok;
    int n_experts;
};
hipError_t launch_drelu_gate_up(const DreluArgs& a, hipStream_t stream);
// MoE gate/up with the pairs of each expert processed together: every
// expert's gate rows are read once per chunk of its tokens.
hipError_t launch_drelu_grouped(const DreluArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- MoE routing and combine
struct MoeRouteArgs {
    const uint16_t* x;       // bf16 [rows, d]
    const uint16_t* wr;      // bf16 router [n_experts, d]
    int64_t rows, d;
    int n_experts, top_k;    // n_experts <= 64
    int32_t* pair_token;     // [rows * top_k]
    int32_t* pair_expert;    // [rows * top_k], ascending within a token
    float* pair_weight;      // [rows * top_k]
    float* logits;           // [rows, n_experts] or null
    int32_t* out_experts;    // [rows, top_k] or null: copy of pair_expert
    float* out_weights;      // [rows, top_k] or null: copy of pair_weight
};
hipError_t launch_moe_route(const MoeRouteArgs& a, hipStream_t stream);
// Lists the pairs of each expert: count[e] of them at list[e * pairs ..], their
// tokens at tok[e * pairs ..] (the order inside an expert is not fixed, and
// nothing computed from it depends on it).
hipError_t launch_moe_group(const int32_t* pair_expert, const int32_t* pair_token, int64_t pairs,
                            int n_experts, int32_t* count, int32_t* list, int32_t* tok,
                            hipStream_t stream);
// y[t] = sum over j < top_k of pair_weight[t * top_k + j] * ypair[t * top_k + j]
// (pair_weight null: weight 1, so top_k == 1 just rounds ypair into y).
hipError_t launch_moe_combine(const float* ypair, const float* pair_weight, int64_t rows,
                              int top_k, int64_t d, void* y, int y_bf16, hipStream_t stream);

// Nonzero compaction of h rows: idx[r, 0..cnt) ascending, cnt[r].
// Gather that selects the top-a.sel_k of each row of a.xs (fp32, not
// sparsified) by magnitude itself: one launch instead of a descriptor launch
// and the gather (the one-token FFN's down projection).  bf16 W^T; the
// accumulate form adds into fp32 y (any rows, one grid layer each), else
// (one row) split partials with the last split finishing (a.partial: nsplit *
// n_out floats, a.counters: n_tiles counters, zero on entry and exit).
bool gather_sel_supported(int64_t rows, int64_t d_in, int64_t n_out);
void gather_sel_plan(int64_t d_in, int64_t n_out, int* n_tiles, int* nsplit, int* cand);
hipError_t launch_gather_sel(const GemvArgs& a, hipStream_t stream);

// Top-k descriptor of each row of fp32 x [rows, d] by |x| (one workgroup per
// row, rowsel::select_desc31): tau -> desc[r], cutoff -> desc[rows + r].
// d % 4 == 0, d <= kDescMaxD.
constexpr int64_t kDescMaxD = 4 * 4096;
inline bool desc31_supported(int64_t d) { return d > 0 && d % 4 == 0 && d <= kDescMaxD; }
hipError_t launch_desc31(const float* x, int64_t rows, int64_t d, int64_t k, uint32_t* desc,
                         hipStream_t stream);

hipError_t launch_nonzero_lists(const float* h, int64_t rows, int64_t n, int32_t* idx,
                                int32_t* cnt, hipStream_t stream);

// Fill an int32 buffer with zeros (a kernel, so graph capture stays clean).
hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t stream);

}  // namespace qs
