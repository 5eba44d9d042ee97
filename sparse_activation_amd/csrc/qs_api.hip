// C ABI of libqs.so: argument validation, workspace layout and dispatch to
// the HIP kernels.  Every check runs before anything is enqueued, so a call
// that fails leaves the outputs untouched.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/qs.h"
#include "qs_error.h"
#include "qs_internal.h"

namespace {

thread_local std::string g_err;

// Process-wide: 1 = every split-K sum in a fixed order (bitwise reproducible).
std::atomic<int> g_deterministic{0};
bool deterministic() { return g_deterministic.load(std::memory_order_relaxed) != 0; }

qs_status fail(qs_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

qs_status ok() {
    g_err.clear();
    return QS_OK;
}

qs_status hip_fail(hipError_t e, const char* where) {
    return fail(QS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Whether the selection launch over rows of length d can write the 16-token
// MFMA gather's packed records (its vector kernel, whole 8-entry chunks).
bool records_ok(int64_t d) { return d % 8 == 0 && d <= 16384; }

// Points a selection launch at the packed records of the gather planned by p
// (when that gather would pack them itself) and marks the gather to read
// them.  frag_lo: the values are not all bf16 numbers.
void route_records(qs::TopkArgs& t, qs::GemvArgs& g, const qs::GemvPlan& p, int wb, int64_t rows,
                   int64_t d_in, float* partial, int frag_lo) {
    if (!qs::gemv_takes_records(p, wb, rows) || !records_ok(d_in)) return;
    t.frag = qs::gemv_records(p, partial, d_in, &t.frag_groups);
    t.frag_lo = frag_lo;
    t.xs = nullptr;   // the gather reads the records only
    g.frag_ready = 2;
}

// Bump allocator over the caller's workspace (256-byte aligned regions).
struct Carve {
    size_t off = 0;
    char* base = nullptr;
    void* take(size_t bytes) {
        void* p = base ? base + off : nullptr;
        off += (bytes + 255) & ~size_t(255);
        return p;
    }
};

// ----------------------------------------------------------------- layouts
// Each layout is computed twice: once with base == nullptr to size it, once
// with the caller's pointer to carve it.  Sizes depend on shapes only.

struct LinearWs {
    int32_t* counters;
    float* xs;          // gather path: X (.) M in fp32
    float* partial;
    uint16_t* xm;       // MFMA path: X (.) M in bf16
    size_t bytes;
};

size_t max_sz(size_t a, size_t b) { return a > b ? a : b; }

LinearWs linear_ws(char* base, int64_t rows, int64_t d_in, int64_t n_out) {
    qs::GemvPlan pb = qs::plan_gemv(rows, d_in, n_out, 1);
    qs::GemvPlan pf = qs::plan_gemv(rows, d_in, n_out, 0);
    Carve c;
    c.base = base;
    LinearWs w{};
    w.counters = (int32_t*)c.take(sizeof(int32_t) * (size_t)(pb.n_counters > pf.n_counters ? pb.n_counters : pf.n_counters));
    w.xs = (float*)c.take(sizeof(float) * (size_t)rows * d_in);
    w.partial = (float*)c.take(sizeof(float) * max_sz(pb.scratch_floats, pf.scratch_floats));
    w.xm = (uint16_t*)c.take(sizeof(uint16_t) * (size_t)rows * d_in);
    w.bytes = c.off;
    return w;
}

struct GatherWs {
    int32_t* counters;
    float* partial;
    size_t bytes;
};

// qs_gather_linear keeps its split-K counters in a fixed header at the start
// of the workspace, which the caller zeroes once and every call leaves zero.
constexpr int kGatherCounters = 4096;

GatherWs gather_ws(char* base, int64_t rows, int64_t d_in, int64_t n_out) {
    qs::GemvPlan pb = qs::plan_gemv(rows, d_in, n_out, 1);
    qs::GemvPlan pf = qs::plan_gemv(rows, d_in, n_out, 0);
    Carve c;
    c.base = base;
    GatherWs w{};
    w.counters = (int32_t*)c.take(sizeof(int32_t) * kGatherCounters);
    w.partial = (float*)c.take(sizeof(float) * max_sz(pb.scratch_floats, pf.scratch_floats));
    w.bytes = c.off;
    return w;
}

struct I8tWs {
    int32_t* counters;
    int8_t* qs;
    float* scale;
    int32_t* partial;
    size_t bytes;
};

I8tWs i8t_ws(char* base, int64_t rows, int64_t d_in, int64_t n_out) {
    qs::I8tPlan p = qs::plan_i8t(rows, d_in, n_out);
    Carve c;
    c.base = base;
    I8tWs w{};
    w.counters = (int32_t*)c.take(sizeof(int32_t) * (size_t)p.n_counters);
    w.qs = (int8_t*)c.take((size_t)rows * d_in);
    w.scale = (float*)c.take(sizeof(float) * (size_t)rows);
    w.partial = (int32_t*)c.take(sizeof(int32_t) * p.partial_ints);
    w.bytes = c.off;
    return w;
}

struct FfnWs {
    uint32_t* desc;        // relu2 kinds: top-k descriptor of h: tau [rows], then cutoff [rows]
    int32_t* ctr_up;
    int32_t* ctr_down;
    int n_ctr;             // ctr_up and ctr_down are contiguous: n_ctr ints in total
    float* xs1;            // relu2: X (.) M1 (fp32)
    uint16_t* xm;          // drelu: X (.) M1 (bf16)
    float* h;
    float* hs;
    float* gacc;           // relu2 kinds: the gate sums of the gated FFN's accumulate form
    float* partial;
    size_t partial_cap;    // floats carved for `partial`
    size_t up_ctr_cap, down_ctr_cap;
    size_t bytes;
};

// Plan of the FFN's down gather.  Without a selection on h the dReLU
// intermediate is ~90% zero, so a candidate range holds few active rows:
// fewer, longer splits (Mistral-7B dReLU FFN at one token: 35.0 us per step
// aiming at 320 workgroups against 35.6 at the default 640).
qs::GemvPlan ffn_down_plan(int64_t rows, int64_t d, int64_t ffn, int wb, bool drelu, int64_t k_mid) {
    return qs::plan_gemv(rows, ffn, d, wb, 16, drelu && k_mid < 0 ? 320 : 0);
}

FfnWs ffn_ws(char* base, int64_t rows, int64_t d, int64_t ffn, bool drelu) {
    Carve c;
    c.base = base;
    FfnWs w{};
    size_t up_ctr = 0, up_part = 0;
    if (!drelu) {
        qs::GemvPlan ub = qs::plan_gemv(rows, d, ffn, 1), uf = qs::plan_gemv(rows, d, ffn, 0);
        up_ctr = (size_t)(ub.n_counters > uf.n_counters ? ub.n_counters : uf.n_counters);
        // The gated FFN's one-pass gather keeps the gate's split partials
        // behind the up projection's.
        up_part = max_sz(ub.scratch_floats, uf.scratch_floats) + max_sz(ub.partial_floats, uf.partial_floats);
    }
    // The down gather's plan as qs_sparse_ffn makes it (ffn_down_plan), for
    // both weight dtypes and both selection forms of dReLU.
    size_t down_ctr = 0, down_part = 0;
    for (int wb = 0; wb < 2; ++wb)
        for (int sel = 0; sel < 2; ++sel) {
            const qs::GemvPlan p = ffn_down_plan(rows, d, ffn, wb, drelu, sel == 0 ? -1 : 0);
            down_ctr = max_sz(down_ctr, (size_t)p.n_counters);
            down_part = max_sz(down_part, p.scratch_floats);
        }
    w.n_ctr = (int)(up_ctr + down_ctr);
    w.ctr_up = (int32_t*)c.take(sizeof(int32_t) * (up_ctr + down_ctr));
    w.desc = drelu ? nullptr : (uint32_t*)c.take(sizeof(uint32_t) * 2 * (size_t)rows);
    w.ctr_down = w.ctr_up ? w.ctr_up + up_ctr : nullptr;
    if (!drelu) w.xs1 = (float*)c.take(sizeof(float) * (size_t)rows * d);
    else w.xm = (uint16_t*)c.take(sizeof(uint16_t) * (size_t)rows * d);
    w.h = (float*)c.take(sizeof(float) * (size_t)rows * ffn);
    w.hs = (float*)c.take(sizeof(float) * (size_t)rows * ffn);
    if (!drelu) w.gacc = (float*)c.take(sizeof(float) * (size_t)rows * ffn);
    w.partial = (float*)c.take(sizeof(float) * max_sz(up_part, down_part));
    w.partial_cap = max_sz(up_part, down_part);
    w.up_ctr_cap = up_ctr;
    w.down_ctr_cap = down_ctr;
    w.bytes = c.off;
    return w;
}

bool valid_float_dtype(qs_dtype t) { return t == QS_F32 || t == QS_BF16; }

// MoE FFN workspace for `pairs` = rows * top_k (token, expert) pairs.
struct MoeWs {
    int32_t* ctr;
    int n_ctr;
    int32_t* pair_token;
    int32_t* pair_expert;
    float* pair_weight;
    int32_t* grp_count;
    int32_t* grp_pairs;
    int32_t* grp_tok;
    float* h;
    float* ypair;
    float* partial;
    size_t bytes;
};

// Batches with more pairs than this keep one launch row per pair (the
// per-expert lists take 512 bytes per pair).
constexpr int64_t kMoeGroupMaxPairs = 8192;

MoeWs moe_ws(char* base, int64_t pairs, int64_t d, int64_t ffn) {
    qs::GemvPlan p = qs::plan_gemv(pairs, ffn, d, 1, 1);
    Carve c;
    c.base = base;
    MoeWs w{};
    w.n_ctr = p.n_counters;
    w.ctr = (int32_t*)c.take(sizeof(int32_t) * (size_t)p.n_counters);
    w.pair_token = (int32_t*)c.take(sizeof(int32_t) * (size_t)pairs);
    w.pair_expert = (int32_t*)c.take(sizeof(int32_t) * (size_t)pairs);
    w.pair_weight = (float*)c.take(sizeof(float) * (size_t)pairs);
    w.grp_count = (int32_t*)c.take(sizeof(int32_t) * 64);
    if (pairs <= kMoeGroupMaxPairs) {
        w.grp_pairs = (int32_t*)c.take(sizeof(int32_t) * 64 * (size_t)pairs);
        w.grp_tok = (int32_t*)c.take(sizeof(int32_t) * 64 * (size_t)pairs);
    }
    w.h = (float*)c.take(sizeof(float) * (size_t)pairs * ffn);
    w.ypair = (float*)c.take(sizeof(float) * (size_t)pairs * d);
    w.partial = (float*)c.take(sizeof(float) * p.scratch_floats);
    w.bytes = c.off;
    return w;
}

}  // namespace

qs_status qs::set_error(qs_status st, const char* msg) {
    g_err = msg;
    return st;
}

extern "C" {

const char* qs_last_error(void) { return g_err.c_str(); }

const char* qs_version(void) { return "qsparse-mi355x 0.1 (gfx950)"; }

qs_status qs_workspace_bytes(qs_op op, int64_t rows, int64_t d, int64_t n, size_t* bytes) {
    if (bytes == nullptr) return fail(QS_ERR_INVALID_ARG, "qs_workspace_bytes: bytes is NULL");
    if (rows < 0 || d <= 0 || n < 0) return fail(QS_ERR_INVALID_ARG, "qs_workspace_bytes: bad shape");
    switch (op) {
    case QS_OP_TOPK_MASK: *bytes = 0; break;
    case QS_OP_SPARSE_LINEAR: *bytes = linear_ws(nullptr, rows, d, n).bytes; break;
    case QS_OP_SPARSE_LINEAR_I8T: *bytes = i8t_ws(nullptr, rows, d, n).bytes; break;
    case QS_OP_SPARSE_FFN_RELU2: *bytes = ffn_ws(nullptr, rows, d, n, false).bytes; break;
    case QS_OP_SPARSE_FFN_DRELU: *bytes = ffn_ws(nullptr, rows, d, n, true).bytes; break;
    case QS_OP_SPARSE_FFN_RELU2_GLU: *bytes = ffn_ws(nullptr, rows, d, n, false).bytes; break;
    case QS_OP_GATHER_LINEAR: *bytes = gather_ws(nullptr, rows, d, n).bytes; break;
    case QS_OP_SPARSE_LINEAR_BACKWARD: *bytes = ((size_t)rows * (size_t)d * 2 + 255) & ~size_t(255); break;
    case QS_OP_BLOCK_SPARSE_LINEAR: *bytes = qs::nm24_packed_bytes(rows, d); break;
    case QS_OP_SPARSE_MOE_FFN: *bytes = moe_ws(nullptr, rows, d, n).bytes; break;
    default: return fail(QS_ERR_INVALID_ARG, "qs_workspace_bytes: unknown op %d", (int)op);
    }
    return ok();
}

qs_status qs_topk_mask(const void* x, qs_dtype xt, int64_t rows, int64_t d, int64_t k,
                       uint8_t* mask, int32_t* idx, uint32_t* tau, int32_t* cutoff,
                       float* xs, void* stream) {
    if (rows < 0 || d <= 0 || d > (int64_t(1) << 24))
        return fail(QS_ERR_INVALID_ARG, "qs_topk_mask: need rows >= 0 and 0 < d <= 2^24");
    if (k < 0 || k > d) return fail(QS_ERR_INVALID_ARG, "qs_topk_mask: need 0 <= k <= d");
    if (xt != QS_F32 && xt != QS_BF16 && xt != QS_I8)
        return fail(QS_ERR_UNSUPPORTED, "qs_topk_mask: dtype must be QS_F32, QS_BF16 or QS_I8");
    if (rows > 0x7FFFFFFF) return fail(QS_ERR_UNSUPPORTED, "qs_topk_mask: too many rows");
    if (rows == 0) return ok();
    if (x == nullptr) return fail(QS_ERR_INVALID_ARG, "qs_topk_mask: x is NULL");
    const void* ptrs[] = {x, mask, idx, tau, cutoff, xs};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(QS_ERR_UNSUPPORTED, "qs_topk_mask: pointer not 16-byte aligned");
    if (xs && xt == QS_I8) return fail(QS_ERR_UNSUPPORTED, "qs_topk_mask: xs needs QS_F32 or QS_BF16 x");
    qs::TopkArgs a{};
    a.x = x;
    a.d = d;
    a.k = k;
    a.mask = mask;
    a.idx = idx;
    a.idx_stride = k;
    a.tau = tau;
    a.cutoff = cutoff;
    a.xs = xs;
    const int kk = xt == QS_F32 ? qs::KEY_F32 : xt == QS_BF16 ? qs::KEY_BF16 : qs::KEY_I8;
    hipError_t e = qs::launch_topk(kk, xs ? qs::XS_F32 : qs::XS_NONE, rows, a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "qs_topk_mask");
    return ok();
}

qs_status qs_sparse_linear(const void* x, qs_dtype xt, int64_t rows, int64_t d_in, int64_t k,
                           const void* w, qs_dtype wt_t, qs_layout w_layout, int64_t n_out,
                           void* y, qs_dtype yt, void* ws, size_t ws_bytes, void* stream) {
    return qs_sparse_linear_pitched(x, xt, rows, d_in, k, w, w_layout == QS_LAYOUT_W ? d_in : n_out,
                                    wt_t, w_layout, n_out, y, yt, ws, ws_bytes, stream);
}

qs_status qs_sparse_linear_pitched(const void* x, qs_dtype xt, int64_t rows, int64_t d_in,
                                   int64_t k, const void* w, int64_t ldw, qs_dtype wt_t,
                                   qs_layout w_layout, int64_t n_out, void* y, qs_dtype yt,
                                   void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "qs_sparse_linear";
    if (rows < 0 || d_in <= 0 || n_out <= 0 || d_in > (int64_t(1) << 24))
        return fail(QS_ERR_INVALID_ARG, "%s: bad shape", fn);
    if (k < 0 || k > d_in) return fail(QS_ERR_INVALID_ARG, "%s: need 0 <= k <= d_in", fn);
    if (!valid_float_dtype(xt) || !valid_float_dtype(wt_t) || !valid_float_dtype(yt))
        return fail(QS_ERR_UNSUPPORTED, "%s: dtypes must be QS_F32 or QS_BF16", fn);
    if (w_layout != QS_LAYOUT_WT && w_layout != QS_LAYOUT_W)
        return fail(QS_ERR_INVALID_ARG, "%s: unknown weight layout", fn);
    if (rows > 0x7FFFFFFF) return fail(QS_ERR_UNSUPPORTED, "%s: too many rows", fn);
    // The row pitch of the weights: the natural one, or (W^T, one bf16 token
    // with bf16 weights: the single-launch path) at least n_out, a multiple of 8.
    const bool pitched = ldw != (w_layout == QS_LAYOUT_W ? d_in : n_out);
    if (pitched) {   // (the gather path reads any pitch; the dense MFMA path natural rows)
        if (w_layout != QS_LAYOUT_WT || ldw < n_out || ldw % 8 != 0)
            return fail(QS_ERR_INVALID_ARG, "%s: need ldw >= n_out, a multiple of 8, with QS_LAYOUT_WT", fn);
        if (d_in * ldw * (wt_t == QS_BF16 ? 2 : 4) >= qs::kMaxGatherWeightBytes)
            return fail(QS_ERR_UNSUPPORTED, "%s: W^T must be smaller than 1 GiB", fn);
    }
    if (w_layout == QS_LAYOUT_W) {
        if (xt != QS_BF16 || wt_t != QS_BF16)
            return fail(QS_ERR_UNSUPPORTED, "%s: QS_LAYOUT_W (MFMA path) needs bf16 x and w", fn);
        if (d_in % 8 != 0) return fail(QS_ERR_UNSUPPORTED, "%s: QS_LAYOUT_W needs d_in %% 8 == 0", fn);
    } else {
        if (n_out % (wt_t == QS_BF16 ? 8 : 4) != 0)
            return fail(QS_ERR_UNSUPPORTED, "%s: n_out must be a multiple of %d", fn,
                        wt_t == QS_BF16 ? 8 : 4);
        if (d_in * n_out * (wt_t == QS_BF16 ? 2 : 4) >= qs::kMaxGatherWeightBytes)
            return fail(QS_ERR_UNSUPPORTED, "%s: W^T must be smaller than 1 GiB", fn);
    }
    if (rows == 0) return ok();
    if (!x || !w || !y) return fail(QS_ERR_INVALID_ARG, "%s: x, w and y must be non-NULL", fn);
    if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (ws && !aligned16(ws)))
        return fail(QS_ERR_UNSUPPORTED, "%s: pointer not 16-byte aligned", fn);
    LinearWs need = linear_ws(nullptr, rows, d_in, n_out);
    if (ws == nullptr || ws_bytes < need.bytes)
        return fail(QS_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need.bytes);
    LinearWs wsp = linear_ws((char*)ws, rows, d_in, n_out);
    hipStream_t st = (hipStream_t)stream;
    const int kk = xt == QS_F32 ? qs::KEY_F32 : qs::KEY_BF16;
    hipError_t e;
    if (w_layout == QS_LAYOUT_W) {
        // Top-K writes X (.) M in bf16; the dense MFMA GEMM then reads it.
        qs::TopkArgs t{};
        t.x = x; t.d = d_in; t.k = k; t.idx_stride = k;
        t.xs = wsp.xm;
        e = qs::launch_topk(kk, qs::XS_BF16, rows, t, st);
        if (e != hipSuccess) return hip_fail(e, fn);
        qs::MfmaArgs m{};
        m.x = wsp.xm;
        m.w = (const uint16_t*)w; m.m = rows; m.n = n_out; m.k = d_in;
        m.y = y; m.y_bf16 = yt == QS_BF16;
        e = qs::launch_masked_gemm(m, st);
        if (e != hipSuccess) return hip_fail(e, fn);
        return ok();
    }
    const int wb = wt_t == QS_BF16;
    if (rows == 1 && xt == QS_BF16 && wb && qs::up_cols_supported(rows, d_in, n_out)) {
        // One bf16 token: a single launch whose workgroups each select the
        // top-k of x and compute whole 64-column tiles of y over the
        // selected rows (fixed-order sums, no K split).
        qs::UpColsArgs u{};
        u.x = (const uint16_t*)x; u.rows = rows; u.d = d_in; u.ffn = n_out; u.k = k;
        u.w = (const uint16_t*)w; u.linear = 1; u.w_ld = ldw;
        if (yt == QS_BF16) u.hb = (uint16_t*)y;
        else u.h = (float*)y;
        e = qs::launch_up_cols(u, st);
        if (e != hipSuccess) return hip_fail(e, fn);
        return ok();
    }
    qs::GemvPlan plan = qs::plan_gemv(rows, d_in, n_out, wb);
    // fp32 y: the selection launch clears y and the gather's workgroups add
    // into it (no split handoff), unless fixed-order sums are asked for.
    const bool acc = !deterministic() && yt == QS_F32 && qs::gemv_accumulate_supported(plan, wb);
    qs::TopkArgs t{};
    t.x = x; t.d = d_in; t.k = k; t.idx_stride = k;
    t.xs = wsp.xs;
    t.zero_ptr = wsp.counters; t.n_zero = plan.n_counters;
    if (acc) { t.zero_rows = (int32_t*)y; t.zero_row_len = n_out; }
    qs::GemvArgs g{};
    g.xs = wsp.xs; g.rows = rows; g.d_in = d_in; g.n_out = n_out; g.w = w; g.w_ld = ldw;
    g.partial = wsp.partial; g.counters = wsp.counters; g.y = y; g.y_bf16 = yt == QS_BF16;
    g.epilogue = qs::EPI_STORE;
    g.accumulate = acc ? 1 : 0;
    g.xs_bf16 = xt == QS_BF16;
    route_records(t, g, plan, wb, rows, d_in, wsp.partial, xt != QS_BF16);
    e = qs::launch_topk(kk, qs::XS_F32, rows, t, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    e = qs::launch_gemv(plan, wb, g, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

namespace {

qs_status gather_linear(const char* fn, bool accumulate, const float* xs, int64_t rows,
                        int64_t d_in, const void* wt, qs_dtype wt_t, int64_t n_out, int64_t ldw,
                        void* y, qs_dtype yt, void* ws, size_t ws_bytes, void* stream) {
    if (rows < 0 || d_in <= 0 || n_out <= 0 || d_in > (int64_t(1) << 24))
        return fail(QS_ERR_INVALID_ARG, "%s: bad shape", fn);
    if (!valid_float_dtype(wt_t) || !valid_float_dtype(yt))
        return fail(QS_ERR_UNSUPPORTED, "%s: dtypes must be QS_F32 or QS_BF16", fn);
    if (n_out % (wt_t == QS_BF16 ? 8 : 4) != 0)
        return fail(QS_ERR_UNSUPPORTED, "%s: n_out must be a multiple of %d", fn,
                    wt_t == QS_BF16 ? 8 : 4);
    if (ldw < n_out || ldw % 8 != 0)
        return fail(QS_ERR_INVALID_ARG, "%s: need ldw >= n_out, a multiple of 8", fn);
    if (d_in * ldw * (wt_t == QS_BF16 ? 2 : 4) >= qs::kMaxGatherWeightBytes)
        return fail(QS_ERR_UNSUPPORTED, "%s: W^T must be smaller than 1 GiB", fn);
    if (rows > 0x7FFFFFFF) return fail(QS_ERR_UNSUPPORTED, "%s: too many rows", fn);
    if (rows == 0) return ok();
    if (!xs || !wt || !y) return fail(QS_ERR_INVALID_ARG, "%s: xs, wt and y must be non-NULL", fn);
    if (!aligned16(xs) || !aligned16(wt) || !aligned16(y) || (ws && !aligned16(ws)))
        return fail(QS_ERR_UNSUPPORTED, "%s: pointer not 16-byte aligned", fn);
    GatherWs need = gather_ws(nullptr, rows, d_in, n_out);
    if (ws == nullptr || ws_bytes < need.bytes)
        return fail(QS_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need.bytes);
    GatherWs wsp = gather_ws((char*)ws, rows, d_in, n_out);
    hipStream_t st = (hipStream_t)stream;
    const int wb = wt_t == QS_BF16;
    qs::GemvPlan plan = qs::plan_gemv(rows, d_in, n_out, wb);
    if (plan.n_counters > kGatherCounters)
        return fail(QS_ERR_UNSUPPORTED, "%s: too many output tiles (n_out or rows too large)", fn);
    if (accumulate && !qs::gemv_accumulate_supported(plan, wb))
        return fail(QS_ERR_UNSUPPORTED, "%s: fp32 weights need at most 8 rows", fn);
    qs::GemvArgs g{};
    g.xs = xs; g.rows = rows; g.d_in = d_in; g.n_out = n_out; g.w = wt; g.w_ld = ldw;
    g.partial = wsp.partial; g.counters = wsp.counters; g.y = y; g.y_bf16 = yt == QS_BF16;
    g.epilogue = qs::EPI_STORE;
    g.accumulate = accumulate ? 1 : 0;
    hipError_t e = qs::launch_gemv(plan, wb, g, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

}  // namespace

qs_status qs_gather_linear(const float* xs, int64_t rows, int64_t d_in, const void* wt,
                           qs_dtype wt_t, int64_t n_out, int64_t ldw, void* y, qs_dtype yt,
                           void* ws, size_t ws_bytes, void* stream) {
    return gather_linear("qs_gather_linear", false, xs, rows, d_in, wt, wt_t, n_out, ldw, y, yt,
                         ws, ws_bytes, stream);
}

qs_status qs_gather_linear_acc(const float* xs, int64_t rows, int64_t d_in, const void* wt,
                               qs_dtype wt_t, int64_t n_out, int64_t ldw, float* y, void* ws,
                               size_t ws_bytes, void* stream) {
    return gather_linear("qs_gather_linear_acc", true, xs, rows, d_in, wt, wt_t, n_out, ldw, y,
                         QS_F32, ws, ws_bytes, stream);
}

qs_status qs_topk_gather_linear_acc(const float* x, int64_t rows, int64_t d_in, int64_t k,
                                    const void* wt, qs_dtype wt_t, int64_t n_out, int64_t ldw,
                                    float* y, void* stream) {
    const char* fn = "qs_topk_gather_linear_acc";
    if (rows < 0 || d_in <= 0 || n_out <= 0) return fail(QS_ERR_INVALID_ARG, "%s: bad shape", fn);
    if (k < 0 || k > d_in) return fail(QS_ERR_INVALID_ARG, "%s: need 0 <= k <= d_in", fn);
    if (wt_t != QS_BF16) return fail(QS_ERR_UNSUPPORTED, "%s: W^T must be bf16", fn);
    if (rows > 65535 || !qs::gather_sel_supported(rows == 0 ? 1 : rows, d_in, n_out))
        return fail(QS_ERR_UNSUPPORTED,
                    "%s: needs d_in %% 4 == 0, d_in <= 16384, n_out %% 8 == 0, rows <= 65535", fn);
    if (ldw < n_out || ldw % 8 != 0)
        return fail(QS_ERR_INVALID_ARG, "%s: need ldw >= n_out, a multiple of 8", fn);
    if (d_in * ldw * 2 >= qs::kMaxGatherWeightBytes)
        return fail(QS_ERR_UNSUPPORTED, "%s: W^T must be smaller than 1 GiB", fn);
    if (rows == 0) return ok();
    if (!x || !wt || !y) return fail(QS_ERR_INVALID_ARG, "%s: x, wt and y must be non-NULL", fn);
    if (!aligned16(x) || !aligned16(wt) || !aligned16(y))
        return fail(QS_ERR_UNSUPPORTED, "%s: pointer not 16-byte aligned", fn);
    qs::GemvArgs g{};
    g.xs = x; g.rows = rows; g.d_in = d_in; g.n_out = n_out; g.w = wt; g.y = y;
    g.epilogue = qs::EPI_STORE;
    g.accumulate = 1;
    g.sel_k = k;
    g.w_ld = ldw;
    hipError_t e = qs::launch_gather_sel(g, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

int qs_set_deterministic(int on) {
    return g_deterministic.exchange(on ? 1 : 0, std::memory_order_relaxed);
}

qs_status qs_sparse_linear_i8t(const float* x, int64_t rows, int64_t d_in, int64_t k,
                               const uint8_t* wt_packed, float alpha, int64_t n_out,
                               int32_t* acc, float* y, int8_t* xq, float* xscale, int32_t* idx,
                               void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "qs_sparse_linear_i8t";
    if (rows < 0 || d_in <= 0 || n_out <= 0 || d_in > (int64_t(1) << 24))
        return fail(QS_ERR_INVALID_ARG, "%s: bad shape", fn);
    if (k < 0 || k > d_in) return fail(QS_ERR_INVALID_ARG, "%s: need 0 <= k <= d_in", fn);
    if (n_out % 16 != 0) return fail(QS_ERR_UNSUPPORTED, "%s: n_out must be a multiple of 16", fn);
    if (d_in * (n_out / 4) >= qs::kMaxGatherWeightBytes)
        return fail(QS_ERR_UNSUPPORTED, "%s: packed W^T must be smaller than 1 GiB", fn);
    if (rows > 0x7FFFFFFF) return fail(QS_ERR_UNSUPPORTED, "%s: too many rows", fn);
    if (rows == 0) return ok();
    if (!x || !wt_packed) return fail(QS_ERR_INVALID_ARG, "%s: x and wt_packed must be non-NULL", fn);
    const void* ptrs[] = {x, wt_packed, acc, y, xq, xscale, idx, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(QS_ERR_UNSUPPORTED, "%s: pointer not 16-byte aligned", fn);
    I8tWs need = i8t_ws(nullptr, rows, d_in, n_out);
    if (ws == nullptr || ws_bytes < need.bytes)
        return fail(QS_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need.bytes);
    I8tWs wsp = i8t_ws((char*)ws, rows, d_in, n_out);
    qs::I8tPlan plan = qs::plan_i8t(rows, d_in, n_out);
    hipStream_t st = (hipStream_t)stream;
    if (qs::i8t_fused_supported(rows, d_in, n_out)) {
        // 1-4 tokens: quantisation, selection and the exact integer sums in
        // one launch (the workspace is not used).
        qs::I8fArgs f{};
        f.x = x; f.rows = rows; f.d_in = d_in; f.n_out = n_out; f.k = k;
        f.wt = wt_packed; f.alpha = alpha; f.acc = acc; f.y = y; f.xq = xq; f.xscale = xscale;
        f.idx = idx;
        const hipError_t e = qs::launch_i8t_fused(f, st);
        if (e != hipSuccess) return hip_fail(e, fn);
        return ok();
    }
    float* scale = xscale ? xscale : wsp.scale;
    qs::TopkArgs t{};
    t.x = x; t.d = d_in; t.k = k; t.idx = idx; t.idx_stride = k;
    t.xs = wsp.qs; t.xq = xq; t.xscale = scale;
    t.zero_ptr = wsp.counters; t.n_zero = plan.n_counters;
    // The matrix-core kernel's splits add into zeroed int32 sums: acc itself
    // when asked for, else scratch; each row's selection workgroup zeroes it.
    int32_t* acc_sum = nullptr;
    if (plan.mfma && plan.nsplit > 1 && (acc || y)) {
        acc_sum = acc ? acc : wsp.partial;
        t.zero_rows = acc_sum;
        t.zero_row_len = n_out;
    }
    hipError_t e = qs::launch_topk(qs::KEY_Q8, qs::XS_I8, rows, t, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (!acc && !y) return ok();
    qs::I8tArgs g{};
    g.qs = wsp.qs; g.xscale = scale; g.rows = rows; g.d_in = d_in; g.n_out = n_out;
    g.wt = wt_packed; g.alpha = alpha; g.partial = wsp.partial; g.counters = wsp.counters;
    g.acc = acc; g.y = y; g.acc_sum = acc_sum;
    e = qs::launch_i8t(plan, g, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

qs_status qs_sparse_ffn(const void* x, qs_dtype dt, int64_t rows, int64_t d, int64_t ffn,
                        qs_act act, int64_t k_in, int64_t k_mid,
                        const void* w_gate, const void* w_up, const void* w_down_t,
                        const float* b_gate, const float* b_up,
                        void* y, qs_dtype yt, float* h, int32_t* mid_idx, int32_t* mid_cnt,
                        void* ws, size_t ws_bytes, void* stream) {
    // (natural pitches: W_up^T / W_gate^T rows of ffn, dReLU's W_up / W_gate rows of d)
    return qs_sparse_ffn_pitched(x, dt, rows, d, ffn, act, k_in, k_mid, w_gate, w_up,
                                 act == QS_ACT_DRELU ? d : ffn, w_down_t, d, b_gate, b_up, y, yt,
                                 h, mid_idx, mid_cnt, ws, ws_bytes, stream);
}

qs_status qs_sparse_ffn_pitched(const void* x, qs_dtype dt, int64_t rows, int64_t d, int64_t ffn,
                                qs_act act, int64_t k_in, int64_t k_mid, const void* w_gate,
                                const void* w_up, int64_t ld_up, const void* w_down_t,
                                int64_t ld_down, const float* b_gate, const float* b_up,
                                void* y, qs_dtype yt, float* h, int32_t* mid_idx,
                                int32_t* mid_cnt, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "qs_sparse_ffn";
    if (rows < 0 || d <= 0 || ffn <= 0 || d > (int64_t(1) << 24) || ffn > (int64_t(1) << 24))
        return fail(QS_ERR_INVALID_ARG, "%s: bad shape", fn);
    if (act != QS_ACT_RELU2 && act != QS_ACT_DRELU && act != QS_ACT_RELU2_GLU)
        return fail(QS_ERR_INVALID_ARG, "%s: unknown activation", fn);
    if (k_in < 0 || k_in > d) return fail(QS_ERR_INVALID_ARG, "%s: need 0 <= k_in <= d", fn);
    if (k_mid > ffn) return fail(QS_ERR_INVALID_ARG, "%s: need k_mid <= ffn", fn);
    if (!valid_float_dtype(dt) || !valid_float_dtype(yt))
        return fail(QS_ERR_UNSUPPORTED, "%s: dtypes must be QS_F32 or QS_BF16", fn);
    if (act == QS_ACT_DRELU && dt != QS_BF16)
        return fail(QS_ERR_UNSUPPORTED, "%s: dReLU path needs bf16 x and weights", fn);
    if (d % 8 != 0 || ffn % 8 != 0)
        return fail(QS_ERR_UNSUPPORTED, "%s: d and ffn must be multiples of 8", fn);
    // Natural pitches: rows of W_up^T (and W_gate^T) hold ffn entries, rows
    // of dReLU's W_up (and W_gate) d entries, rows of W_down^T d entries.
    const int64_t up_len = act == QS_ACT_DRELU ? d : ffn;
    const int64_t up_rows = act == QS_ACT_DRELU ? ffn : d;
    if (ld_up < up_len || ld_down < d || ld_up % 8 != 0 || ld_down % 8 != 0)
        return fail(QS_ERR_INVALID_ARG,
                    "%s: need row pitches of at least the row lengths, multiples of 8", fn);
    if (up_rows * ld_up * (dt == QS_BF16 ? 2 : 4) >= qs::kMaxGatherWeightBytes ||
        ffn * ld_down * (dt == QS_BF16 ? 2 : 4) >= qs::kMaxGatherWeightBytes)
        return fail(QS_ERR_UNSUPPORTED, "%s: each weight matrix must be smaller than 1 GiB", fn);
    if (rows > 0x7FFFFFFF) return fail(QS_ERR_UNSUPPORTED, "%s: too many rows", fn);
    if (rows == 0) return ok();
    if (!x || !w_up || !w_down_t || !y)
        return fail(QS_ERR_INVALID_ARG, "%s: x, w_up, w_down_t and y must be non-NULL", fn);
    if (act == QS_ACT_DRELU && !w_gate) return fail(QS_ERR_INVALID_ARG, "%s: dReLU needs w_gate", fn);
    if (act == QS_ACT_RELU2 && (w_gate || b_gate || b_up))
        return fail(QS_ERR_INVALID_ARG, "%s: squared ReLU takes no gate weights or biases", fn);
    if (act == QS_ACT_RELU2_GLU && (!w_gate || b_gate || b_up))
        return fail(QS_ERR_INVALID_ARG, "%s: gated squared ReLU needs w_gate and takes no biases", fn);
    const void* ptrs[] = {x, w_gate, w_up, w_down_t, b_gate, b_up, y, h, mid_idx, mid_cnt, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(QS_ERR_UNSUPPORTED, "%s: pointer not 16-byte aligned", fn);
    const bool drelu = act == QS_ACT_DRELU;
    FfnWs need = ffn_ws(nullptr, rows, d, ffn, drelu);
    if (ws == nullptr || ws_bytes < need.bytes)
        return fail(QS_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need.bytes);
    FfnWs wsp = ffn_ws((char*)ws, rows, d, ffn, drelu);
    hipStream_t st = (hipStream_t)stream;
    const int wb = dt == QS_BF16;
    const int kk = wb ? qs::KEY_BF16 : qs::KEY_F32;
    float* hbuf = h ? h : wsp.h;
    hipError_t e;
    if (drelu && ld_up != up_len)   // (the dReLU gate/up kernels read whole natural rows)
        return fail(QS_ERR_UNSUPPORTED, "%s: dReLU takes W_gate and W_up with natural rows", fn);

    // Small batches of the squared-ReLU kinds with bf16 weights.  The up
    // launch (for one token selecting the top-k_in of x in every workgroup,
    // else after a selection launch) computes whole column tiles of u over
    // all selected rows (fixed-order sums, no K split, no atomics), writing
    // h; the selection of h writes only its descriptor (tau, cutoff) (and the
    // index list if asked for); the down gather applies it to h and gathers
    // only the selected rows of W_down^T.
    if (!drelu && wb && qs::up_cols_supported(rows, d, ffn)) {
        const qs::GemvPlan pdn = qs::plan_gemv(rows, ffn, d, wb);
        if (pdn.bt <= 8 && pdn.scratch_floats <= wsp.partial_cap &&
            (size_t)pdn.n_counters <= wsp.down_ctr_cap) {
            const bool acc = !deterministic() && yt == QS_F32 && qs::gemv_accumulate_supported(pdn, wb);
            qs::UpColsArgs u{};
            u.x = (const uint16_t*)x; u.rows = rows; u.d = d; u.ffn = ffn; u.k = k_in;
            u.w_ld = ld_up;
            if (rows == 1) {
                // One token: the up launch selects it itself and clears what
                // the down gather needs cleared.
                if (acc) { u.zero = (float*)y; u.n_zero = rows * d; }
                else { u.zero_i = wsp.ctr_down; u.n_zero_i = pdn.n_counters; }
            } else {
                // Several tokens: one selection launch (a workgroup per token)
                // beats selecting every token in every up workgroup.
                qs::TopkArgs t{};
                t.x = x; t.d = d; t.k = k_in; t.idx_stride = k_in;
                t.xs = wsp.xs1;
                t.zero_ptr = wsp.ctr_down; t.n_zero = pdn.n_counters;
                if (acc) { t.zero_rows = (int32_t*)y; t.zero_row_len = d; }
                e = qs::launch_topk(kk, qs::XS_F32, rows, t, st);
                if (e != hipSuccess) return hip_fail(e, fn);
                u.xs = wsp.xs1;
            }
            u.w = (const uint16_t*)w_up;
            u.w2 = act == QS_ACT_RELU2_GLU ? (const uint16_t*)w_gate : nullptr;
            u.h = hbuf;
            // One token without the index list or count of h: the down
            // gather's workgroups select h themselves (one launch less).
            int fs_tiles = 0, fs_split = 0, fs_cand = 0;
            if (rows == 1) qs::gather_sel_plan(ffn, d, &fs_tiles, &fs_split, &fs_cand);
            const bool fused_sel = rows == 1 && k_mid >= 0 && !mid_idx && !mid_cnt &&
                                   qs::gather_sel_supported(rows, ffn, d) &&
                                   (size_t)fs_split * d <= wsp.partial_cap &&
                                   (size_t)fs_tiles <= wsp.down_ctr_cap;
            if (fused_sel && !acc && u.n_zero_i < fs_tiles) u.n_zero_i = fs_tiles;
            e = qs::launch_up_cols(u, st);
            if (e != hipSuccess) return hip_fail(e, fn);
            if (fused_sel) {
                qs::GemvArgs g{};
                g.xs = hbuf; g.rows = rows; g.d_in = ffn; g.n_out = d; g.w = w_down_t;
                g.partial = wsp.partial; g.counters = wsp.ctr_down; g.y = y; g.y_bf16 = yt == QS_BF16;
                g.epilogue = qs::EPI_STORE;
                g.accumulate = acc ? 1 : 0;
                g.sel_k = k_mid;
                g.w_ld = ld_down;
                e = qs::launch_gather_sel(g, st);
                if (e != hipSuccess) return hip_fail(e, fn);
                return ok();
            }
            if (k_mid >= 0 && !mid_idx && !mid_cnt && qs::desc31_supported(ffn)) {
                // Only the descriptor: the lean selection.
                e = qs::launch_desc31(hbuf, rows, ffn, k_mid, wsp.desc, st);
                if (e != hipSuccess) return hip_fail(e, fn);
            } else if (k_mid >= 0) {
                qs::TopkArgs tm{};
                tm.x = hbuf; tm.d = ffn; tm.k = k_mid;
                tm.tau = wsp.desc; tm.cutoff = (int32_t*)wsp.desc + rows; tm.cutoff_any = 1;
                tm.idx = mid_idx; tm.idx_stride = ffn; tm.count = mid_cnt;
                e = qs::launch_topk(qs::KEY_F32, qs::XS_NONE, rows, tm, st);
                if (e != hipSuccess) return hip_fail(e, fn);
            } else if (mid_idx || mid_cnt) {
                e = qs::launch_nonzero_lists(hbuf, rows, ffn, mid_idx, mid_cnt, st);
                if (e != hipSuccess) return hip_fail(e, fn);
            }
            qs::GemvArgs g{};
            g.xs = hbuf; g.rows = rows; g.d_in = ffn; g.n_out = d; g.w = w_down_t; g.w_ld = ld_down;
            g.partial = wsp.partial; g.counters = wsp.ctr_down; g.y = y; g.y_bf16 = yt == QS_BF16;
            g.epilogue = qs::EPI_STORE;
            g.accumulate = acc ? 1 : 0;
            g.sel_desc = k_mid >= 0 ? wsp.desc : nullptr;   // k_mid < 0: every nonzero entry
            e = qs::launch_gemv(pdn, wb, g, st);
            if (e != hipSuccess) return hip_fail(e, fn);
            return ok();
        }
    }

    // Accumulate forms (unless fixed-order sums are asked for): the gathers'
    // workgroups add their partial tiles into zeroed fp32 buffers instead of
    // handing them to a last workgroup.  Up projection: the input selection
    // clears the sums, and the selection of h maps them to h (so only with
    // k_mid >= 0).  Down projection: the selection of h clears y.
    const qs::GemvPlan pd = ffn_down_plan(rows, d, ffn, wb, drelu, k_mid);
    // The carved regions hold every plan this call launches (by construction;
    // checked on the host before anything is enqueued).
    if (pd.scratch_floats > wsp.partial_cap || (size_t)pd.n_counters > wsp.down_ctr_cap)
        return fail(QS_ERR_WORKSPACE, "%s: internal: down-gather plan exceeds its workspace", fn);
    if (!drelu) {
        const qs::GemvPlan pu = qs::plan_gemv(rows, d, ffn, wb);
        if (pu.scratch_floats + pu.partial_floats > wsp.partial_cap ||
            (size_t)pu.n_counters > wsp.up_ctr_cap)
            return fail(QS_ERR_WORKSPACE, "%s: internal: up-gather plan exceeds its workspace", fn);
    }
    // (y is cleared by the selection of h, or without one by the dReLU
    // gate/up launch.)
    const bool acc_down = !deterministic() && (k_mid >= 0 || drelu) && yt == QS_F32 &&
                          qs::gemv_accumulate_supported(pd, wb);
    bool acc_up = false, dual = false;

    // Stage 1: the intermediate h.
    if (!drelu) {
        qs::GemvPlan pu = qs::plan_gemv(rows, d, ffn, wb);
        dual = act == QS_ACT_RELU2_GLU && qs::gemv_dual_supported(pu, wb);
        acc_up = !deterministic() && k_mid >= 0 && qs::topk_xform_supported(ffn) &&
                 qs::gemv_accumulate_supported(pu, wb) && (act == QS_ACT_RELU2 || dual);
        qs::TopkArgs t{};
        t.x = x; t.d = d; t.k = k_in; t.idx_stride = k_in;
        t.xs = wsp.xs1;
        t.zero_ptr = wsp.ctr_up; t.n_zero = wsp.n_ctr;
        if (acc_up) {
            t.zero_rows = (int32_t*)hbuf;
            t.zero_rows2 = dual ? (int32_t*)wsp.gacc : nullptr;
            t.zero_row_len = ffn;
        }
        qs::GemvArgs g{};
        g.xs = wsp.xs1; g.rows = rows; g.d_in = d; g.n_out = ffn; g.w = w_up; g.w_ld = ld_up;
        g.partial = wsp.partial; g.counters = wsp.ctr_up; g.y = hbuf; g.y_bf16 = 0;
        g.epilogue = acc_up ? qs::EPI_STORE : qs::EPI_RELU2;
        g.accumulate = acc_up ? 1 : 0;
        g.xs_bf16 = dt == QS_BF16;
        // (The non-dual gated form runs two gathers over the same xs.)
        // (Not for the gated forms: the dual gather measured slower reading
        // records at its register budget, and the non-dual one runs two
        // gathers over the same xs.)
        if (act == QS_ACT_RELU2) route_records(t, g, pu, wb, rows, d, wsp.partial, dt != QS_BF16);
        e = qs::launch_topk(kk, qs::XS_F32, rows, t, st);
        if (e != hipSuccess) return hip_fail(e, fn);
        if (dual) {
            // Both projections in one gather: the gate's and the up rows of
            // each selected feature are streamed together, and the last
            // split (or, in the accumulate form, the selection of h) forms
            // h = relu(g)^2 * u.
            g.w2 = w_gate;
            if (acc_up) g.y2 = wsp.gacc;
            else g.partial2 = wsp.partial + pu.scratch_floats;   // behind the partials and records
            e = qs::launch_gemv_dual(pu, wb, g, st);
            if (e != hipSuccess) return hip_fail(e, fn);
        } else if (act == QS_ACT_RELU2_GLU) {
            // Gate first, kept in fp32 in the buffer that later holds the
            // selected intermediate; the up gather then forms h in its epilogue.
            // Both gathers read the same selected rows; the split counters
            // are left zero by each.
            qs::GemvArgs gg = g;
            gg.w = w_gate; gg.y = wsp.hs; gg.epilogue = qs::EPI_STORE;
            e = qs::launch_gemv(pu, wb, gg, st);
            if (e != hipSuccess) return hip_fail(e, fn);
            g.epilogue = qs::EPI_RELU2_GLU;
            g.gate = wsp.hs;
            g.frag_ready = 1;   // the gate gather packed the same coefficients
            e = qs::launch_gemv(pu, wb, g, st);
            if (e != hipSuccess) return hip_fail(e, fn);
        } else {
            e = qs::launch_gemv(pu, wb, g, st);
            if (e != hipSuccess) return hip_fail(e, fn);
        }
    } else {
        const uint16_t* xin = (const uint16_t*)x;
        bool zeroed = false;
        if (k_in < d) {
            qs::TopkArgs t{};
            t.x = x; t.d = d; t.k = k_in; t.idx_stride = k_in;
            t.xs = wsp.xm;
            t.zero_ptr = wsp.ctr_up; t.n_zero = wsp.n_ctr;
            e = qs::launch_topk(qs::KEY_BF16, qs::XS_BF16, rows, t, st);
            if (e != hipSuccess) return hip_fail(e, fn);
            xin = wsp.xm;
            zeroed = true;
        }
        qs::DreluArgs g{};
        g.x = xin; g.rows = rows; g.d = d; g.ffn = ffn;
        g.wg = (const uint16_t*)w_gate; g.wu = (const uint16_t*)w_up;
        g.bg = b_gate; g.bu = b_up; g.h = hbuf;
        g.zero_ptr = zeroed ? nullptr : wsp.ctr_up; g.n_zero = zeroed ? 0 : wsp.n_ctr;
        if (acc_down && k_mid < 0) { g.zero_out = (float*)y; g.n_zero_out = rows * d; }
        e = qs::launch_drelu_gate_up(g, st);
        if (e != hipSuccess) return hip_fail(e, fn);
    }

    // Stage 2: select the intermediate entries that enter W_down.
    qs::GemvArgs g{};   // the down gather (stage 3)
    g.rows = rows; g.d_in = ffn; g.n_out = d; g.w = w_down_t; g.w_ld = ld_down;
    g.partial = wsp.partial; g.counters = wsp.ctr_down; g.y = y; g.y_bf16 = yt == QS_BF16;
    g.epilogue = qs::EPI_STORE;
    g.accumulate = acc_down ? 1 : 0;
    const float* hsel = hbuf;
    if (k_mid >= 0) {
        qs::TopkArgs t{};
        t.x = hbuf; t.d = ffn; t.k = k_mid;
        t.idx = mid_idx; t.idx_stride = ffn; t.count = mid_cnt;
        t.xs = wsp.hs;
        if (acc_up) {
            // hbuf holds the raw up sums (and gacc the gate's): map them to h
            // here, and write h back where the caller asked for it.
            t.xform = dual ? qs::XF_RELU2_GLU : qs::XF_RELU2;
            t.x2 = wsp.gacc;
            t.h_out = h;
        }
        if (acc_down) { t.zero_rows = (int32_t*)y; t.zero_row_len = d; }
        route_records(t, g, pd, wb, rows, ffn, wsp.partial, 1);
        e = qs::launch_topk(qs::KEY_F32, qs::XS_F32, rows, t, st);
        if (e != hipSuccess) return hip_fail(e, fn);
        hsel = wsp.hs;
    } else if (mid_idx || mid_cnt) {
        e = qs::launch_nonzero_lists(hbuf, rows, ffn, mid_idx, mid_cnt, st);
        if (e != hipSuccess) return hip_fail(e, fn);
    }

    // Stage 3: gathered down projection.
    g.xs = hsel;
    e = qs::launch_gemv(pd, wb, g, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

}  // extern "C"

// ----------------------------------------------------------------- allocation-free FFN
// Scratch of qs_sparse_ffn_static: one array per GPU, held until the process
// ends.  Host code never passes the array's name to a kernel or a copy (on
// the host it is a stand-in, not a device address): each device's address is
// looked up once with hipGetSymbolAddress, with that device current, and the
// kernels receive it as their workspace.
static __device__ __align__(256) unsigned char scratch[QS_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device

// The current device's address of the scratch array (looked up on the first
// call on that device).
qs_status static_scratch(const char* fn, void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (dev < 0 || dev >= kMaxDevices)
        return fail(QS_ERR_UNSUPPORTED, "%s: device index %d is beyond %d", fn, dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, fn);
        if (p == nullptr) return fail(QS_ERR_HIP, "%s: no device address for the scratch array", fn);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return QS_OK;
}

}  // namespace

extern "C" {

qs_status qs_sparse_ffn_static(const void* x, qs_dtype dt, int64_t rows, int64_t d, int64_t ffn,
                               qs_act act, int64_t k_in, int64_t k_mid,
                               const void* w_gate, const void* w_up, const void* w_down_t,
                               const float* b_gate, const float* b_up,
                               void* y, qs_dtype yt, float* h, int32_t* mid_idx,
                               int32_t* mid_cnt, void* stream) {
    const char* fn = "qs_sparse_ffn_static";
    // qs_sparse_ffn's own validation first: without a workspace it enqueues
    // nothing and, for valid arguments, stops at the workspace check.
    const qs_status v = qs_sparse_ffn(x, dt, rows, d, ffn, act, k_in, k_mid, w_gate, w_up, w_down_t,
                                      b_gate, b_up, y, yt, h, mid_idx, mid_cnt, nullptr, 0, stream);
    if (v != QS_ERR_WORKSPACE) return v;   // QS_OK (rows == 0) or an argument error
    const size_t need = ffn_ws(nullptr, rows, d, ffn, act == QS_ACT_DRELU).bytes;
    if (need > (size_t)QS_STATIC_SCRATCH_BYTES)
        return fail(QS_ERR_UNSUPPORTED,
                    "%s: this shape needs %zu bytes of scratch, more than the %zu the library "
                    "holds per GPU (use qs_sparse_ffn with a workspace)",
                    fn, need, (size_t)QS_STATIC_SCRATCH_BYTES);
    void* ws = nullptr;
    const qs_status st = static_scratch(fn, &ws);
    if (st != QS_OK) return st;
    return qs_sparse_ffn(x, dt, rows, d, ffn, act, k_in, k_mid, w_gate, w_up, w_down_t, b_gate,
                         b_up, y, yt, h, mid_idx, mid_cnt, ws, (size_t)QS_STATIC_SCRATCH_BYTES,
                         stream);
}

qs_status qs_sparse_linear_backward(const void* x, qs_dtype xt, int64_t rows, int64_t d_in,
                                    int64_t k, const void* w, qs_dtype wt_t, qs_layout w_layout,
                                    int64_t n_out, const void* dy, qs_dtype dyt, void* dx,
                                    qs_dtype dxt, void* dw, qs_dtype dwt, void* ws,
                                    size_t ws_bytes, void* stream) {
    const char* fn = "qs_sparse_linear_backward";
    if (rows < 0 || d_in <= 0 || n_out <= 0 || d_in > (int64_t(1) << 24))
        return fail(QS_ERR_INVALID_ARG, "%s: bad shape", fn);
    if (k < 0 || k > d_in) return fail(QS_ERR_INVALID_ARG, "%s: need 0 <= k <= d_in", fn);
    if (w_layout != QS_LAYOUT_WT && w_layout != QS_LAYOUT_W)
        return fail(QS_ERR_INVALID_ARG, "%s: unknown weight layout", fn);
    if (xt != QS_BF16 || wt_t != QS_BF16 || dyt != QS_BF16)
        return fail(QS_ERR_UNSUPPORTED, "%s: x, w and dy must be QS_BF16", fn);
    if ((dx && !valid_float_dtype(dxt)) || (dw && !valid_float_dtype(dwt)))
        return fail(QS_ERR_UNSUPPORTED, "%s: dx and dw dtypes must be QS_F32 or QS_BF16", fn);
    if (d_in % 8 != 0 || n_out % 8 != 0)
        return fail(QS_ERR_UNSUPPORTED, "%s: d_in and n_out must be multiples of 8", fn);
    const int64_t lim = int64_t(1) << 30;
    if (rows * d_in >= lim || rows * n_out >= lim || d_in * n_out >= lim)
        return fail(QS_ERR_UNSUPPORTED, "%s: every operand must hold fewer than 2^30 elements", fn);
    if (dx == nullptr && dw == nullptr) return ok();
    if ((rows > 0 && (!x || !dy)) || (dx && !w))
        return fail(QS_ERR_INVALID_ARG, "%s: x, dy (and w for dx) must be non-NULL", fn);
    const void* ptrs[] = {x, w, dy, dx, dw};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(QS_ERR_UNSUPPORTED, "%s: pointer not 16-byte aligned", fn);
    const size_t need = ((size_t)rows * (size_t)d_in * 2 + 255) & ~size_t(255);
    if (dw && rows > 0 && (ws == nullptr || ws_bytes < need || !aligned16(ws)))
        return fail(QS_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
    hipStream_t st = (hipStream_t)stream;
    hipError_t e;
    if (dw) {
        // dW = dY^T . (X (.) M): the mask recomputed from x (same k, same
        // selection as the forward), X (.) M written in bf16, then a GEMM
        // contracting over the tokens, both operands k-major.  rows == 0
        // gives a zero gradient (every load is out of range).
        const uint16_t* xm = (const uint16_t*)dw;
        if (rows > 0) {
            qs::TopkArgs t{};
            t.x = x; t.d = d_in; t.k = k; t.idx_stride = k;
            t.xs = ws;
            e = qs::launch_topk(qs::KEY_BF16, qs::XS_BF16, rows, t, st);
            if (e != hipSuccess) return hip_fail(e, fn);
            xm = (const uint16_t*)ws;
        }
        const uint16_t* gy = rows > 0 ? (const uint16_t*)dy : (const uint16_t*)dw;
        qs::GemmArgs g{};
        g.a_kmajor = 1; g.b_kmajor = 1; g.k = rows; g.c = dw; g.c_bf16 = dwt == QS_BF16;
        if (w_layout == QS_LAYOUT_WT) {     // dW^T [d_in, n_out]
            g.a = xm; g.lda = d_in; g.m = d_in;
            g.b = gy; g.ldb = n_out; g.n = n_out;
        } else {                            // dW [n_out, d_in]
            g.a = gy; g.lda = n_out; g.m = n_out;
            g.b = xm; g.ldb = d_in; g.n = d_in;
        }
        e = qs::launch_gemm_bf16(g, st);
        if (e != hipSuccess) return hip_fail(e, fn);
    }
    if (dx && rows > 0) {
        // dX = dY . W, not masked (straight-through estimator).
        qs::GemmArgs g{};
        g.a = (const uint16_t*)dy; g.a_kmajor = 0; g.lda = n_out;
        g.m = rows; g.n = d_in; g.k = n_out;
        g.b = (const uint16_t*)w;
        if (w_layout == QS_LAYOUT_WT) { g.b_kmajor = 0; g.ldb = n_out; }   // W^T [d_in, n_out]
        else { g.b_kmajor = 1; g.ldb = d_in; }                            // W [n_out, d_in]
        g.c = dx; g.c_bf16 = dxt == QS_BF16;
        e = qs::launch_gemm_bf16(g, st);
        if (e != hipSuccess) return hip_fail(e, fn);
    }
    return ok();
}

qs_status qs_block_sparse_linear(const void* x, qs_dtype xt, int64_t rows, int64_t d_in,
                                 const void* w, qs_dtype wt_t, int64_t n_out, void* y,
                                 qs_dtype yt, uint8_t* mask, void* ws, size_t ws_bytes,
                                 void* stream) {
    const char* fn = "qs_block_sparse_linear";
    if (rows < 0 || d_in <= 0 || n_out <= 0) return fail(QS_ERR_INVALID_ARG, "%s: bad shape", fn);
    if (xt != QS_BF16 || wt_t != QS_BF16)
        return fail(QS_ERR_UNSUPPORTED, "%s: x and w must be QS_BF16", fn);
    if (!valid_float_dtype(yt)) return fail(QS_ERR_UNSUPPORTED, "%s: y must be QS_F32 or QS_BF16", fn);
    if (d_in % 32 != 0 || n_out % 8 != 0)
        return fail(QS_ERR_UNSUPPORTED, "%s: need d_in %% 32 == 0 and n_out %% 8 == 0", fn);
    const int64_t lim = int64_t(1) << 30;
    if (rows * d_in >= lim || n_out * d_in >= lim || rows * n_out >= (int64_t(1) << 31))
        return fail(QS_ERR_UNSUPPORTED, "%s: x and w must hold fewer than 2^30 elements", fn);
    if (rows == 0) return ok();
    if (!x || !w || !y) return fail(QS_ERR_INVALID_ARG, "%s: x, w and y must be non-NULL", fn);
    const void* ptrs[] = {x, w, y, mask, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(QS_ERR_UNSUPPORTED, "%s: pointer not 16-byte aligned", fn);
    const size_t need = qs::nm24_packed_bytes(rows, d_in);
    if (ws == nullptr || ws_bytes < need)
        return fail(QS_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need);
    qs::BlockSparseArgs a{};
    a.x = (const uint16_t*)x; a.rows = rows; a.d = d_in; a.n = n_out;
    a.w = (const uint16_t*)w; a.y = y; a.y_bf16 = yt == QS_BF16; a.mask = mask; a.ws = ws;
    hipError_t e = qs::launch_block_sparse_linear(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

qs_status qs_sparse_moe_ffn(const void* x, qs_dtype dt, int64_t rows, int64_t d, int64_t ffn,
                            int64_t n_experts, int64_t top_k, const void* w_router,
                            const void* w_gate, const void* w_up, const void* w_down_t,
                            const float* b_gate, const float* b_up, void* y, qs_dtype yt,
                            float* router_logits, int32_t* experts, float* expert_weights,
                            float* h, void* ws, size_t ws_bytes, void* stream) {
    const char* fn = "qs_sparse_moe_ffn";
    if (rows < 0 || d <= 0 || ffn <= 0) return fail(QS_ERR_INVALID_ARG, "%s: bad shape", fn);
    if (n_experts < 1 || top_k < 1 || top_k > n_experts)
        return fail(QS_ERR_INVALID_ARG, "%s: need 1 <= top_k <= n_experts", fn);
    if (n_experts > 64) return fail(QS_ERR_UNSUPPORTED, "%s: at most 64 experts", fn);
    if (dt != QS_BF16) return fail(QS_ERR_UNSUPPORTED, "%s: x and the weights must be QS_BF16", fn);
    if (!valid_float_dtype(yt)) return fail(QS_ERR_UNSUPPORTED, "%s: y must be QS_F32 or QS_BF16", fn);
    if (d % 8 != 0 || ffn % 8 != 0 || d > 8192)
        return fail(QS_ERR_UNSUPPORTED, "%s: need d %% 8 == 0, ffn %% 8 == 0 and d <= 8192", fn);
    if (ffn * d * 2 >= qs::kMaxGatherWeightBytes)
        return fail(QS_ERR_UNSUPPORTED, "%s: an expert matrix must be smaller than 1 GiB", fn);
    if (rows * top_k > 0x7FFFFFFF) return fail(QS_ERR_UNSUPPORTED, "%s: too many rows", fn);
    if (rows == 0) return ok();
    if (!x || !w_router || !w_gate || !w_up || !w_down_t || !y)
        return fail(QS_ERR_INVALID_ARG, "%s: x, the weights and y must be non-NULL", fn);
    const void* ptrs[] = {x, w_router, w_gate, w_up, w_down_t, b_gate, b_up, y, router_logits,
                          experts, expert_weights, h, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return fail(QS_ERR_UNSUPPORTED, "%s: pointer not 16-byte aligned", fn);
    const int64_t pairs = rows * top_k;
    MoeWs need = moe_ws(nullptr, pairs, d, ffn);
    if (ws == nullptr || ws_bytes < need.bytes)
        return fail(QS_ERR_WORKSPACE, "%s: workspace needs %zu bytes", fn, need.bytes);
    MoeWs wsp = moe_ws((char*)ws, pairs, d, ffn);
    hipStream_t st = (hipStream_t)stream;

    // Router: (token, expert, weight) pairs.
    qs::MoeRouteArgs r{};
    r.x = (const uint16_t*)x; r.wr = (const uint16_t*)w_router; r.rows = rows; r.d = d;
    r.n_experts = (int)n_experts; r.top_k = (int)top_k;
    r.pair_token = wsp.pair_token; r.pair_expert = wsp.pair_expert; r.pair_weight = wsp.pair_weight;
    r.logits = router_logits; r.out_experts = experts; r.out_weights = expert_weights;
    hipError_t e = qs::launch_moe_route(r, st);
    if (e != hipSuccess) return hip_fail(e, fn);

    // Gate, then up only where the gate is positive, per pair (dReLU).
    // Accumulate form of the down gather (unless fixed-order sums are asked
    // for): each pair's workgroups add weight * partial into its token's row
    // of an fp32 sum that this launch clears: y itself (no combine launch),
    // or for a bf16 y the pair buffer, which one pass then rounds into y.
    qs::GemvPlan pd = qs::plan_gemv(pairs, ffn, d, 1, 1);
    const bool acc = !deterministic() && qs::gemv_accumulate_supported(pd, 1);
    float* yacc = yt == QS_F32 ? (float*)y : wsp.ypair;   // ypair holds pairs >= rows rows
    float* hbuf = h ? h : wsp.h;
    qs::DreluArgs g{};
    g.x = (const uint16_t*)x; g.rows = rows; g.d = d; g.ffn = ffn;
    g.wg = (const uint16_t*)w_gate; g.wu = (const uint16_t*)w_up; g.bg = b_gate; g.bu = b_up;
    g.h = hbuf; g.zero_ptr = wsp.ctr; g.n_zero = wsp.n_ctr;
    if (acc) { g.zero_out = yacc; g.n_zero_out = rows * d; }
    g.pair_token = wsp.pair_token; g.pair_expert = wsp.pair_expert; g.pairs = pairs;
    if (rows > 1 && pairs <= kMoeGroupMaxPairs && rows * d * 2 < (int64_t(1) << 31)) {
        // Several tokens: group the pairs by expert so that each expert's gate
        // rows are read once per chunk of its tokens, not once per pair.
        e = qs::launch_moe_group(wsp.pair_expert, wsp.pair_token, pairs, (int)n_experts,
                                 wsp.grp_count, wsp.grp_pairs, wsp.grp_tok, st);
        if (e != hipSuccess) return hip_fail(e, fn);
        g.grp_count = wsp.grp_count; g.grp_pairs = wsp.grp_pairs; g.grp_tok = wsp.grp_tok;
        g.n_experts = (int)n_experts;
        e = qs::launch_drelu_grouped(g, st);
    } else {
        e = qs::launch_drelu_gate_up(g, st);
    }
    if (e != hipSuccess) return hip_fail(e, fn);

    // Down: each pair gathers the rows of its expert's W_down^T where h != 0.
    qs::GemvArgs gd{};
    gd.xs = hbuf; gd.rows = pairs; gd.d_in = ffn; gd.n_out = d; gd.w = w_down_t;
    gd.partial = wsp.partial; gd.counters = wsp.ctr; gd.y = wsp.ypair; gd.y_bf16 = 0;
    gd.epilogue = qs::EPI_STORE;
    gd.row_expert = wsp.pair_expert; gd.expert_bytes = ffn * d * 2;
    if (acc) {
        gd.y = yacc; gd.accumulate = 1;
        gd.row_scale = wsp.pair_weight; gd.row_out = wsp.pair_token;
    }
    e = qs::launch_gemv(pd, 1, gd, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    if (acc) {
        if (yt == QS_F32) return ok();
        e = qs::launch_moe_combine(yacc, nullptr, rows, 1, d, y, 1, st);   // weights already applied
        if (e != hipSuccess) return hip_fail(e, fn);
        return ok();
    }

    e = qs::launch_moe_combine(wsp.ypair, wsp.pair_weight, rows, (int)top_k, d, y, yt == QS_BF16, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

}  // extern "C"
