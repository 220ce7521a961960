// C-ABI entry points of libtpshard.so: argument validation, shard planning,
// workspace sizing and kernel dispatch. Every check runs on the host before
// anything is enqueued; nothing here allocates device memory or synchronises.
#include "tp_shard.h"

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_err;

tp_status fail(tp_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

tp_status ok() {
    g_err.clear();
    return TP_OK;
}

tp_status hip_fail(hipError_t e, const char* what) {
    return fail(TP_ERR_HIP, "%s: HIP error %s (%s); check that the pointers are device memory of the current "
                "device and the stream belongs to it", what, hipGetErrorName(e), hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

size_t esize(tp_dtype dt) { return dt == TP_BF16 ? 2 : 4; }
size_t vec_elems(tp_dtype dt) { return dt == TP_BF16 ? 8 : 4; }
size_t round256(size_t b) { return (b + 255) / 256 * 256; }

constexpr int64_t kMaxDim = int64_t(1) << 30;
// Up to this many tokens a bf16 projection runs on the decode projections (blocks of 16 tokens, each
// streaming the weights), above it on the MFMA GEMM, whose 256-row tiles at a few dozen rows leave most
// of their matrix work idle and split K into float32 tiles. Measured per step: the 70B layer at t=8 with
// 32 / 64 / 128 sequences 938 / 1624 / 3009 us on the decode projections against 1517 / 1690 / 2172 us
// on the GEMM, the Llama-3-8B MLP at t=4 with 32 / 64 / 128 tokens 148 / 258 / 467 us against
// 423 / 425 / 433 us.
constexpr int kGemvMaxM = 64;
// Above kGemvMaxM tokens a projection still stays on the decode projections when its output is this
// narrow (a router's logits): a 256 x 256 GEMM tile would leave most of its matrix work idle and split
// its few tiles' K into float32 tiles, while the decode projections read the activations once in blocks
// of 16 tokens against one tile of weight rows (the Mixtral router at 4096 tokens: 21 + 38 us on the
// GEMM and its tail kernel)
constexpr int kGemmMinN = 65;
// The stacked experts of a decode batch (every expert's blocks in one projection, hundreds of MB per
// rank) go to the GEMM above one block of 16 tokens: there every further block of the decode
// projections streams all of them again (Mixtral t=2 MoE step at 32 / 64 tokens: 913 / 920 us on the
// GEMM against 996 / 1917 us on the decode projections).
constexpr int kStackedGemvMaxM = 16;

tp_status check_dtype(tp_dtype dt) {
    if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_DTYPE, "dtype %d is neither TP_F32 nor TP_BF16", (int)dt);
    return TP_OK;
}

tp_status check_dims(int64_t m, int64_t k, int64_t n) {
    if (m < 1 || k < 1 || n < 1)
        return fail(TP_ERR_SHAPE, "sizes must be >= 1 (m=%lld k=%lld n=%lld)", (long long)m, (long long)k, (long long)n);
    if (m > kMaxDim || k > kMaxDim || n > kMaxDim || m * n > (int64_t(1) << 40) || n * k > (int64_t(1) << 40))
        return fail(TP_ERR_SHAPE, "sizes too large (m=%lld k=%lld n=%lld); each must be <= 2^30",
                    (long long)m, (long long)k, (long long)n);
    return TP_OK;
}

tp_status check_ptr(const void* p, const char* name) {
    if (!p) return fail(TP_ERR_NULL, "%s is NULL", name);
    if (!aligned16(p)) return fail(TP_ERR_ALIGN, "%s=%p is not 16-byte aligned; allocate with the default "
                                   "allocator or pad to 16 bytes", name, p);
    return TP_OK;
}

tp_status check_ws(void* ws, size_t have, size_t need) {
    if (need == 0) return TP_OK;
    if (!ws) return fail(TP_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
    if (reinterpret_cast<uintptr_t>(ws) & 255u)
        return fail(TP_ERR_WORKSPACE, "workspace %p is not 256-byte aligned", ws);
    if (have < need)
        return fail(TP_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed; size it with the matching "
                    "*_workspace_bytes call", have, need);
    return TP_OK;
}

#define TRY(expr)                       \
    do {                                \
        tp_status st_ = (expr);         \
        if (st_ != TP_OK) return st_;   \
    } while (0)

bool use_gemm(int64_t m, int64_t k, int64_t n, tp_dtype dt, int epi, int gemv_max_m = kGemvMaxM) {
    return dt == TP_BF16 && epi != tpk::EPI_QKV && m > gemv_max_m && n >= kGemmMinN &&
           tpk::gemm_supported((int)m, (int)n, (int)k, epi);
}

// Scratch bytes (after the counter header) a projection needs: on the GEMM
// path the normalised activations (with a norm) and the K-range sums of its
// last partial round of tiles; on the GEMV path the split-K slices.
size_t gemm_norm_bytes(int64_t m, int64_t k, tp_dtype dt, bool norm) {
    return norm ? round256((size_t)m * k * esize(dt)) : 0;
}

size_t linear_scratch(int64_t m, int64_t k, int64_t n, tp_dtype dt, int epi, bool norm,
                      int gemv_max_m = kGemvMaxM) {
    if (use_gemm(m, k, n, dt, epi, gemv_max_m))
        return gemm_norm_bytes(m, k, dt, norm) + round256(tpk::gemm_scratch_bytes((int)m, (int)n, (int)k, epi));
    return round256(tpk::gemv_plan((int)m, (int)k, (int)n, dt == TP_BF16, epi).ws_bytes);
}

bool linear_needs_ws(int64_t m, int64_t k, int64_t n, tp_dtype dt, int epi, bool norm) {
    if (use_gemm(m, k, n, dt, epi)) return linear_scratch(m, k, n, dt, epi, norm) > 0;
    return tpk::gemv_plan((int)m, (int)k, (int)n, dt == TP_BF16, epi).splits > 1;
}

// Whole workspace of a standalone projection: header + scratch, or 0.
size_t linear_ws(int64_t m, int64_t k, int64_t n, tp_dtype dt, int epi, bool norm) {
    return linear_needs_ws(m, k, n, dt, epi, norm) ? tpk::WS_HEADER + linear_scratch(m, k, n, dt, epi, norm) : 0;
}

// Enqueue one projection. x [m,k], w (and w_up) [n,k]; y per epilogue.
// counters: the workspace header; scratch: this call's scratch region.
tp_status run_linear(const void* x, const void* w, const void* w_up, const void* gamma, float eps, void* y,
                     int64_t m, int64_t k, int64_t n, tp_dtype dt, int epi, unsigned* counters, void* scratch,
                     hipStream_t s, const tpk::GemvArgs* qkv = nullptr, int gemv_max_m = kGemvMaxM) {
    const bool norm = gamma != nullptr;
    if (use_gemm(m, k, n, dt, epi, gemv_max_m)) {
        const void* xin = x;
        if (norm) {
            hipError_t e = tpk::rmsnorm_launch(x, gamma, scratch, (int)m, (int)k, eps, 1, s);
            if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
            xin = scratch;
        }
        tpk::GemmArgs g{};
        g.x = xin; g.w = w; g.w_up = w_up; g.y = y;
        g.M = (int)m; g.N = (int)n; g.K = (int)k; g.epi = epi;
        g.scratch = scratch ? reinterpret_cast<char*>(scratch) + gemm_norm_bytes(m, k, dt, norm) : nullptr;
        hipError_t e = tpk::gemm_launch(g, s);
        if (e != hipSuccess) return hip_fail(e, "MFMA GEMM launch");
        return ok();
    }
    tpk::GemvArgs a{};
    if (qkv) a = *qkv;
    a.x = x; a.w = w; a.w_up = w_up; a.gamma = gamma; a.y = y;
    a.m = (int)m; a.K = (int)k; a.N = (int)n; a.eps = eps;
    a.is_bf16 = dt == TP_BF16;
    a.epi = epi;
    a.norm = norm;
    const tpk::GemvPlan p = tpk::gemv_plan(a.m, a.K, a.N, a.is_bf16, epi);
    hipError_t e = tpk::gemv_launch(a, p, counters, scratch, s);
    if (e != hipSuccess) return hip_fail(e, "GEMV launch");
    return ok();
}

unsigned* ws_counters(void* ws) { return reinterpret_cast<unsigned*>(ws); }
void* ws_scratch(void* ws) { return ws ? reinterpret_cast<char*>(ws) + tpk::WS_HEADER : nullptr; }

tp_status plan_impl(const tp_model_desc* d, int32_t t, int32_t rank, tp_rank_plan* out) {
    if (!d) return fail(TP_ERR_NULL, "desc is NULL");
    if (!out) return fail(TP_ERR_NULL, "out is NULL");
    if (t < 1 || t > 8) return fail(TP_ERR_RANK, "t=%d outside 1..8 (tensor parallelism stays inside one node)", t);
    if (rank < 0 || rank >= t) return fail(TP_ERR_RANK, "rank=%d outside 0..%d", rank, t - 1);
    if (d->hidden <= 0 || d->intermediate < 0 || d->n_q_heads < 0)
        return fail(TP_ERR_SHAPE, "hidden must be > 0, intermediate and n_q_heads >= 0");
    const bool attn = d->n_q_heads > 0;
    if (attn) {
        if (d->n_kv_heads <= 0 || d->head_dim <= 0)
            return fail(TP_ERR_SHAPE, "attention needs n_kv_heads > 0 and head_dim > 0");
        if (d->n_q_heads % d->n_kv_heads)
            return fail(TP_ERR_INDIVISIBLE, "n_q_heads=%d is not a multiple of n_kv_heads=%d", d->n_q_heads,
                        d->n_kv_heads);
        if (d->n_q_heads % t)
            return fail(TP_ERR_INDIVISIBLE, "t=%d must divide n_q_heads=%d", t, d->n_q_heads);
        if (d->n_kv_heads % t && t % d->n_kv_heads)
            return fail(TP_ERR_INDIVISIBLE, "t=%d must divide n_kv_heads=%d or be a multiple of it (then each "
                        "rank keeps a copy of the kv head its q heads read)", t, d->n_kv_heads);
    }
    if (d->intermediate % t)
        return fail(TP_ERR_INDIVISIBLE, "t=%d must divide intermediate=%lld", t, (long long)d->intermediate);
    const int64_t H = d->hidden;
    const int32_t q_r = attn ? d->n_q_heads / t : 0;
    // t > n_kv: every rank keeps the one kv head its q heads read (t / n_kv copies of each).
    const bool replicate = attn && (d->n_kv_heads % t) != 0;
    const int32_t kv_r = attn ? (replicate ? 1 : d->n_kv_heads / t) : 0;
    const int64_t hd = attn ? d->head_dim : 0;
    const int64_t i_r = d->intermediate / t;
    tp_rank_plan p{};
    p.t = t;
    p.rank = rank;
    p.q_head_begin = rank * q_r;
    p.q_heads = q_r;
    p.kv_head_begin = replicate ? rank / (t / d->n_kv_heads) : rank * kv_r;
    p.kv_heads = kv_r;
    p.inter_begin = rank * i_r;
    p.inter_cols = i_r;
    p.qkv_cols = (q_r + 2 * kv_r) * hd;
    p.o_rows = q_r * hd;
    p.weight_elems = H * (q_r + 2 * kv_r) * hd + q_r * hd * H + 3 * H * i_r;
    if (attn) {
        const int64_t per_seq = 2 * (int64_t)d->n_layers * d->n_kv_heads * hd * d->seq_len;
        const int64_t total = per_seq * d->bytes_per_elem * d->batch;
        p.kv_elems_per_seq_all_layers = per_seq;
        p.kv_bytes_rank = replicate ? total / d->n_kv_heads : total / t;   // replicated: one head's cache
    }
    *out = p;
    return ok();
}

// The plan the caller passes must be the one tp_shard_plan gives for its t and rank.
tp_status check_plan(const tp_model_desc* d, const tp_rank_plan* p) {
    if (!d) return fail(TP_ERR_NULL, "desc is NULL");
    if (!p) return fail(TP_ERR_NULL, "plan is NULL");
    tp_rank_plan ref{};
    TRY(plan_impl(d, p->t, p->rank, &ref));
    if (ref.q_head_begin != p->q_head_begin || ref.q_heads != p->q_heads || ref.kv_heads != p->kv_heads ||
        ref.inter_begin != p->inter_begin || ref.inter_cols != p->inter_cols || ref.qkv_cols != p->qkv_cols ||
        ref.o_rows != p->o_rows)
        return fail(TP_ERR_SHAPE, "plan does not match desc for t=%d rank=%d; build it with tp_shard_plan",
                    p->t, p->rank);
    return TP_OK;
}

// Layer workspace: [counter header][act1][act2][projection scratch][attention scratch].
struct LayerWs {
    size_t act1, act2, lin, attn, total;
};

LayerWs layer_ws(const tp_model_desc* d, const tp_rank_plan* p, tp_stage stage, int64_t m, tp_dtype dt,
                 bool prefill) {
    LayerWs w{};
    const int64_t H = d->hidden;
    if (stage == TP_STAGE_ATTN && prefill) {
        w.act1 = round256((size_t)m * p->qkv_cols * 2);  // [q | k | v] of every token
        w.act2 = round256((size_t)m * p->o_rows * 2);    // attention output
        const size_t l1 = linear_scratch(m, H, p->qkv_cols, dt, tpk::EPI_STORE, true);
        const size_t l2 = linear_scratch(m, p->o_rows, H, dt, tpk::EPI_PARTIAL, false);
        w.lin = l1 > l2 ? l1 : l2;
    } else if (stage == TP_STAGE_ATTN) {
        w.act1 = round256((size_t)m * p->o_rows * 2);   // q
        w.act2 = round256((size_t)m * p->o_rows * 2);   // attention output
        const size_t l1 = linear_scratch(m, H, p->qkv_cols, dt, tpk::EPI_QKV, true);
        const size_t l2 = linear_scratch(m, p->o_rows, H, dt, tpk::EPI_PARTIAL, false);
        w.lin = l1 > l2 ? l1 : l2;
        // sized for every kv_len up to the cache capacity
        w.attn = round256(tpk::attn_ws_bound((int)m, p->q_heads, p->kv_heads, d->head_dim, (int)d->seq_len));
    } else {
        w.act1 = round256((size_t)m * p->inter_cols * esize(dt));  // SwiGLU output
        const size_t l1 = linear_scratch(m, H, p->inter_cols, dt, tpk::EPI_SWIGLU, true);
        const size_t l2 = linear_scratch(m, p->inter_cols, H, dt, tpk::EPI_PARTIAL, false);
        w.lin = l1 > l2 ? l1 : l2;
    }
    w.total = tpk::WS_HEADER + w.act1 + w.act2 + w.lin + w.attn;
    return w;
}

}  // namespace

extern "C" {

const char* tp_status_name(tp_status s) {
    switch (s) {
        case TP_OK: return "TP_OK";
        case TP_ERR_NULL: return "TP_ERR_NULL";
        case TP_ERR_SHAPE: return "TP_ERR_SHAPE";
        case TP_ERR_INDIVISIBLE: return "TP_ERR_INDIVISIBLE";
        case TP_ERR_RANK: return "TP_ERR_RANK";
        case TP_ERR_DTYPE: return "TP_ERR_DTYPE";
        case TP_ERR_ALIGN: return "TP_ERR_ALIGN";
        case TP_ERR_WORKSPACE: return "TP_ERR_WORKSPACE";
        case TP_ERR_KV: return "TP_ERR_KV";
        case TP_ERR_ALIAS: return "TP_ERR_ALIAS";
        case TP_ERR_HIP: return "TP_ERR_HIP";
    }
    return "TP_ERR_UNKNOWN";
}

const char* tp_last_error(void) { return g_err.c_str(); }

tp_status tp_shard_plan(const tp_model_desc* desc, int32_t t, int32_t rank, tp_rank_plan* out) {
    return plan_impl(desc, t, rank, out);
}

size_t tp_linear_workspace_bytes(int64_t m, int64_t k, int64_t n, tp_dtype dtype, int32_t flags) {
    if (m < 1 || k < 1 || n < 1 || (dtype != TP_F32 && dtype != TP_BF16)) return 0;
    const int epi = (flags & TP_LINEAR_SWIGLU) ? tpk::EPI_SWIGLU : tpk::EPI_STORE;
    const size_t a = linear_ws(m, k, n, dtype, epi, (flags & TP_LINEAR_NORM) != 0);
    const size_t b = linear_ws(m, k, n, dtype, tpk::EPI_PARTIAL, false);
    return a > b ? a : b;
}

tp_status tp_column_linear(const void* x, const void* w, const void* w_up, const void* gamma, float eps, void* y,
                           int64_t m, int64_t k, int64_t n, tp_dtype dtype, void* ws, size_t ws_bytes,
                           void* stream) {
    TRY(check_dtype(dtype));
    TRY(check_ptr(x, "x"));
    TRY(check_ptr(w, "w"));
    TRY(check_ptr(y, "y"));
    if (w_up) TRY(check_ptr(w_up, "w_up"));
    if (gamma) TRY(check_ptr(gamma, "gamma"));
    TRY(check_dims(m, k, n));
    if (k % (int64_t)vec_elems(dtype))
        return fail(TP_ERR_ALIGN, "k=%lld is not a multiple of %zu (rows are read in 128-bit vectors)",
                    (long long)k, vec_elems(dtype));
    if (!(eps >= 0.0f)) return fail(TP_ERR_SHAPE, "eps must be >= 0");
    const size_t es = esize(dtype);
    const size_t ny = (size_t)m * n * es;
    if (overlaps(y, ny, x, (size_t)m * k * es) || overlaps(y, ny, w, (size_t)n * k * es) ||
        overlaps(y, ny, w_up, (size_t)n * k * es) || overlaps(y, ny, gamma, (size_t)k * es))
        return fail(TP_ERR_ALIAS, "y overlaps an input; use a separate output buffer");
    if (ws && overlaps(ws, ws_bytes, y, ny)) return fail(TP_ERR_ALIAS, "workspace overlaps y");
    const int epi = w_up ? tpk::EPI_SWIGLU : tpk::EPI_STORE;
    TRY(check_ws(ws, ws_bytes, linear_ws(m, k, n, dtype, epi, gamma != nullptr)));
    return run_linear(x, w, w_up, gamma, eps, y, m, k, n, dtype, epi, ws_counters(ws), ws_scratch(ws),
                      (hipStream_t)stream);
}

tp_status tp_row_linear_partial(const void* a, const void* w, float* partial, int64_t m, int64_t k, int64_t n,
                                tp_dtype dtype, void* ws, size_t ws_bytes, void* stream) {
    TRY(check_dtype(dtype));
    TRY(check_ptr(a, "a"));
    TRY(check_ptr(w, "w"));
    TRY(check_ptr(partial, "partial"));
    TRY(check_dims(m, k, n));
    if (k % (int64_t)vec_elems(dtype))
        return fail(TP_ERR_ALIGN, "k=%lld is not a multiple of %zu (rows are read in 128-bit vectors)",
                    (long long)k, vec_elems(dtype));
    const size_t es = esize(dtype);
    const size_t np = (size_t)m * n * 4;
    if (overlaps(partial, np, a, (size_t)m * k * es) || overlaps(partial, np, w, (size_t)n * k * es))
        return fail(TP_ERR_ALIAS, "partial overlaps an input");
    if (ws && overlaps(ws, ws_bytes, partial, np)) return fail(TP_ERR_ALIAS, "workspace overlaps partial");
    TRY(check_ws(ws, ws_bytes, linear_ws(m, k, n, dtype, tpk::EPI_PARTIAL, false)));
    return run_linear(a, w, nullptr, nullptr, 0.f, partial, m, k, n, dtype, tpk::EPI_PARTIAL, ws_counters(ws),
                      ws_scratch(ws), (hipStream_t)stream);
}

tp_status tp_swiglu(const void* gate, const void* up, void* out, int64_t m, int64_t n, tp_dtype dtype,
                    void* stream) {
    TRY(check_dtype(dtype));
    TRY(check_ptr(gate, "gate"));
    TRY(check_ptr(up, "up"));
    TRY(check_ptr(out, "out"));
    TRY(check_dims(m, 1, n));
    const size_t nb = (size_t)m * n * esize(dtype);
    if ((out != gate && overlaps(out, nb, gate, nb)) || (out != up && overlaps(out, nb, up, nb)))
        return fail(TP_ERR_ALIAS, "out partially overlaps gate or up (only exact in-place is allowed)");
    hipError_t e = tpk::swiglu_launch(gate, up, out, m * n, dtype == TP_BF16, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "SwiGLU launch");
    return ok();
}

}  // extern "C"

namespace {

tp_status partial_sum_impl(const void* const* partials, int in_bf16, int32_t t, const void* residual, void* out,
                           int64_t m, int64_t n, tp_dtype out_dtype, void* stream) {
    TRY(check_dtype(out_dtype));
    if (!partials) return fail(TP_ERR_NULL, "partials is NULL");
    if (t < 1 || t > 8) return fail(TP_ERR_RANK, "t=%d outside 1..8", t);
    TRY(check_ptr(out, "out"));
    if (residual) TRY(check_ptr(residual, "residual"));
    TRY(check_dims(m, 1, n));
    tpk::PartialPtrs ps{};
    const size_t np = (size_t)m * n * (in_bf16 ? 2 : 4);
    const size_t no = (size_t)m * n * esize(out_dtype);
    for (int r = 0; r < t; ++r) {
        char name[32];
        snprintf(name, sizeof name, "partials[%d]", r);
        TRY(check_ptr(partials[r], name));
        if (overlaps(out, no, partials[r], np)) return fail(TP_ERR_ALIAS, "out overlaps %s", name);
        ps.p[r] = partials[r];
    }
    if (residual && residual != out && overlaps(out, no, residual, no))
        return fail(TP_ERR_ALIAS, "out partially overlaps residual (only exact in-place is allowed)");
    hipError_t e = tpk::partial_sum_launch(ps, t, residual, out, m * n, in_bf16, out_dtype == TP_BF16,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "partial-sum launch");
    return ok();
}

}  // namespace

extern "C" {

tp_status tp_partial_sum(const float* const* partials, int32_t t, const void* residual, void* out, int64_t m,
                         int64_t n, tp_dtype out_dtype, void* stream) {
    return partial_sum_impl(reinterpret_cast<const void* const*>(partials), 0, t, residual, out, m, n, out_dtype,
                            stream);
}

tp_status tp_partial_sum_bf16(const void* const* partials, int32_t t, const void* residual, void* out, int64_t m,
                              int64_t n, tp_dtype out_dtype, void* stream) {
    return partial_sum_impl(partials, 1, t, residual, out, m, n, out_dtype, stream);
}

tp_status tp_row_linear_partial_bf16(const void* a, const void* w, void* partial, int64_t m, int64_t k, int64_t n,
                                     void* ws, size_t ws_bytes, void* stream) {
    TRY(check_ptr(a, "a"));
    TRY(check_ptr(w, "w"));
    TRY(check_ptr(partial, "partial"));
    TRY(check_dims(m, k, n));
    if (k % 8) return fail(TP_ERR_ALIGN, "k=%lld is not a multiple of 8 (rows are read in 128-bit vectors)",
                           (long long)k);
    const size_t np = (size_t)m * n * 2;
    if (overlaps(partial, np, a, (size_t)m * k * 2) || overlaps(partial, np, w, (size_t)n * k * 2))
        return fail(TP_ERR_ALIAS, "partial overlaps an input");
    if (ws && overlaps(ws, ws_bytes, partial, np)) return fail(TP_ERR_ALIAS, "workspace overlaps partial");
    TRY(check_ws(ws, ws_bytes, linear_ws(m, k, n, TP_BF16, tpk::EPI_STORE, false)));
    // A bf16 partial is the plain projection rounded to bf16: the store epilogue.
    return run_linear(a, w, nullptr, nullptr, 0.f, partial, m, k, n, TP_BF16, tpk::EPI_STORE, ws_counters(ws),
                      ws_scratch(ws), (hipStream_t)stream);
}

}  // extern "C"

namespace {

// Tokens up to which the router's logits and gates come from one fused launch
// (every workgroup reads all of W_router, cheap for a decode batch).
constexpr int64_t MOE_FUSED_ROUTER_MAX_M = 64;
// Larger batches compute each expert over its own tokens (grouped GEMMs),
// when a token's experts fit the partial sum's eight inputs.
constexpr int MOE_GROUPED_MAX_K = 8;

bool moe_grouped(int64_t m, int32_t top_k) { return m > MOE_FUSED_ROUTER_MAX_M && top_k <= MOE_GROUPED_MAX_K; }

// MoE workspace: [header][u (normalised x)][logits][gates] then, for a decode
// batch, [expert activations, every expert][projection scratch]; for a grouped
// batch, [slots][lists][counts][activations, packed by expert][slot partials
// [top_k, m, H] float32][projection scratch].
struct MoeWs {
    size_t u, logits, gates, act, lin, slots, lists, counts, parts, total;
};

MoeWs moe_ws(int64_t m, int64_t H, int32_t E, int64_t cols, bool norm, int32_t top_k) {
    MoeWs w{};
    const int64_t ecols = (int64_t)E * cols;
    w.u = norm ? round256((size_t)m * H * 2) : 0;
    w.logits = round256((size_t)m * E * 4);
    w.gates = round256((size_t)m * E * 4);
    size_t l = linear_scratch(m, H, E, TP_BF16, tpk::EPI_PARTIAL, false);
    if (moe_grouped(m, top_k)) {
        w.slots = round256((size_t)m * E * 4);
        w.lists = round256((size_t)m * E * 4);
        w.counts = round256((size_t)E * 4);
        w.act = round256((size_t)m * top_k * cols * 2);
        w.parts = round256((size_t)top_k * m * H * 4);
    } else {
        w.act = round256((size_t)m * ecols * 2);
        const size_t l2 = linear_scratch(m, H, ecols, TP_BF16, tpk::EPI_SWIGLU, false, kStackedGemvMaxM);
        const size_t l3 = linear_scratch(m, ecols, H, TP_BF16, tpk::EPI_PARTIAL, false, kStackedGemvMaxM);
        if (l2 > l) l = l2;
        if (l3 > l) l = l3;
    }
    w.lin = l;
    w.total = tpk::WS_HEADER + w.u + w.logits + w.gates + w.slots + w.lists + w.counts + w.act + w.parts + w.lin;
    return w;
}

}  // namespace

extern "C" {

size_t tp_moe_workspace_bytes(int64_t m, int64_t hidden, int32_t n_experts, int32_t top_k, int64_t inter_cols,
                              int32_t has_norm) {
    if (m < 1 || hidden < 1 || n_experts < 1 || n_experts > 64 || inter_cols < 1) return 0;
    if (top_k < 1 || top_k > n_experts) return 0;
    return moe_ws(m, hidden, n_experts, inter_cols, has_norm != 0, top_k).total;
}

tp_status tp_moe_shard_forward(const tp_moe_weights* w, const void* x, float* partial, float* gates_out,
                               float* logits_out, int64_t m, int64_t hidden, int32_t n_experts, int32_t top_k,
                               int64_t inter_cols, float eps, void* ws, size_t ws_bytes, void* stream) {
    if (!w) return fail(TP_ERR_NULL, "weights is NULL");
    TRY(check_ptr(x, "x"));
    TRY(check_ptr(partial, "partial"));
    TRY(check_ptr(w->w_router, "weights->w_router"));
    TRY(check_ptr(w->w_gate, "weights->w_gate"));
    TRY(check_ptr(w->w_up, "weights->w_up"));
    TRY(check_ptr(w->w_down, "weights->w_down"));
    if (w->norm) TRY(check_ptr(w->norm, "weights->norm"));
    if (gates_out) TRY(check_ptr(gates_out, "gates_out"));
    if (logits_out) TRY(check_ptr(logits_out, "logits_out"));
    if (n_experts < 1 || n_experts > 64) return fail(TP_ERR_SHAPE, "n_experts=%d outside 1..64", n_experts);
    if (top_k < 1 || top_k > n_experts) return fail(TP_ERR_SHAPE, "top_k=%d outside 1..n_experts", top_k);
    if (!(eps >= 0.0f)) return fail(TP_ERR_SHAPE, "eps must be >= 0");
    TRY(check_dims(m, hidden, (int64_t)n_experts * inter_cols));
    if (hidden % 8 || inter_cols % 8)
        return fail(TP_ERR_ALIGN, "hidden=%lld and inter_cols=%lld must be multiples of 8", (long long)hidden,
                    (long long)inter_cols);
    const int64_t ecols = (int64_t)n_experts * inter_cols;
    const size_t np = (size_t)m * hidden * 4;
    if (overlaps(partial, np, x, (size_t)m * hidden * 2)) return fail(TP_ERR_ALIAS, "partial overlaps x");
    const MoeWs L = moe_ws(m, hidden, n_experts, inter_cols, w->norm != nullptr, top_k);
    TRY(check_ws(ws, ws_bytes, L.total));
    if (overlaps(ws, ws_bytes, partial, np)) return fail(TP_ERR_ALIAS, "workspace overlaps partial");
    char* b = reinterpret_cast<char*>(ws) + tpk::WS_HEADER;
    unsigned* cnt = ws_counters(ws);
    void* u = b;
    b += L.u;
    float* logits = logits_out ? logits_out : reinterpret_cast<float*>(b);
    b += L.logits;
    float* gates = gates_out ? gates_out : reinterpret_cast<float*>(b);
    b += L.gates;
    int* slots = reinterpret_cast<int*>(b);
    b += L.slots;
    int* lists = reinterpret_cast<int*>(b);
    b += L.lists;
    int* counts = reinterpret_cast<int*>(b);
    b += L.counts;
    void* act = b;
    b += L.act;
    float* parts = reinterpret_cast<float*>(b);
    b += L.parts;
    void* lin = b;
    hipStream_t s = (hipStream_t)stream;
    const void* xin = x;
    if (w->norm) {
        hipError_t e = tpk::rmsnorm_launch(x, w->norm, u, (int)m, (int)hidden, eps, 1, s);
        if (e != hipSuccess) return hip_fail(e, "rmsnorm launch");
        xin = u;
    }
    // The router is replicated on every rank: logits = u @ W_router^T, float32,
    // then the top-k gates. A decode batch takes both in one launch; larger
    // batches form the logits as a projection.
    hipError_t e;
    if (m <= MOE_FUSED_ROUTER_MAX_M) {
        e = tpk::moe_router_launch(xin, w->w_router, logits, gates, (int)m, (int)hidden, n_experts, top_k, s);
        if (e != hipSuccess) return hip_fail(e, "router launch");
    } else {
        TRY(run_linear(xin, w->w_router, nullptr, nullptr, 0.f, logits, m, hidden, n_experts, TP_BF16,
                       tpk::EPI_PARTIAL, cnt, lin, s));
        e = tpk::moe_gates_launch(logits, gates, (int)m, n_experts, top_k, s, moe_grouped(m, top_k) ? slots : nullptr);
        if (e != hipSuccess) return hip_fail(e, "router gates launch");
    }
    if (moe_grouped(m, top_k)) {
        // Each expert over its own tokens: the token lists, gate/up + SwiGLU on
        // the gathered rows (activations packed expert after expert), down on
        // the packed rows into the token's slot times its gate, then the top_k
        // slots of every token added in slot (expert) order.
        e = tpk::moe_lists_launch(slots, lists, counts, (int)m, n_experts, s);
        if (e != hipSuccess) return hip_fail(e, "expert token lists launch");
        tpk::GemmGroups gg{};
        gg.counts = counts; gg.lists = lists; gg.slots = slots; gg.gates = gates; gg.G = n_experts;
        gg.rows_total = (int)(m * top_k);
        tpk::GemmArgs ga{};
        ga.x = xin; ga.w = w->w_gate; ga.w_up = w->w_up; ga.y = act;
        ga.M = (int)m; ga.N = (int)inter_cols; ga.K = (int)hidden; ga.epi = tpk::EPI_SWIGLU;
        gg.b_group_stride = inter_cols * hidden;
        gg.ldb = (int)hidden;
        e = tpk::gemm_grouped_launch(ga, gg, s);
        if (e != hipSuccess) return hip_fail(e, "grouped expert gate/up launch");
        tpk::GemmArgs gd{};
        gd.x = act; gd.w = w->w_down; gd.y = parts;
        gd.M = (int)m; gd.N = (int)hidden; gd.K = (int)inter_cols; gd.epi = tpk::EPI_PARTIAL;
        gg.b_group_stride = inter_cols;
        gg.ldb = (int)ecols;
        e = tpk::gemm_grouped_launch(gd, gg, s);
        if (e != hipSuccess) return hip_fail(e, "grouped expert down launch");
        tpk::PartialPtrs ps{};
        for (int k = 0; k < top_k; ++k) ps.p[k] = parts + (size_t)k * m * hidden;
        e = tpk::partial_sum_launch(ps, top_k, nullptr, partial, m * hidden, 0, 0, s);
        if (e != hipSuccess) return hip_fail(e, "expert slot sum launch");
        return ok();
    }
    // Every expert's gate/up column block at once (rows stacked expert by expert).
    TRY(run_linear(xin, w->w_gate, w->w_up, nullptr, 0.f, act, m, hidden, ecols, TP_BF16, tpk::EPI_SWIGLU, cnt,
                   lin, s, nullptr, kStackedGemvMaxM));
    e = tpk::moe_scale_launch(act, gates, (int)m, n_experts, inter_cols, s);
    if (e != hipSuccess) return hip_fail(e, "expert gate scaling launch");
    // Every expert's down row block at once: the gate-weighted sum over experts is the contraction over the
    // stacked intermediate columns.
    return run_linear(act, w->w_down, nullptr, nullptr, 0.f, partial, m, ecols, hidden, TP_BF16, tpk::EPI_PARTIAL,
                      cnt, lin, s, nullptr, kStackedGemvMaxM);
}

size_t tp_attention_workspace_bytes(int64_t batch, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                    int64_t kv_len) {
    if (batch < 1 || q_heads < 1 || kv_heads < 1 || q_heads % kv_heads || kv_len < 1) return 0;
    const tpk::AttnPlan p = tpk::attn_plan((int)batch, q_heads, kv_heads, head_dim, (int)kv_len);
    return p.n_chunks > 1 ? tpk::WS_HEADER + round256(p.ws_bytes) : 0;
}

static tp_status check_attention(const void* q, const void* k, const void* v, const void* out, int64_t batch,
                                 int32_t q_heads, int32_t kv_heads, int32_t head_dim, int64_t capacity,
                                 int64_t kv_len, tp_dtype dtype) {
    if (dtype != TP_BF16) return fail(TP_ERR_DTYPE, "decode attention supports bf16 only");
    TRY(check_ptr(q, "q"));
    TRY(check_ptr(k, "k"));
    TRY(check_ptr(v, "v"));
    TRY(check_ptr(out, "out"));
    if (batch < 1 || batch > (1 << 20)) return fail(TP_ERR_SHAPE, "batch=%lld outside 1..2^20", (long long)batch);
    if (q_heads < 1 || kv_heads < 1) return fail(TP_ERR_SHAPE, "q_heads and kv_heads must be >= 1");
    if (q_heads % kv_heads) return fail(TP_ERR_INDIVISIBLE, "q_heads=%d not a multiple of kv_heads=%d", q_heads, kv_heads);
    const int gq = q_heads / kv_heads;
    if (gq != 1 && gq != 2 && gq != 4 && gq != 8 && gq != 16)
        return fail(TP_ERR_SHAPE, "q_heads/kv_heads=%d must be 1, 2, 4, 8 or 16", gq);
    if (head_dim != 64 && head_dim != 128) return fail(TP_ERR_SHAPE, "head_dim=%d must be 64 or 128", head_dim);
    if (capacity < 1 || capacity > (int64_t(1) << 24)) return fail(TP_ERR_SHAPE, "capacity outside 1..2^24");
    if (kv_len < 1 || kv_len > capacity)
        return fail(TP_ERR_KV, "kv_len=%lld outside 1..capacity=%lld", (long long)kv_len, (long long)capacity);
    if ((kv_len + 255) / 256 > 128LL * 1024) return fail(TP_ERR_KV, "kv_len too large");
    const size_t no = (size_t)batch * q_heads * head_dim * 2;
    const size_t nc = (size_t)batch * kv_heads * capacity * head_dim * 2;
    if (overlaps(out, no, q, no) || overlaps(out, no, k, nc) || overlaps(out, no, v, nc))
        return fail(TP_ERR_ALIAS, "out overlaps q or the caches");
    return TP_OK;
}

tp_status tp_decode_attention(const void* q, const void* k, const void* v, void* out, int64_t batch, int32_t q_heads,
                              int32_t kv_heads, int32_t head_dim, int64_t capacity, int64_t kv_len, tp_dtype dtype,
                              void* ws, size_t ws_bytes, void* stream) {
    TRY(check_attention(q, k, v, out, batch, q_heads, kv_heads, head_dim, capacity, kv_len, dtype));
    const tpk::AttnPlan p = tpk::attn_plan((int)batch, q_heads, kv_heads, head_dim, (int)kv_len);
    TRY(check_ws(ws, ws_bytes, p.n_chunks > 1 ? tpk::WS_HEADER + round256(p.ws_bytes) : 0));
    tpk::AttnArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out;
    a.capacity = capacity; a.kv_len = (int)kv_len;
    a.batch = (int)batch; a.q_heads = q_heads; a.kv_heads = kv_heads; a.head_dim = head_dim;
    hipError_t e = tpk::attn_launch(a, p, ws_counters(ws), ws_scratch(ws), (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    return ok();
}

tp_status tp_prefill_attention(const void* q, const void* k, const void* v, void* out, int64_t batch, int64_t seq,
                               int32_t q_heads, int32_t kv_heads, int32_t head_dim, int64_t capacity, int64_t kv_len,
                               tp_dtype dtype, void* stream) {
    if (dtype != TP_BF16) return fail(TP_ERR_DTYPE, "prefill attention supports bf16 only");
    TRY(check_ptr(q, "q"));
    TRY(check_ptr(k, "k"));
    TRY(check_ptr(v, "v"));
    TRY(check_ptr(out, "out"));
    if (batch < 1 || batch > 65535) return fail(TP_ERR_SHAPE, "batch=%lld outside 1..65535", (long long)batch);
    if (q_heads < 1 || kv_heads < 1 || kv_heads > 65535) return fail(TP_ERR_SHAPE, "bad head counts");
    if (q_heads % kv_heads) return fail(TP_ERR_INDIVISIBLE, "q_heads=%d not a multiple of kv_heads=%d", q_heads, kv_heads);
    const int gq = q_heads / kv_heads;
    if (gq != 1 && gq != 2 && gq != 4 && gq != 8 && gq != 16)
        return fail(TP_ERR_SHAPE, "q_heads/kv_heads=%d must be 1, 2, 4, 8 or 16", gq);
    if (head_dim != 64 && head_dim != 128) return fail(TP_ERR_SHAPE, "head_dim=%d must be 64 or 128", head_dim);
    if (capacity < 1 || capacity > (int64_t(1) << 24)) return fail(TP_ERR_SHAPE, "capacity outside 1..2^24");
    if (kv_len < 1 || kv_len > capacity)
        return fail(TP_ERR_KV, "kv_len=%lld outside 1..capacity=%lld", (long long)kv_len, (long long)capacity);
    if (seq < 1 || seq > kv_len)
        return fail(TP_ERR_KV, "seq=%lld outside 1..kv_len=%lld", (long long)seq, (long long)kv_len);
    const size_t nq = (size_t)batch * seq * q_heads * head_dim * 2;
    const size_t nc = (size_t)batch * kv_heads * capacity * head_dim * 2;
    if (overlaps(out, nq, q, nq) || overlaps(out, nq, k, nc) || overlaps(out, nq, v, nc))
        return fail(TP_ERR_ALIAS, "out overlaps q or the caches");
    tpk::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.out = out;
    a.capacity = capacity; a.q_stride = (int64_t)q_heads * head_dim; a.kv_len = (int)kv_len;
    a.batch = (int)batch; a.seq = (int)seq; a.q_heads = q_heads; a.kv_heads = kv_heads; a.head_dim = head_dim;
    hipError_t e = tpk::prefill_attn_launch(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
    return ok();
}

tp_status tp_hbm_stream_read(const void* buf, size_t bytes, void* flag, uint32_t never, void* stream) {
    TRY(check_ptr(buf, "buf"));
    TRY(check_ptr(flag, "flag"));
    if (bytes == 0 || bytes % 16) return fail(TP_ERR_SHAPE, "bytes=%zu must be a positive multiple of 16", bytes);
    if (overlaps(flag, 4, buf, bytes)) return fail(TP_ERR_ALIAS, "flag lies inside buf");
    hipError_t e = tpk::stream_read_launch(buf, (int64_t)(bytes / 16), reinterpret_cast<unsigned*>(flag), never,
                                           (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "stream read launch");
    return ok();
}

size_t tp_layer_workspace_bytes(const tp_model_desc* desc, const tp_rank_plan* plan, tp_stage stage, int64_t m,
                                tp_dtype dtype) {
    if (!desc || !plan || m < 1 || (stage != TP_STAGE_ATTN && stage != TP_STAGE_MLP)) return 0;
    if (dtype != TP_F32 && dtype != TP_BF16) return 0;
    if (stage == TP_STAGE_ATTN && (plan->q_heads < 1 || desc->seq_len < 1)) return 0;
    if (stage == TP_STAGE_MLP && plan->inter_cols < 1) return 0;
    // m rows serve either m sequences of one new token or a block of tokens;
    // the larger of the two layouts covers both.
    const size_t dec = layer_ws(desc, plan, stage, m, dtype, false).total;
    if (stage != TP_STAGE_ATTN) return dec;
    const size_t pre = layer_ws(desc, plan, stage, m, dtype, true).total;
    return dec > pre ? dec : pre;
}

}  // extern "C"

namespace {

// The layer stage. With dry set, every check runs and nothing is enqueued.
tp_status layer_forward_impl(const tp_model_desc* desc, const tp_rank_plan* plan, tp_stage stage,
                             const tp_rank_weights* wts, const void* in, const tp_kv_view* kv, float* partial,
                             int64_t m, tp_dtype dtype, void* ws, size_t ws_bytes, void* stream, bool dry) {
    TRY(check_dtype(dtype));
    TRY(check_plan(desc, plan));
    if (!wts) return fail(TP_ERR_NULL, "weights is NULL");
    if (stage != TP_STAGE_ATTN && stage != TP_STAGE_MLP) return fail(TP_ERR_SHAPE, "unknown stage %d", (int)stage);
    TRY(check_ptr(in, "in"));
    TRY(check_ptr(partial, "partial"));
    const int64_t H = desc->hidden;
    TRY(check_dims(m, H, H));
    if (H % (int64_t)vec_elems(dtype))
        return fail(TP_ERR_ALIGN, "hidden=%lld is not a multiple of %zu", (long long)H, vec_elems(dtype));
    const size_t es = esize(dtype);
    if (overlaps(partial, (size_t)m * H * 4, in, (size_t)m * H * es)) return fail(TP_ERR_ALIAS, "partial overlaps in");
    hipStream_t s = (hipStream_t)stream;

    if (stage == TP_STAGE_ATTN) {
        if (dtype != TP_BF16) return fail(TP_ERR_DTYPE, "the attention stage supports bf16 only");
        if (plan->q_heads < 1) return fail(TP_ERR_SHAPE, "desc has no attention heads");
        if (!kv) return fail(TP_ERR_NULL, "kv is NULL for the attention stage");
        TRY(check_ptr(wts->w_qkv, "weights->w_qkv"));
        TRY(check_ptr(wts->w_o, "weights->w_o"));
        if (wts->attn_norm) TRY(check_ptr(wts->attn_norm, "weights->attn_norm"));
        if (plan->o_rows % 8) return fail(TP_ERR_ALIGN, "q_heads*head_dim=%lld not a multiple of 8", (long long)plan->o_rows);
        TRY(check_ptr(kv->k, "kv->k"));
        TRY(check_ptr(kv->v, "kv->v"));
        const int gq = plan->q_heads / plan->kv_heads;
        if (gq != 1 && gq != 2 && gq != 4 && gq != 8 && gq != 16)
            return fail(TP_ERR_SHAPE, "q heads per kv head = %d must be 1, 2, 4, 8 or 16", gq);
        if (desc->head_dim != 64 && desc->head_dim != 128)
            return fail(TP_ERR_SHAPE, "head_dim=%d must be 64 or 128", desc->head_dim);
        if (m > (1 << 20)) return fail(TP_ERR_SHAPE, "m=%lld too large", (long long)m);
        if (kv->capacity < 1 || kv->capacity > (int64_t(1) << 24))
            return fail(TP_ERR_SHAPE, "kv capacity outside 1..2^24");
        if (kv->kv_len < 1 || kv->kv_len > kv->capacity)
            return fail(TP_ERR_KV, "kv_len=%lld outside 1..capacity=%lld", (long long)kv->kv_len,
                        (long long)kv->capacity);
        if (kv->new_tokens < 0) return fail(TP_ERR_SHAPE, "kv->new_tokens=%lld is negative", (long long)kv->new_tokens);
        const int64_t S = kv->new_tokens > 1 ? kv->new_tokens : 1;   // new tokens per sequence
        if (m % S)
            return fail(TP_ERR_SHAPE, "m=%lld rows are not a whole number of %lld-token blocks", (long long)m,
                        (long long)S);
        if (S > kv->kv_len)
            return fail(TP_ERR_KV, "new_tokens=%lld exceeds kv_len=%lld", (long long)S, (long long)kv->kv_len);
        const int64_t B = m / S;                                     // sequences
        if (S > 1 && B > 65535) return fail(TP_ERR_SHAPE, "%lld sequences exceed 65535", (long long)B);
        {
            const size_t nc = (size_t)B * plan->kv_heads * kv->capacity * desc->head_dim * 2;
            if (overlaps(kv->k, nc, kv->v, nc)) return fail(TP_ERR_ALIAS, "kv->k overlaps kv->v");
            if (overlaps(kv->k, nc, in, (size_t)m * H * 2) || overlaps(kv->v, nc, in, (size_t)m * H * 2) ||
                overlaps(kv->k, nc, partial, (size_t)m * H * 4) || overlaps(kv->v, nc, partial, (size_t)m * H * 4))
                return fail(TP_ERR_ALIAS, "the KV cache overlaps in or partial");
        }
        if (kv->capacity != desc->seq_len)
            return fail(TP_ERR_KV, "kv capacity %lld differs from desc seq_len %lld", (long long)kv->capacity,
                        (long long)desc->seq_len);
        const LayerWs L = layer_ws(desc, plan, stage, m, dtype, S > 1);
        TRY(check_ws(ws, ws_bytes, L.total));
        char* b = reinterpret_cast<char*>(ws) + tpk::WS_HEADER;
        unsigned* cnt = ws_counters(ws);
        void* act1 = b;
        void* obuf = b + L.act1;
        void* lin = b + L.act1 + L.act2;
        void* aws = b + L.act1 + L.act2 + L.lin;
        if (S > 1) {
            if (dry) return ok();
            // A block of S tokens per sequence: [q | k | v] of every token, the
            // block's k, v into the cache, causal attention reading q from the
            // projected rows, W_o partial.
            TRY(run_linear(in, wts->w_qkv, nullptr, wts->attn_norm, desc->eps, act1, m, H, plan->qkv_cols, dtype,
                           tpk::EPI_STORE, cnt, lin, s));
            tpk::KvAppendArgs ka{};
            ka.qkv = act1; ka.k_cache = kv->k; ka.v_cache = kv->v; ka.capacity = kv->capacity;
            ka.row_stride = plan->qkv_cols; ka.rows = (int)m; ka.seq = (int)S; ka.kv_heads = plan->kv_heads;
            ka.head_dim = desc->head_dim; ka.pos0 = (int)(kv->kv_len - S);
            ka.k_col0 = (int)plan->o_rows; ka.v_col0 = (int)(plan->o_rows + plan->kv_heads * desc->head_dim);
            hipError_t e = tpk::kv_append_launch(ka, s);
            if (e != hipSuccess) return hip_fail(e, "KV append launch");
            tpk::PrefillArgs pa{};
            pa.q = act1; pa.k = kv->k; pa.v = kv->v; pa.out = obuf;
            pa.capacity = kv->capacity; pa.q_stride = plan->qkv_cols; pa.kv_len = (int)kv->kv_len;
            pa.batch = (int)B; pa.seq = (int)S; pa.q_heads = plan->q_heads; pa.kv_heads = plan->kv_heads;
            pa.head_dim = desc->head_dim;
            e = tpk::prefill_attn_launch(pa, s);
            if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
            return run_linear(obuf, wts->w_o, nullptr, nullptr, 0.f, partial, m, plan->o_rows, H, dtype,
                              tpk::EPI_PARTIAL, cnt, lin, s);
        }
        // Every check before the first launch: the attention plan of this kv_len
        // must fit the scratch sized for the capacity.
        const tpk::AttnPlan ap_len = tpk::attn_plan((int)m, plan->q_heads, plan->kv_heads, desc->head_dim,
                                                    (int)kv->kv_len);
        if (round256(ap_len.ws_bytes) > L.attn)
            return fail(TP_ERR_WORKSPACE, "attention scratch of %zu bytes exceeds the %zu sized for capacity %lld",
                        (size_t)round256(ap_len.ws_bytes), L.attn, (long long)kv->capacity);
        if (dry) return ok();
        tpk::GemvArgs extra{};
        extra.k_cache = kv->k;
        extra.v_cache = kv->v;
        extra.capacity = kv->capacity;
        extra.pos = kv->kv_len - 1;
        extra.q_cols = (int)plan->o_rows;
        extra.kv_cols = plan->kv_heads * desc->head_dim;
        extra.head_dim = desc->head_dim;
        extra.kv_heads = plan->kv_heads;
        TRY(run_linear(in, wts->w_qkv, nullptr, wts->attn_norm, desc->eps, act1, m, H, plan->qkv_cols, dtype,
                       tpk::EPI_QKV, cnt, lin, s, &extra));
        tpk::AttnArgs a{};
        a.q = act1; a.k = kv->k; a.v = kv->v; a.out = obuf;
        a.capacity = kv->capacity; a.kv_len = (int)kv->kv_len;
        a.batch = (int)m; a.q_heads = plan->q_heads; a.kv_heads = plan->kv_heads; a.head_dim = desc->head_dim;
        hipError_t e = tpk::attn_launch(a, ap_len, cnt, aws, s);
        if (e != hipSuccess) return hip_fail(e, "attention launch");
        return run_linear(obuf, wts->w_o, nullptr, nullptr, 0.f, partial, m, plan->o_rows, H, dtype,
                          tpk::EPI_PARTIAL, cnt, lin, s);
    }

    if (plan->inter_cols < 1) return fail(TP_ERR_SHAPE, "desc has no MLP");
    TRY(check_ptr(wts->w_gate, "weights->w_gate"));
    TRY(check_ptr(wts->w_up, "weights->w_up"));
    TRY(check_ptr(wts->w_down, "weights->w_down"));
    if (wts->mlp_norm) TRY(check_ptr(wts->mlp_norm, "weights->mlp_norm"));
    if (plan->inter_cols % (int64_t)vec_elems(dtype))
        return fail(TP_ERR_ALIGN, "inter_cols=%lld not a multiple of %zu", (long long)plan->inter_cols, vec_elems(dtype));
    const LayerWs L = layer_ws(desc, plan, stage, m, dtype, false);
    TRY(check_ws(ws, ws_bytes, L.total));
    if (dry) return ok();
    char* b = reinterpret_cast<char*>(ws) + tpk::WS_HEADER;
    unsigned* cnt = ws_counters(ws);
    void* abuf = b;
    void* lin = b + L.act1;
    TRY(run_linear(in, wts->w_gate, wts->w_up, wts->mlp_norm, desc->eps, abuf, m, H, plan->inter_cols, dtype,
                   tpk::EPI_SWIGLU, cnt, lin, s));
    return run_linear(abuf, wts->w_down, nullptr, nullptr, 0.f, partial, m, plan->inter_cols, H, dtype,
                      tpk::EPI_PARTIAL, cnt, lin, s);
}

// Scratch of tp_layer_shard_forward_static: one array per GPU, held until
// the process ends. Its device address is looked up once per device (with
// that device current) and kept here; host code never passes the array's
// name to a kernel, only that address.
static __device__ __align__(256) unsigned char scratch[TP_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
bool g_scratch_cleared[kMaxDevices] = {};

tp_status static_scratch(int dev, void** ptr) {
    if (dev < 0 || dev >= kMaxDevices) return fail(TP_ERR_HIP, "device ordinal %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "static scratch address lookup");
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return TP_OK;
}

}  // namespace

extern "C" {

tp_status tp_layer_shard_forward(const tp_model_desc* desc, const tp_rank_plan* plan, tp_stage stage,
                                 const tp_rank_weights* wts, const void* in, const tp_kv_view* kv, float* partial,
                                 int64_t m, tp_dtype dtype, void* ws, size_t ws_bytes, void* stream) {
    return layer_forward_impl(desc, plan, stage, wts, in, kv, partial, m, dtype, ws, ws_bytes, stream, false);
}

tp_status tp_layer_shard_forward_static(const tp_model_desc* desc, const tp_rank_plan* plan, tp_stage stage,
                                        const tp_rank_weights* wts, const void* in, const tp_kv_view* kv,
                                        float* partial, int64_t m, tp_dtype dtype, void* stream) {
    // The call's workspace must fit the static scratch: refuse before any HIP call.
    if (desc && plan && (stage == TP_STAGE_ATTN || stage == TP_STAGE_MLP) && m >= 1 &&
        (dtype == TP_F32 || dtype == TP_BF16)) {
        const bool pre = stage == TP_STAGE_ATTN && kv && kv->new_tokens > 1;
        const size_t need = layer_ws(desc, plan, stage, m, dtype, pre).total;
        if (need > TP_STATIC_SCRATCH_BYTES)
            return fail(TP_ERR_WORKSPACE, "this call needs %zu bytes of scratch, beyond the %d bytes of the static "
                        "scratch; call tp_layer_shard_forward with a workspace instead", need,
                        TP_STATIC_SCRATCH_BYTES);
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    void* ws = nullptr;
    TRY(static_scratch(dev, &ws));
    TRY(layer_forward_impl(desc, plan, stage, wts, in, kv, partial, m, dtype, ws, TP_STATIC_SCRATCH_BYTES, stream,
                           true));
    {
        // The counter header must start at zero; every call leaves it zero, so
        // it is cleared once per device, by a kernel on the caller's stream
        // ordered before this call's work (a graph may capture it).
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_cleared[dev]) {
            e = tpk::fill_zero_launch(ws, tpk::WS_HEADER, (hipStream_t)stream);
            if (e != hipSuccess) return hip_fail(e, "static scratch clear");
            g_scratch_cleared[dev] = true;
        }
    }
    return layer_forward_impl(desc, plan, stage, wts, in, kv, partial, m, dtype, ws, TP_STATIC_SCRATCH_BYTES, stream,
                              false);
}

}  // extern "C"
