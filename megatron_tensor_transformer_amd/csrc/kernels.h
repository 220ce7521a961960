// Launch interface between the C-ABI host code (api.cpp) and the HIP kernels.
// Host-side only types: no device code here.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tpk {

// Every workspace starts with a fixed header of split-K / split-KV counters
// shared by all entry points: each call finds its counters zero and leaves
// them zero, so one workspace can serve calls of any shape in sequence.
// Scratch data always lives after the header, never inside it.
constexpr size_t WS_HEADER = 32768;   // TP_WORKSPACE_HEADER
constexpr int WS_MAX_COUNTERS = (int)(WS_HEADER / 4);

enum Epilogue : int {
    EPI_STORE = 0,    // y[m, n] in the input dtype (column projection)
    EPI_PARTIAL = 1,  // y[m, n] float32 (row-parallel partial)
    EPI_SWIGLU = 2,   // y[m, n] = silu(gate) * up in the input dtype
    EPI_QKV = 3       // q -> y, new k/v -> cache position (decode attention block)
};

// Thin-M projection (decode): y = epilogue(u @ W^T), u = optional RMSNorm(x).
struct GemvArgs {
    const void* x;      // [m, K]
    const void* w;      // [N, K] (gate rows for EPI_SWIGLU)
    const void* w_up;   // [N, K] for EPI_SWIGLU
    const void* gamma;  // [K] or null
    void* y;            // output
    void* k_cache;      // EPI_QKV: [m, kv_heads, capacity, d]
    void* v_cache;
    int64_t capacity;
    int64_t pos;        // cache position written (kv_len - 1)
    int q_cols, kv_cols, head_dim, kv_heads;
    int m, K, N;        // N: output columns
    float eps;
    int is_bf16;
    int epi;
    int norm;
};

struct GemvPlan {
    int mfma;      // 1: matrix-core kernel (bf16, 16-token blocks), 0: v_dot2 / fma kernel
    int mt;        // tokens per block (1, 2, 4, 8, 16)
    int nw;        // waves per workgroup
    int rg, ks;    // matrix-core kernels: (4, 1) 64-row tiles split over workgroups, (2, 2) two K ranges of
                   // 2 waves; (2, 4) and (1, 8) the wide kernel's 32- and 16-row tiles, 8 waves, one K range each
    int mblocks;   // ceil(m / mt)
    int mbw;       // token blocks one workgroup of the wide matrix-core kernel takes per weight fetch (1 or 2)
    int mb_per_launch;  // m-blocks per launch, so a launch's tiles fit the counter header
    int tiles_per_launch;  // row tiles per launch (all of them unless the counters would not fit)
    int rows_per_tile;  // weight rows a workgroup covers
    int out_per_tile;   // outputs a workgroup covers
    int n_tiles;
    int kc;        // K elements per split
    int splits;    // S
    int threads;
    size_t lds_bytes;
    size_t ws_bytes;   // scratch bytes after the header; 0 when splits == 1
};

// Smallest bf16 token count that goes to the matrix-core kernel.
constexpr int GEMV_MFMA_MIN_M = 2;
GemvPlan gemv_plan(int m, int K, int N, int is_bf16, int epi);        // picks one of the two below
GemvPlan gemv_plan_dot2(int m, int K, int N, int is_bf16, int epi);
GemvPlan gemv_plan_mfma(int m, int K, int N, int epi);                // bf16 only
hipError_t gemv_launch(const GemvArgs& a, const GemvPlan& p, unsigned* counters, void* scratch, hipStream_t stream);

// Row-wise RMSNorm into a bf16/f32 buffer: u = x * gamma / sqrt(mean(x^2) + eps).
hipError_t rmsnorm_launch(const void* x, const void* gamma, void* u, int m, int K, float eps, int is_bf16,
                          hipStream_t stream);

// out = silu(gate) * up, elementwise.
hipError_t swiglu_launch(const void* gate, const void* up, void* out, int64_t count, int is_bf16,
                         hipStream_t stream);

// out = sum_r partials[r] (+ residual), rank order, float32 arithmetic;
// partials float32 or bf16.
struct PartialPtrs { const void* p[8]; };
hipError_t partial_sum_launch(const PartialPtrs& ptrs, int t, const void* residual, void* out, int64_t count,
                              int in_bf16, int out_bf16, hipStream_t stream);

// Split-KV grouped-query decode attention.
struct AttnArgs {
    const void* q;      // [B, q_heads * d]
    const void* k;      // [B, kv_heads, capacity, d]
    const void* v;
    void* out;          // [B, q_heads * d]
    int64_t capacity;
    int kv_len;
    int batch, q_heads, kv_heads, head_dim;
};
struct AttnPlan {
    int chunk;      // keys per workgroup
    int n_chunks;
    size_t ws_bytes;   // scratch bytes after the header; 0 when n_chunks == 1
};
AttnPlan attn_plan(int batch, int q_heads, int kv_heads, int head_dim, int kv_len);
// Largest attn_plan(...).ws_bytes over every kv_len in 1..max_kv_len.
size_t attn_ws_bound(int batch, int q_heads, int kv_heads, int head_dim, int max_kv_len);
hipError_t attn_launch(const AttnArgs& a, const AttnPlan& p, unsigned* counters, void* scratch, hipStream_t stream);

// Prefill projection on bf16 MFMA: y = epilogue(x @ W^T) for large m.
struct GemmArgs {
    const void* x;      // [M, K] bf16
    const void* w;      // [N, K] bf16 (gate rows for EPI_SWIGLU)
    const void* w_up;   // [N, K] bf16 for EPI_SWIGLU
    void* y;            // [M, N] bf16 (EPI_STORE, EPI_SWIGLU) or float32 (EPI_PARTIAL)
    int M, N, K;
    int epi;
    void* scratch;      // gemm_scratch_bytes(M, N, K, epi) bytes (ungrouped launches)
};
bool gemm_supported(int M, int N, int K, int epi);
// Scratch an ungrouped launch needs: the float32 sums of the K ranges its
// last, partly filled round of tiles is split into (0 when it is not split).
size_t gemm_scratch_bytes(int M, int N, int K, int epi);
hipError_t gemm_launch(const GemmArgs& a, hipStream_t stream);

// Grouped prefill projections of a mixture of experts: G independent GEMMs,
// one per expert g, whose row counts live on the device (counts[g] <= M).
// Rows of group g are packed after those of groups 0..g-1 (offset = the sum
// of the earlier counts). Column-parallel gate/up + SwiGLU (EPI_SWIGLU): A
// rows gathered through lists[g * M + r] from x [M, K]; B = w (and w_up) +
// g * b_group_stride, rows of ldb elements; y [sum of counts, N] packed.
// Row-parallel down (EPI_PARTIAL): A = x rows offset + r (packed); B as
// above; row r of group g is token t = lists[g * M + r] and is written,
// times gates[t * G + g], to y[(slots[t * G + g] * M + t) * N + n].
struct GemmGroups {
    const int* counts;      // [G]
    const int* lists;       // [G][M] token indices in ascending order
    const int* slots;       // [M][G] rank of expert g among the token's experts, -1 if not chosen
    const float* gates;     // [M][G]
    int64_t b_group_stride; // elements between consecutive groups' B blocks
    int ldb;                // B row stride (elements)
    int G;
    int rows_total;         // sum of the counts (M * top_k): bounds the groups' row tiles
};
hipError_t gemm_grouped_launch(const GemmArgs& a, const GemmGroups& g, hipStream_t stream);

// Mixture of experts: top-k router gates from float32 logits [m, E] (E <= 64),
// and a[t, e * cols + i] *= gates[t, e] on bf16 expert activations
// (cols a multiple of 8).
hipError_t moe_gates_launch(const float* logits, float* gates, int m, int E, int top_k, hipStream_t stream,
                            int* slots = nullptr);
// Per-expert token lists from the routing slots [m, E]: lists[e * m + i] the
// i-th token (ascending) routed to expert e, counts[e] how many.
hipError_t moe_lists_launch(const int* slots, int* lists, int* counts, int m, int E, hipStream_t stream);
// Router logits (written when logits is not null) and gates of m tokens in one
// launch, from bf16 u [m, H] and W_router [E, H] (H a multiple of 8; few
// tokens: one workgroup each reads all of W_router).
hipError_t moe_router_launch(const void* u, const void* w_router, float* logits, float* gates, int m, int H, int E,
                             int top_k, hipStream_t stream);
hipError_t moe_scale_launch(void* a, const float* gates, int m, int E, int64_t cols, hipStream_t stream);

// Block KV append: k, v columns of rows [batch * seq] of a [q | k | v] buffer
// (row_stride elements per row) to cache positions pos0 .. pos0 + seq - 1 (bf16).
struct KvAppendArgs {
    const void* qkv;
    void* k_cache;      // [batch, kv_heads, capacity, d]
    void* v_cache;
    int64_t capacity;
    int64_t row_stride;
    int rows, seq, kv_heads, head_dim;
    int pos0, k_col0, v_col0;
};
hipError_t kv_append_launch(const KvAppendArgs& a, hipStream_t stream);

// Causal grouped-query attention over a block of seq new tokens (bf16).
struct PrefillArgs {
    const void* q;      // [batch, seq] rows of q_stride elements; a row holds q_heads * d
    const void* k;      // [batch, kv_heads, capacity, d]
    const void* v;
    void* out;          // [batch, seq, q_heads * d]
    int64_t capacity;
    int64_t q_stride;   // elements between consecutive tokens' q rows
    int kv_len;         // token i of the block sits at position kv_len - seq + i
    int batch, seq, q_heads, kv_heads, head_dim;
};
hipError_t prefill_attn_launch(const PrefillArgs& a, hipStream_t stream);

// Plain streaming read of n16 128-bit words (the practical HBM read rate);
// out[0] is written only if the folded words equal never.
hipError_t stream_read_launch(const void* buf, int64_t n16, unsigned* out, unsigned never, hipStream_t stream);

// Zero bytes (a multiple of 16) of device memory with a kernel.
hipError_t fill_zero_launch(void* p, size_t bytes, hipStream_t stream);

}  // namespace tpk
