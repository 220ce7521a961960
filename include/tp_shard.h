/*
 * tp_shard.h - one GPU's shard of a Megatron-style tensor-parallel transformer
 * layer on MI355X (gfx950). C ABI of libtpshard.so.
 *
 * What is computed. Each transformer layer's projections are split over t
 * GPUs ("Tensor parallel scaling curves", section "What tensor parallelism
 * actually splits"): Q, K, V are split by columns so each rank owns a
 * contiguous block of attention heads, the attention output projection W_o by
 * rows, the MLP gate and up projections by columns and the down projection by
 * rows. A column-parallel projection takes the replicated input and yields
 * this rank's slice of output columns; a row-parallel projection takes the
 * column-parallel output directly and yields a partial sum of the full output;
 * an all-reduce adds the t partials ("Tensor Parallelism Fundamentals",
 * section "Mechanics of Matrix Slicing"). Two such sums occur per layer,
 * after W_o and after the down projection. On one GPU the all-reduce is
 * replaced by tp_partial_sum over t partials held in device memory.
 *
 * Readings where the pages are silent: SwiGLU, silu(gate) * up, between the
 * gate/up and down projections; RMSNorm x * gamma / sqrt(mean(x^2) + eps) in
 * front of the column projections; decode attention with one query per
 * sequence, scale 1/sqrt(head_dim), no mask and no rotary embedding, query
 * head h reading kv head h / (n_q / n_kv); no biases.
 *
 * Conventions shared by every entry point
 *  - Memory. The caller owns and allocates all memory. Pointers named as
 *    device pointers refer to device memory of the current HIP device; the
 *    library never allocates, frees, synchronises or changes the device.
 *    Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *    and the call returns before it completes.
 *  - Layouts. Matrices are row-major. Activations are [m, features]. A
 *    weight is stored [out, in] with `in` (the contraction dimension K)
 *    contiguous. Row partials are float32. bf16 is IEEE bfloat16 bits;
 *    float32 and bf16 inputs are multiplied with float32 accumulation.
 *  - Alignment. Every device pointer must be 16-byte aligned and K a multiple
 *    of 8 (bf16) or 4 (float32), so that rows stream in 128-bit loads.
 *  - Workspace. Entry points with `ws` need device scratch memory of at least
 *    the size the matching *_workspace_bytes function returns (0 means `ws`
 *    may be NULL), 256-byte aligned. Its first TP_WORKSPACE_HEADER bytes hold
 *    completion counters that every entry point shares: the caller zero-fills
 *    them once, before the first use, and every call leaves them zero again.
 *    Scratch data lives only after the header, so one workspace, sized for the
 *    largest call, serves calls of any shape in sequence without clearing.
 *    Calls sharing one workspace must not overlap in time (same stream, or
 *    ordered by events).
 *  - Errors. Arguments are validated on the host before anything is
 *    enqueued; on failure nothing is enqueued and a tp_status other than
 *    TP_OK is returned. tp_last_error() then gives a thread-local message
 *    naming the argument and a hint for the fix. A failed HIP launch returns
 *    TP_ERR_HIP with the HIP error name in that message.
 *  - Determinism. No floating-point atomics are used: repeated calls on the
 *    same inputs give bitwise identical outputs.
 */
#ifndef TP_SHARD_H
#define TP_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tp_dtype { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

/* Bytes of shared completion counters at the start of every workspace. */
#define TP_WORKSPACE_HEADER 32768

/* Bytes of the per-GPU scratch tp_layer_shard_forward_static uses (16 MiB). */
#define TP_STATIC_SCRATCH_BYTES 16777216

typedef enum tp_status {
    TP_OK = 0,
    TP_ERR_NULL = 1,        /* a required pointer is NULL */
    TP_ERR_SHAPE = 2,       /* a size is zero, negative or beyond a supported limit */
    TP_ERR_INDIVISIBLE = 3, /* t does not divide the heads or intermediate size, or n_q % n_kv != 0 */
    TP_ERR_RANK = 4,        /* t outside 1..8, or rank outside 0..t-1 */
    TP_ERR_DTYPE = 5,       /* dtype not supported by this entry point */
    TP_ERR_ALIGN = 6,       /* a pointer not 16-byte aligned, or K not a multiple of the 128-bit vector */
    TP_ERR_WORKSPACE = 7,   /* workspace NULL, misaligned or smaller than required */
    TP_ERR_KV = 8,          /* kv_len outside 1..capacity */
    TP_ERR_ALIAS = 9,       /* an output range overlaps an input range */
    TP_ERR_HIP = 10         /* a HIP launch failed */
} tp_status;

/* A layer's unsharded shape. n_q_heads = 0 means no attention block,
 * intermediate = 0 no MLP block. n_layers, seq_len, batch and bytes_per_elem
 * only feed the footprints of tp_shard_plan. */
typedef struct tp_model_desc {
    int64_t hidden;          /* H */
    int64_t intermediate;    /* I */
    int32_t n_q_heads;       /* n_q */
    int32_t n_kv_heads;      /* n_kv */
    int32_t head_dim;        /* d */
    int32_t n_layers;        /* L */
    int64_t seq_len;         /* cached tokens per sequence S */
    int64_t batch;           /* sequences B */
    int32_t bytes_per_elem;  /* bytes per cached element */
    float eps;               /* RMSNorm epsilon */
} tp_model_desc;

/* What one rank owns. Blocks are contiguous and in rank order. */
typedef struct tp_rank_plan {
    int32_t t, rank;
    int32_t q_head_begin, q_heads;    /* q heads [q_head_begin, q_head_begin + q_heads) */
    int32_t kv_head_begin, kv_heads;  /* kv heads, likewise */
    int64_t inter_begin, inter_cols;  /* intermediate columns of gate, up and rows of down */
    int64_t qkv_cols;                 /* (q_heads + 2 kv_heads) * d: rows of this rank's W_qkv */
    int64_t o_rows;                   /* q_heads * d: the K of this rank's W_o */
    int64_t weight_elems;             /* this rank's projection weights, one layer (norms excluded) */
    int64_t kv_elems_per_seq_all_layers; /* 2 L n_kv d S: one sequence, all layers, unsharded */
    int64_t kv_bytes_rank;            /* 2 L n_kv d S bytes_per_elem B / t (/ n_kv when replicated) */
} tp_rank_plan;

/*
 * tp_shard_plan - what rank `rank` of `t` owns ("Tensor parallel scaling
 * curves", section "What tensor parallelism actually splits": the rank holds
 * heads[rank*h_per_gpu : (rank+1)*h_per_gpu]; "Tensor Parallelism
 * Fundamentals", section "Memory Overhead and Communication Bottlenecks":
 * weights and KV cache per GPU are the totals divided by t).
 * Host only; touches no device. Intermediate columns follow the same
 * contiguous rank order as heads; t must divide n_q and I, and either divide
 * n_kv or be a multiple of it (TP_ERR_INDIVISIBLE); 1 <= t <= 8 and
 * 0 <= rank < t (TP_ERR_RANK). When t > n_kv every rank keeps a copy of the
 * one kv head its q heads read (kv_heads = 1, head rank / (t / n_kv)), and
 * its KV cache is that head's: the total divided by n_kv, not by t.
 */
tp_status tp_shard_plan(const tp_model_desc* desc, int32_t t, int32_t rank, tp_rank_plan* out);

/* Flags for tp_linear_workspace_bytes. */
#define TP_LINEAR_SWIGLU 1   /* column projection with fused SwiGLU (w_up given) */
#define TP_LINEAR_NORM   2   /* column projection with fused RMSNorm (gamma given) */

/* Workspace bytes tp_column_linear / tp_row_linear_partial need for these sizes. */
size_t tp_linear_workspace_bytes(int64_t m, int64_t k, int64_t n, tp_dtype dtype, int32_t flags);

/*
 * tp_column_linear - column-parallel projection ("Tensor Parallelism
 * Fundamentals", section "Mechanics of Matrix Slicing": the weight is split
 * by columns, the input is replicated, each GPU computes its slice of output
 * columns with no communication).
 *   u = gamma ? RMSNorm(x; gamma, eps) : x
 *   y = w_up ? silu(u @ w^T) * (u @ w_up^T)  :  u @ w^T
 * x      device [m, k] activations (dtype)
 * w      device [n, k] this rank's column block, stored [out, in] (dtype)
 * w_up   device [n, k] or NULL: the paired up projection; enables fused SwiGLU
 * gamma  device [k] or NULL: RMSNorm scale; enables fused RMSNorm
 * y      device [m, n] output (dtype)
 * ws     workspace of tp_linear_workspace_bytes(m, k, n, dtype, flags)
 * Errors: TP_ERR_NULL (x, w, y), TP_ERR_SHAPE (m, k, n < 1), TP_ERR_ALIGN,
 * TP_ERR_WORKSPACE, TP_ERR_ALIAS (y overlaps x, w, w_up or gamma), TP_ERR_DTYPE.
 */
tp_status tp_column_linear(const void* x, const void* w, const void* w_up, const void* gamma, float eps,
                           void* y, int64_t m, int64_t k, int64_t n, tp_dtype dtype,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * tp_swiglu - the rank-local gating between the column-parallel gate/up and
 * the row-parallel down projection: out = silu(gate) * up, silu(z) = z /
 * (1 + e^-z), elementwise over [m, n]. The pages name the gate and up
 * projections ("Tensor parallel scaling curves", section "What tensor
 * parallelism actually splits"); the gating itself is the SwiGLU reading.
 * gate, up, out: device [m, n] (dtype). out may equal gate or up (in place);
 * any other overlap is TP_ERR_ALIAS.
 */
tp_status tp_swiglu(const void* gate, const void* up, void* out, int64_t m, int64_t n, tp_dtype dtype,
                    void* stream);

/*
 * tp_row_linear_partial - row-parallel projection ("Tensor Parallelism
 * Fundamentals", section "Mechanics of Matrix Slicing": the weight is split
 * by rows, the column-parallel output is fed in directly, each GPU yields a
 * partial sum of the full output).
 *   partial = a @ w^T, float32
 * a       device [m, k] this rank's column-parallel output (dtype)
 * w       device [n, k] this rank's row block, stored [out, in] (dtype)
 * partial device [m, n] float32
 * ws      workspace of tp_linear_workspace_bytes(m, k, n, dtype, 0)
 */
tp_status tp_row_linear_partial(const void* a, const void* w, float* partial, int64_t m, int64_t k, int64_t n,
                                tp_dtype dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * tp_partial_sum - the value the all-reduce after a row-parallel projection
 * returns ("Tensor parallel scaling curves", section "What tensor parallelism
 * actually splits": the row-wise splits need an all-reduce to sum the
 * partial results), computed on one device:
 *   out = sum_{r=0}^{t-1} partials[r]  (+ residual), in rank order, float32.
 * partials  host array of t device pointers, each [m, n] float32, 1 <= t <= 8
 * residual  device [m, n] (out_dtype) or NULL; added once, after the sum
 * out       device [m, n] (out_dtype); must not overlap any partial
 */
tp_status tp_partial_sum(const float* const* partials, int32_t t, const void* residual, void* out,
                         int64_t m, int64_t n, tp_dtype out_dtype, void* stream);

/*
 * bf16 partials. The partial sums a row-parallel projection emits are what
 * the all-reduce moves ("Tensor parallel scaling curves", section "What
 * tensor parallelism actually splits"; the bandwidth term of "The scaling
 * math" is proportional to the message bytes). Emitting them in bf16 halves
 * that message; the sum still adds in float32.
 *
 * tp_row_linear_partial_bf16 - as tp_row_linear_partial with bf16 a, w and
 *   partial: partial = bf16(a @ w^T). ws: tp_linear_workspace_bytes(m, k, n,
 *   TP_BF16, 0). k must be a multiple of 8 (TP_ERR_ALIGN).
 * tp_partial_sum_bf16 - as tp_partial_sum over t bf16 partials:
 *   out = sum_r float32(partials[r]) (+ residual), in rank order.
 */
tp_status tp_row_linear_partial_bf16(const void* a, const void* w, void* partial, int64_t m, int64_t k,
                                     int64_t n, void* ws, size_t ws_bytes, void* stream);
tp_status tp_partial_sum_bf16(const void* const* partials, int32_t t, const void* residual, void* out,
                              int64_t m, int64_t n, tp_dtype out_dtype, void* stream);

/* Workspace bytes of tp_decode_attention. */
size_t tp_attention_workspace_bytes(int64_t batch, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                                    int64_t kv_len);

/*
 * tp_decode_attention - attention over the heads this rank owns ("Tensor
 * parallel scaling curves", section "What tensor parallelism actually
 * splits": local attention on owned heads, no communication). For sequence
 * b and owned query head h with kv head g = h / (q_heads / kv_heads):
 *   o[b, h] = sum_j softmax_j(q[b, h] . K[b, g, j] / sqrt(d)) V[b, g, j],
 *   j = 0 .. kv_len - 1.
 * q      device [batch, q_heads * d] bf16
 * k, v   device [batch, kv_heads, capacity, d] bf16 caches
 * out    device [batch, q_heads * d] bf16
 * d must be 64 or 128; q_heads / kv_heads at most 16 (TP_ERR_SHAPE);
 * 1 <= kv_len <= capacity (TP_ERR_KV). bf16 only (TP_ERR_DTYPE).
 */
tp_status tp_decode_attention(const void* q, const void* k, const void* v, void* out, int64_t batch,
                              int32_t q_heads, int32_t kv_heads, int32_t head_dim, int64_t capacity,
                              int64_t kv_len, tp_dtype dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * tp_prefill_attention - causal attention over the heads this rank owns for
 * a block of seq new tokens ("Tensor parallel scaling curves", section "What
 * tensor parallelism actually splits": local attention on owned heads, no
 * communication; causal masking is the standard decoder rule, token at
 * position p sees positions 0..p). Token i of sequence b sits at position
 * p = kv_len - seq + i and its k, v are already in the caches. For owned
 * query head h with kv head g = h / (q_heads / kv_heads):
 *   o[b, i, h] = sum_j softmax_j(q[b, i, h] . K[b, g, j] / sqrt(d)) V[b, g, j],
 *   j = 0 .. p.
 * q      device [batch, seq, q_heads * d] bf16
 * k, v   device [batch, kv_heads, capacity, d] bf16 caches
 * out    device [batch, seq, q_heads * d] bf16; must not overlap q or the caches
 * d must be 64 or 128, q_heads / kv_heads one of 1, 2, 4, 8, 16, batch and
 * kv_heads at most 65535 (TP_ERR_SHAPE); 1 <= seq <= kv_len <= capacity
 * (TP_ERR_KV). bf16 only
 * (TP_ERR_DTYPE). Needs no workspace.
 */
tp_status tp_prefill_attention(const void* q, const void* k, const void* v, void* out, int64_t batch,
                               int64_t seq, int32_t q_heads, int32_t kv_heads, int32_t head_dim,
                               int64_t capacity, int64_t kv_len, tp_dtype dtype, void* stream);

typedef enum tp_stage { TP_STAGE_ATTN = 0, TP_STAGE_MLP = 1 } tp_stage;

/* One rank's weights for one layer, all device pointers, stored [out, in]. */
typedef struct tp_rank_weights {
    const void* attn_norm;  /* [H] gamma in front of QKV, or NULL for no norm */
    const void* w_qkv;      /* [qkv_cols, H]: this rank's Q rows, then K rows, then V rows */
    const void* w_o;        /* [H, o_rows] */
    const void* mlp_norm;   /* [H] gamma in front of gate/up, or NULL */
    const void* w_gate;     /* [inter_cols, H] */
    const void* w_up;       /* [inter_cols, H] */
    const void* w_down;     /* [H, inter_cols] */
} tp_rank_weights;

/* This rank's KV cache for one layer: k, v device [batch, kv_heads, capacity, d]. */
typedef struct tp_kv_view {
    void* k;
    void* v;
    int64_t capacity;
    int64_t kv_len;          /* keys attended over, the new tokens included */
    int64_t new_tokens;      /* new tokens per sequence: 0 or 1 for a decode step, S > 1 for a
                                block of S tokens at positions kv_len - S .. kv_len - 1 */
} tp_kv_view;

/* Workspace bytes of tp_layer_shard_forward for this stage and m. */
size_t tp_layer_workspace_bytes(const tp_model_desc* desc, const tp_rank_plan* plan, tp_stage stage,
                                int64_t m, tp_dtype dtype);

/*
 * tp_layer_shard_forward - one rank's share of one block of the layer,
 * ending in the row-parallel partial that the all-reduce would sum ("Tensor
 * parallel scaling curves", section "What tensor parallelism actually
 * splits", pseudocode for the attention block and the two all-reduces per
 * layer).
 * TP_STAGE_ATTN (bf16): u = RMSNorm(in; attn_norm); [q|k|v] = u @ W_qkv^T.
 *   Decode (kv->new_tokens 0 or 1; m is the batch, one new token per
 *   sequence): the new k, v are written to the cache at position kv_len - 1
 *   and o = decode attention over the owned heads. Prefill (new_tokens =
 *   S > 1; m = batch * S rows, sequence-major): the block's k, v are written
 *   to positions kv_len - S .. kv_len - 1 and o = causal prefill attention
 *   over the owned heads (as tp_prefill_attention), with S <= kv_len and at
 *   most 65535 sequences (TP_ERR_KV / TP_ERR_SHAPE). Then
 *   partial = o @ W_o^T. A prefill block of one token is a decode step.
 * TP_STAGE_MLP (bf16 or float32, any m): u = RMSNorm(in; mlp_norm);
 *   a = silu(u @ W_gate^T) * (u @ W_up^T); partial = a @ W_down^T.
 * in       device [m, H] (dtype): x for ATTN; h = x + sum of attention
 *          partials for MLP
 * kv       ATTN only: this rank's cache view; ignored (may be NULL) for MLP
 * partial  device [m, H] float32
 * The caller sums the t ranks' partials with tp_partial_sum.
 */
tp_status tp_layer_shard_forward(const tp_model_desc* desc, const tp_rank_plan* plan, tp_stage stage,
                                 const tp_rank_weights* weights, const void* in, const tp_kv_view* kv,
                                 float* partial, int64_t m, tp_dtype dtype, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * tp_layer_shard_forward_static - tp_layer_shard_forward for callers that
 * cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation and kernels, with
 * the workspace taken from a library-owned device array of
 * TP_STATIC_SCRATCH_BYTES per GPU instead of a caller's buffer. It calls no
 * allocating routine. The caller still passes inputs and outputs.
 * - A call whose workspace (tp_layer_workspace_bytes) exceeds
 *   TP_STATIC_SCRATCH_BYTES returns TP_ERR_WORKSPACE before any HIP call.
 *   Decode stages of the 70B-shaped layer at t=8 over 16 sequences need
 *   about 2 MB; long prefill blocks need more and take the workspace entry
 *   point.
 * - The first call on a device looks the array up with that device current
 *   and enqueues one small kernel on the caller's stream that zeroes its
 *   counter header; every call leaves the header zero again.
 * - Every call on one GPU shares that GPU's array: calls that overlap in time
 *   on one GPU (different streams without ordering, or several host threads)
 *   race on it and must not be issued.
 */
tp_status tp_layer_shard_forward_static(const tp_model_desc* desc, const tp_rank_plan* plan, tp_stage stage,
                                        const tp_rank_weights* weights, const void* in, const tp_kv_view* kv,
                                        float* partial, int64_t m, tp_dtype dtype, void* stream);

/*
 * Mixture of experts. "Tensor Parallelism Fundamentals", section "Sizing
 * Heuristics and Limits": for a mixture-of-experts model tensor parallelism
 * shards the expert feed-forward layers as well as attention. Each expert's
 * FFN is split like the dense MLP: this rank holds the same column block of
 * every expert's gate and up projections and the matching row block of its
 * down projection. The router is replicated on every rank.
 *
 * One rank's MoE FFN (bf16, float32 accumulation):
 *   u = RMSNorm(x; norm) (or x when norm is NULL)
 *   logits = u @ W_router^T                       [m, E] float32
 *   gates  = top_k of each row of logits (ties to the lower expert), softmax
 *            over the selected logits, 0 for the other experts
 *   a_e = gates[:, e] * silu(u @ W_gate_e^T) * (u @ W_up_e^T)
 *   partial = sum_e a_e @ W_down_e^T              [m, H] float32
 * The caller sums the t ranks' partials with tp_partial_sum; all ranks must
 * see the same gates (the router weights are identical on every rank).
 * Experts a token is not routed to carry gate 0, so the result is the sum
 * over its top_k experts. Up to 64 tokens (a decode batch) every expert is
 * computed for every token (its weights are read anyway); above that, with
 * top_k <= 8, each expert runs only over the tokens routed to it (grouped
 * GEMMs over per-expert token lists: top_k / E of the dense flops), and a
 * token's top_k expert outputs are added in expert order.
 */
typedef struct tp_moe_weights {
    const void* norm;      /* [H] gamma in front of the router and experts, or NULL */
    const void* w_router;  /* [E, H] */
    const void* w_gate;    /* [E * inter_cols, H]: expert e's rows e*inter_cols .. (e+1)*inter_cols - 1 */
    const void* w_up;      /* [E * inter_cols, H], stacked the same way */
    const void* w_down;    /* [H, E * inter_cols]: expert e's columns e*inter_cols .. (e+1)*inter_cols - 1 */
} tp_moe_weights;

/* Workspace bytes of tp_moe_shard_forward (has_norm: weights->norm != NULL);
 * 0 for invalid sizes. */
size_t tp_moe_workspace_bytes(int64_t m, int64_t hidden, int32_t n_experts, int32_t top_k, int64_t inter_cols,
                              int32_t has_norm);

/*
 * tp_moe_shard_forward - the MoE FFN above for m tokens x [m, hidden] (bf16).
 * partial     device [m, hidden] float32
 * gates_out   device [m, n_experts] float32, or NULL
 * logits_out  device [m, n_experts] float32, or NULL
 * 1 <= n_experts <= 64, 1 <= top_k <= n_experts (TP_ERR_SHAPE); hidden and
 * inter_cols (this rank's columns of one expert, intermediate / t) multiples
 * of 8 (TP_ERR_ALIGN).
 */
tp_status tp_moe_shard_forward(const tp_moe_weights* weights, const void* x, float* partial, float* gates_out,
                               float* logits_out, int64_t m, int64_t hidden, int32_t n_experts, int32_t top_k,
                               int64_t inter_cols, float eps, void* ws, size_t ws_bytes, void* stream);

/*
 * tp_hbm_stream_read - measurement helper, not a step of the layer: reads
 * bytes of device memory at buf once with 128-bit non-temporal loads (the
 * practical HBM read rate a decode projection's weight stream is compared
 * with; "Tensor parallel scaling curves", The scaling math: decode is bound by
 * reading the weights). flag: device, 4 bytes, written only in the unlikely
 * case that the folded words equal never. bytes must be a positive multiple
 * of 16 (TP_ERR_SHAPE); buf and flag 16-byte aligned (TP_ERR_ALIGN).
 */
tp_status tp_hbm_stream_read(const void* buf, size_t bytes, void* flag, uint32_t never, void* stream);

/* Name of a status code, e.g. "TP_ERR_SHAPE". */
const char* tp_status_name(tp_status status);

/* Thread-local message of the last failing call on this thread ("" if none). */
const char* tp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TP_SHARD_H */
