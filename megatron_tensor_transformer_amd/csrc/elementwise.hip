// Bandwidth-bound elementwise kernels: the on-device sum of the t row-parallel
// partials (the value the all-reduce returns), standalone SwiGLU, the
// row-wise RMSNorm used in front of the prefill GEMM, and the append of a
// block of tokens' k, v to the cache. All use 128-bit loads
// and grid-stride loops sized to a few workgroups per compute unit.
#include "device_common.h"
#include "kernels.h"

namespace tpk {

constexpr int EW_THREADS = 256;

static int ew_blocks(int64_t items) {
    int64_t b = (items + EW_THREADS - 1) / EW_THREADS;
    if (b > 256 * 8) b = 256 * 8;
    if (b < 1) b = 1;
    return (int)b;
}

// Sum of partials: each thread handles 4 elements of every partial (one
// 128-bit float32 or 64-bit bf16 load from each), added in float32 in rank
// order, then the residual.
template <bool IN_BF16>
__device__ __forceinline__ float4 load4(const void* p, int64_t i) {
    if (IN_BF16) {
        const uint2 v = reinterpret_cast<const uint2*>(p)[i];
        return make_float4(bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y));
    }
    return reinterpret_cast<const float4*>(p)[i];
}
template <bool IN_BF16>
__device__ __forceinline__ float load1(const void* p, int64_t i) {
    if (IN_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
    return reinterpret_cast<const float*>(p)[i];
}

template <bool IN_BF16, bool OUT_BF16>
__global__ __launch_bounds__(EW_THREADS) void partial_sum_kernel(PartialPtrs ps, int t, const void* residual,
                                                                 void* out, int64_t count) {
    const int64_t n4 = count / 4;
    const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
    for (int64_t i = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; i < n4; i += stride) {
        // every partial requested before the first add; added in rank order
        float4 v[8];
#pragma unroll
        for (int r = 0; r < 8; ++r)
            if (r < t) v[r] = load4<IN_BF16>(ps.p[r], i);
        float4 acc = v[0];
#pragma unroll
        for (int r = 1; r < 8; ++r)
            if (r < t) { acc.x += v[r].x; acc.y += v[r].y; acc.z += v[r].z; acc.w += v[r].w; }
        if (OUT_BF16) {
            if (residual) {
                const uint2 rv = reinterpret_cast<const uint2*>(residual)[i];
                acc.x += bf16lo(rv.x); acc.y += bf16hi(rv.x); acc.z += bf16lo(rv.y); acc.w += bf16hi(rv.y);
            }
            uint2 o;
            o.x = pack_bf16x2(acc.x, acc.y);
            o.y = pack_bf16x2(acc.z, acc.w);
            reinterpret_cast<uint2*>(out)[i] = o;
        } else {
            if (residual) {
                const float4 rv = reinterpret_cast<const float4*>(residual)[i];
                acc.x += rv.x; acc.y += rv.y; acc.z += rv.z; acc.w += rv.w;
            }
            reinterpret_cast<float4*>(out)[i] = acc;
        }
    }
    // tail (count not a multiple of 4)
    const int64_t tail0 = n4 * 4;
    for (int64_t i = tail0 + (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; i < count; i += stride) {
        float acc = load1<IN_BF16>(ps.p[0], i);
        for (int r = 1; r < t; ++r) acc += load1<IN_BF16>(ps.p[r], i);
        if (OUT_BF16) {
            if (residual) acc += bf16_to_f32(reinterpret_cast<const uint16_t*>(residual)[i]);
            reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_bf16_bits(acc);
        } else {
            if (residual) acc += reinterpret_cast<const float*>(residual)[i];
            reinterpret_cast<float*>(out)[i] = acc;
        }
    }
}

hipError_t partial_sum_launch(const PartialPtrs& ps, int t, const void* residual, void* out, int64_t count,
                              int in_bf16, int out_bf16, hipStream_t s) {
    const int blocks = ew_blocks((count + 3) / 4);
    if (in_bf16 && out_bf16)
        hipLaunchKernelGGL((partial_sum_kernel<true, true>), dim3(blocks), dim3(EW_THREADS), 0, s, ps, t, residual, out, count);
    else if (in_bf16)
        hipLaunchKernelGGL((partial_sum_kernel<true, false>), dim3(blocks), dim3(EW_THREADS), 0, s, ps, t, residual, out, count);
    else if (out_bf16)
        hipLaunchKernelGGL((partial_sum_kernel<false, true>), dim3(blocks), dim3(EW_THREADS), 0, s, ps, t, residual, out, count);
    else
        hipLaunchKernelGGL((partial_sum_kernel<false, false>), dim3(blocks), dim3(EW_THREADS), 0, s, ps, t, residual, out, count);
    return hipGetLastError();
}

template <bool BF16>
__global__ __launch_bounds__(EW_THREADS) void swiglu_kernel(const void* gate, const void* up, void* out,
                                                            int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
    if (BF16) {
        const int64_t n8 = count / 8;
        for (int64_t i = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; i < n8; i += stride) {
            const uint4 g = reinterpret_cast<const uint4*>(gate)[i];
            const uint4 u = reinterpret_cast<const uint4*>(up)[i];
            const uint32_t* gp = &g.x;
            const uint32_t* up_ = &u.x;
            uint4 o;
            uint32_t* op = &o.x;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                op[j] = pack_bf16x2(silu_f32(bf16lo(gp[j])) * bf16lo(up_[j]), silu_f32(bf16hi(gp[j])) * bf16hi(up_[j]));
            reinterpret_cast<uint4*>(out)[i] = o;
        }
        for (int64_t i = n8 * 8 + (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; i < count; i += stride) {
            const float g = bf16_to_f32(reinterpret_cast<const uint16_t*>(gate)[i]);
            const float u = bf16_to_f32(reinterpret_cast<const uint16_t*>(up)[i]);
            reinterpret_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_bf16_bits(silu_f32(g) * u);
        }
    } else {
        const int64_t n4 = count / 4;
        for (int64_t i = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; i < n4; i += stride) {
            const float4 g = reinterpret_cast<const float4*>(gate)[i];
            const float4 u = reinterpret_cast<const float4*>(up)[i];
            float4 o;
            o.x = silu_f32(g.x) * u.x; o.y = silu_f32(g.y) * u.y;
            o.z = silu_f32(g.z) * u.z; o.w = silu_f32(g.w) * u.w;
            reinterpret_cast<float4*>(out)[i] = o;
        }
        for (int64_t i = n4 * 4 + (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; i < count; i += stride) {
            const float g = reinterpret_cast<const float*>(gate)[i];
            reinterpret_cast<float*>(out)[i] = silu_f32(g) * reinterpret_cast<const float*>(up)[i];
        }
    }
}

hipError_t swiglu_launch(const void* gate, const void* up, void* out, int64_t count, int is_bf16, hipStream_t s) {
    const int blocks = ew_blocks((count + 7) / 8);
    if (is_bf16)
        hipLaunchKernelGGL(swiglu_kernel<true>, dim3(blocks), dim3(EW_THREADS), 0, s, gate, up, out, count);
    else
        hipLaunchKernelGGL(swiglu_kernel<false>, dim3(blocks), dim3(EW_THREADS), 0, s, gate, up, out, count);
    return hipGetLastError();
}

// One workgroup per row: sum of squares, then u = x * gamma * inv_rms.
template <bool BF16>
__global__ __launch_bounds__(EW_THREADS) void rmsnorm_kernel(const void* x, const void* gamma, void* u, int K,
                                                             float eps) {
    constexpr int VEC = BF16 ? 8 : 4;
    const int row = blockIdx.x;
    const int nv = K / VEC;
    __shared__ float wsum[EW_THREADS / 64];
    const uint4* xr = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(x) + (size_t)row * K * (BF16 ? 2 : 4));
    const uint4* gr = reinterpret_cast<const uint4*>(gamma);
    uint4* ur = reinterpret_cast<uint4*>(reinterpret_cast<char*>(u) + (size_t)row * K * (BF16 ? 2 : 4));
    float ss = 0.f;
    for (int c = threadIdx.x; c < nv; c += EW_THREADS) {
        const uint4 v = xr[c];
        const uint32_t* p = &v.x;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (BF16) {
                const float a = bf16lo(p[j]), b = bf16hi(p[j]);
                ss = fmaf(a, a, ss); ss = fmaf(b, b, ss);
            } else {
                const float a = __uint_as_float(p[j]);
                ss = fmaf(a, a, ss);
            }
        }
    }
    ss = group_sum<64>(ss);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < EW_THREADS / 64; ++w) tot += wsum[w];
    const float inv = 1.0f / sqrtf(tot / (float)K + eps);
    for (int c = threadIdx.x; c < nv; c += EW_THREADS) {
        const uint4 v = xr[c];
        const uint4 g = gr[c];
        const uint32_t* p = &v.x;
        const uint32_t* q = &g.x;
        uint4 o;
        uint32_t* op = &o.x;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (BF16) {
                op[j] = pack_bf16x2(bf16lo(p[j]) * inv * bf16lo(q[j]), bf16hi(p[j]) * inv * bf16hi(q[j]));
            } else {
                op[j] = __float_as_uint(__uint_as_float(p[j]) * inv * __uint_as_float(q[j]));
            }
        }
        ur[c] = o;
    }
}

hipError_t rmsnorm_launch(const void* x, const void* gamma, void* u, int m, int K, float eps, int is_bf16,
                          hipStream_t s) {
    if (is_bf16)
        hipLaunchKernelGGL(rmsnorm_kernel<true>, dim3(m), dim3(EW_THREADS), 0, s, x, gamma, u, K, eps);
    else
        hipLaunchKernelGGL(rmsnorm_kernel<false>, dim3(m), dim3(EW_THREADS), 0, s, x, gamma, u, K, eps);
    return hipGetLastError();
}

// Block KV append: the k and v columns of each token row of the projected
// [q | k | v] buffer go to cache positions pos0 .. pos0 + S - 1. A thread moves
// one 16-byte chunk of k and the matching chunk of v; consecutive threads
// take consecutive chunks of one row, so reads and writes are contiguous runs
// of a head's d elements.
__global__ __launch_bounds__(EW_THREADS) void kv_append_kernel(KvAppendArgs a) {
    const int dc = a.head_dim / 8;                 // chunks per head
    const int per_row = a.kv_heads * dc;
    const int64_t total = (int64_t)a.rows * per_row;
    const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(a.qkv);
    for (int64_t i = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / per_row;             // token row, sequence-major
        const int c = (int)(i - r * per_row);
        const int g = c / dc, off = (c - g * dc) * 8;
        const int64_t b = r / a.seq, t = r - b * a.seq;
        const uint16_t* row = src + r * a.row_stride + g * a.head_dim + off;
        const size_t dst = (((size_t)b * a.kv_heads + g) * a.capacity + a.pos0 + t) * a.head_dim + off;
        const uint4 k = load_u4(row + a.k_col0);
        const uint4 v = load_u4(row + a.v_col0);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.k_cache) + dst) = k;
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.v_cache) + dst) = v;
    }
}

hipError_t kv_append_launch(const KvAppendArgs& a, hipStream_t s) {
    const int blocks = ew_blocks((int64_t)a.rows * a.kv_heads * (a.head_dim / 8));
    hipLaunchKernelGGL(kv_append_kernel, dim3(blocks), dim3(EW_THREADS), 0, s, a);
    return hipGetLastError();
}

// Top-k routing of one token in one wave: lane e holds expert e's logit
// (lanes past E hold nothing). The k experts with the largest logits are
// chosen one at a time, the lowest index first among equal logits; their gates
// are the softmax of their logits (exponentials relative to the largest,
// added in expert order), every other gate 0.
__device__ __forceinline__ void route_wave(float l, int E, int top_k, float* logits_row, float* gates_row,
                                           int* slots_row = nullptr) {
    const int e = threadIdx.x & 63;
    const bool valid = e < E;
    bool chosen = false;
    float mx0 = 0.f;
    for (int j = 0; j < top_k; ++j) {
        float v = (valid && !chosen) ? l : -INFINITY;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
        const uint64_t cand = __ballot(valid && !chosen && l == v);
        const int best = __ffsll((unsigned long long)cand) - 1;
        chosen = chosen || e == best;
        if (j == 0) mx0 = v;
    }
    const float ex = chosen ? expf(l - mx0) : 0.f;
    const uint64_t chosen_mask = __ballot(chosen);
    uint64_t mask = chosen_mask;
    float den = 0.f;
    while (mask) {
        const int b = __ffsll((unsigned long long)mask) - 1;
        den += __shfl(ex, b, 64);
        mask &= mask - 1;
    }
    if (valid) {
        if (logits_row) logits_row[e] = l;
        gates_row[e] = chosen ? ex / den : 0.f;
        // rank of this expert among the chosen ones, in expert order
        if (slots_row) slots_row[e] = chosen ? __popcll(chosen_mask & ((1ull << e) - 1ull)) : -1;
    }
}

// Gates from float32 logits [m, E]: one wave per token.
__global__ __launch_bounds__(EW_THREADS) void moe_gates_kernel(const float* logits, float* gates, int* slots, int m,
                                                               int E, int top_k) {
    const int t = blockIdx.x * (EW_THREADS / 64) + (threadIdx.x >> 6);
    if (t >= m) return;                             // whole waves
    const int e = threadIdx.x & 63;
    const float l = e < E ? logits[(size_t)t * E + e] : 0.f;
    route_wave(l, E, top_k, nullptr, gates + (size_t)t * E, slots ? slots + (size_t)t * E : nullptr);
}

hipError_t moe_gates_launch(const float* logits, float* gates, int m, int E, int top_k, hipStream_t s, int* slots) {
    constexpr int per = EW_THREADS / 64;
    hipLaunchKernelGGL(moe_gates_kernel, dim3((m + per - 1) / per), dim3(EW_THREADS), 0, s, logits, gates, slots, m,
                       E, top_k);
    return hipGetLastError();
}

// Token lists per expert: one workgroup per expert walks the tokens in order,
// 256 at a time; the routed ones are compacted by a ballot, the lanes below in
// the wave (mbcnt) and the waves before in the workgroup, so the list is in
// ascending token order.
__global__ __launch_bounds__(EW_THREADS) void moe_lists_kernel(const int* slots, int* lists, int* counts, int m,
                                                               int E) {
    constexpr int NW = EW_THREADS / 64;
    __shared__ int wave_n[NW];
    const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int* list = lists + (size_t)e * m;
    int base = 0;
    for (int t0 = 0; t0 < m; t0 += EW_THREADS) {
        const int t = t0 + tid;
        const bool sel = t < m && slots[(size_t)t * E + e] >= 0;
        const uint64_t bal = __ballot(sel);
        const int below = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 0) wave_n[wave] = __popcll(bal);
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            before += w < wave ? wave_n[w] : 0;
            total += wave_n[w];
        }
        if (sel) list[base + before + below] = t;
        base += total;
        __syncthreads();
    }
    if (tid == 0) counts[e] = base;
}

hipError_t moe_lists_launch(const int* slots, int* lists, int* counts, int m, int E, hipStream_t s) {
    hipLaunchKernelGGL(moe_lists_kernel, dim3(E), dim3(EW_THREADS), 0, s, slots, lists, counts, m, E);
    return hipGetLastError();
}

// Router logits and gates of a few tokens in one launch: one workgroup per
// token forms its E logits (u[t] . W_router[e], bf16 products summed in
// float32: each thread over 8-element chunks tid, tid + 256, ..., then the
// wave's lanes, then the 4 waves in order) and its first wave routes them.
template <int EM>
__global__ __launch_bounds__(EW_THREADS) void moe_router_kernel(const uint16_t* u, const uint16_t* w, float* logits,
                                                                float* gates, int H, int E, int top_k) {
    __shared__ float red[EW_THREADS / 64][EM];
    const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint16_t* x = u + (size_t)t * H;
    float acc[EM];
#pragma unroll
    for (int e = 0; e < EM; ++e) acc[e] = 0.f;
    for (int c = tid; c < H / 8; c += EW_THREADS) {
        const uint4 xv = reinterpret_cast<const uint4*>(x)[c];
#pragma unroll
        for (int e = 0; e < EM; ++e) {
            if (e < E) {
                const uint4 wv = reinterpret_cast<const uint4*>(w + (size_t)e * H)[c];
                acc[e] = dot2_bf16(xv.x, wv.x, acc[e]);
                acc[e] = dot2_bf16(xv.y, wv.y, acc[e]);
                acc[e] = dot2_bf16(xv.z, wv.z, acc[e]);
                acc[e] = dot2_bf16(xv.w, wv.w, acc[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < EM; ++e) {
        if (e < E) {
            float v = acc[e];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            if (lane == 0) red[wave][e] = v;
        }
    }
    __syncthreads();
    if (wave != 0) return;
    float l = 0.f;
    if (lane < E) {
#pragma unroll
        for (int wv = 0; wv < EW_THREADS / 64; ++wv) l += red[wv][lane];
    }
    route_wave(l, E, top_k, logits + (size_t)t * E, gates + (size_t)t * E);
}

hipError_t moe_router_launch(const void* u, const void* w_router, float* logits, float* gates, int m, int H, int E,
                             int top_k, hipStream_t s) {
    const uint16_t* uu = reinterpret_cast<const uint16_t*>(u);
    const uint16_t* ww = reinterpret_cast<const uint16_t*>(w_router);
    if (E <= 8)
        hipLaunchKernelGGL(moe_router_kernel<8>, dim3(m), dim3(EW_THREADS), 0, s, uu, ww, logits, gates, H, E, top_k);
    else if (E <= 16)
        hipLaunchKernelGGL(moe_router_kernel<16>, dim3(m), dim3(EW_THREADS), 0, s, uu, ww, logits, gates, H, E, top_k);
    else if (E <= 32)
        hipLaunchKernelGGL(moe_router_kernel<32>, dim3(m), dim3(EW_THREADS), 0, s, uu, ww, logits, gates, H, E, top_k);
    else
        hipLaunchKernelGGL(moe_router_kernel<64>, dim3(m), dim3(EW_THREADS), 0, s, uu, ww, logits, gates, H, E, top_k);
    return hipGetLastError();
}

// a[t, e * cols + i] *= gates[t, e] in place (bf16), 8 elements per thread.
__global__ __launch_bounds__(EW_THREADS) void moe_scale_kernel(uint16_t* a, const float* gates, int m, int E,
                                                               int64_t cols) {
    const int64_t row8 = (int64_t)E * cols / 8;
    const int64_t total = (int64_t)m * row8;
    const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
    for (int64_t i = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; i < total; i += stride) {
        const int64_t t = i / row8;
        const int e = (int)((i - t * row8) * 8 / cols);
        const float w = gates[t * E + e];
        uint4 v = reinterpret_cast<const uint4*>(a)[i];
        uint32_t* p = &v.x;
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = pack_bf16x2(bf16lo(p[j]) * w, bf16hi(p[j]) * w);
        reinterpret_cast<uint4*>(a)[i] = v;
    }
}

hipError_t moe_scale_launch(void* a, const float* gates, int m, int E, int64_t cols, hipStream_t s) {
    const int blocks = ew_blocks((int64_t)m * E * cols / 8);
    hipLaunchKernelGGL(moe_scale_kernel, dim3(blocks), dim3(EW_THREADS), 0, s, reinterpret_cast<uint16_t*>(a), gates,
                       m, E, cols);
    return hipGetLastError();
}

}  // namespace tpk

namespace tpk {

// Plain streaming read of a buffer, the reference point for the decode
// kernels' bandwidth: every lane keeps SR_UNR 128-bit non-temporal loads in
// flight over a grid-stride loop and folds them into one word. The word is
// stored only if it equals a value the caller passes and never expects, so
// the loads stay live and the kernel writes (almost) nothing.
constexpr int SR_UNR = 8;

__global__ __launch_bounds__(EW_THREADS) void stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                                 unsigned* out, unsigned never) {
    const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
    int64_t i = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x;
    unsigned acc = 0;
    for (; i + (SR_UNR - 1) * stride < n16; i += SR_UNR * stride) {
        uint4 v[SR_UNR];
#pragma unroll
        for (int u = 0; u < SR_UNR; ++u) v[u] = load_stream_u4(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < SR_UNR; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = load_stream_u4(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == never) out[0] = acc;
}

hipError_t stream_read_launch(const void* buf, int64_t n16, unsigned* out, unsigned never, hipStream_t s) {
    int64_t blocks = (n16 + (int64_t)EW_THREADS * SR_UNR - 1) / ((int64_t)EW_THREADS * SR_UNR);
    if (blocks > 256 * 16) blocks = 256 * 16;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(EW_THREADS), 0, s,
                       reinterpret_cast<const uint4*>(buf), n16, out, never);
    return hipGetLastError();
}

}  // namespace tpk

namespace tpk {

// Zero n16 128-bit words with vector stores (a kernel, so a caller may
// capture it in a graph).
__global__ __launch_bounds__(EW_THREADS) void fill_zero_kernel(uint4* p, int64_t n16) {
    const int64_t stride = (int64_t)gridDim.x * EW_THREADS;
    for (int64_t i = (int64_t)blockIdx.x * EW_THREADS + threadIdx.x; i < n16; i += stride)
        p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t fill_zero_launch(void* p, size_t bytes, hipStream_t s) {
    const int64_t n16 = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(ew_blocks(n16)), dim3(EW_THREADS), 0, s, reinterpret_cast<uint4*>(p),
                       n16);
    return hipGetLastError();
}

}  // namespace tpk
