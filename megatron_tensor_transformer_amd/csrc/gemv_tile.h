// Shared end of the decode projections: the split-K merge of a workgroup's
// result tile and the epilogues (store, float32 partial, SwiGLU, QKV with
// KV-cache append). Device code; included by the projection kernels only.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace tpk {

struct GemvDev {
    GemvArgs a;
    int kc, splits, n_tiles;
    int opt;           // outputs per tile
    int mb0;           // first m-block of this launch
    int tile0;         // first row tile of this launch (v_dot2 kernel)
    float* part;       // [tiles*mblocks][S][MT*RPT], tiles and m-blocks of one launch
    float* ssq;        // [tiles*mblocks][S][MT]
    unsigned* cnt;     // [tiles*mblocks]
};

// Matrix-core variant (gemv_mfma.hip); same workspace layout as the v_dot2 kernel.
hipError_t gemv_mfma_launch(const GemvDev& d, const GemvPlan& p, hipStream_t s);

__device__ __forceinline__ void store_out(void* y, size_t idx, float v, uint16_t*) {
    reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)f32_to_bf16_bits(v);
}
__device__ __forceinline__ void store_out(void* y, size_t idx, float v, float*) {
    reinterpret_cast<float*>(y)[idx] = v;
}

// Sum of squares of a vector and the vector scaled by gamma (rounded back to T).
__device__ __forceinline__ float vsumsq(const uint4& v, uint16_t*) {
    float s = 0.f;
    const uint32_t* p = &v.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float a = bf16lo(p[i]), b = bf16hi(p[i]);
        s = fmaf(a, a, s);
        s = fmaf(b, b, s);
    }
    return s;
}
__device__ __forceinline__ float vsumsq(const uint4& v, float*) {
    const uint32_t* p = &v.x;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s = fmaf(__uint_as_float(p[i]), __uint_as_float(p[i]), s);
    return s;
}
__device__ __forceinline__ uint4 vscale(const uint4& v, const uint4& g, uint16_t*) {
    uint4 r;
    const uint32_t* a = &v.x;
    const uint32_t* b = &g.x;
    uint32_t* o = &r.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(bf16lo(a[i]) * bf16lo(b[i]), bf16hi(a[i]) * bf16hi(b[i]));
    return r;
}
__device__ __forceinline__ uint4 vscale(const uint4& v, const uint4& g, float*) {
    uint4 r;
    r.x = __float_as_uint(__uint_as_float(v.x) * __uint_as_float(g.x));
    r.y = __float_as_uint(__uint_as_float(v.y) * __uint_as_float(g.y));
    r.z = __float_as_uint(__uint_as_float(v.z) * __uint_as_float(g.z));
    r.w = __float_as_uint(__uint_as_float(v.w) * __uint_as_float(g.w));
    return r;
}

// The epilogue of one output tile: res[m][RPT] are the full K sums of the
// tile's rows for tokens m < mvalid (for SwiGLU the gate rows first, then the
// up rows of the same outputs), ssl[m] the activations' sums of squares when
// RMSNorm is fused. A tile holds opt outputs (at most RPT, or RPT / 2 for
// SwiGLU; rows past them are padding).
template <typename T, int MT, int RPT, int EPI, bool NORM, int NT>
__device__ __forceinline__ void gemv_epilogue(const GemvArgs& a, const float* res, const float* ssl, int tile, int m0,
                                              int mvalid, int opt = EPI == EPI_SWIGLU ? RPT / 2 : RPT) {
    constexpr bool SWI = (EPI == EPI_SWIGLU);
    constexpr int HALF = RPT / 2;
    constexpr int OUTS = SWI ? HALF : RPT;
    const int tid = threadIdx.x;
    const int N = a.N;
    for (int i = tid; i < mvalid * OUTS; i += NT) {
        const int m = i / OUTS, o = i - m * OUTS;
        if (o >= opt) continue;
        const float inv = NORM ? 1.0f / sqrtf(ssl[m] / (float)a.K + a.eps) : 1.0f;
        const int row = m0 + m;
        if (SWI) {
            const int n = tile * opt + o;
            if (n < N) {
                const float g = res[m * RPT + o] * inv;
                const float u = res[m * RPT + HALF + o] * inv;
                store_out(a.y, (size_t)row * N + n, silu_f32(g) * u, (T*)nullptr);
            }
        } else {
            const int n = tile * opt + o;
            if (n >= N) continue;
            const float v = res[m * RPT + o] * inv;
            if (EPI == EPI_PARTIAL) {
                reinterpret_cast<float*>(a.y)[(size_t)row * N + n] = v;
            } else if (EPI == EPI_STORE) {
                store_out(a.y, (size_t)row * N + n, v, (T*)nullptr);
            } else {  // EPI_QKV
                if (n < a.q_cols) {
                    store_out(a.y, (size_t)row * a.q_cols + n, v, (T*)nullptr);
                } else {
                    const int r = n - a.q_cols;
                    const bool is_k = r < a.kv_cols;
                    const int rr = is_k ? r : r - a.kv_cols;
                    const int g = rr / a.head_dim, e = rr - g * a.head_dim;
                    const size_t idx = (((size_t)row * a.kv_heads + g) * a.capacity + a.pos) * a.head_dim + e;
                    store_out(is_k ? a.k_cache : a.v_cache, idx, v, (T*)nullptr);
                }
            }
        }
    }
}

// res[MT][RPT] holds this workgroup's sums of its K chunk (rows of the tile in
// the order the epilogue expects: for SwiGLU the gate rows, then the up rows
// of the same outputs), ssl[MT] its sums of squares of the activations when
// RMSNorm is fused. When K is split, every split publishes its tile with
// coherent stores and the last to arrive adds the slices in split order
// (deterministic) and runs the epilogue; the others return.
template <typename T, int MT, int RPT, int EPI, bool NORM, int NT>
__device__ __forceinline__ void gemv_finish(const GemvDev& d, float* res, float* ssl, int* s_last, int tile,
                                            int split, int m0, int mvalid) {
    const GemvArgs& a = d.a;
    const int tid = threadIdx.x;
    // slot of this (tile, m-block) among the launch's: the counters and slices
    // of one launch never exceed the header and the scratch the plan sized
    const int tile_id = blockIdx.z * gridDim.x + blockIdx.x;
    if (d.splits > 1) {
        float* base = d.part + (size_t)tile_id * d.splits * (MT * RPT);
        float* mine = base + (size_t)split * (MT * RPT);
        const int live = mvalid * RPT;      // token rows past m are never read back
        for (int i = tid; i < live; i += NT) store_coherent(mine + i, res[i]);
        if (NORM && tid < MT) store_coherent(d.ssq + ((size_t)tile_id * d.splits + split) * MT + tid, ssl[tid]);
        if (!last_arriver(&d.cnt[tile_id], (unsigned)d.splits, s_last)) return;
        // Sum the slices in split order. A thread owns PER elements and
        // requests UNR splits of each at once, so the coherent loads are in
        // flight together rather than one round trip each.
        constexpr int PER = 4, UNR = 8;
        const int S = d.splits;
        for (int i0 = tid; i0 < live; i0 += NT * PER) {
            float acc[PER];
#pragma unroll
            for (int p = 0; p < PER; ++p) acc[p] = 0.f;
            for (int sp0 = 0; sp0 < S; sp0 += UNR) {
                float v[PER][UNR];
#pragma unroll
                for (int p = 0; p < PER; ++p)
#pragma unroll
                    for (int u = 0; u < UNR; ++u)
                        v[p][u] = load_coherent(base + (size_t)min(sp0 + u, S - 1) * (MT * RPT) + min(i0 + p * NT, live - 1));
#pragma unroll
                for (int p = 0; p < PER; ++p)
#pragma unroll
                    for (int u = 0; u < UNR; ++u)
                        if (sp0 + u < S) acc[p] += v[p][u];
            }
#pragma unroll
            for (int p = 0; p < PER; ++p)
                if (i0 + p * NT < live) res[i0 + p * NT] = acc[p];
        }
        if (NORM && tid < MT) {
            float s = 0.f;
            for (int sp = 0; sp < S; ++sp) s += load_coherent(d.ssq + ((size_t)tile_id * S + sp) * MT + tid);
            ssl[tid] = s;
        }
        __syncthreads();
    }

    gemv_epilogue<T, MT, RPT, EPI, NORM, NT>(a, res, ssl, tile, m0, mvalid);
}

}  // namespace tpk
