// Grouped-query decode attention over the heads one rank owns, split over the
// cached keys ("split-KV").
//
// Grid: (key chunks, kv heads, sequences). A workgroup takes the GQ query
// heads that share one kv head and one chunk of keys, walks the chunk in
// passes of 256 keys with a running (max, sum, output) per head, and leaves
// an unnormalised partial with its max and sum in the workspace. The last
// workgroup of a (sequence, kv head) to finish, found with a counter, merges
// the chunk partials in chunk order by their log-sum-exp weights and writes
// the bf16 output. Partials travel through agent-scope coherent stores and
// loads, so no cache-wide fence is needed. Reading K and V once is the
// cost; q is staged in LDS and read by broadcast.
#include "device_common.h"
#include "kernels.h"

namespace tpk {

constexpr int AT_NT = 256;       // threads; one key per thread while scoring
constexpr int AT_PASS = 256;     // keys per pass
constexpr int AT_MAX_CHUNKS = 128;

struct AttnDev {
    AttnArgs a;
    int chunk, n_chunks;
    unsigned* cnt;   // [B * kv_heads]
    float* pml;      // [B * kv_heads][n_chunks][GQ][2] (max, sum)
    float* po;       // [B * kv_heads][n_chunks][GQ][D]
};

template <int D, int GQ>
__global__ __launch_bounds__(AT_NT) void attn_decode_kernel(AttnDev d) {
    constexpr int QD = D / 4;          // threads per V row (4 dims each)
    constexpr int KG = AT_NT / QD;     // key groups in the PV phase
    const AttnArgs& a = d.a;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bg = b * a.kv_heads + g;
    const int jbeg = c * d.chunk;
    const int jend = min(jbeg + d.chunk, a.kv_len);

    __shared__ uint32_t qs[GQ][D / 2];
    __shared__ float ps[GQ][AT_PASS];
    __shared__ float mrun[GQ], lrun[GQ], alpha[GQ];
    __shared__ float red[4][GQ][D];
    __shared__ int s_last;

    const uint32_t* q = reinterpret_cast<const uint32_t*>(a.q) + ((size_t)b * a.q_heads + (size_t)g * GQ) * (D / 2);
    for (int i = tid; i < GQ * D / 2; i += AT_NT) qs[i / (D / 2)][i % (D / 2)] = q[i];
    if (tid < GQ) { mrun[tid] = -INFINITY; lrun[tid] = 0.f; }
    __syncthreads();

    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + (size_t)bg * a.capacity * D;
    const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + (size_t)bg * a.capacity * D;
    const float scale = 1.0f / sqrtf((float)D);
    const int dq = tid % QD, kg = tid / QD;
    float o[GQ][4];
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[h][e] = 0.f;

    for (int j0 = jbeg; j0 < jend; j0 += AT_PASS) {
        const int nk = min(AT_PASS, jend - j0);
        // scores: thread tid scores key j0 + tid for every head of the group
        float s[GQ];
#pragma unroll
        for (int h = 0; h < GQ; ++h) s[h] = 0.f;
        if (tid < nk) {
            const uint4* kr = reinterpret_cast<const uint4*>(kbase + (size_t)(j0 + tid) * D);
            uint4 kv[D / 8];
#pragma unroll
            for (int v = 0; v < D / 8; ++v) kv[v] = load_stream_u4(kr + v);
#pragma unroll
            for (int v = 0; v < D / 8; ++v) {
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    const uint4 qv = *reinterpret_cast<const uint4*>(&qs[h][4 * v]);
                    s[h] = dot2_bf16(kv[v].x, qv.x, s[h]);
                    s[h] = dot2_bf16(kv[v].y, qv.y, s[h]);
                    s[h] = dot2_bf16(kv[v].z, qv.z, s[h]);
                    s[h] = dot2_bf16(kv[v].w, qv.w, s[h]);
                }
            }
        }
#pragma unroll
        for (int h = 0; h < GQ; ++h) ps[h][tid] = (tid < nk) ? s[h] * scale : -INFINITY;
        __syncthreads();

        // per-head running max and sum; probabilities relative to the new max
        for (int h = wave; h < GQ; h += 4) {
            float mx = -INFINITY;
            for (int i = lane; i < AT_PASS; i += 64) mx = fmaxf(mx, ps[h][i]);
            mx = group_max<64>(mx);
            const float mnew = fmaxf(mrun[h], mx);
            float sum = 0.f;
            for (int i = lane; i < AT_PASS; i += 64) {
                const float p = __expf(ps[h][i] - mnew);
                ps[h][i] = p;
                sum += p;
            }
            sum = group_sum<64>(sum);
            if (lane == 0) {
                const float al = __expf(mrun[h] - mnew);
                alpha[h] = al;
                lrun[h] = lrun[h] * al + sum;
                mrun[h] = mnew;
            }
        }
        __syncthreads();

        // PV: thread (kg, dq) accumulates dims 4dq..4dq+3 over keys kg, kg+KG, ...
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            const float al = alpha[h];
#pragma unroll
            for (int e = 0; e < 4; ++e) o[h][e] *= al;
        }
        for (int j = kg; j < nk; j += KG) {
            const uint2 vv = *reinterpret_cast<const uint2*>(vbase + (size_t)(j0 + j) * D + 4 * dq);
            const float v0 = bf16lo(vv.x), v1 = bf16hi(vv.x), v2 = bf16lo(vv.y), v3 = bf16hi(vv.y);
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                const float p = ps[h][j];
                o[h][0] = fmaf(p, v0, o[h][0]);
                o[h][1] = fmaf(p, v1, o[h][1]);
                o[h][2] = fmaf(p, v2, o[h][2]);
                o[h][3] = fmaf(p, v3, o[h][3]);
            }
        }
        __syncthreads();
    }

    // reduce the key groups: lanes of a wave first, then the 4 waves via LDS
#pragma unroll
    for (int h = 0; h < GQ; ++h)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = o[h][e];
#pragma unroll
            for (int off = QD; off < 64; off <<= 1) v += __shfl_xor(v, off, 64);
            o[h][e] = v;
        }
    if (lane < QD) {
#pragma unroll
        for (int h = 0; h < GQ; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[wave][h][4 * dq + e] = o[h][e];
    }
    __syncthreads();

    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((size_t)b * a.q_heads + (size_t)g * GQ) * D;
    if (d.n_chunks == 1) {
        for (int i = tid; i < GQ * D; i += AT_NT) {
            const int h = i / D, e = i % D;
            const float v = red[0][h][e] + red[1][h][e] + red[2][h][e] + red[3][h][e];
            out[i] = (uint16_t)f32_to_bf16_bits(v / lrun[h]);
        }
        return;
    }

    float* po = d.po + ((size_t)bg * d.n_chunks + c) * GQ * D;
    for (int i = tid; i < GQ * D; i += AT_NT) {
        const int h = i / D, e = i % D;
        store_coherent(po + i, red[0][h][e] + red[1][h][e] + red[2][h][e] + red[3][h][e]);
    }
    if (tid < GQ) {
        float* ml = d.pml + (((size_t)bg * d.n_chunks + c) * GQ + tid) * 2;
        store_coherent(ml, mrun[tid]);
        store_coherent(ml + 1, lrun[tid]);
    }
    if (!last_arriver(&d.cnt[bg], (unsigned)d.n_chunks, &s_last)) return;

    // merge the chunks in chunk order
    __shared__ float wgt[AT_MAX_CHUNKS][GQ];
    const float* mlb = d.pml + (size_t)bg * d.n_chunks * GQ * 2;
    for (int h = wave; h < GQ; h += 4) {
        float mx = -INFINITY;
        for (int cc = lane; cc < d.n_chunks; cc += 64) mx = fmaxf(mx, load_coherent(mlb + (cc * GQ + h) * 2));
        mx = group_max<64>(mx);
        float l = 0.f;
        for (int cc = lane; cc < d.n_chunks; cc += 64) {
            const float w = __expf(load_coherent(mlb + (cc * GQ + h) * 2) - mx);
            wgt[cc][h] = w;
            l += w * load_coherent(mlb + (cc * GQ + h) * 2 + 1);
        }
        l = group_sum<64>(l);
        if (lane == 0) alpha[h] = 1.0f / l;
    }
    __syncthreads();
    const float* pob = d.po + (size_t)bg * d.n_chunks * GQ * D;
    for (int i = tid; i < GQ * D; i += AT_NT) {
        const int h = i / D;
        float v = 0.f;
        for (int cc = 0; cc < d.n_chunks; ++cc) v = fmaf(wgt[cc][h], load_coherent(pob + (size_t)cc * GQ * D + i), v);
        out[i] = (uint16_t)f32_to_bf16_bits(v * alpha[h]);
    }
}

AttnPlan attn_plan(int batch, int q_heads, int kv_heads, int head_dim, int kv_len) {
    AttnPlan p{};
    const int gq = q_heads / kv_heads;
    const long pairs = (long)batch * kv_heads;
    // chunks of whole passes; aim for about two workgroups per compute unit
    int passes_total = (kv_len + AT_PASS - 1) / AT_PASS;
    int want = (int)((512 + pairs - 1) / pairs);
    if (want < 1) want = 1;
    if (want > passes_total) want = passes_total;
    int passes_per_chunk = (passes_total + want - 1) / want;
    int n_chunks = (passes_total + passes_per_chunk - 1) / passes_per_chunk;
    while (n_chunks > AT_MAX_CHUNKS) {
        ++passes_per_chunk;
        n_chunks = (passes_total + passes_per_chunk - 1) / passes_per_chunk;
    }
    if (pairs > WS_MAX_COUNTERS) {   // one counter per (sequence, kv head): no split beyond that
        passes_per_chunk = passes_total;
        n_chunks = 1;
    }
    p.chunk = passes_per_chunk * AT_PASS;
    p.n_chunks = n_chunks;
    if (n_chunks > 1) {
        const size_t ml = ((size_t)pairs * n_chunks * gq * 2 * 4 + 255) / 256 * 256;
        const size_t o = (size_t)pairs * n_chunks * gq * head_dim * 4;
        p.ws_bytes = ml + (o + 255) / 256 * 256;
    } else {
        p.ws_bytes = 0;
    }
    return p;
}

template <int D, int GQ>
static hipError_t attn_launch_t(const AttnDev& d, hipStream_t s) {
    dim3 grid(d.n_chunks, d.a.kv_heads, d.a.batch);
    hipLaunchKernelGGL((attn_decode_kernel<D, GQ>), grid, dim3(AT_NT), 0, s, d);
    return hipGetLastError();
}

template <int D>
static hipError_t attn_launch_d(const AttnDev& d, int gq, hipStream_t s) {
    switch (gq) {
        case 1: return attn_launch_t<D, 1>(d, s);
        case 2: return attn_launch_t<D, 2>(d, s);
        case 4: return attn_launch_t<D, 4>(d, s);
        case 8: return attn_launch_t<D, 8>(d, s);
        case 16: return attn_launch_t<D, 16>(d, s);
    }
    return hipErrorInvalidValue;
}

hipError_t attn_launch(const AttnArgs& a, const AttnPlan& p, unsigned* counters, void* scratch, hipStream_t s) {
    AttnDev d{};
    d.a = a;
    d.chunk = p.chunk;
    d.n_chunks = p.n_chunks;
    const int gq = a.q_heads / a.kv_heads;
    if (p.n_chunks > 1) {
        const size_t pairs = (size_t)a.batch * a.kv_heads;
        char* b = reinterpret_cast<char*>(scratch);
        const size_t ml = (pairs * p.n_chunks * gq * 2 * 4 + 255) / 256 * 256;
        d.cnt = counters;
        d.pml = reinterpret_cast<float*>(b);
        d.po = reinterpret_cast<float*>(b + ml);
    }
    if (a.head_dim == 64) return attn_launch_d<64>(d, gq, s);
    if (a.head_dim == 128) return attn_launch_d<128>(d, gq, s);
    return hipErrorInvalidValue;
}

}  // namespace tpk
