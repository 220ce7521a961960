// Grouped-query decode attention over the heads one rank owns, split over the
// cached keys ("split-KV").
//
// Grid: (key chunks, kv heads, sequences). A workgroup (4 waves) takes the GQ
// query heads that share one kv head and one chunk of keys, walks the chunk
// in passes of 256 keys (64 per wave) with a running (max, sum, output) per
// head, and leaves an unnormalised partial with its max and sum.
//
// Memory is read coalesced: a key's row of D bf16 is read by D/8 lanes with
// one 128-bit load each, so one wave instruction covers 64/(D/8) whole keys.
// A wave requests its pass's K and V rows before any arithmetic.
//  - Scores: each lane dots its 8 dimensions of a key with the same 8
//    dimensions of every head of the group (v_dot2), then a DPP
//    reduce-scatter over the key's lanes leaves each lane with one head's
//    score.
//  - Probabilities go to LDS as packed bf16 pairs of consecutive keys; the
//    value pass forms (V[j][d], V[j+1][d]) pairs with one v_perm each and
//    accumulates with v_dot2, two keys per instruction. The running sum adds
//    the same rounded probabilities the values are weighted with.
//  - The key groups of a wave are reduced with permlane swaps, the 4 waves
//    through LDS.
// When the keys are split over several chunks, a second small kernel (one
// workgroup per sequence, kv head and query head) merges the chunk partials
// in chunk order by their log-sum-exp weights and writes the bf16 output; the
// kernel boundary makes the partials visible, so no counters or fences are
// needed.
#include "device_common.h"
#include "kernels.h"

namespace tpk {

constexpr int AT_NT = 256;       // threads
constexpr int AT_PASS = 256;     // keys per pass (64 per wave)
constexpr int AT_MAX_CHUNKS = 128;

struct AttnDev {
    AttnArgs a;
    int chunk, n_chunks;
    float* pml;      // [B * kv_heads][n_chunks][GQ][2] (max, sum)
    float* po;       // [B * kv_heads][n_chunks][GQ][D]
};

template <int D, int GQ>
__global__ __launch_bounds__(AT_NT) void attn_decode_kernel(AttnDev d) {
    constexpr int LPK = D / 8;             // lanes per key row
    constexpr int KPW = 64 / LPK;          // keys per wave instruction
    constexpr int KW = AT_PASS / 4;        // keys per wave per pass
    constexpr int NK = KW / KPW;           // K rows a lane loads per pass
    constexpr int NP = KW / 2 / KPW;       // V row pairs a lane loads per pass
    constexpr bool PREFETCH_V = GQ <= 8;   // keep V loads in flight during the scores
    constexpr int NO = GQ * 8;             // output accumulators per lane
    const AttnArgs& a = d.a;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kq = lane / LPK, dq = lane % LPK;
    const int bg = b * a.kv_heads + g;
    const int jbeg = c * d.chunk;
    const int jend = min(jbeg + d.chunk, a.kv_len);

    __shared__ float sc[GQ][AT_PASS];                          // scores
    __shared__ __align__(16) uint32_t pp[AT_PASS / 2][GQ];     // probabilities of key pairs, packed bf16
    __shared__ float mrun[GQ], lrun[GQ], alpha[GQ];
    __shared__ float red[4][GQ][D];

    // this lane's 8 dimensions of every query head of the group
    uint4 qv[GQ];
    {
        const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.q_heads + (size_t)g * GQ) * D;
#pragma unroll
        for (int h = 0; h < GQ; ++h) qv[h] = load_u4(q + (size_t)h * D + dq * 8);
    }
    if (tid < GQ) { mrun[tid] = -INFINITY; lrun[tid] = 0.f; }

    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + (size_t)bg * a.capacity * D;
    const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + (size_t)bg * a.capacity * D;
    const float scale = 1.0f / sqrtf((float)D);
    float o[NO];
#pragma unroll
    for (int i = 0; i < NO; ++i) o[i] = 0.f;

    for (int j0 = jbeg; j0 < jend; j0 += AT_PASS) {
        const int kw0 = j0 + wave * KW;              // this wave's first key
        // K rows (and V row pairs) of the pass, clamped to the last valid key.
        uint4 kr[NK];
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int key = min(kw0 + i * KPW + kq, jend - 1);
            kr[i] = load_stream_u4(kbase + (size_t)key * D + dq * 8);
        }
        uint4 va[NP], vb[NP];
        auto load_v = [&]() {
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const int key = kw0 + 2 * (i * KPW + kq);
                va[i] = load_stream_u4(vbase + (size_t)min(key, jend - 1) * D + dq * 8);
                vb[i] = load_stream_u4(vbase + (size_t)min(key + 1, jend - 1) * D + dq * 8);
            }
        };
        if (PREFETCH_V) load_v();

        // scores
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            float s[GQ];
#pragma unroll
            for (int h = 0; h < GQ; ++h) {
                float t = dot2_bf16(kr[i].x, qv[h].x, 0.f);
                t = dot2_bf16(kr[i].y, qv[h].y, t);
                t = dot2_bf16(kr[i].z, qv[h].z, t);
                s[h] = dot2_bf16(kr[i].w, qv[h].w, t);
            }
            reduce_scatter_group<LPK, GQ>(s, lane);
            const int lk = wave * KW + i * KPW + kq;            // key within the pass
#pragma unroll
            for (int j = 0; j < (GQ > LPK ? GQ / LPK : 1); ++j) {
                bool owner;
                const int h = reduce_group_index<LPK, GQ>(lane, j, owner);
                if (owner) sc[h][lk] = (j0 + lk < jend) ? s[j] * scale : -INFINITY;
            }
        }
        if (!PREFETCH_V) load_v();
        __syncthreads();

        // running max and sum per head; probabilities relative to the new max
        for (int h = wave; h < GQ; h += 4) {
            float mx = -INFINITY;
            for (int i = lane; i < AT_PASS; i += 64) mx = fmaxf(mx, sc[h][i]);
            mx = group_max<64>(mx);
            const float mnew = fmaxf(mrun[h], mx);
            float sum = 0.f;
            for (int i = lane; i < AT_PASS / 2; i += 64) {
                const float p0 = __expf(sc[h][2 * i] - mnew);
                const float p1 = __expf(sc[h][2 * i + 1] - mnew);
                const uint32_t pk = pack_bf16x2(p0, p1);
                pp[i][h] = pk;
                sum += bf16lo(pk) + bf16hi(pk);
            }
            sum = wave_sum(sum);
            if (lane == 0) {
                const float al = __expf(mrun[h] - mnew);
                alpha[h] = al;
                lrun[h] = lrun[h] * al + sum;
                mrun[h] = mnew;
            }
        }
        __syncthreads();

        // values: two keys per v_dot2
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            const float al = alpha[h];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h * 8 + e] *= al;
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int lp = (wave * KW) / 2 + i * KPW + kq;      // key pair within the pass
            uint32_t pw[GQ];
            if constexpr (GQ >= 4) {
#pragma unroll
                for (int h4 = 0; h4 < GQ; h4 += 4) {
                    const uint4 t = *reinterpret_cast<const uint4*>(&pp[lp][h4]);
                    pw[h4] = t.x; pw[h4 + 1] = t.y; pw[h4 + 2] = t.z; pw[h4 + 3] = t.w;
                }
            } else {
#pragma unroll
                for (int h = 0; h < GQ; ++h) pw[h] = pp[lp][h];
            }
            const uint32_t* A = &va[i].x;
            const uint32_t* Bv = &vb[i].x;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t lo = __builtin_amdgcn_perm(Bv[t], A[t], 0x05040100u);   // (V[j][2t],   V[j+1][2t])
                const uint32_t hi = __builtin_amdgcn_perm(Bv[t], A[t], 0x07060302u);   // (V[j][2t+1], V[j+1][2t+1])
#pragma unroll
                for (int h = 0; h < GQ; ++h) {
                    o[h * 8 + 2 * t] = dot2_bf16(pw[h], lo, o[h * 8 + 2 * t]);
                    o[h * 8 + 2 * t + 1] = dot2_bf16(pw[h], hi, o[h * 8 + 2 * t + 1]);
                }
            }
        }
        __syncthreads();
    }

    // Reduce over the key groups of the wave (lanes with the same dq). For
    // D = 128 the groups differ in lane bits 4 and 5 (two permlane stages);
    // for D = 64 also in bit 3 (a DPP stage first).
    constexpr int N0 = (LPK == 8) ? NO / 2 : NO;
    if constexpr (LPK == 8) {
        const bool upper = (lane >> 3) & 1;
#pragma unroll
        for (int j = 0; j < NO / 2; ++j) {
            const float kp = upper ? o[NO / 2 + j] : o[j];
            const float sd = upper ? o[j] : o[NO / 2 + j];
            o[j] = kp + dpp_mov<DPP_ROW_ROR8>(sd);
        }
    }
#pragma unroll
    for (int j = 0; j < N0 / 2; ++j) xrow_pair<0>(o[j], o[N0 / 2 + j]);      // lane bit 5
#pragma unroll
    for (int j = 0; j < N0 / 4; ++j) xrow_pair<1>(o[j], o[N0 / 4 + j]);      // lane bit 4
    // slot j of this lane now holds flat index base + j (flat index = head * 8 + element)
    {
        int base = ((lane >> 5) & 1) * (N0 / 2) + ((lane >> 4) & 1) * (N0 / 4);
        if constexpr (LPK == 8) base += ((lane >> 3) & 1) * (NO / 2);
#pragma unroll
        for (int j = 0; j < N0 / 4; ++j) {
            const int idx = base + j;
            const int h = idx / 8, e = idx % 8;
            red[wave][h][dq * 8 + e] = o[j];
        }
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
        po[i] = red[0][h][e] + red[1][h][e] + red[2][h][e] + red[3][h][e];
    }
    if (tid < GQ) {
        float* ml = d.pml + (((size_t)bg * d.n_chunks + c) * GQ + tid) * 2;
        ml[0] = mrun[tid];
        ml[1] = lrun[tid];
    }
}

// Merge of the chunk partials of one (sequence, kv head, query head): weights
// exp(m_c - max) in chunk order, out = sum_c w_c o_c / sum_c w_c l_c. One
// thread per dimension. The chunk maxima and sums and the first MR chunks'
// partial outputs are requested together, so the merge costs one memory
// round trip for up to MR chunks.
template <int D, int GQ>
__global__ __launch_bounds__(D) void attn_merge_kernel(AttnDev d) {
    constexpr int MR = 32;
    const AttnArgs& a = d.a;
    const int h = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int e = threadIdx.x;
    const int bg = b * a.kv_heads + g;
    const int nc = d.n_chunks;
    __shared__ float wgt[AT_MAX_CHUNKS];
    __shared__ float red[D / 64];
    __shared__ float s_max, s_inv;
    const float* mlb = d.pml + (size_t)bg * nc * GQ * 2;
    const float* pob = d.po + (size_t)bg * nc * GQ * D + (size_t)h * D + e;
    // chunk maxima and sums (nc <= AT_MAX_CHUNKS <= 2 D): each thread reads up to two of each
    const int c0 = min(e, nc - 1), c1 = min(e + D, nc - 1);
    const float m0r = mlb[((size_t)c0 * GQ + h) * 2], l0r = mlb[((size_t)c0 * GQ + h) * 2 + 1];
    const float m1r = mlb[((size_t)c1 * GQ + h) * 2], l1r = mlb[((size_t)c1 * GQ + h) * 2 + 1];
    float v[MR];
#pragma unroll
    for (int u = 0; u < MR; ++u) v[u] = pob[(size_t)min(u, nc - 1) * GQ * D];
    const float m0 = e < nc ? m0r : -INFINITY;
    const float m1 = e + D < nc ? m1r : -INFINITY;
    float mx = group_max<64>(fmaxf(m0, m1));
    if ((e & 63) == 0) red[e >> 6] = mx;
    __syncthreads();
    if (e == 0) {
        float t = red[0];
        for (int w = 1; w < D / 64; ++w) t = fmaxf(t, red[w]);
        s_max = t;
    }
    __syncthreads();
    const float M = s_max;
    float l = 0.f;
    if (e < nc) {
        const float w = __expf(m0 - M);
        wgt[e] = w;
        l += w * l0r;
    }
    if (e + D < nc) {
        const float w = __expf(m1 - M);
        wgt[e + D] = w;
        l += w * l1r;
    }
    l = wave_sum(l);
    __syncthreads();
    if ((e & 63) == 0) red[e >> 6] = l;
    __syncthreads();
    if (e == 0) {
        float t = 0.f;
        for (int w = 0; w < D / 64; ++w) t += red[w];
        s_inv = 1.0f / t;
    }
    __syncthreads();
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < MR; ++u)
        if (u < nc) acc = fmaf(wgt[u], v[u], acc);
    for (int c = MR; c < nc; ++c) acc = fmaf(wgt[c], pob[(size_t)c * GQ * D], acc);
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((size_t)b * a.q_heads + (size_t)g * GQ + h) * D;
    out[e] = (uint16_t)f32_to_bf16_bits(acc * s_inv);
}

AttnPlan attn_plan(int batch, int q_heads, int kv_heads, int head_dim, int kv_len) {
    AttnPlan p{};
    const int gq = q_heads / kv_heads;
    const long pairs = (long)batch * kv_heads;
    // chunks of whole passes; aim for about two workgroups per compute unit
    const int passes_total = (kv_len + AT_PASS - 1) / AT_PASS;
    int want = (int)((512 + pairs - 1) / pairs);
    if (want < 1) want = 1;
    if (want > passes_total) want = passes_total;
    int passes_per_chunk = (passes_total + want - 1) / want;
    int n_chunks = (passes_total + passes_per_chunk - 1) / passes_per_chunk;
    while (n_chunks > AT_MAX_CHUNKS) {
        ++passes_per_chunk;
        n_chunks = (passes_total + passes_per_chunk - 1) / passes_per_chunk;
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
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || d.n_chunks == 1) return e;
    hipLaunchKernelGGL((attn_merge_kernel<D, GQ>), dim3(GQ, d.a.kv_heads, d.a.batch), dim3(D), 0, s, d);
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

hipError_t attn_launch(const AttnArgs& a, const AttnPlan& p, unsigned* /*counters: unused*/, void* scratch,
                       hipStream_t s) {
    AttnDev d{};
    d.a = a;
    d.chunk = p.chunk;
    d.n_chunks = p.n_chunks;
    const int gq = a.q_heads / a.kv_heads;
    if (p.n_chunks > 1) {
        const size_t pairs = (size_t)a.batch * a.kv_heads;
        char* b = reinterpret_cast<char*>(scratch);
        const size_t ml = (pairs * p.n_chunks * gq * 2 * 4 + 255) / 256 * 256;
        d.pml = reinterpret_cast<float*>(b);
        d.po = reinterpret_cast<float*>(b + ml);
    }
    if (a.head_dim == 64) return attn_launch_d<64>(d, gq, s);
    if (a.head_dim == 128) return attn_launch_d<128>(d, gq, s);
    return hipErrorInvalidValue;
}

}  // namespace tpk
