// Grouped-query decode attention over the heads one rank owns, split over the
// cached keys ("split-KV").
//
// Grid: (key chunks, kv heads, sequences). A workgroup (4 waves) takes the GQ
// query heads that share one kv head and one chunk of keys, in passes of 128
// keys; each wave owns 32 keys of every pass and keeps its own running max,
// sum and output per head, so the waves never synchronise inside the chunk.
//
// Memory is read coalesced: a key's row of D bf16 is read by D/8 lanes with
// one 128-bit load each, so one wave instruction covers 64/(D/8) whole keys,
// and a wave requests its pass's K rows, then its V rows, before anything
// else.
//  - Scores are a [keys x D] x [D x heads] contraction and go to the matrix
//    cores (v_mfma_f32_16x16x32_bf16, heads padded to 16 with zero queries).
//    The K rows pass through a wave-private LDS tile (rows padded by 16
//    bytes) on their way to the operand registers: read in the operand
//    layout straight from HBM they would stream at a fraction of the rate.
//    A lane then holds one head's scores for four keys of each 16-key block.
//  - The softmax runs in registers: maxima and sums over the four lanes of a
//    head are two permlane swaps each. Probabilities are rounded to bf16 and
//    the running sum adds exactly the rounded values the outputs are weighted
//    with.
//  - Values: probabilities go to LDS as packed bf16 pairs of consecutive keys;
//    the value pass forms (V[j][d], V[j+1][d]) pairs with one v_perm each and
//    accumulates two keys per v_dot2.
//  - At the end of the chunk each wave reduces its outputs over its key
//    groups (permlane swaps, DPP), and the four waves are merged by their
//    log-sum-exp weights through LDS.
// When the keys are split over several chunks, a second small kernel (one
// workgroup per sequence, kv head and query head) merges the chunk partials
// in chunk order by their log-sum-exp weights and writes the bf16 output; the
// kernel boundary makes the partials visible, so no counters or fences are
// needed.
#include "device_common.h"
#include "kernels.h"

namespace tpk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int AT_NT = 256;       // threads
constexpr int AT_KW = 32;        // keys per wave per pass
constexpr int AT_PASS = 4 * AT_KW;   // keys per workgroup pass
constexpr int AT_MAX_CHUNKS = 128;

struct AttnDev {
    AttnArgs a;
    int chunk, n_chunks;
    float* pml;      // [B * kv_heads][n_chunks][GQ][2] (max, sum)
    float* po;       // [B * kv_heads][n_chunks][GQ][D]
};

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// op over the lanes l, l ^ 16, l ^ 32, l ^ 48: each permlane swap of a value
// with itself leaves, between the two results, the lane's own value and its
// partner's in every lane, so op(a, b) combines them with no selects.
__device__ __forceinline__ float max_over_kg(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float sum_over_kg(float v) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

template <int D, int GQ>
__global__ __launch_bounds__(AT_NT) void attn_decode_kernel(AttnDev d) {
    constexpr int LPK = D / 8;             // lanes per key row
    constexpr int KPW = 64 / LPK;          // keys per wave instruction
    constexpr int NK = AT_KW / KPW;        // K rows a lane loads per pass
    constexpr int NP = AT_KW / 2 / KPW;    // V row pairs a lane loads per pass
    constexpr int NO = GQ * 8;             // output accumulators per lane
    constexpr int KP = D + 8;              // K tile row pitch (elements)
    constexpr int DS = D / 32;             // MFMA steps over d
    constexpr int KB = AT_KW / 16;         // 16-key blocks per wave per pass
    constexpr int NPAIR = AT_KW / 2;
    static_assert(AT_KW * KP * 2 >= GQ * D * 4, "the end-of-chunk reduction reuses the K tile");
    const AttnArgs& a = d.a;
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kq = lane / LPK, dq = lane % LPK;        // load / value-pass role
    const int hc = lane & 15, kg = lane >> 4;          // score role: head hc, keys 4 kg .. 4 kg + 3 of a block
    const int bg = b * a.kv_heads + g;
    const int jbeg = c * d.chunk;
    const int jend = min(jbeg + d.chunk, a.kv_len);

    __shared__ __align__(16) uint16_t kt[4][AT_KW * KP];       // K tiles; at the end, each wave's outputs
    __shared__ __align__(16) uint32_t pp[4][NPAIR][16];        // probabilities of key pairs, packed bf16
    __shared__ float alpha_w[4][16];
    __shared__ float m_w[4][16], l_w[4][16];

    // query fragments: head hc, elements 32 s + 8 kg .. + 7 (zero for padding heads)
    uint4 qf[DS];
    {
        const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.q_heads + (size_t)g * GQ) * D;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            const uint4 v = load_u4(q + (size_t)min(hc, GQ - 1) * D + s * 32 + kg * 8);
            qf[s] = hc < GQ ? v : make_uint4(0, 0, 0, 0);
        }
    }
    const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + (size_t)bg * a.capacity * D;
    const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.v) + (size_t)bg * a.capacity * D;
    const float scale = 1.0f / sqrtf((float)D);
    uint16_t* ktw = kt[wave];
    float mrun = -INFINITY, lrun = 0.f;                // of head hc, this wave's keys
    float o[NO];
#pragma unroll
    for (int i = 0; i < NO; ++i) o[i] = 0.f;

    for (int j0 = jbeg; j0 < jend; j0 += AT_PASS) {
        const int kw0 = j0 + wave * AT_KW;             // this wave's first key
        // K rows, then V row pairs, clamped to the last valid key.
        uint4 kr[NK];
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int key = min(kw0 + i * KPW + kq, jend - 1);
            kr[i] = load_stream_u4(kbase + (size_t)key * D + dq * 8);
        }
        uint4 va[NP], vb[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int key = kw0 + 2 * (i * KPW + kq);
            va[i] = load_stream_u4(vbase + (size_t)min(key, jend - 1) * D + dq * 8);
            vb[i] = load_stream_u4(vbase + (size_t)min(key + 1, jend - 1) * D + dq * 8);
        }
#pragma unroll
        for (int i = 0; i < NK; ++i) *reinterpret_cast<uint4*>(ktw + (i * KPW + kq) * KP + dq * 8) = kr[i];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // scores: block kb, lane holds head hc for keys 16 kb + 4 kg + r
        f32x4_t sc[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            sc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < DS; ++s) {
                const uint4 kf = *reinterpret_cast<const uint4*>(ktw + (kb * 16 + hc) * KP + s * 32 + kg * 8);
                sc[kb] = mfma16(kf, qf[s], sc[kb]);
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool valid = kw0 + kb * 16 + 4 * kg + r < jend;
                sc[kb][r] = valid ? sc[kb][r] * scale : -INFINITY;
                mx = fmaxf(mx, sc[kb][r]);
            }
        mx = max_over_kg(mx);
        const float mnew = fmaxf(mrun, mx);
        const float mref = mnew == -INFINITY ? 0.f : mnew;    // a wave may see no valid key yet
        const float al = __expf(mrun - mref);
        float sum = 0.f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const uint32_t pk = pack_bf16x2(__expf(sc[kb][2 * r2] - mref), __expf(sc[kb][2 * r2 + 1] - mref));
                sum += bf16lo(pk) + bf16hi(pk);
                pp[wave][kb * 8 + 2 * kg + r2][hc] = pk;
            }
        sum = sum_over_kg(sum);
        lrun = lrun * al + sum;
        mrun = mnew;
        if (kg == 0) alpha_w[wave][hc] = al;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // values: two keys per v_dot2
#pragma unroll
        for (int h = 0; h < GQ; ++h) {
            const float ah = alpha_w[wave][h];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[h * 8 + e] *= ah;
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int lp = i * KPW + kq;                // key pair within the wave's keys
            uint32_t pw[GQ];
            if constexpr (GQ >= 4) {
#pragma unroll
                for (int h4 = 0; h4 < GQ; h4 += 4) {
                    const uint4 t = *reinterpret_cast<const uint4*>(&pp[wave][lp][h4]);
                    pw[h4] = t.x; pw[h4 + 1] = t.y; pw[h4 + 2] = t.z; pw[h4 + 3] = t.w;
                }
            } else {
#pragma unroll
                for (int h = 0; h < GQ; ++h) pw[h] = pp[wave][lp][h];
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
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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
    float* ow = reinterpret_cast<float*>(kt[wave]);                          // [GQ][D] of this wave
    {
        int base = ((lane >> 5) & 1) * (N0 / 2) + ((lane >> 4) & 1) * (N0 / 4);
        if constexpr (LPK == 8) base += ((lane >> 3) & 1) * (NO / 2);
#pragma unroll
        for (int j = 0; j < N0 / 4; ++j) {
            const int idx = base + j;
            const int h = idx / 8, e = idx % 8;
            ow[h * D + dq * 8 + e] = o[j];
        }
    }
    if (kg == 0) {
        m_w[wave][hc] = mrun;
        l_w[wave][hc] = lrun;
    }
    __syncthreads();

    // Merge the four waves: weights exp(m_w - max), in wave order.
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((size_t)b * a.q_heads + (size_t)g * GQ) * D;
    float* po = d.po + ((size_t)bg * d.n_chunks + c) * GQ * D;
    for (int i = tid; i < GQ * D; i += AT_NT) {
        const int h = i / D;
        const float M = fmaxf(fmaxf(m_w[0][h], m_w[1][h]), fmaxf(m_w[2][h], m_w[3][h]));
        float acc = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float wt = m_w[w][h] == -INFINITY ? 0.f : __expf(m_w[w][h] - M);
            acc += wt * reinterpret_cast<const float*>(kt[w])[i];
            l += wt * l_w[w][h];
        }
        if (d.n_chunks == 1) {
            out[i] = (uint16_t)f32_to_bf16_bits(acc / l);
        } else {
            po[i] = acc;
            if (i % D == 0) {
                float* ml = d.pml + (((size_t)bg * d.n_chunks + c) * GQ + h) * 2;
                ml[0] = M;
                ml[1] = l;
            }
        }
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

// Scratch of n chunk partials per (sequence, kv head): running max and sum per
// q head, then the unnormalised outputs; none for a single chunk.
static size_t attn_chunk_bytes(long pairs, int n_chunks, int gq, int head_dim) {
    if (n_chunks <= 1) return 0;
    const size_t ml = ((size_t)pairs * n_chunks * gq * 2 * 4 + 255) / 256 * 256;
    const size_t o = (size_t)pairs * n_chunks * gq * head_dim * 4;
    return ml + (o + 255) / 256 * 256;
}

AttnPlan attn_plan(int batch, int q_heads, int kv_heads, int head_dim, int kv_len) {
    AttnPlan p{};
    const int gq = q_heads / kv_heads;
    const long pairs = (long)batch * kv_heads;
    // Chunks of whole passes, about one workgroup per compute unit: measured
    // on 16 x 8192-key caches, 256 workgroups beat 192 (idle units), 384
    // (uneven) and 512 (shorter workgroups, more partials).
    const int passes_total = (kv_len + AT_PASS - 1) / AT_PASS;
    int want = (int)((256 + pairs - 1) / pairs);
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
    p.ws_bytes = attn_chunk_bytes(pairs, n_chunks, gq, head_dim);
    return p;
}

size_t attn_ws_bound(int batch, int q_heads, int kv_heads, int head_dim, int max_kv_len) {
    // attn_plan's chunk count is at most the requested workgroups per (sequence,
    // kv head), at most AT_MAX_CHUNKS and at most the passes of the longest
    // cache; it is not monotone in kv_len, so bound it by all three.
    const long pairs = (long)batch * kv_heads;
    long n = (256 + pairs - 1) / pairs;
    if (n < 1) n = 1;
    if (n > AT_MAX_CHUNKS) n = AT_MAX_CHUNKS;
    const long passes = (max_kv_len + AT_PASS - 1) / AT_PASS;
    if (n > passes) n = passes;
    return attn_chunk_bytes(pairs, (int)n, q_heads / kv_heads, head_dim);
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
