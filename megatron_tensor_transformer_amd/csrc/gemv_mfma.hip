// Decode projections of a few to 16 tokens on the matrix cores
// (v_mfma_f32_16x16x32_bf16).
//
// At 16 tokens a v_dot2 projection needs more VALU issue slots than the
// weight stream leaves, although the work is still a dense contraction of a
// [16, K] activation block with [K, N] weights. One MFMA multiplies the 16
// tokens' slice of 32 K elements (A) with 16 weight rows' slice of the same
// 32 elements (B); in both operands a lane holds 8 consecutive K elements of
// one row.
//
// Loading B straight from HBM in that layout reads 16 rows x 64 bytes per
// wave instruction, which streams at well under the HBM rate; runs of 256
// bytes or more per row stream at full rate. So weights are read as 2 rows x
// 512 bytes per instruction and pass through a small wave-private LDS tile
// on their way to the operand registers.
//  - A workgroup (4 waves) owns 64 weight rows (16 per wave) and a K chunk,
//    walked in stages of 256 elements with two stages of loads in flight:
//    the loads of stage i + 1 are requested before stage i is used. Loads
//    return in order, so each stage's activations and weights are requested
//    together, in the order they are consumed.
//  - Per stage the activations (16 tokens x 256, padded with zeros, times
//    gamma when RMSNorm is fused, their squares summed) are staged once for
//    the workgroup, so activation reads are a quarter of the weight bytes;
//    each wave stages its own 16 weight rows. Rows are padded by 16 bytes so
//    the operand reads of 16 rows hit distinct banks.
//  - K is split over at most about four workgroups per tile. Unsplit, the
//    results (lane: one weight row, four tokens) go through an LDS tile to the
//    epilogue shared with the v_dot2 kernel. Split, each workgroup writes its
//    float32 slice with plain stores and a small merge kernel (one workgroup
//    per tile) adds the slices in split order and runs that epilogue: no
//    counter vote, whose memory round trips would sit at the end of the
//    projection kernel.
#include "gemv_tile.h"

namespace tpk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int SK_NW = 4;                       // waves per workgroup
constexpr int SK_MT = 16;                      // tokens per block
constexpr int SK_RPT = SK_NW * 16;             // weight rows per workgroup
constexpr int SK_SUB = 256;                    // K elements per stage
constexpr int SK_PITCH = SK_SUB + 8;           // LDS row pitch in elements
constexpr int SK_WL = 16 * SK_SUB / 8 / 64;    // weight vectors per lane per stage (8)
constexpr int SK_MAX_STAGES = 8;               // K chunk of at most 2048

__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// NST: stages per workgroup; the K chunk is NST * 256.
template <int EPI, bool NORM, int NST>
__global__ __launch_bounds__(SK_NW * 64) void gemv_mfma_kernel(GemvDev d) {
    constexpr int NT = SK_NW * 64;
    constexpr bool SWI = (EPI == EPI_SWIGLU);
    constexpr int HALF = SK_RPT / 2;
    __shared__ __align__(16) uint16_t wl[SK_NW][16 * SK_PITCH];
    __shared__ __align__(16) uint16_t xl[SK_MT * SK_PITCH];
    __shared__ float res[SK_MT * SK_RPT];
    __shared__ float ssl[SK_MT];

    const GemvArgs& a = d.a;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tile = blockIdx.x, split = blockIdx.y, mb = d.mb0 + blockIdx.z;
    const int K = a.K, N = a.N;
    const int kbase = split * (NST * SK_SUB);
    const int m0 = mb * SK_MT;
    const int mvalid = min(SK_MT, a.m - m0);
    const int col = lane & 15, kg = lane >> 4;

    // Loads of a stage. Lane: element offset (lane & 31) * 8 of the stage.
    //  - weights: vector q covers the wave's rows 2q and 2q + 1 (half-waves);
    //  - activations: tokens t0 and t0 + 8 (t0 = tid / 32), and gamma.
    // Rows past N and tokens past m are clamped to valid ones (their results
    // are never stored or are zeroed), elements past K are clamped in bounds
    // and zeroed when staged; no load is conditional.
    const int ve = (lane & 31) * 8;
    const uint16_t* wrow[SK_WL];
#pragma unroll
    for (int q = 0; q < SK_WL; ++q) {
        const int r = 2 * q + (lane >> 5);     // row within the wave's 16
        int n;
        const uint16_t* base;
        if (SWI) {                             // waves 0-1: gate rows, waves 2-3: up rows of the same outputs
            n = tile * HALF + (wave & 1) * 16 + r;
            base = reinterpret_cast<const uint16_t*>(wave < 2 ? a.w : a.w_up);
        } else {
            n = tile * SK_RPT + wave * 16 + r;
            base = reinterpret_cast<const uint16_t*>(a.w);
        }
        wrow[q] = base + (size_t)min(n, N - 1) * K;
    }
    const int t0 = tid >> 5;
    const uint16_t* xrow[2];
    bool tok_ok[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int t = t0 + 8 * i;
        tok_ok[i] = t < mvalid;
        xrow[i] = reinterpret_cast<const uint16_t*>(a.x) + (size_t)(m0 + min(t, mvalid - 1)) * K;
    }
    const uint16_t* gam = reinterpret_cast<const uint16_t*>(a.gamma);

    struct Stage { uint4 w[SK_WL]; uint4 x[2]; uint4 g; };
    auto issue = [&](Stage& b, int st) {
        const int kk = min(kbase + st * SK_SUB + ve, K - 8);
#pragma unroll
        for (int i = 0; i < 2; ++i) b.x[i] = load_u4(xrow[i] + kk);
        if (NORM) b.g = load_u4(gam + kk);
#pragma unroll
        for (int q = 0; q < SK_WL; ++q) b.w[q] = load_stream_u4(wrow[q] + kk);
    };

    const uint4 zero = make_uint4(0, 0, 0, 0);
    float ss[2] = {0.f, 0.f};
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // One stage: request the next stage's loads, stage this one in LDS, multiply.
    auto run = [&](Stage& cur, Stage& nxt, int st) {
        if (st + 1 < NST) {
            issue(nxt, st + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        const bool kin = kbase + st * SK_SUB + ve < K;
        if (st > 0) __syncthreads();           // every wave is done reading the previous stage
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint4 v = cur.x[i];
            if (!(tok_ok[i] && kin)) v = zero;
            if (NORM) {
                ss[i] += vsumsq(v, (uint16_t*)nullptr);
                v = vscale(v, cur.g, (uint16_t*)nullptr);
            }
            *reinterpret_cast<uint4*>(xl + (t0 + 8 * i) * SK_PITCH + ve) = v;
        }
#pragma unroll
        for (int q = 0; q < SK_WL; ++q) {
            uint4 v = cur.w[q];
            if (!kin) v = zero;
            *reinterpret_cast<uint4*>(&wl[wave][(2 * q + (lane >> 5)) * SK_PITCH + ve]) = v;
        }
        __syncthreads();
#pragma unroll
        for (int s = 0; s < SK_SUB / 32; ++s) {
            const uint4 xa = *reinterpret_cast<const uint4*>(xl + col * SK_PITCH + s * 32 + kg * 8);
            const uint4 wb = *reinterpret_cast<const uint4*>(&wl[wave][col * SK_PITCH + s * 32 + kg * 8]);
            acc = mfma16(xa, wb, acc);
        }
    };
    Stage s0, s1;
    issue(s0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NST; st += 2) {
        run(s0, s1, st);
        if (st + 1 < NST) run(s1, s0, st + 1);
    }

    if (NORM) {
        // the 32 lanes of a half-wave hold the same two tokens
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float v = ss[i];
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            if ((lane & 31) == 0) ssl[t0 + 8 * i] = v;
        }
    }
    if (d.splits > 1) {
        if (NORM) __syncthreads();             // ssl written by the stagers
        // This split's slice goes out with plain stores; the merge kernel that
        // follows on the stream adds the slices and runs the epilogue.
        const int tile_id = blockIdx.z * d.n_tiles + tile;
        float* mine = d.part + ((size_t)tile_id * d.splits + split) * (SK_MT * SK_RPT);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (4 * kg + j < mvalid) mine[(4 * kg + j) * SK_RPT + wave * 16 + col] = acc[j];
        if (NORM && tid < mvalid) d.ssq[((size_t)tile_id * d.splits + split) * SK_MT + tid] = ssl[tid];
        return;
    }
    // lane holds tokens 4 kg + j of row wave * 16 + col
#pragma unroll
    for (int j = 0; j < 4; ++j) res[(4 * kg + j) * SK_RPT + wave * 16 + col] = acc[j];
    __syncthreads();
    gemv_epilogue<uint16_t, SK_MT, SK_RPT, EPI, NORM, NT>(a, res, ssl, tile, m0, mvalid);
}

// Split-K merge: one workgroup per output tile adds the tile's slices in
// split order (a thread requests the slices of its outputs together) and runs
// the epilogue.
template <int EPI, bool NORM>
__global__ __launch_bounds__(256) void gemv_mfma_merge_kernel(GemvDev d) {
    // The plan splits K about four ways, so one batch of loads usually
    // covers every slice; the squared-sum slices of a fused RMSNorm travel in
    // the same batch.
    constexpr int NT = 256, PER = SK_MT * SK_RPT / NT, UNR = 4;
    __shared__ float res[SK_MT * SK_RPT];
    __shared__ float ssl[SK_MT];
    const int tid = threadIdx.x, tile = blockIdx.x, mb = d.mb0 + blockIdx.z;
    const int m0 = mb * SK_MT;
    const int mvalid = min(SK_MT, d.a.m - m0);
    const int S = d.splits;
    const int tile_id = blockIdx.z * d.n_tiles + tile;
    const float* base = d.part + (size_t)tile_id * S * (SK_MT * SK_RPT);
    const float* sqb = NORM ? d.ssq + (size_t)tile_id * S * SK_MT + min(tid, mvalid - 1) : nullptr;
    const int live = mvalid * SK_RPT;
    float acc[PER], sq = 0.f;
#pragma unroll
    for (int p = 0; p < PER; ++p) acc[p] = 0.f;
    for (int sp0 = 0; sp0 < S; sp0 += UNR) {
        float v[PER][UNR], q[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u)
            if (NORM) q[u] = sqb[(size_t)min(sp0 + u, S - 1) * SK_MT];
#pragma unroll
        for (int p = 0; p < PER; ++p)
#pragma unroll
            for (int u = 0; u < UNR; ++u)
                v[p][u] = base[(size_t)min(sp0 + u, S - 1) * (SK_MT * SK_RPT) + min(tid + p * NT, live - 1)];
#pragma unroll
        for (int u = 0; u < UNR; ++u)
            if (sp0 + u < S) {
                if (NORM) sq += q[u];
#pragma unroll
                for (int p = 0; p < PER; ++p) acc[p] += v[p][u];
            }
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) res[tid + p * NT] = acc[p];
    if (NORM && tid < mvalid) ssl[tid] = sq;
    __syncthreads();
    gemv_epilogue<uint16_t, SK_MT, SK_RPT, EPI, NORM, NT>(d.a, res, ssl, tile, m0, mvalid);
}

GemvPlan gemv_plan_mfma(int m, int K, int N, int epi) {
    GemvPlan p{};
    p.mfma = 1;
    p.mt = SK_MT;
    p.mblocks = (m + SK_MT - 1) / SK_MT;
    p.nw = SK_NW;
    p.rows_per_tile = SK_RPT;
    p.out_per_tile = (epi == EPI_SWIGLU) ? SK_RPT / 2 : SK_RPT;
    p.n_tiles = (N + p.out_per_tile - 1) / p.out_per_tile;
    // K chunk: 1024 or 2048 elements, the smaller when the launch then has
    // at most 256 workgroups (512 for SwiGLU tiles), and shorter chunks only
    // for launches that would otherwise have fewer than 128 workgroups. Measured
    // in replayed graphs on the 8B MLP and 70B attention and MLP shard shapes:
    // about one workgroup per compute unit streams best, more splits cost
    // merge traffic and a longer tail, and chunks under 1024 gain nothing
    // once about half the compute units are busy.
    const int64_t tiles = (int64_t)p.n_tiles * p.mblocks;
    const int64_t lim = (epi == EPI_SWIGLU) ? 512 : 256;
    auto wgs = [&](int c) { return tiles * ((K + c - 1) / c); };
    int kc = 4 * SK_SUB;
    while (kc < SK_MAX_STAGES * SK_SUB && wgs(kc) > lim) kc *= 2;
    while (kc > SK_SUB && wgs(kc) < 128 && wgs(kc / 2) <= lim) kc /= 2;
    while (kc > SK_SUB && kc / 2 >= K) kc /= 2;   // no stage past the end of K
    const int S = (K + kc - 1) / kc;
    p.mb_per_launch = p.mblocks;                // the merge uses no counters
    p.kc = kc;
    p.splits = S;
    p.threads = SK_NW * 64;
    p.lds_bytes = 0;                           // static LDS only
    if (S > 1) {
        const size_t tl = (size_t)p.n_tiles * p.mb_per_launch;
        const size_t part = tl * S * SK_MT * SK_RPT * 4;
        const size_t ssq = tl * S * SK_MT * 4;
        p.ws_bytes = (part + 255) / 256 * 256 + (ssq + 255) / 256 * 256;
    }
    return p;
}

template <int EPI, bool NORM, int NST>
static hipError_t mfma_launch_t(const GemvDev& d, const GemvPlan& p, hipStream_t s) {
    for (int mb0 = 0; mb0 < p.mblocks; mb0 += p.mb_per_launch) {
        GemvDev dl = d;
        dl.mb0 = mb0;
        dim3 grid(p.n_tiles, p.splits, min(p.mb_per_launch, p.mblocks - mb0));
        hipLaunchKernelGGL((gemv_mfma_kernel<EPI, NORM, NST>), grid, dim3(p.threads), 0, s, dl);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (p.splits > 1) {
            hipLaunchKernelGGL((gemv_mfma_merge_kernel<EPI, NORM>), dim3(p.n_tiles, 1, grid.z), dim3(256), 0, s, dl);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

template <int EPI, bool NORM>
static hipError_t mfma_launch_kc(const GemvDev& d, const GemvPlan& p, hipStream_t s) {
    switch (p.kc) {
        case 8 * SK_SUB: return mfma_launch_t<EPI, NORM, 8>(d, p, s);
        case 4 * SK_SUB: return mfma_launch_t<EPI, NORM, 4>(d, p, s);
        case 2 * SK_SUB: return mfma_launch_t<EPI, NORM, 2>(d, p, s);
        case SK_SUB: return mfma_launch_t<EPI, NORM, 1>(d, p, s);
    }
    return hipErrorInvalidValue;
}

hipError_t gemv_mfma_launch(const GemvDev& d, const GemvPlan& p, hipStream_t s) {
    const bool nrm = d.a.norm != 0;
    switch (d.a.epi) {
        case EPI_STORE:
            return nrm ? mfma_launch_kc<EPI_STORE, true>(d, p, s) : mfma_launch_kc<EPI_STORE, false>(d, p, s);
        case EPI_PARTIAL: return mfma_launch_kc<EPI_PARTIAL, false>(d, p, s);
        case EPI_SWIGLU:
            return nrm ? mfma_launch_kc<EPI_SWIGLU, true>(d, p, s) : mfma_launch_kc<EPI_SWIGLU, false>(d, p, s);
        case EPI_QKV:
            return nrm ? mfma_launch_kc<EPI_QKV, true>(d, p, s) : mfma_launch_kc<EPI_QKV, false>(d, p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tpk
