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
//  - A wave owns 16 weight rows and a K range, walked in stages of 256
//    elements with two stages of loads in flight: the loads of stage i + 1
//    are requested before stage i is used. Loads return in order, so each
//    stage's activations and weights are requested together, in the order
//    they are consumed.
//  - The waves that share a K range share its activations: per stage they
//    are staged once (16 tokens x 256, padded with zeros, times gamma when
//    RMSNorm is fused, their squares summed); each wave stages its own 16
//    weight rows. Rows are padded by 16 bytes so the operand reads of 16
//    rows hit distinct banks.
//  - Wide projections: 8 waves per workgroup, 2 per K range (32 rows: for
//    SwiGLU the gate and up rows of 16 outputs) and 4 K ranges, whose sums
//    are added in LDS before the epilogue (SwiGLU over 512 tiles or more: 2
//    K ranges, 4 waves, three workgroups per compute unit). One kernel,
//    nothing in memory between the slices.
//  - Narrow projections (too few 32-row tiles to fill the chip): 4 waves
//    share one K range of a 64-row tile and K is split over workgroups. Each
//    writes its float32 slice with plain stores and a small merge kernel (one
//    workgroup per tile) adds the slices in split order and runs the
//    epilogue: no counter vote, whose memory round trips would sit at the
//    end of the projection kernel.
//  - Unsplit, the results (lane: one weight row, four tokens) go through an
//    LDS tile to the epilogue shared with the v_dot2 kernel.
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

// NST: stages per K range (a K range is NST * 256 elements). RG: waves that
// share a K range, 16 weight rows each (the tile is 16 * RG rows). KS: K
// ranges a workgroup covers, its wave groups' sums added in LDS at the end.
// Split across workgroups (gridDim.y > 1) only with KS == 1.
template <int EPI, bool NORM, int NST, int RG, int KS>
__global__ __launch_bounds__(RG * KS * 64) void gemv_mfma_kernel(GemvDev d) {
    constexpr int NT = RG * KS * 64;
    constexpr int GT = RG * 64;                 // threads of a wave group
    constexpr int RPT = RG * 16;                // weight rows per workgroup
    constexpr int XV = 8 / RG;                  // activation vectors a thread stages per stage
    constexpr int TSTEP = 2 * RG;               // tokens between them
    constexpr bool SWI = (EPI == EPI_SWIGLU);
    constexpr int HALF = RPT / 2;
    static_assert(!SWI || RG % 2 == 0, "a SwiGLU tile pairs gate and up waves");
    __shared__ __align__(16) uint16_t wl[RG * KS][16 * SK_PITCH];
    __shared__ __align__(16) uint16_t xl[KS][SK_MT * SK_PITCH];
    __shared__ float res[SK_MT * RPT];
    __shared__ float ssl[KS][SK_MT];

    const GemvArgs& a = d.a;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rg = wave % RG, grp = wave / RG, gtid = tid % GT;
    const int tile = blockIdx.x, split = blockIdx.y, mb = d.mb0 + blockIdx.z;
    const int K = a.K, N = a.N;
    const int kbase = (split * KS + grp) * (NST * SK_SUB);
    const int m0 = mb * SK_MT;
    const int mvalid = min(SK_MT, a.m - m0);
    const int col = lane & 15, kg = lane >> 4;

    // Loads of a stage. Lane: element offset (lane & 31) * 8 of the stage.
    //  - weights: vector q covers the wave's rows 2q and 2q + 1 (half-waves);
    //  - activations: the group's thread g stages tokens g / 32 + 2 RG i and
    //    gamma.
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
        if (SWI) {                             // first half of the group: gate rows, second: up rows of the same outputs
            constexpr int HR = RG / 2;
            n = tile * HALF + (rg % HR) * 16 + r;
            base = reinterpret_cast<const uint16_t*>(rg < HR ? a.w : a.w_up);
        } else {
            n = tile * RPT + rg * 16 + r;
            base = reinterpret_cast<const uint16_t*>(a.w);
        }
        wrow[q] = base + (size_t)min(n, N - 1) * K;
    }
    const int t0 = gtid >> 5;
    const uint16_t* xrow[XV];
    bool tok_ok[XV];
#pragma unroll
    for (int i = 0; i < XV; ++i) {
        const int t = t0 + TSTEP * i;
        tok_ok[i] = t < mvalid;
        xrow[i] = reinterpret_cast<const uint16_t*>(a.x) + (size_t)(m0 + min(t, mvalid - 1)) * K;
    }
    const uint16_t* gam = reinterpret_cast<const uint16_t*>(a.gamma);
    uint16_t* xg = xl[grp];

    struct Stage { uint4 w[SK_WL]; uint4 x[XV]; uint4 g; };
    auto issue = [&](Stage& b, int st) {
        const int kk = min(kbase + st * SK_SUB + ve, K - 8);
#pragma unroll
        for (int i = 0; i < XV; ++i) b.x[i] = load_u4(xrow[i] + kk);
        if (NORM) b.g = load_u4(gam + kk);
#pragma unroll
        for (int q = 0; q < SK_WL; ++q) b.w[q] = load_stream_u4(wrow[q] + kk);
    };

    const uint4 zero = make_uint4(0, 0, 0, 0);
    float ss[XV];
#pragma unroll
    for (int i = 0; i < XV; ++i) ss[i] = 0.f;
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
        for (int i = 0; i < XV; ++i) {
            uint4 v = cur.x[i];
            if (!(tok_ok[i] && kin)) v = zero;
            if (NORM) {
                ss[i] += vsumsq(v, (uint16_t*)nullptr);
                v = vscale(v, cur.g, (uint16_t*)nullptr);
            }
            *reinterpret_cast<uint4*>(xg + (t0 + TSTEP * i) * SK_PITCH + ve) = v;
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
            const uint4 xa = *reinterpret_cast<const uint4*>(xg + col * SK_PITCH + s * 32 + kg * 8);
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
        // the 32 lanes of a half-wave hold the same tokens
#pragma unroll
        for (int i = 0; i < XV; ++i) {
            float v = ss[i];
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
            if ((lane & 31) == 0) ssl[grp][t0 + TSTEP * i] = v;
        }
    }
    if (KS == 1 && d.splits > 1) {
        if (NORM) __syncthreads();             // ssl written by the stagers
        // This split's slice goes out with plain stores; the merge kernel that
        // follows on the stream adds the slices and runs the epilogue.
        const int tile_id = blockIdx.z * d.n_tiles + tile;
        float* mine = d.part + ((size_t)tile_id * d.splits + split) * (SK_MT * RPT);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (4 * kg + j < mvalid) mine[(4 * kg + j) * RPT + rg * 16 + col] = acc[j];
        if (NORM && tid < mvalid) d.ssq[((size_t)tile_id * d.splits + split) * SK_MT + tid] = ssl[0][tid];
        return;
    }
    if (KS == 1) {
        // lane holds tokens 4 kg + j of row rg * 16 + col
#pragma unroll
        for (int j = 0; j < 4; ++j) res[(4 * kg + j) * RPT + rg * 16 + col] = acc[j];
    } else {
        // Every wave parks its sums in its own weight tile; the K ranges'
        // sums are then added in range order (deterministic).
        __syncthreads();
        float* park = reinterpret_cast<float*>(wl[wave]);
#pragma unroll
        for (int j = 0; j < 4; ++j) park[(4 * kg + j) * 16 + col] = acc[j];
        __syncthreads();
        for (int e = tid; e < SK_MT * RPT; e += NT) {
            const int m = e / RPT, rr = e - m * RPT;
            float v = 0.f;
#pragma unroll
            for (int g = 0; g < KS; ++g)
                v += reinterpret_cast<const float*>(wl[g * RG + (rr >> 4)])[m * 16 + (rr & 15)];
            res[e] = v;
        }
        if (NORM && tid < SK_MT) {
            float v = 0.f;
#pragma unroll
            for (int g = 0; g < KS; ++g) v += ssl[g][tid];
            ssl[0][tid] = v;
        }
    }
    __syncthreads();
    gemv_epilogue<uint16_t, SK_MT, RPT, EPI, NORM, NT>(a, res, ssl[0], tile, m0, mvalid);
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
    p.mb_per_launch = p.mblocks;                // the merge uses no counters
    p.lds_bytes = 0;                            // static LDS only
    const bool swi = epi == EPI_SWIGLU;
    const int64_t mb = p.mblocks;
    // Wide projections: one workgroup per tile of 16 outputs (SwiGLU: 16
    // gate and 16 up rows; otherwise 32 rows), its K range split over 4 wave
    // groups of 2 waves (2 groups for SwiGLU over 512 tiles or more) whose
    // sums meet in LDS: no second kernel and no float32 slices in memory.
    // Taken when that gives at least 128 (SwiGLU) or 192 workgroups;
    // measured on replayed 8B MLP and 70B attention projection steps,
    // narrower projections stream better as 64-row tiles split over
    // workgroups.
    const int64_t t2 = swi ? (N + 15) / 16 : (N + 31) / 32;
    int rg = SK_NW, ks = 1;
    if (t2 * mb >= (swi ? 128 : 192) && K <= 4 * SK_MAX_STAGES * SK_SUB) {
        rg = 2;
        // SwiGLU over many tiles (the stacked experts): two K ranges, so three
        // 4-wave workgroups share a compute unit.
        ks = (swi && t2 * mb >= 512 && K <= 2 * SK_MAX_STAGES * SK_SUB) ? 2 : 4;
    }
    p.rg = rg;
    p.ks = ks;
    p.nw = rg * ks;
    p.threads = p.nw * 64;
    p.rows_per_tile = 16 * rg;
    p.out_per_tile = swi ? 8 * rg : 16 * rg;
    p.n_tiles = (N + p.out_per_tile - 1) / p.out_per_tile;
    if (ks > 1) {
        int kc = SK_SUB;
        while (kc * ks < K) kc *= 2;            // at most SK_MAX_STAGES stages by the guard above
        p.kc = kc;
        p.splits = 1;
        return p;
    }
    // Narrow projections, 4 waves per 64-row tile, K split over workgroups.
    // K chunk: 1024 or 2048 elements, the smaller when the launch then has
    // at most 256 workgroups (512 for SwiGLU tiles), and shorter chunks only
    // for launches that would otherwise have fewer than 128 workgroups. Measured
    // in replayed graphs on the 8B MLP and 70B attention and MLP shard shapes:
    // about one workgroup per compute unit streams best, more splits cost
    // merge traffic and a longer tail, and chunks under 1024 gain nothing
    // once about half the compute units are busy.
    const int64_t tiles = (int64_t)p.n_tiles * mb;
    const int64_t lim = swi ? 512 : 256;
    auto wgs = [&](int c) { return tiles * ((K + c - 1) / c); };
    int kc = 4 * SK_SUB;
    while (kc < SK_MAX_STAGES * SK_SUB && wgs(kc) > lim) kc *= 2;
    while (kc > SK_SUB && wgs(kc) < 128 && wgs(kc / 2) <= lim) kc /= 2;
    while (kc > SK_SUB && kc / 2 >= K) kc /= 2;   // no stage past the end of K
    const int S = (K + kc - 1) / kc;
    p.kc = kc;
    p.splits = S;
    if (S > 1) {
        const size_t tl = (size_t)p.n_tiles * p.mb_per_launch;
        const size_t part = tl * S * SK_MT * SK_RPT * 4;
        const size_t ssq = tl * S * SK_MT * 4;
        p.ws_bytes = (part + 255) / 256 * 256 + (ssq + 255) / 256 * 256;
    }
    return p;
}

template <int EPI, bool NORM, int NST, int RG, int KS>
static hipError_t mfma_launch_t(const GemvDev& d, const GemvPlan& p, hipStream_t s) {
    for (int mb0 = 0; mb0 < p.mblocks; mb0 += p.mb_per_launch) {
        GemvDev dl = d;
        dl.mb0 = mb0;
        dim3 grid(p.n_tiles, p.splits, min(p.mb_per_launch, p.mblocks - mb0));
        hipLaunchKernelGGL((gemv_mfma_kernel<EPI, NORM, NST, RG, KS>), grid, dim3(RG * KS * 64), 0, s, dl);
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

template <int EPI, bool NORM, int RG, int KS>
static hipError_t mfma_launch_kc(const GemvDev& d, const GemvPlan& p, hipStream_t s) {
    switch (p.kc) {
        case 8 * SK_SUB: return mfma_launch_t<EPI, NORM, 8, RG, KS>(d, p, s);
        case 4 * SK_SUB: return mfma_launch_t<EPI, NORM, 4, RG, KS>(d, p, s);
        case 2 * SK_SUB: return mfma_launch_t<EPI, NORM, 2, RG, KS>(d, p, s);
        case SK_SUB: return mfma_launch_t<EPI, NORM, 1, RG, KS>(d, p, s);
    }
    return hipErrorInvalidValue;
}

template <int EPI, bool NORM>
static hipError_t mfma_launch_shape(const GemvDev& d, const GemvPlan& p, hipStream_t s) {
    if (p.rg == SK_NW && p.ks == 1) return mfma_launch_kc<EPI, NORM, SK_NW, 1>(d, p, s);
    if (p.rg == 2 && p.ks == 4) return mfma_launch_kc<EPI, NORM, 2, 4>(d, p, s);
    if constexpr (EPI == EPI_SWIGLU) {
        if (p.rg == 2 && p.ks == 2) return mfma_launch_kc<EPI, NORM, 2, 2>(d, p, s);
    }
    return hipErrorInvalidValue;
}

hipError_t gemv_mfma_launch(const GemvDev& d, const GemvPlan& p, hipStream_t s) {
    if (p.splits > 1 && p.ks != 1) return hipErrorInvalidValue;
    const bool nrm = d.a.norm != 0;
    switch (d.a.epi) {
        case EPI_STORE:
            return nrm ? mfma_launch_shape<EPI_STORE, true>(d, p, s) : mfma_launch_shape<EPI_STORE, false>(d, p, s);
        case EPI_PARTIAL: return mfma_launch_shape<EPI_PARTIAL, false>(d, p, s);
        case EPI_SWIGLU:
            return nrm ? mfma_launch_shape<EPI_SWIGLU, true>(d, p, s) : mfma_launch_shape<EPI_SWIGLU, false>(d, p, s);
        case EPI_QKV:
            return nrm ? mfma_launch_shape<EPI_QKV, true>(d, p, s) : mfma_launch_shape<EPI_QKV, false>(d, p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tpk
