// Thin-M projections for decode on gfx950: column-parallel (optionally with
// fused RMSNorm, SwiGLU or KV-cache append) and row-parallel partials.
//
// Decode reads each weight byte once and does M multiply-adds with it, so the
// kernel is bound by HBM for small M and close to the VALU limit at M = 16.
// A decode-sized matrix is only a few HBM latencies' worth of bytes, so the
// design goal is to have every byte requested as early as possible:
//  - A workgroup (4 waves) owns a tile of weight rows and one K chunk. Each
//    wave owns RW rows; one load instruction reads 1 KB of one row (64 lanes
//    x 128 bits), and the plan sizes the chunk so that a lane's whole share
//    (at most PF vectors per row) is requested at the start, before anything
//    else happens. No loop carries loads.
//  - The activation chunk [MT, kc] is staged in LDS once per workgroup (gamma
//    folded in when RMSNorm is fused) and read by every row of the tile.
//  - bf16 products use v_dot2 (two multiply-adds per lane per instruction,
//    float32 accumulation, no unpacking); float32 inputs use fma.
//  - The 64 lanes of a row are reduced by a reduce-scatter: permlane32/16 swaps
//    across rows, then DPP within rows, in a fixed order; each lane ends with
//    its share of the sums, which pass through a small LDS tile so the
//    epilogue writes outputs in coalesced order.
//  - When K is split over S workgroups, each publishes its float32 tile with
//    agent-scope coherent stores and bumps a per-tile counter; the last to
//    arrive sums the S slices in split order (deterministic), runs the
//    epilogue and resets the counter. No cache-wide fence is needed. RMSNorm's
//    sum of squares travels the same way, so the normalisation stays fused:
//    inv_rms multiplies the contraction result.
#include "gemv_tile.h"

namespace tpk {

constexpr size_t GEMV_X_LDS = 64 * 1024;   // LDS budget for the staged activation chunk
constexpr int GEMV_NW = 4;                 // waves per workgroup

// Per token-block size: rows per wave (RW) and the most K steps a lane keeps
// in flight (PF). A step is one 128-bit vector per lane, 64 lanes wide.
template <int MT> struct RowsPerWave { static constexpr int v = MT >= 8 ? 4 : 2; };
template <int MT> struct StepsInFlight { static constexpr int v = MT >= 8 ? 4 : 8; };
static int rows_per_wave(int mt) { return mt >= 8 ? 4 : 2; }
static int steps_in_flight(int mt) { return mt >= 8 ? 4 : 8; }

template <typename T> struct Elem;
template <> struct Elem<uint16_t> { static constexpr int vec = 8; };
template <> struct Elem<float> { static constexpr int vec = 4; };

// acc[m] += dot(w, x) over one 128-bit vector.
__device__ __forceinline__ float vdot(const uint4& w, const uint4& x, float acc, uint16_t*) {
    acc = dot2_bf16(w.x, x.x, acc);
    acc = dot2_bf16(w.y, x.y, acc);
    acc = dot2_bf16(w.z, x.z, acc);
    acc = dot2_bf16(w.w, x.w, acc);
    return acc;
}
__device__ __forceinline__ float vdot(const uint4& w, const uint4& x, float acc, float*) {
    acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
    acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
    acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
    acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
    return acc;
}

template <typename T, int MT, int EPI, bool NORM>
__global__ __launch_bounds__(GEMV_NW * 64) void gemv_kernel(GemvDev d) {
    constexpr int NW = GEMV_NW;
    constexpr int NT = NW * 64;
    constexpr int VEC = Elem<T>::vec;
    constexpr int RW = RowsPerWave<MT>::v;
    constexpr int PF = StepsInFlight<MT>::v;
    constexpr int RPT = NW * RW;             // weight rows per workgroup
    constexpr bool SWI = (EPI == EPI_SWIGLU);
    constexpr int HALF = RPT / 2;
    constexpr int STEP = 64 * VEC;           // K elements of one row per wave instruction
    constexpr int NV = RW * MT;              // sums per lane before the wave reduction
    constexpr int NKEEP = NV >= 64 ? NV / 64 : 1;

    const GemvArgs& a = d.a;
    constexpr int XW = PF * STEP;            // staged activation row length (elements)
    constexpr int RPWV = (MT + NW - 1) / NW; // activation rows a wave stages
    extern __shared__ __align__(16) unsigned char smem[];
    T* xs = reinterpret_cast<T*>(smem);                                        // [MT][XW]
    float* res = reinterpret_cast<float*>(smem + (size_t)MT * XW * sizeof(T));  // [MT][RPT]
    float* ssl = res + MT * RPT;                                               // [MT]
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tile = d.tile0 + blockIdx.x, split = blockIdx.y, mb = d.mb0 + blockIdx.z;
    const int K = a.K, N = a.N;
    const int k0 = split * d.kc;
    const int klen = min(d.kc, K - k0);      // a multiple of VEC, at most XW
    const int m0 = mb * MT;
    const int mvalid = min(MT, a.m - m0);

    // Weight rows of this wave. Rows past N are clamped to a valid row; their
    // results are never stored.
    const T* wrow[RW];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int rho = wave * RW + r;
        int n;
        const T* base;
        if (SWI) {
            n = tile * HALF + (rho < HALF ? rho : rho - HALF);
            base = reinterpret_cast<const T*>(rho < HALF ? a.w : a.w_up);
        } else {
            n = tile * RPT + rho;
            base = reinterpret_cast<const T*>(a.w);
        }
        n = min(n, N - 1);
        wrow[r] = base + (size_t)n * K + k0;
    }

    // Loads are issued in the order they are needed and without control flow:
    // activations (and gamma) first, then the lane's whole share of weights.
    // Offsets past the chunk are clamped to its last vector and the value
    // zeroed, so every load is in bounds and none is conditional; waiting for
    // the activations then leaves every weight load in flight.
    const T* x = reinterpret_cast<const T*>(a.x);
    const T* gam = reinterpret_cast<const T*>(a.gamma);
    const bool stager = (MT >= NW) || (wave < MT);   // waves with activation rows to stage
    uint4 xr[RPWV][PF];
    uint4 gr[PF];
    if (stager) {
#pragma unroll
        for (int i = 0; i < RPWV; ++i) {
            const int mm = wave + i * NW;
            const int row = m0 + min(mm, mvalid - 1);
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const int k = (u * 64 + lane) * VEC;
                const bool ok = mm < mvalid && k < klen;
                const uint4 v = load_u4(x + (size_t)row * K + k0 + min(k, klen - VEC));
                xr[i][u] = ok ? v : make_uint4(0, 0, 0, 0);
            }
        }
        if (NORM) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                const int k = (u * 64 + lane) * VEC;
                gr[u] = load_u4(gam + k0 + min(k, klen - VEC));
            }
        }
    }
    uint4 wv[PF][RW];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        const int k = (u * 64 + lane) * VEC;
        const int kk = min(k, klen - VEC);
#pragma unroll
        for (int r = 0; r < RW; ++r) {
            const uint4 v = load_stream_u4(wrow[r] + kk);
            wv[u][r] = k < klen ? v : make_uint4(0, 0, 0, 0);
        }
    }

    // Stage the activation rows (times gamma) in LDS with their sums of squares.
    if (stager) {
#pragma unroll
        for (int i = 0; i < RPWV; ++i) {
            const int mm = wave + i * NW;
            if (mm >= MT) break;
            float ss = 0.f;
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                uint4 v = xr[i][u];
                if (NORM) {
                    ss += vsumsq(v, (T*)nullptr);
                    v = vscale(v, gr[u], (T*)nullptr);
                }
                *reinterpret_cast<uint4*>(xs + (size_t)mm * XW + (u * 64 + lane) * VEC) = v;
            }
            if (NORM) {
                ss = wave_sum(ss);
                if (lane == 0) ssl[mm] = ss;
            }
        }
    }
    __syncthreads();

    float acc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) acc[i] = 0.f;
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        const int k = (u * 64 + lane) * VEC;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4 xv = *reinterpret_cast<const uint4*>(xs + (size_t)m * XW + k);
#pragma unroll
            for (int r = 0; r < RW; ++r) acc[r * MT + m] = vdot(wv[u][r], xv, acc[r * MT + m], (T*)nullptr);
        }
    }

    // Reduce every (row, token) sum over the wave's 64 lanes and scatter the
    // results; each lane writes its share of the tile to LDS.
    reduce_scatter64<NV>(acc, lane);
#pragma unroll
    for (int j = 0; j < NKEEP; ++j) {
        bool owner;
        const int idx = reduce64_index<NV>(lane, j, owner);
        if (owner) {
            const int r = idx / MT, m = idx % MT;
            res[m * RPT + wave * RW + r] = acc[j];
        }
    }
    __syncthreads();

    gemv_finish<T, MT, RPT, EPI, NORM, NT>(d, res, ssl, &s_last, tile, split, m0, mvalid);
}

GemvPlan gemv_plan_dot2(int m, int K, int N, int is_bf16, int epi) {
    GemvPlan p{};
    p.mt = m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : m <= 8 ? 8 : 16;
    if (!is_bf16 && p.mt != 1 && p.mt != 4) p.mt = (m <= 4) ? 4 : 16;
    p.mblocks = (m + p.mt - 1) / p.mt;
    p.mbw = 1;
    p.nw = GEMV_NW;
    p.rows_per_tile = GEMV_NW * rows_per_wave(p.mt);
    p.out_per_tile = (epi == EPI_SWIGLU) ? p.rows_per_tile / 2 : p.rows_per_tile;
    p.n_tiles = (N + p.out_per_tile - 1) / p.out_per_tile;
    const int esz = is_bf16 ? 2 : 4;
    const int step = 64 * (16 / esz);
    const int kround = (K + step - 1) / step * step;
    // A chunk is at most PF steps (every load of a lane in flight at once) and
    // its activations must fit the LDS budget.
    int kc_max = steps_in_flight(p.mt) * step;
    const int kc_lds = (int)(GEMV_X_LDS / ((size_t)p.mt * esz)) / step * step;
    if (kc_lds < kc_max) kc_max = kc_lds;
    if (kc_max > kround) kc_max = kround;
    // Shrink the chunk (more K splits) while the grid is short of about two
    // workgroups per compute unit, down to two steps per chunk.
    const long target = 512;
    int kc = kc_max;
    while (kc > 2 * step && (long)p.n_tiles * ((kround + kc - 1) / kc) * p.mblocks < target) kc -= step;
    int S = (K + kc - 1) / kc;
    p.mb_per_launch = p.mblocks;
    p.tiles_per_launch = p.n_tiles;
    if (S > 1 && (size_t)p.n_tiles * p.mblocks > (size_t)WS_MAX_COUNTERS) {
        // One counter per (tile, m-block) of a launch: run the m-blocks, and
        // when the tiles alone are too many, ranges of tiles, in launches that
        // fit the header.
        if (p.n_tiles > WS_MAX_COUNTERS) {
            p.tiles_per_launch = WS_MAX_COUNTERS;
            p.mb_per_launch = 1;
        } else {
            p.mb_per_launch = WS_MAX_COUNTERS / p.n_tiles;
        }
    }
    const size_t tiles = (size_t)p.tiles_per_launch * p.mb_per_launch;
    p.kc = kc;
    p.splits = S;
    p.threads = GEMV_NW * 64;
    p.lds_bytes = (size_t)p.mt * steps_in_flight(p.mt) * step * esz + (size_t)p.mt * p.rows_per_tile * 4 +
                  (size_t)p.mt * 4;
    if (S > 1) {
        const size_t part = tiles * S * p.mt * p.rows_per_tile * 4;
        const size_t ssq = tiles * S * p.mt * 4;
        p.ws_bytes = (part + 255) / 256 * 256 + (ssq + 255) / 256 * 256;
    } else {
        p.ws_bytes = 0;
    }
    return p;
}

GemvPlan gemv_plan(int m, int K, int N, int is_bf16, int epi) {
    // bf16 blocks of two tokens or more go to the matrix cores (measured on the
    // 8B and 70B shard projections: 2-4 tokens up to 24% faster there than on
    // v_dot2 and at most 3% slower, a single token 8% slower on the 8B
    // gate/up); one token (and float32) stays on v_dot2 / fma
    if (is_bf16 && m >= GEMV_MFMA_MIN_M) return gemv_plan_mfma(m, K, N, epi);
    return gemv_plan_dot2(m, K, N, is_bf16, epi);
}

template <typename T, int MT, int EPI, bool NORM>
static hipError_t launch_t(const GemvDev& d, const GemvPlan& p, hipStream_t s) {
    auto kern = gemv_kernel<T, MT, EPI, NORM>;
    // Raise the dynamic LDS limit once per instantiation (outside any graph capture
    // in practice: the first call of a shape is an eager one).
    static bool lds_raised = false;
    if (p.lds_bytes > 64 * 1024 && !lds_raised) {
        // the most this instantiation can ask for: the activation budget plus its result tile
        const int most = (int)p.lds_bytes;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, most);
        if (e != hipSuccess) {
            (void)hipGetLastError();   // do not leave the error pending for the caller's next HIP call
            return e;
        }
        lds_raised = true;
    }
    for (int mb0 = 0; mb0 < p.mblocks; mb0 += p.mb_per_launch) {
        for (int t0 = 0; t0 < p.n_tiles; t0 += p.tiles_per_launch) {
            GemvDev dl = d;
            dl.mb0 = mb0;
            dl.tile0 = t0;
            dim3 grid(min(p.tiles_per_launch, p.n_tiles - t0), p.splits, min(p.mb_per_launch, p.mblocks - mb0));
            hipLaunchKernelGGL(kern, grid, dim3(p.threads), p.lds_bytes, s, dl);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

template <typename T, int MT>
static hipError_t launch_mt(const GemvDev& d, const GemvPlan& p, hipStream_t s) {
    const bool nrm = d.a.norm != 0;
    switch (d.a.epi) {
        case EPI_STORE:
            return nrm ? launch_t<T, MT, EPI_STORE, true>(d, p, s) : launch_t<T, MT, EPI_STORE, false>(d, p, s);
        case EPI_PARTIAL: return launch_t<T, MT, EPI_PARTIAL, false>(d, p, s);
        case EPI_SWIGLU:
            return nrm ? launch_t<T, MT, EPI_SWIGLU, true>(d, p, s) : launch_t<T, MT, EPI_SWIGLU, false>(d, p, s);
        case EPI_QKV:
            if constexpr (sizeof(T) == 2)
                return nrm ? launch_t<T, MT, EPI_QKV, true>(d, p, s) : launch_t<T, MT, EPI_QKV, false>(d, p, s);
            break;
    }
    return hipErrorInvalidValue;
}

hipError_t gemv_launch(const GemvArgs& a, const GemvPlan& p, unsigned* counters, void* scratch, hipStream_t s) {
    GemvDev d{};
    d.a = a;
    d.kc = p.kc;
    d.splits = p.splits;
    d.n_tiles = p.n_tiles;
    d.opt = p.out_per_tile;
    if (p.splits > 1) {
        const size_t tiles = (size_t)p.tiles_per_launch * p.mb_per_launch;
        char* b = reinterpret_cast<char*>(scratch);
        const size_t part = (tiles * p.splits * p.mt * p.rows_per_tile * 4 + 255) / 256 * 256;
        d.cnt = counters;
        d.part = reinterpret_cast<float*>(b);
        d.ssq = reinterpret_cast<float*>(b + part);
    }
    if (p.mfma) return a.is_bf16 ? gemv_mfma_launch(d, p, s) : hipErrorInvalidValue;
    if (a.is_bf16) {
        switch (p.mt) {
            case 1: return launch_mt<uint16_t, 1>(d, p, s);
            case 2: return launch_mt<uint16_t, 2>(d, p, s);
            case 4: return launch_mt<uint16_t, 4>(d, p, s);
            case 8: return launch_mt<uint16_t, 8>(d, p, s);
            case 16: return launch_mt<uint16_t, 16>(d, p, s);
        }
    } else {
        if (a.epi == EPI_QKV) return hipErrorInvalidValue;
        switch (p.mt) {
            case 1: return launch_mt<float, 1>(d, p, s);
            case 4: return launch_mt<float, 4>(d, p, s);
            case 16: return launch_mt<float, 16>(d, p, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace tpk
