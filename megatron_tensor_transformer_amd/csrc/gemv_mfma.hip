// Decode projections of 2 to 64 tokens on the matrix cores
// (v_mfma_f32_16x16x32_bf16), in blocks of 16 tokens.
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
// bytes or more per row stream at full rate. So weights pass through LDS on
// their way to the operand registers. Two kernels:
//  - Wide projections (gemv_mfma_wide_kernel): a workgroup of 8 waves takes
//    32 or 16 weight rows over all of K, one K range per wave. Weights go by
//    DMA into the wave's own LDS tiles (4 rows x 256 bytes per transfer),
//    activation operands are read straight from memory, and the waves meet
//    only when their sums are added at the end: no workgroup barrier while
//    streaming. Above 16 tokens, unless K is split over workgroups, a
//    workgroup takes two token blocks, each weight fragment feeding one MFMA
//    per block, so the weights stream once per 32 tokens. Where K is also
//    split over workgroups (narrow outputs), each
//    publishes its float32 slice with coherent stores and the last of them
//    to arrive adds the slices and runs the epilogue: no second kernel.
//  - Narrow projections and the stacked experts (gemv_mfma_kernel): waves
//    own 16 rows each and share a K range, walked in stages of 256 elements
//    with two stages of loads in flight; weights are read as 2 rows x 512
//    bytes per instruction and written to a wave-private LDS tile (rows
//    padded by 16 bytes so the operand reads of 16 rows hit distinct banks),
//    and the waves sharing a K range stage its activations once per stage
//    (16 tokens x 256, zero-padded, times gamma when RMSNorm is fused, their
//    squares summed), alternating between two LDS stages so a stage costs
//    one barrier. Narrow projections (too few tiles to fill the chip) use 4
//    waves per 64-row tile and split K over workgroups: each writes its
//    float32 slice with plain stores and a small merge kernel (one workgroup
//    per tile) adds the slices in split order and runs the epilogue. The
//    stacked experts' SwiGLU uses 4-wave workgroups of two K ranges whose
//    sums meet in LDS, three workgroups per compute unit.
//  - Either way the results (lane: one weight row, four tokens) reach the
//    epilogue shared with the v_dot2 kernel through an LDS tile.
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

// K split over workgroups: every split publishes its tile's sums res[m][RPT]
// (and, with a fused RMSNorm, its squared-sum slice ssl[m]) with coherent
// stores, and the last of the tile's splits to arrive adds the slices in
// split order (deterministic) into res and ssl. Returns true in that
// workgroup, which then runs the epilogue; the others return. A thread's
// loads of its element's slices are in flight together.
template <int RPT, bool NORM, int NT>
__device__ __forceinline__ bool split_merge(const GemvDev& d, float* res, float* ssl, int tile_id, int split,
                                            int mvalid, int* s_last) {
    const int tid = threadIdx.x, S = d.splits;
    float* base = d.part + (size_t)tile_id * S * (SK_MT * RPT);
    float* sqb = d.ssq + (size_t)tile_id * S * SK_MT;
    const int live = mvalid * RPT;              // token rows past m are never read back
    for (int e = tid; e < live; e += NT) store_coherent(base + (size_t)split * (SK_MT * RPT) + e, res[e]);
    if (NORM && tid < mvalid) store_coherent(sqb + (size_t)split * SK_MT + tid, ssl[tid]);
    if (!last_arriver(&d.cnt[tile_id], (unsigned)S, s_last)) return false;
    constexpr int UNR = 4;
    for (int e = tid; e < live; e += NT) {
        float v = 0.f;
        for (int sp0 = 0; sp0 < S; sp0 += UNR) {
            float u[UNR];
#pragma unroll
            for (int i = 0; i < UNR; ++i) u[i] = load_coherent(base + (size_t)min(sp0 + i, S - 1) * (SK_MT * RPT) + e);
#pragma unroll
            for (int i = 0; i < UNR; ++i)
                if (sp0 + i < S) v += u[i];
        }
        res[e] = v;
    }
    if (NORM && tid < mvalid) {
        float v = 0.f;
        for (int sp = 0; sp < S; ++sp) v += load_coherent(sqb + (size_t)sp * SK_MT + tid);
        ssl[tid] = v;
    }
    __syncthreads();
    return true;
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
    // Activation stages in LDS: two let a stage be written while the other is
    // still being read, so one barrier per stage suffices. The layout that
    // packs three workgroups per compute unit keeps one (LDS decides how many
    // fit).
    constexpr int XB = (RG == 2 && KS == 2) ? 1 : 2;
    static_assert(!SWI || RG % 2 == 0, "a SwiGLU tile pairs gate and up waves");
    __shared__ __align__(16) uint16_t wl[RG * KS][16 * SK_PITCH];
    __shared__ __align__(16) uint16_t xl[XB][KS][SK_MT * SK_PITCH];
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
        // With one activation stage, every wave must be done reading the
        // previous one. With two, the barrier that ended the previous stage's
        // writes also ended the reads of the one before it. The weight tile is
        // the wave's own: its reads of the previous stage precede these writes.
        if (XB == 1 && st > 0) __syncthreads();
        uint16_t* xg = xl[st % XB][grp];
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
        // follows on the stream adds the slices and runs the epilogue (an
        // in-kernel merge by the last split to arrive measured slower here:
        // 70B attention projections at t=4, 89.2 -> 93.2 us per step).
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

// Wide projections, one wave per K range. A workgroup of 8 waves covers ROWS
// (32 or 16) weight rows over all of K (for SwiGLU the gate and up rows of
// ROWS / 2 outputs); wave w takes the w-th eighth of K in stages of 128
// elements. Each wave moves its stage of weights (ROWS rows x 256 bytes) from
// HBM into its own ring of LDS tiles by DMA (two for 32 rows, four for 16), and reads its
// activation operands straight from memory (the 16 tokens' rows stay in L2;
// their bytes are 16 / ROWS of the weights'). No wave waits for another until
// the K ranges' sums meet in LDS, and no weight passes through registers on
// its way to LDS. Rows are 256 bytes, unpadded: a row's 16-byte chunks are
// XOR-swizzled by the row index, so the 16 rows of an operand read fall in
// distinct banks. Chunks past K and rows past N are fetched out of their
// buffer's range and arrive as zeros. 16-row workgroups serve projections
// with too few 32-row tiles to fill the chip, without splitting K over
// workgroups.
constexpr int WD_NW = 8;                        // waves, one K range each
constexpr int WD_SUB = 128;                     // K elements per stage
constexpr int WD16_NBUF = 4;                    // stage tiles per wave with 16 rows (32 rows: 2, LDS-bound)
constexpr unsigned WD_OOB = 0x80000000u;        // an offset past every buffer's range

// s_waitcnt immediate waiting until at most n vector-memory operations are
// outstanding (LDS and export counts left at their maxima).
__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wd_view(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// Weights are read once: the transfer is marked non-temporal (the nt bit of
// the cache policy), like the streamed loads of the other kernels.
__device__ __forceinline__ void wd_dma16(__amdgpu_buffer_rsrc_t r, unsigned off, uint16_t* lds_base) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, off, 0, 0, 2);
}
__device__ __forceinline__ uint4 wd_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

template <int EPI, bool NORM, int NST, int ROWS, int MB>
__global__ __launch_bounds__(WD_NW * 64) void gemv_mfma_wide_kernel(GemvDev d) {
    static_assert(ROWS == 16 || ROWS == 32, "one or two 16-row operand tiles");
    static_assert(MB == 1 || MB == 2, "one or two token blocks per weight fetch");
    constexpr int NT = WD_NW * 64;
    constexpr bool SWI = (EPI == EPI_SWIGLU);
    constexpr int NQ = ROWS / 4;                // transfers per stage, 4 rows x 256 bytes each
    constexpr int NTT = ROWS / 16;              // 16-row operand tiles
    constexpr int MT = MB * SK_MT;              // tokens of the workgroup
    constexpr int WD_STAGE = ROWS * WD_SUB;     // elements of a wave's stage
    constexpr int VM = 4 * MB + (NORM ? 4 : 0) + NQ;   // vector-memory operations per stage
    // A ring of NBUF stage tiles per wave, NBUF - 1 stages requested ahead;
    // each tile of the ring is its own array, so the compiler can tell one
    // stage's transfers from another stage's reads. Two token blocks hold
    // twice the activation registers per stage in flight, so 16-row tiles
    // then keep three stages, not four.
    constexpr int NBUF = ROWS == 32 ? 2 : (MB == 1 ? WD16_NBUF : 3);
    static_assert(NBUF >= 2 && NBUF <= 4 && VM * (NBUF - 1) <= 63, "the ring and the wait counter");
    // a wave's first tile holds its MT x ROWS float32 sums at the end
    static_assert(MT * ROWS * 4 <= WD_STAGE * 2, "the parked sums fit a stage tile");
    __shared__ __align__(16) uint16_t w0[WD_NW][WD_STAGE];
    __shared__ __align__(16) uint16_t w1[WD_NW][WD_STAGE];
    __shared__ __align__(16) uint16_t w2[WD_NW][NBUF > 2 ? WD_STAGE : 8];
    __shared__ __align__(16) uint16_t w3[WD_NW][NBUF > 3 ? WD_STAGE : 8];
    __shared__ float res[MT * ROWS];
    __shared__ float ssl[WD_NW][MT];

    const GemvArgs& a = d.a;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases stay scalar
    const int tile = blockIdx.x, mb = d.mb0 + blockIdx.z * MB;  // first token block of the workgroup
    const int K = a.K, N = a.N;
    const int kw = (blockIdx.y * WD_NW + wave) * (NST * WD_SUB);   // first K element of this wave's range
    const int m0 = mb * SK_MT;
    const int mvalid = min(MT, a.m - m0);
    const int col = lane & 15, kg = lane >> 4;

    // Weight views: for SwiGLU the gate rows and the up rows of outputs
    // opt tile .. + opt - 1 (opt <= ROWS / 2), else rows opt tile .. +
    // opt - 1 (opt <= ROWS); the rest of the tile is padding, fetched out
    // of range.
    constexpr int HALF = ROWS / 2;
    const int opt = d.opt;
    const int n0 = tile * opt;
    const int nrows = min(N - n0, opt);
    const int64_t rowb = (int64_t)K * 2;
    const __amdgpu_buffer_rsrc_t wv0 =
        wd_view(reinterpret_cast<const uint16_t*>(a.w) + (size_t)n0 * K, nrows * rowb);
    const __amdgpu_buffer_rsrc_t wv1 =
        SWI ? wd_view(reinterpret_cast<const uint16_t*>(a.w_up) + (size_t)n0 * K, nrows * rowb) : wv0;
    // Transfer q moves rows 4q .. 4q + 3 of the tile: lane l fetches chunk
    // (l & 15) ^ (row & 15) of row 4q + l / 16 into position l & 15 of it.
    const int dr = lane >> 4;
    int wrowb[NQ], wck[4];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int r = 4 * q + dr;
        wrowb[q] = (SWI ? r % HALF : r) * K * 2;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) wck[q] = ((lane & 15) ^ ((4 * q + dr) & 15)) * 8;
    // Activation and gamma views: token col's row of each token block, chunk
    // kg of each 32. Rows past m lie past the view and arrive as zeros.
    const __amdgpu_buffer_rsrc_t xv = wd_view(reinterpret_cast<const uint16_t*>(a.x) + (size_t)m0 * K, mvalid * rowb);
    const __amdgpu_buffer_rsrc_t gv = wd_view(a.gamma, NORM ? rowb : 0);
    const unsigned xrow = col * K * 2;

    struct Act { uint4 x[MB][4]; uint4 g[4]; };
    auto issue = [&](Act& ac, uint16_t* dst, int st) {
        const int k0 = kw + st * WD_SUB;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int k = k0 + s * 32 + kg * 8;
#pragma unroll
            for (int b = 0; b < MB; ++b)
                ac.x[b][s] = wd_load16(xv, k < K ? xrow + (unsigned)(b * SK_MT * K * 2) + k * 2 : WD_OOB);
            if (NORM) ac.g[s] = wd_load16(gv, k < K ? k * 2 : WD_OOB);
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int k = k0 + wck[q & 3];
            wd_dma16(q < NQ / 2 ? wv0 : wv1, k < K ? wrowb[q] + k * 2 : WD_OOB, dst + q * 512);
        }
    };

    float ss[MB];
    f32x4_t acc[MB][NTT];
#pragma unroll
    for (int b = 0; b < MB; ++b) {
        ss[b] = 0.f;
#pragma unroll
        for (int t = 0; t < NTT; ++t) acc[b][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // One stage: the weight fragments are read from LDS once and serve every
    // token block.
    auto run = [&](Act& cur, const uint16_t* tl) {
        uint4 wf[NTT][4];
#pragma unroll
        for (int t = 0; t < NTT; ++t)
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int r = t * 16 + col;
                wf[t][s] = *reinterpret_cast<const uint4*>(&tl[r * WD_SUB + (((s * 4 + kg) ^ (r & 15)) * 8)]);
            }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int b = 0; b < MB; ++b) {
                uint4 xa = cur.x[b][s];
                if (NORM) {
                    if constexpr (MB == 1) {
                        ss[b] += vsumsq(xa, (uint16_t*)nullptr);
                    } else {            // squares by v_dot2 on the packed pairs: no unpacked copy kept
                        float q = dot2_bf16(xa.x, xa.x, 0.f);
                        q = dot2_bf16(xa.y, xa.y, q);
                        q = dot2_bf16(xa.z, xa.z, q);
                        ss[b] += dot2_bf16(xa.w, xa.w, q);
                        // the sum is consumed only after the last stage: left free, the
                        // compiler sinks the chain there and keeps every stage's
                        // activations live; an empty asm reading it pins it to this stage
                        asm volatile("" : "+v"(ss[b]));
                    }
                    xa = vscale(xa, cur.g[s], (uint16_t*)nullptr);
                }
#pragma unroll
                for (int t = 0; t < NTT; ++t) acc[b][t] = mfma16(xa, wf[t][s], acc[b][t]);
                // with two token blocks, one 32-element slice at a time: scheduled
                // as one region the unpacked activations and gamma of all four
                // slices stay live together and spill
                if constexpr (MB > 1) __builtin_amdgcn_sched_barrier(0);
            }
    };
    // stage i's tile (i is a constant once the loops are unrolled)
    auto tile_of = [&](int i) -> uint16_t* {
        switch (i % NBUF) {
            case 0: return w0[wave];
            case 1: return w1[wave];
            case 2: return w2[wave];
            default: return w3[wave];
        }
    };
    Act ac[NBUF];
#pragma unroll
    for (int i = 0; i < NBUF - 1; ++i)
        if (i < NST) issue(ac[i], tile_of(i), i);
#pragma unroll
    for (int st = 0; st < NST; ++st) {
        // Stage st + NBUF - 1 reuses the tile and registers of stage st - 1,
        // whose reads are complete.
        if (st + NBUF - 1 < NST) issue(ac[(st + NBUF - 1) % NBUF], tile_of(st + NBUF - 1), st + NBUF - 1);
        // this stage's loads and transfers are done when only the later
        // stages' are outstanding
        const int later = min(NBUF - 1, NST - 1 - st);
        if (later == 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * VM));
        else if (later == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * VM));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(VM));
        else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_sched_barrier(0);
        run(ac[st % NBUF], tile_of(st));
        __builtin_amdgcn_sched_barrier(0);
    }

    // Sums of the K ranges, added in wave order (deterministic): every wave
    // parks its MT tokens x ROWS rows in its first tile (its own reads of it
    // and transfers into it are complete).
    float* park = reinterpret_cast<float*>(w0[wave]);
#pragma unroll
    for (int b = 0; b < MB; ++b)
#pragma unroll
        for (int t = 0; t < NTT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) park[(b * SK_MT + 4 * kg + j) * ROWS + t * 16 + col] = acc[b][t][j];
    if (NORM) {
        // lanes col, col + 16, col + 32, col + 48 hold token col's squares
#pragma unroll
        for (int b = 0; b < MB; ++b) {
            float v = ss[b];
            v += __shfl_xor(v, 16, 64);
            v += __shfl_xor(v, 32, 64);
            if (lane < 16) ssl[wave][b * SK_MT + lane] = v;
        }
    }
    __syncthreads();
    for (int e = tid; e < MT * ROWS; e += NT) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < WD_NW; ++w) v += reinterpret_cast<const float*>(w0[w])[e];
        res[e] = v;
    }
    if (NORM && tid < MT) {
        float v = 0.f;
#pragma unroll
        for (int w = 0; w < WD_NW; ++w) v += ssl[w][tid];
        ssl[0][tid] = v;
    }
    __syncthreads();
    if constexpr (MB == 1) {                    // the plan splits K over workgroups only for one token block
        if (d.splits > 1) {
            __shared__ int s_last;
            if (!split_merge<ROWS, NORM, NT>(d, res, ssl[0], blockIdx.z * d.n_tiles + tile, blockIdx.y, mvalid,
                                             &s_last))
                return;
        }
    }
    gemv_epilogue<uint16_t, MT, ROWS, EPI, NORM, NT>(a, res, ssl[0], tile, m0, mvalid, opt);
}

// Split-K merge: one workgroup per output tile adds the tile's slices in
// split order (a thread requests the slices of its outputs together) and runs
// the epilogue.
template <int EPI, bool NORM, int RPT>
__global__ __launch_bounds__(256) void gemv_mfma_merge_kernel(GemvDev d) {
    // The plan splits K about four ways, so one batch of loads usually
    // covers every slice; the squared-sum slices of a fused RMSNorm travel in
    // the same batch. RPT: rows of a slice (64, the narrow kernel's tile).
    constexpr int NT = 256, PER = SK_MT * RPT / NT, UNR = 4;
    __shared__ float res[SK_MT * RPT];
    __shared__ float ssl[SK_MT];
    const int tid = threadIdx.x, tile = blockIdx.x, mb = d.mb0 + blockIdx.z;
    const int m0 = mb * SK_MT;
    const int mvalid = min(SK_MT, d.a.m - m0);
    const int S = d.splits;
    const int tile_id = blockIdx.z * d.n_tiles + tile;
    const float* base = d.part + (size_t)tile_id * S * (SK_MT * RPT);
    const float* sqb = NORM ? d.ssq + (size_t)tile_id * S * SK_MT + min(tid, mvalid - 1) : nullptr;
    const int live = mvalid * RPT;
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
                v[p][u] = base[(size_t)min(sp0 + u, S - 1) * (SK_MT * RPT) + min(tid + p * NT, live - 1)];
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
    gemv_epilogue<uint16_t, SK_MT, RPT, EPI, NORM, NT>(d.a, res, ssl, tile, m0, mvalid, d.opt);
}

constexpr int64_t WIDE_MIN_ROWS = 16;          // rows of the shortest wide tile

static GemvPlan plan_mfma(int m, int K, int N, int epi) {
    GemvPlan p{};
    p.mfma = 1;
    p.mt = SK_MT;
    p.mblocks = (m + SK_MT - 1) / SK_MT;
    p.mbw = 1;
    p.mb_per_launch = p.mblocks;                // capped below where split workgroups count arrivals
    p.lds_bytes = 0;                            // static LDS only
    const bool swi = epi == EPI_SWIGLU;
    const int64_t mb = p.mblocks;
    // Wide projections: one workgroup of 8 waves per tile of rows, its K
    // range split over the waves, whose sums meet in LDS: no second kernel
    // and no float32 slices in memory. A tile holds as many outputs as make
    // about 256 workgroups (one per compute unit, none idle; the rest of the
    // tile is padding that is never fetched): up to 32 rows, or the gate and
    // up rows of 16 outputs, in two 16-row operand tiles, and up to 16 rows
    // (8 outputs) in one, down to WIDE_MIN_ROWS. SwiGLU over 512 tiles of
    // 16 outputs or more (the stacked experts) takes 4-wave workgroups of two
    // K ranges instead, three per compute unit. Otherwise 64-row tiles split
    // over workgroups. Measured on replayed 8B MLP and 70B attention
    // projection steps and the 70B layer: tiles of 10 rows (70B QKV, t=4)
    // or 5 (t=8) lose to the split, by 0.3 and 3 us per call.
    // A wide workgroup takes two blocks of 16 tokens per weight fetch (the
    // weight fragments it reads from LDS serve both), so 17 to 32 tokens
    // stream the weights once and 33 to 64 twice; the tiles are sized as for
    // the blocks of 16 tokens a launch then has in z (wb).
    const int64_t mbw = mb >= 2 ? 2 : 1;
    const int64_t wb = (mb + mbw - 1) / mbw;
    const int64_t t2 = swi ? (N + 15) / 16 : (N + 31) / 32;
    const int64_t want = std::max<int64_t>(1, 256 / wb);
    const int64_t per = (N + want - 1) / want;  // outputs per tile for ~256 workgroups
    const int64_t cap16 = swi ? 8 : 16, cap32 = swi ? 16 : 32;
    int rg = SK_NW, ks = 1, opt = swi ? 8 * SK_NW : 16 * SK_NW;
    if (K <= 4 * SK_MAX_STAGES * SK_SUB) {
        if (swi && t2 * wb >= 512 && K <= 2 * SK_MAX_STAGES * SK_SUB) {
            rg = 2, ks = 2, opt = 16;
        } else if (per > cap16) {
            rg = 2, ks = 4, opt = (int)std::min(cap32, per);
        } else if (per >= (swi ? WIDE_MIN_ROWS / 2 : WIDE_MIN_ROWS)) {
            rg = 1, ks = 8, opt = (int)per;
        }
    }
    p.rg = rg;
    p.ks = ks;
    p.nw = rg * ks;
    p.threads = p.nw * 64;
    p.rows_per_tile = 16 * rg;
    p.out_per_tile = opt;
    p.n_tiles = (N + p.out_per_tile - 1) / p.out_per_tile;
    if (ks > 1) {
        // a workgroup covers 4 kc elements of K (8 waves of kc / 2), or 2 kc
        // (two K ranges of kc)
        const int span = rg * ks == WD_NW ? 4 : ks;
        int kc = SK_SUB;
        while (kc * span < K) kc *= 2;          // at most SK_MAX_STAGES stages by the guard above
        p.kc = kc;
        p.splits = 1;
        if (rg * ks == WD_NW) p.mbw = (int)mbw; // the wide kernel
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
    // When that chunk is 1024 or shorter, a workgroup spends much of its time
    // filling and draining; 8-wave workgroups of 16 to 32 rows stream longer
    // K ranges: K split S ways (2 to 16), the fewest splits whose tiles,
    // sized to about 256 workgroups, hold at least WIDE_MIN_ROWS rows and
    // leave no split without K to cover; the last split to finish a tile
    // adds its slices (a counter per tile and m-block in the header).
    // The 70B QKV shard at t=8 (1280 rows, K 8192): 4 splits of 20-row
    // tiles, 557 -> 546 us per layer step; at t=4 (chunk 2048) two splits
    // of 20-row tiles measured 1 us per step slower, so it stays here.
    // SwiGLU keeps the 64-row tiles.
    if (!swi && kc <= 4 * SK_SUB) {
        for (int S2 = 2; S2 <= 16; S2 *= 2) {
            const int64_t want2 = std::max<int64_t>(1, 256 / (mb * S2));
            const int64_t per2 = (N + want2 - 1) / want2;
            if (per2 > 32) break;               // more splits only lengthen the tiles
            int kc2 = SK_SUB;
            while (kc2 * 4 * S2 < K) kc2 *= 2;  // a workgroup covers 4 kc2 elements of K
            if (kc2 > SK_MAX_STAGES * SK_SUB) continue;      // K too long for S2 splits
            if (per2 < WIDE_MIN_ROWS || (int64_t)(S2 - 1) * 4 * kc2 >= K) continue;   // tiles too short, or a split idle
            p.rg = 2;
            p.ks = 4;
            p.nw = WD_NW;
            p.threads = WD_NW * 64;
            p.rows_per_tile = 32;
            p.out_per_tile = (int)per2;
            p.n_tiles = (N + p.out_per_tile - 1) / p.out_per_tile;
            p.kc = kc2;
            p.splits = S2;
            // one counter per (tile, m-block) of a launch
            if ((int64_t)p.n_tiles * p.mb_per_launch > WS_MAX_COUNTERS)
                p.mb_per_launch = std::max(1, WS_MAX_COUNTERS / p.n_tiles);
            const size_t tl = (size_t)p.n_tiles * p.mb_per_launch;
            p.ws_bytes = (tl * S2 * SK_MT * 32 * 4 + 255) / 256 * 256 + (tl * S2 * SK_MT * 4 + 255) / 256 * 256;
            return p;
        }
    }
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

GemvPlan gemv_plan_mfma(int m, int K, int N, int epi) {
    GemvPlan p = plan_mfma(m, K, N, epi);
    p.tiles_per_launch = p.n_tiles;             // slices and counters are indexed by tile and m-block
    return p;
}

template <int EPI, bool NORM, int NST, int RG, int KS>
static hipError_t mfma_launch_t(const GemvDev& d, const GemvPlan& p, hipStream_t s) {
    for (int mb0 = 0; mb0 < p.mblocks; mb0 += p.mb_per_launch) {
        GemvDev dl = d;
        dl.mb0 = mb0;
        const int blocks = min(p.mb_per_launch, p.mblocks - mb0);
        dim3 grid(p.n_tiles, p.splits, (blocks + p.mbw - 1) / p.mbw);   // z: groups of mbw token blocks
        if constexpr (RG * KS == WD_NW) {       // 16 RG rows; 8 K ranges of NST stages of 128
            if (p.mbw == 2)
                hipLaunchKernelGGL((gemv_mfma_wide_kernel<EPI, NORM, NST, 16 * RG, 2>), grid, dim3(WD_NW * 64), 0, s,
                                   dl);
            else
                hipLaunchKernelGGL((gemv_mfma_wide_kernel<EPI, NORM, NST, 16 * RG, 1>), grid, dim3(WD_NW * 64), 0, s,
                                   dl);
        } else {
            hipLaunchKernelGGL((gemv_mfma_kernel<EPI, NORM, NST, RG, KS>), grid, dim3(RG * KS * 64), 0, s, dl);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if (RG * KS != WD_NW && p.splits > 1) {  // the wide kernel merges its splits itself
            hipLaunchKernelGGL((gemv_mfma_merge_kernel<EPI, NORM, SK_RPT>), dim3(p.n_tiles, 1, grid.z), dim3(256), 0, s, dl);
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
    if (p.rg == 1 && p.ks == 8) return mfma_launch_kc<EPI, NORM, 1, 8>(d, p, s);
    if constexpr (EPI == EPI_SWIGLU) {
        if (p.rg == 2 && p.ks == 2) return mfma_launch_kc<EPI, NORM, 2, 2>(d, p, s);
    }
    return hipErrorInvalidValue;
}

hipError_t gemv_mfma_launch(const GemvDev& d, const GemvPlan& p, hipStream_t s) {
    if (p.splits > 1 && p.ks != 1 && p.rg * p.ks != WD_NW) return hipErrorInvalidValue;
    // two token blocks per workgroup: the wide kernel only, K not split over workgroups
    if (p.mbw != 1 && (p.mbw != 2 || p.splits != 1 || p.rg * p.ks != WD_NW)) return hipErrorInvalidValue;
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
