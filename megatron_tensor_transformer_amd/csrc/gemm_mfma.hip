// Prefill projections on gfx950 bf16 MFMA: y = epilogue(x @ W^T), x [M, K],
// W [N, K] (both K-contiguous), float32 accumulation.
//
// Macro-tile 256 x 256 x 64 per workgroup of 8 waves (two per SIMD, so one
// wave's LDS reads and waits overlap the other's matrix work). Waves form a
// 2 x 4 grid; each owns a 128 x 64 block as 4 x 2 tiles of
// v_mfma_f32_32x32x16_bf16 (128 float32 accumulators per lane).
//
// Operand tiles go from global memory straight to LDS (global_load_lds: each
// lane's 16 bytes land at the instruction's LDS base + lane * 16, so no
// registers or LDS-write instructions are spent on staging), double
// buffered: the next K tile streams into one buffer while the other is
// multiplied, with one barrier per K tile. Rows are 128 bytes; the 16-byte
// chunk c of row r is stored at slot c ^ ((r / 2) % 8), so the fragment
// reads of 16 consecutive rows hit 16 distinct bank groups without padding.
// A lane picks which global chunk it fetches so that the swizzled slot it
// lands in is the one the reads expect. Within a K tile the fragments of the
// next 16-element step are read before the current step's MFMAs are issued.
//
// Epilogues: bf16 store; float32 store (row-parallel partial); SwiGLU, where
// the B tile holds 128 gate rows and the same 128 up rows and every wave owns
// matching gate and up accumulators, so silu(gate) * up is formed in registers
// and only the activation is written.
//
// Grouped launches (mixture of experts): the same tiles over each expert's own
// tokens, whose counts are read on the device; a workgroup finds its expert
// and tile row from them, and workgroups past the last expert's tiles return
// before any transfer. Gate/up gathers the expert's token rows
// through its list and packs the activations expert after expert; down reads
// those packed rows and writes each row, times the token's gate, to the
// token's slot (its rank among its experts) of a [top_k, M, N] buffer.
//
// MFMA operand layout (32x32x16): lane l supplies row (l % 32) of A and column
// (l % 32) of B, 8 consecutive k each, the two lane halves covering k 0-7 and
// 8-15. Accumulator register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4,
// column l % 32.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace tpk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int GM_BM = 256, GM_BN = 256, GM_BK = 64;
constexpr int GM_NT = 512;                                  // 8 waves
constexpr int GM_TILE_BYTES = GM_BM * GM_BK * 2;            // one operand tile (32 KiB)
constexpr int GM_STAGE = 2 * GM_TILE_BYTES;                 // A and B tiles of one K step
constexpr int GM_DMA = GM_BM * GM_BK / 8 / GM_NT;           // 16-byte chunks per thread per operand (4)
constexpr int GM_GROUP_M = 8;                               // tile rows walked together for L2 reuse

struct GemmDev {
    const uint16_t* x;
    const uint16_t* w;
    const uint16_t* w_up;
    void* y;
    int M, N, K;
    int tiles_m, tiles_n;
    int ldb;              // B row stride (elements): K unless grouped
    GemmGroups grp;       // grouped launches only
    // Tail split (ungrouped): workgroups past full_tiles take one of split
    // K ranges of kts K tiles of a tail tile and store their float32 sums to
    // part; gemm_tail_kernel adds them and runs the epilogue.
    int full_tiles, split, kts;
    float* part;          // [tail tiles][split][GM_BM][GM_BN]
};

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// Byte offset of chunk c of row r in an operand tile.
__device__ __forceinline__ int tile_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

__device__ __forceinline__ void dma16(const uint16_t* src, unsigned char* lds_base) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                     (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

// Tile (tm, tn) of workgroup w of an ungrouped launch: workgroups are
// dispatched to the 8 XCDs round robin; renumber them so each XCD gets a
// contiguous run of tiles. Then groups of GM_GROUP_M tile rows sweep the tile
// columns together, so the A rows of a group and the B columns in flight stay
// in that XCD's L2.
__device__ __forceinline__ void gemm_tile_of(const GemmDev& d, int w, int& tm, int& tn) {
    const int nblocks = d.tiles_m * d.tiles_n;
    const int per_xcd = nblocks / 8;
    int pid = w;
    if (pid < per_xcd * 8) pid = (pid % 8) * per_xcd + pid / 8;
    const int per_group = GM_GROUP_M * d.tiles_n;
    const int group = pid / per_group;
    const int first_m = group * GM_GROUP_M;
    const int gsize = min(d.tiles_m - first_m, GM_GROUP_M);
    tm = first_m + (pid % per_group) % gsize;
    tn = (pid % per_group) / gsize;
}

template <int EPI, bool GRP>
__global__ __launch_bounds__(GM_NT, 1) void gemm_bf16_kernel(GemmDev d) {
    constexpr bool SWI = (EPI == EPI_SWIGLU);
    constexpr int BN_OUT = SWI ? GM_BN / 2 : GM_BN;
    // Two stages, A tile then B tile each. Separate objects let the compiler see
    // that the transfers into one stage never alias the reads of the other, so
    // it does not wait for them before reading.
    __shared__ __align__(16) unsigned char stage0[GM_STAGE];
    __shared__ __align__(16) unsigned char stage1[GM_STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 2, wn = wave & 3;

    // Ungrouped: the tile order of gemm_tile_of; a tail tile's K is split over
    // d.split workgroups. A grouped launch learns each group's row count on the device. Its grid
    // covers the most tile rows the groups can need (sum of counts / 256 + G)
    // times the tile columns; workgroup (rt, tn) takes tile row rt of the
    // groups' rows laid end to end, tile column tn. Numbered row by row, the
    // live tiles are spread over all XCDs by the round-robin dispatch.
    int tm = 0, tn;
    int g = 0, M = d.M, grow0 = 0;
    int kt0 = 0, kt1 = (d.K + GM_BK - 1) / GM_BK;   // K tiles of this workgroup
    int tail = -1, tail_part = 0;                  // tail tile index and K range, or -1
    if (GRP) {
        int rt = (int)blockIdx.x / d.tiles_n;
        tn = (int)blockIdx.x % d.tiles_n;
        g = -1;
        for (int e = 0; e < d.grp.G; ++e) {
            const int c = d.grp.counts[e];
            const int nt = (c + GM_BM - 1) / GM_BM;
            if (g < 0) {
                if (rt < nt) {
                    g = e;
                    tm = rt;
                    M = c;
                } else {
                    rt -= nt;
                    grow0 += c;
                }
            }
        }
        if (g < 0) return;      // past the last group's tiles
    } else {
        int w = blockIdx.x;
        if (w >= d.full_tiles) {
            const int q = w - d.full_tiles;
            tail = q / d.split;
            tail_part = q - tail * d.split;
            w = d.full_tiles + tail;
            kt0 = tail_part * d.kts;
            kt1 = min(kt1, kt0 + d.kts);
        }
        gemm_tile_of(d, w, tm, tn);
    }
    const int m0 = tm * GM_BM;
    const int n0 = tn * BN_OUT;
    const int N = d.N, K = d.K;
    const int KT = (K + GM_BK - 1) / GM_BK;        // K tiles of the whole contraction
    const int KL = kt1 - kt0;                      // K tiles of this workgroup
    const uint16_t* wb = d.w + (GRP ? (size_t)g * d.grp.b_group_stride : 0);
    const uint16_t* wub = SWI ? d.w_up + (GRP ? (size_t)g * d.grp.b_group_stride : 0) : nullptr;

    // Chunks this thread moves per K tile: transfer j of wave w fills slots
    // p = (j * 8 + w) * 64 + lane of each tile, i.e. row p / 8, slot p % 8,
    // which holds logical chunk (p % 8) ^ ((row / 2) % 8). Rows past M or N
    // are clamped to the last row: they only feed accumulator rows or columns
    // that are never stored.
    const uint16_t* a_src[GM_DMA];
    const uint16_t* b_src[GM_DMA];
    int kc[GM_DMA];
#pragma unroll
    for (int j = 0; j < GM_DMA; ++j) {
        const int p = (j * 8 + wave) * 64 + lane;
        const int row = p >> 3;
        kc[j] = ((p & 7) ^ ((row >> 1) & 7)) * 8;
        const int r = min(m0 + row, M - 1);
        int arow = r;
        if (GRP) arow = SWI ? d.grp.lists[(size_t)g * d.M + r] : grow0 + r;   // gathered tokens / packed rows
        a_src[j] = d.x + (size_t)arow * K + kc[j];
        int bn;
        const uint16_t* base;
        if (SWI) {
            bn = n0 + (row & 127);
            base = row < 128 ? wb : wub;
        } else {
            bn = n0 + row;
            base = wb;
        }
        b_src[j] = base + (size_t)min(bn, N - 1) * d.ldb + kc[j];
    }
    // Chunks past K (ragged last tile) are fetched from a clamped in-bounds
    // offset and zeroed in LDS once they have landed.
    auto load_stage = [&](int k0, unsigned char* sa) {
        unsigned char* sb = sa + GM_TILE_BYTES;
#pragma unroll
        for (int j = 0; j < GM_DMA; ++j) {
            const int off = (k0 + kc[j] < K) ? k0 : K - 8 - kc[j];
            dma16(a_src[j] + off, sa + (j * 8 + wave) * 1024);
            dma16(b_src[j] + off, sb + (j * 8 + wave) * 1024);
        }
    };
    auto zero_tail = [&](int k0, unsigned char* sa) {
        unsigned char* sb = sa + GM_TILE_BYTES;
#pragma unroll
        for (int j = 0; j < GM_DMA; ++j) {
            if (k0 + kc[j] >= K) {
                const int off = (j * 8 + wave) * 1024 + lane * 16;
                *reinterpret_cast<uint4*>(sa + off) = make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4*>(sb + off) = make_uint4(0, 0, 0, 0);
            }
        }
    };
    const bool ragged = (K % GM_BK) != 0;

    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Tile rows of this lane's A and B fragments.
    const int lrow = lane & 31;
    int a_row[4], b_row[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a_row[i] = wm * 128 + i * 32 + lrow;
#pragma unroll
    for (int j = 0; j < 2; ++j) b_row[j] = SWI ? (j * 128 + wn * 32 + lrow) : (wn * 64 + j * 32 + lrow);

    auto compute = [&](const unsigned char* sa) {
        const unsigned char* sb = sa + GM_TILE_BYTES;
        uint4 fa[2][4], fb[2][2];
        auto read = [&](int kk, uint4 (&a)[4], uint4 (&b)[2]) {
            const int c = kk * 2 + (lane >> 5);
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const uint4*>(sa + tile_off(a_row[i], c));
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = *reinterpret_cast<const uint4*>(sb + tile_off(b_row[j], c));
        };
        read(0, fa[0], fb[0]);
#pragma unroll
        for (int kk = 0; kk < GM_BK / 16; ++kk) {
            if (kk + 1 < GM_BK / 16) read(kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fa[kk & 1][i], fb[kk & 1][j], acc[i][j]);
        }
    };

    // K tile kt lives in stage kt % 2; the loop body covers two tiles so each
    // access names its stage statically.
    // kt counts this workgroup's K tiles from kt0; only the contraction's last
    // K tile can be ragged.
    auto step = [&](int kt, unsigned char* cur, unsigned char* nxt) {
        const bool more = kt + 1 < KL;
        if (more) load_stage((kt0 + kt + 1) * GM_BK, nxt);
        compute(cur);
        if (more) {
            __builtin_amdgcn_s_waitcnt(0);     // the next tile has landed in LDS
            if (ragged && kt0 + kt + 2 == KT) zero_tail((kt0 + kt + 1) * GM_BK, nxt);
        }
        __syncthreads();
    };
    load_stage(kt0 * GM_BK, stage0);
    __builtin_amdgcn_s_waitcnt(0);
    if (ragged && kt0 + 1 == KT) zero_tail(kt0 * GM_BK, stage0);
    __syncthreads();
    for (int kt = 0; kt < KL; kt += 2) {
        step(kt, stage0, stage1);
        if (kt + 1 < KL) step(kt + 1, stage1, stage0);
    }

    if (!GRP && tail >= 0) {
        // A part of a tail tile: its float32 sums, [row][B row of the tile].
        float* pt = d.part + ((size_t)tail * d.split + tail_part) * GM_BM * GM_BN;
        const int row_l = 4 * (lane >> 5);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = wm * 128 + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
#pragma unroll
                for (int j = 0; j < 2; ++j) pt[(size_t)row * GM_BN + b_row[j]] = acc[i][j][r];   // column lane % 32
            }
        return;
    }

    // Epilogue.
    const int col_l = lane & 31;
    const int row_l = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + row_l + (r & 3);
            if (row >= M) continue;
            if (SWI) {
                const int col = n0 + wn * 32 + col_l;
                if (col < N) {
                    const float gt = acc[i][0][r], u = acc[i][1][r];
                    const size_t orow = GRP ? (size_t)grow0 + row : (size_t)row;   // grouped: packed rows
                    reinterpret_cast<uint16_t*>(d.y)[orow * N + col] = (uint16_t)f32_to_bf16_bits(silu_f32(gt) * u);
                }
            } else {
                size_t orow = (size_t)row;
                float scl = 1.0f;
                if (GRP) {
                    // token of this row, its slot among its experts, its gate
                    const int t = d.grp.lists[(size_t)g * d.M + row];
                    orow = (size_t)d.grp.slots[(size_t)t * d.grp.G + g] * d.M + t;
                    scl = d.grp.gates[(size_t)t * d.grp.G + g];
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = n0 + wn * 64 + j * 32 + col_l;
                    if (col >= N) continue;
                    const float v = acc[i][j][r];
                    if (EPI == EPI_PARTIAL)
                        reinterpret_cast<float*>(d.y)[orow * N + col] = GRP ? v * scl : v;
                    else
                        reinterpret_cast<uint16_t*>(d.y)[orow * N + col] = (uint16_t)f32_to_bf16_bits(v);
                }
            }
        }
    }
}


// The tail tiles of an ungrouped launch: the sum of their K ranges' float32
// partials in range order, then the epilogue. One workgroup per 8 rows of a
// tail tile, a thread per column.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_tail_kernel(GemmDev d) {
    constexpr bool SWI = (EPI == EPI_SWIGLU);
    constexpr int BN_OUT = SWI ? GM_BN / 2 : GM_BN;
    constexpr int ROWS = 8;
    const int t = blockIdx.x / (GM_BM / ROWS);
    const int r0 = (blockIdx.x % (GM_BM / ROWS)) * ROWS;
    int tm, tn;
    gemm_tile_of(d, d.full_tiles + t, tm, tn);
    const int c = threadIdx.x;
    if (c >= BN_OUT) return;
    const int n = tn * BN_OUT + c;
    if (n >= d.N) return;
    const float* pt = d.part + (size_t)t * d.split * GM_BM * GM_BN;
    for (int rr = 0; rr < ROWS; ++rr) {
        const int row = r0 + rr;
        const int m = tm * GM_BM + row;
        if (m >= d.M) break;
        float v = 0.f, u = 0.f;
        for (int q = 0; q < d.split; ++q) {
            const float* pr = pt + ((size_t)q * GM_BM + row) * GM_BN;
            v += pr[c];
            if (SWI) u += pr[GM_BN / 2 + c];
        }
        if (SWI)
            reinterpret_cast<uint16_t*>(d.y)[(size_t)m * d.N + n] = (uint16_t)f32_to_bf16_bits(silu_f32(v) * u);
        else if (EPI == EPI_PARTIAL)
            reinterpret_cast<float*>(d.y)[(size_t)m * d.N + n] = v;
        else
            reinterpret_cast<uint16_t*>(d.y)[(size_t)m * d.N + n] = (uint16_t)f32_to_bf16_bits(v);
    }
}

// How an ungrouped launch splits the K of its tail tiles. With fewer than 256
// tiles all of them are tail tiles; otherwise those of the last partial round
// of 256. Each tail tile's K goes to `split` workgroups (at least 4 K tiles
// each, at most one per compute unit in the last round); split 1 means none.
struct TailPlan {
    int tiles, full, tail, split, kts;
};
static TailPlan gemm_tail_plan(int M, int N, int K, int epi) {
    TailPlan t{};
    const int bn_out = epi == EPI_SWIGLU ? GM_BN / 2 : GM_BN;
    t.tiles = ((M + GM_BM - 1) / GM_BM) * ((N + bn_out - 1) / bn_out);
    const int KT = (K + GM_BK - 1) / GM_BK;
    t.tail = t.tiles % 256;
    t.full = t.tiles - t.tail;
    int sp = t.tail ? std::min(256 / t.tail, KT / 4) : 1;
    if (sp < 2) {
        t.full = t.tiles;
        t.tail = 0;
        t.split = 1;
        t.kts = KT;
        return t;
    }
    t.kts = (KT + sp - 1) / sp;
    t.split = (KT + t.kts - 1) / t.kts;           // no empty range
    return t;
}

size_t gemm_scratch_bytes(int M, int N, int K, int epi) {
    if (epi == EPI_QKV) return 0;
    const TailPlan t = gemm_tail_plan(M, N, K, epi);
    return (size_t)t.tail * t.split * GM_BM * GM_BN * 4;
}

bool gemm_supported(int M, int N, int K, int epi) {
    return M > 0 && N > 0 && K > 0 && (K % 8) == 0 && epi != EPI_QKV;
}

template <int EPI, bool GRP>
static hipError_t gemm_launch_t(const GemmDev& d, int grid, hipStream_t s) {
    hipLaunchKernelGGL((gemm_bf16_kernel<EPI, GRP>), dim3(grid), dim3(GM_NT), 0, s, d);
    return hipGetLastError();
}

hipError_t gemm_launch(const GemmArgs& a, hipStream_t s) {
    GemmDev d{};
    d.x = reinterpret_cast<const uint16_t*>(a.x);
    d.w = reinterpret_cast<const uint16_t*>(a.w);
    d.w_up = reinterpret_cast<const uint16_t*>(a.w_up);
    d.y = a.y;
    d.M = a.M; d.N = a.N; d.K = a.K;
    const int bn_out = a.epi == EPI_SWIGLU ? GM_BN / 2 : GM_BN;
    d.tiles_m = (a.M + GM_BM - 1) / GM_BM;
    d.tiles_n = (a.N + bn_out - 1) / bn_out;
    d.ldb = a.K;
    const TailPlan t = gemm_tail_plan(a.M, a.N, a.K, a.epi);
    d.full_tiles = t.full;
    d.split = t.split;
    d.kts = t.kts;
    d.part = reinterpret_cast<float*>(a.scratch);
    if (t.tail && !a.scratch) return hipErrorInvalidValue;
    const int grid = t.full + t.tail * t.split;
    hipError_t e = hipErrorInvalidValue;
    switch (a.epi) {
        case EPI_STORE: e = gemm_launch_t<EPI_STORE, false>(d, grid, s); break;
        case EPI_PARTIAL: e = gemm_launch_t<EPI_PARTIAL, false>(d, grid, s); break;
        case EPI_SWIGLU: e = gemm_launch_t<EPI_SWIGLU, false>(d, grid, s); break;
    }
    if (e != hipSuccess || !t.tail) return e;
    const dim3 fg(t.tail * (GM_BM / 8));
    switch (a.epi) {
        case EPI_STORE: hipLaunchKernelGGL(gemm_tail_kernel<EPI_STORE>, fg, dim3(256), 0, s, d); break;
        case EPI_PARTIAL: hipLaunchKernelGGL(gemm_tail_kernel<EPI_PARTIAL>, fg, dim3(256), 0, s, d); break;
        case EPI_SWIGLU: hipLaunchKernelGGL(gemm_tail_kernel<EPI_SWIGLU>, fg, dim3(256), 0, s, d); break;
    }
    return hipGetLastError();
}

hipError_t gemm_grouped_launch(const GemmArgs& a, const GemmGroups& g, hipStream_t s) {
    GemmDev d{};
    d.x = reinterpret_cast<const uint16_t*>(a.x);
    d.w = reinterpret_cast<const uint16_t*>(a.w);
    d.w_up = reinterpret_cast<const uint16_t*>(a.w_up);
    d.y = a.y;
    d.M = a.M; d.N = a.N; d.K = a.K;
    const int bn_out = a.epi == EPI_SWIGLU ? GM_BN / 2 : GM_BN;
    d.tiles_m = (g.rows_total + GM_BM - 1) / GM_BM + g.G;   // sum over groups of ceil(count / 256), at most
    d.tiles_n = (a.N + bn_out - 1) / bn_out;
    d.ldb = g.ldb;
    d.grp = g;
    const int grid = d.tiles_m * d.tiles_n;
    switch (a.epi) {
        case EPI_PARTIAL: return gemm_launch_t<EPI_PARTIAL, true>(d, grid, s);
        case EPI_SWIGLU: return gemm_launch_t<EPI_SWIGLU, true>(d, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tpk
