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
// MFMA operand layout (32x32x16): lane l supplies row (l % 32) of A and column
// (l % 32) of B, 8 consecutive k each, the two lane halves covering k 0-7 and
// 8-15. Accumulator register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4,
// column l % 32.
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

template <int EPI>
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

    // Workgroups are dispatched to the 8 XCDs round robin; renumber them so
    // each XCD gets a contiguous run of tiles. Then groups of GM_GROUP_M tile
    // rows sweep the tile columns together, so the A rows of a group and the
    // B columns in flight stay in that XCD's L2.
    const int nblocks = d.tiles_m * d.tiles_n;
    const int per_xcd = nblocks / 8;
    int pid = blockIdx.x;
    if (pid < per_xcd * 8) pid = (pid % 8) * per_xcd + pid / 8;
    const int per_group = GM_GROUP_M * d.tiles_n;
    const int group = pid / per_group;
    const int first_m = group * GM_GROUP_M;
    const int gsize = min(d.tiles_m - first_m, GM_GROUP_M);
    const int tm = first_m + (pid % per_group) % gsize;
    const int tn = (pid % per_group) / gsize;
    const int m0 = tm * GM_BM;
    const int n0 = tn * BN_OUT;
    const int M = d.M, N = d.N, K = d.K;
    const int KT = (K + GM_BK - 1) / GM_BK;

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
        a_src[j] = d.x + (size_t)min(m0 + row, M - 1) * K + kc[j];
        int bn;
        const uint16_t* base;
        if (SWI) {
            bn = n0 + (row & 127);
            base = row < 128 ? d.w : d.w_up;
        } else {
            bn = n0 + row;
            base = d.w;
        }
        b_src[j] = base + (size_t)min(bn, N - 1) * K + kc[j];
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
    auto step = [&](int kt, unsigned char* cur, unsigned char* nxt) {
        const bool more = kt + 1 < KT;
        if (more) load_stage((kt + 1) * GM_BK, nxt);
        compute(cur);
        if (more) {
            __builtin_amdgcn_s_waitcnt(0);     // the next tile has landed in LDS
            if (ragged && kt + 2 == KT) zero_tail((kt + 1) * GM_BK, nxt);
        }
        __syncthreads();
    };
    load_stage(0, stage0);
    __builtin_amdgcn_s_waitcnt(0);
    if (ragged && KT == 1) zero_tail(0, stage0);
    __syncthreads();
    for (int kt = 0; kt < KT; kt += 2) {
        step(kt, stage0, stage1);
        if (kt + 1 < KT) step(kt + 1, stage1, stage0);
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
                    const float g = acc[i][0][r], u = acc[i][1][r];
                    reinterpret_cast<uint16_t*>(d.y)[(size_t)row * N + col] = (uint16_t)f32_to_bf16_bits(silu_f32(g) * u);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = n0 + wn * 64 + j * 32 + col_l;
                    if (col >= N) continue;
                    const float v = acc[i][j][r];
                    if (EPI == EPI_PARTIAL)
                        reinterpret_cast<float*>(d.y)[(size_t)row * N + col] = v;
                    else
                        reinterpret_cast<uint16_t*>(d.y)[(size_t)row * N + col] = (uint16_t)f32_to_bf16_bits(v);
                }
            }
        }
    }
}


bool gemm_supported(int M, int N, int K, int epi) {
    return M > 0 && N > 0 && K > 0 && (K % 8) == 0 && epi != EPI_QKV;
}

template <int EPI>
static hipError_t gemm_launch_t(const GemmDev& d, hipStream_t s) {
    hipLaunchKernelGGL(gemm_bf16_kernel<EPI>, dim3(d.tiles_m * d.tiles_n), dim3(GM_NT), 0, s, d);
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
    switch (a.epi) {
        case EPI_STORE: return gemm_launch_t<EPI_STORE>(d, s);
        case EPI_PARTIAL: return gemm_launch_t<EPI_PARTIAL>(d, s);
        case EPI_SWIGLU: return gemm_launch_t<EPI_SWIGLU>(d, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace tpk
