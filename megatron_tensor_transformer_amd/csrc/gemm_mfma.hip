// Prefill projections on gfx950 bf16 MFMA: y = epilogue(x @ W^T), x [M, K],
// W [N, K] (both K-contiguous), float32 accumulation.
//
// Macro-tile 256 x 256 x 64 per workgroup of 4 waves; waves form a 2 x 2 grid
// and each owns a 128 x 128 block as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16
// (256 float32 accumulators per lane). Operand tiles are staged in LDS, double
// buffered, with rows padded to 72 elements so the 16-byte fragment reads of
// 32 consecutive rows land in distinct banks. The next K-tile is fetched into
// registers while the current one is multiplied; one barrier per K-step.
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
constexpr int GM_LDK = GM_BK + 8;          // padded row stride (elements)
constexpr int GM_NT = 256;
constexpr int GM_CHUNKS = GM_BM * GM_BK / 8 / GM_NT;   // 16-byte chunks per thread per operand tile (8)
constexpr int GM_GROUP_M = 8;              // tile rows walked together for L2 reuse

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

template <int EPI>
__global__ __launch_bounds__(GM_NT, 1) void gemm_bf16_kernel(GemmDev d) {
    constexpr bool SWI = (EPI == EPI_SWIGLU);
    constexpr int BN_OUT = SWI ? GM_BN / 2 : GM_BN;
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* As = reinterpret_cast<uint16_t*>(smem);                  // [2][BM][LDK]
    uint16_t* Bs = As + 2 * GM_BM * GM_LDK;                            // [2][BN][LDK]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

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

    // Global source of each thread's chunks: chunk c = tid + 256 i covers
    // row c / 8 and k offset (c % 8) * 8 of the tile. Rows past M or N are
    // clamped to the last row: they only feed accumulator rows or columns that
    // are never stored, so they need no masking.
    const uint16_t* a_src[GM_CHUNKS];
    const uint16_t* b_src[GM_CHUNKS];
#pragma unroll
    for (int i = 0; i < GM_CHUNKS; ++i) {
        const int c = tid + GM_NT * i;
        const int row = c >> 3, kc = (c & 7) * 8;
        a_src[i] = d.x + (size_t)min(m0 + row, M - 1) * K + kc;
        int bn;
        const uint16_t* base;
        if (SWI) {
            bn = n0 + (row & 127);
            base = row < 128 ? d.w : d.w_up;
        } else {
            bn = n0 + row;
            base = d.w;
        }
        b_src[i] = base + (size_t)min(bn, N - 1) * K + kc;
    }

    uint4 ra[GM_CHUNKS], rb[GM_CHUNKS];
    // A whole K tile: straight-line, unmasked loads.
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < GM_CHUNKS; ++i) {
            ra[i] = load_u4(a_src[i] + k0);
            rb[i] = load_u4(b_src[i] + k0);
        }
    };
    // The ragged last K tile: offsets past K are clamped and zeroed.
    auto fetch_tail = [&](int k0) {
#pragma unroll
        for (int i = 0; i < GM_CHUNKS; ++i) {
            const int kc = ((tid + GM_NT * i) & 7) * 8;
            const bool kin = k0 + kc < K;
            const int off = kin ? k0 : K - 8 - kc;
            const uint4 va = load_u4(a_src[i] + off);
            const uint4 vb = load_u4(b_src[i] + off);
            ra[i] = kin ? va : make_uint4(0, 0, 0, 0);
            rb[i] = kin ? vb : make_uint4(0, 0, 0, 0);
        }
    };
    auto stash = [&](int buf) {
        uint16_t* a = As + buf * GM_BM * GM_LDK;
        uint16_t* b = Bs + buf * GM_BN * GM_LDK;
#pragma unroll
        for (int i = 0; i < GM_CHUNKS; ++i) {
            const int c = tid + GM_NT * i;
            const int off = (c >> 3) * GM_LDK + (c & 7) * 8;
            *reinterpret_cast<uint4*>(a + off) = ra[i];
            *reinterpret_cast<uint4*>(b + off) = rb[i];
        }
    };

    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // LDS rows this lane reads for its A and B fragments.
    const int lrow = lane & 31;
    const int lk = (lane >> 5) * 8;
    int a_row[4], b_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a_row[i] = wm * 128 + i * 32 + lrow;
        b_row[i] = SWI ? ((i < 2 ? 0 : 128) + wn * 64 + (i & 1) * 32 + lrow) : (wn * 128 + i * 32 + lrow);
    }

    const int KT = (K + GM_BK - 1) / GM_BK;
    const int KT_full = K / GM_BK;           // tiles with every k inside K

    auto compute = [&](int buf) {
        const uint16_t* a = As + buf * GM_BM * GM_LDK;
        const uint16_t* b = Bs + buf * GM_BN * GM_LDK;
#pragma unroll
        for (int kk = 0; kk < GM_BK / 16; ++kk) {
            uint4 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fa[i] = *reinterpret_cast<const uint4*>(a + a_row[i] * GM_LDK + kk * 16 + lk);
                fb[i] = *reinterpret_cast<const uint4*>(b + b_row[i] * GM_LDK + kk * 16 + lk);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fa[i], fb[j], acc[i][j]);
        }
    };

    if (KT_full > 0) fetch(0);
    else fetch_tail(0);
    stash(0);
    __syncthreads();
    for (int kt = 0; kt + 1 < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT_full) fetch((kt + 1) * GM_BK);
        else fetch_tail((kt + 1) * GM_BK);
        compute(buf);
        stash(buf ^ 1);
        __syncthreads();
    }
    compute((KT - 1) & 1);

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
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int col = n0 + wn * 64 + j * 32 + col_l;
                    if (col < N) {
                        const float g = acc[i][j][r], u = acc[i][j + 2][r];
                        reinterpret_cast<uint16_t*>(d.y)[(size_t)row * N + col] =
                            (uint16_t)f32_to_bf16_bits(silu_f32(g) * u);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = n0 + wn * 128 + j * 32 + col_l;
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

constexpr size_t GM_LDS = 2 * (size_t)(GM_BM + GM_BN) * GM_LDK * 2;   // 147,456 bytes

bool gemm_supported(int M, int N, int K, int epi) {
    return M > 0 && N > 0 && K > 0 && (K % 8) == 0 && epi != EPI_QKV;
}

template <int EPI>
static hipError_t gemm_launch_t(const GemmDev& d, hipStream_t s) {
    static bool lds_raised = false;
    if (!lds_raised) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_bf16_kernel<EPI>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)GM_LDS);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return e;
        }
        lds_raised = true;
    }
    hipLaunchKernelGGL(gemm_bf16_kernel<EPI>, dim3(d.tiles_m * d.tiles_n), dim3(GM_NT), GM_LDS, s, d);
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
