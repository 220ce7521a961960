// Device helpers shared by the gfx950 kernels: bf16 packing, 128-bit vectors,
// dot products on packed bf16 pairs, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpk {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 bits <-> float. The low half of a packed pair is the element with the
// lower address.
__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// float -> bf16 with round-to-nearest-even (one v_cvt_pk_bf16_f32 per pair on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    const __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// acc + a.lo*b.lo + a.hi*b.hi on packed bf16 pairs (v_dot2 on gfx950).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                           acc, false);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

// Sum over groups of G consecutive lanes (G a power of two <= 64); every lane
// of the group ends with the group's sum. Butterfly order is fixed, so the
// result is deterministic.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Lane exchange within rows of 16 lanes (DPP). Each control is an involution
// pairing the lower and upper half of a block: mirror (i <-> 15-i, block 16),
// half mirror (i <-> 7-i, block 8), quad xor 2 and quad xor 1.
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int ST>
__device__ __forceinline__ float dpp_stage(float v) {
    if constexpr (ST == 0) return dpp_mov<DPP_ROW_MIRROR>(v);
    else if constexpr (ST == 1) return dpp_mov<DPP_ROW_HALF_MIRROR>(v);
    else if constexpr (ST == 2) return dpp_mov<DPP_QUAD_XOR2>(v);
    else return dpp_mov<DPP_QUAD_XOR1>(v);
}

// DPP rotate by 8 within 16 lanes: lane i reads lane i ^ 8.
constexpr int DPP_ROW_ROR8 = 0x128;

template <int ST, int N>
__device__ __forceinline__ void rs_stage(float* v, int sub) {
    if constexpr (ST < 4) {
        if constexpr (N > 1) {
            constexpr int H = N / 2;
            const bool upper = (sub >> (3 - ST)) & 1;
#pragma unroll
            for (int j = 0; j < H; ++j) {
                const float keep = upper ? v[H + j] : v[j];
                const float send = upper ? v[j] : v[H + j];
                v[j] = keep + dpp_stage<ST>(send);
            }
            rs_stage<ST + 1, H>(v, sub);
        } else {
            v[0] += dpp_stage<ST>(v[0]);
            rs_stage<ST + 1, 1>(v, sub);
        }
    }
}

// Reduce V values over each group of 16 lanes and scatter the sums: stage s
// pairs the lanes of a block of 16 >> s and keeps half of the remaining values
// (the upper lane of a pair keeps the upper half). After log2(V) stages (at
// most 4) each lane holds V/16 sums in v[0 .. V/16) (or, for V < 16, one sum
// duplicated over 16/V lanes); reduce16_index names them.
template <int V>
__device__ __forceinline__ void reduce_scatter16(float* v, int sub) {
    static_assert(V >= 1 && (V & (V - 1)) == 0, "V must be a power of two");
    rs_stage<0, V>(v, sub);
}

// Cross-row exchange stages for 64-lane reductions. v_permlane32_swap on the
// pair (x, y) leaves x with its upper 32 lanes replaced by the lower 32 lanes
// of y, and y with its lower 32 lanes replaced by the upper 32 lanes of x; the
// sum of the two results is, in lanes 0-31, x plus its partner's x and, in
// lanes 32-63, y plus its partner's y. permlane16_swap does the same for the
// 16-lane halves of each 32-lane half. So one swap and one add reduce a pair
// of values across the exchange with no lane-dependent selects.
template <int ST>
__device__ __forceinline__ void xrow_pair(float& x, float& y) {
    const uint32_t xi = __float_as_uint(x), yi = __float_as_uint(y);
    uint32_t a, b;
    if constexpr (ST == 0) {
        const auto r = __builtin_amdgcn_permlane32_swap(xi, yi, false, false);
        a = r[0]; b = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(xi, yi, false, false);
        a = r[0]; b = r[1];
    }
    x = __uint_as_float(a) + __uint_as_float(b);
}

template <int ST, int N>
__device__ __forceinline__ void rs64_stage(float* v, int lane) {
    if constexpr (ST < 2) {
        if constexpr (N > 1) {
            constexpr int H = N / 2;
#pragma unroll
            for (int j = 0; j < H; ++j) xrow_pair<ST>(v[j], v[H + j]);
            rs64_stage<ST + 1, H>(v, lane);
        } else {
            float y = v[0];
            xrow_pair<ST>(v[0], y);
            rs64_stage<ST + 1, 1>(v, lane);
        }
    } else {
        rs_stage<ST - 2, N>(v, lane & 15);
    }
}

// Reduce V values over all 64 lanes and scatter the sums: the two cross-row
// stages (lane bit 5, then bit 4) use permlane swaps, the four in-row stages
// (bits 3..0) use DPP. Each lane ends with max(V/64, 1) sums in v[0..);
// reduce64_index names them.
template <int V>
__device__ __forceinline__ void reduce_scatter64(float* v, int lane) {
    static_assert(V >= 1 && (V & (V - 1)) == 0, "V must be a power of two");
    rs64_stage<0, V>(v, lane);
}

template <int V>
__device__ __forceinline__ int reduce64_index(int lane, int j, bool& owner) {
    int idx = 0, n = V;
    owner = true;
#pragma unroll
    for (int st = 0; st < 6; ++st) {
        const int bit = (lane >> (5 - st)) & 1;
        if (n > 1) {
            n /= 2;
            idx += bit * n;
        } else if (bit) {
            owner = false;
        }
    }
    return idx + j;
}

// Sum over the 64 lanes of a wave, every lane receiving it (permlane + DPP).
__device__ __forceinline__ float wave_sum(float v) {
    float t[1] = {v};
    rs64_stage<0, 1>(t, threadIdx.x & 63);
    return t[0];
}

// Reduce V values over groups of LANES (8 or 16) consecutive lanes, scattering
// the sums as reduce_scatter16 does (an 8-lane group uses its last 3 stages).
template <int LANES, int V>
__device__ __forceinline__ void reduce_scatter_group(float* v, int lane) {
    static_assert(LANES == 8 || LANES == 16, "groups of 8 or 16 lanes");
    if constexpr (LANES == 16) rs_stage<0, V>(v, lane & 15);
    else rs_stage<1, V>(v, lane & 7);
}
template <int LANES, int V>
__device__ __forceinline__ int reduce_group_index(int lane, int j, bool& owner) {
    const int sub = lane & (LANES - 1);
    int idx = 0, n = V;
    owner = true;
#pragma unroll
    for (int st = (LANES == 16 ? 0 : 1); st < 4; ++st) {
        const int bit = (sub >> (3 - st)) & 1;
        if (n > 1) {
            n /= 2;
            idx += bit * n;
        } else if (bit) {
            owner = false;
        }
    }
    return idx + j;
}

// Value index held in slot j of lane `sub` after reduce_scatter16<V>; lanes
// that hold a duplicate (V < 16) are those with owner == false.
template <int V>
__device__ __forceinline__ int reduce16_index(int sub, int j, bool& owner) {
    int idx = 0, n = V;
    owner = true;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
        const int bit = (sub >> (3 - st)) & 1;
        if (n > 1) {
            n /= 2;
            idx += bit * n;
        } else if (bit) {
            owner = false;
        }
    }
    return idx + j;
}

// Agent-scope relaxed atomics: coherent per location across the XCDs without
// the cache-wide writeback/invalidate of an agent-scope fence.
__device__ __forceinline__ void store_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup-level "last one to finish" vote over `total` workgroups sharing a
// counter. Every thread's coherent stores must be complete before the vote;
// the caller's threads all call this. Returns true in every thread of the
// last workgroup, which also resets the counter for the next use.
__device__ __forceinline__ bool last_arriver(unsigned* counter, unsigned total, int* s_flag) {
    __builtin_amdgcn_s_waitcnt(0);           // this thread's stores are acknowledged
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old == total - 1;
        if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = last;
    }
    __syncthreads();
    return *s_flag != 0;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 128-bit global load that marks the line as streamed (used once).
__device__ __forceinline__ uint4 load_stream_u4(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 load_u4(const void* p) { return *reinterpret_cast<const uint4*>(p); }

}  // namespace tpk
