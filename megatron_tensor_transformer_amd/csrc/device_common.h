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

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
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

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 128-bit global load that marks the line as streamed (used once).
__device__ __forceinline__ uint4 load_stream_u4(const void* p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 load_u4(const void* p) { return *reinterpret_cast<const uint4*>(p); }

}  // namespace tpk
