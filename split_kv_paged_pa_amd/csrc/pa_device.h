// pa_device.h -- device helpers shared by the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlockTokens = 16;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp_e(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Store written through to the device's point of coherence (a device-scope
// relaxed atomic store: global_store ... sc1).  Used for the partials, which the
// next kernel reads: leaving no dirty lines in the L2s shortens the end of the
// kernel (measured: 0.4-0.5 us per Phase-1 launch).
__device__ __forceinline__ void store_through(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// max over lanes l, l^16, l^32, l^48 (the four rows of a column), on the
// gfx950 permlane swaps: permlane32_swap(v, v) returns {v[l % 32], v[l % 32 + 32]}
// and permlane16_swap(v, v) returns the two rows of each row pair.
__device__ __forceinline__ float column_max(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float column_sum(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_max(float v) {
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// float -> bf16 with v_cvt_pk_bf16_f32 (round to nearest even, two per instruction).
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ s16x4 pack_bf16(float a, float b, float c, float d) {
    return __builtin_bit_cast(s16x4, u32x2{pack2_bf16(a, b), pack2_bf16(c, d)});
}

__device__ __forceinline__ s16x4 pack_bf16(f32x4 v) { return pack_bf16(v[0], v[1], v[2], v[3]); }

// Non-temporal loads (the "nt" bit): for data read exactly once, which gains
// nothing from being kept in the L2 or the last-level cache.
__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
    typedef uint32_t v4 __attribute__((ext_vector_type(4)));
    const v4 x = __builtin_nontemporal_load(reinterpret_cast<const v4 *>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ u32x2 load_nt(const u32x2 *p) { return __builtin_nontemporal_load(p); }

// Buffer descriptor word 3 of a raw (untyped) buffer on CDNA3/4, and the
// cache-policy bit of a device-scope write-through store (sc1).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kCachePolicySc1 = 16;

// Four consecutive output values base[4 i .. 4 i + 3] written through to the
// device's point of coherence with one store (8 bytes of bf16 or 16 of float):
// an output leaves no dirty L2 line behind for the end-of-kernel release to
// write back.  base must be wave-uniform and 16-byte aligned; n = elements from
// base the descriptor covers.
__device__ __forceinline__ void store_out4(uint16_t *base, int n, int i, float a, float b, float c,
                                           float d) {
    const u32x2 v = {pack2_bf16(a, b), pack2_bf16(c, d)};
    __builtin_amdgcn_raw_buffer_store_b64(v, __builtin_amdgcn_make_buffer_rsrc(base, 0, 2 * n, kBufferWord3),
                                          8 * i, 0, kCachePolicySc1);
}
__device__ __forceinline__ void store_out4(float *base, int n, int i, float a, float b, float c,
                                           float d) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v v = {__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(d)};
    __builtin_amdgcn_raw_buffer_store_b128(v, __builtin_amdgcn_make_buffer_rsrc(base, 0, 4 * n, kBufferWord3),
                                           16 * i, 0, kCachePolicySc1);
}

__device__ __forceinline__ s16x4 lo_half(uint4 v) { return __builtin_bit_cast(s16x4, u32x2{v.x, v.y}); }
__device__ __forceinline__ s16x4 hi_half(uint4 v) { return __builtin_bit_cast(s16x4, u32x2{v.z, v.w}); }

}  // namespace pa
