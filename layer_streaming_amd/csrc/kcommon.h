// Device-side helpers shared by the gfx950 kernels: bf16 storage as
// uint16_t, float <-> bf16 conversion, wave64 reductions, vector types.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// fp16 <-> float (hardware conversion, round to nearest even).
__device__ __forceinline__ float h2f(uint16_t h) { return float(__builtin_bit_cast(_Float16, h)); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, _Float16(f)); }
__device__ __forceinline__ f16x8_t as_f16x8(const uint4& v) { return __builtin_bit_cast(f16x8_t, v); }

// bf16 -> float is exact: the bf16 bits are the top half of the float.
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16, IEEE round to nearest, ties to even; NaN stays a NaN.  The
// conversion is gfx950's v_cvt_pk_bf16_f32 (one instruction per two values).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, __bf16(f)); }
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Unpack 8 bf16 held in a uint4 into floats.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
    f[0] = bflo(v.x); f[1] = bfhi(v.x); f[2] = bflo(v.y); f[3] = bfhi(v.y);
    f[4] = bflo(v.z); f[5] = bfhi(v.z); f[6] = bflo(v.w); f[7] = bfhi(v.w);
}
__device__ __forceinline__ uint4 pack8(const float* f) {
    return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
}

// Sum / max over the 64 lanes of a wave; every lane receives the result.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

// 8 fp16 in a uint4 <-> floats.
__device__ __forceinline__ void unpack8h(const uint4& v, float* f) {
    f[0] = h2f(v.x & 0xFFFF); f[1] = h2f(v.x >> 16); f[2] = h2f(v.y & 0xFFFF); f[3] = h2f(v.y >> 16);
    f[4] = h2f(v.z & 0xFFFF); f[5] = h2f(v.z >> 16); f[6] = h2f(v.w & 0xFFFF); f[7] = h2f(v.w >> 16);
}
__device__ __forceinline__ uint4 pack8h(const float* f) {
    auto p = [](float a, float b) { return uint32_t(f2h(a)) | (uint32_t(f2h(b)) << 16); };
    return make_uint4(p(f[0], f[1]), p(f[2], f[3]), p(f[4], f[5]), p(f[6], f[7]));
}

// Range guard of the fp16 operands.  A value whose magnitude rounds beyond
// the largest finite fp16 (|x| >= 65520, or not finite) is counted in n and
// saturated to +-65504 (a NaN stays a NaN); every other value converts with
// round to nearest even.  Values below fp16's normal range (2^-14) become
// subnormals with an absolute error of at most 2^-25.
__device__ __forceinline__ uint16_t f2h_sat(float f, uint32_t& n) {
    if (!(fabsf(f) < 65520.f)) {
        ++n;
        if (f == f) f = copysignf(65504.f, f);
    }
    return f2h(f);
}
__device__ __forceinline__ uint32_t pack2h_sat(float a, float b, uint32_t& n) {
    return uint32_t(f2h_sat(a, n)) | (uint32_t(f2h_sat(b, n)) << 16);
}
__device__ __forceinline__ uint4 pack8h_sat(const float* f, uint32_t& n) {
    return make_uint4(pack2h_sat(f[0], f[1], n), pack2h_sat(f[2], f[3], n), pack2h_sat(f[4], f[5], n),
                      pack2h_sat(f[6], f[7], n));
}
// Add a lane's overflow count to the caller's counter (only lanes that saw
// one: the common case issues no atomic at all).
__device__ __forceinline__ void count_ovf(uint32_t* ovf, uint32_t n) {
    if (ovf && n) atomicAdd(ovf, n);
}
