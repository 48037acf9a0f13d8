// Device-side helpers shared by the gfx950 kernels: storage formats, bf16
// rounding, MFMA operand types and small wave utilities.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint16_t u16x4;
typedef __attribute__((ext_vector_type(8))) uint16_t u16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 with the hardware converter (v_cvt_pk_bf16_f32): round to
// nearest even, NaN stays NaN.
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t h = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, h);
}

// Split x into hi + lo, both bf16: hi = RNE(x), lo = RNE(x - hi).  hi + lo
// carries about 16 significant bits, enough that a pair of bf16 MFMAs
// reproduces an fp32-operand product to well below the parity tolerance.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
    hi = f32_to_bf16_bits(x);
    lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}
// Two values at once: packed hi pair and lo pair.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf16x2(a, b);
    const float ha = __uint_as_float(hi << 16);
    const float hb = __uint_as_float(hi & 0xffff0000u);
    lo = pack_bf16x2(a - ha, b - hb);
}

// Smallest decay the chunked kernels take the logarithm of: a gate of exactly
// 0 (a complete reset) becomes 2^-126, whose contribution is below fp32
// resolution of any state it multiplies, instead of log(0) = -inf turning
// differences of log decays into NaN.
constexpr float kMinDecay = 1.17549435e-38f;

// ---------------------------------------------------------------- storage types
struct F32 {
    using T = float;
    static constexpr int bytes = 4;
    __device__ __forceinline__ static float load(const T* p, long i) { return p[i]; }
    __device__ __forceinline__ static void store(T* p, long i, float x) { p[i] = x; }
};
struct BF16 {
    using T = uint16_t;
    static constexpr int bytes = 2;
    __device__ __forceinline__ static float load(const T* p, long i) { return bf16_bits_to_f32(p[i]); }
    __device__ __forceinline__ static void store(T* p, long i, float x) { p[i] = f32_to_bf16_bits(x); }
};

// 4 consecutive elements <-> float4
template <class S> struct Vec4;
template <> struct Vec4<F32> {
    __device__ __forceinline__ static f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
    __device__ __forceinline__ static void store(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
};
template <> struct Vec4<BF16> {
    __device__ __forceinline__ static f32x4 load(const uint16_t* p) {
        u32x2 w = *reinterpret_cast<const u32x2*>(p);
        f32x4 r;
        r.x = __uint_as_float(w.x << 16);
        r.y = __uint_as_float(w.x & 0xffff0000u);
        r.z = __uint_as_float(w.y << 16);
        r.w = __uint_as_float(w.y & 0xffff0000u);
        return r;
    }
    __device__ __forceinline__ static void store(uint16_t* p, f32x4 x) {
        u32x2 w;
        w.x = pack_bf16x2(x.x, x.y);
        w.y = pack_bf16x2(x.z, x.w);
        *reinterpret_cast<u32x2*>(p) = w;
    }
};

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_bf16: D(16x16) += A(16x32) B(32x16).  Lane l supplies
// row (l % 16) of A and column (l % 16) of B, each as 8 k-values; lane group
// l / 16 selects which 8 of the 32 k.  Any fixed assignment of k-values to
// (lane group, slot) works as long as A and B use the same one.  D: lane l
// holds column l % 16, rows 4 * (l / 16) + {0,1,2,3}.
__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x4_f32: same row/column/accumulator layout, one k-value
// per lane, k = l / 16.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// ---------------------------------------------------------------- misc
__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
    return x;
}

}  // namespace gla
