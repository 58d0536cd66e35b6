// kda_device.h -- device-side building blocks shared by the KDA kernels (gfx950).
//
// MFMA conventions (v_mfma_f32_16x16x32_{f16,bf16}, wave64):
//   A (16 x 32): lane l holds row (l % 16), eight K-slots of K-group (l / 16).
//   B (32 x 16): lane l holds column (l % 16), the same eight K-slots of group (l / 16).
//   C/D (16 x 16): lane l holds rows 4*(l/16) + j, j = 0..3, of column (l % 16).
// Only the pairing of K-slots between A and B matters for a product, so an
// operand may list its 32 reduction indices in any order, as long as the other
// operand lists them in the same order. The kernels use the order in which two
// stacked accumulator tiles (rows 0-15 and 16-31) already sit in registers:
//   group g, slot j  <->  index  4g + j (j < 4),  16 + 4g + (j - 4) (j >= 4).
// This lets a 32-row slice of the fp32 state S (held as accumulators) feed the
// next product as a B operand with no data movement. kperm() gives, for an
// index i in 0..31, its position 8g + j in that order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int D = 128;   // K = V = 128

__device__ __forceinline__ constexpr int kperm(int i) {
    return 8 * ((i & 15) >> 2) + 4 * (i >> 4) + (i & 3);
}

__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x4(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Round to fp16 / bf16 exactly once. The compiler may otherwise materialise
// the same conversion twice with different instructions (a packed convert for
// the stored operand, a mixed-precision FMA inside the remainder), and those
// do not round exact ties the same way; a split whose two halves saw
// different "hi" values is off by 2*lo. The empty asm makes the converted
// value opaque, so every use reads the one rounded result.
__device__ __forceinline__ _Float16 cvt16_once(float x) {
    _Float16 h = (_Float16)x;
    __asm__ volatile("" : "+v"(h));
    return h;
}
__device__ __forceinline__ __bf16 cvtbf_once(float x) {
    __bf16 h = (__bf16)x;
    __asm__ volatile("" : "+v"(h));
    return h;
}

// Two-term fp16 split: x ~= hi + lo with about 22 significant bits.
__device__ __forceinline__ void split16(float x, _Float16& hi, _Float16& lo) {
    const _Float16 h = cvt16_once(x);
    hi = h;
    lo = (_Float16)(x - (float)h);
}
struct half2s { _Float16 hi, lo; };
__device__ __forceinline__ half2s split16(float x) {
    half2s r;
    r.hi = cvt16_once(x);
    r.lo = (_Float16)(x - (float)r.hi);
    return r;
}
// Two-term bf16 split: x ~= hi + lo with about 16 significant bits, fp32 range.
__device__ __forceinline__ void splitbf(float x, __bf16& hi, __bf16& lo) {
    const __bf16 h = cvtbf_once(x);
    hi = h;
    lo = (__bf16)(x - (float)h);
}

// Pairs: two values rounded together and returned as one packed 32-bit word,
// the low half holding the first value.
__device__ __forceinline__ uint32_t pack_f16(float x0, float x1) {
    f16x2 h = {(_Float16)x0, (_Float16)x1};
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ void split_f16x2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    f16x2 h = {(_Float16)x0, (_Float16)x1};
    __asm__ volatile("" : "+v"(h));
    f16x2 l = {(_Float16)(x0 - (float)h[0]), (_Float16)(x1 - (float)h[1])};
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}
__device__ __forceinline__ void split_bf16x2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    bf16x2 h = {(__bf16)x0, (__bf16)x1};
    __asm__ volatile("" : "+v"(h));
    bf16x2 l = {(__bf16)(x0 - (float)h[0]), (__bf16)(x1 - (float)h[1])};
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}

// Load one element of q/k/v as float.
template <bool F32>
__device__ __forceinline__ float ld_in(const void* p, long long i) {
    if constexpr (F32) {
        return static_cast<const float*>(p)[i];
    } else {
        const uint16_t u = static_cast<const uint16_t*>(p)[i];
        return __uint_as_float(static_cast<uint32_t>(u) << 16);
    }
}

template <typename T>
__device__ __forceinline__ T lds_vec(const void* p) {
    return *reinterpret_cast<const T*>(p);
}

}  // namespace kda
