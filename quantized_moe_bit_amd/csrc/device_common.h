// Device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qmoe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2_t;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// (t & mask) | c in one VALU instruction. The mask comes from a scalar register and c from a
// vector register (one scalar operand per VALU instruction on gfx9).
__device__ __forceinline__ uint32_t and_or(uint32_t t, uint32_t mask, uint32_t c) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(t), "s"(mask), "v"(c));
    return r;
}

// Two bf16 values (1 + q/16) built from the nibbles of one device-layout word.
// Pair p (0..3) holds elements 2p and 2p+1 of the word's eight inputs; element j sits in
// nibble (j even ? j/2 : 4 + j/2), so pair p is nibbles p and 4+p: shifting them to bits 3..6
// and 19..22 and or-ing the exponent of 1.0 gives bf16 values 1 + q/16 (exact).
template <int P>
__device__ __forceinline__ uint32_t nib_pair(uint32_t w) {
    uint32_t t;
    if constexpr (P == 0) t = w << 3;
    else t = w >> (4 * P - 3);
    return and_or(t, 0x00780078u, 0x3F803F80u);
}

// One 16-byte MFMA B fragment (8 bf16) from one device-layout word.
__device__ __forceinline__ bf16x8_t nib_frag(uint32_t w) {
    u32x4_t v = {nib_pair<0>(w), nib_pair<1>(w), nib_pair<2>(w), nib_pair<3>(w)};
    return __builtin_bit_cast(bf16x8_t, v);
}

// float -> fp16 bits, round to nearest even, saturating at +-65504 (the expert hidden activation).
__device__ __forceinline__ uint32_t f32_to_f16_sat(float f) {
    f = fminf(fmaxf(f, -65504.0f), 65504.0f);
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// fp16 version of nib_pair: 1 + q/16 is 0x3C00 | q << 6 in fp16.
template <int P>
__device__ __forceinline__ uint32_t nib_pair_f16(uint32_t w) {
    uint32_t t;
    if constexpr (P == 0) t = w << 6;
    else if constexpr (P == 1) t = w << 2;
    else if constexpr (P == 2) t = w >> 2;
    else t = w >> 6;
    return and_or(t, 0x03C003C0u, 0x3C003C00u);
}

__device__ __forceinline__ f16x8_t nib_frag_f16(uint32_t w) {
    u32x4_t v = {nib_pair_f16<0>(w), nib_pair_f16<1>(w), nib_pair_f16<2>(w), nib_pair_f16<3>(w)};
    return __builtin_bit_cast(f16x8_t, v);
}

__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b), c, false);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                          false);
}

// tanh-form GELU, fp32.
__device__ __forceinline__ float gelu_tanh_f32(float v) {
    const float c = 0.7978845608028654f;
    float z = c * (v + 0.044715f * v * v * v);
    // tanh(z) = 1 - 2 / (exp(2z) + 1), saturating for large |z|
    // 0.5 (1 + tanh z) = 1 - 1 / (exp(2z) + 1); saturates correctly as exp(2z) -> 0 or inf
    const float e = __expf(2.0f * z);
    return v * (1.0f - __builtin_amdgcn_rcpf(e + 1.0f));
}

__device__ __forceinline__ u32x4_t ld16(const void *p) { return *reinterpret_cast<const u32x4_t *>(p); }

}  // namespace qmoe
