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

// float -> fp16 bits, round to nearest even; magnitudes that round above 65504 become +-inf and
// NaN stays NaN, so a value outside fp16's range makes the layer output non-finite (reported
// under MOE_FLAG_CHECK_FINITE) instead of silently changing it.
__device__ __forceinline__ uint32_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

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

// The four fp16 pairs of one device-layout word as subnormals: pair p holds nibbles p and
// 4 + p (elements 2p, 2p + 1). Masked in place, nibble n sits in mantissa bits 0..3 of its
// half (value q 2^-24) for n = 0, 4 and bits 4..7 (value 16 q 2^-24) for n = 1, 5; the word
// shifted down by 8 gives nibbles 2, 6 and 3, 7 the same way. Pairs 0 and 2 therefore carry
// q 2^-24 and pairs 1 and 3 carry 16 q 2^-24, all exact. One shift and four ands.
__device__ __forceinline__ u32x4_t nib_sub(uint32_t w) {
    const uint32_t w8 = w >> 8;
    return u32x4_t{w & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x000F000Fu, w8 & 0x00F000F0u};
}

// Eight bf16 values -> eight fp16 values, each rounded to nearest even as f32_to_f16 does (exact
// for |v| in fp16's normal range; values that round above 65504 become infinite and smaller
// ones fp16 subnormals, the same conversion the prefill path applies to x).
__device__ __forceinline__ u32x4_t bf16x8_to_f16x8(u32x4_t v) {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = f32_to_f16(__uint_as_float(v[i] << 16)) | (f32_to_f16(__uint_as_float(v[i] & 0xFFFF0000u)) << 16);
    return r;
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
// 16-byte load of data read once per call (decode weight streams): non-temporal, so it does
// not displace what the caches hold for the rest of the call
__device__ __forceinline__ u32x4_t ld16_nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}

// 16-byte store with the non-temporal hint (streamed past the caches), for a large output no
// later kernel of the call reads.
__device__ __forceinline__ void st16_nt(void *p, u32x4_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(p));
}

// fp64 -> bf16 bits, round to nearest even with a single rounding: fp64 -> fp32 with
// round-to-odd (24 significant bits, at least two more than bf16 keeps), then fp32 -> bf16
// with round-to-nearest-even. Inputs are finite and within the fp32 range.
__device__ __forceinline__ uint32_t f64_to_bf16(double v) {
    const float f = (float)v;   // round to nearest even
    uint32_t u = __float_as_uint(f);
    if ((double)f != v && (u & 1u) == 0u && (u & 0x7FFFFFFFu) != 0u) {
        // inexact with an even last bit: the odd neighbour on v's side is the round-to-odd value
        if (fabs((double)f) > fabs(v)) u -= 1u;
        else u += 1u;
    }
    return f32_to_bf16(__uint_as_float(u));
}

__device__ __forceinline__ double bf16_to_f64(uint32_t bits16) { return (double)bf16_to_f32(bits16); }


// Residual step between stacked layers for one token, by one workgroup of kGlueWG threads,
// with the tail of the layer that produced y (Mference system design, "Decode", cb2: post-FFN
// norm, residual add, layer scalar):
//   z  = post ? (y / sqrt(mean(y^2) + 1e-6)) * post : y
//   h' = bf16((h + z) * scalar)      x = bf16(h' / sqrt(mean(h'^2) + 1e-6))
// in fp64 in that order, each rounded once to bf16 (y may be null: h' = h). post: bf16 [d] or
// null; scalar: one bf16 or null (1). Thread i owns the 8-element chunks i, i + kGlueWG, ...
// and issues all of its loads before any arithmetic; the fp64 sums of squares are reduced in
// a fixed order. d % 8 == 0, d <= 8 kGlueWG kGlueChunks. h' goes to h_next unless it is null
// (h_next may alias h); x goes to x_next (global or LDS). red: LDS for kGlueWG / 64 doubles.
// Every thread of the workgroup must call it.
constexpr int kGlueWG = 256;
constexpr int kGlueChunks = 4;

// Largest float of the wave: DPP within rows of 16 (swap pairs, swap halves of quads,
// half-row mirror, row mirror), then the four row results through scalar registers.
template <int CTRL>
__device__ __forceinline__ float max_dpp(float x) {
    const float y = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
    return fmaxf(x, y);
}

__device__ __forceinline__ float wave_max(float x) {
    x = max_dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    x = max_dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    x = max_dpp<0x141>(x);   // row_half_mirror
    x = max_dpp<0x140>(x);   // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Inclusive fp64 sum within each 16-lane row of the wave (every lane of the row active): lane
// 15 of the row gets the row's total, added in a fixed tree (DPP row shifts by 1, 2, 4, 8;
// lanes shifted in from outside the row add 0).
template <int SH>
__device__ __forceinline__ double row_shr_f64(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, 0x110 + SH, 0xF, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), 0x110 + SH, 0xF, 0xF, true);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double row_scan16_f64(double v) {
    v += row_shr_f64<1>(v);
    v += row_shr_f64<2>(v);
    v += row_shr_f64<4>(v);
    v += row_shr_f64<8>(v);
    return v;
}
__device__ __forceinline__ double lane_f64(double v, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// fp64 sum over a full wave in a fixed order (the same value in every lane)
__device__ __forceinline__ double wave_sum_f64(double v) {
    v = row_scan16_f64(v);
    return (lane_f64(v, 15) + lane_f64(v, 31)) + (lane_f64(v, 47) + lane_f64(v, 63));
}

// fixed-order fp64 sum over the workgroup (every thread gets the total; red reusable after)
__device__ __forceinline__ double glue_block_sum(double v, double *red) {
    const int tid = threadIdx.x;
    v = wave_sum_f64(v);
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kGlueWG / 64; ++w) tot += red[w];
    __syncthreads();
    return tot;
}

__device__ __forceinline__ void glue_token(const uint16_t *h, const float *y, const uint16_t *post,
                                           const uint16_t *scalar, uint16_t *h_next, uint16_t *x_next, int d,
                                           double *red) {
    const int tid = threadIdx.x;
    const int nc = d / 8;
    u32x4_t hv[kGlueChunks], pv[kGlueChunks];
    f32x4_t yv[kGlueChunks][2];
    const bool tail = y && post;
#pragma unroll
    for (int c = 0; c < kGlueChunks; ++c) {
        const int i = tid + kGlueWG * c;
        if (i < nc) {
            hv[c] = ld16(h + 8 * i);
            if (y) {
                yv[c][0] = *reinterpret_cast<const f32x4_t *>(y + 8 * i);
                yv[c][1] = *reinterpret_cast<const f32x4_t *>(y + 8 * i + 4);
            }
            if (tail) pv[c] = ld16(post + 8 * i);
        }
    }
    const double sc = (y && scalar) ? bf16_to_f64(*scalar) : 1.0;
    double inv_y = 1.0;
    if (tail) {
        double sy = 0.0;
#pragma unroll
        for (int c = 0; c < kGlueChunks; ++c)
            if (tid + kGlueWG * c < nc) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const double f = (double)yv[c][j >> 2][j & 3];
                    sy = fma(f, f, sy);
                }
            }
        inv_y = 1.0 / sqrt(glue_block_sum(sy, red) / (double)d + 1e-6);
    }
    uint32_t hb[kGlueChunks][8];
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < kGlueChunks; ++c) {
        if (tid + kGlueWG * c < nc) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                double v = bf16_to_f64((hv[c][j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
                if (y) {
                    double z = (double)yv[c][j >> 2][j & 3];
                    if (tail) z = (z * inv_y) * bf16_to_f64((pv[c][j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
                    v = (v + z) * sc;
                }
                hb[c][j] = f64_to_bf16(v);
                const double r = bf16_to_f64(hb[c][j]);
                ss = fma(r, r, ss);
            }
        }
    }
    const double inv = 1.0 / sqrt(glue_block_sum(ss, red) / (double)d + 1e-6);
#pragma unroll
    for (int c = 0; c < kGlueChunks; ++c) {
        const int i = tid + kGlueWG * c;
        if (i < nc) {
            u32x4_t ho, xo;
#pragma unroll
            for (int j2 = 0; j2 < 4; ++j2) {
                ho[j2] = hb[c][2 * j2] | (hb[c][2 * j2 + 1] << 16);
                xo[j2] = f64_to_bf16(bf16_to_f64(hb[c][2 * j2]) * inv) |
                         (f64_to_bf16(bf16_to_f64(hb[c][2 * j2 + 1]) * inv) << 16);
            }
            if (h_next) *reinterpret_cast<u32x4_t *>(h_next + 8 * i) = ho;
            *reinterpret_cast<u32x4_t *>(x_next + 8 * i) = xo;
        }
    }
}

// Slot of routed expert e when the layer keeps its experts in slots (eslot non-null): an absent
// or out-of-range slot is replaced by slot 0, so no access leaves the slab, and counted in
// *faults by the callers that pass count (one per workgroup or wave); the caller's output is
// then void. Without slots the expert's own index.
__device__ __forceinline__ int expert_slot_of(const int32_t *eslot, int n_slots, int32_t *faults, int e,
                                              bool count) {
    if (!eslot) return e;
    int s = eslot[e];
    if (s < 0 || s >= n_slots) {
        if (count) atomicAdd(faults, 1);
        s = 0;
    }
    return s;
}

// Shared-expert gate of one token, by one full workgroup of kGlueWG threads (Mference system
// design, "Scope and limitations": a gated shared expert): a = 1 / (1 + exp(-z)) with
// z = sum_i x_i g_i, x fp16 (global or LDS), g bf16 in global memory, d a multiple of 8.
// Thread i accumulates inputs 8 (i + kGlueWG c) + j in fp32, c then j ascending; the
// partial sums are added by a fixed butterfly within each wave and then wave by wave, so
// every caller gets the same bits for the same x. red: kGlueWG / 64 floats of LDS.
__device__ __forceinline__ float shared_gate_token(const uint16_t *x, const uint16_t *g, int d, float *red) {
    const int tid = threadIdx.x;
    float z = 0.0f;
    for (int i = tid; i < d / 8; i += kGlueWG) {
        const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(x + 8 * i);
        const u32x4_t gv = ld16(g + 8 * i);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float xf = f16_to_f32((xv[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
            z = fmaf(xf, bf16_to_f32((gv[j >> 1] >> (16 * (j & 1))) & 0xFFFFu), z);
        }
    }
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
    if ((tid & 63) == 0) red[tid >> 6] = z;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < kGlueWG / 64; ++w) tot += red[w];
    __syncthreads();
    return 1.0f / (1.0f + __expf(-tot));
}

// Router prologue of one token held in LDS (bf16 [d], d a multiple of 8), in place, by one
// full workgroup of kGlueWG threads: x -> bf16(((x / sqrt(mean(x^2) + 1e-6)) * rs) / sqrt(d)),
// float64 in that order and rounded once (Mference system design, "Decode", router listing).
// rs: bf16 [d] in global memory, 16-byte aligned. red: kGlueWG / 64 doubles of LDS.
__device__ __forceinline__ void prologue_token(uint16_t *xs, const uint16_t *rs, int d, double *red) {
    const int tid = threadIdx.x;
    const int nc = d / 8;
    double ss = 0.0;
    for (int i = tid; i < nc; i += kGlueWG) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(xs + 8 * i);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const double f = bf16_to_f64((v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
            ss = fma(f, f, ss);
        }
    }
    ss = wave_sum_f64(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kGlueWG / 64; ++w) tot += red[w];
    __syncthreads();   // red may be reused by the caller
    const double inv = 1.0 / sqrt(tot / (double)d + 1e-6), sd = sqrt((double)d);
    for (int i = tid; i < nc; i += kGlueWG) {   // each thread rewrites the chunks it alone reads
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(xs + 8 * i);
        const u32x4_t r = *reinterpret_cast<const u32x4_t *>(rs + 8 * i);
        u32x4_t o;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            uint32_t ub[2];
#pragma unroll
            for (int h = 0; h < 2; ++h)
                ub[h] = f64_to_bf16(((bf16_to_f64((v[w] >> (16 * h)) & 0xFFFFu) * inv) *
                                     bf16_to_f64((r[w] >> (16 * h)) & 0xFFFFu)) / sd);
            o[w] = ub[0] | (ub[1] << 16);
        }
        *reinterpret_cast<u32x4_t *>(xs + 8 * i) = o;
    }
}

}  // namespace qmoe
