// Residual stream between the MoE FFN layers of a decode stack.
//
// The Mference system design ends each decode layer with post-FFN norms, the residual add
// and a per-layer scalar ("Decode", the layer tail) and opens the next layer with a norm
// without a learned scale before its projections ("Decode", the router listing). The stack
// here keeps the two steps that carry state from one FFN to the next:
//   h_next = bf16(h + y)
//   x_next = bf16(h_next / sqrt(mean(h_next^2) + 1e-6))
// Both are computed in fp64 and rounded once to bf16 (round to nearest even), so the bf16
// results are the correctly rounded values of the exact expressions up to the fp64 rounding
// of the mean; the learned norm scales and the layer scalar are not applied.
#include "device_common.h"
#include "moe_internal.h"

namespace qmoe {
namespace {

constexpr int kGlueWG = 256;
constexpr int kGlueChunks = 4;   // 8-element chunks per thread: d <= 8192

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

// One workgroup per token; thread i owns the 8-element chunks i, i + kGlueWG, ... and issues
// all of their loads before any arithmetic (the inputs were just written by another kernel).
// grid T; block kGlueWG; d <= 8 kGlueWG kGlueChunks, d % 8 == 0
__global__ __launch_bounds__(kGlueWG) void k_glue(const uint16_t *h, const float *__restrict__ y,
                                                  uint16_t *h_next, uint16_t *__restrict__ x_next, int d) {
    __shared__ double red[kGlueWG / 64];
    const int t = blockIdx.x, tid = threadIdx.x;
    const int nc = d / 8;
    u32x4_t hv[kGlueChunks];
    f32x4_t yv[kGlueChunks][2];
#pragma unroll
    for (int c = 0; c < kGlueChunks; ++c) {
        const int i = tid + kGlueWG * c;
        if (i < nc) {
            hv[c] = ld16(h + (size_t)t * d + 8 * i);
            if (y) {
                yv[c][0] = *reinterpret_cast<const f32x4_t *>(y + (size_t)t * d + 8 * i);
                yv[c][1] = *reinterpret_cast<const f32x4_t *>(y + (size_t)t * d + 8 * i + 4);
            }
        }
    }
    uint32_t hb[kGlueChunks][8];
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < kGlueChunks; ++c) {
        if (tid + kGlueWG * c < nc) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                double v = bf16_to_f64((hv[c][j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
                if (y) v += (double)yv[c][j >> 2][j & 3];
                hb[c][j] = f64_to_bf16(v);
                const double r = bf16_to_f64(hb[c][j]);
                ss = fma(r, r, ss);
            }
        }
    }
    // wave sums, then the wave partials in a fixed order
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kGlueWG / 64; ++w) tot += red[w];
    const double inv = 1.0 / sqrt(tot / (double)d + 1e-6);
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
            *reinterpret_cast<u32x4_t *>(h_next + (size_t)t * d + 8 * i) = ho;
            *reinterpret_cast<u32x4_t *>(x_next + (size_t)t * d + 8 * i) = xo;
        }
    }
}

}  // namespace

hipError_t launch_glue(const uint16_t *h, const float *y, uint16_t *h_next, uint16_t *x_next, int T, int d,
                       hipStream_t s) {
    launch(k_glue, dim3(T), dim3(kGlueWG), 0, s, h, y, h_next, x_next, d);
    return hipGetLastError();
}

}  // namespace qmoe
