// Residual stream between the MoE FFN layers of a decode stack.
//
// The Mference system design ends each decode layer with the post-FFN norm, the residual add
// and a per-layer scalar ("Decode", cb2) and opens the next layer with a norm without a
// learned scale before its projections ("Decode", the router listing). The stack keeps the
// two steps that carry state from one FFN to the next, with the tail of the layer that made y:
//   z      = post ? y / sqrt(mean(y^2) + 1e-6) * post : y
//   h_next = bf16((h + z) * scalar)
//   x_next = bf16(h_next / sqrt(mean(h_next^2) + 1e-6))
// Both are computed in fp64 and rounded once to bf16 (round to nearest even), so the bf16
// results are the correctly rounded values of the exact expressions up to the fp64 rounding
// of the means. Without post and scalar this is the plain residual add.
#include <algorithm>

#include "device_common.h"
#include "moe_internal.h"

namespace qmoe {
namespace {


// One workgroup per token. grid T; block kGlueWG
__global__ __launch_bounds__(kGlueWG) void k_glue(const uint16_t *h, const float *__restrict__ y,
                                                  const uint16_t *post, const uint16_t *scalar,
                                                  uint16_t *h_next, uint16_t *__restrict__ x_next, int d) {
    __shared__ double red[kGlueWG / 64];
    const int t = blockIdx.x;
    glue_token(h + (size_t)t * d, y ? y + (size_t)t * d : nullptr, post, scalar, h_next + (size_t)t * d, x_next + (size_t)t * d, d,
               red);
}

// Debug check (layers created with MOE_FLAG_CHECK_FINITE): *count += number of NaN or infinite
// values among n bf16 (f32: fp32) values. Grid-stride over 16-byte chunks plus a scalar tail;
// a workgroup adds its count once, and only when it is non-zero.
__global__ __launch_bounds__(256) void k_count_nonfinite(const void *__restrict__ p, size_t n, int f32,
                                                         int32_t *__restrict__ count) {
    const size_t per = f32 ? 4 : 8;   // values per 16-byte chunk
    const size_t nchunk = n / per;
    int bad = 0;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nchunk; i += (size_t)gridDim.x * 256) {
        const u32x4_t v = ld16(static_cast<const uint8_t *>(p) + 16 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (f32) {
                bad += (v[j] & 0x7F800000u) == 0x7F800000u;
            } else {
                bad += (v[j] & 0x7F80u) == 0x7F80u;
                bad += (v[j] & 0x7F800000u) == 0x7F800000u;
            }
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < n - nchunk * per) {
        const size_t i = nchunk * per + threadIdx.x;
        if (f32) bad += (static_cast<const uint32_t *>(p)[i] & 0x7F800000u) == 0x7F800000u;
        else bad += (static_cast<const uint16_t *>(p)[i] & 0x7F80u) == 0x7F80u;
    }
    for (int off = 32; off > 0; off >>= 1) bad += __shfl_xor(bad, off);
    __shared__ int red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = bad;
    __syncthreads();
    if (threadIdx.x == 0) {
        const int tot = red[0] + red[1] + red[2] + red[3];
        if (tot) atomicAdd(count, tot);
    }
}

}  // namespace

hipError_t launch_count_nonfinite(const void *p, size_t n, bool f32, int32_t *count, hipStream_t s) {
    const size_t chunks = n / (f32 ? 4 : 8);
    const unsigned grid = (unsigned)std::min<size_t>(1024, std::max<size_t>(1, (chunks + 255) / 256));
    launch(k_count_nonfinite, dim3(grid), dim3(256), 0, s, p, n, (int)f32, count);
    return hipGetLastError();
}

hipError_t launch_glue(const uint16_t *h, const float *y, const uint16_t *post, const uint16_t *scalar,
                       uint16_t *h_next, uint16_t *x_next, int T, int d, hipStream_t s) {
    launch(k_glue, dim3(T), dim3(kGlueWG), 0, s, h, y, post, scalar, h_next, x_next, d);
    return hipGetLastError();
}

}  // namespace qmoe
