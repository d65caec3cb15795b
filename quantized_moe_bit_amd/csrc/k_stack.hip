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

}  // namespace

hipError_t launch_glue(const uint16_t *h, const float *y, const uint16_t *post, const uint16_t *scalar,
                       uint16_t *h_next, uint16_t *x_next, int T, int d, hipStream_t s) {
    launch(k_glue, dim3(T), dim3(kGlueWG), 0, s, h, y, post, scalar, h_next, x_next, d);
    return hipGetLastError();
}

}  // namespace qmoe
