// GPU slot map lookup (Mference system design, "Decode": the router's top-k IDs are resolved
// against the layer's expert-to-slot table on the GPU). One workgroup marks every selected
// expert whose slot is absent in an LDS bitmap, then one wave lists the marked experts in
// ascending order: missing[0] = their number, missing[1 ..] = the experts.
#include "device_common.h"
#include "moe_internal.h"

namespace qmoe {
namespace {

// grid 1; block 256; E <= MOE_MAX_EXPERTS
__global__ __launch_bounds__(256) void k_slot_lookup(const int32_t *__restrict__ idx, int n, int E,
                                                     const int32_t *__restrict__ eslot, int n_slots,
                                                     int32_t *__restrict__ missing) {
    __shared__ int flag[MOE_MAX_EXPERTS];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 256) flag[e] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
        const int e = idx[i];
        if (e >= 0 && e < E) {
            const int s = eslot[e];
            if (s < 0 || s >= n_slots) flag[e] = 1;
        }
    }
    __syncthreads();
    if (tid < 64) {
        int base = 0;
        for (int c = 0; c < E; c += 64) {
            const int e = c + tid;
            const bool f = e < E && flag[e];
            const uint64_t m = __ballot(f);
            if (f) missing[1 + base + __popcll(m & ((1ull << tid) - 1ull))] = e;
            base += __popcll(m);
        }
        if (tid == 0) missing[0] = base;
    }
}

}  // namespace

hipError_t launch_slot_lookup(const moe_layer *L, const int32_t *idx, int T, int32_t *missing, hipStream_t s) {
    launch(k_slot_lookup, dim3(1), dim3(256), 0, s, idx, T * L->dims.top_k, L->dims.n_experts, L->w.expert_slot,
           L->w.n_slots, missing);
    return hipGetLastError();
}

}  // namespace qmoe
