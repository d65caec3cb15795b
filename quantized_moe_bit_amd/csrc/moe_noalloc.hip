// Decode without a layer handle and without allocating: moe_forward_decode_noalloc.
//
// The same three decode launches as moe_forward_decode (router, routed and shared gate/up,
// down with the fixed-order combine), with their scratch (logits, top-k, group sums of x,
// hidden activations and their 16-value sums, shared-expert gate values, the router
// prologue's output) placed in one file-scope device array instead of a layer workspace. The
// entry point calls no hipMalloc, hipFree or other allocating routine; it is meant for callers
// that cannot allocate (code under stream capture, tight serving loops).
//
// In host code the name `scratch` stands for a host-side shadow, not the device array: the
// device address is taken with hipGetSymbolAddress, once per device with that device current,
// and only that address is handed to kernels.
#include <mutex>

#include "moe_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(1) << 20;   // the stated maximum: 1 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (hipGetSymbolAddress on the first call
// per device, with that device current).
moe_status scratch_ptr(int dev, void **out) {
    if (dev < 0 || dev >= kMaxDevices) return qmoe::fail(MOE_E_DEVICE, "device %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
        void *p = nullptr;
        const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !p)
            return qmoe::fail(MOE_E_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(err));
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return MOE_OK;
}

// Regions of the decode scratch for T tokens, 256-byte aligned, laid out from offset 0.
struct ScratchPlan {
    size_t off = 0;
    template <class T>
    size_t take(size_t count) {
        off = (off + 255) & ~size_t(255);
        const size_t at = off;
        off += sizeof(T) * (count ? count : 1);
        return at;
    }
};

}  // namespace

extern "C" moe_status moe_forward_decode_noalloc(const moe_dims *dims, const moe_weights *w, const uint16_t *x,
                                                 int32_t T, float *y, void *hip_stream) {
    using namespace qmoe;
    clear_error();
    if (!dims || !w) return fail(MOE_E_INVALID, "moe_forward_decode_noalloc: NULL dims or weights");
    moe_status st = check_layer_args(dims, w);
    if (st != MOE_OK) return st;
    if (w->expert_slot)
        return fail(MOE_E_INVALID, "moe_forward_decode_noalloc: expert slots need a layer handle (moe_layer_create)");
    if (T < 0) return fail(MOE_E_SHAPE, "moe_forward_decode_noalloc: T = %d is negative", T);
    const int cap = dims->max_tokens < MOE_MAX_DECODE_TOKENS ? dims->max_tokens : MOE_MAX_DECODE_TOKENS;
    if (T > cap) return fail(MOE_E_CAPACITY, "moe_forward_decode_noalloc: T = %d exceeds the decode capacity %d", T, cap);
    if (T == 0) return MOE_OK;
    if (!x || !y) return fail(MOE_E_INVALID, "moe_forward_decode_noalloc: NULL input or output");
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) & 15u)
        return fail(MOE_E_ALIGN, "moe_forward_decode_noalloc: input/output not 16-byte aligned");

    // the layer description the launchers read, with its decode scratch in `scratch`
    moe_layer L;
    L.dims = *dims;
    L.w = *w;
    L.G_d = dims->d_model / 64;
    L.G_I = dims->d_expert / 64;
    L.G_Is = dims->d_shared / 64;
    L.max_dec = T;
    L.n_mats = dims->n_experts;
    L.flags = 0;
    L.routed_T = -1;
    L.last_T = T;
    L.ws_base = nullptr;
    L.ws_bytes = 0;
    L.ws = Workspace{};
    L.prof_on = false;
    const moe_dims &D = *dims;
    ScratchPlan plan;
    const size_t o_logits = plan.take<float>((size_t)T * D.n_experts);
    const size_t o_idx = plan.take<int32_t>((size_t)T * D.top_k);
    const size_t o_wts = plan.take<float>((size_t)T * D.top_k);
    const size_t o_u = plan.take<uint16_t>(w->router_scale ? (size_t)T * D.d_model : 0);
    const size_t o_sgate = plan.take<float>(w->shared_gate ? (size_t)T : 0);
    const size_t o_dxg = plan.take<float>(dec_workspace_floats(D, T, 0));
    const size_t o_dhr = plan.take<uint16_t>(2 * dec_workspace_floats(D, T, 1));
    const size_t o_dhs = plan.take<uint16_t>(2 * dec_workspace_floats(D, T, 2));
    const size_t o_dhsr = plan.take<float>(dec_workspace_floats(D, T, 3));
    const size_t o_dhss = plan.take<float>(dec_workspace_floats(D, T, 4));
    if (plan.off > kScratchBytes)
        return fail(MOE_E_CAPACITY,
                    "moe_forward_decode_noalloc: %d tokens of this layer need %zu bytes of scratch; the static "
                    "scratch holds %zu (use moe_layer_create / moe_forward_decode)",
                    T, plan.off, kScratchBytes);

    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return fail(MOE_E_DEVICE, "hipGetDevice: %s", hipGetErrorString(err));
    void *base = nullptr;
    if ((st = scratch_ptr(dev, &base)) != MOE_OK) return st;
    char *b = static_cast<char *>(base);
    L.device = dev;
    L.ws.logits = reinterpret_cast<float *>(b + o_logits);
    L.ws.idx = reinterpret_cast<int32_t *>(b + o_idx);
    L.ws.wts = reinterpret_cast<float *>(b + o_wts);
    L.ws.u = reinterpret_cast<uint16_t *>(b + o_u);
    L.ws.sgate = reinterpret_cast<float *>(b + o_sgate);
    L.ws.dxg = reinterpret_cast<float *>(b + o_dxg);
    L.ws.dh_r = reinterpret_cast<uint16_t *>(b + o_dhr);
    L.ws.dh_s = reinterpret_cast<uint16_t *>(b + o_dhs);
    L.ws.dhs_r = reinterpret_cast<float *>(b + o_dhsr);
    L.ws.dhs_s = reinterpret_cast<float *>(b + o_dhss);
    // Nothing here must start at zero: every value a decode launch reads was written by an
    // earlier launch of the same call (logits and group sums by the router, top-k, hidden
    // activations, their sums and the gate values by gate/up), so the array's previous
    // contents never reach the output.

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (w->router_scale && dec_router_glue_fits(D, T)) {
        err = launch_dec_router_pro(&L, x, T, L.ws.logits, s);
    } else if (w->router_scale) {
        err = launch_router_prologue(&L, x, T, false, s);
        if (err == hipSuccess) err = launch_dec_router(&L, L.ws.u, T, L.ws.logits, s, false);
    } else {
        err = launch_dec_router(&L, x, T, L.ws.logits, s, true);
    }
    if (err == hipSuccess) err = launch_dec_gateup(&L, x, T, s);
    if (err == hipSuccess) err = launch_dec_down(&L, T, y, s);
    if (err != hipSuccess) return fail(MOE_E_DEVICE, "moe_forward_decode_noalloc: %s", hipGetErrorString(err));
    return MOE_OK;
}
