// Host side of the C ABI: argument validation (entirely before any enqueue), the
// layer-owned workspace, and the stream-ordered kernel sequences of the decode and
// prefill paths. Errors never cross the ABI as exceptions; a failed call leaves the
// handle usable and writes nothing.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <utility>
#include <vector>

#include "moe_internal.h"

namespace qmoe {

static thread_local char g_err[512] = "";
thread_local LaunchTiming g_timing;

moe_status fail(moe_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { g_err[0] = 0; }

namespace {

const char *kKernelNames[K_COUNT] = {"router",     "topk",       "bucket_rank", "bucket_scan", "bucket_scatter",
                                     "dec_router", "dec_gateup", "dec_down", "pre_gateup",  "pre_down",
                                     "combine",    "glue",       "router_prologue", "slot_lookup"};

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_dims(const moe_dims *D) {
    if (!D) return fail(MOE_E_INVALID, "dims is NULL");
    if (D->group != 64) return fail(MOE_E_QUANT, "group must be 64, got %d", D->group);
    if (D->router_bits != 8) return fail(MOE_E_QUANT, "router_bits must be 8, got %d", D->router_bits);
    if (D->expert_bits != 4) return fail(MOE_E_QUANT, "expert_bits must be 4, got %d", D->expert_bits);
    if (D->expert_format != MOE_FORMAT_AFFINE_G64 && D->expert_format != MOE_FORMAT_Q4_0)
        return fail(MOE_E_QUANT, "expert_format %d is neither MOE_FORMAT_AFFINE_G64 nor MOE_FORMAT_Q4_0",
                    D->expert_format);
    if (D->d_model < 64 || D->d_model % 64 || D->d_model > 8192)
        return fail(MOE_E_SHAPE, "d_model %d must be a multiple of 64 in [64, 8192]", D->d_model);
    if (D->d_expert < 64 || D->d_expert % 64)
        return fail(MOE_E_SHAPE, "d_expert %d must be a positive multiple of 64", D->d_expert);
    if (D->d_shared < 64 || D->d_shared % 64)
        return fail(MOE_E_SHAPE, "d_shared %d must be a positive multiple of 64", D->d_shared);
    if (D->n_experts < 1 || D->n_experts > MOE_MAX_EXPERTS)
        return fail(MOE_E_SHAPE, "n_experts %d out of range [1, %d]", D->n_experts, MOE_MAX_EXPERTS);
    if (D->top_k < 1 || D->top_k > D->n_experts || D->top_k > MOE_MAX_TOP_K)
        return fail(MOE_E_SHAPE, "top_k %d out of range [1, min(n_experts, %d)]", D->top_k, MOE_MAX_TOP_K);
    if (D->max_tokens < 1 || D->max_tokens > (1 << 20))
        return fail(MOE_E_SHAPE, "max_tokens %d out of range [1, 2^20]", D->max_tokens);
    if (D->d_expert > 16384 || D->d_shared > 16384)
        return fail(MOE_E_SHAPE, "d_expert %d / d_shared %d above 16384", D->d_expert, D->d_shared);
    {
        // the prefill GEMMs address activation rows with 32-bit byte offsets
        const uint64_t P = (uint64_t)D->max_tokens * D->top_k;
        const uint64_t wmax = (uint64_t)(D->d_model > D->d_expert ? D->d_model : D->d_expert);
        if (P * wmax * 2 >= (1ull << 32) || (uint64_t)D->max_tokens * D->d_shared * 2 >= (1ull << 32))
            return fail(MOE_E_SHAPE, "max_tokens %d too large: activation buffers exceed 4 GiB", D->max_tokens);
    }
    if (max_routed_tiles(D->max_tokens, D->top_k, D->n_experts) > kTileTabMax)
        return fail(MOE_E_SHAPE, "max_tokens %d too large: a chunk could hold more than %d routed row tiles "
                    "(ceil(max_tokens top_k / 128) + min(n_experts, max_tokens top_k))", D->max_tokens, kTileTabMax);
    if (dec_down_lds(*D) > 65536)
        return fail(MOE_E_SHAPE, "top_k * d_expert + d_shared = %d too large for the decode down projection (LDS)",
                    D->top_k * D->d_expert + D->d_shared);
    return MOE_OK;
}

moe_status check_qmat(const moe_qmat &m, const char *name) {
    if (!m.codes || !m.sb) return fail(MOE_E_INVALID, "weight %s: NULL pointer", name);
    if (!aligned16(m.codes) || !aligned16(m.sb)) return fail(MOE_E_ALIGN, "weight %s: pointer not 16-byte aligned", name);
    return MOE_OK;
}

moe_status check_weights(const moe_weights *w) {
    if (!w) return fail(MOE_E_INVALID, "weights is NULL");
    moe_status s;
    if ((s = check_qmat(w->router, "router")) != MOE_OK) return s;
    if ((s = check_qmat(w->gate, "gate")) != MOE_OK) return s;
    if ((s = check_qmat(w->up, "up")) != MOE_OK) return s;
    if ((s = check_qmat(w->down, "down")) != MOE_OK) return s;
    if ((s = check_qmat(w->sh_gate, "sh_gate")) != MOE_OK) return s;
    if ((s = check_qmat(w->sh_up, "sh_up")) != MOE_OK) return s;
    if ((s = check_qmat(w->sh_down, "sh_down")) != MOE_OK) return s;
    if (w->logit_bias && !aligned16(w->logit_bias)) return fail(MOE_E_ALIGN, "logit_bias not 16-byte aligned");
    if (w->router_scale && !aligned16(w->router_scale)) return fail(MOE_E_ALIGN, "router_scale not 16-byte aligned");
    if (w->post_ffn_norm && !aligned16(w->post_ffn_norm)) return fail(MOE_E_ALIGN, "post_ffn_norm not 16-byte aligned");
    if (w->shared_gate && !aligned16(w->shared_gate)) return fail(MOE_E_ALIGN, "shared_gate not 16-byte aligned");
    if (w->expert_slot) {
        if (reinterpret_cast<uintptr_t>(w->expert_slot) & 3u) return fail(MOE_E_ALIGN, "expert_slot not 4-byte aligned");
        if (w->n_slots < 1 || w->n_slots > MOE_MAX_EXPERTS)
            return fail(MOE_E_SHAPE, "n_slots %d out of range [1, %d]", w->n_slots, MOE_MAX_EXPERTS);
    }
    return MOE_OK;
}

}  // namespace

moe_status check_layer_args(const moe_dims *D, const moe_weights *w) {
    moe_status st = check_dims(D);
    return st != MOE_OK ? st : check_weights(w);
}

namespace {

moe_status check_tokens(moe_layer *L, int32_t T, const char *what) {
    if (!L) return fail(MOE_E_INVALID, "%s: layer is NULL", what);
    if (T < 0) return fail(MOE_E_SHAPE, "%s: T = %d is negative", what, T);
    if (T > L->dims.max_tokens)
        return fail(MOE_E_CAPACITY, "%s: T = %d exceeds max_tokens %d", what, T, L->dims.max_tokens);
    return MOE_OK;
}

moe_status check_call(moe_layer *L, const void *x, int32_t T, const void *out, const char *what) {
    moe_status st = check_tokens(L, T, what);
    if (st != MOE_OK || T == 0) return st;
    if (!x || !out) return fail(MOE_E_INVALID, "%s: NULL input or output", what);
    if (!aligned16(x) || !aligned16(out)) return fail(MOE_E_ALIGN, "%s: input/output not 16-byte aligned", what);
    return MOE_OK;
}

// Bump allocator over one device allocation; every region 256-byte aligned. take() records
// where each region's pointer lives, and rebase() turns every recorded offset into an address
// inside the allocation, so no region can be left holding a bare offset.
struct Plan {
    size_t off = 0;
    std::vector<std::pair<void *, size_t>> slots;   // (address of the pointer, byte offset)
    template <class T>
    void take(T **p, size_t count) {
        off = (off + 255) & ~size_t(255);
        slots.emplace_back(static_cast<void *>(p), off);
        *p = nullptr;
        off += sizeof(T) * (count ? count : 1);
    }
    void rebase(char *base) const {
        for (const auto &sl : slots) {
            char *addr = base + sl.second;
            std::memcpy(sl.first, &addr, sizeof(addr));   // every object pointer has one representation
        }
    }
};

hipError_t prof_begin(moe_layer *L, int id, hipStream_t s, hipEvent_t *a, hipEvent_t *b) {
    (void)id;
    if (!L->prof_on) return hipSuccess;
    auto grab = [&](hipEvent_t *e) -> hipError_t {
        if (!L->prof_pool.empty()) {
            *e = L->prof_pool.back();
            L->prof_pool.pop_back();
            return hipSuccess;
        }
        return hipEventCreate(e);
    };
    hipError_t err = grab(a);
    if (err != hipSuccess) return err;
    if ((err = grab(b)) != hipSuccess) return err;
    (void)s;
    g_timing.start = *a;   // consumed by the launcher's kernel launches
    g_timing.stop = *b;
    return hipSuccess;
}

hipError_t prof_end(moe_layer *L, int id, hipStream_t s, hipEvent_t a, hipEvent_t b) {
    (void)s;
    if (!L->prof_on) return hipSuccess;
    g_timing = LaunchTiming{};
    L->prof_pending.push_back(ProfEvent{id, a, b});
    return hipSuccess;
}

// Runs one launcher, with optional event timing, mapping errors to MOE_E_DEVICE.
template <class F>
moe_status run(moe_layer *L, int id, hipStream_t s, F &&f) {
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t err = prof_begin(L, id, s, &a, &b);
    if (err == hipSuccess) err = f();
    if (err == hipSuccess) err = prof_end(L, id, s, a, b);
    else g_timing = LaunchTiming{};
    if (err != hipSuccess) return fail(MOE_E_DEVICE, "kernel %s: %s", kKernelNames[id], hipGetErrorString(err));
    return MOE_OK;
}

#define RUN(id, expr)                                              \
    do {                                                           \
        moe_status _st = run(L, id, s, [&]() { return (expr); }); \
        if (_st != MOE_OK) return _st;                             \
    } while (0)

// MOE_FLAG_CHECK_FINITE: the number of NaN / infinite values among n values at p (bf16, or fp32
// with f32), counted on the stream and read back (the stream is synchronized). MOE_E_NONFINITE
// when there are any.
moe_status check_finite(moe_layer *L, const void *p, size_t n, bool f32, hipStream_t s, const char *what) {
    int32_t cnt = 0;
    hipError_t err = hipMemsetAsync(L->ws.flag, 0, sizeof(int32_t), s);
    if (err == hipSuccess) err = launch_count_nonfinite(p, n, f32, L->ws.flag, s);
    if (err == hipSuccess) err = hipMemcpyAsync(&cnt, L->ws.flag, sizeof(cnt), hipMemcpyDeviceToHost, s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (err != hipSuccess) return fail(MOE_E_DEVICE, "%s: finite check: %s", what, hipGetErrorString(err));
    if (cnt) return fail(MOE_E_NONFINITE, "%s: %d NaN or infinite %s values", what, cnt, f32 ? "output" : "input");
    return MOE_OK;
}

#define CHECK_FINITE(p, n, f32, what)                                               \
    do {                                                                            \
        if (L->flags & MOE_FLAG_CHECK_FINITE) {                                     \
            moe_status _st = check_finite(L, (p), (size_t)(n), (f32), s, (what));   \
            if (_st != MOE_OK) return _st;                                          \
        }                                                                           \
    } while (0)

// Routed experts of a layer with expert slots: the fp16 staging exponents of the matrices now in
// the slots (they are filled after creation), with unstageable ones counted as slot faults.
moe_status slot_stage_shift(moe_layer *L, hipStream_t s) {
    if (!L->w.expert_slot) return MOE_OK;
    hipError_t err = launch_stage_shift(L, true, false, L->ws.slot_faults, s);
    if (err != hipSuccess) return fail(MOE_E_DEVICE, "kernel stage_shift: %s", hipGetErrorString(err));
    return MOE_OK;
}

// The router's input: x itself, or the router prologue's output (which also writes what the
// router would have derived from x: the fp16 copy for prefill, the group sums for decode).
moe_status router_input(moe_layer *L, const uint16_t *x, int T, bool for_prefill, hipStream_t s, const uint16_t **u) {
    *u = x;
    if (!L->w.router_scale) return MOE_OK;
    RUN(K_ROUTER_PROLOGUE, launch_router_prologue(L, x, T, for_prefill, s));
    *u = L->ws.u;
    return MOE_OK;
}

moe_status route_impl(moe_layer *L, const uint16_t *x, int T, hipStream_t s, float *logits, int32_t *idx,
                      float *w, bool bucket, int32_t *perm_out, bool prefill) {
    const bool dec = !prefill && T <= L->max_dec;
    if (dec && L->w.router_scale && dec_router_glue_fits(L->dims, T)) {
        RUN(K_ROUTER, launch_dec_router_pro(L, x, T, logits, s));
    } else {
        const uint16_t *u = x;
        moe_status st = router_input(L, x, T, !dec, s, &u);
        if (st != MOE_OK) return st;
        if (dec) RUN(K_ROUTER, launch_dec_router(L, u, T, logits, s, u == x));
        else RUN(K_ROUTER, launch_router(L, u, T, logits, s, u == x));
    }
    RUN(K_TOPK, launch_topk(L, T, logits, idx, w, s));
    if (bucket) {
        RUN(K_BUCKET_RANK, launch_bucket_rank(L, T, idx, s));
        RUN(K_BUCKET_SCAN, launch_bucket_scan(L, T, s));
        RUN(K_BUCKET_SCATTER, launch_bucket_scatter(L, T, idx, perm_out, s));
    }
    return MOE_OK;
}

}  // namespace
}  // namespace qmoe

using namespace qmoe;

extern "C" {

const char *moe_status_str(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_E_INVALID: return "MOE_E_INVALID";
        case MOE_E_SHAPE: return "MOE_E_SHAPE";
        case MOE_E_QUANT: return "MOE_E_QUANT";
        case MOE_E_ALIGN: return "MOE_E_ALIGN";
        case MOE_E_CAPACITY: return "MOE_E_CAPACITY";
        case MOE_E_NOMEM: return "MOE_E_NOMEM";
        case MOE_E_DEVICE: return "MOE_E_DEVICE";
        case MOE_E_NONFINITE: return "MOE_E_NONFINITE";
    }
    return "MOE_E_UNKNOWN";
}

const char *moe_last_error(void) { return g_err; }

#ifndef QMOE_SOURCE_HASH
#define QMOE_SOURCE_HASH "unknown"
#endif
const char *moe_build_id(void) { return QMOE_SOURCE_HASH; }

const char *moe_kernel_name(int32_t id) { return (id >= 0 && id < K_COUNT) ? kKernelNames[id] : nullptr; }

moe_status moe_layer_create(const moe_dims *dims, const moe_weights *w, uint32_t flags, moe_layer **out) {
    clear_error();
    if (!out) return fail(MOE_E_INVALID, "out is NULL");
    moe_status st = check_dims(dims);
    if (st != MOE_OK) return st;
    if ((st = check_weights(w)) != MOE_OK) return st;
    if (flags & ~(MOE_FLAG_CHECK_FINITE | MOE_FLAG_WS_BUDGET_MIB(0xFFFFFFu)))
        return fail(MOE_E_INVALID, "unknown flags 0x%x", flags);

    moe_layer *L = new (std::nothrow) moe_layer();
    if (!L) return fail(MOE_E_NOMEM, "host allocation failed");
    L->dims = *dims;
    L->w = *w;
    L->flags = flags;
    L->routed_T = -1;
    L->last_T = -1;
    L->n_mats = w->expert_slot ? w->n_slots : dims->n_experts;
    L->prof_on = false;
    for (int i = 0; i < K_COUNT; ++i) {
        L->prof_ms[i] = 0.0;
        L->prof_n[i] = 0;
    }
    const moe_dims &D = *dims;
    const int E = D.n_experts, k = D.top_k, d = D.d_model, I = D.d_expert, Is = D.d_shared;
    const size_t Tm = (size_t)D.max_tokens, P = Tm * k;
    L->G_d = d / 64;
    L->G_I = I / 64;
    L->G_Is = Is / 64;
    L->max_dec = D.max_tokens < MOE_MAX_DECODE_TOKENS ? D.max_tokens : MOE_MAX_DECODE_TOKENS;
    const size_t nchunks = (size_t)cdiv((int)P, kChunk);

    Plan plan;
    Workspace &ws = L->ws;
    plan.take(&ws.logits, Tm * E);
    plan.take(&ws.idx, P);
    plan.take(&ws.wts, P);
    plan.take(&ws.x16, Tm * d);
    plan.take(&ws.u, w->router_scale ? Tm * d : 0);
    plan.take(&ws.counts, E);
    plan.take(&ws.offsets, E + 1);
    plan.take(&ws.list[0], (size_t)kXcds * gemm_list_cap(D, (int)Tm, 0));
    plan.take(&ws.list[1], (size_t)kXcds * gemm_list_cap(D, (int)Tm, 1));
    plan.take(&ws.list_n, 2 * kXcds);
    plan.take(&ws.chunk_base, nchunks * E);
    plan.take(&ws.rank, P);
    plan.take(&ws.perm, P);
    plan.take(&ws.pos, P);
    plan.take(&ws.h_r, P * I);
    plan.take(&ws.h_s, Tm * Is);
    plan.take(&ws.r, P * d);
    plan.take(&ws.sh, Tm * d);
    plan.take(&ws.sgate, w->shared_gate ? Tm : 0);
    plan.take(&ws.slot_faults, 1);
    plan.take(&ws.rqf, router_table_floats(D));
    plan.take(&ws.rqm, router_mtable_floats(D));
    plan.take(&ws.flag, 1);
    plan.take(&ws.shift, 3 * (size_t)L->n_mats + 3);
    plan.take(&ws.dxg, dec_workspace_floats(D, L->max_dec, 0));
    plan.take(&ws.dh_r, 2 * dec_workspace_floats(D, L->max_dec, 1));
    plan.take(&ws.dh_s, 2 * dec_workspace_floats(D, L->max_dec, 2));
    plan.take(&ws.dhs_r, dec_workspace_floats(D, L->max_dec, 3));
    plan.take(&ws.dhs_s, dec_workspace_floats(D, L->max_dec, 4));
    plan.take(&ws.dss, (size_t)L->max_dec * (d / 16));
    L->ws_bytes = (plan.off + 255) & ~size_t(255);
    const uint64_t budget_mib = flags >> 8;
    if (budget_mib && L->ws_bytes > (budget_mib << 20)) {
        const size_t need = L->ws_bytes;
        delete L;
        return fail(MOE_E_NOMEM, "workspace of %zu bytes exceeds the budget of %llu MiB", need,
                    (unsigned long long)budget_mib);
    }

    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) {
        delete L;
        return fail(MOE_E_DEVICE, "hipGetDevice: %s", hipGetErrorString(err));
    }
    L->device = dev;
    err = hipMalloc(&L->ws_base, L->ws_bytes);
    if (err != hipSuccess) {
        (void)hipGetLastError();
        delete L;
        return fail(MOE_E_NOMEM, "workspace of %zu bytes: %s", plan.off, hipGetErrorString(err));
    }
    plan.rebase(static_cast<char *>(L->ws_base));
    // zero once: padding columns of the split sums rely on it
    err = hipMemset(L->ws_base, 0, L->ws_bytes);
    // derived bias-term tables of the prefill GEMMs (read from the borrowed scale/bias words)
    if (err == hipSuccess) err = launch_router_table(L, nullptr);
    // fp16 staging exponents of the prefill GEMMs, and the check that every expert matrix can be
    // staged (routed ones of a layer with slots: at each prefill call, once the slots are filled)
    int32_t bad = 0;
    if (err == hipSuccess) err = launch_stage_shift(L, !w->expert_slot, true, ws.flag, nullptr);
    if (err == hipSuccess) err = hipMemcpy(&bad, ws.flag, sizeof(bad), hipMemcpyDeviceToHost);
    if (err == hipSuccess) err = hipDeviceSynchronize();
    if (err != hipSuccess) {
        (void)hipFree(L->ws_base);
        delete L;
        return fail(MOE_E_DEVICE, "workspace init: %s", hipGetErrorString(err));
    }
    if (bad) {
        (void)hipFree(L->ws_base);
        delete L;
        return fail(MOE_E_QUANT,
                    "%d expert matrices have scales or biases the fp16 staging cannot carry (NaN or infinite, "
                    "largest |scale| outside [2^-73, 2^56), or floor(log2 |bias|) >= floor(log2 max |scale|) + 24; "
                    "Q4_0: a NaN or infinite d)",
                    bad);
    }
    *out = L;
    return MOE_OK;
}

void moe_layer_destroy(moe_layer *L) {
    if (!L) return;
    int cur = 0;
    (void)hipGetDevice(&cur);
    (void)hipSetDevice(L->device);
    (void)hipDeviceSynchronize();
    if (L->ws_base) (void)hipFree(L->ws_base);
    for (auto &p : L->prof_pending) {
        (void)hipEventDestroy(p.a);
        (void)hipEventDestroy(p.b);
    }
    for (auto e : L->prof_pool) (void)hipEventDestroy(e);
    (void)hipSetDevice(cur);
    delete L;
}

moe_status moe_route(moe_layer *L, const uint16_t *x, int32_t T, int32_t *topk_idx, float *topk_w, float *logits,
                     int32_t *expert_offsets, int32_t *pair_perm, void *hip_stream) {
    clear_error();
    moe_status st = check_call(L, x, T, topk_idx, "moe_route");
    if (st != MOE_OK || T == 0) return st;
    if (!topk_w) return fail(MOE_E_INVALID, "moe_route: topk_w is NULL");
    if (!aligned16(topk_w) || (logits && !aligned16(logits)))
        return fail(MOE_E_ALIGN, "moe_route: output not 16-byte aligned");
    if ((expert_offsets == nullptr) != (pair_perm == nullptr))
        return fail(MOE_E_INVALID, "moe_route: expert_offsets and pair_perm must be given together");
    if (expert_offsets && (!aligned16(expert_offsets) || !aligned16(pair_perm)))
        return fail(MOE_E_ALIGN, "moe_route: grouping outputs not 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    CHECK_FINITE(x, (size_t)T * L->dims.d_model, false, "moe_route");
    float *lg = logits ? logits : L->ws.logits;
    L->routed_T = -1;   // the router and grouping kernels reuse the workspace of a routed chunk
    st = route_impl(L, x, T, s, lg, topk_idx, topk_w, expert_offsets != nullptr, pair_perm, false);
    if (st != MOE_OK) return st;
    if (expert_offsets) {
        hipError_t err = hipMemcpyAsync(expert_offsets, L->ws.offsets, sizeof(int32_t) * (L->dims.n_experts + 1),
                                        hipMemcpyDeviceToDevice, s);
        if (err != hipSuccess) return fail(MOE_E_DEVICE, "offsets copy: %s", hipGetErrorString(err));
    }
    return MOE_OK;
}

moe_status moe_forward_decode(moe_layer *L, const uint16_t *x, int32_t T, float *y, void *hip_stream) {
    clear_error();
    moe_status st = check_call(L, x, T, y, "moe_forward_decode");
    if (st != MOE_OK || T == 0) return st;
    if (T > L->max_dec)
        return fail(MOE_E_CAPACITY, "moe_forward_decode: T = %d exceeds the decode capacity %d", T, L->max_dec);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    CHECK_FINITE(x, (size_t)T * L->dims.d_model, false, "moe_forward_decode");
    L->routed_T = -1;
    L->last_T = T;
    if (L->w.router_scale && dec_router_glue_fits(L->dims, T)) {
        RUN(K_DEC_ROUTER, launch_dec_router_pro(L, x, T, L->ws.logits, s));
    } else {
        const uint16_t *u = x;
        if ((st = router_input(L, x, T, false, s, &u)) != MOE_OK) return st;
        RUN(K_DEC_ROUTER, launch_dec_router(L, u, T, L->ws.logits, s, u == x));
    }
    RUN(K_DEC_GATEUP, launch_dec_gateup(L, x, T, s));
    RUN(K_DEC_DOWN, launch_dec_down(L, T, y, s));
    CHECK_FINITE(y, (size_t)T * L->dims.d_model, true, "moe_forward_decode");
    return MOE_OK;
}

moe_status moe_forward_prefill(moe_layer *L, const uint16_t *x, int32_t T, float *y, void *hip_stream) {
    clear_error();
    moe_status st = check_call(L, x, T, y, "moe_forward_prefill");
    if (st != MOE_OK || T == 0) return st;
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    CHECK_FINITE(x, (size_t)T * L->dims.d_model, false, "moe_forward_prefill");
    L->routed_T = T;
    L->last_T = T;
    st = route_impl(L, x, T, s, L->ws.logits, L->ws.idx, L->ws.wts, true, nullptr, true);
    if (st != MOE_OK) return st;
    if ((st = slot_stage_shift(L, s)) != MOE_OK) return st;
    RUN(K_PRE_GATEUP, launch_pre_gateup(L, x, T, s));
    RUN(K_PRE_DOWN, launch_pre_down(L, T, s));
    RUN(K_COMBINE, launch_combine(L, T, y, s));
    CHECK_FINITE(y, (size_t)T * L->dims.d_model, true, "moe_forward_prefill");
    return MOE_OK;
}

moe_status moe_last_routing(moe_layer *L, int32_t T, int32_t *idx, float *w, void *hip_stream) {
    clear_error();
    if (!L) return fail(MOE_E_INVALID, "moe_last_routing: layer is NULL");
    if (T < 0) return fail(MOE_E_SHAPE, "moe_last_routing: T = %d is negative", T);
    if (L->last_T < 0) return fail(MOE_E_INVALID, "moe_last_routing: no forward call has run on the layer");
    if (T > L->last_T)
        return fail(MOE_E_INVALID, "moe_last_routing: T = %d exceeds the last call's %d tokens", T, L->last_T);
    if (T == 0) return MOE_OK;
    if (!idx || !w) return fail(MOE_E_INVALID, "moe_last_routing: NULL output");
    if (!aligned16(idx) || !aligned16(w)) return fail(MOE_E_ALIGN, "moe_last_routing: output not 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const size_t n = (size_t)T * L->dims.top_k;
    hipError_t err = hipMemcpyAsync(idx, L->ws.idx, n * sizeof(int32_t), hipMemcpyDeviceToDevice, s);
    if (err == hipSuccess) err = hipMemcpyAsync(w, L->ws.wts, n * sizeof(float), hipMemcpyDeviceToDevice, s);
    if (err != hipSuccess) return fail(MOE_E_DEVICE, "moe_last_routing: %s", hipGetErrorString(err));
    return MOE_OK;
}

moe_status moe_stack_glue(const uint16_t *h, const float *y, const uint16_t *post, const uint16_t *scalar,
                          uint16_t *h_next, uint16_t *x_next, int32_t T, int32_t d, void *hip_stream) {
    clear_error();
    if (T < 0) return fail(MOE_E_SHAPE, "moe_stack_glue: T = %d is negative", T);
    if (d < 8 || d % 8 || d > 8192)
        return fail(MOE_E_SHAPE, "moe_stack_glue: d = %d must be a multiple of 8 in [8, 8192]", d);
    if (T == 0) return MOE_OK;
    if (!h || !h_next || !x_next) return fail(MOE_E_INVALID, "moe_stack_glue: NULL pointer");
    if (!aligned16(h) || !aligned16(h_next) || !aligned16(x_next) || (y && !aligned16(y)) ||
        (post && !aligned16(post)))
        return fail(MOE_E_ALIGN, "moe_stack_glue: pointer not 16-byte aligned");
    hipError_t err = launch_glue(h, y, post, scalar, h_next, x_next, T, d, static_cast<hipStream_t>(hip_stream));
    if (err != hipSuccess) return fail(MOE_E_DEVICE, "kernel glue: %s", hipGetErrorString(err));
    return MOE_OK;
}

moe_status moe_stack_forward_decode(moe_layer *const *layers, int32_t n_layers, uint16_t *h, int32_t T,
                                    uint16_t *x_buf, float *y_buf, uint16_t *h_buf, void *hip_stream) {
    clear_error();
    if (n_layers < 1 || !layers) return fail(MOE_E_INVALID, "moe_stack_forward_decode: no layers");
    if (T < 0) return fail(MOE_E_SHAPE, "moe_stack_forward_decode: T = %d is negative", T);
    for (int l = 0; l < n_layers; ++l) {
        const moe_layer *L = layers[l];
        if (!L) return fail(MOE_E_INVALID, "moe_stack_forward_decode: layer %d is NULL", l);
        if (L->dims.d_model != layers[0]->dims.d_model)
            return fail(MOE_E_SHAPE, "moe_stack_forward_decode: layer %d has d_model %d, layer 0 has %d", l,
                        L->dims.d_model, layers[0]->dims.d_model);
        if (T > L->max_dec)
            return fail(MOE_E_CAPACITY, "moe_stack_forward_decode: T = %d exceeds layer %d's decode capacity %d", T,
                        l, L->max_dec);
    }
    if (T == 0) return MOE_OK;
    if (!h || !x_buf || !y_buf || !h_buf) return fail(MOE_E_INVALID, "moe_stack_forward_decode: NULL buffer");
    if (!aligned16(h) || !aligned16(x_buf) || !aligned16(y_buf) || !aligned16(h_buf))
        return fail(MOE_E_ALIGN, "moe_stack_forward_decode: buffer not 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int d = layers[0]->dims.d_model;
    moe_layer *check = nullptr;   // a layer created with MOE_FLAG_CHECK_FINITE: its flag workspace counts
    for (int l = 0; l < n_layers; ++l)
        if (layers[l]->flags & MOE_FLAG_CHECK_FINITE) check = layers[l];
    if (check) {
        moe_status st = check_finite(check, h, (size_t)T * d, false, s, "moe_stack_forward_decode");
        if (st != MOE_OK) return st;
    }
    // The residual stream alternates between h and h_buf: layer l's stream (after the previous
    // layer's residual add) goes to dst_l = (l odd ? h : h_buf). The residual step before layer
    // l >= 1 runs either inside layer l's router launch (with layer l-1's post-FFN norm, from
    // dst_{l-1} and y) or, for a layer l-1 without one, already in layer l-1's down launch, which
    // writes dst_l and the sums of squares that layer l's router then reads.
    const bool fused = dec_router_glue_fits(layers[0]->dims, T);
    bool formed = false;   // dst_l was formed by the previous down launch
    for (int l = 0; l < n_layers; ++l) {
        moe_layer *L = layers[l];
        L->routed_T = -1;
        L->last_T = T;
        uint16_t *src = (l & 1) ? h_buf : h, *dst = (l & 1) ? h : h_buf;
        const float *yp = l ? y_buf : nullptr;
        // the previous layer's tail goes with its output y into this layer's residual step
        const uint16_t *post = l ? layers[l - 1]->w.post_ffn_norm : nullptr;
        const uint16_t *scalar = l ? layers[l - 1]->w.layer_scalar : nullptr;
        if (formed) {
            RUN(K_DEC_ROUTER, launch_dec_router_norm(L, dst, layers[l - 1]->ws.dss, x_buf, T, s));
        } else if (fused) {
            RUN(K_DEC_ROUTER, launch_dec_router_glue(L, src, yp, post, scalar, dst, x_buf, T, s));
        } else {
            RUN(K_GLUE, launch_glue(src, yp, post, scalar, dst, x_buf, T, d, s));
            const uint16_t *u = x_buf;
            moe_status st = router_input(L, x_buf, T, false, s, &u);
            if (st != MOE_OK) return st;
            RUN(K_DEC_ROUTER, launch_dec_router(L, u, T, L->ws.logits, s, u == x_buf));
        }
        RUN(K_DEC_GATEUP, launch_dec_gateup(L, x_buf, T, s));
        // this layer's residual step in its down launch when it has no post-FFN norm and the
        // next step takes a formed stream (the next router holds x in LDS, or the final step)
        const bool last = l == n_layers - 1;
        formed = fused && !L->w.post_ffn_norm;
        uint16_t *next = last ? h : (((l + 1) & 1) ? h : h_buf);
        RUN(K_DEC_DOWN, launch_dec_down(L, T, y_buf, s, formed ? dst : nullptr, formed ? next : nullptr));
    }
    moe_layer *L = layers[n_layers - 1];
    if (formed) {   // the final stream is in h already: x_buf = its norm
        RUN(K_GLUE, launch_glue(h, nullptr, nullptr, nullptr, h, x_buf, T, d, s));
    } else {   // the last layer's residual add, into h
        uint16_t *src = ((n_layers - 1) & 1) ? h : h_buf;
        RUN(K_GLUE, launch_glue(src, y_buf, L->w.post_ffn_norm, L->w.layer_scalar, h, x_buf, T, d, s));
    }
    if (check) {
        moe_status st = check_finite(check, h, (size_t)T * d, false, s, "moe_stack_forward_decode");
        if (st != MOE_OK) return st;
    }
    return MOE_OK;
}

struct moe_stack_plan {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};

void moe_stack_plan_destroy(moe_stack_plan *plan) {
    if (!plan) return;
    if (plan->exec) (void)hipGraphExecDestroy(plan->exec);
    if (plan->graph) (void)hipGraphDestroy(plan->graph);
    delete plan;
}

moe_status moe_stack_plan_create(moe_layer *const *layers, int32_t n_layers, uint16_t *h, int32_t T,
                                 uint16_t *x_buf, float *y_buf, uint16_t *h_buf, moe_stack_plan **out) {
    clear_error();
    if (!out) return fail(MOE_E_INVALID, "moe_stack_plan_create: out is NULL");
    *out = nullptr;
    if (n_layers < 1 || !layers) return fail(MOE_E_INVALID, "moe_stack_plan_create: no layers");
    if (T == 0) return fail(MOE_E_SHAPE, "moe_stack_plan_create: T = 0 (nothing to record)");
    for (int l = 0; l < n_layers; ++l) {
        const moe_layer *L = layers[l];
        if (!L) return fail(MOE_E_INVALID, "moe_stack_plan_create: layer %d is NULL", l);
        if (L->flags & MOE_FLAG_CHECK_FINITE)
            return fail(MOE_E_INVALID, "moe_stack_plan_create: layer %d has MOE_FLAG_CHECK_FINITE (reads back)", l);
        if (L->prof_on) return fail(MOE_E_INVALID, "moe_stack_plan_create: layer %d has profiling on", l);
    }
    moe_stack_plan *P = new (std::nothrow) moe_stack_plan();
    if (!P) return fail(MOE_E_NOMEM, "moe_stack_plan_create: host allocation failed");
    hipStream_t cs = nullptr;
    hipError_t err = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (err != hipSuccess) {
        delete P;
        return fail(MOE_E_DEVICE, "moe_stack_plan_create: stream: %s", hipGetErrorString(err));
    }
    err = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (err != hipSuccess) {
        (void)hipStreamDestroy(cs);
        delete P;
        return fail(MOE_E_DEVICE, "moe_stack_plan_create: begin capture: %s", hipGetErrorString(err));
    }
    // the same validation and kernels as an ordinary call, recorded instead of run
    const moe_status st = moe_stack_forward_decode(layers, n_layers, h, T, x_buf, y_buf, h_buf, cs);
    char msg[sizeof g_err];
    std::memcpy(msg, g_err, sizeof msg);
    err = hipStreamEndCapture(cs, &P->graph);
    (void)hipStreamDestroy(cs);
    if (st != MOE_OK) {
        moe_stack_plan_destroy(P);
        clear_error();
        return fail(st, "moe_stack_plan_create: %s", msg);
    }
    if (err == hipSuccess) err = hipGraphInstantiate(&P->exec, P->graph, nullptr, nullptr, 0);
    if (err != hipSuccess) {
        moe_stack_plan_destroy(P);
        return fail(MOE_E_DEVICE, "moe_stack_plan_create: capture: %s", hipGetErrorString(err));
    }
    *out = P;
    return MOE_OK;
}

moe_status moe_stack_plan_run(moe_stack_plan *plan, void *hip_stream) {
    clear_error();
    if (!plan) return fail(MOE_E_INVALID, "moe_stack_plan_run: plan is NULL");
    const hipError_t err = hipGraphLaunch(plan->exec, static_cast<hipStream_t>(hip_stream));
    if (err != hipSuccess) return fail(MOE_E_DEVICE, "moe_stack_plan_run: %s", hipGetErrorString(err));
    return MOE_OK;
}

moe_status moe_prefill_route(moe_layer *L, const uint16_t *x, int32_t T, int32_t *expert_counts, void *hip_stream) {
    clear_error();
    moe_status st = check_tokens(L, T, "moe_prefill_route");
    if (st != MOE_OK || T == 0) return st;
    if (!x) return fail(MOE_E_INVALID, "moe_prefill_route: x is NULL");
    if (!aligned16(x)) return fail(MOE_E_ALIGN, "moe_prefill_route: x not 16-byte aligned");
    if (expert_counts && !aligned16(expert_counts))
        return fail(MOE_E_ALIGN, "moe_prefill_route: expert_counts not 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    CHECK_FINITE(x, (size_t)T * L->dims.d_model, false, "moe_prefill_route");
    L->routed_T = T;
    L->last_T = T;
    st = route_impl(L, x, T, s, L->ws.logits, L->ws.idx, L->ws.wts, true, nullptr, true);
    if (st != MOE_OK) return st;
    if (expert_counts) {
        hipError_t err = hipMemcpyAsync(expert_counts, L->ws.counts, sizeof(int32_t) * L->dims.n_experts,
                                        hipMemcpyDeviceToDevice, s);
        if (err != hipSuccess) return fail(MOE_E_DEVICE, "moe_prefill_route: %s", hipGetErrorString(err));
    }
    return MOE_OK;
}

moe_status moe_prefill_tile(moe_layer *L, int32_t T, int32_t tile, void *hip_stream) {
    clear_error();
    moe_status st = check_tokens(L, T, "moe_prefill_tile");
    if (st != MOE_OK) return st;
    if (!L->w.expert_slot) return fail(MOE_E_INVALID, "moe_prefill_tile: the layer has no expert slots");
    if (tile < 0) return fail(MOE_E_INVALID, "moe_prefill_tile: tile = %d is negative", tile);
    if (T == 0) return MOE_OK;
    if (L->routed_T != T)
        return fail(MOE_E_INVALID, "moe_prefill_tile: T = %d is not the routed chunk's (%d; -1: none)", T, L->routed_T);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if ((st = slot_stage_shift(L, s)) != MOE_OK) return st;
    RUN(K_PRE_GATEUP, launch_pre_gateup(L, nullptr, T, s, tile));
    RUN(K_PRE_DOWN, launch_pre_down(L, T, s, tile));
    return MOE_OK;
}

moe_status moe_prefill_combine(moe_layer *L, int32_t T, float *y, void *hip_stream) {
    clear_error();
    moe_status st = check_tokens(L, T, "moe_prefill_combine");
    if (st != MOE_OK || T == 0) return st;
    if (!y) return fail(MOE_E_INVALID, "moe_prefill_combine: y is NULL");
    if (!aligned16(y)) return fail(MOE_E_ALIGN, "moe_prefill_combine: y not 16-byte aligned");
    if (L->routed_T != T)
        return fail(MOE_E_INVALID, "moe_prefill_combine: T = %d is not the routed chunk's (%d; -1: none)", T,
                    L->routed_T);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    RUN(K_COMBINE, launch_combine(L, T, y, s));
    CHECK_FINITE(y, (size_t)T * L->dims.d_model, true, "moe_prefill_combine");
    return MOE_OK;
}

moe_status moe_slot_lookup(moe_layer *L, const int32_t *topk_idx, int32_t T, int32_t *missing, void *hip_stream) {
    clear_error();
    if (!L) return fail(MOE_E_INVALID, "moe_slot_lookup: layer is NULL");
    if (!L->w.expert_slot) return fail(MOE_E_INVALID, "moe_slot_lookup: the layer has no expert slots");
    if (T < 0) return fail(MOE_E_SHAPE, "moe_slot_lookup: T = %d is negative", T);
    if (!missing || (T > 0 && !topk_idx)) return fail(MOE_E_INVALID, "moe_slot_lookup: NULL pointer");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    RUN(K_SLOT_LOOKUP, launch_slot_lookup(L, topk_idx, T, missing, s));
    return MOE_OK;
}

moe_status moe_slot_faults(moe_layer *L, int32_t reset, int32_t *count, void *hip_stream) {
    clear_error();
    if (!L || !count) return fail(MOE_E_INVALID, "moe_slot_faults: NULL argument");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    int32_t v = 0;
    hipError_t err = hipMemcpyAsync(&v, L->ws.slot_faults, sizeof(v), hipMemcpyDeviceToHost, s);
    if (err == hipSuccess) err = hipStreamSynchronize(s);
    if (err == hipSuccess && reset) err = hipMemsetAsync(L->ws.slot_faults, 0, sizeof(int32_t), s);
    if (err != hipSuccess) return fail(MOE_E_DEVICE, "moe_slot_faults: %s", hipGetErrorString(err));
    *count = v;
    return MOE_OK;
}

moe_status moe_profile_enable(moe_layer *L, int32_t on) {
    clear_error();
    if (!L) return fail(MOE_E_INVALID, "layer is NULL");
    L->prof_on = on != 0;
    return MOE_OK;
}

static moe_status prof_drain(moe_layer *L) {
    for (auto &p : L->prof_pending) {
        hipError_t err = hipEventSynchronize(p.b);
        float ms = 0.0f;
        if (err == hipSuccess) err = hipEventElapsedTime(&ms, p.a, p.b);
        if (err != hipSuccess) return fail(MOE_E_DEVICE, "profile events: %s", hipGetErrorString(err));
        L->prof_ms[p.id] += ms;
        L->prof_n[p.id] += 1;
        L->prof_pool.push_back(p.a);
        L->prof_pool.push_back(p.b);
    }
    L->prof_pending.clear();
    return MOE_OK;
}

moe_status moe_profile_read(moe_layer *L, int32_t id, double *total_ms, int64_t *launches) {
    clear_error();
    if (!L || !total_ms || !launches) return fail(MOE_E_INVALID, "NULL argument");
    if (id < 0 || id >= K_COUNT) return fail(MOE_E_INVALID, "kernel id %d out of range", id);
    moe_status st = prof_drain(L);
    if (st != MOE_OK) return st;
    *total_ms = L->prof_ms[id];
    *launches = L->prof_n[id];
    return MOE_OK;
}

moe_status moe_profile_reset(moe_layer *L) {
    clear_error();
    if (!L) return fail(MOE_E_INVALID, "layer is NULL");
    moe_status st = prof_drain(L);
    for (int i = 0; i < K_COUNT; ++i) {
        L->prof_ms[i] = 0.0;
        L->prof_n[i] = 0;
    }
    return st;
}

}  // extern "C"
