// Internal definitions shared by the host runtime and the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <utility>
#include <vector>

#include "moe.h"

namespace qmoe {

// ----------------------------------------------------------------------------- errors
moe_status fail(moe_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
// dims and weight pointers of moe_layer_create (validation only)
moe_status check_layer_args(const moe_dims *D, const moe_weights *w);

// ----------------------------------------------------------------------------- tiling constants
constexpr int kGroup = 64;          // quantization group (inputs per scale/bias)
constexpr int kTileRows = 32;       // rows per 1 KiB weight tile
constexpr int kMT = 128;            // prefill GEMM rows per workgroup tile
constexpr int kChunk = 256;         // pairs per bucketing chunk

// Routed row tiles of a prefill chunk of T tokens: at most ceil(T k / kMT) + min(E, T k)
// (every expert with pairs adds at most one partially filled tile).
inline int max_routed_tiles(int T, int k, int E) {
    const int P = T * k;
    return (P + kMT - 1) / kMT + (E < P ? E : P);
}

__host__ __device__ inline int roundup(int a, int b) { return (a + b - 1) / b * b; }
constexpr int cdiv_c(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Work lists of the prefill GEMM launches. A launch has kXcds * cap workgroups; workgroup b runs
// on XCD b % kXcds and takes item b / kXcds of that XCD's list (the lists are built with the
// grouping, so each XCD gets about the same work: every shared-expert item is dealt on its own,
// routed row tiles whole, class by class from the longest). Output tiles per row tile:
//   shared 128-row tile nts, routed 128-row tile ntr, routed tile of at most 32 rows ntn.
constexpr int kXcds = 8;
constexpr int kTileTabMax = 16384;   // routed row tiles per chunk the list builder holds
struct GemmTiles {
    int nts, ntr, ntn;
};
inline GemmTiles gemm_tiles(const moe_dims &D, int mode) {   // mode 0: gate/up, 1: down
    if (mode == 0) return GemmTiles{cdiv(D.d_shared / 32, 4), cdiv(D.d_expert / 32, 4), cdiv(D.d_expert / 32, 8)};
    return GemmTiles{cdiv(D.d_model / 64, 4), cdiv(D.d_model / 64, 4), cdiv(D.d_model / 32, 16)};
}
// Items per XCD list for a chunk of T tokens. The shared items are dealt one by one (at most
// ceil(S / 8) per XCD) and each of the four routed classes by whole tiles (at most
// ceil(m_c / 8) tiles of n_c items), so a list holds at most worst / 8 + 1 + sum n_c items,
// worst = S + (routed row tiles) ntr >= every chunk's item count (ntn <= ntr).
inline int gemm_list_cap(const moe_dims &D, int T, int mode) {
    const GemmTiles g = gemm_tiles(D, mode);
    const int worst = cdiv(T, kMT) * g.nts + max_routed_tiles(T, D.top_k, D.n_experts) * g.ntr;
    return cdiv(worst, kXcds) + 1 + 3 * g.ntr + g.ntn;
}
// Kind of a work-list item (bits 28.. of its .y)
enum { kItemShared = 0, kItemWide = 1, kItemNarrow = 2 };

// Kernel ids for per-kernel timing.
enum KernelId {
    K_ROUTER = 0,
    K_TOPK,
    K_BUCKET_RANK,
    K_BUCKET_SCAN,
    K_BUCKET_SCATTER,
    K_DEC_ROUTER,
    K_DEC_GATEUP,
    K_DEC_DOWN,
    K_PRE_GATEUP,
    K_PRE_DOWN,
    K_COMBINE,
    K_GLUE,
    K_ROUTER_PROLOGUE,
    K_SLOT_LOOKUP,
    K_COUNT
};

// Device pointers of the layer workspace.
struct Workspace {
    float *logits;        // [maxT, E]
    int32_t *idx;         // [maxT, k]
    float *wts;           // [maxT, k]
    uint16_t *x16;        // [maxT, d]          fp16 copy of x (prefill gate/up operand, written by the router)
    uint16_t *u;          // [maxT, d]          router input after the router prologue (bf16), if the layer has one
    int32_t *counts;      // [E]
    int32_t *offsets;     // [E+1]
    int4 *list[2];        // [kXcds, cap]        GEMM work lists (gate/up, down): item q of XCD x at
                          //                    x cap + q: (expert | nt << 16, row tile | kind << 28,
                          //                    first pair row, pairs of the expert); shared: (nt << 16,
                          //                    row tile, 0, T)
    int32_t *list_n;      // [2, kXcds]          items in each XCD's list
    int32_t *chunk_base;  // [nchunks, E]
    int32_t *rank;        // [maxT*k]
    int32_t *perm;        // [maxT*k]
    int32_t *pos;         // [maxT*k]
    uint16_t *h_r;        // [maxT*k, I]        routed hidden activations, fp16 bits (bucket order)
    uint16_t *h_s;        // [maxT, I_s]        shared hidden activations, fp16 bits
    float *r;             // [maxT*k, d]        routed expert outputs (bucket order)
    float *sh;            // [maxT, d]          shared expert outputs
    float *sgate;         // [maxT]             decode: shared-expert gate values (layers with a gate)
    int32_t *slot_faults; // [1]                absent expert slots the kernels met (layers with slots)
    float *rqf;           // router weights fma(scale, q, bias) as fp32 (prefill router table)
    float *rqm;           // the same weights in the matrix-core router's operand order
    int32_t *flag;        // [1]                layer-creation checks, non-finite counts
    int32_t *shift;       // [3 n_mats + 3]     fp16 staging exponents of the prefill GEMMs: routed
                          //                    gate, up, down (kind * n_mats + matrix), then shared
    // decode path (D = decode capacity, KSd/KSs = input pieces of d / of I_s)
    float *dxg;           // [D, d/64]          decode: group sums of x (Q4_0 experts: [D, d/32] half sums)
    uint16_t *dh_r;       // [D*k, I]           decode: routed hidden activations, fp16 bits
    uint16_t *dh_s;       // [D, I_s]           decode: shared hidden activations, fp16 bits
    float *dhs_r;         // [D*k, I/16]        decode: sums of 16 consecutive routed h values
    float *dhs_s;         // [D, I_s/16]        decode: sums of 16 consecutive shared h values
    double *dss;          // [D, d/16]          decode stack: fp64 sums of squares of 16-row pieces of the
                          //                    stream this layer's down launch formed
};

struct ProfEvent {
    int id;
    hipEvent_t a, b;
};

}  // namespace qmoe

struct moe_layer {
    moe_dims dims;
    moe_weights w;
    int device;
    int G_d, G_I, G_Is;        // groups along d, I, I_s
    int max_dec;               // decode capacity = min(max_tokens, MOE_MAX_DECODE_TOKENS)
    int n_mats;                // routed matrices per kind in the weight arrays (experts, or slots)
    uint32_t flags;            // MOE_FLAG_* of the creation
    int routed_T;              // tokens of the chunk whose routing and grouping the workspace holds (-1: none)
    int last_T;                // tokens of the last call whose top-k ws.idx / ws.wts hold (-1: none)
    void *ws_base;
    size_t ws_bytes;
    qmoe::Workspace ws;
    // profiling
    bool prof_on;
    std::vector<qmoe::ProfEvent> prof_pending;
    std::vector<hipEvent_t> prof_pool;
    double prof_ms[qmoe::K_COUNT];
    int64_t prof_n[qmoe::K_COUNT];
};

namespace qmoe {

// Kernel timing hook. While `stop` is set (per-kernel profiling of one call), launches go
// through hipExtLaunchKernelGGL, which attaches the events to the dispatch itself, so the
// elapsed time is the kernel's execution interval (the same interval a kernel trace reports)
// rather than the gap between two separately queued markers. A launcher issuing several
// kernels records `start` on the first and `stop` on each, so the interval spans all of them.
struct LaunchTiming {
    hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local LaunchTiming g_timing;

template <typename F, typename... Args>
inline void launch(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, Args... args) {
    if (g_timing.stop) {
        hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)lds, s, g_timing.start, g_timing.stop, 0u, args...);
        g_timing.start = nullptr;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
    }
}

// Kernel launchers (each enqueues on stream, returns hipGetLastError()).
hipError_t launch_dec_router(const moe_layer *L, const uint16_t *x, int T, float *logits, hipStream_t s,
                             bool write_aux = true);
// write_aux: the prefill router also writes the fp16 copy of x from its input, the decode router
// the group sums of x; both are off when the router reads the prologue's output instead of x.
hipError_t launch_router(const moe_layer *L, const uint16_t *x, int T, float *logits, hipStream_t s,
                         bool write_aux = true);
// Router prologue: u = bf16(((x / rms(x)) * router_scale) / sqrt(d)) into ws.u, plus the fp16
// copy of x (for_prefill) or the decode group sums of x (otherwise).
hipError_t launch_router_prologue(const moe_layer *L, const uint16_t *x, int T, bool for_prefill, hipStream_t s);
bool dec_router_glue_fits(const moe_dims &D, int T);
// decode router with the router prologue fused (every workgroup forms the router input in LDS;
// needs dec_router_glue_fits); writes the group sums of x itself
hipError_t launch_dec_router_pro(const moe_layer *L, const uint16_t *x, int T, float *logits, hipStream_t s);
hipError_t launch_dec_router_glue(const moe_layer *L, const uint16_t *h_in, const float *y_in,
                                  const uint16_t *post_in, const uint16_t *scalar_in, uint16_t *h_out,
                                  uint16_t *x_out, int T, hipStream_t s);
hipError_t launch_router_table(const moe_layer *L, hipStream_t s);
size_t router_table_floats(const moe_dims &D);
size_t router_mtable_floats(const moe_dims &D);
hipError_t launch_topk(const moe_layer *L, int T, const float *logits, int32_t *idx, float *w, hipStream_t s);
hipError_t launch_bucket_rank(const moe_layer *L, int T, const int32_t *idx, hipStream_t s);
hipError_t launch_bucket_scan(const moe_layer *L, int T, hipStream_t s);
hipError_t launch_bucket_scatter(const moe_layer *L, int T, const int32_t *idx, int32_t *perm, hipStream_t s);
hipError_t launch_dec_gateup(const moe_layer *L, const uint16_t *x, int T, hipStream_t s);
// res_out: also the next layer's residual step of a stack, res_out = bf16((res_h + y) * layer_scalar)
// (a layer without a post-FFN norm), and the fp64 sums of squares of its 16-row pieces into ws.dss
hipError_t launch_dec_down(const moe_layer *L, int T, float *y, hipStream_t s, const uint16_t *res_h = nullptr,
                           uint16_t *res_out = nullptr);
// decode router whose input is x = norm(h_in), h_in formed by the previous layer's down launch
// with its sums of squares ss_in (that layer's ws.dss); workgroup 0 stores x_out. Needs
// dec_router_glue_fits.
hipError_t launch_dec_router_norm(const moe_layer *L, const uint16_t *h_in, const double *ss_in, uint16_t *x_out,
                                  int T, hipStream_t s);
size_t dec_gateup_lds(const moe_dims &D);
size_t dec_down_lds(const moe_dims &D);
size_t dec_workspace_floats(const moe_dims &D, int max_dec, int which);
// fp16 staging exponents of the prefill GEMMs (ws.shift) from the scale/bias words of the
// routed matrices (routed) and of the shared expert (shared). Matrices that cannot be staged
// add to *faults.
hipError_t launch_stage_shift(const moe_layer *L, bool routed, bool shared, int32_t *faults, hipStream_t s);
// *count += the number of NaN / infinite values among n bf16 (f32: fp32) values at p
hipError_t launch_count_nonfinite(const void *p, size_t n, bool f32, int32_t *count, hipStream_t s);
// tile: -1 for a whole chunk; otherwise the index of an expert tile of a chunk (routed items
// whose expert has no slot are skipped; the shared expert runs with tile 0 only)
hipError_t launch_pre_gateup(const moe_layer *L, const uint16_t *x, int T, hipStream_t s, int tile = -1);
hipError_t launch_pre_down(const moe_layer *L, int T, hipStream_t s, int tile = -1);
hipError_t launch_combine(const moe_layer *L, int T, float *y, hipStream_t s);
// GPU slot lookup of the top-k experts (layers with expert slots)
hipError_t launch_slot_lookup(const moe_layer *L, const int32_t *idx, int T, int32_t *missing, hipStream_t s);
hipError_t launch_glue(const uint16_t *h, const float *y, const uint16_t *post, const uint16_t *scalar,
                       uint16_t *h_next, uint16_t *x_next, int T, int d,
                       hipStream_t s);

}  // namespace qmoe
