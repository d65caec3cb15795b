/*
 * moe.h -- C ABI of the MI355X quantized mixture-of-experts FFN layer.
 *
 * One layer of a Gemma-4-style MoE transformer FFN, as the Mference system
 * design describes it ("Why the runtime has this shape"; "Decode"; "Prefill"):
 *
 *   - an 8-bit group-64 affine router projection gives one logit per routed
 *     expert (no softcap); the top-k logits are kept, largest first, ties going
 *     to the lower expert index, and their softmax gives the routing weights;
 *   - each routed expert is a GELU-gated FFN (gate and up projections, tanh-form
 *     GELU of the gate times up, down projection) with 4-bit group-64 affine
 *     weights: weight = scale * code + bias, one BF16 scale and one BF16 bias
 *     per 64 consecutive input elements;
 *   - a dense shared expert of the same form runs on the same input and is added
 *     without a routing weight;
 *   - the routed outputs are reduced with their routing weights (Mference,
 *     "Decode", cb2 phase) in the fixed slot order 0..k-1, in fp32.
 *
 * All compute runs in gfx950 HIP kernels on the stream the caller passes. Every
 * entry point validates its arguments on the host before enqueuing anything; on
 * error nothing is enqueued, nothing is written, and the handle stays usable.
 * Calls enqueue work and return without waiting for it, with these exceptions, which
 * read device memory back to the host: moe_layer_create (it checks the quantization
 * metadata once and waits for that check), moe_slot_faults, moe_profile_read, and every
 * call on a layer created with MOE_FLAG_CHECK_FINITE (see there).
 *
 * Memory ownership:
 *   - weights are caller-owned device buffers in the device layout moe_repack
 *     produces; the layer borrows them (never copies or writes them) and they
 *     must stay valid and unchanged until moe_layer_destroy;
 *   - the layer owns one workspace, allocated at moe_layer_create for
 *     dims.max_tokens tokens and reused in stream order; calls on one handle must
 *     be issued on one stream, or serialized by the caller, because a queued
 *     kernel owns the workspace until it completes (Mference, "Correctness and
 *     safety invariants");
 *   - activations and outputs are caller-owned device buffers.
 *
 * Device pointers must be 16-byte aligned. Activations are bf16 bit patterns
 * (uint16_t), outputs fp32.
 */
#ifndef QMOE_MOE_H
#define QMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct moe_layer moe_layer; /* opaque handle */

typedef enum {
    MOE_OK = 0,
    MOE_E_INVALID = 1,  /* null required pointer, unknown flag, bad enum value */
    MOE_E_SHAPE = 2,    /* dimension not a multiple of 64, top_k out of range, T < 0 */
    MOE_E_QUANT = 3,    /* group != 64, router bits != 8, expert bits != 4, expert scales or
                           biases the prefill path cannot stage (see moe_layer_create) */
    MOE_E_ALIGN = 4,    /* a device pointer is not 16-byte aligned */
    MOE_E_CAPACITY = 5, /* T above max_tokens (or above MOE_MAX_DECODE_TOKENS for decode) */
    MOE_E_NOMEM = 6,    /* workspace allocation failed, or the workspace exceeds the budget in the flags */
    MOE_E_DEVICE = 7,   /* a HIP call or kernel launch reported an error */
    MOE_E_NONFINITE = 8 /* MOE_FLAG_CHECK_FINITE only: an input or output holds a NaN or infinity */
} moe_status;

/*
 * Flags of moe_layer_create (Mference system design, "Correctness and safety invariants": a
 * step refuses rather than emitting corrupt output).
 *   MOE_FLAG_CHECK_FINITE: debug mode. moe_route, moe_forward_decode, moe_forward_prefill,
 *     moe_prefill_route and moe_stack_forward_decode first count the NaN and infinite values
 *     of their input on the stream and wait for the count; a non-zero count returns
 *     MOE_E_NONFINITE with nothing else enqueued and no output written. The forward calls
 *     (and moe_prefill_combine) then count those of their output y (the stack: of the final
 *     residual stream) and return MOE_E_NONFINITE if there are any; y has then been written.
 *     Without the flag, inputs are assumed finite and nothing is checked or waited for.
 *   MOE_FLAG_WS_BUDGET_MIB(n): the workspace may take at most n MiB (1 <= n < 2^24); a layer
 *     whose workspace would be larger is refused with MOE_E_NOMEM before anything is
 *     allocated. n = 0 (the default) sets no budget.
 * Other bits are MOE_E_INVALID.
 */
#define MOE_FLAG_CHECK_FINITE 0x1u
#define MOE_FLAG_WS_BUDGET_MIB(n) (((uint32_t)(n) & 0xFFFFFFu) << 8)

/* Largest token count moe_forward_decode accepts; larger chunks use moe_forward_prefill. */
#define MOE_MAX_DECODE_TOKENS 16
/* Largest top_k the kernels support. */
#define MOE_MAX_TOP_K 16
/* Largest number of routed experts the kernels support. */
#define MOE_MAX_EXPERTS 1024

/*
 * Formats of the expert matrices (routed and shared; the router is always 8-bit affine):
 *   MOE_FORMAT_AFFINE_G64: weight = scale * code + bias, 4-bit codes, one BF16 scale and one
 *     BF16 bias per 64 consecutive inputs (Mference system design, "Why the runtime has this
 *     shape").
 *   MOE_FORMAT_Q4_0: weight = d * (code - 8), 4-bit codes, one fp16 scale d per 32 consecutive
 *     inputs (Gem native architecture, "M4 Max operating assumptions": 32 weights in an 18-byte
 *     block; "Ownership boundaries": the GGUF loader accepts Q4_0 matrices). Host blocks are
 *     converted with moe_repack_q4_0.
 */
#define MOE_FORMAT_AFFINE_G64 0
#define MOE_FORMAT_Q4_0 1

typedef struct {
    int32_t d_model;     /* model width d; multiple of 64 in [64, 8192] */
    int32_t n_experts;   /* routed experts E, 1..MOE_MAX_EXPERTS */
    int32_t top_k;       /* experts per token k, 1..min(E, MOE_MAX_TOP_K) */
    int32_t d_expert;    /* routed expert width I; multiple of 64 */
    int32_t d_shared;    /* shared expert width I_s; multiple of 64 */
    int32_t group;       /* quantization group; must be 64 */
    int32_t router_bits; /* must be 8 */
    int32_t expert_bits; /* must be 4 */
    int32_t max_tokens;  /* workspace capacity in tokens per call, in [1, 2^20], with the fp16
                            activation buffers (max_tokens top_k max(d, I) and max_tokens I_s
                            values) below 4 GiB and at most 16384 routed row tiles per chunk
                            (ceil(max_tokens top_k / 128) + min(E, max_tokens top_k), the
                            prefill GEMMs' work-list bound); else MOE_E_SHAPE */
    int32_t expert_format; /* MOE_FORMAT_AFFINE_G64 (0) or MOE_FORMAT_Q4_0 (1); other values are
                              MOE_E_QUANT */
} moe_dims;

/*
 * One quantized matrix (or a stack of E of them) in the device layout:
 *   codes: device bytes, layout per moe_repack;
 *   sb:    device uint32 words, one per (row, group of 64 inputs), layout per moe_repack:
 *          affine: (bf16 scale) | (bf16 bias << 16);
 *          Q4_0 expert matrices: (fp16 d of inputs 0..31 of the group) | (fp16 d of inputs
 *          32..63 << 16).
 */
typedef struct {
    const void *codes;
    const uint32_t *sb;
} moe_qmat;

typedef struct {
    moe_qmat router;          /* [E, d] 8-bit */
    moe_qmat gate, up;        /* E x [I, d] 4-bit */
    moe_qmat down;            /* E x [d, I] 4-bit */
    moe_qmat sh_gate, sh_up;  /* [I_s, d] 4-bit */
    moe_qmat sh_down;         /* [d, I_s] 4-bit */
    const float *logit_bias;  /* optional fp32 [E] added to every token's router logits (routing skew); may be NULL */
    /*
     * Optional router prologue and epilogue (Mference system design, "Decode", router listing);
     * NULL leaves the router as above.
     *   router_scale: bf16 [d], 16-byte aligned. The router reads
     *       u = bf16(((x / sqrt(mean(x^2) + 1e-6)) * router_scale) / sqrt(d))
     *     (float64, rounded once) instead of x; the experts still read x.
     *   per_expert_scale: bf16 [E]. Each routing weight is multiplied by the scale of its expert
     *     (the weights then no longer sum to 1).
     */
    const uint16_t *router_scale;
    const uint16_t *per_expert_scale;
    /*
     * Optional layer tail (Mference system design, "Decode", cb2: post-FFN norm, residual add,
     * layer scalar), applied to this layer's output y by the residual step that follows it in
     * a stack (moe_stack_forward_decode); moe_forward_* return y without it. NULL leaves the
     * step out.
     *   post_ffn_norm: bf16 [d], 16-byte aligned: y -> (y / sqrt(mean(y^2) + 1e-6)) * post_ffn_norm
     *   layer_scalar: one bf16 in device memory: h_next = bf16((h + y) * layer_scalar)
     */
    const uint16_t *post_ffn_norm;
    const uint16_t *layer_scalar;
    /*
     * Optional shared-expert gate (Mference system design, "Scope and limitations": the Qwen
     * 3.6 layers carry a gated shared expert): bf16 [d], 16-byte aligned. The shared branch
     * is multiplied by a = 1 / (1 + exp(-(g . x))) per token, the dot product in fp32 over the
     * fp16 copy of x; NULL leaves the branch ungated.
     */
    const uint16_t *shared_gate;
    /*
     * Optional expert slots (Mference system design, "Load and ownership": each layer keeps
     * its routed experts in a slab of slots and a GPU-visible expert-to-slot table, -1 for an
     * absent expert). When expert_slot is non-NULL (device int32 [E]), the routed gate, up and
     * down arrays hold n_slots experts (slot n at n times the per-expert size) and routed
     * expert e is read from slot expert_slot[e]. The caller fills slots and updates the table
     * between calls (moe_slot_cache_* plan which expert goes where); every expert a call
     * selects must be resident when its routed kernels run. A kernel that meets an absent or
     * out-of-range slot reads slot 0 instead, so nothing outside the slab is touched, and
     * records the fault: moe_slot_faults returns the count, and the call's output must then
     * be discarded. The prefill calls check the scale/bias words of the experts in slots (the
     * checks moe_layer_create makes for resident layers) and count an expert they cannot
     * stage as a fault too.
     */
    const int32_t *expert_slot;
    int32_t n_slots;
} moe_weights;

/*
 * Create a layer handle for one MoE FFN layer (Mference system design, "Why the runtime has
 * this shape": 8-bit group-64 affine router, 4-bit group-64 affine experts with BF16 scale and
 * bias; ".gturbo directory": weights are bound in place, incompatible quantization metadata is
 * rejected). Validates dims (MOE_E_QUANT, MOE_E_SHAPE), the weight pointers (MOE_E_INVALID if
 * any required pointer is NULL, MOE_E_ALIGN if not 16-byte aligned) and flags (MOE_FLAG_*,
 * else MOE_E_INVALID), then allocates the workspace for dims->max_tokens tokens on the current
 * HIP device (MOE_E_NOMEM, also when it exceeds the flags' budget).
 *
 * The prefill GEMMs stage each dequantized expert weight as one fp16 value, fp16(2^m (s q + b)),
 * with a power-of-two exponent m per matrix chosen from the matrix's largest |scale| (the
 * accumulated products are scaled back by 2^-m in fp32, exactly), so the staging keeps 11
 * significant bits for scales of any magnitude. At creation the library reads every expert
 * matrix's scale/bias words once and waits for the result: a NaN or infinite scale or bias, a
 * largest |scale| outside [2^-73, 2^56), or a bias with floor(log2 |bias|) >=
 * floor(log2 max |scale|) + 24 in its matrix is MOE_E_QUANT. For Q4_0 experts (weight
 * d (q - 8)) the staged value is fp16(2^m (d q - 8 d)) and only a NaN or infinite d is refused
 * (every finite fp16 d can be staged). Layers with expert slots check the routed experts'
 * words in every prefill call instead (see expert_slot), since the slots are filled later.
 * *out is written only on MOE_OK.
 */
moe_status moe_layer_create(const moe_dims *dims, const moe_weights *w, uint32_t flags,
                            moe_layer **out);

/* Frees the workspace. Waits for the device to finish work that may use it. NULL is a no-op. */
void moe_layer_destroy(moe_layer *layer);

/*
 * Router and grouping only (Mference, "Decode": the router listing, with its prologue
 * and per-expert scale when the layer has them; "Prefill": token/expert pairs grouped by
 * expert). For T tokens x (bf16 [T, d]):
 *   logits     fp32 [T, E]   optional (NULL to skip): router logits (+ logit_bias)
 *   topk_idx   int32 [T, k]  the k selected experts, largest logit first, ties to lower index
 *   topk_w     fp32 [T, k]   softmax of the selected logits (times per_expert_scale if given)
 *   expert_offsets int32 [E+1] optional: offsets[e] = number of pairs routed to experts < e
 *   pair_perm  int32 [T*k]   optional: pair ids p = t*k + slot ordered by (expert, token)
 * expert_offsets and pair_perm must be both given or both NULL.
 * T = 0 is a no-op; T > max_tokens is MOE_E_CAPACITY.
 */
moe_status moe_route(moe_layer *layer, const uint16_t *x, int32_t T, int32_t *topk_idx,
                     float *topk_w, float *logits, int32_t *expert_offsets, int32_t *pair_perm,
                     void *hip_stream);

/*
 * Full layer, decode path (wavefront GEMV kernels; Mference system design, "Decode": router,
 * top-8 IDs and weights, shared branch, routed experts, weighted reduction (cb2); "Metal
 * execution": custom affine INT4/INT8 GEMV kernels for single-token decode), for
 * 1 <= T <= MOE_MAX_DECODE_TOKENS:
 *   y[t] = a[t] * shared(x[t]) + sum_{s<k} w[t,s] * expert_{idx[t,s]}(x[t])      fp32 [T, d]
 * with a[t] the shared-expert gate (1 without shared_gate) and the routing of moe_route
 * (including the router prologue and per-expert scale when the weights carry them). With
 * expert slots every selected expert must be resident (see expert_slot).
 * T = 0 is a no-op; T above MOE_MAX_DECODE_TOKENS or max_tokens is MOE_E_CAPACITY.
 * Range: the experts read x and the hidden activation h = gelu(gate x) * (up x) in fp16 (as
 * moe_forward_prefill does). Values that round above 65504 in magnitude become infinite and a
 * NaN stays NaN, so the output is then non-finite (MOE_FLAG_CHECK_FINITE reports it) rather
 * than silently wrong; magnitudes below 2^-14 are fp16 subnormals and keep fewer significant
 * bits (a layer input normalized to unit rms, and the hidden activations of weights with
 * scales near the usual 2^-9 .. 2^-5, lie well inside the normal range).
 */
moe_status moe_forward_decode(moe_layer *layer, const uint16_t *x, int32_t T, float *y,
                              void *hip_stream);

/*
 * Full layer, prefill path (Mference system design, "Prefill": token/expert pairs grouped by
 * expert and each expert's rows run as one dense product against its dequantized tiles;
 * "Metal execution": matrix units for multi-row prefill): grouped MFMA GEMMs over
 * expert-bucketed rows, for 1 <= T <= max_tokens. Same result definition as
 * moe_forward_decode.
 */
moe_status moe_forward_prefill(moe_layer *layer, const uint16_t *x, int32_t T, float *y,
                               void *hip_stream);

/*
 * moe_forward_decode for callers that cannot allocate (code under HIP stream capture, tight
 * serving loops, harnesses that forbid allocation): the same computation and the same results,
 * without a layer handle. dims and w are as for moe_layer_create (validated the same way;
 * expert slots and flags are not available here); x, T and y as for moe_forward_decode, with
 * 1 <= T <= min(dims->max_tokens, MOE_MAX_DECODE_TOKENS). The call's scratch (logits, top-k,
 * hidden activations and their sums, about 0.4 MiB for 16 tokens of the 2816-wide layer) lives
 * in one static device array of 1 MiB per device that the library holds until the process
 * ends: a call whose scratch would not fit (the widest layers at 16 tokens) returns
 * MOE_E_CAPACITY before enqueuing anything.
 * The entry point allocates nothing (no hipMalloc, hipFree or allocating library routine); on
 * its first call on a device it looks up that device's array (hipGetSymbolAddress). Every
 * call on one device shares that device's array: calls that overlap on one device (on
 * different streams, or from several threads) race and must be serialized by the caller.
 */
moe_status moe_forward_decode_noalloc(const moe_dims *dims, const moe_weights *w, const uint16_t *x, int32_t T,
                                      float *y, void *hip_stream);

/*
 * Routing of the last moe_forward_decode or moe_forward_prefill (or moe_prefill_route) on
 * this layer, as that call's own kernels selected it: copies, in stream order, the top-k
 * expert ids (int32 [T, k]) and routing weights (fp32 [T, k]) of its first T tokens to the
 * device buffers idx and w (Mference system design, "Decode": the router hands eight IDs and
 * eight weights to the expert stage). T must be at most that call's T; MOE_E_INVALID if no
 * such call has run or T is larger. An inspection aid for tests; the forward calls need it
 * not.
 */
moe_status moe_last_routing(moe_layer *layer, int32_t T, int32_t *idx, float *w, void *hip_stream);

/*
 * Residual stream between stacked layers (device, bf16 bit patterns), with the tail of the
 * layer that produced y (Mference system design, "Decode", cb2):
 *   z      = post ? (y / sqrt(mean(y^2) + 1e-6)) * post : y
 *   h_next = bf16((h + z) * scalar)                       (y may be NULL: h_next = h)
 *   x_next = bf16(h_next / sqrt(mean(h_next^2) + 1e-6))   (norm without a learned scale)
 * h, h_next, x_next: [T, d] bf16; y: [T, d] fp32; post: bf16 [d] or NULL (no post-FFN norm);
 * scalar: one bf16 or NULL (1); all device memory. h_next may alias h. d must be a multiple
 * of 8 in [8, 8192] (MOE_E_SHAPE); h, y, h_next, x_next and post 16-byte aligned (MOE_E_ALIGN).
 * Both results are computed in fp64 in that order and rounded once to bf16 (round to nearest
 * even).
 */
moe_status moe_stack_glue(const uint16_t *h, const float *y, const uint16_t *post, const uint16_t *scalar,
                          uint16_t *h_next, uint16_t *x_next, int32_t T, int32_t d, void *hip_stream);

/*
 * A stack of decode layers with the residual stream between them, for
 * 1 <= T <= every layer's decode capacity. h (bf16 [T, d]) is the residual stream on entry
 * and is updated in place; for l = 0 .. n_layers-1 in order:
 *   x = bf16(h / sqrt(mean(h^2) + 1e-6));  y = layer_l(x);
 *   h = bf16((h + post_l(y)) * scalar_l)
 * with post_l, scalar_l the layer's optional post_ffn_norm and layer_scalar (moe_stack_glue's
 * steps around moe_forward_decode; when T * d_model <= 16384 the residual step after a layer
 * without a post-FFN norm runs in that layer's down launch, and after one with it in the next
 * layer's router launch). x_buf, h_buf (bf16 [T, d]) and y_buf (fp32
 * [T, d]) are caller-owned scratch; on return x_buf holds the norm of the final stream (what
 * a next layer would read) and y_buf the last layer's y. All layers must have the same d_model (MOE_E_SHAPE); every layer handle is used on this
 * stream. MOE_E_INVALID for NULL arguments or n_layers < 1, MOE_E_CAPACITY for T above a
 * layer's decode capacity; T = 0 is a no-op.
 */
moe_status moe_stack_forward_decode(moe_layer *const *layers, int32_t n_layers, uint16_t *h, int32_t T,
                                    uint16_t *x_buf, float *y_buf, uint16_t *h_buf, void *hip_stream);

/*
 * A decode stack recorded once, for callers that run the same layers on the same buffers
 * token after token (Mference system design, "Decode": each token runs the layer stack in
 * order). moe_stack_plan_create records exactly the kernels moe_stack_forward_decode(layers,
 * n_layers, h, T, x_buf, y_buf, h_buf) enqueues, with the same arguments, as a HIP graph
 * (captured on a stream of its own; nothing runs); moe_stack_plan_run launches that graph on
 * hip_stream. A run computes what moe_stack_forward_decode computes on the buffers' contents
 * at that point, bit for bit: the caller writes each token's stream into h before a run and
 * reads h, x_buf and y_buf after it. The plan borrows the layers and the buffers: they must
 * stay valid until moe_stack_plan_destroy, and runs on one plan, like calls on its layers,
 * must be ordered on one stream. Create validates its arguments as moe_stack_forward_decode
 * does and returns the same errors, except that T = 0 is MOE_E_SHAPE (nothing to record); it
 * refuses (MOE_E_INVALID) layers created with MOE_FLAG_CHECK_FINITE or with profiling on, whose
 * calls read device memory back, and a NULL out; MOE_E_DEVICE if HIP refuses the capture,
 * MOE_E_NOMEM if the plan cannot be allocated. *out is NULL on error. Run: MOE_E_INVALID for a
 * NULL plan, MOE_E_DEVICE if the launch fails. Destroy accepts NULL.
 */
typedef struct moe_stack_plan moe_stack_plan; /* opaque handle */
moe_status moe_stack_plan_create(moe_layer *const *layers, int32_t n_layers, uint16_t *h, int32_t T,
                                 uint16_t *x_buf, float *y_buf, uint16_t *h_buf, moe_stack_plan **out);
moe_status moe_stack_plan_run(moe_stack_plan *plan, void *hip_stream);
void moe_stack_plan_destroy(moe_stack_plan *plan);

/* ---------------------------------------------------------------- host-side weight layout */

/* Canonical host layout of one matrix or a stack of n_mats matrices [out, in]:
 *   codes  [n_mats, out, in*bits/8] bytes; 4-bit codes two per byte, the lower-indexed
 *          element in the low nibble (eight per little-endian u32); 8-bit one per byte
 *   scales [n_mats, out, in/64] bf16 bits;  biases [n_mats, out, in/64] bf16 bits */
typedef struct {
    const uint8_t *codes;
    const uint16_t *scales;
    const uint16_t *biases;
} moe_host_qmat;

/* Bytes of the device layout: part 0 = codes, part 1 = sb words. 0 on invalid arguments. */
size_t moe_packed_bytes(int32_t bits, int32_t n_mats, int32_t out_dim, int32_t in_dim, int32_t part);

/*
 * Host-to-host lossless repack from the canonical layout to the device layout: codes
 * are moved, never re-quantized (Mference, "Source weights and bounded repack";
 * "Correctness and safety invariants": repack must be exactly invertible).
 *   bits 8 (router): codes stay [n_mats, out, in]; sb is [n_mats, out, in/64].
 *   bits 4 (experts): out must be a multiple of 32. Per matrix, 1 KiB tiles of 32 rows x
 *     64 inputs, ordered (row block, group); inside a tile, 64 lanes x 16 bytes, lane l
 *     holding row (l % 32), inputs 16*s + 8*(l / 32) + j for step s = 0..3 and j = 0..7,
 *     one u32 per step with element j in nibble (j even ? j/2 : 4 + j/2).
 *     sb words ordered (row block, group, row in block).
 * Returns MOE_E_SHAPE / MOE_E_QUANT / MOE_E_INVALID on bad arguments (nothing written).
 */
moe_status moe_repack(int32_t bits, int32_t n_mats, int32_t out_dim, int32_t in_dim,
                      const moe_host_qmat *canonical, void *codes_out, uint32_t *sb_out);

/* Exact inverse of moe_repack (host to host). */
moe_status moe_unrepack(int32_t bits, int32_t n_mats, int32_t out_dim, int32_t in_dim,
                        const void *codes_in, const uint32_t *sb_in, uint8_t *codes,
                        uint16_t *scales, uint16_t *biases);

/*
 * Host-to-host lossless repack of Q4_0 expert matrices (MOE_FORMAT_Q4_0) into the device
 * layout (Mference, "Source weights and bounded repack": a packed sidecar derived
 * reproducibly, codes moved and never re-quantized).
 *   blocks: [n_mats, out, in/32] blocks of 18 bytes: fp16 d (little-endian), then 16 bytes,
 *           byte j holding the code of element j in its low nibble and of element j + 16 in
 *           its high nibble; weight = d * (code - 8).
 *   codes_out: the 4-bit tile layout of moe_repack (moe_packed_bytes(4, ..., 0) bytes), codes
 *           unchanged (0..15); sb_out: one word per (row, group of 64 inputs) in moe_repack's
 *           order, d of the group's first block in the low half, of its second block in the
 *           high half.
 * out must be a multiple of 32 and in a multiple of 64 (MOE_E_SHAPE); NULL pointers are
 * MOE_E_INVALID. Nothing is written on error. Scales are copied as bit patterns; NaN or
 * infinite scales are refused later by moe_layer_create (MOE_E_QUANT).
 */
moe_status moe_repack_q4_0(int32_t n_mats, int32_t out_dim, int32_t in_dim, const uint8_t *blocks,
                           void *codes_out, uint32_t *sb_out);

/* Exact inverse of moe_repack_q4_0 (host to host): device layout back to the 18-byte blocks. */
moe_status moe_unrepack_q4_0(int32_t n_mats, int32_t out_dim, int32_t in_dim, const void *codes_in,
                             const uint32_t *sb_in, uint8_t *blocks);

/* ---------------------------------------------------------------- diagnostics */

const char *moe_status_str(moe_status s);
/* Message of the last failed call on this thread ("" if none). */
const char *moe_last_error(void);

/* Build identity of the library: a hash over the sources it was compiled from (a binding can
 * refuse a library older than its sources). */
const char *moe_build_id(void);

/* ---------------------------------------------------------------- expert slot cache */
/*
 * GPU slot lookup (Mference system design, "Decode": the slot map resolves the router's
 * top-k IDs against the layer's expert-to-slot table on the GPU). topk_idx: device int32
 * [T, k] (as moe_route writes it); missing: device int32 [1 + E]: missing[0] = the number of
 * distinct selected experts without a slot, then those experts in ascending order. Needs a
 * layer created with expert_slot (MOE_E_INVALID otherwise); T = 0 writes a count of 0.
 */
moe_status moe_slot_lookup(moe_layer *layer, const int32_t *topk_idx, int32_t T, int32_t *missing,
                           void *hip_stream);

/*
 * Prefill in expert tiles (Mference system design, "Prefill": a chunk's routed experts are
 * streamed through the slot cache in tiles; each tile's work runs while its experts occupy
 * slots), for layers with expert slots. Three stream-ordered steps on one chunk of T tokens
 * (the layer's workspace holds it between them; no other call on the layer in between):
 *   moe_prefill_route: routing and grouping of the chunk, as moe_forward_prefill starts;
 *     expert_counts (device int32 [E], may be NULL) gets each expert's number of pairs.
 *   moe_prefill_tile: the gate/up and down projections of the routed pairs whose expert has
 *     a slot in the table at that point of the stream (pairs of absent experts are skipped,
 *     not faults), and with tile = 0 also the shared expert. The caller maps each expert of
 *     the chunk in exactly one tile's table.
 *   moe_prefill_combine: y (fp32 [T, d]) from the shared and routed outputs.
 * moe_prefill_tile on a layer without slots is MOE_E_INVALID, and so are moe_prefill_tile and
 * moe_prefill_combine when no chunk has been routed on the layer or T differs from the routed
 * chunk's T. moe_prefill_tile first checks the scale/bias words of the experts its slot table
 * maps (as moe_layer_create does for resident layers); an expert the prefill GEMMs cannot
 * stage counts as a slot fault.
 */
moe_status moe_prefill_route(moe_layer *layer, const uint16_t *x, int32_t T, int32_t *expert_counts,
                             void *hip_stream);
moe_status moe_prefill_tile(moe_layer *layer, int32_t T, int32_t tile, void *hip_stream);
moe_status moe_prefill_combine(moe_layer *layer, int32_t T, float *y, void *hip_stream);

/* Number of absent or out-of-range slots the layer's kernels have met since creation (or
 * the last reset); synchronizes the layer's stream. */
moe_status moe_slot_faults(moe_layer *layer, int32_t reset, int32_t *count, void *hip_stream);

/*
 * Host-side slot planner (Mference system design, "Load and ownership": least-frequently
 * used eviction with recency as the tie-breaker; a hit reuses its slot, a miss takes an
 * evictable slot). Each slot counts the uses of its expert since it was filled and the
 * request of its last use. moe_slot_cache_plan takes one request (the experts one call
 * needs, in any order, duplicates allowed): every listed resident expert is a hit (count + 1,
 * last use = this request); the missing ones, in ascending expert order, take free slots in
 * ascending slot order, then evict, among the residents this request does not list, the one
 * with the lowest count, then the oldest last use, then the lowest slot. A request with more
 * distinct experts than slots is MOE_E_CAPACITY and changes nothing. slot_of (host [n]) gets
 * each listed expert's slot; fill_expert / fill_slot (host, room for n) get the fills the
 * caller must perform before the call runs, n_fill their number.
 */
typedef struct moe_slot_cache moe_slot_cache;
moe_status moe_slot_cache_create(int32_t n_experts, int32_t n_slots, moe_slot_cache **out);
void moe_slot_cache_destroy(moe_slot_cache *cache);
moe_status moe_slot_cache_plan(moe_slot_cache *cache, const int32_t *experts, int32_t n, int32_t *slot_of,
                               int32_t *fill_expert, int32_t *fill_slot, int32_t *n_fill);
/*
 * moe_slot_cache_plan with protected experts (host int32 [n_protect]): those that are resident
 * and not in the request keep their slots (this request evicts none of them) and count no use,
 * so a caller can plan the next tile of a chunk while the current tile's experts still serve
 * queued work (Mference system design, "Prefill"; "Correctness and safety invariants"). The
 * request's distinct experts plus the kept protected ones must fit the slots (MOE_E_CAPACITY
 * otherwise, nothing changed). moe_slot_cache_plan is this call with no protected experts.
 */
moe_status moe_slot_cache_plan_protected(moe_slot_cache *cache, const int32_t *experts, int32_t n,
                                         const int32_t *protect, int32_t n_protect, int32_t *slot_of,
                                         int32_t *fill_expert, int32_t *fill_slot, int32_t *n_fill);
/* The current expert-to-slot table (host int32 [n_experts], -1 for absent experts). */
moe_status moe_slot_cache_table(const moe_slot_cache *cache, int32_t *expert_slot);

/*
 * Per-kernel timing with HIP events attached to each kernel dispatch on the caller's stream
 * (Gem native architecture, "Ownership boundaries": a profiled run must give the same results
 * as the ordinary one). Off by default; it never changes results. moe_profile_read
 * synchronizes the recorded events and returns the summed milliseconds and launch count of
 * kernel id since the last reset. moe_kernel_name(id) is NULL past the last id.
 */
moe_status moe_profile_enable(moe_layer *layer, int32_t on);
moe_status moe_profile_read(moe_layer *layer, int32_t kernel_id, double *total_ms, int64_t *launches);
moe_status moe_profile_reset(moe_layer *layer);
const char *moe_kernel_name(int32_t kernel_id);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_MOE_H */
