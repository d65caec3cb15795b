// Decode path (up to 16 tokens): three launches of wavefront GEMV kernels over 4-bit
// group-64 affine weights, with no communication between workgroups of a launch.
//
// Each selected expert is a GELU-gated FFN whose weights are w = scale * q + bias per group
// of 64 inputs (Mference system design, "Why the runtime has this shape"; "Metal
// execution": decode uses custom affine INT4/INT8 GEMV kernels that consume the packed codes
// and BF16 scale/bias directly, and the routed kernels fuse the affine decode, GeGLU and the
// weighted reduction).
//
// Affine split per group (x the 64 inputs of the group):
//   sum_j x_j (s q_j + b) = (2^24 s) * sum_j x_j (q_j 2^-24) + b * sum_j x_j.
// Q4_0 expert matrices (weight d (q - 8), one fp16 d per 32 inputs) split per block the same
// way, with scale d and bias -8 d: the two halves of a group keep their own dot products and
// input sums (the router and the 16-value h sums provide half-group sums instead).
// q 2^-24 is the fp16 subnormal whose mantissa is q, so masking a device-layout word gives
// two of them at once (exact; see nib_sub), and v_dot2_f32_f16 forms x_j q_j 2^-24 with fp32
// accumulation. The inputs enter as fp16: h is fp16; x is converted when it is staged, which
// is exact for |x| in fp16's normal range (a layer input normalized to unit rms has
// |x| <= sqrt(d)). The group sums of the inputs are formed once (x: by the router, from the
// bf16 x in its fixed order; h: from 16-value sums the gate/up units write) and enter once
// per (row, group).
//
// A decode launch moves a few MB of weights; one compute unit streams only some tens of
// GB/s, so the work of every launch is cut into units of 16 weight rows (half of a 1 KiB
// 32-row tile) and spread over all compute units. One 16-byte load per lane then covers two
// input groups: lane l takes row l % 16, input half (l / 16) % 2 and group (l / 32) of the
// pair; the four lanes of a row are added with two cross-lane steps.
//
// Launch A (k_dec_router): router logits in the fixed fp32 order the oracle uses (one wave
//   per expert, one lane per input group), and the group sums of x.
// Launch B (k_dec_gateup): one workgroup per (token, routed slot, 16 rows of I) and per
//   (token, 16 rows of I_s): h = fp16(gelu(gate x) * (up x)) over the whole input. A routed
//   unit first derives its token's top-k from the logits (each wave, DPP argmax); shared
//   units do not depend on routing and stream meanwhile (Mference "Decode" likewise starts
//   the shared branch before the routed one).
// Launch C (k_dec_down): one workgroup per (token, 16 output rows): one wave per routed slot
//   (down projection of that slot's h) and a few waves for the shared down projection, then
//   y = shared + w_0 r_0 + ... + w_{k-1} r_{k-1} in slot order (Mference "Decode", cb2;
//   TinyTitan architecture "Invariants": fixed reduction order).
// In a layer stack the residual step between layers (Mference "Decode", cb2) runs in launch A
// of the next layer (from h and y), or, after a layer without a post-FFN norm, already in
// launch C: each workgroup forms its 16 rows of the next stream, bf16((h + y) * scalar), and
// their fp64 sum of squares, and the next layer's launch A normalizes that stream.
#include "device_common.h"
#include "moe_internal.h"

namespace qmoe {
namespace {

constexpr int kRW = 4;      // router experts (waves) per workgroup
constexpr int kBW = 4;      // waves per gate/up workgroup
constexpr int kMPB = 6;     // group pairs a gate/up wave loads before computing
constexpr int kMPC = 6;     // group pairs a down wave loads before computing
constexpr int kXC = 4;      // 16-byte x chunks per gate/up thread: d <= 64 kBW * 8 * kXC
constexpr size_t kGlueLdsMax = 32768;   // bf16 bytes of x the fused residual step keeps in LDS

// ----------------------------------------------------------------------------- router
// The wave's expert e; lane g handles input group g (and g + 64, ... for d > 4096).
// A[t][g] into Ps, then lanes t < T sum over g in ascending order. Fixed fp32 order:
//   w_j = fma(s, q_j, b); A = fma chain of x_j w_j, ascending j; L = ((0 + A_0) + A_1) + ...
// The group sums X = ((0 + x_0) + x_1) + ... go to xg_out when it is given (the gate/up
// units' bias terms use them; they are not part of the logits); with halves = 2 (Q4_0
// experts) the sums of the group's two halves of 32, each in the same order.
// The 64 codes and the scale/bias word of expert e's input group g.
struct RouterCodes {
    u32x4_t c[4];
    uint32_t sbw;
};
__device__ __forceinline__ RouterCodes router_codes(const uint8_t *__restrict__ rq, const uint32_t *__restrict__ rsb,
                                                    int d, int e, int g) {
    RouterCodes r;
    const u32x4_t *cp = reinterpret_cast<const u32x4_t *>(rq + (size_t)e * d + 64 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) r.c[i] = cp[i];
    r.sbw = rsb[(size_t)e * (d / 64) + g];
    return r;
}

// pre: the codes of group `lane` when the caller loaded them ahead (or null)
__device__ __forceinline__ void router_wave(const uint16_t *__restrict__ x, int T, int d, int e, const uint8_t *__restrict__ rq,
                            const uint32_t *__restrict__ rsb, float *Ps, float *xg_out, const RouterCodes *pre,
                            int halves) {
#pragma clang fp contract(off)
    const int G = d / 64, lane = threadIdx.x & 63;
    for (int g = lane; g < G; g += 64) {
        const RouterCodes rc = (pre && g == lane) ? *pre : router_codes(rq, rsb, d, e, g);
        const u32x4_t c0 = rc.c[0], c1 = rc.c[1], c2 = rc.c[2], c3 = rc.c[3];
        const uint32_t cw[16] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3],
                                 c2[0], c2[1], c2[2], c2[3], c3[0], c3[1], c3[2], c3[3]};
        const uint32_t sbw = rc.sbw;
        const float sc = bf16_to_f32(sbw & 0xFFFFu), bi = bf16_to_f32(sbw >> 16);
        for (int t = 0; t < T; ++t) {
            const u32x4_t *xp = reinterpret_cast<const u32x4_t *>(x + (size_t)t * d + 64 * g);
            u32x4_t xv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[i] = xp[i];
            float X = 0.0f, X0 = 0.0f, A = 0.0f;
#pragma unroll
            for (int j2 = 0; j2 < 32; ++j2) {          // element pair (2 j2, 2 j2 + 1)
                if (j2 == 16 && halves == 2) {   // the first half's sum is complete
                    X0 = X;
                    X = 0.0f;
                }
                const uint32_t xw = xv[j2 >> 2][j2 & 3];
                const float xa = bf16_to_f32(xw & 0xFFFFu), xb = bf16_to_f32(xw >> 16);
                const uint32_t c = cw[j2 >> 1];
                const int sh = (j2 & 1) * 16;
                const float qa = (float)((c >> sh) & 0xFFu), qb = (float)((c >> (sh + 8)) & 0xFFu);
                X = X + xa;
                X = X + xb;
                A = __builtin_fmaf(xa, __builtin_fmaf(sc, qa, bi), A);
                A = __builtin_fmaf(xb, __builtin_fmaf(sc, qb, bi), A);
            }
            Ps[t * G + g] = A;
            if (xg_out && halves == 2) {
                xg_out[(size_t)t * 2 * G + 2 * g] = X0;
                xg_out[(size_t)t * 2 * G + 2 * g + 1] = X;
            } else if (xg_out) {
                xg_out[t * G + g] = X;
            }
        }
    }
}

// ----------------------------------------------------------------------------- top-k
// Slot `slot` of a token's top-k, derived by one wave from its logits row (identical on
// every lane and every wave): each round takes the largest remaining logit, ties to the
// lowest expert index (the lowest lane of the lowest 64-expert block holding the maximum).
// If no remaining logit equals the maximum (only NaNs remain), the lowest remaining index
// is taken. With all_rounds, runs all k rounds and returns the slot's softmax weight over
// the k selected logits (fp32) in w_out.
template <int kPer>   // logits per lane: E <= 64 * kPer
__device__ __forceinline__ int wave_topk(const float *__restrict__ l, int E, int k, int slot, bool all_rounds,
                                         float &w_out) {
    const int lane = threadIdx.x & 63;
    float v[kPer];
    bool live[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        live[i] = e < E;
        v[i] = live[i] ? l[e] : 0.0f;
    }
    const int rounds = all_rounds ? k : slot + 1;
    int target_e = 0;
    float target_v = 0.0f, m = 0.0f, z = 0.0f;
    for (int s = 0; s < rounds; ++s) {
        float lb = -INFINITY;
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if (live[i]) lb = fmaxf(lb, v[i]);
        const float mx = wave_max(lb);
        int e = -1;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const uint64_t bal = __ballot(live[i] && v[i] == mx);
            if (e < 0 && bal) e = 64 * i + __ffsll((long long)bal) - 1;
        }
        if (e < 0) {
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const uint64_t bal = __ballot(live[i]);
                if (e < 0 && bal) e = 64 * i + __ffsll((long long)bal) - 1;
            }
        }
        e = max(e, 0);
        float val = 0.0f;
#pragma unroll
        for (int i = 0; i < kPer; ++i)
            if ((e >> 6) == i) {
                val = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[i]), e & 63));
                if (lane == (e & 63)) live[i] = false;
            }
        if (s == 0) m = val;
        z += __expf(val - m);
        if (s == slot) {
            target_e = min(e, E - 1);
            target_v = val;
        }
    }
    w_out = __expf(target_v - m) / z;
    return target_e;
}

// ----------------------------------------------------------------------------- 16-row units
// Lane roles for 16 rows (block hb of the 32-row tile rb): row l % 16, input half (l/16) % 2,
// group 2p + l/32 of pair p.
struct Lane16 {
    int row, khalf, gsel;
};
__device__ __forceinline__ Lane16 lane16() {
    const int l = threadIdx.x & 63;
    return Lane16{l & 15, (l >> 4) & 1, l >> 5};
}
// Within the tiles of row block rb (starting at W + rb * G * 1024, scale/bias words at
// S + rb * G * 32), this lane's 16 bytes of group g sit at g * 1024 + code_lane(hb) and its
// scale/bias word at index g * 32 + sb_lane(hb).
__device__ __forceinline__ uint32_t code_lane(int hb, const Lane16 &L) { return (32 * L.khalf + 16 * hb + L.row) * 16; }
__device__ __forceinline__ uint32_t sb_lane(int hb, const Lane16 &L) { return 16 * hb + L.row; }
// sum of the four lanes holding one row (lanes l, l^16, l^32, l^48); result in lanes 0..15
__device__ __forceinline__ float row_sum16(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

// Gate and up sums of 16 rows over the group pairs p = p0, p0 + PS, ... (< cdiv(G, 2)), MP
// pairs per batch. load(i0) issues one batch (unconditionally: pairs past the input re-read
// a valid group and are masked later), so a caller can put the first batch in flight before
// it stages the input; compute(i0) consumes it with x (fp16) and its group sums Xs in LDS.
template <int MP, bool Q4>
struct GateUp16 {
    const uint8_t *Wg, *Wu;
    const uint32_t *Sg, *Su;
    int G, p0, PS;
    uint32_t co, so;
    int gsel, khalf;
    u32x4_t wg[MP], wu[MP];
    uint32_t sg[MP], su[MP];

    __device__ __forceinline__ GateUp16(const uint8_t *wg_, const uint8_t *wu_, const uint32_t *sg_, const uint32_t *su_,
                                        int rb, int hb, int G_, int p0_, int PS_) {
        const Lane16 L = lane16();
        Wg = wg_ + (size_t)rb * G_ * 1024;
        Wu = wu_ + (size_t)rb * G_ * 1024;
        Sg = sg_ + (size_t)rb * G_ * 32;
        Su = su_ + (size_t)rb * G_ * 32;
        G = G_;
        p0 = p0_;
        PS = PS_;
        co = code_lane(hb, L);
        so = sb_lane(hb, L);
        gsel = L.gsel;
        khalf = L.khalf;
    }
    __device__ __forceinline__ bool more(int i0) const { return p0 + PS * i0 < cdiv(G, 2); }
    __device__ __forceinline__ void load(int i0) {
#pragma unroll
        for (int i = 0; i < MP; ++i) {
            const int g = min(2 * (p0 + PS * (i0 + i)) + gsel, G - 1);
            wg[i] = ld16_nt(Wg + ((uint32_t)g * 1024 + co));
            wu[i] = ld16_nt(Wu + ((uint32_t)g * 1024 + co));
            sg[i] = Sg[(uint32_t)g * 32 + so];
            su[i] = Su[(uint32_t)g * 32 + so];
        }
    }
    // Xs: the group sums of x (Q4_0: half-group sums, two per group)
    __device__ __forceinline__ void compute(int i0, const uint16_t *xs, const float *Xs, float &accg, float &accu) const {
#pragma unroll
        for (int i = 0; i < MP; ++i) {
            const int g = 2 * (p0 + PS * (i0 + i)) + gsel;
            const int gc = min(g, G - 1);
            // pairs 0 and 2 of a word carry q 2^-24, pairs 1 and 3 carry 16 q 2^-24; [h]: K-steps
            // 2 h, 2 h + 1 (inputs 32 h .. 32 h + 31 of the group)
            float ag0[2] = {0.0f, 0.0f}, ag1[2] = {0.0f, 0.0f}, au0[2] = {0.0f, 0.0f}, au1[2] = {0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int h = Q4 ? s >> 1 : 0;
                const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(xs + 64 * gc + 16 * s + 8 * khalf);
                const u32x4_t pg = nib_sub(wg[i][s]), pu = nib_sub(wu[i][s]);
                ag0[h] = dot2_f16(xv[0], pg[0], ag0[h]);
                ag1[h] = dot2_f16(xv[1], pg[1], ag1[h]);
                au0[h] = dot2_f16(xv[0], pu[0], au0[h]);
                au1[h] = dot2_f16(xv[1], pu[1], au1[h]);
                ag0[h] = dot2_f16(xv[2], pg[2], ag0[h]);
                ag1[h] = dot2_f16(xv[3], pg[3], ag1[h]);
                au0[h] = dot2_f16(xv[2], pu[2], au0[h]);
                au1[h] = dot2_f16(xv[3], pu[3], au1[h]);
            }
            const float on = g < G ? 1.0f : 0.0f;
            const float first = khalf == 0 ? 1.0f : 0.0f;   // the input-sum terms once per (row, group)
            if constexpr (Q4) {
                // d (2^24 A - 8 X) per block, A = sum x q 2^-24 over the block, X its input sum
                const float X0 = Xs[2 * gc] * first, X1 = Xs[2 * gc + 1] * first;
                const float g0 = fmaf(16777216.0f, fmaf(ag1[0], 0.0625f, ag0[0]), -8.0f * X0);
                const float g1 = fmaf(16777216.0f, fmaf(ag1[1], 0.0625f, ag0[1]), -8.0f * X1);
                const float u0 = fmaf(16777216.0f, fmaf(au1[0], 0.0625f, au0[0]), -8.0f * X0);
                const float u1 = fmaf(16777216.0f, fmaf(au1[1], 0.0625f, au0[1]), -8.0f * X1);
                accg = fmaf(on, fmaf(f16_to_f32(sg[i] & 0xFFFFu), g0, f16_to_f32(sg[i] >> 16) * g1), accg);
                accu = fmaf(on, fmaf(f16_to_f32(su[i] & 0xFFFFu), u0, f16_to_f32(su[i] >> 16) * u1), accu);
            } else {
                const float ag = fmaf(ag1[0], 0.0625f, ag0[0]), au = fmaf(au1[0], 0.0625f, au0[0]);
                const float X = Xs[gc] * first;
                const float s24g = 16777216.0f * bf16_to_f32(sg[i] & 0xFFFFu);
                const float s24u = 16777216.0f * bf16_to_f32(su[i] & 0xFFFFu);
                accg = fmaf(on, fmaf(s24g, ag, bf16_to_f32(sg[i] >> 16) * X), accg);
                accu = fmaf(on, fmaf(s24u, au, bf16_to_f32(su[i] >> 16) * X), accu);
            }
        }
    }
};

// Down sum of 16 rows over group pairs p = p0, p0 + PS, ... of an fp16 input h (LDS, with its
// group sums Hs), MP pairs per batch; load / compute as in GateUp16.
template <int MP, bool Q4>
struct Down16 {
    const uint8_t *W;
    const uint32_t *S;
    int G, p0, PS;
    uint32_t co, so;
    int gsel, khalf;
    u32x4_t w[MP];
    uint32_t sb[MP];

    __device__ __forceinline__ Down16(const uint8_t *w_, const uint32_t *s_, int rb, int hb, int G_, int p0_, int PS_) {
        const Lane16 L = lane16();
        W = w_ + (size_t)rb * G_ * 1024;
        S = s_ + (size_t)rb * G_ * 32;
        G = G_;
        p0 = p0_;
        PS = PS_;
        co = code_lane(hb, L);
        so = sb_lane(hb, L);
        gsel = L.gsel;
        khalf = L.khalf;
    }
    __device__ __forceinline__ bool more(int i0) const { return p0 + PS * i0 < cdiv(G, 2); }
    __device__ __forceinline__ void load(int i0) {
#pragma unroll
        for (int i = 0; i < MP; ++i) {
            const int g = min(2 * (p0 + PS * (i0 + i)) + gsel, G - 1);
            w[i] = ld16_nt(W + ((uint32_t)g * 1024 + co));
            sb[i] = S[(uint32_t)g * 32 + so];
        }
    }
    __device__ __forceinline__ float compute(int i0, const uint16_t *hl, const float *Hs) const {
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < MP; ++i) {
            // keeps the LDS reads of pair i after the arithmetic of pair i - 1 (register use)
            asm volatile("" ::: "memory");
            const int g = 2 * (p0 + PS * (i0 + i)) + gsel;
            const int gc = min(g, G - 1);
            float a0[2] = {0.0f, 0.0f}, a1[2] = {0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int h = Q4 ? s >> 1 : 0;
                const u32x4_t hv = *reinterpret_cast<const u32x4_t *>(hl + 64 * gc + 16 * s + 8 * khalf);
                const u32x4_t p = nib_sub(w[i][s]);
                a0[h] = dot2_f16(hv[0], p[0], a0[h]);
                a1[h] = dot2_f16(hv[1], p[1], a1[h]);
                a0[h] = dot2_f16(hv[2], p[2], a0[h]);
                a1[h] = dot2_f16(hv[3], p[3], a1[h]);
            }
            const float on = g < G ? 1.0f : 0.0f;
            const float first = khalf == 0 ? 1.0f : 0.0f;
            if constexpr (Q4) {   // Hs: half-group sums of h
                const float r0 = fmaf(16777216.0f, fmaf(a1[0], 0.0625f, a0[0]), -8.0f * (Hs[2 * gc] * first));
                const float r1 = fmaf(16777216.0f, fmaf(a1[1], 0.0625f, a0[1]), -8.0f * (Hs[2 * gc + 1] * first));
                acc = fmaf(on, fmaf(f16_to_f32(sb[i] & 0xFFFFu), r0, f16_to_f32(sb[i] >> 16) * r1), acc);
            } else {
                const float H = Hs[gc] * first;
                const float s24 = 16777216.0f * bf16_to_f32(sb[i] & 0xFFFFu);
                acc = fmaf(on, fmaf(s24, fmaf(a1[0], 0.0625f, a0[0]), bf16_to_f32(sb[i] >> 16) * H), acc);
            }
        }
        return acc;
    }
};

struct DecArgs {
    const uint16_t *x;
    int T, d, E, k, I, Is;
    const uint8_t *rq;
    const uint32_t *rsb;
    const float *logit_bias;
    const uint16_t *pes;    // [E]              optional per-expert scale of the routing weights (bf16)
    float *logits;
    int32_t *idx;
    float *wts;
    moe_qmat gate, up, down, sh_gate, sh_up, sh_down;
    float *xg;              // [T][d/64]        group sums of x (router, fixed order); Q4_0: [T][d/32] half sums
    int q4_0;               // expert matrices in Q4_0 (1) or affine (0)
    uint16_t *h_r;          // [T*k][I]         routed hidden activations (fp16 bits)
    uint16_t *h_s;          // [T][I_s]         shared hidden activations (fp16 bits)
    float *hs_r;            // [T*k][I/16]      sums of 16 consecutive routed h values
    float *hs_s;            // [T][I_s/16]      sums of 16 consecutive shared h values
    float *y;
    // fused residual step of a layer stack (router launch only): h_in, y_in (null before the
    // first layer) with the previous layer's tail post_in, scalar_in (optional) -> h_out
    // (written by workgroup 0) and x (written by workgroup 0 to x_out, and kept in LDS by
    // every workgroup for its own router waves)
    const uint16_t *h_in;
    const float *y_in;
    const uint16_t *post_in, *scalar_in;
    uint16_t *h_out, *x_out;
    const double *ss_in;    // [T][d/16] router launch with the stream formed by the previous down launch:
                            // fp64 sums of squares of its 16-row pieces (h_in is that stream)
    // the next layer's residual step in the down launch: res_out = bf16((res_h + y) * res_scalar)
    // (res_scalar optional) and the fp64 sums of squares of its 16-row pieces into res_ss
    const uint16_t *res_h, *res_scalar;
    uint16_t *res_out;
    double *res_ss;
    // router prologue fused into the router launch: router_scale (bf16 [d])
    const uint16_t *router_scale;
    // shared-expert gate: g (bf16 [d]) and the per-token gate values (gate/up -> down)
    const uint16_t *shared_gate;
    float *sgate;
    // expert slots (null: routed expert e is matrix e of the routed arrays)
    const int32_t *eslot;
    int n_slots;
    int32_t *slot_faults;
};

// x = bf16(h / sqrt(mean(h^2) + 1e-6)) of one token (one full workgroup), h the stream a down
// launch formed together with the fp64 sums of squares of its 16-row pieces (ssp, d / 16 of
// them): the sums are added per thread and then over the workgroup in a fixed order, and
// inv and x follow glue_token's expressions.
__device__ __forceinline__ void norm_token(const uint16_t *h, const double *ssp, uint16_t *x_next, int d, double *red) {
    const int tid = threadIdx.x, nc = d / 8, np = d / 16;
    u32x4_t hv[kGlueChunks];
#pragma unroll
    for (int c = 0; c < kGlueChunks; ++c) {
        const int i = tid + kGlueWG * c;
        if (i < nc) hv[c] = ld16(h + 8 * i);
    }
    double ss = 0.0;
    for (int i = tid; i < np; i += kGlueWG) ss += ssp[i];
    const double inv = 1.0 / sqrt(glue_block_sum(ss, red) / (double)d + 1e-6);
#pragma unroll
    for (int c = 0; c < kGlueChunks; ++c) {
        const int i = tid + kGlueWG * c;
        if (i < nc) {
            u32x4_t xo;
#pragma unroll
            for (int j2 = 0; j2 < 4; ++j2)
                xo[j2] = f64_to_bf16(bf16_to_f64(hv[c][j2] & 0xFFFFu) * inv) |
                         (f64_to_bf16(bf16_to_f64(hv[c][j2] >> 16) * inv) << 16);
            *reinterpret_cast<u32x4_t *>(x_next + 8 * i) = xo;
        }
    }
}

// ----------------------------------------------------------------------------- launch A
// grid: ceil(E / kRW); block 64 * kRW; LDS kRW * T * (d/64) floats, plus (GLUE or PRO) T * d
// bf16 and 4 doubles. With GLUE == 2 every workgroup forms x = norm(h_in) from the stream the
// previous layer's down launch formed, with that launch's sums of squares (ss_in; workgroup 0
// stores x_out). With GLUE == 1 every workgroup first forms x = norm(bf16(h_in + y_in)) for its
// own use (the same fp64 residual step as the stack glue kernel; workgroup 0 also stores h_out
// and x_out for the later launches), so the stack needs no separate residual launch. With PRO
// every workgroup applies the router prologue to its copy of x (workgroup 0 first stores the
// group sums of x itself for the gate/up launch), so the router reads the prologue's output.
template <int GLUE, bool PRO>
__global__ __launch_bounds__(64 * kRW) void k_dec_router(DecArgs a) {
    static_assert(64 * kRW == kGlueWG, "the residual step runs on one full workgroup");
    extern __shared__ __align__(16) unsigned char smem[];
    const int G = a.d / 64;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    float *Ps = reinterpret_cast<float *>(smem);     // [kRW][T][G]
    const uint16_t *x = a.x;
    const int e = blockIdx.x * kRW + wave;
    // with the residual step in front, the codes of the wave's first group are requested
    // before it, so their latency overlaps the step's own loads
    constexpr bool LDSX = GLUE != 0 || PRO;   // x (then u) kept in LDS
    RouterCodes pre;
    if (LDSX && e < a.E) pre = router_codes(a.rq, a.rsb, a.d, e, min(lane, G - 1));
    if (LDSX) {
        uint16_t *xs = reinterpret_cast<uint16_t *>(smem + sizeof(float) * kRW * a.T * G);
        double *red = reinterpret_cast<double *>(xs + (size_t)a.T * a.d);
        if (GLUE == 2) {
            for (int t = 0; t < a.T; ++t)
                norm_token(a.h_in + (size_t)t * a.d, a.ss_in + (size_t)t * (a.d / 16), xs + (size_t)t * a.d, a.d, red);
            __syncthreads();
            if (blockIdx.x == 0)
                for (int i = tid; i < a.T * a.d / 8; i += 64 * kRW)
                    *reinterpret_cast<u32x4_t *>(a.x_out + 8 * i) = *reinterpret_cast<const u32x4_t *>(xs + 8 * i);
        } else if (GLUE == 1) {
            for (int t = 0; t < a.T; ++t)
                glue_token(a.h_in + (size_t)t * a.d, a.y_in ? a.y_in + (size_t)t * a.d : nullptr, a.post_in,
                           a.scalar_in, blockIdx.x == 0 ? a.h_out + (size_t)t * a.d : nullptr, xs + (size_t)t * a.d, a.d, red);
            __syncthreads();
            if (blockIdx.x == 0)
                for (int i = tid; i < a.T * a.d / 8; i += 64 * kRW)
                    *reinterpret_cast<u32x4_t *>(a.x_out + 8 * i) = *reinterpret_cast<const u32x4_t *>(xs + 8 * i);
        } else {
            for (int i = tid; i < a.T * a.d / 8; i += 64 * kRW)
                *reinterpret_cast<u32x4_t *>(xs + 8 * i) = ld16(a.x + 8 * i);
        }
        if (PRO) {
            __syncthreads();
            const int NX = a.q4_0 ? 2 * G : G, NL = 64 * G / NX;   // sums per token, inputs per sum
            if (blockIdx.x == 0 && tid < NX) {   // X = ((0 + x_0) + x_1) + ... over NL inputs, fp32
#pragma clang fp contract(off)
                for (int t = 0; t < a.T; ++t) {
                    float X = 0.0f;
                    for (int j = 0; j < NL; ++j) X = X + bf16_to_f32(xs[(size_t)t * a.d + NL * tid + j]);
                    a.xg[(size_t)t * NX + tid] = X;
                }
            }
            __syncthreads();   // x_out and the group sums are read from xs before it is rewritten
            for (int t = 0; t < a.T; ++t) prologue_token(xs + (size_t)t * a.d, a.router_scale, a.d, red);
        }
        __syncthreads();
        x = xs;
    }
    float *P = Ps + (size_t)wave * a.T * G;
    if (e < a.E)
        router_wave(x, a.T, a.d, e, a.rq, a.rsb, P, (!PRO && e == 0) ? a.xg : nullptr, LDSX ? &pre : nullptr,
                    a.q4_0 ? 2 : 1);
    __syncthreads();
    if (e < a.E && lane < a.T) {
#pragma clang fp contract(off)
        float L = 0.0f;
        for (int g = 0; g < G; ++g) L = L + P[lane * G + g];
        if (a.logit_bias) L = L + a.logit_bias[e];
        a.logits[(size_t)lane * a.E + e] = L;
    }
}

// ----------------------------------------------------------------------------- launch B
// grid: T * k * (I / 16) routed units, then T * (I_s / 16) shared units; block 64 * kBW.
// LDS: x [d fp16] | Xs [NX floats] | red [kBW][2][16], NX = d/64 group sums (Q4_0: d/32 half sums)
template <int kPer, bool Q4>
__global__ __launch_bounds__(64 * kBW) void k_dec_gateup(DecArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int G = a.d / 64, NX = Q4 ? 2 * G : G;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    uint16_t *xs = reinterpret_cast<uint16_t *>(smem);
    float *Xs = reinterpret_cast<float *>(smem + sizeof(uint16_t) * a.d);
    float(*red)[2][16] = reinterpret_cast<float(*)[2][16]>(smem + sizeof(uint16_t) * a.d + sizeof(float) * NX);
    const int JBr = a.I / 16, JBs = a.Is / 16;
    const int nR = a.T * a.k * JBr;
    const bool routed = (int)blockIdx.x < nR;
    int t, jb, pr = 0;
    if (routed) {
        jb = blockIdx.x % JBr;
        pr = blockIdx.x / JBr;
        t = pr / a.k;
    } else {
        const int u = blockIdx.x - nR;
        jb = u % JBs;
        t = u / JBs;
    }
    // the token's x and group sums, fetched before any selection
    const uint16_t *xrow = a.x + (size_t)t * a.d;
    u32x4_t xv[kXC];
#pragma unroll
    for (int c = 0; c < kXC; ++c) xv[c] = ld16(xrow + 8 * min(tid + 64 * kBW * c, a.d / 8 - 1));
    const float xgv = a.xg[(size_t)t * NX + min(tid, NX - 1)];   // NX <= 256 threads

    const moe_qmat *mg = &a.sh_gate, *mu = &a.sh_up;
    size_t cbase = 0, sbase = 0;
    if (routed) {
        // every wave derives the token's selection itself; one unit of the pair records it
        const int slot = pr % a.k;
        const bool record = (jb == 0 && wave == 0);
        float wsel;
        const int e = __builtin_amdgcn_readfirstlane(wave_topk<kPer>(a.logits + (size_t)t * a.E, a.E, a.k, slot, record, wsel));
        if (record && lane == 0) {
            a.idx[pr] = e;
            a.wts[pr] = a.pes ? wsel * bf16_to_f32(a.pes[e]) : wsel;   // router epilogue
        }
        mg = &a.gate;
        mu = &a.up;
        const int es = __builtin_amdgcn_readfirstlane(
            expert_slot_of(a.eslot, a.n_slots, a.slot_faults, e, record && lane == 0));
        cbase = (size_t)es * a.I * a.d / 2;
        sbase = (size_t)es * a.I * G;
    }
    // the first batch of weights goes out before x is staged
    GateUp16<kMPB, Q4> gu(static_cast<const uint8_t *>(mg->codes) + cbase, static_cast<const uint8_t *>(mu->codes) + cbase,
                      mg->sb + sbase, mu->sb + sbase, jb >> 1, jb & 1, G, wave, kBW);
    gu.load(0);
#pragma unroll
    for (int c = 0; c < kXC; ++c) {
        const int i = tid + 64 * kBW * c;
        if (i < a.d / 8) *reinterpret_cast<u32x4_t *>(xs + 8 * i) = bf16x8_to_f16x8(xv[c]);
    }
    if (tid < NX) Xs[tid] = xgv;
    __syncthreads();
    float accg = 0.0f, accu = 0.0f;
    gu.compute(0, xs, Xs, accg, accu);
    for (int i0 = kMPB; gu.more(i0); i0 += kMPB) {
        gu.load(i0);
        gu.compute(i0, xs, Xs, accg, accu);
    }
    if (!routed && jb == 0 && a.shared_gate) {   // one unit per token forms its shared-expert gate
        __shared__ float gred[kBW];
        static_assert(64 * kBW == kGlueWG, "the gate runs on one full workgroup");
        const float gv = shared_gate_token(xs, a.shared_gate, a.d, gred);
        if (tid == 0) a.sgate[t] = gv;
    }
    accg = row_sum16(accg);
    accu = row_sum16(accu);
    if (lane < 16) {
        red[wave][0][lane] = accg;
        red[wave][1][lane] = accu;
    }
    __syncthreads();
    if (wave == 0) {
        float hv = 0.0f;
        if (lane < 16) {
            float gv = 0.0f, uv = 0.0f;
#pragma unroll
            for (int w = 0; w < kBW; ++w) {
                gv += red[w][0][lane];
                uv += red[w][1][lane];
            }
            const uint32_t hb = f32_to_f16(gelu_tanh_f32(gv) * uv);
            if (routed) a.h_r[(size_t)pr * a.I + 16 * jb + lane] = (uint16_t)hb;
            else a.h_s[(size_t)t * a.Is + 16 * jb + lane] = (uint16_t)hb;
            hv = f16_to_f32(hb);
        }
        hv += __shfl_xor(hv, 8);
        hv += __shfl_xor(hv, 4);
        hv += __shfl_xor(hv, 2);
        hv += __shfl_xor(hv, 1);
        if (lane == 0) {
            if (routed) a.hs_r[(size_t)pr * JBr + jb] = hv;
            else a.hs_s[(size_t)t * JBs + jb] = hv;
        }
    }
}

// ----------------------------------------------------------------------------- launch C
// grid: T * (d / 16); block 64 * NW with NW = min(16, k + 4). Wave s < k: routed slot s. The
// shared down projection's group pairs go round-robin to waves k..NW-1 (to all waves when
// k == 16).
// LDS: h_r of the k slots [k][I] | h_s [I_s] | Hr [k][I/64] | Hsh [I_s/64] | Ws [k] |
//      part_r [k][16] | part_s [NW][16]; Q4_0: Hr [k][I/32] and Hsh [I_s/32] half-group sums
template <int MAXT, bool Q4>
__global__ __launch_bounds__(MAXT) void k_dec_down(DecArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int RB = a.d / 16, GI = a.I / 64, GS = a.Is / 64;
    const int t = blockIdx.x / RB, db = blockIdx.x % RB;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int NW = blockDim.x >> 6, nth = blockDim.x;
    const int s0 = NW > a.k ? a.k : 0, SN = NW - s0;   // shared waves [s0, NW)
    uint16_t *hr = reinterpret_cast<uint16_t *>(smem);
    uint16_t *hsh = hr + (size_t)a.k * a.I;
    float *Hr = reinterpret_cast<float *>(hsh + a.Is);
    constexpr int NH = Q4 ? 2 : 1;   // input sums per group
    float *Hsh = Hr + a.k * GI * NH;
    float *Ws = Hsh + GS * NH;
    float *part_r = Ws + a.k;
    float *part_s = part_r + a.k * 16;
    // the expert indices, then the (small) staging reads, then this wave's first batch of
    // weights; loads retire in order, so the staging stores below wait only for the former
    const int sw = wave >= s0 ? wave - s0 : 0;
    int e = 0;
    if (wave < a.k) {
        e = __builtin_amdgcn_readfirstlane(a.idx[(size_t)t * a.k + wave]);
        e = __builtin_amdgcn_readfirstlane(expert_slot_of(a.eslot, a.n_slots, a.slot_faults, e, false));
    }
    constexpr int kHC = 2;   // 16-byte chunks of the slot h per thread: k I / 8 <= kHC * 64 * NW
    u32x4_t hrv[kHC];
#pragma unroll
    for (int c = 0; c < kHC; ++c) hrv[c] = ld16(a.h_r + (size_t)t * a.k * a.I + 8 * min(tid + nth * c, a.k * a.I / 8 - 1));
    const u32x4_t hsv = ld16(a.h_s + (size_t)t * a.Is + 8 * min(tid, a.Is / 8 - 1));
    const int ih = min(tid, a.k * GI - 1), ihs = min(tid, GS - 1);
    const float *qr = a.hs_r + (size_t)t * a.k * (a.I / 16) + 4 * ih;
    const float *qs = a.hs_s + (size_t)t * (a.Is / 16) + 4 * ihs;
    const float qr0 = qr[0], qr1 = qr[1], qr2 = qr[2], qr3 = qr[3];
    const float qs0 = qs[0], qs1 = qs[1], qs2 = qs[2], qs3 = qs[3];
    const float wv = a.wts[(size_t)t * a.k + min(tid, a.k - 1)];
    const float sgv = a.shared_gate ? a.sgate[t] : 1.0f;
    const uint32_t hres = (a.res_out && tid < 16) ? a.res_h[(size_t)t * a.d + 16 * db + tid] : 0u;
    Down16<kMPC, Q4> dr(static_cast<const uint8_t *>(a.down.codes) + (size_t)e * a.d * a.I / 2,
                    a.down.sb + (size_t)e * a.d * GI, db >> 1, db & 1, GI, 0, 1);
    Down16<kMPC, Q4> ds(static_cast<const uint8_t *>(a.sh_down.codes), a.sh_down.sb, db >> 1, db & 1, GS, sw, SN);
    if (wave < a.k) dr.load(0);
    if (wave >= s0) ds.load(0);
    if (a.k * a.I / 8 <= kHC * nth) {
#pragma unroll
        for (int c = 0; c < kHC; ++c)
            if (tid + nth * c < a.k * a.I / 8) *reinterpret_cast<u32x4_t *>(hr + 8 * (tid + nth * c)) = hrv[c];
    } else {
        for (int i = tid; i < a.k * a.I / 8; i += nth)
            *reinterpret_cast<u32x4_t *>(hr + 8 * i) = ld16(a.h_r + (size_t)t * a.k * a.I + 8 * i);
    }
    if (a.Is / 8 <= nth) {
        if (tid < a.Is / 8) *reinterpret_cast<u32x4_t *>(hsh + 8 * tid) = hsv;
    } else {
        for (int i = tid; i < a.Is / 8; i += nth)
            *reinterpret_cast<u32x4_t *>(hsh + 8 * i) = ld16(a.h_s + (size_t)t * a.Is + 8 * i);
    }
    // group sums of h from its 16-value sums (Q4_0: the two half-group sums)
    auto put = [&](float *dst, int i, float q0, float q1, float q2, float q3) {
        if (Q4) {
            dst[2 * i] = q0 + q1;
            dst[2 * i + 1] = q2 + q3;
        } else {
            dst[i] = (q0 + q1) + (q2 + q3);
        }
    };
    if (tid < a.k * GI) put(Hr, tid, qr0, qr1, qr2, qr3);
    for (int i = tid + nth; i < a.k * GI; i += nth) {
        const float *q = a.hs_r + (size_t)t * a.k * (a.I / 16) + 4 * i;
        put(Hr, i, q[0], q[1], q[2], q[3]);
    }
    if (tid < GS) put(Hsh, tid, qs0, qs1, qs2, qs3);
    for (int i = tid + nth; i < GS; i += nth) {
        const float *q = a.hs_s + (size_t)t * (a.Is / 16) + 4 * i;
        put(Hsh, i, q[0], q[1], q[2], q[3]);
    }
    if (tid < a.k) Ws[tid] = wv;
    __syncthreads();
    if (wave < a.k) {
        float r = dr.compute(0, hr + (size_t)wave * a.I, Hr + wave * GI * NH);
        for (int i0 = kMPC; dr.more(i0); i0 += kMPC) {
            dr.load(i0);
            r += dr.compute(i0, hr + (size_t)wave * a.I, Hr + wave * GI * NH);
        }
        r = row_sum16(r);
        if (lane < 16) part_r[wave * 16 + lane] = r;
    }
    if (wave >= s0) {
        float r = ds.compute(0, hsh, Hsh);
        for (int i0 = kMPC; ds.more(i0); i0 += kMPC) {
            ds.load(i0);
            r += ds.compute(i0, hsh, Hsh);
        }
        r = row_sum16(r);
        if (lane < 16) part_s[wave * 16 + lane] = r;
    }
    __syncthreads();
    if (tid < 16) {
        float out = 0.0f;
        for (int w = s0; w < NW; ++w) out += part_s[w * 16 + tid];
        out *= sgv;   // gated shared expert (1 without a gate)
        for (int s = 0; s < a.k; ++s) out = fmaf(Ws[s], part_r[s * 16 + tid], out);
        a.y[(size_t)t * a.d + 16 * db + tid] = out;
        if (a.res_out) {   // the next layer's residual step (glue_token's expression, no post-FFN norm)
            const double sc = a.res_scalar ? bf16_to_f64(*a.res_scalar) : 1.0;
            const uint32_t hb = f64_to_bf16((bf16_to_f64(hres) + (double)out) * sc);
            a.res_out[(size_t)t * a.d + 16 * db + tid] = (uint16_t)hb;
            const double r = bf16_to_f64(hb);
            const double ss = row_scan16_f64(r * r);   // lanes 0-15: row 0 of wave 0
            if (tid == 15) a.res_ss[(size_t)t * (a.d / 16) + db] = ss;
        }
    }
}

DecArgs dec_args(const moe_layer *L, const uint16_t *x, int T, float *y) {
    const moe_dims &D = L->dims;
    DecArgs a{};
    a.x = x;
    a.T = T;
    a.d = D.d_model;
    a.E = D.n_experts;
    a.k = D.top_k;
    a.I = D.d_expert;
    a.Is = D.d_shared;
    a.rq = static_cast<const uint8_t *>(L->w.router.codes);
    a.rsb = L->w.router.sb;
    a.logit_bias = L->w.logit_bias;
    a.pes = L->w.per_expert_scale;
    a.logits = L->ws.logits;
    a.idx = L->ws.idx;
    a.wts = L->ws.wts;
    a.gate = L->w.gate;
    a.up = L->w.up;
    a.down = L->w.down;
    a.sh_gate = L->w.sh_gate;
    a.sh_up = L->w.sh_up;
    a.sh_down = L->w.sh_down;
    a.xg = L->ws.dxg;
    a.q4_0 = D.expert_format == MOE_FORMAT_Q4_0;
    a.h_r = L->ws.dh_r;
    a.h_s = L->ws.dh_s;
    a.hs_r = L->ws.dhs_r;
    a.hs_s = L->ws.dhs_s;
    a.y = y;
    a.shared_gate = L->w.shared_gate;
    a.sgate = L->ws.sgate;
    a.eslot = L->w.expert_slot;
    a.n_slots = L->w.n_slots;
    a.slot_faults = L->ws.slot_faults;
    return a;
}

}  // namespace

int dec_down_waves(const moe_dims &D) { return D.top_k + 4 < 16 ? D.top_k + 4 : 16; }

// input sums per 64-input group the decode kernels use (Q4_0: one per 32-input block)
static size_t sums_per_group(const moe_dims &D) { return D.expert_format == MOE_FORMAT_Q4_0 ? 2 : 1; }

size_t dec_down_lds(const moe_dims &D) {
    const size_t k = D.top_k, I = D.d_expert, Is = D.d_shared, nh = sums_per_group(D);
    return sizeof(uint16_t) * (k * I + Is) +
           sizeof(float) * (nh * (k * I / 64 + Is / 64) + k + 16 * k + 16 * dec_down_waves(D));
}

size_t dec_gateup_lds(const moe_dims &D) {
    return sizeof(uint16_t) * D.d_model + sizeof(float) * (sums_per_group(D) * (D.d_model / 64) + kBW * 2 * 16);
}

size_t dec_workspace_floats(const moe_dims &D, int max_dec, int which) {
    switch (which) {
        case 0: return (size_t)max_dec * (D.d_model / 64) * sums_per_group(D);  // x group (Q4_0: half) sums
        case 1: return (size_t)max_dec * D.top_k * D.d_expert / 2;              // routed h (fp16)
        case 2: return (size_t)max_dec * D.d_shared / 2;                        // shared h (fp16)
        case 3: return (size_t)max_dec * D.top_k * (D.d_expert / 16);           // routed 16-value h sums
        default: return (size_t)max_dec * (D.d_shared / 16);                    // shared 16-value h sums
    }
}

hipError_t launch_dec_router(const moe_layer *L, const uint16_t *x, int T, float *logits, hipStream_t s,
                             bool write_aux) {
    const moe_dims &D = L->dims;
    DecArgs a = dec_args(L, x, T, nullptr);
    a.logits = logits;
    if (!write_aux) a.xg = nullptr;   // the group sums of x come from the router prologue
    const size_t lds = sizeof(float) * kRW * T * (D.d_model / 64);
    launch(k_dec_router<0, false>, dim3(cdiv(D.n_experts, kRW)), dim3(64 * kRW), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_dec_router_pro(const moe_layer *L, const uint16_t *x, int T, float *logits, hipStream_t s) {
    const moe_dims &D = L->dims;
    DecArgs a = dec_args(L, x, T, nullptr);
    a.logits = logits;
    a.router_scale = L->w.router_scale;
    const size_t lds = sizeof(float) * kRW * T * (D.d_model / 64) + sizeof(uint16_t) * T * D.d_model +
                       sizeof(double) * (kGlueWG / 64);
    launch(k_dec_router<0, true>, dim3(cdiv(D.n_experts, kRW)), dim3(64 * kRW), lds, s, a);
    return hipGetLastError();
}

bool dec_router_glue_fits(const moe_dims &D, int T) { return (size_t)T * D.d_model * 2 <= kGlueLdsMax; }

hipError_t launch_dec_router_glue(const moe_layer *L, const uint16_t *h_in, const float *y_in,
                                  const uint16_t *post_in, const uint16_t *scalar_in, uint16_t *h_out,
                                  uint16_t *x_out, int T, hipStream_t s) {
    const moe_dims &D = L->dims;
    DecArgs a = dec_args(L, x_out, T, nullptr);
    a.h_in = h_in;
    a.y_in = y_in;
    a.post_in = post_in;
    a.scalar_in = scalar_in;
    a.h_out = h_out;
    a.x_out = x_out;
    const size_t lds = sizeof(float) * kRW * T * (D.d_model / 64) + sizeof(uint16_t) * T * D.d_model +
                       sizeof(double) * (kGlueWG / 64);
    a.router_scale = L->w.router_scale;
    if (a.router_scale)
        launch(k_dec_router<1, true>, dim3(cdiv(D.n_experts, kRW)), dim3(64 * kRW), lds, s, a);
    else
        launch(k_dec_router<1, false>, dim3(cdiv(D.n_experts, kRW)), dim3(64 * kRW), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_dec_router_norm(const moe_layer *L, const uint16_t *h_in, const double *ss_in, uint16_t *x_out,
                                  int T, hipStream_t s) {
    const moe_dims &D = L->dims;
    DecArgs a = dec_args(L, x_out, T, nullptr);
    a.h_in = h_in;
    a.ss_in = ss_in;
    a.x_out = x_out;
    const size_t lds = sizeof(float) * kRW * T * (D.d_model / 64) + sizeof(uint16_t) * T * D.d_model +
                       sizeof(double) * (kGlueWG / 64);
    a.router_scale = L->w.router_scale;
    if (a.router_scale)
        launch(k_dec_router<2, true>, dim3(cdiv(D.n_experts, kRW)), dim3(64 * kRW), lds, s, a);
    else
        launch(k_dec_router<2, false>, dim3(cdiv(D.n_experts, kRW)), dim3(64 * kRW), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_dec_gateup(const moe_layer *L, const uint16_t *x, int T, hipStream_t s) {
    const moe_dims &D = L->dims;
    const DecArgs a = dec_args(L, x, T, nullptr);
    const int grid = T * D.top_k * (D.d_expert / 16) + T * (D.d_shared / 16);
    const size_t lds = dec_gateup_lds(D);
    if (a.q4_0) {
        if (D.n_experts <= 128) launch(k_dec_gateup<2, true>, dim3(grid), dim3(64 * kBW), lds, s, a);
        else if (D.n_experts <= 256) launch(k_dec_gateup<4, true>, dim3(grid), dim3(64 * kBW), lds, s, a);
        else launch(k_dec_gateup<MOE_MAX_EXPERTS / 64, true>, dim3(grid), dim3(64 * kBW), lds, s, a);
    } else {
        if (D.n_experts <= 128) launch(k_dec_gateup<2, false>, dim3(grid), dim3(64 * kBW), lds, s, a);
        else if (D.n_experts <= 256) launch(k_dec_gateup<4, false>, dim3(grid), dim3(64 * kBW), lds, s, a);
        else launch(k_dec_gateup<MOE_MAX_EXPERTS / 64, false>, dim3(grid), dim3(64 * kBW), lds, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_dec_down(const moe_layer *L, int T, float *y, hipStream_t s, const uint16_t *res_h,
                           uint16_t *res_out) {
    const moe_dims &D = L->dims;
    DecArgs a = dec_args(L, nullptr, T, y);
    if (res_out) {
        a.res_h = res_h;
        a.res_out = res_out;
        a.res_scalar = L->w.layer_scalar;
        a.res_ss = L->ws.dss;
    }
    const int nw = dec_down_waves(D);
    const dim3 grid(T * (D.d_model / 16)), block(64 * nw);
    if (a.q4_0) {
        if (nw <= 12) launch(k_dec_down<768, true>, grid, block, dec_down_lds(D), s, a);
        else launch(k_dec_down<1024, true>, grid, block, dec_down_lds(D), s, a);
    } else {
        if (nw <= 12) launch(k_dec_down<768, false>, grid, block, dec_down_lds(D), s, a);
        else launch(k_dec_down<1024, false>, grid, block, dec_down_lds(D), s, a);
    }
    return hipGetLastError();
}

}  // namespace qmoe
