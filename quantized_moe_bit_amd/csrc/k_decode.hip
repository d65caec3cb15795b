// Decode path (up to 16 tokens): three launches of wavefront GEMV kernels over 4-bit
// group-64 affine weights, with no communication between workgroups of a launch.
//
// Each selected expert is a GELU-gated FFN whose weights are w = scale * q + bias per group
// of 64 inputs (Mference system design, "Why the runtime has this shape"; "Metal
// execution": decode uses custom affine INT4/INT8 GEMV kernels that consume the packed codes
// and BF16 scale/bias directly, and the routed kernels fuse the affine decode, GeGLU and the
// weighted reduction).
//
// Exact affine split per group (x the 64 inputs of the group):
//   sum_j x_j (s q_j + b) = 16 s * sum_j x_j (1 + q_j/16) + (b - 16 s) * sum_j x_j.
// A lane holds half of a group's inputs; it adds 16 s * (its half of the first sum) +
// (b - 16 s) * (its half of sum x), which is linear, so the halves add up to the exact group
// term. 1 + q/16 comes from the nibbles with one shift and one and-or; v_dot2_f32_bf16
// (gate/up, x is bf16) and v_dot2_f32_f16 (down, h is fp16) accumulate in fp32.
//
// Work is cut into many thin units: every projection is split along its input dimension into
// pieces of kGPS groups, each piece a 256-thread workgroup streaming ~25 KB, and the consumer
// of a projection adds its partial sums in piece order (fixed order, deterministic).
//
// Launch 1 (k_dec_stage1): router logits in the fixed fp32 order the oracle uses (one wave
//   per expert, one lane per input group), and the shared expert's gate/up partial sums (the
//   shared branch does not depend on routing; Mference "Decode" likewise starts it before
//   the routed branch).
// Launch 2 (k_dec_stage2): routed gate/up partial sums per (pair, 32 rows, input piece); each
//   wave first derives its token's top-k from the logits with a DPP argmax over packed
//   (logit, index) keys, identical on every wave. Other workgroups: the shared down
//   projection per (token, 32 rows, input piece), forming h = fp16(gelu(g) * u) for their
//   piece from the launch-1 partials.
// Launch 3 (k_dec_stage3): one workgroup per (token, 32 output rows), one wave per routed
//   slot: h of the slot from the launch-2 partials, the down projection, then
//   y = shared + w_0 r_0 + ... + w_{k-1} r_{k-1} in slot order (Mference "Decode", cb2;
//   TinyTitan architecture "Invariants": fixed reduction order).
#include "device_common.h"
#include "moe_internal.h"

namespace qmoe {
namespace {

constexpr int kRW = 4;      // router experts (waves) per workgroup
constexpr int kPW = 4;      // waves per partial-sum workgroup
constexpr int kPB = cdiv_c(kGPS, kPW);   // groups per wave in a piece
constexpr int kW2 = 8;      // waves per launch-2 workgroup
constexpr int kB2 = 6;      // groups per wave of a routed gate/up unit (kW2 * kB2 >= 48 input groups)
constexpr uint32_t kOneBf16x2 = 0x3F803F80u;
constexpr uint32_t kOneF16x2 = 0x3C003C00u;

// ----------------------------------------------------------------------------- router
// The wave's expert e; lane g handles input group g (and g + 64, ... for d > 4096).
// P[t][g] into Ps, then lanes t < T sum over g in ascending order (the group sums X also go
// to xg_out when it is given). Fixed fp32 order:
//   X = ((0 + x_0) + x_1) + ...; A = fma chain; P = fma(s, A, fl(b * X)); L = ((0 + P_0) + ...)
__device__ __forceinline__ void router_wave(const uint16_t *__restrict__ x, int T, int d, int e, const uint8_t *__restrict__ rq,
                            const uint32_t *__restrict__ rsb, float *Ps, float *xg_out) {
#pragma clang fp contract(off)
    const int G = d / 64, lane = threadIdx.x & 63;
    for (int g = lane; g < G; g += 64) {
        const u32x4_t *cp = reinterpret_cast<const u32x4_t *>(rq + (size_t)e * d + 64 * g);
        const u32x4_t c0 = cp[0], c1 = cp[1], c2 = cp[2], c3 = cp[3];
        const uint32_t cw[16] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3],
                                 c2[0], c2[1], c2[2], c2[3], c3[0], c3[1], c3[2], c3[3]};
        const uint32_t sbw = rsb[(size_t)e * G + g];
        const float sc = bf16_to_f32(sbw & 0xFFFFu), bi = bf16_to_f32(sbw >> 16);
        for (int t = 0; t < T; ++t) {
            const u32x4_t *xp = reinterpret_cast<const u32x4_t *>(x + (size_t)t * d + 64 * g);
            u32x4_t xv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) xv[i] = xp[i];
            float X = 0.0f, A = 0.0f;
#pragma unroll
            for (int j2 = 0; j2 < 32; ++j2) {          // element pair (2 j2, 2 j2 + 1)
                const uint32_t xw = xv[j2 >> 2][j2 & 3];
                const float xa = bf16_to_f32(xw & 0xFFFFu), xb = bf16_to_f32(xw >> 16);
                const uint32_t c = cw[j2 >> 1];
                const int sh = (j2 & 1) * 16;
                const float qa = (float)((c >> sh) & 0xFFu), qb = (float)((c >> (sh + 8)) & 0xFFu);
                X = X + xa;
                X = X + xb;
                A = __builtin_fmaf(xa, qa, A);
                A = __builtin_fmaf(xb, qb, A);
            }
            const float bX = bi * X;
            Ps[t * G + g] = __builtin_fmaf(sc, A, bX);
            if (xg_out) xg_out[t * G + g] = X;
        }
    }
}

// ----------------------------------------------------------------------------- gate/up piece
// Partial gate and up sums of 32 rows (block jb) over input groups [g0, g1) (at most kGPS)
// for one token, x of those groups staged in LDS (xs, indexed from g0). Wave w takes groups
// g0 + w, g0 + w + kPW, ...; the four waves' sums are added in wave order.
template <int PB>
struct GUTiles {
    u32x4_t wg[PB], wu[PB];
    uint32_t sbg[PB], sbu[PB];
};

template <int NW, int PB>
__device__ __forceinline__ void gu_load(GUTiles<PB> &r, const uint8_t *Wg, const uint8_t *Wu, const uint32_t *Sg,
                                        const uint32_t *Su, int G, int jb, int g0, int g1) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 31;
    const size_t tb = (size_t)jb * G;
#pragma unroll
    for (int b = 0; b < PB; ++b) {
        const int g = g0 + wave + b * NW;
        if (g < g1) {
            r.wg[b] = ld16(Wg + (tb + g) * 1024 + lane * 16);
            r.wu[b] = ld16(Wu + (tb + g) * 1024 + lane * 16);
            r.sbg[b] = Sg[(tb + g) * 32 + n];
            r.sbu[b] = Su[(tb + g) * 32 + n];
        }
    }
}

template <int NW, int PB>
__device__ __forceinline__ void gu_compute(const GUTiles<PB> &r, const uint16_t *xs, const float *Xs, int g0, int g1,
                                           float &accg, float &accu) {
    const int wave = threadIdx.x >> 6, half = (threadIdx.x >> 5) & 1;
#pragma unroll
    for (int b = 0; b < PB; ++b) {
        const int g = g0 + wave + b * NW;
        if (g < g1) {
            float ag = 0.0f, au = 0.0f;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(xs + 64 * (g - g0) + 16 * s + 8 * half);
                ag = dot2_bf16(xv[0], nib_pair<0>(r.wg[b][s]), ag);
                ag = dot2_bf16(xv[1], nib_pair<1>(r.wg[b][s]), ag);
                ag = dot2_bf16(xv[2], nib_pair<2>(r.wg[b][s]), ag);
                ag = dot2_bf16(xv[3], nib_pair<3>(r.wg[b][s]), ag);
                au = dot2_bf16(xv[0], nib_pair<0>(r.wu[b][s]), au);
                au = dot2_bf16(xv[1], nib_pair<1>(r.wu[b][s]), au);
                au = dot2_bf16(xv[2], nib_pair<2>(r.wu[b][s]), au);
                au = dot2_bf16(xv[3], nib_pair<3>(r.wu[b][s]), au);
            }
            // the (b - 16 s) X_g term once per group (lanes of half 0)
            const float xsum = half == 0 ? Xs[g - g0] : 0.0f;
            const float s16g = 16.0f * bf16_to_f32(r.sbg[b] & 0xFFFFu);
            const float s16u = 16.0f * bf16_to_f32(r.sbu[b] & 0xFFFFu);
            accg = fmaf(s16g, ag, fmaf(bf16_to_f32(r.sbg[b] >> 16) - s16g, xsum, accg));
            accu = fmaf(s16u, au, fmaf(bf16_to_f32(r.sbu[b] >> 16) - s16u, xsum, accu));
        }
    }
}

// One gate/up piece over input groups [g0, g1) (at most NW * PB) with NW waves: loads tiles,
// stages x[g0:g1] of token row xrow, computes, adds the waves' sums in wave order, and either
// writes the 32 partial gate and up sums to out_g[n], out_u[n] (hout == nullptr) or, when the
// piece covers the whole input, h = fp16(gelu(g) * u) to hout[n] (and, with hsum_out, the
// sum of those 32 values to *hsum_out). With x_staged, xs and Xs already hold x[g0:g1] and
// its group sums (written before the call; the call's barrier publishes them); otherwise
// they are staged here. LDS: xs (NW * PB * 64 bf16), Xs (NW * PB floats), red.
template <int NW, int PB>
__device__ __forceinline__ void gateup_piece(const uint16_t *xrow, const uint8_t *Wg, const uint8_t *Wu,
                                             const uint32_t *Sg, const uint32_t *Su, int G, int jb, int g0, int g1,
                                             uint16_t *xs, float *Xs, float (*red)[2][32], float *out_g, float *out_u,
                                             uint16_t *hout, bool x_staged = false, float *hsum_out = nullptr) {
    static_assert(PB <= 8, "one 16-byte x chunk per thread");
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31;
    GUTiles<PB> r;
    gu_load<NW, PB>(r, Wg, Wu, Sg, Su, G, jb, g0, g1);
    if (!x_staged) {
        // stage x[g0:g1] and its group sums (eight consecutive threads per group)
        const int nch = (g1 - g0) * 8;
        float ps = 0.0f;
        if (tid < nch) {
            const u32x4_t v = ld16(xrow + 64 * g0 + 8 * tid);
            *reinterpret_cast<u32x4_t *>(xs + 8 * tid) = v;
#pragma unroll
            for (int w = 0; w < 4; ++w) ps += bf16_to_f32(v[w] & 0xFFFFu) + bf16_to_f32(v[w] >> 16);
        }
        ps += __shfl_xor(ps, 1);
        ps += __shfl_xor(ps, 2);
        ps += __shfl_xor(ps, 4);
        if (tid < nch && (tid & 7) == 0) Xs[tid >> 3] = ps;
    }
    __syncthreads();
    float accg = 0.0f, accu = 0.0f;
    gu_compute<NW, PB>(r, xs, Xs, g0, g1, accg, accu);
    accg += __shfl_xor(accg, 32);
    accu += __shfl_xor(accu, 32);
    if (lane < 32) {
        red[wave][0][n] = accg;
        red[wave][1][n] = accu;
    }
    __syncthreads();
    if (tid < 32) {
        float gv = 0.0f, uv = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            gv += red[w][0][tid];
            uv += red[w][1][tid];
        }
        if (hout) {
            const uint32_t hb = f32_to_f16_sat(gelu_tanh_f32(gv) * uv);
            hout[tid] = (uint16_t)hb;
            if (hsum_out) red[0][0][tid] = f16_to_f32(hb);
        } else {
            out_g[tid] = gv;
            out_u[tid] = uv;
        }
    }
    if (hout && hsum_out && wave == 0) {
        // sum of the 32 stored h values (after every lane of wave 0 has read red above)
        float hs = lane < 32 ? red[0][0][lane] : 0.0f;
        hs += __shfl_xor(hs, 16);
        hs += __shfl_xor(hs, 8);
        hs += __shfl_xor(hs, 4);
        hs += __shfl_xor(hs, 2);
        hs += __shfl_xor(hs, 1);
        if (lane == 0) *hsum_out = hs;
    }
}

// h = fp16(gelu(g) * u) for inputs [j0, j0 + nj) of a projection whose gate/up partial sums
// (KS pieces) are at part[(ks * 2 + {0: gate, 1: up}) * J + j]; pieces added in order. Each
// thread handles at most NPT inputs; for KS <= kKSFast every partial is loaded before any is
// used (one round trip), otherwise piece by piece.
constexpr int kKSFast = 4;
template <int NPT>
__device__ __forceinline__ void form_h(const float *part, int KS, int J, int j0, int nj, uint16_t *hl, int tid,
                                       int nthreads) {
    float gv[NPT], uv[NPT];
    if (KS <= kKSFast) {
        float gp[kKSFast][NPT], up[kKSFast][NPT];
#pragma unroll
        for (int ks = 0; ks < kKSFast; ++ks)
#pragma unroll
            for (int i = 0; i < NPT; ++i) {
                const int j = tid + i * nthreads;
                const bool ok = ks < KS && j < nj;
                gp[ks][i] = ok ? part[(size_t)(ks * 2) * J + j0 + j] : 0.0f;
                up[ks][i] = ok ? part[(size_t)(ks * 2 + 1) * J + j0 + j] : 0.0f;
            }
#pragma unroll
        for (int i = 0; i < NPT; ++i) {
            gv[i] = gp[0][i];
            uv[i] = up[0][i];
#pragma unroll
            for (int ks = 1; ks < kKSFast; ++ks) {
                gv[i] += gp[ks][i];
                uv[i] += up[ks][i];
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < NPT; ++i) gv[i] = uv[i] = 0.0f;
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int i = 0; i < NPT; ++i) {
                const int j = tid + i * nthreads;
                if (j < nj) {
                    gv[i] += part[(size_t)(ks * 2) * J + j0 + j];
                    uv[i] += part[(size_t)(ks * 2 + 1) * J + j0 + j];
                }
            }
    }
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
        const int j = tid + i * nthreads;
        if (j < nj) hl[j] = (uint16_t)f32_to_f16_sat(gelu_tanh_f32(gv[i]) * uv[i]);
    }
}

// ----------------------------------------------------------------------------- down part
// One wave: 32 output rows (block rb) of a down projection over input groups [g0, g1)
// (at most kDecodeChunkGroups) of its fp16 input h, staged in LDS at hl (indexed from g0).
struct DTiles {
    u32x4_t w4[kDecodeChunkGroups];
    uint32_t sbw[kDecodeChunkGroups];
};

__device__ __forceinline__ void down_load(DTiles &r, const uint8_t *W, const uint32_t *S, int rb, int Gk, int g0,
                                          int g1) {
    const int lane = threadIdx.x & 63, n = lane & 31;
    const size_t tb = (size_t)rb * Gk;
#pragma unroll
    for (int b = 0; b < kDecodeChunkGroups; ++b)
        if (g0 + b < g1) {
            r.w4[b] = ld16(W + (tb + g0 + b) * 1024 + lane * 16);
            r.sbw[b] = S[(tb + g0 + b) * 32 + n];
        }
}

// Hs: group sums of h (indexed from g0), or nullptr to form them from hl here.
__device__ __forceinline__ float down_compute(const DTiles &r, const uint16_t *hl, const float *Hs, int g0, int g1) {
    const int half = (threadIdx.x >> 5) & 1;
    float acc = 0.0f;
#pragma unroll
    for (int b = 0; b < kDecodeChunkGroups; ++b)
        if (g0 + b < g1) {
            float a = 0.0f, hsum = 0.0f;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4_t hv = *reinterpret_cast<const u32x4_t *>(hl + 64 * b + 16 * s + 8 * half);
                a = dot2_f16(hv[0], nib_pair_f16<0>(r.w4[b][s]), a);
                a = dot2_f16(hv[1], nib_pair_f16<1>(r.w4[b][s]), a);
                a = dot2_f16(hv[2], nib_pair_f16<2>(r.w4[b][s]), a);
                a = dot2_f16(hv[3], nib_pair_f16<3>(r.w4[b][s]), a);
                if (!Hs) {
                    hsum = dot2_f16(hv[0], kOneF16x2, hsum);
                    hsum = dot2_f16(hv[1], kOneF16x2, hsum);
                    hsum = dot2_f16(hv[2], kOneF16x2, hsum);
                    hsum = dot2_f16(hv[3], kOneF16x2, hsum);
                }
            }
            if (Hs) hsum = half == 0 ? Hs[b] : 0.0f;
            const float s16 = 16.0f * bf16_to_f32(r.sbw[b] & 0xFFFFu);
            acc = fmaf(s16, a, fmaf(bf16_to_f32(r.sbw[b] >> 16) - s16, hsum, acc));
        }
    return acc + __shfl_xor(acc, 32);
}

// ----------------------------------------------------------------------------- top-k
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

struct DecArgs {
    const uint16_t *x;
    int T, d, E, k, I, Is;
    int KSd, KSs;           // input pieces of the d-wide gate/up inputs and of the shared down input
    const uint8_t *rq;
    const uint32_t *rsb;
    const float *logit_bias;
    float *logits;
    int32_t *idx;
    float *wts;
    moe_qmat gate, up, down, sh_gate, sh_up, sh_down;
    float *gus;             // [T][KSd][2][I_s] shared gate/up partials
    uint16_t *h_r;          // [T*k][I]         routed hidden activations (fp16 bits)
    float *shp;             // [T][KSs][d]      shared down partials
    float *xg;              // [T][d/64]        group sums of x (router, fixed order)
    float *hs;              // [T*k][I/32]      sums of 32 consecutive routed h values
    float *y;
};

// grid: ceil(E / kRW) router workgroups + T * (I_s / 32) * KSd shared gate/up pieces; block 256
__global__ __launch_bounds__(64 * kPW) void k_dec_stage1(DecArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int RW = cdiv(a.E, kRW);
    const int G = a.d / 64;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if ((int)blockIdx.x < RW) {
        float *Ps = reinterpret_cast<float *>(smem);     // [kRW][T][G]
        const int e = blockIdx.x * kRW + wave;
        float *P = Ps + (size_t)wave * a.T * G;
        if (e < a.E) router_wave(a.x, a.T, a.d, e, a.rq, a.rsb, P, e == 0 ? a.xg : nullptr);
        __syncthreads();
        if (e < a.E && lane < a.T) {
#pragma clang fp contract(off)
            float L = 0.0f;
            for (int g = 0; g < G; ++g) L = L + P[lane * G + g];
            if (a.logit_bias) L = L + a.logit_bias[e];
            a.logits[(size_t)lane * a.E + e] = L;
        }
        return;
    }
    uint16_t *xs = reinterpret_cast<uint16_t *>(smem);
    float *Xs = reinterpret_cast<float *>(smem + sizeof(uint16_t) * 64 * kGPS);
    float(*red)[2][32] = reinterpret_cast<float(*)[2][32]>(smem + sizeof(uint16_t) * 64 * kGPS + sizeof(float) * 16);
    const int JBs = a.Is / 32;
    int u = blockIdx.x - RW;
    const int ks = u % a.KSd;
    u /= a.KSd;
    const int jb = u % JBs, t = u / JBs;
    const int g0 = ks * kGPS, g1 = min(G, g0 + kGPS);
    float *out = a.gus + ((size_t)t * a.KSd + ks) * 2 * a.Is + jb * 32;
    gateup_piece<kPW, kPB>(a.x + (size_t)t * a.d, static_cast<const uint8_t *>(a.sh_gate.codes),
                           static_cast<const uint8_t *>(a.sh_up.codes), a.sh_gate.sb, a.sh_up.sb, G, jb, g0, g1, xs,
                           Xs, red, out, out + a.Is, nullptr);
}

// grid: T * k * (I / 32) routed gate/up units + T * (d / 32) * KSs shared down pieces;
// block 64 * kW2
template <int kPer>
__global__ __launch_bounds__(64 * kW2) void k_dec_stage2(DecArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int G = a.d / 64, JB = a.I / 32;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int nR = a.T * a.k * JB;
    if ((int)blockIdx.x < nR) {
        const int jb = blockIdx.x % JB, pr = blockIdx.x / JB, t = pr / a.k, slot = pr % a.k;
        uint16_t *xs = reinterpret_cast<uint16_t *>(smem);
        // the token's x is fetched while the selection is derived
        const bool narrow = G <= kW2 * kB2;
        u32x4_t xv = u32x4_t{0u, 0u, 0u, 0u};
        float xgv = 0.0f;
        if (narrow && tid < G * 8) xv = ld16(a.x + (size_t)t * a.d + 8 * tid);
        if (narrow && tid < G) xgv = a.xg[(size_t)t * G + tid];
        // every wave derives the token's selection itself; one unit of the pair records it
        const bool record = (jb == 0 && wave == 0);
        float wsel;
        const int e = wave_topk<kPer>(a.logits + (size_t)t * a.E, a.E, a.k, slot, record, wsel);
        if (record && lane == 0) {
            a.idx[pr] = e;
            a.wts[pr] = wsel;
        }
        // LDS: xs [min(d, 64 kW2 kB2) bf16] | Xs [64 floats] | red [kW2][2][32] | wide-path totals
        const int XE = min(a.d, 64 * kW2 * kB2);
        float *Xs = reinterpret_cast<float *>(smem + sizeof(uint16_t) * XE);
        float(*red)[2][32] = reinterpret_cast<float(*)[2][32]>(smem + sizeof(uint16_t) * XE + sizeof(float) * 64);
        if (narrow && tid < G * 8) *reinterpret_cast<u32x4_t *>(xs + 8 * tid) = xv;
        if (narrow && tid < G) Xs[tid] = xgv;
        const size_t cstride = (size_t)a.I * a.d / 2, sstride = (size_t)a.I * G;
        const uint8_t *Wg = static_cast<const uint8_t *>(a.gate.codes) + e * cstride;
        const uint8_t *Wu = static_cast<const uint8_t *>(a.up.codes) + e * cstride;
        uint16_t *hout = a.h_r + (size_t)pr * a.I + jb * 32;
        if (narrow) {
            gateup_piece<kW2, kB2>(a.x + (size_t)t * a.d, Wg, Wu, a.gate.sb + e * sstride, a.up.sb + e * sstride, G,
                                   jb, 0, G, xs, Xs, red, nullptr, nullptr, hout, true, a.hs + (size_t)pr * JB + jb);
        } else {
            // wide inputs: kW2 * kB2 groups at a time, partial sums carried through red
            float *acc = reinterpret_cast<float *>(red);   // reuse: [2][32] totals after each batch
            float tg = 0.0f, tu = 0.0f;
            for (int g0 = 0; g0 < G; g0 += kW2 * kB2) {
                gateup_piece<kW2, kB2>(a.x + (size_t)t * a.d, Wg, Wu, a.gate.sb + e * sstride,
                                       a.up.sb + e * sstride, G, jb, g0, min(G, g0 + kW2 * kB2), xs, Xs, red,
                                       acc + 2 * 64 * kW2, acc + 2 * 64 * kW2 + 32, nullptr);
                __syncthreads();
                if (tid < 32) {
                    tg += acc[2 * 64 * kW2 + tid];
                    tu += acc[2 * 64 * kW2 + 32 + tid];
                }
                __syncthreads();
            }
            float hv = 0.0f;
            if (tid < 32) {
                const uint32_t hb = f32_to_f16_sat(gelu_tanh_f32(tg) * tu);
                hout[tid] = (uint16_t)hb;
                hv = f16_to_f32(hb);
            }
            if (wave == 0) {
                hv += __shfl_xor(hv, 16);
                hv += __shfl_xor(hv, 8);
                hv += __shfl_xor(hv, 4);
                hv += __shfl_xor(hv, 2);
                hv += __shfl_xor(hv, 1);
                if (lane == 0) a.hs[(size_t)pr * JB + jb] = hv;
            }
        }
        return;
    }
    // shared down piece: (token, 32 output rows, input groups [g0, g1) of I_s)
    const int RB = a.d / 32, GIs = a.Is / 64;
    int u = blockIdx.x - nR;
    const int ks = u % a.KSs;
    u /= a.KSs;
    const int rb = u % RB, t = u / RB;
    const int g0 = ks * kGPS, g1 = min(GIs, g0 + kGPS);
    uint16_t *hl = reinterpret_cast<uint16_t *>(smem);                              // [kGPS * 64]
    float *part = reinterpret_cast<float *>(smem + sizeof(uint16_t) * 64 * kGPS);   // [kW2][32]
    // wave w takes a contiguous sub-range of at most kSB groups
    constexpr int kSB = cdiv_c(kGPS, kW2);
    const int wg0 = min(g1, g0 + wave * kSB), wg1 = min(g1, wg0 + kSB);
    const uint8_t *W = static_cast<const uint8_t *>(a.sh_down.codes);
    DTiles r;
    down_load(r, W, a.sh_down.sb, rb, GIs, wg0, wg1);
    form_h<cdiv_c(64 * kGPS, 64 * kW2)>(a.gus + (size_t)t * a.KSd * 2 * a.Is, a.KSd, a.Is, 64 * g0, 64 * (g1 - g0),
                                        hl, tid, 64 * kW2);
    __syncthreads();
    const float rsum = down_compute(r, hl + 64 * (wg0 - g0), nullptr, wg0, wg1);
    if (lane < 32) part[wave * 32 + lane] = rsum;
    __syncthreads();
    if (tid < 32) {
        float sacc = 0.0f;
#pragma unroll
        for (int w = 0; w < kW2; ++w) sacc += part[w * 32 + tid];
        a.shp[((size_t)t * a.KSs + ks) * a.d + rb * 32 + tid] = sacc;
    }
}

// grid: T * (d / 32); block 64 * k (k <= MAXW): wave s = routed slot s
template <int MAXW>
__global__ __launch_bounds__(64 * MAXW) void k_dec_stage3(DecArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int RB = a.d / 32, GI = a.I / 64;
    const int t = blockIdx.x / RB, rb = blockIdx.x % RB;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    uint16_t *hl = reinterpret_cast<uint16_t *>(smem);                              // [k][I]
    float *part = reinterpret_cast<float *>(smem + sizeof(uint16_t) * a.k * a.I);  // [k][32]
    float *Hs = part + a.k * 32;                                                    // [k][I/64]
    const int pr = t * a.k + wave;
    const int e = a.idx[pr];
    // loads that do not depend on the expert go out first: the slot's h, and (first 32
    // threads) the shared-expert partial sums and the slot weights of the combine
    constexpr int kHL = 4;   // h chunks of 16 bytes per lane: I <= 64 * 8 * kHL
    u32x4_t hv[kHL];
#pragma unroll
    for (int c = 0; c < kHL; ++c) {
        const int i = lane + 64 * c;
        hv[c] = i < a.I / 8 ? ld16(a.h_r + (size_t)pr * a.I + 8 * i) : u32x4_t{0u, 0u, 0u, 0u};
    }
    // group sums of the slot's h from the 32-value sums its gate/up units wrote
    float hg = 0.0f;
    if (lane < GI && GI <= 64)
        hg = a.hs[(size_t)pr * (2 * GI) + 2 * lane] + a.hs[(size_t)pr * (2 * GI) + 2 * lane + 1];
    constexpr int kSP = 4, kWP = MAXW;
    float shv[kSP], wv[kWP];
    if (tid < 32) {
        const int row = rb * 32 + tid;
#pragma unroll
        for (int ks = 0; ks < kSP; ++ks) shv[ks] = ks < a.KSs ? a.shp[((size_t)t * a.KSs + ks) * a.d + row] : 0.0f;
#pragma unroll
        for (int s = 0; s < kWP; ++s) wv[s] = s < a.k ? a.wts[(size_t)t * a.k + s] : 0.0f;
    }
    const uint8_t *W = static_cast<const uint8_t *>(a.down.codes) + (size_t)e * a.d * a.I / 2;
    const uint32_t *S = a.down.sb + (size_t)e * a.d * GI;
    float rsum = 0.0f;
    for (int gb = 0; gb < GI; gb += kDecodeChunkGroups) {
        const int gb1 = min(GI, gb + kDecodeChunkGroups);
        DTiles r;
        down_load(r, W, S, rb, GI, gb, gb1);
        if (gb == 0) {
            if (lane < GI && GI <= 64) Hs[wave * GI + lane] = hg;
            if (a.I <= 64 * 8 * kHL) {
#pragma unroll
                for (int c = 0; c < kHL; ++c) {
                    const int i = lane + 64 * c;
                    if (i < a.I / 8) *reinterpret_cast<u32x4_t *>(hl + (size_t)wave * a.I + 8 * i) = hv[c];
                }
            } else {
                for (int i = lane; i < a.I / 8; i += 64)
                    *reinterpret_cast<u32x4_t *>(hl + (size_t)wave * a.I + 8 * i) =
                        ld16(a.h_r + (size_t)pr * a.I + 8 * i);
            }
        }
        __syncthreads();
        rsum += down_compute(r, hl + (size_t)wave * a.I + 64 * gb, GI <= 64 ? Hs + wave * GI + gb : nullptr, gb, gb1);
    }
    if (lane < 32) part[wave * 32 + lane] = rsum;
    __syncthreads();
    if (tid < 32) {
        const int row = rb * 32 + tid;
        float out = 0.0f;
        if (a.KSs <= kSP) {
#pragma unroll
            for (int ks = 0; ks < kSP; ++ks)
                if (ks < a.KSs) out += shv[ks];
        } else {
            for (int ks = 0; ks < a.KSs; ++ks) out += a.shp[((size_t)t * a.KSs + ks) * a.d + row];
        }
#pragma unroll
        for (int s = 0; s < kWP; ++s)
            if (s < a.k) out = fmaf(wv[s], part[s * 32 + tid], out);
        a.y[(size_t)t * a.d + row] = out;
    }
}

DecArgs dec_args(const moe_layer *L, const uint16_t *x, int T, float *y) {
    const moe_dims &D = L->dims;
    DecArgs a;
    a.x = x;
    a.T = T;
    a.d = D.d_model;
    a.E = D.n_experts;
    a.k = D.top_k;
    a.I = D.d_expert;
    a.Is = D.d_shared;
    a.KSd = cdiv(D.d_model / 64, kGPS);
    a.KSs = cdiv(D.d_shared / 64, kGPS);
    a.rq = static_cast<const uint8_t *>(L->w.router.codes);
    a.rsb = L->w.router.sb;
    a.logit_bias = L->w.logit_bias;
    a.logits = L->ws.logits;
    a.idx = L->ws.idx;
    a.wts = L->ws.wts;
    a.gate = L->w.gate;
    a.up = L->w.up;
    a.down = L->w.down;
    a.sh_gate = L->w.sh_gate;
    a.sh_up = L->w.sh_up;
    a.sh_down = L->w.sh_down;
    a.gus = L->ws.dgus;
    a.h_r = L->ws.dh_r;
    a.shp = L->ws.dshp;
    a.xg = L->ws.dxg;
    a.hs = L->ws.dhs;
    a.y = y;
    return a;
}

}  // namespace

size_t dec_stage3_lds(const moe_dims &D) {
    return sizeof(uint16_t) * D.top_k * D.d_expert + sizeof(float) * D.top_k * (32 + D.d_expert / 64);
}

size_t dec_workspace_floats(const moe_dims &D, int max_dec, int which) {
    const size_t KSd = cdiv(D.d_model / 64, kGPS), KSs = cdiv(D.d_shared / 64, kGPS);
    if (which == 0) return (size_t)max_dec * KSd * 2 * D.d_shared;
    if (which == 1) return (size_t)max_dec * D.top_k * D.d_expert / 2;   // fp16 h, in floats
    if (which == 3) return (size_t)max_dec * (D.d_model / 64);           // x group sums
    if (which == 4) return (size_t)max_dec * D.top_k * (D.d_expert / 32); // h 32-value sums
    return (size_t)max_dec * KSs * D.d_model;
}

hipError_t launch_dec_stage1(const moe_layer *L, const uint16_t *x, int T, hipStream_t s) {
    const moe_dims &D = L->dims;
    const DecArgs a = dec_args(L, x, T, nullptr);
    const int G = D.d_model / 64;
    const int grid = cdiv(D.n_experts, kRW) + T * (D.d_shared / 32) * a.KSd;
    const size_t lds_router = sizeof(float) * kRW * T * G;
    const size_t lds_gu = sizeof(uint16_t) * 64 * kGPS + sizeof(float) * (16 + kPW * 2 * 32);
    hipLaunchKernelGGL(k_dec_stage1, dim3(grid), dim3(64 * kPW), lds_router > lds_gu ? lds_router : lds_gu, s, a);
    return hipGetLastError();
}

// Router logits only (the stage-1 router workgroups), for moe_route on a few tokens.
hipError_t launch_dec_router(const moe_layer *L, const uint16_t *x, int T, float *logits, hipStream_t s) {
    const moe_dims &D = L->dims;
    DecArgs a = dec_args(L, x, T, nullptr);
    a.logits = logits;
    const size_t lds = sizeof(float) * kRW * T * (D.d_model / 64);
    hipLaunchKernelGGL(k_dec_stage1, dim3(cdiv(D.n_experts, kRW)), dim3(64 * kPW), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_dec_stage2(const moe_layer *L, const uint16_t *x, int T, hipStream_t s) {
    const moe_dims &D = L->dims;
    const DecArgs a = dec_args(L, x, T, nullptr);
    const int grid = T * D.top_k * (D.d_expert / 32) + T * (D.d_model / 32) * a.KSs;
    const size_t lds_gu = sizeof(uint16_t) * (D.d_model < 64 * kW2 * kB2 ? D.d_model : 64 * kW2 * kB2) +
                          sizeof(float) * (64 + kW2 * 2 * 32 + 2 * 64 * kW2 + 64);
    const size_t lds_sd = sizeof(uint16_t) * 64 * kGPS + sizeof(float) * kW2 * 32;
    const size_t lds = lds_gu > lds_sd ? lds_gu : lds_sd;
    if (D.n_experts <= 128) hipLaunchKernelGGL(k_dec_stage2<2>, dim3(grid), dim3(64 * kW2), lds, s, a);
    else if (D.n_experts <= 256) hipLaunchKernelGGL(k_dec_stage2<4>, dim3(grid), dim3(64 * kW2), lds, s, a);
    else hipLaunchKernelGGL(k_dec_stage2<MOE_MAX_EXPERTS / 64>, dim3(grid), dim3(64 * kW2), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_dec_stage3(const moe_layer *L, int T, float *y, hipStream_t s) {
    const moe_dims &D = L->dims;
    const DecArgs a = dec_args(L, nullptr, T, y);
    if (D.top_k <= 8)
        hipLaunchKernelGGL(k_dec_stage3<8>, dim3(T * (D.d_model / 32)), dim3(64 * D.top_k), dec_stage3_lds(D), s, a);
    else
        hipLaunchKernelGGL(k_dec_stage3<MOE_MAX_TOP_K>, dim3(T * (D.d_model / 32)), dim3(64 * D.top_k),
                           dec_stage3_lds(D), s, a);
    return hipGetLastError();
}

}  // namespace qmoe
