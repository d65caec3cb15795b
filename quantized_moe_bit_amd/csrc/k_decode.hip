// Decode path (a few tokens): wavefront GEMV kernels over 4-bit group-64 weights.
//
// Each selected expert is a GELU-gated FFN (gate, up, tanh-GELU, down) whose weights
// are affine-quantized: w = scale * q + bias per group of 64 inputs (Mference system
// design, "Why the runtime has this shape"; "Metal execution": decode uses custom
// affine INT4 GEMV kernels that consume packed codes and BF16 scale/bias directly, and
// the routed kernels fuse the affine decode, GeGLU and the weighted reduction).
//
// Per group the dot product is split exactly as
//   sum_j x_j (s q_j + b) = 16 s * sum_j x_j (1 + q_j/16) + (b - 16 s) * X_g,
// where X_g = sum_j x_j. The bf16 values 1 + q/16 come from the nibbles with a shift and
// an and-or, and v_dot2_f32_bf16 accumulates x * (1 + q/16) in fp32.
//
// Kernels:
//   k_dec_gateup: one workgroup per (pair or shared token, 32-row block of the expert
//     width); streams the gate and up tiles, writes h = fp16(gelu(g) * u) and the sums
//     of each 32 consecutive h values (for the down projection's bias term). The down
//     projection reads h with v_dot2_f32_f16 against fp16 values 1 + q/16.
//   k_dec_down: one wave per (token, part, 32 output rows); a part is one routed slot
//     or one chunk of the shared expert's input groups. Each wave writes its partial
//     rows; the last wave to arrive for a (token, row block) adds the shared parts, then
//     the routed slots weighted by their routing weights in slot order 0..k-1 (Mference,
//     "Decode", cb2; fixed reduction order as in TinyTitan, "Invariants").
#include "device_common.h"
#include "moe_internal.h"

namespace qmoe {
namespace {

constexpr int kGUWaves = 8;     // waves per gate/up workgroup
constexpr int kGUBatch = 6;     // groups whose tiles a wave loads before computing

// grid: T*k*(I/32) + T*(I_s/32); block 64*kGUWaves
__global__ __launch_bounds__(64 * kGUWaves) void k_dec_gateup(
    const uint16_t *__restrict__ x, int T, int d, int k, int I, int Is, const int32_t *__restrict__ idx,
    const float *__restrict__ xsum, moe_qmat gate, moe_qmat up, moe_qmat sh_gate, moe_qmat sh_up,
    uint16_t *__restrict__ h_r, uint16_t *__restrict__ h_s, float *__restrict__ hsum_r, float *__restrict__ hsum_s) {
    __shared__ __align__(16) uint16_t xs[8192];
    __shared__ float red[kGUWaves][2][32];
    __shared__ float hv[32];
    const int G = d / 64;
    const int JB = I / 32, JBs = Is / 32;
    int u = blockIdx.x;
    const uint8_t *Wg, *Wu;
    const uint32_t *Sg, *Su;
    uint16_t *hout;
    float *hsum;
    int t, jb;
    if (u < T * k * JB) {
        const int p = u / JB;
        jb = u % JB;
        t = p / k;
        const int e = idx[p];
        const size_t cstride = (size_t)I * d / 2, sstride = (size_t)I * G;
        Wg = static_cast<const uint8_t *>(gate.codes) + e * cstride;
        Wu = static_cast<const uint8_t *>(up.codes) + e * cstride;
        Sg = gate.sb + e * sstride;
        Su = up.sb + e * sstride;
        hout = h_r + (size_t)p * I;
        hsum = hsum_r + (size_t)p * JB;
    } else {
        u -= T * k * JB;
        t = u / JBs;
        jb = u % JBs;
        Wg = static_cast<const uint8_t *>(sh_gate.codes);
        Wu = static_cast<const uint8_t *>(sh_up.codes);
        Sg = sh_gate.sb;
        Su = sh_up.sb;
        hout = h_s + (size_t)t * Is;
        hsum = hsum_s + (size_t)t * JBs;
    }
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, n = lane & 31, half = lane >> 5;
    const float *X = xsum + (size_t)t * G;
    Wg += (size_t)jb * G * 1024 + lane * 16;
    Wu += (size_t)jb * G * 1024 + lane * 16;
    Sg += (size_t)jb * G * 32 + n;
    Su += (size_t)jb * G * 32 + n;
    float accg = 0.0f, accu = 0.0f;
    // every wave runs the same number of iterations, so the barrier below is uniform
    for (int gb0 = 0; gb0 < G; gb0 += kGUWaves * kGUBatch) {
        const int gb = gb0 + wave;
        u32x4_t wg[kGUBatch], wu[kGUBatch];
        uint32_t sbg[kGUBatch], sbu[kGUBatch];
#pragma unroll
        for (int b = 0; b < kGUBatch; ++b) {
            const int g = gb + b * kGUWaves;
            if (g < G) {
                wg[b] = ld16(Wg + (size_t)g * 1024);
                wu[b] = ld16(Wu + (size_t)g * 1024);
                sbg[b] = Sg[g * 32];
                sbu[b] = Su[g * 32];
            }
        }
        if (gb0 == 0)
            for (int i = tid; i < d / 8; i += 64 * kGUWaves)
                *reinterpret_cast<u32x4_t *>(xs + 8 * i) = ld16(x + (size_t)t * d + 8 * i);
        __syncthreads();
#pragma unroll
        for (int b = 0; b < kGUBatch; ++b) {
            const int g = gb + b * kGUWaves;
            if (g < G) {
                float ag = 0.0f, au = 0.0f;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const u32x4_t xv = *reinterpret_cast<const u32x4_t *>(xs + 64 * g + 16 * s + 8 * half);
                    ag = dot2_bf16(xv[0], nib_pair<0>(wg[b][s]), ag);
                    ag = dot2_bf16(xv[1], nib_pair<1>(wg[b][s]), ag);
                    ag = dot2_bf16(xv[2], nib_pair<2>(wg[b][s]), ag);
                    ag = dot2_bf16(xv[3], nib_pair<3>(wg[b][s]), ag);
                    au = dot2_bf16(xv[0], nib_pair<0>(wu[b][s]), au);
                    au = dot2_bf16(xv[1], nib_pair<1>(wu[b][s]), au);
                    au = dot2_bf16(xv[2], nib_pair<2>(wu[b][s]), au);
                    au = dot2_bf16(xv[3], nib_pair<3>(wu[b][s]), au);
                }
                const float s16g = 16.0f * bf16_to_f32(sbg[b] & 0xFFFFu);
                const float s16u = 16.0f * bf16_to_f32(sbu[b] & 0xFFFFu);
                accg = fmaf(s16g, ag, accg);
                accu = fmaf(s16u, au, accu);
                if (half == 0) {
                    const float Xg = X[g];
                    accg = fmaf(bf16_to_f32(sbg[b] >> 16) - s16g, Xg, accg);
                    accu = fmaf(bf16_to_f32(sbu[b] >> 16) - s16u, Xg, accu);
                }
            }
        }
    }
    accg += __shfl_xor(accg, 32);
    accu += __shfl_xor(accu, 32);
    if (lane < 32) {
        red[wave][0][n] = accg;
        red[wave][1][n] = accu;
    }
    __syncthreads();
    if (tid < 32) {
        float gv = 0.0f, uv = 0.0f;
        for (int w = 0; w < kGUWaves; ++w) {
            gv += red[w][0][tid];
            uv += red[w][1][tid];
        }
        const uint32_t hb = f32_to_f16_sat(gelu_tanh_f32(gv) * uv);
        hout[jb * 32 + tid] = (uint16_t)hb;
        hv[tid] = f16_to_f32(hb);
    }
    __syncthreads();
    if (tid == 0) {
        float s = 0.0f;
        for (int i = 0; i < 32; ++i) s += hv[i];
        hsum[jb] = s;
    }
}

// grid: T * NP * (d/32); block 64
__global__ __launch_bounds__(64) void k_dec_down(int T, int d, int k, int I, int Is, int nR, int nS,
                                                 const int32_t *__restrict__ idx, const float *__restrict__ wts,
                                                 moe_qmat down, moe_qmat sh_down, const uint16_t *__restrict__ h_r,
                                                 const uint16_t *__restrict__ h_s, const float *__restrict__ hsum_r,
                                                 const float *__restrict__ hsum_s, float *__restrict__ part,
                                                 uint32_t *__restrict__ counter, float *__restrict__ y) {
    __shared__ __align__(16) uint16_t hl[kDecodeChunkGroups * 64];
    const int RB = d / 32, NP = k * nR + nS;
    int u = blockIdx.x;
    const int rb = u % RB;
    u /= RB;
    const int pidx = u % NP;
    const int t = u / NP;
    const int GI = I / 64, GIs = Is / 64;
    const uint8_t *W;
    const uint32_t *S;
    const uint16_t *hin;
    const float *hs;
    int Gk, g0, g1;
    if (pidx < k * nR) {
        const int slot = pidx / nR, c = pidx % nR;
        const int p = t * k + slot;
        const int e = idx[p];
        W = static_cast<const uint8_t *>(down.codes) + (size_t)e * d * I / 2;
        S = down.sb + (size_t)e * d * GI;
        hin = h_r + (size_t)p * I;
        hs = hsum_r + (size_t)p * (I / 32);
        Gk = GI;
        g0 = c * kDecodeChunkGroups;
        g1 = min(GI, g0 + kDecodeChunkGroups);
    } else {
        const int c = pidx - k * nR;
        W = static_cast<const uint8_t *>(sh_down.codes);
        S = sh_down.sb;
        hin = h_s + (size_t)t * Is;
        hs = hsum_s + (size_t)t * (Is / 32);
        Gk = GIs;
        g0 = c * kDecodeChunkGroups;
        g1 = min(GIs, g0 + kDecodeChunkGroups);
    }
    const int lane = threadIdx.x, n = lane & 31, half = lane >> 5;
    const int ng = g1 - g0;
    W += ((size_t)rb * Gk + g0) * 1024 + lane * 16;
    S += ((size_t)rb * Gk + g0) * 32 + n;
    u32x4_t w4[kDecodeChunkGroups];
    uint32_t sbw[kDecodeChunkGroups];
#pragma unroll
    for (int b = 0; b < kDecodeChunkGroups; ++b)
        if (b < ng) {
            w4[b] = ld16(W + (size_t)b * 1024);
            sbw[b] = S[b * 32];
        }
    for (int i = lane; i < ng * 8; i += 64)
        *reinterpret_cast<u32x4_t *>(hl + 8 * i) = ld16(hin + 64 * g0 + 8 * i);
    __syncthreads();
    float acc = 0.0f;
#pragma unroll
    for (int b = 0; b < kDecodeChunkGroups; ++b)
        if (b < ng) {
            float a = 0.0f;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4_t hv = *reinterpret_cast<const u32x4_t *>(hl + 64 * b + 16 * s + 8 * half);
                a = dot2_f16(hv[0], nib_pair_f16<0>(w4[b][s]), a);
                a = dot2_f16(hv[1], nib_pair_f16<1>(w4[b][s]), a);
                a = dot2_f16(hv[2], nib_pair_f16<2>(w4[b][s]), a);
                a = dot2_f16(hv[3], nib_pair_f16<3>(w4[b][s]), a);
            }
            const float s16 = 16.0f * bf16_to_f32(sbw[b] & 0xFFFFu);
            acc = fmaf(s16, a, acc);
            if (half == 0) {
                const int g = g0 + b;
                acc = fmaf(bf16_to_f32(sbw[b] >> 16) - s16, hs[2 * g] + hs[2 * g + 1], acc);
            }
        }
    acc += __shfl_xor(acc, 32);
    const int row = rb * 32 + n;
    if (lane < 32) part[((size_t)t * NP + pidx) * d + row] = acc;
    __threadfence();
    uint32_t old = 0;
    if (lane == 0) old = atomicAdd(&counter[(size_t)t * RB + rb], 1u);
    old = __shfl(old, 0);
    if (old != (uint32_t)(NP - 1)) return;
    __threadfence();
    if (lane < 32) {
        const float *pt = part + (size_t)t * NP * d + row;
        float sh = 0.0f;
        for (int c = 0; c < nS; ++c) sh += __builtin_nontemporal_load(pt + (size_t)(k * nR + c) * d);
        float out = sh;
        for (int s = 0; s < k; ++s) {
            float r = 0.0f;
            for (int c = 0; c < nR; ++c) r += __builtin_nontemporal_load(pt + (size_t)(s * nR + c) * d);
            out = fmaf(wts[(size_t)t * k + s], r, out);
        }
        y[(size_t)t * d + row] = out;
    }
    if (lane == 0) counter[(size_t)t * RB + rb] = 0u;
}

}  // namespace

hipError_t launch_dec_gateup(const moe_layer *L, const uint16_t *x, int T, hipStream_t s) {
    const moe_dims &D = L->dims;
    const int units = T * D.top_k * (D.d_expert / 32) + T * (D.d_shared / 32);
    hipLaunchKernelGGL(k_dec_gateup, dim3(units), dim3(64 * kGUWaves), 0, s, x, T, D.d_model, D.top_k, D.d_expert,
                       D.d_shared, L->ws.idx, L->ws.xsum, L->w.gate, L->w.up, L->w.sh_gate, L->w.sh_up, L->ws.dh_r,
                       L->ws.dh_s, L->ws.dhsum_r, L->ws.dhsum_s);
    return hipGetLastError();
}

hipError_t launch_dec_down(const moe_layer *L, int T, float *y, hipStream_t s) {
    const moe_dims &D = L->dims;
    const int NP = D.top_k * L->dec_parts_r + L->dec_parts_s;
    const int units = T * NP * (D.d_model / 32);
    hipLaunchKernelGGL(k_dec_down, dim3(units), dim3(64), 0, s, T, D.d_model, D.top_k, D.d_expert, D.d_shared,
                       L->dec_parts_r, L->dec_parts_s, L->ws.idx, L->ws.wts, L->w.down, L->w.sh_down, L->ws.dh_r,
                       L->ws.dh_s, L->ws.dhsum_r, L->ws.dhsum_s, L->ws.dpart, L->ws.dcount, y);
    return hipGetLastError();
}

}  // namespace qmoe
