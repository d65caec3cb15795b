// Prefill path: grouped GEMM over expert-bucketed token rows on gfx950 MFMA.
//
// Token/expert pairs of a chunk are grouped by expert (Mference system design,
// "Prefill"); each expert's rows then form one dense GEMM against its 4-bit
// group-64 affine weights. The Mference design unpacks an affine tile into bounded
// FP16 staging and hands it to a matrix unit ("Prefill"; "Metal execution"); here the
// codes become bf16 MFMA operands directly in registers.
//
// Exact affine split per 64-input group g of output n:
//   sum_j x_j (s q_j + b) = 16 s * A''_g + (b - 16 s) * X_g,   A''_g = sum_j x_j (1 + q_j/16)
// A''_g comes from four 32x32x16 MFMA steps with fp32 accumulation: bf16 for the gate/up
// projections (x is bf16; 1 + q/16 is exact in bf16), fp16 for the down projection, whose
// input, the hidden activation h = gelu(g) * u, is carried in fp16 (11 significant bits;
// the Mference prefill likewise stages FP16 tensors for its matrix unit). 16 s is applied
// per group on the VALU. The (b - 16 s) X_g terms for
// all groups form a small GEMM with K = 3 * Gp (Gp = groups padded to 16) done on MFMA
// after the main loop, with both factors split into bf16 hi + lo parts:
//   c X ~= c_hi X_hi + c_hi X_lo + c_lo X_hi.
//
// Work items: (expert or shared, 128-row tile, output tile). A persistent grid walks them
// with a static schedule: items are cut into 8 contiguous ranges, one per XCD (workgroup
// i runs on XCD i % 8), so all tiles of one expert share an L2.
#include "device_common.h"
#include "moe_internal.h"

namespace qmoe {
namespace {

constexpr int kAPitch = 72;   // bf16 per staged A row in LDS (64 + 8 pad: conflict-free 16 B reads)
constexpr int kPreWG = 256;

struct PreArgs {
    int T, d, k, I, Is, E;
    const uint16_t *x;          // gate/up A rows [T, d]
    const int32_t *perm, *offsets, *tile_off;
    const uint16_t *xsplit;     // [T, 3 Gp_d]
    moe_qmat gate, up, sh_gate, sh_up, down, sh_down;
    uint16_t *h_r, *hsplit_r, *h_s, *hsplit_s;
    int Gp_d, Gp_I, Gp_Is;
    float *r, *sh;
    const uint8_t *bt_gate, *bt_up, *bt_down, *bt_sh_gate, *bt_sh_up, *bt_sh_down;   // bias-term B' tables
};

__device__ __forceinline__ int find_expert(const int32_t *tile_off, int E, int m) {
    int lo = 0, hi = E;  // tile_off[lo] <= m < tile_off[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tile_off[mid] <= m) lo = mid;
        else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16_t mfma32(f16x8_t a, f16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// MFMA operand type: bf16 for the gate/up projections (x is bf16), fp16 for the down
// projection (the hidden activation is carried in fp16).
template <int MODE> struct OpT;
template <> struct OpT<0> {
    typedef bf16x8_t type;
    static __device__ __forceinline__ type frag(uint32_t w) { return nib_frag(w); }
};
template <> struct OpT<1> {
    typedef f16x8_t type;
    static __device__ __forceinline__ type frag(uint32_t w) { return nib_frag_f16(w); }
};

// c = bias - 16*scale as bf16 hi (part 0, 1) or lo (part 2) for the bias-term GEMM.
__device__ __forceinline__ uint32_t bias_part(uint32_t sbw, int part) {
    const float c = bf16_to_f32(sbw >> 16) - 16.0f * bf16_to_f32(sbw & 0xFFFFu);
    const uint32_t hi = f32_to_bf16(c);
    if (part < 2) return hi;
    return f32_to_bf16(c - bf16_to_f32(hi));
}

template <int MODE>  // 0: gate/up + GeGLU, 1: down
__global__ __launch_bounds__(kPreWG, 2) void k_pre_gemm(PreArgs a) {
    __shared__ __align__(16) uint16_t As[2][kMT * kAPitch];
    __shared__ __align__(16) uint16_t Bs[2][4 * 512];   // four 1 KiB weight tiles (codes) per group
    __shared__ int32_t srow[kMT];   // A source row (-1: padding)
    __shared__ int32_t drow[kMT];   // destination row

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1, n = lane & 31, half = lane >> 5;
    const int E = a.E;

    // item space
    const int Ms = cdiv(a.T, kMT);
    const int NTs = MODE == 0 ? a.Is / 64 : a.d / 128;
    const int NTr = MODE == 0 ? a.I / 64 : a.d / 128;
    const int S_items = Ms * NTs;
    const int N = S_items + a.tile_off[E] * NTr;
    const int nwg = gridDim.x, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per_xcd = nwg >> 3;
    const int lo = (int)((long long)N * xcd / 8), hi = (int)((long long)N * (xcd + 1) / 8);

    for (int item = lo + slot; item < hi; item += per_xcd) {
        bool shared_item;
        int e = 0, mt, nt, count, rowbase;
        if (item < S_items) {
            shared_item = true;
            mt = item / NTs;
            nt = item % NTs;
            count = a.T;
            rowbase = 0;
        } else {
            shared_item = false;
            const int j = item - S_items;
            const int mg = j / NTr;
            nt = j % NTr;
            e = find_expert(a.tile_off, E, mg);
            mt = mg - a.tile_off[e];
            rowbase = a.offsets[e];
            count = a.offsets[e + 1] - rowbase;
        }
        const int K = MODE == 0 ? a.d : (shared_item ? a.Is : a.I);
        const int G = K / 64;
        const int Gp = MODE == 0 ? a.Gp_d : (shared_item ? a.Gp_Is : a.Gp_I);
        const uint16_t *Asrc;
        const uint16_t *Bsrc;   // split sums for the bias-term GEMM
        if (MODE == 0) {
            Asrc = a.x;
            Bsrc = a.xsplit;
        } else {
            Asrc = shared_item ? a.h_s : a.h_r;
            Bsrc = shared_item ? a.hsplit_s : a.hsplit_r;
        }

        __syncthreads();   // previous item is done with the LDS tables
        if (tid < kMT) {
            const int r = mt * kMT + tid;
            int src = -1, dst = -1;
            if (r < count) {
                if (shared_item) {
                    src = r;
                    dst = r;
                } else {
                    dst = rowbase + r;
                    src = MODE == 0 ? a.perm[dst] / a.k : dst;
                }
            }
            srow[tid] = src;
            drow[tid] = dst;
        }
        __syncthreads();

        // The workgroup's four weight tiles per input group (32 rows each): gate/up -> gate
        // blocks 2nt, 2nt+1 then up blocks 2nt, 2nt+1; down -> blocks 4nt .. 4nt+3. Wave (wm, wn)
        // uses tiles t0 = wn and t1 = 2 + wn (gate/up) or t0 = 2wn, t1 = 2wn + 1 (down).
        const int t0 = MODE == 0 ? wn : 2 * wn, t1 = MODE == 0 ? 2 + wn : 2 * wn + 1;
        const uint8_t *Bt;        // this thread's copy source: tile tid/64, 16 B at lane tid%64
        const uint32_t *S0, *S1;  // scale/bias words of the wave's two tiles
        {
            const moe_qmat *mg = MODE == 0 ? (shared_item ? &a.sh_gate : &a.gate) : (shared_item ? &a.sh_down : &a.down);
            const moe_qmat *mu = MODE == 0 ? (shared_item ? &a.sh_up : &a.up) : mg;
            const int rows = MODE == 0 ? (shared_item ? a.Is : a.I) : a.d;
            const size_t cstride = (size_t)rows * K / 2, sstride = (size_t)rows * G;
            auto rb_of = [&](int ti) { return MODE == 0 ? nt * 2 + (ti & 1) : nt * 4 + ti; };
            auto mat_of = [&](int ti) { return (MODE == 0 && ti >= 2) ? mu : mg; };
            const int ti = tid >> 6;
            Bt = static_cast<const uint8_t *>(mat_of(ti)->codes) + e * cstride + (size_t)rb_of(ti) * G * 1024 +
                 (tid & 63) * 16;
            S0 = mat_of(t0)->sb + e * sstride + (size_t)rb_of(t0) * G * 32 + n;
            S1 = mat_of(t1)->sb + e * sstride + (size_t)rb_of(t1) * G * 32 + n;
        }

        // 2-deep pipeline: register sets hold groups g+1 and g+2 while group g computes from LDS.
        // A staging: thread covers 4 pieces of 16 B (row q/8, column chunk q%8), q = tid + 256 i.
        u32x4_t ra0[4], ra1[4], rb0, rb1;
        auto fetch = [&](int g, u32x4_t(&ra)[4], u32x4_t &rbv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = tid + kPreWG * i;
                const int src = srow[q >> 3];
                ra[i] = src >= 0 ? ld16(Asrc + (size_t)src * K + 64 * g + 8 * (q & 7)) : u32x4_t{0u, 0u, 0u, 0u};
            }
            rbv = ld16(Bt + (size_t)g * 1024);
        };
        auto put = [&](int buf, const u32x4_t(&ra)[4], const u32x4_t &rbv) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = tid + kPreWG * i;
                *reinterpret_cast<u32x4_t *>(&As[buf][(q >> 3) * kAPitch + 8 * (q & 7)]) = ra[i];
            }
            *reinterpret_cast<u32x4_t *>(&Bs[buf][tid * 8]) = rbv;
        };

        f32x16_t tot[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) tot[i][j][v] = 0.0f;
        const f32x16_t zero = tot[0][0];

        // 32-row subtiles of this wave that hold at least one real row (wave-uniform)
        const int live_rows = count - mt * kMT - wm * 64;
        const bool live0 = live_rows > 0, live1 = live_rows > 32;
        auto compute = [&](int buf, uint32_t sb0, uint32_t sb1) {
            typedef typename OpT<MODE>::type op_t;
            if (!live0) return;
            const u32x4_t bw0 = *reinterpret_cast<const u32x4_t *>(&Bs[buf][(t0 * 64 + lane) * 8]);
            const u32x4_t bw1 = *reinterpret_cast<const u32x4_t *>(&Bs[buf][(t1 * 64 + lane) * 8]);
            f32x16_t acc[2][2];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const op_t b0 = OpT<MODE>::frag(bw0[s]);
                const op_t b1 = OpT<MODE>::frag(bw1[s]);
#pragma unroll
                for (int ms = 0; ms < 2; ++ms) {
                    if (ms == 1 && !live1) continue;
                    const int row = wm * 64 + ms * 32 + n;
                    const op_t av = __builtin_bit_cast(
                        op_t, *reinterpret_cast<const u32x4_t *>(&As[buf][row * kAPitch + 16 * s + 8 * half]));
                    acc[ms][0] = mfma32(av, b0, s == 0 ? zero : acc[ms][0]);
                    acc[ms][1] = mfma32(av, b1, s == 0 ? zero : acc[ms][1]);
                }
            }
            const float s16_0 = 16.0f * bf16_to_f32(sb0 & 0xFFFFu);
            const float s16_1 = 16.0f * bf16_to_f32(sb1 & 0xFFFFu);
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
                if (ms == 1 && !live1) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    tot[ms][0][v] = fmaf(s16_0, acc[ms][0][v], tot[ms][0][v]);
                    tot[ms][1][v] = fmaf(s16_1, acc[ms][1][v], tot[ms][1][v]);
                }
            }
        };

        fetch(0, ra0, rb0);
        if (G > 1) fetch(1, ra1, rb1);
        uint32_t sc0 = S0[0], sc1 = S1[0];
        uint32_t sn0 = G > 1 ? S0[32] : 0u, sn1 = G > 1 ? S1[32] : 0u;
        put(0, ra0, rb0);
        __syncthreads();
        for (int g = 0; g < G; g += 2) {
            // even step: group g from buffer 0; ra0 refills with g+2; ra1 (g+1) goes to buffer 1
            if (g + 2 < G) fetch(g + 2, ra0, rb0);
            compute(0, sc0, sc1);
            if (g + 1 < G) put(1, ra1, rb1);
            sc0 = sn0;
            sc1 = sn1;
            if (g + 2 < G) {
                sn0 = S0[(g + 2) * 32];
                sn1 = S1[(g + 2) * 32];
            }
            __syncthreads();
            if (g + 1 >= G) break;
            // odd step: group g+1 from buffer 1; ra1 refills with g+3; ra0 (g+2) goes to buffer 0
            if (g + 3 < G) fetch(g + 3, ra1, rb1);
            compute(1, sc0, sc1);
            if (g + 2 < G) put(0, ra0, rb0);
            sc0 = sn0;
            sc1 = sn1;
            if (g + 3 < G) {
                sn0 = S0[(g + 3) * 32];
                sn1 = S1[(g + 3) * 32];
            }
            __syncthreads();
        }

        // bias-term GEMM: K' = 3 Gp; A' = [X_hi | X_lo | X_hi], B' = [c_hi | c_hi | c_lo] with
        // c = bias - 16 scale. B' fragments come from the table built at layer creation.
        if (live0) {
            const int steps = 3 * Gp / 16;
            const uint8_t *T0, *T1;
            {
                const uint8_t *tg = MODE == 0 ? (shared_item ? a.bt_sh_gate : a.bt_gate)
                                              : (shared_item ? a.bt_sh_down : a.bt_down);
                const uint8_t *tu = MODE == 0 ? (shared_item ? a.bt_sh_up : a.bt_up) : tg;
                const int rows = MODE == 0 ? (shared_item ? a.Is : a.I) : a.d;
                const size_t estride = (size_t)(rows / 32) * steps * 1024;
                auto rb_of = [&](int ti) { return MODE == 0 ? nt * 2 + (ti & 1) : nt * 4 + ti; };
                T0 = ((MODE == 0 && t0 >= 2) ? tu : tg) + e * estride + (size_t)rb_of(t0) * steps * 1024 + lane * 16;
                T1 = ((MODE == 0 && t1 >= 2) ? tu : tg) + e * estride + (size_t)rb_of(t1) * steps * 1024 + lane * 16;
            }
            const int src0 = srow[wm * 64 + n], src1 = srow[wm * 64 + 32 + n];
            for (int st = 0; st < steps; ++st) {
                const int kk0 = 16 * st + 8 * half;
                const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, ld16(T0 + (size_t)st * 1024));
                const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, ld16(T1 + (size_t)st * 1024));
#pragma unroll
                for (int ms = 0; ms < 2; ++ms) {
                    if (ms == 1 && !live1) continue;
                    u32x4_t av = u32x4_t{0u, 0u, 0u, 0u};
                    const int sr = ms == 0 ? src0 : src1;
                    if (sr >= 0) av = ld16(Bsrc + (size_t)sr * 3 * Gp + kk0);
                    const bf16x8_t avb = __builtin_bit_cast(bf16x8_t, av);
                    tot[ms][0] = mfma32(avb, b0, tot[ms][0]);
                    tot[ms][1] = mfma32(avb, b1, tot[ms][1]);
                }
            }
        }

        // epilogue. Accumulator element v of lane l: row 8*(v/4) + 4*(l/32) + v%4, column l%32.
        if (MODE == 0) {
            // h = fp16(gelu(g) * u) into an LDS tile [128 rows][64 columns] (reusing As[0]), then
            // each row leaves as 16-byte stores and its 64-column sum feeds the down bias term
            const int J = shared_item ? a.Is : a.I;
            uint16_t *hout = shared_item ? a.h_s : a.h_r;
            uint16_t *Hs = As[0];
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = wm * 64 + ms * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                    Hs[row * kAPitch + wn * 32 + n] =
                        (uint16_t)f32_to_f16_sat(gelu_tanh_f32(tot[ms][0][v]) * tot[ms][1][v]);
                }
            __syncthreads();
            const int row = tid >> 1, hh = tid & 1;
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(Hs + row * kAPitch + hh * 32);
            u32x4_t hv[4];
            float hsum_part = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                hv[i] = src[i];
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    hsum_part += f16_to_f32(hv[i][w] & 0xFFFFu) + f16_to_f32(hv[i][w] >> 16);
            }
            const float H = hsum_part + __shfl_xor(hsum_part, 1);
            const int dst = drow[row];
            if (dst >= 0) {
                u32x4_t *o = reinterpret_cast<u32x4_t *>(hout + (size_t)dst * J + nt * 64 + hh * 32);
#pragma unroll
                for (int i = 0; i < 4; ++i) o[i] = hv[i];
                if (hh == 0) {
                    const int Gpo = shared_item ? a.Gp_Is : a.Gp_I;
                    uint16_t *hs = (shared_item ? a.hsplit_s : a.hsplit_r) + (size_t)dst * 3 * Gpo;
                    const uint32_t hi = f32_to_bf16(H);
                    const uint32_t lo = f32_to_bf16(H - bf16_to_f32(hi));
                    hs[nt] = (uint16_t)hi;
                    hs[Gpo + nt] = (uint16_t)lo;
                    hs[2 * Gpo + nt] = (uint16_t)hi;
                }
            }
        } else {
            float *out = shared_item ? a.sh : a.r;
            const int c0 = (nt * 4 + wn * 2) * 32 + n;
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = wm * 64 + ms * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                    const int dst = drow[row];
                    if (dst >= 0) {
                        out[(size_t)dst * a.d + c0] = tot[ms][0][v];
                        out[(size_t)dst * a.d + c0 + 32] = tot[ms][1][v];
                    }
                }
        }
    }
}

// Bias-term B' fragments of one quantized matrix stack (n_mats x [rows, in]): for each
// (matrix, 32-row block rb, 16-step st, lane l) eight bf16 values for K' indices
// kk = 16 st + 8 (l / 32) + j, j = 0..7, of row rb*32 + l%32: with part = kk / Gp and
// g = kk % Gp, c = bias - 16 scale of group g, value c_hi (part 0, 1) or c_lo (part 2),
// 0 for padding groups g >= G. grid: ceil(n_mats * rows/32 * steps * 64 / 256); block 256
__global__ __launch_bounds__(256) void k_bias_table(const uint32_t *__restrict__ sb, int n_mats, int rows, int G,
                                                    int Gp, uint8_t *__restrict__ out) {
    const int steps = 3 * Gp / 16;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t total = (size_t)n_mats * (rows / 32) * steps * 64;
    if (i >= total) return;
    const int lane = (int)(i % 64);
    size_t r = i / 64;
    const int st = (int)(r % steps);
    r /= steps;
    const int rb = (int)(r % (rows / 32));
    const size_t m = r / (rows / 32);
    const uint32_t *sbm = sb + m * (size_t)rows * G + (size_t)rb * G * 32 + (lane & 31);
    uint32_t w[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        uint32_t v2[2];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int kk = 16 * st + 8 * (lane >> 5) + 2 * jj + h2;
            const int part = kk / Gp, gg = kk % Gp;
            v2[h2] = gg < G ? bias_part(sbm[gg * 32], part) : 0u;
        }
        w[jj] = v2[0] | (v2[1] << 16);
    }
    *reinterpret_cast<u32x4_t *>(out + i * 16) = u32x4_t{w[0], w[1], w[2], w[3]};
}

// y[t] = sh[t] + sum_s w[t,s] * r[pos[t*k+s]] in slot order. grid (cdiv(d,1024), T); block 256
__global__ __launch_bounds__(256) void k_combine(int d, int k, const float *__restrict__ sh,
                                                 const float *__restrict__ r, const int32_t *__restrict__ pos,
                                                 const float *__restrict__ wts, float *__restrict__ y) {
    const int t = blockIdx.y;
    const int c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= d) return;
    f32x4_t acc = *reinterpret_cast<const f32x4_t *>(sh + (size_t)t * d + c);
    for (int s = 0; s < k; ++s) {
        const float w = wts[(size_t)t * k + s];
        const f32x4_t rv = *reinterpret_cast<const f32x4_t *>(r + (size_t)pos[(size_t)t * k + s] * d + c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, rv[i], acc[i]);
    }
    *reinterpret_cast<f32x4_t *>(y + (size_t)t * d + c) = acc;
}

// Residual stream between stacked layers. grid T; block 256
__global__ __launch_bounds__(256) void k_glue(const uint16_t *h, const float *y, uint16_t *h_next,
                                              uint16_t *x_next, int d) {
    __shared__ float red[256];
    const int t = blockIdx.x, tid = threadIdx.x;
    float ss = 0.0f;
    for (int i = tid; i < d; i += 256) {
        const size_t o = (size_t)t * d + i;
        float v = bf16_to_f32(h[o]);
        if (y) v = v + y[o];
        const uint32_t b = f32_to_bf16(v);
        h_next[o] = (uint16_t)b;
        const float hv = bf16_to_f32(b);
        ss = fmaf(hv, hv, ss);
    }
    red[tid] = ss;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
        if (tid < w) red[tid] += red[tid + w];
        __syncthreads();
    }
    const float inv = 1.0f / sqrtf(red[0] / (float)d + 1e-6f);
    for (int i = tid; i < d; i += 256) {
        const size_t o = (size_t)t * d + i;
        x_next[o] = (uint16_t)f32_to_bf16(bf16_to_f32(h_next[o]) * inv);
    }
}

PreArgs make_args(const moe_layer *L, const uint16_t *x, int T) {
    PreArgs a;
    const moe_dims &D = L->dims;
    a.T = T;
    a.d = D.d_model;
    a.k = D.top_k;
    a.I = D.d_expert;
    a.Is = D.d_shared;
    a.E = D.n_experts;
    a.x = x;
    a.perm = L->ws.perm;
    a.offsets = L->ws.offsets;
    a.tile_off = L->ws.tile_off;
    a.xsplit = L->ws.xsplit;
    a.gate = L->w.gate;
    a.up = L->w.up;
    a.sh_gate = L->w.sh_gate;
    a.sh_up = L->w.sh_up;
    a.down = L->w.down;
    a.sh_down = L->w.sh_down;
    a.h_r = L->ws.h_r;
    a.hsplit_r = L->ws.hsplit_r;
    a.h_s = L->ws.h_s;
    a.hsplit_s = L->ws.hsplit_s;
    a.Gp_d = L->Gp_d;
    a.Gp_I = L->Gp_I;
    a.Gp_Is = L->Gp_Is;
    a.r = L->ws.r;
    a.sh = L->ws.sh;
    a.bt_gate = L->ws.bt[0];
    a.bt_up = L->ws.bt[1];
    a.bt_down = L->ws.bt[2];
    a.bt_sh_gate = L->ws.bt[3];
    a.bt_sh_up = L->ws.bt[4];
    a.bt_sh_down = L->ws.bt[5];
    return a;
}

int persistent_grid() {
    static int grid = 0;
    if (!grid) {
        int dev = 0, cus = 256;
        if (hipGetDevice(&dev) == hipSuccess)
            (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        grid = ((cus * 2 + 7) / 8) * 8;
    }
    return grid;
}

}  // namespace

hipError_t launch_pre_gateup(const moe_layer *L, const uint16_t *x, int T, hipStream_t s) {
    hipLaunchKernelGGL(k_pre_gemm<0>, dim3(persistent_grid()), dim3(kPreWG), 0, s, make_args(L, x, T));
    return hipGetLastError();
}

hipError_t launch_pre_down(const moe_layer *L, int T, hipStream_t s) {
    hipLaunchKernelGGL(k_pre_gemm<1>, dim3(persistent_grid()), dim3(kPreWG), 0, s, make_args(L, nullptr, T));
    return hipGetLastError();
}

size_t bias_table_bytes(int n_mats, int rows, int in_dim) {
    const int Gp = roundup(in_dim / 64, 16);
    return (size_t)n_mats * (rows / 32) * (3 * Gp / 16) * 1024;
}

hipError_t launch_bias_table(const moe_qmat &m, int n_mats, int rows, int in_dim, uint8_t *out, hipStream_t s) {
    const int G = in_dim / 64, Gp = roundup(G, 16);
    const size_t total = (size_t)n_mats * (rows / 32) * (3 * Gp / 16) * 64;
    hipLaunchKernelGGL(k_bias_table, dim3((unsigned)cdiv((int)total, 256)), dim3(256), 0, s, m.sb, n_mats, rows, G, Gp,
                       out);
    return hipGetLastError();
}

hipError_t launch_combine(const moe_layer *L, int T, float *y, hipStream_t s) {
    const int d = L->dims.d_model;
    hipLaunchKernelGGL(k_combine, dim3(cdiv(d, 1024), T), dim3(256), 0, s, d, L->dims.top_k, L->ws.sh, L->ws.r,
                       L->ws.pos, L->ws.wts, y);
    return hipGetLastError();
}

hipError_t launch_glue(const uint16_t *h, const float *y, uint16_t *h_next, uint16_t *x_next, int T, int d,
                       hipStream_t s) {
    hipLaunchKernelGGL(k_glue, dim3(T), dim3(256), 0, s, h, y, h_next, x_next, d);
    return hipGetLastError();
}

}  // namespace qmoe
