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
    __shared__ int32_t srow[kMT];   // A source row (-1: padding)
    __shared__ int32_t drow[kMT];   // destination row
    __shared__ float hsum[2][kMT];

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

        // this wave's two weight tiles (32 rows each)
        const uint8_t *B0, *B1;
        const uint32_t *S0, *S1;
        {
            const moe_qmat *m0, *m1;
            int rb0, rb1, rows;
            if (MODE == 0) {
                m0 = shared_item ? &a.sh_gate : &a.gate;
                m1 = shared_item ? &a.sh_up : &a.up;
                rb0 = rb1 = nt * 2 + wn;
                rows = shared_item ? a.Is : a.I;
            } else {
                m0 = m1 = shared_item ? &a.sh_down : &a.down;
                rb0 = nt * 4 + wn * 2;
                rb1 = rb0 + 1;
                rows = a.d;
            }
            const size_t cstride = (size_t)rows * K / 2, sstride = (size_t)rows * G;
            B0 = static_cast<const uint8_t *>(m0->codes) + e * cstride + (size_t)rb0 * G * 1024 + lane * 16;
            B1 = static_cast<const uint8_t *>(m1->codes) + e * cstride + (size_t)rb1 * G * 1024 + lane * 16;
            S0 = m0->sb + e * sstride + (size_t)rb0 * G * 32 + n;
            S1 = m1->sb + e * sstride + (size_t)rb1 * G * 32 + n;
        }

        // A staging: thread covers 4 pieces of 16 B (row q/8, column chunk q%8)
        u32x4_t stage[4];
        auto load_A = [&](int g) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = tid + kPreWG * i;
                const int row = q >> 3, c8 = q & 7;
                const int src = srow[row];
                if (src >= 0) stage[i] = ld16(Asrc + (size_t)src * K + 64 * g + 8 * c8);
                else stage[i] = u32x4_t{0u, 0u, 0u, 0u};
            }
        };
        auto store_A = [&](int buf) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = tid + kPreWG * i;
                const int row = q >> 3, c8 = q & 7;
                *reinterpret_cast<u32x4_t *>(&As[buf][row * kAPitch + 8 * c8]) = stage[i];
            }
        };

        f32x16_t tot[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) tot[i][j][v] = 0.0f;
        const f32x16_t zero = tot[0][0];

        load_A(0);
        u32x4_t bw0 = ld16(B0), bw1 = ld16(B1);
        uint32_t sb0 = S0[0], sb1 = S1[0];
        store_A(0);
        __syncthreads();

        for (int g = 0; g < G; ++g) {
            const int buf = g & 1;
            u32x4_t nb0 = bw0, nb1 = bw1;
            uint32_t ns0 = sb0, ns1 = sb1;
            if (g + 1 < G) {
                load_A(g + 1);
                nb0 = ld16(B0 + (size_t)(g + 1) * 1024);
                nb1 = ld16(B1 + (size_t)(g + 1) * 1024);
                ns0 = S0[(g + 1) * 32];
                ns1 = S1[(g + 1) * 32];
            }
            f32x16_t acc[2][2];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                typedef typename OpT<MODE>::type op_t;
                const op_t b0 = OpT<MODE>::frag(bw0[s]);
                const op_t b1 = OpT<MODE>::frag(bw1[s]);
#pragma unroll
                for (int ms = 0; ms < 2; ++ms) {
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
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    tot[ms][0][v] = fmaf(s16_0, acc[ms][0][v], tot[ms][0][v]);
                    tot[ms][1][v] = fmaf(s16_1, acc[ms][1][v], tot[ms][1][v]);
                }
            if (g + 1 < G) {
                store_A(buf ^ 1);
                bw0 = nb0;
                bw1 = nb1;
                sb0 = ns0;
                sb1 = ns1;
            }
            __syncthreads();
        }

        // bias-term GEMM: K' = 3 Gp; A' = [X_hi | X_lo | X_hi], B' = [c_hi | c_hi | c_lo]
        {
            const int steps = 3 * Gp / 16;
            int srcs[2];
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) srcs[ms] = srow[wm * 64 + ms * 32 + n];
            for (int st = 0; st < steps; ++st) {
                const int kk0 = 16 * st + 8 * half;
                uint32_t w0[4], w1[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    uint32_t lo0 = 0, hi0 = 0, lo1 = 0, hi1 = 0;
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int kk = kk0 + 2 * jj + h2;
                        const int part = kk / Gp, gg = kk % Gp;
                        uint32_t v0 = 0, v1 = 0;
                        if (gg < G) {
                            v0 = bias_part(S0[gg * 32], part);
                            v1 = bias_part(S1[gg * 32], part);
                        }
                        if (h2 == 0) {
                            lo0 = v0;
                            lo1 = v1;
                        } else {
                            hi0 = v0;
                            hi1 = v1;
                        }
                    }
                    w0[jj] = lo0 | (hi0 << 16);
                    w1[jj] = lo1 | (hi1 << 16);
                }
                const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w0[2], w0[3]});
                const bf16x8_t b1 = __builtin_bit_cast(bf16x8_t, u32x4_t{w1[0], w1[1], w1[2], w1[3]});
#pragma unroll
                for (int ms = 0; ms < 2; ++ms) {
                    u32x4_t av = u32x4_t{0u, 0u, 0u, 0u};
                    if (srcs[ms] >= 0) av = ld16(Bsrc + (size_t)srcs[ms] * 3 * Gp + kk0);
                    const bf16x8_t avb = __builtin_bit_cast(bf16x8_t, av);
                    tot[ms][0] = mfma32(avb, b0, tot[ms][0]);
                    tot[ms][1] = mfma32(avb, b1, tot[ms][1]);
                }
            }
        }

        // epilogue. Accumulator element v of lane l: row 8*(v/4) + 4*(l/32) + v%4, column l%32.
        if (MODE == 0) {
            const int J = shared_item ? a.Is : a.I;
            uint16_t *hout = shared_item ? a.h_s : a.h_r;
            const int j = (nt * 2 + wn) * 32 + n;
            float rsum[2][16];
#pragma unroll
            for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = wm * 64 + ms * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
                    const uint32_t hb = f32_to_f16_sat(gelu_tanh_f32(tot[ms][0][v]) * tot[ms][1][v]);
                    const int dst = drow[row];
                    if (dst >= 0) hout[(size_t)dst * J + j] = (uint16_t)hb;
                    rsum[ms][v] = f16_to_f32(hb);
                }
            // sum over this wave's 32 columns (lanes of one half share rows)
#pragma unroll
            for (int off = 1; off < 32; off <<= 1)
#pragma unroll
                for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                    for (int v = 0; v < 16; ++v) rsum[ms][v] += __shfl_xor(rsum[ms][v], off);
            if (n == 0) {
#pragma unroll
                for (int ms = 0; ms < 2; ++ms)
#pragma unroll
                    for (int v = 0; v < 16; ++v)
                        hsum[wn][wm * 64 + ms * 32 + 8 * (v >> 2) + 4 * half + (v & 3)] = rsum[ms][v];
            }
            __syncthreads();
            if (tid < kMT) {
                const int dst = drow[tid];
                if (dst >= 0) {
                    const int Gpo = shared_item ? a.Gp_Is : a.Gp_I;
                    uint16_t *hs = (shared_item ? a.hsplit_s : a.hsplit_r) + (size_t)dst * 3 * Gpo;
                    const float H = hsum[0][tid] + hsum[1][tid];
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
