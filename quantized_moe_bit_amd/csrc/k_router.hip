// Router, top-k and token/expert grouping kernels (gfx950).
//
// Router: one logit per (token, expert) from the 8-bit group-64 affine router
// projection, with no softcap (Mference system design, "Why the runtime has this
// shape"; "Decode", router listing), plus an optional per-expert logit bias. The
// logits decide an integer result (the top-k set), so they are computed in one fixed
// fp32 order, the same one the CPU oracle writes out:
//   X_g = x_{64g} + ... + x_{64g+63}               (fp32 adds, ascending)
//   A_g = fma chain of x_j * q_j, ascending j         (fp32, starting from 0)
//   P_g = fma(scale_g, A_g, fl(bias_g * X_g))
//   logit = (P_0 + P_1 + ... + P_{G-1}) [+ logit_bias]   (fp32 adds, ascending g)
// Contraction is disabled in this file so the compiler cannot fuse or reorder these.
//
// Top-k: the k largest logits, largest first, equal values ordered by lower expert
// index (TinyTitan architecture, "Invariants": top-k index sets must match exactly),
// and the softmax of the selected logits as routing weights.
//
// Grouping: token/expert pairs of a chunk grouped by expert (Mference, "Prefill"),
// stable in token order: offsets[e] = pairs routed to experts below e, perm lists pair
// ids t*k + slot by (expert, token), pos is its inverse.
#include "device_common.h"
#include "moe_internal.h"

#pragma clang fp contract(off)

namespace qmoe {
namespace {

constexpr int kRouterWaves = 4;                  // experts per workgroup
constexpr int kXPitch = 66;                      // bf16 per group in LDS (64 + 2 pad: conflict-free dword reads)

// grid: (ceil(E / 4), ceil(T / kRouterTokens)); block 256
__global__ __launch_bounds__(256) void k_router(const uint16_t *__restrict__ x, int T, int d, int E,
                                                const uint8_t *__restrict__ rq, const uint32_t *__restrict__ rsb,
                                                const float *__restrict__ logit_bias, float *__restrict__ logits,
                                                float *__restrict__ xsum, uint16_t *__restrict__ xsplit, int Gp) {
    extern __shared__ __align__(16) unsigned char smem[];
    const int G = d / 64;
    const int t0 = blockIdx.y * kRouterTokens;
    const int nt = min(kRouterTokens, T - t0);
    uint16_t *xs = reinterpret_cast<uint16_t *>(smem);                  // [kRouterTokens][G][kXPitch]
    float *Xs = reinterpret_cast<float *>(smem + sizeof(uint16_t) * kRouterTokens * G * kXPitch);  // [tok][G]
    float *Ps = Xs + kRouterTokens * G;                                  // [4 waves][tok][G]
    const int tid = threadIdx.x;

    // stage the token tile (bf16) into LDS, padded per group
    for (int i = tid; i < kRouterTokens * d / 2; i += 256) {
        const int t = i / (d / 2), c = (i % (d / 2)) * 2;
        uint32_t v = 0;
        if (t < nt) v = *reinterpret_cast<const uint32_t *>(x + (size_t)(t0 + t) * d + c);
        const int g = c / 64, j = c % 64;
        *reinterpret_cast<uint32_t *>(xs + (t * G + g) * kXPitch + j) = v;
    }
    __syncthreads();
    // group sums X_g in the fixed ascending order
    for (int i = tid; i < kRouterTokens * G; i += 256) {
        const int t = i / G, g = i % G;
        const uint16_t *row = xs + (t * G + g) * kXPitch;
        float s = 0.0f;
        for (int j = 0; j < 64; ++j) s = s + bf16_to_f32(row[j]);
        Xs[i] = s;
        if (blockIdx.x == 0 && t < nt) {
            const size_t tt = (size_t)(t0 + t);
            xsum[tt * G + g] = s;
            const uint32_t hi = f32_to_bf16(s);
            const uint32_t lo = f32_to_bf16(s - bf16_to_f32(hi));
            xsplit[tt * 3 * Gp + g] = (uint16_t)hi;
            xsplit[tt * 3 * Gp + Gp + g] = (uint16_t)lo;
            xsplit[tt * 3 * Gp + 2 * Gp + g] = (uint16_t)hi;
        }
    }
    __syncthreads();

    const int wave = tid >> 6, lane = tid & 63;
    const int e = blockIdx.x * kRouterWaves + wave;
    if (e < E) {
        for (int g = lane; g < G; g += 64) {
            // this lane's 64 codes
            const u32x4_t *cp = reinterpret_cast<const u32x4_t *>(rq + (size_t)e * d + 64 * g);
            u32x4_t c4[4] = {cp[0], cp[1], cp[2], cp[3]};
            const uint32_t sbw = rsb[(size_t)e * G + g];
            const float sc = bf16_to_f32(sbw & 0xFFFFu), bi = bf16_to_f32(sbw >> 16);
            float A[kRouterTokens];
#pragma unroll
            for (int t = 0; t < kRouterTokens; ++t) A[t] = 0.0f;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
#pragma unroll
                for (int wi = 0; wi < 4; ++wi) {
                    const uint32_t cw = c4[q4][wi];
#pragma unroll
                    for (int b = 0; b < 4; b += 2) {
                        const int j = q4 * 16 + wi * 4 + b;     // element index within the group
                        const float qa = (float)((cw >> (8 * b)) & 0xFFu);
                        const float qb = (float)((cw >> (8 * (b + 1))) & 0xFFu);
#pragma unroll
                        for (int t = 0; t < kRouterTokens; ++t) {
                            const uint32_t xv =
                                *reinterpret_cast<const uint32_t *>(xs + (t * G + g) * kXPitch + j);
                            A[t] = __builtin_fmaf(bf16_to_f32(xv & 0xFFFFu), qa, A[t]);
                            A[t] = __builtin_fmaf(bf16_to_f32(xv >> 16), qb, A[t]);
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < kRouterTokens; ++t) {
                const float bX = bi * Xs[t * G + g];
                Ps[(wave * kRouterTokens + t) * G + g] = __builtin_fmaf(sc, A[t], bX);
            }
        }
    }
    __syncthreads();
    if (e < E && lane < nt) {
        const float *p = Ps + (wave * kRouterTokens + lane) * G;
        float L = 0.0f;
        for (int g = 0; g < G; ++g) L = L + p[g];
        if (logit_bias) L = L + logit_bias[e];
        logits[(size_t)(t0 + lane) * E + e] = L;
    }
}

// (value desc, index asc) ordering
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
    return va > vb || (va == vb && ia < ib);
}

// grid: ceil(T / 4); block 256 -- one wave per token
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, int T, int E, int k,
                                              int32_t *__restrict__ idx, float *__restrict__ wout) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    const float *l = logits + (size_t)t * E;
    constexpr int kPer = MOE_MAX_EXPERTS / 64;
    float v[kPer];
    const int nper = (E + 63) / 64;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        v[i] = (i < nper && e < E) ? l[e] : -__builtin_inff();
    }
    uint32_t taken = 0;   // bit i: element lane + 64 i already selected
    float sel_v[MOE_MAX_TOP_K];
    int sel_i[MOE_MAX_TOP_K];
    for (int s = 0; s < k; ++s) {
        float bv = -__builtin_inff();
        int bi = 0x7FFFFFFF;
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int e = lane + 64 * i;
            // an unset best (bi == INT_MAX) takes any candidate, so the index stays valid even for NaN
            if (i < nper && e < E && !((taken >> i) & 1u) && (bi == 0x7FFFFFFF || better(v[i], e, bv, bi))) {
                bv = v[i];
                bi = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (oi != 0x7FFFFFFF && (bi == 0x7FFFFFFF || better(ov, oi, bv, bi))) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
        sel_v[s] = bv;
        sel_i[s] = bi;
    }
    if (lane == 0) {
        const float m = sel_v[0];
        float z = 0.0f;
        float ex[MOE_MAX_TOP_K];
        for (int s = 0; s < k; ++s) {
            ex[s] = __expf(sel_v[s] - m);
            z += ex[s];
        }
        const float inv = 1.0f / z;
        for (int s = 0; s < k; ++s) {
            idx[(size_t)t * k + s] = min(max(sel_i[s], 0), E - 1);
            wout[(size_t)t * k + s] = ex[s] * inv;
        }
    }
}

// Within-chunk stable ranks. grid: nchunks; block kChunk (256)
__global__ __launch_bounds__(256) void k_bucket_rank(const int32_t *__restrict__ idx, int P, int E,
                                                     int32_t *__restrict__ rank, int32_t *__restrict__ chunk_cnt) {
    __shared__ int32_t wcnt[4][MOE_MAX_EXPERTS];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int i = tid; i < 4 * E; i += 256) wcnt[i / E][i % E] = 0;
    __syncthreads();
    const int p = blockIdx.x * kChunk + tid;
    const bool valid = p < P;
    const int e = valid ? idx[p] : 0;
    // lanes of this wave with the same expert
    uint64_t peers = __ballot(valid);
    for (int b = 0; (1 << b) < MOE_MAX_EXPERTS; ++b) {
        const uint64_t m = __ballot(valid && ((e >> b) & 1));
        peers &= ((e >> b) & 1) ? m : ~m;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int r_w = __popcll(peers & below);
    if (valid && r_w == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
        int r = r_w;
        for (int w = 0; w < wave; ++w) r += wcnt[w][e];
        rank[p] = r;
    }
    for (int i = tid; i < E; i += 256)
        chunk_cnt[(size_t)blockIdx.x * E + i] = wcnt[0][i] + wcnt[1][i] + wcnt[2][i] + wcnt[3][i];
}

// Counts, offsets, per-chunk bases and GEMM tile offsets. grid 1; block 1024
__global__ __launch_bounds__(1024) void k_bucket_scan(int nchunks, int E, int32_t *__restrict__ chunk_base,
                                                      int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                      int32_t *__restrict__ tile_off, int mt) {
    __shared__ int32_t sc[MOE_MAX_EXPERTS];
    __shared__ int32_t st[MOE_MAX_EXPERTS];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int c = 0; c < nchunks; ++c) {
            const int v = chunk_base[(size_t)c * E + e];
            chunk_base[(size_t)c * E + e] = run;
            run += v;
        }
        counts[e] = run;
        sc[e] = run;
        st[e] = (run + mt - 1) / mt;
    }
    __syncthreads();
    if (e == 0) {
        int a = 0, b = 0;
        for (int i = 0; i < E; ++i) {
            offsets[i] = a;
            tile_off[i] = b;
            const int ca = sc[i], cb = st[i];
            sc[i] = a;
            a += ca;
            b += cb;
        }
        offsets[E] = a;
        tile_off[E] = b;
    }
    __syncthreads();
    if (e < E) {
        const int base = sc[e];
        for (int c = 0; c < nchunks; ++c) chunk_base[(size_t)c * E + e] += base;
    }
}

// grid: nchunks; block 256
__global__ __launch_bounds__(256) void k_bucket_scatter(const int32_t *__restrict__ idx, int P, int E,
                                                        const int32_t *__restrict__ rank,
                                                        const int32_t *__restrict__ chunk_base,
                                                        int32_t *__restrict__ perm, int32_t *__restrict__ pos,
                                                        int32_t *__restrict__ perm_out) {
    const int p = blockIdx.x * kChunk + threadIdx.x;
    if (p >= P) return;
    const int e = idx[p];
    const int q = chunk_base[(size_t)blockIdx.x * E + e] + rank[p];
    perm[q] = p;
    pos[p] = q;
    if (perm_out) perm_out[q] = p;
}

}  // namespace

hipError_t launch_router(const moe_layer *L, const uint16_t *x, int T, float *logits, hipStream_t s) {
    const int d = L->dims.d_model, E = L->dims.n_experts, G = d / 64;
    dim3 grid(cdiv(E, kRouterWaves), cdiv(T, kRouterTokens));
    const size_t lds = sizeof(uint16_t) * kRouterTokens * G * kXPitch + sizeof(float) * kRouterTokens * G * 5;
    hipLaunchKernelGGL(k_router, grid, dim3(256), lds, s, x, T, d, E,
                       static_cast<const uint8_t *>(L->w.router.codes), L->w.router.sb, L->w.logit_bias, logits,
                       L->ws.xsum, L->ws.xsplit, L->Gp_d);
    return hipGetLastError();
}

hipError_t launch_topk(const moe_layer *L, int T, const float *logits, int32_t *idx, float *w, hipStream_t s) {
    hipLaunchKernelGGL(k_topk, dim3(cdiv(T, 4)), dim3(256), 0, s, logits, T, L->dims.n_experts, L->dims.top_k,
                       idx, w);
    return hipGetLastError();
}

hipError_t launch_bucket_rank(const moe_layer *L, int T, const int32_t *idx, hipStream_t s) {
    const int P = T * L->dims.top_k;
    hipLaunchKernelGGL(k_bucket_rank, dim3(cdiv(P, kChunk)), dim3(kChunk), 0, s, idx, P, L->dims.n_experts,
                       L->ws.rank, L->ws.chunk_base);
    return hipGetLastError();
}

hipError_t launch_bucket_scan(const moe_layer *L, int T, hipStream_t s) {
    const int P = T * L->dims.top_k;
    hipLaunchKernelGGL(k_bucket_scan, dim3(1), dim3(1024), 0, s, cdiv(P, kChunk), L->dims.n_experts,
                       L->ws.chunk_base, L->ws.counts, L->ws.offsets, L->ws.tile_off, kMT);
    return hipGetLastError();
}

hipError_t launch_bucket_scatter(const moe_layer *L, int T, const int32_t *idx, int32_t *perm_out, hipStream_t s) {
    const int P = T * L->dims.top_k;
    hipLaunchKernelGGL(k_bucket_scatter, dim3(cdiv(P, kChunk)), dim3(kChunk), 0, s, idx, P, L->dims.n_experts,
                       L->ws.rank, L->ws.chunk_base, L->ws.perm, L->ws.pos, perm_out);
    return hipGetLastError();
}

}  // namespace qmoe
