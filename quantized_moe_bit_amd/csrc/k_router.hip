// Router, top-k and token/expert grouping kernels (gfx950).
//
// Router (prefill chunks; decode has its own router in k_decode.hip with the same
// arithmetic): one logit per (token, expert) from the 8-bit group-64 affine router
// projection, with no softcap (Mference system design, "Why the runtime has this
// shape"; "Decode", router listing), plus an optional per-expert logit bias. The
// logits decide an integer result (the top-k set), so they are computed in one fixed
// fp32 order, the same one the CPU oracle writes out:
//   w_j = fma(scale_g, q_j, bias_g)                   (the dequantized weight, fp32)
//   A_g = fma chain of x_j * w_j, ascending j         (fp32, starting from 0)
//   logit = (A_0 + A_1 + ... + A_{G-1}) [+ logit_bias]   (fp32 adds, ascending g)
// Contraction is disabled in this file so the compiler cannot fuse or reorder these.
// Two kernels compute it: k_router_ksplit (lane = token, the groups of a token spread over
// eight waves, fma chains with row-broadcast weights, each A_g kept in LDS and folded in
// ascending g by one wave) for chunks up to about a thousand tokens, and k_router_mfma (the
// chains on the matrix cores, whose fp32 multiply-add is an ordered fma) for larger ones;
// both give the same bits.
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

constexpr int kRNE = 4;                  // experts per wave of the prefill router
constexpr long kRouterKsplitMaxWG = 512;    // see router_ksplit
constexpr int kRBlk = 64 * kRNE;   // router table floats per (expert block, group)

// Router prologue (Mference system design, "Decode", router listing): the router reads
//   u = bf16(((x / sqrt(mean(x^2) + 1e-6)) * router_scale) / sqrt(d))
// computed in float64 in that order and rounded once, the same expression the oracle writes
// out (its sum of squares runs in another order; the bf16 rounding absorbs the difference).
// Also writes the fp16 copy of x (x16, prefill) or the fixed-order group sums of x (xg,
// decode; nl = 32 for Q4_0 experts: sums of 32 inputs), which the router would otherwise
// derive from its own input.
// grid: T; block 256 (d <= 8192: at most four 16-byte chunks per thread)
constexpr int kProChunks = 4;
__global__ __launch_bounds__(256) void k_router_prologue(const uint16_t *__restrict__ x, int d,
                                                         const uint16_t *__restrict__ rs, uint16_t *__restrict__ u,
                                                         uint16_t *__restrict__ x16, float *__restrict__ xg, int nl) {
    __shared__ double red[4];
    const int t = blockIdx.x, tid = threadIdx.x, nc = d / 8;
    const uint16_t *xt = x + (size_t)t * d;
    u32x4_t xv[kProChunks], rv[kProChunks];
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < kProChunks; ++c) {
        const int i = tid + 256 * c;
        if (i < nc) {
            xv[c] = ld16(xt + 8 * i);
            rv[c] = ld16(rs + 8 * i);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const double v = bf16_to_f64((xv[c][j >> 1] >> (16 * (j & 1))) & 0xFFFFu);
                ss = fma(v, v, ss);
            }
        }
    }
    ss = wave_sum_f64(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const double tot = (red[0] + red[1]) + (red[2] + red[3]);
    const double inv = 1.0 / sqrt(tot / (double)d + 1e-6), sd = sqrt((double)d);
#pragma unroll
    for (int c = 0; c < kProChunks; ++c) {
        const int i = tid + 256 * c;
        if (i < nc) {
            u32x4_t uo, ho;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t ub[2], hb[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t xb = (xv[c][w] >> (16 * h)) & 0xFFFFu, rb = (rv[c][w] >> (16 * h)) & 0xFFFFu;
                    ub[h] = f64_to_bf16(((bf16_to_f64(xb) * inv) * bf16_to_f64(rb)) / sd);
                    hb[h] = f32_to_f16(bf16_to_f32(xb));
                }
                uo[w] = ub[0] | (ub[1] << 16);
                ho[w] = hb[0] | (hb[1] << 16);
            }
            *reinterpret_cast<u32x4_t *>(u + (size_t)t * d + 8 * i) = uo;
            if (x16) *reinterpret_cast<u32x4_t *>(x16 + (size_t)t * d + 8 * i) = ho;
        }
    }
    if (xg && tid < d / nl) {   // X = ((0 + x_0) + x_1) + ... over nl inputs, fp32
        float X = 0.0f;
        for (int j = 0; j < nl; ++j) X = X + bf16_to_f32(xt[nl * tid + j]);
        xg[(size_t)t * (d / nl) + tid] = X;
    }
}

// Router weight table (built at layer creation, k_router_table): the weights dequantized to
// fp32, per block of kRNE experts eb and group g kRBlk floats [4 jc][16 j][kRNE] (input
// 16 jc + j of expert kRNE eb + i at [jc][j][i]); experts past E are zero.
static_assert(kRNE == 4, "one 16-byte load per lane holds the four experts' codes of an input");

// a += x * (lane J of q's 16-lane row), one instruction (the DPP source is a loaded register,
// never one a VALU instruction has just written)
template <int J>
__device__ __forceinline__ void fma_rowbcast(float &a, float x, float q) {
    asm("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf" : "+v"(a) : "v"(q), "v"(x), "n"(J));
}
template <int J>
__device__ __forceinline__ void chunk_fmas(float (&A)[kRNE], const f32x4_t (&xv)[4], const f32x4_t &q) {
#pragma unroll
    for (int i = 0; i < kRNE; ++i) fma_rowbcast<J>(A[i], xv[J >> 2][J & 3], q[i]);
    if constexpr (J + 1 < 16) chunk_fmas<J + 1>(A, xv, q);
}

// Prefill router with the groups split across the waves of a workgroup: lane = token, the
// workgroup = 64 tokens x kRNE experts, wave w computes the group sums A_g of groups
// [w gw, (w + 1) gw) (gw = ceil(G / kKW)) as fma chains, each weight taken from lane j of a
// 16-lane row by a row broadcast (DPP row_newbcast, no instruction spent on moving weights),
// and stores them in LDS; after one barrier, wave i < kRNE folds expert i's sums in group
// order, L = ((0 + A_0) + A_1) + ... + A_{G-1}.
// A wave brings its groups' inputs in with coalesced loads (eight lanes per token row) into a
// staging tile of its own in LDS and reads them back one token row per lane, so it waits on no
// other wave until the fold. A workgroup carries 64 tokens x 4 experts and an eighth of each
// chain, which fills the chip when the chunk has few tokens (512 tokens: 256 workgroups of 8
// waves; the matrix-core router has 64 of 4 there). LDS: G x kRNE x 64 fp32 of group sums
// (d <= 4096) and 8 staging tiles of 64 x 64 bf16.
// grid: (ceil(T / 64), ceil(E / kRNE)); block 64 kKW
constexpr int kKW = 8;
constexpr int kKSplitMaxG = 64;
constexpr int kKXP = 72;   // bf16 per staged token row (144 B: row t's 16-byte chunks spread over the banks)
__global__ __launch_bounds__(64 * kKW) void k_router_ksplit(const uint16_t *__restrict__ x, int T, int d, int E,
                                                           const float *__restrict__ tab,
                                                           const float *__restrict__ logit_bias,
                                                           float *__restrict__ logits, uint16_t *__restrict__ x16) {
    __shared__ float As[kKSplitMaxG][kRNE][64];
    __shared__ __align__(16) uint16_t xsw[kKW][64][kKXP];
    const int G = d / 64;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int eb = blockIdx.y, e0 = eb * kRNE;
    const int t = blockIdx.x * 64 + lane;
    const int gw = cdiv(G, kKW), g0 = wave * gw, g1 = min(G, g0 + gw);
    // coalesced loads: this lane moves chunk lc = lane % 8 (inputs 8 lc .. 8 lc + 7 of the group)
    // of token rows lane / 8 + 8 i, i = 0..7
    const int lc = lane & 7, lr = lane >> 3;
    uint16_t (*xw)[kKXP] = xsw[wave];
    const float *blk = tab + (size_t)eb * G * kRBlk;
    auto load_q = [&](int g, f32x4_t (&q)[4]) {
#pragma unroll
        for (int jc = 0; jc < 4; ++jc)
            q[jc] = *reinterpret_cast<const f32x4_t *>(blk + (size_t)g * kRBlk + (16 * jc + (lane & 15)) * kRNE);
    };
    auto load_x = [&](int g, u32x4_t (&v)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = min((int)blockIdx.x * 64 + lr + 8 * i, T - 1);
            v[i] = ld16(x + (size_t)r * d + 64 * g + 8 * lc);
        }
    };
    // loaded chunks into the staging tile (and, for the first expert block, the fp16 copy of x)
    auto put_x = [&](int g, const u32x4_t (&v)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int rl = lr + 8 * i;
            *reinterpret_cast<u32x4_t *>(&xw[rl][8 * lc]) = v[i];
            const int r = (int)blockIdx.x * 64 + rl;
            if (x16 && eb == 0 && r < T) {
                u32x4_t h;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    h[w] = f32_to_f16(bf16_to_f32(v[i][w] & 0xFFFFu)) | (f32_to_f16(bf16_to_f32(v[i][w] >> 16)) << 16);
                *reinterpret_cast<u32x4_t *>(x16 + (size_t)r * d + 64 * g + 8 * lc) = h;
            }
        }
    };
    if (g0 < g1) {
        u32x4_t nv[8];
        f32x4_t qa[4], qb[4];
        load_x(g0, nv);
        load_q(g0, qa);
        put_x(g0, nv);
        // one group: the next group's loads go out first; its inputs replace this group's in the
        // staging tile after this group's reads (LDS operations of a wave complete in order)
        auto group = [&](int g, const f32x4_t (&q)[4], f32x4_t (&qn)[4]) {
            const bool more = g + 1 < g1;
            if (more) {
                load_x(g + 1, nv);
                load_q(g + 1, qn);
            }
            float A[kRNE];
#pragma unroll
            for (int i = 0; i < kRNE; ++i) A[i] = 0.0f;
#pragma unroll
            for (int jc = 0; jc < 4; ++jc) {
                // inputs 16 jc .. 16 jc + 15 of this lane's token as fp32 (bf16 -> fp32 is exact)
                const u32x4_t c0 = *reinterpret_cast<const u32x4_t *>(&xw[lane][16 * jc]);
                const u32x4_t c1 = *reinterpret_cast<const u32x4_t *>(&xw[lane][16 * jc + 8]);
                f32x4_t xf[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    xf[w >> 1][2 * (w & 1)] = __uint_as_float(c0[w] << 16);
                    xf[w >> 1][2 * (w & 1) + 1] = __uint_as_float(c0[w] & 0xFFFF0000u);
                    xf[2 + (w >> 1)][2 * (w & 1)] = __uint_as_float(c1[w] << 16);
                    xf[2 + (w >> 1)][2 * (w & 1) + 1] = __uint_as_float(c1[w] & 0xFFFF0000u);
                }
                chunk_fmas<0>(A, xf, q[jc]);
            }
#pragma unroll
            for (int i = 0; i < kRNE; ++i) As[g][i][lane] = A[i];
            if (more) put_x(g + 1, nv);
        };
        for (int g = g0; g < g1; g += 2) {
            group(g, qa, qb);
            if (g + 1 < g1) group(g + 1, qb, qa);
        }
    }
    __syncthreads();
    if (wave >= kRNE || t >= T) return;
    const int e = e0 + wave;
    if (e >= E) return;
    float L = 0.0f;   // contraction is off for this file: the fold is L = L + A_g, in group order
    for (int g = 0; g < G; ++g) L = L + As[g][wave][lane];
    logits[(size_t)t * E + e] = logit_bias ? L + logit_bias[e] : L;
}

// Prefill router on the matrix cores. v_mfma_f32_16x16x4_f32 performs its four fp32
// multiply-adds in k order, each rounded once like an fma (checked on the device against
// sequential fmaf over normal, subnormal and mixed operands), so 16 of them over one group's
// 64 inputs (step s takes inputs 4 s .. 4 s + 3 as its k = 0..3) form exactly the chain
// A_g = fma(x_63, w_63, ... fma(x_0, w_0, 0)) of the fixed order, for 16 tokens x 16 experts at
// once; the group sums are then added in group order in registers, L = ((0 + A_0) + A_1) + ...
// Operand layout: lane l holds A[row l % 16][k l / 16] and B[k l / 16][column l % 16]; result
// element v of lane l is row 4 (l / 16) + v, column l % 16.
// Workgroup: 64 tokens (wave w: tokens 16 w .. 16 w + 15) x 16 experts. The MFMA router table
// (below) stores each lane's 16 weight operands of a group contiguously; a K step of kMG
// groups copies the step's table rows (4 KB per group, shared by the four waves) into LDS with
// 80 B between lanes, and each wave writes the x rows of its 16 tokens into a tile of its own,
// transposed so that a lane's 16 x operands of a group (input 4 s + k, s = 0..15) are
// contiguous; a lane's operands then come in with two (x) and four (weights) 16-byte reads.
// The 16-byte pieces of x row r sit at piece u ^ xswz(r), which keeps the tile's writes (16
// lanes x 8 B per pass) and reads (8 lanes x 16 B) free of bank conflicts for 32 as for 64 LDS
// banks; the weights' 80-B lane pitch does the same for theirs. The LDS (53 KB) and registers
// leave room for two workgroups per compute unit.
// Software pipeline over two LDS stages, two register sets of operands and two of global loads,
// one barrier per K step: step st runs its kMG chains (one accumulator each, interleaved) on
// operands read during step st - 1, while the operands of step st + 1 come in from LDS, step
// st + 2 (loaded into registers during step st - 2) is written into the stage step st's operands
// came from, and the global loads of step st + 4 are issued; the group sums are folded into L in
// group order last.
// The loads are issued on every path (past the last group they re-read it), so each wait is for
// exactly its own step's data.
// Tile order: workgroup b runs on XCD b % 8 and takes token block 8 (b / 8 / NEB) + b % 8 and
// expert block (b / 8) % NEB, so an XCD runs the NEB expert blocks of a token block back to
// back (its x rows fetched into that XCD's L2 once). Expert block eb also writes the fp16 copy
// of x for the groups g with g % NEB = eb of its tokens, so the stores are spread evenly.
// grid: 8 ceil(ceil(T / 64) / 8) ceil(E / 16); block 256
constexpr int kMG = 2;                         // groups per K step
constexpr int kMXR = 64 * kMG;                 // bf16 per staged x row (256 B: 16 pieces of 16 B)
constexpr int kMTile = 1024;                   // MFMA table floats per (16-expert block, group)
constexpr int kMWL = 20;                       // staged weight floats per lane (80 B)
// physical 16-byte piece of logical piece u in row r of the x tile: u ^ xswz(r)
__device__ __forceinline__ int xswz(int r) { return (2 * (r & 3) + ((r >> 2) & 3)) & 15; }
struct alignas(16) RouterMfmaSmem {
    alignas(16) uint16_t xs[2][4][16][kMXR];
    alignas(16) float wsm[2][kMG][64][kMWL];
};
template <bool X16>
__device__ __forceinline__ f32x4_t router_mfma_tile(RouterMfmaSmem &sm, const uint16_t *__restrict__ x, int T, int d,
                                                    int G, int tb, int eb, int NEB, const float *__restrict__ tab,
                                                    uint16_t *__restrict__ x16) {
    const int NS = cdiv(G, kMG);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // x loads: lane l takes row l / 4 of its wave's 16, inputs 16 (l % 4) .. 16 (l % 4) + 15 of each group
    const int xr = lane >> 2, xc = (lane & 3) * 16;
    const int tx = 64 * tb + 16 * wave + xr;
    const uint16_t *xrow = x + (size_t)min(tx, T - 1) * d + xc;
    const bool wx16 = X16 && tx < T;
    // weight loads: thread tid copies half (tid / 64) % 2 of table lane tid % 64 of group kMG st + tid / 128
    const int wq = tid >> 7, wl = tid & 63, wh = (tid >> 6) & 1;
    const float *wsrc = tab + ((size_t)eb * G * 64 + wl) * 16 + 8 * wh;
    struct Loaded {   // one step's global loads
        f32x4_t wv[2];
        u32x4_t xv[kMG][2];
    };
    // weights first, so that staging waits for them alone before it waits for x
    auto load = [&](Loaded &ld, int st) {
        const f32x4_t *p = reinterpret_cast<const f32x4_t *>(wsrc + (size_t)min(kMG * st + wq, G - 1) * kMTile);
        ld.wv[0] = p[0];
        ld.wv[1] = p[1];
        __builtin_amdgcn_sched_barrier(0);   // keeps this order of the loads on every path
#pragma unroll
        for (int q = 0; q < kMG; ++q) {
            const int g = min(kMG * st + q, G - 1);
            ld.xv[q][0] = ld16(xrow + 64 * g);
            ld.xv[q][1] = ld16(xrow + 64 * g + 8);
        }
    };
    // the loaded step into LDS stage b: x input xc + i of group q -> logical element
    // 16 (4 q + i % 4) + xc / 4 + i / 4 of row xr (16-byte piece 2 (4 q + i % 4) + xc / 32);
    // the fp16 copy of x is stored last
    auto stage = [&](int b, int st, const Loaded &ld) {
        *reinterpret_cast<f32x4_t *>(&sm.wsm[b][wq][wl][8 * wh]) = ld.wv[0];
        *reinterpret_cast<f32x4_t *>(&sm.wsm[b][wq][wl][8 * wh + 4]) = ld.wv[1];
#pragma unroll
        for (int q = 0; q < kMG; ++q) {
            const uint32_t *w32 = reinterpret_cast<const uint32_t *>(&ld.xv[q][0]);   // 8 words, 16 bf16
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                // inputs kk, kk + 4, kk + 8, kk + 12 of the lane's 16: the same half (kk % 2) of
                // words kk / 2, 2 + kk / 2, 4 + kk / 2, 6 + kk / 2, two per byte permute
                const uint32_t sel = (kk & 1) ? 0x07060302u : 0x05040100u;
                uint2 pk;
                pk.x = __builtin_amdgcn_perm(w32[2 + (kk >> 1)], w32[kk >> 1], sel);
                pk.y = __builtin_amdgcn_perm(w32[6 + (kk >> 1)], w32[4 + (kk >> 1)], sel);
                const int u = 2 * (4 * q + kk) + (xc >> 5);
                *reinterpret_cast<uint2 *>(&sm.xs[b][wave][xr][8 * (u ^ xswz(xr)) + ((xc >> 2) & 4)]) = pk;
            }
        }
        if constexpr (X16) {
            if (wx16) {
#pragma unroll
                for (int q = 0; q < kMG; ++q) {
                    const int g = kMG * st + q;
                    if (g < G && g % NEB == eb) {
                        uint16_t *xo = x16 + (size_t)tx * d + 64 * g + xc;
                        *reinterpret_cast<u32x4_t *>(xo) = bf16x8_to_f16x8(ld.xv[q][0]);
                        *reinterpret_cast<u32x4_t *>(xo + 8) = bf16x8_to_f16x8(ld.xv[q][1]);
                    }
                }
            }
        }
    };
    const int r = lane & 15, k = lane >> 4;
    struct Ops {
        u32x4_t xa[kMG][2];   // a lane's 16 x operands (bf16) of each group
        f32x4_t wb[kMG][4];   // and its 16 weight operands
    };
    auto read_ops = [&](Ops &o, int b) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < kMG; ++q) {
                o.wb[q][i] = *reinterpret_cast<const f32x4_t *>(&sm.wsm[b][q][lane][4 * i]);
                if (i < 2)
                    o.xa[q][i] = *reinterpret_cast<const u32x4_t *>(&sm.xs[b][wave][r][8 * ((2 * (4 * q + k) + i) ^ xswz(r))]);
            }
    };
    f32x4_t L = {0.0f, 0.0f, 0.0f, 0.0f};
    // the chains of step st (operands o), folded into L in group order; the next step's operands
    // are read from LDS stage nb into `next` meanwhile, one read between every two MFMAs (a wave
    // keeps at most 15 LDS reads in flight; issued all at once they would stall it)
    auto mfma_step = [&](const Ops &o, int st, Ops &next, int nb, f32x4_t (&a)[kMG]) {
        auto xval = [&](int q, int s4) {
            const uint32_t v = o.xa[q][s4 >> 3][(s4 >> 1) & 3];
            return bf16_to_f32((s4 & 1) ? (v >> 16) : (v & 0xFFFFu));
        };
        // every x operand converted before the first MFMA, each into a register of its own: a
        // register an MFMA is still reading is never rewritten by the next conversion
        float xf[kMG][16];
#pragma unroll
        for (int q = 0; q < kMG; ++q)
#pragma unroll
            for (int s4 = 0; s4 < 16; ++s4) xf[q][s4] = xval(q, s4);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < kMG; ++q) a[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        const int ng = min(kMG, G - kMG * st);
        if (ng == kMG) {   // the chains interleaved
            read_ops(next, nb);
#pragma unroll
            for (int s4 = 0; s4 < 16; ++s4)
#pragma unroll
                for (int q = 0; q < kMG; ++q)
                    a[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[q][s4], o.wb[q][s4 >> 2][s4 & 3], a[q], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 6 * kMG; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // two MFMAs
            }
        } else {
            read_ops(next, nb);
#pragma unroll
            for (int q = 0; q < kMG; ++q)
                if (q < ng)
#pragma unroll
                    for (int s4 = 0; s4 < 16; ++s4)
                        a[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[q][s4], o.wb[q][s4 >> 2][s4 & 3], a[q], 0, 0, 0);
        }
    };
    // fold step st's group sums into L in group order (contraction is off for this file); the
    // caller does this after staging, so the MFMAs run while the staging instructions issue
    auto fold = [&](const f32x4_t (&a)[kMG], int st) {
        const int ng = min(kMG, G - kMG * st);
#pragma unroll
        for (int q = 0; q < kMG; ++q)
            if (q < ng)
#pragma unroll
                for (int v = 0; v < 4; ++v) L[v] = L[v] + a[q][v];
    };
    // prologue: steps 0 and 1 staged, step 0's operands in registers, steps 2 and 3 loading
    Ops o0, o1;
    Loaded la, lb;
    load(la, 0);
    load(lb, 1);
    stage(0, 0, la);
    load(la, 2);
    __syncthreads();
    read_ops(o0, 0);
    stage(1, 1, lb);
    load(lb, 3);
    __syncthreads();
    // step st: its operands are in registers, step st + 1 is staged in LDS stage (st + 1) % 2 and
    // steps st + 2 and st + 3 are loading; read step st + 1's operands, run step st's MFMAs, stage
    // step st + 2 into stage st % 2 (every wave has read it: barrier of step st - 1), issue step
    // st + 4's loads
    f32x4_t acc[kMG];
    for (int st = 0; st < NS; st += 2) {
        mfma_step(o0, st, o1, 1, acc);
        stage(0, st + 2, la);
        load(la, st + 4);
        fold(acc, st);
        __syncthreads();
        if (st + 1 >= NS) break;
        mfma_step(o1, st + 1, o0, 0, acc);
        stage(1, st + 3, lb);
        load(lb, st + 5);
        fold(acc, st + 1);
        __syncthreads();
    }
    return L;
}
__global__ __launch_bounds__(256) void k_router_mfma(const uint16_t *__restrict__ x, int T, int d, int E,
                                                     const float *__restrict__ tab, const float *__restrict__ logit_bias,
                                                     float *__restrict__ logits, uint16_t *__restrict__ x16) {
    __shared__ RouterMfmaSmem sm;
    const int G = d / 64, NEB = cdiv(E, 16), NTB = cdiv(T, 64);
    const int xq = blockIdx.x / kXcds;
    const int eb = xq % NEB, tb = (xq / NEB) * kXcds + (int)(blockIdx.x % kXcds);
    if (tb >= NTB) return;   // the whole workgroup
    const f32x4_t L = x16 != nullptr ? router_mfma_tile<true>(sm, x, T, d, G, tb, eb, NEB, tab, x16)
                                     : router_mfma_tile<false>(sm, x, T, d, G, tb, eb, NEB, tab, x16);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int e = 16 * eb + (lane & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int t = 64 * tb + 16 * wave + 4 * (lane >> 4) + v;
        if (t < T && e < E) logits[(size_t)t * E + e] = logit_bias ? L[v] + logit_bias[e] : L[v];
    }
}

// MFMA router table (built at layer creation, k_router_mtable): per 16-expert block eb and
// group g, kMTile floats [lane l][s] with lane l = 16 k + c holding the weight of expert
// 16 eb + c, input 4 s + k of the group (fp32 fma(scale, q, bias); experts past E are zero).
// grid ceil(n / 256) with n = ceil(E / 16) * G * kMTile; block 256
__global__ __launch_bounds__(256) void k_router_mtable(const uint8_t *__restrict__ q, const uint32_t *__restrict__ sb,
                                                       int E, int d, float *__restrict__ out) {
    const int G = d / 64;
    const size_t n = (size_t)cdiv(E, 16) * G * kMTile;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int sidx = (int)(i % 16), l = (int)((i / 16) % 64);
    const size_t bg = i / kMTile;
    const int g = (int)(bg % G), eb = (int)(bg / G);
    const int e = 16 * eb + (l & 15), j = 4 * sidx + (l >> 4);
    float v = 0.0f;
    if (e < E) {
        const uint32_t w = sb[(size_t)e * G + g];
        v = __builtin_fmaf(bf16_to_f32(w & 0xFFFFu), (float)q[(size_t)e * d + 64 * g + j], bf16_to_f32(w >> 16));
    }
    out[i] = v;
}

// The router table the prefill routers read (weights fma(scale, q, bias) in fp32; layout above).
// grid ceil(n / 256) with n = ceil(E / kRNE) * G * kRBlk; block 256
__global__ __launch_bounds__(256) void k_router_table(const uint8_t *__restrict__ q, const uint32_t *__restrict__ sb,
                                                      int E, int d, float *__restrict__ out) {
    const int G = d / 64;
    const size_t n = (size_t)cdiv(E, kRNE) * G * kRBlk;
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int r = (int)(i % kRBlk);
    const size_t bg = i / kRBlk;
    const int g = (int)(bg % G), eb = (int)(bg / G);
    const int jc = r / (16 * kRNE), j = (r / kRNE) % 16, ii = r % kRNE;
    const int e = eb * kRNE + ii;
    float v = 0.0f;
    if (e < E) {
        const uint32_t w = sb[(size_t)e * G + g];
        v = __builtin_fmaf(bf16_to_f32(w & 0xFFFFu), (float)q[(size_t)e * d + 64 * g + 16 * jc + j], bf16_to_f32(w >> 16));
    }
    out[i] = v;
}

// (value desc, index asc) ordering
// grid: ceil(T / 4); block 256 -- one wave per token; kPer logits per lane (E <= 64 kPer).
// Round s takes the largest remaining logit (wave_max over DPP), ties to the lowest expert
// (the lowest set bit of a ballot); if every remaining logit is NaN, the lowest remaining
// expert, so the index stays valid.
template <int kPer>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ logits, int T, int E, int k,
                                              const uint16_t *__restrict__ pes, int32_t *__restrict__ idx,
                                              float *__restrict__ wout) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    const float *l = logits + (size_t)t * E;
    float v[kPer];
    bool live[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        live[i] = e < E;
        v[i] = live[i] ? l[e] : -__builtin_inff();
    }
    float my_v = 0.0f, m = 0.0f, z = 0.0f;   // lane s keeps slot s
    int my_i = 0;
    for (int s = 0; s < k; ++s) {
        float lb = -__builtin_inff();
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
        if (e < 0) {   // only NaN left
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
        if (lane == s) {
            my_v = val;
            my_i = e;
        }
    }
    if (lane < k) {
        const int e = min(max(my_i, 0), E - 1);
        idx[(size_t)t * k + lane] = e;
        const float w = __expf(my_v - m) / z;
        wout[(size_t)t * k + lane] = pes ? w * bf16_to_f32(pes[e]) : w;   // router epilogue
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

// Exclusive prefix sums of NV values per thread over threads 0 .. 64 nw - 1 of the block (v is
// replaced by its prefix; tot receives the totals; threads past them must hold zeros). ws: LDS
// of 16 x NV.
template <int NV>
__device__ __forceinline__ void block_scan(int (&v)[NV], int (&tot)[NV], int32_t (*ws)[NV], int nw) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int inc[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) inc[i] = v[i];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int t = __shfl_up(inc[i], o);
            if (lane >= o) inc[i] += t;
        }
    if (lane == 63)
#pragma unroll
        for (int i = 0; i < NV; ++i) ws[wave][i] = inc[i];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        int base = 0, total = 0;
        for (int w = 0; w < nw; ++w) {
            const int x = ws[w][i];
            if (w < wave) base += x;
            total += x;
        }
        v[i] = base + inc[i] - v[i];
        tot[i] = total;
    }
    __syncthreads();
}

constexpr int kScanPiece = 16384;   // chunk counts per LDS piece of the scan

// Class dealt o-th in launch m's lists: the classes by live rows of the tile (0: 97-128, 1: 65-96,
// 2: 33-64, 3: at most 32, narrow) in the order of their measured item durations, longest
// first (gate/up: 0, 1, 3, 2; down: 0, 1, 2, 3)
__device__ __forceinline__ int list_class(int m, int o) { return (m == 0 && o >= 2) ? 5 - o : o; }

// Arguments of the GEMM work-list build (gemm_list_cap has the list bound)
struct ListArgs {
    int T;                           // tokens of the chunk: cdiv(T, kMT) shared row tiles
    int nts[2], ntr[2], ntn[2];      // output tiles per row tile (shared, routed 128-row, narrow), per launch
    int cap[2];                      // list capacity per XCD, per launch
    int4 *list[2];                   // [kXcds][cap]: gate/up, down
    int32_t *list_n;                 // [2][kXcds]
};

// Counts, offsets, per-chunk bases and the work lists of the two GEMM launches. grid 1;
// block 1024 (thread e: expert e).
//  * chunk_base[c][e] becomes the number of pairs of expert e in chunks before c (the expert's
//    own start is added by the scatter), in pieces of whole chunks staged in LDS with coalesced
//    loads and stores.
//  * counts[e], offsets[e] (exclusive prefix; offsets[E] = all pairs).
//  * Work lists (one per launch and XCD; gemm_list_cap). Routed row tiles fall in four classes by
//    their live rows (97-128, 65-96, 33-64: 128-row items; at most 32: narrow items), dealt in
//    the order list_class gives (longest items first). A list holds, in this order, its share
//    of the shared-expert items (item i of S = cdiv(T, kMT) nts to XCD i % 8, in order) and,
//    per class, whole routed tiles (all their output tiles, so a tile's rows are fetched into
//    one L2): rank r of class c (expert order) goes to the XCD in position r % 8 of that
//    class's order, the XCDs sorted by the items they hold before the class (ties to the lower
//    XCD). The workgroups of an XCD start in list order, so the longest items start first and
//    the XCDs end together.
__global__ __launch_bounds__(1024) void k_bucket_scan(int nchunks, int E, int32_t *__restrict__ chunk_base,
                                                      int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                                      ListArgs la) {
    static_assert(kTileTabMax <= kScanPiece, "the tile table reuses the scan's piece buffer");
    __shared__ int32_t piece[kScanPiece];
    __shared__ int32_t ws[16][5];
    __shared__ int32_t seg[8][MOE_MAX_EXPERTS];
    __shared__ int32_t plan_sh[2][kXcds], plan_n[2][kXcds];
    __shared__ int32_t plan_start[2][4][kXcds], plan_pos[2][4][kXcds], plan_unit[2][4][kXcds];
    __shared__ int32_t carry[MOE_MAX_EXPERTS];   // pairs of each expert in the pieces so far
    const int tid = threadIdx.x, e = tid;
    const int pc = kScanPiece / E;   // chunks per piece (E <= 1024)
    if (e < E) carry[e] = 0;
    for (int c0 = 0; c0 < nchunks; c0 += pc) {
        const int nc = min(pc, nchunks - c0), n = nc * E;
        int32_t *blk = chunk_base + (size_t)c0 * E;
#pragma unroll
        for (int k0 = 0; k0 < kScanPiece / 1024; k0 += 8) {   // eight independent loads at a time
            int v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = tid + 1024 * (k0 + k);
                v[k] = i < n ? blk[i] : 0;
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = tid + 1024 * (k0 + k);
                if (i < n) piece[i] = v[k];
            }
        }
        __syncthreads();
        // thread (segment sg, expert ee) scans its segment of L consecutive chunks of the piece
        // for expert ee, starting from the totals of the expert's earlier segments and pieces
        {
            const int nseg = min(8, 1024 / E), L = (nc + nseg - 1) / nseg;
            const int sg = tid / E, ee = tid % E;
            const int c_lo = sg * L, c_hi = min(nc, c_lo + L);
            int tsum = 0;
            if (sg < nseg)
                for (int c = c_lo; c < c_hi; ++c) tsum += piece[c * E + ee];
            if (sg < nseg) seg[sg][ee] = tsum;
            __syncthreads();
            if (sg < nseg) {
                int r = carry[ee];
                for (int q = 0; q < sg; ++q) r += seg[q][ee];
                for (int c = c_lo; c < c_hi; ++c) {
                    const int x = piece[c * E + ee];
                    piece[c * E + ee] = r;
                    r += x;
                }
            }
            __syncthreads();
            if (e < E)
                for (int q = 0; q < nseg; ++q) carry[e] += seg[q][e];
        }
#pragma unroll
        for (int k = 0; k < kScanPiece / 1024; ++k) {
            const int i = tid + 1024 * k;
            if (i < n) blk[i] = piece[i];
        }
        __syncthreads();   // the piece is refilled
    }
    const bool ok = e < E;
    const int cnt = ok ? carry[e] : 0;
    // the expert's full row tiles and the class of its last one (-1: none past the full ones)
    const int nfull = cnt / kMT, rem = cnt - nfull * kMT;
    const int lastc = rem == 0 ? -1 : rem > 3 * kMT / 4 ? 0 : rem > kMT / 2 ? 1 : rem > kMT / 4 ? 2 : 3;
    int v[5] = {cnt, nfull + (lastc == 0 ? 1 : 0), lastc == 1 ? 1 : 0, lastc == 2 ? 1 : 0, lastc == 3 ? 1 : 0};
    int tot[5];
    block_scan<5>(v, tot, ws, min(16, (E + 63) / 64));
    if (ok) {
        counts[e] = cnt;
        offsets[e] = v[0];
    }
    if (tid == 0) offsets[E] = tot[0];

    // routed row tiles by class in LDS (the scan's piece buffer is free): class c from 0, cb1,
    // cb2, cb3, in expert order, each as expert << 20 | tile; the expert's first pair row and
    // pairs in seg
    const int cb1 = tot[1], cb2 = cb1 + tot[2], cb3 = cb2 + tot[3];
    if (ok) {
        seg[0][e] = v[0];
        seg[1][e] = cnt;
        const int n0 = nfull + (lastc == 0 ? 1 : 0);   // class-0 tiles: the full ones and a last one of 97+ rows
        for (int j = 0; j < n0; ++j)
            if (v[1] + j < kTileTabMax) piece[v[1] + j] = (e << 20) | j;
        if (lastc > 0) {
            const int i = (lastc == 1 ? cb1 : lastc == 2 ? cb2 : cb3) + v[1 + lastc];
            if (i < kTileTabMax) piece[i] = (e << 20) | nfull;
        }
    }

    // The plan of each launch (wave 0: gate/up, wave 1: down; lane x < 8: XCD x). Units of an
    // XCD's list, in order: its shared items (one item each), then per class in the launch's
    // order its routed tiles (n items each). Per XCD and class: the first unit, the first item
    // and the XCD's position in the class's dealing order.
    if (tid < 128 && (tid & 63) < kXcds) {
        const int m = tid >> 6, x = tid & 63;
        const int S = cdiv(la.T, kMT) * la.nts[m];
        int load = S > x ? (S - 1 - x) / kXcds + 1 : 0, units = load;
        plan_sh[m][x] = load;
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            const int c = list_class(m, o);
            const int n = c < 3 ? la.ntr[m] : la.ntn[m];
            const int mc = c == 0 ? tot[1] : c == 1 ? tot[2] : c == 2 ? tot[3] : tot[4];
            int pos = 0;   // XCDs holding fewer items (ties: lower XCDs) come first
#pragma unroll
            for (int y = 0; y < kXcds; ++y) {
                const int ly = __builtin_amdgcn_readlane(load, y);
                pos += (ly < load || (ly == load && y < x)) ? 1 : 0;
            }
            const int tiles = mc > pos ? (mc - 1 - pos) / kXcds + 1 : 0;
            plan_pos[m][o][x] = pos;
            plan_start[m][o][x] = load;
            plan_unit[m][o][x] = units;
            load += tiles * n;
            units += tiles;
        }
        plan_n[m][x] = units;
        la.list_n[m * kXcds + x] = min(load, la.cap[m]);   // load <= cap (gemm_list_cap)
    }
    __syncthreads();

    // The lists (threads [0, 512): gate/up, [512, 1024): down): thread tid takes units u, u + 64,
    // ... (u = tid % 512 / 8) of XCD tid % 8 and writes their items (item q of XCD x at x cap + q)
    {
        const int m = tid >> 9, x = tid & (kXcds - 1);
        const int cap = la.cap[m], nts = la.nts[m], nsh = plan_sh[m][x], nu = plan_n[m][x];
        int u0[4], q0[4], p0[4];
#pragma unroll
        for (int o = 0; o < 4; ++o) {
            u0[o] = plan_unit[m][o][x];
            q0[o] = plan_start[m][o][x];
            p0[o] = plan_pos[m][o][x];
        }
        int4 *list = la.list[m] + (size_t)x * cap;
        for (int u = (tid & 511) >> 3; u < nu; u += 512 / kXcds) {
            if (u < nsh) {   // shared item i = 8 u + x: row tile i / nts, output tile i % nts
                const int i = kXcds * u + x;
                if (u < cap) list[u] = make_int4((i % nts) << 16, (i / nts) | (kItemShared << 28), 0, la.T);
                continue;
            }
            int o = 0;
#pragma unroll
            for (int oo = 1; oo < 4; ++oo)
                if (u0[oo] <= u) o = oo;
            const int c = list_class(m, o);
            const int n = c < 3 ? la.ntr[m] : la.ntn[m];
            const int k = u - (o == 0 ? u0[0] : o == 1 ? u0[1] : o == 2 ? u0[2] : u0[3]);
            const int po = o == 0 ? p0[0] : o == 1 ? p0[1] : o == 2 ? p0[2] : p0[3];
            const int qs = (o == 0 ? q0[0] : o == 1 ? q0[1] : o == 2 ? q0[2] : q0[3]) + k * n;
            const int r = (c == 0 ? 0 : c == 1 ? cb1 : c == 2 ? cb2 : cb3) + po + kXcds * k;
            const int tv = piece[min(r, kTileTabMax - 1)];
            const int ex = min(tv >> 20, E - 1), j = tv & 0xFFFFF;
            const int kind = c < 3 ? kItemWide : kItemNarrow;
            const int oe = seg[0][ex], ce = seg[1][ex];
            for (int nt = 0; nt < n && qs + nt < cap; ++nt)
                list[qs + nt] = make_int4(ex | (nt << 16), j | (kind << 28), oe, ce);
        }
    }
}

// grid: nchunks; block 256
__global__ __launch_bounds__(256) void k_bucket_scatter(const int32_t *__restrict__ idx, int P, int E,
                                                        const int32_t *__restrict__ rank,
                                                        const int32_t *__restrict__ chunk_base,
                                                        const int32_t *__restrict__ offsets,
                                                        int32_t *__restrict__ perm, int32_t *__restrict__ pos,
                                                        int32_t *__restrict__ perm_out) {
    const int p = blockIdx.x * kChunk + threadIdx.x;
    if (p >= P) return;
    const int e = idx[p];
    const int q = offsets[e] + chunk_base[(size_t)blockIdx.x * E + e] + rank[p];
    perm[q] = p;
    pos[p] = q;
    if (perm_out) perm_out[q] = p;
}

}  // namespace

// k_router_ksplit while its launch has at most kRouterKsplitMaxWG workgroups (two per compute
// unit), k_router_mfma above; both give the same bits. Measured on the 2816-wide, 128-expert
// layer (router kernel, ksplit / mfma): 256 tokens 17.0 / 29.0 us, 512: 18.6 / 28.7, 1024:
// 31.0 / 30.2, 1536: 42.3 / 30.1, 2048: 53.7 / 30.9, 3072: 44.5 (mfma), 4096: 46 (mfma). The
// mfma kernel's floor at small chunks is one wave's 704 chained MFMAs, ~50 cycles apart in
// this loop (32 for the instruction alone).
static bool router_ksplit(int T, int E) { return (long)cdiv(T, 64) * cdiv(E, kRNE) <= kRouterKsplitMaxWG; }

hipError_t launch_router(const moe_layer *L, const uint16_t *x, int T, float *logits, hipStream_t s,
                         bool write_aux) {
    const int d = L->dims.d_model, E = L->dims.n_experts;
    if (d / 64 <= kKSplitMaxG && router_ksplit(T, E))
        launch(k_router_ksplit, dim3(cdiv(T, 64), cdiv(E, kRNE)), dim3(64 * kKW), 0, s, x, T, d, E, L->ws.rqf,
               L->w.logit_bias, logits, write_aux ? L->ws.x16 : nullptr);
    else
        launch(k_router_mfma, dim3(kXcds * cdiv(cdiv(T, 64), kXcds) * cdiv(E, 16)), dim3(256), 0, s, x, T, d, E,
               L->ws.rqm, L->w.logit_bias, logits, write_aux ? L->ws.x16 : nullptr);
    return hipGetLastError();
}

size_t router_table_floats(const moe_dims &D) { return (size_t)cdiv(D.n_experts, kRNE) * (D.d_model / 64) * kRBlk; }
size_t router_mtable_floats(const moe_dims &D) { return (size_t)cdiv(D.n_experts, 16) * (D.d_model / 64) * kMTile; }

hipError_t launch_router_table(const moe_layer *L, hipStream_t s) {
    const uint8_t *q = static_cast<const uint8_t *>(L->w.router.codes);
    const size_t n = router_table_floats(L->dims), nm = router_mtable_floats(L->dims);
    launch(k_router_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, q, L->w.router.sb, L->dims.n_experts,
           L->dims.d_model, L->ws.rqf);
    launch(k_router_mtable, dim3((unsigned)((nm + 255) / 256)), dim3(256), 0, s, q, L->w.router.sb,
           L->dims.n_experts, L->dims.d_model, L->ws.rqm);
    return hipGetLastError();
}

hipError_t launch_topk(const moe_layer *L, int T, const float *logits, int32_t *idx, float *w, hipStream_t s) {
    const int E = L->dims.n_experts, k = L->dims.top_k;
    const uint16_t *pes = L->w.per_expert_scale;
    if (E <= 128) launch(k_topk<2>, dim3(cdiv(T, 4)), dim3(256), 0, s, logits, T, E, k, pes, idx, w);
    else if (E <= 256) launch(k_topk<4>, dim3(cdiv(T, 4)), dim3(256), 0, s, logits, T, E, k, pes, idx, w);
    else launch(k_topk<MOE_MAX_EXPERTS / 64>, dim3(cdiv(T, 4)), dim3(256), 0, s, logits, T, E, k, pes, idx, w);
    return hipGetLastError();
}

hipError_t launch_bucket_rank(const moe_layer *L, int T, const int32_t *idx, hipStream_t s) {
    const int P = T * L->dims.top_k;
    launch(k_bucket_rank, dim3(cdiv(P, kChunk)), dim3(kChunk), 0, s, idx, P, L->dims.n_experts,
                       L->ws.rank, L->ws.chunk_base);
    return hipGetLastError();
}

hipError_t launch_bucket_scan(const moe_layer *L, int T, hipStream_t s) {
    const int P = T * L->dims.top_k;
    ListArgs la{};
    la.T = T;
    for (int m = 0; m < 2; ++m) {
        const GemmTiles g = gemm_tiles(L->dims, m);
        la.nts[m] = g.nts;
        la.ntr[m] = g.ntr;
        la.ntn[m] = g.ntn;
        la.cap[m] = gemm_list_cap(L->dims, T, m);
        la.list[m] = L->ws.list[m];
    }
    la.list_n = L->ws.list_n;
    launch(k_bucket_scan, dim3(1), dim3(1024), 0, s, cdiv(P, kChunk), L->dims.n_experts, L->ws.chunk_base,
           L->ws.counts, L->ws.offsets, la);
    return hipGetLastError();
}

hipError_t launch_bucket_scatter(const moe_layer *L, int T, const int32_t *idx, int32_t *perm_out, hipStream_t s) {
    const int P = T * L->dims.top_k;
    launch(k_bucket_scatter, dim3(cdiv(P, kChunk)), dim3(kChunk), 0, s, idx, P, L->dims.n_experts,
                       L->ws.rank, L->ws.chunk_base, L->ws.offsets, L->ws.perm, L->ws.pos, perm_out);
    return hipGetLastError();
}

hipError_t launch_router_prologue(const moe_layer *L, const uint16_t *x, int T, bool for_prefill, hipStream_t s) {
    launch(k_router_prologue, dim3(T), dim3(256), 0, s, x, L->dims.d_model, L->w.router_scale, L->ws.u,
           for_prefill ? L->ws.x16 : nullptr, for_prefill ? nullptr : L->ws.dxg,
           L->dims.expert_format == MOE_FORMAT_Q4_0 ? 32 : 64);
    return hipGetLastError();
}

}  // namespace qmoe
