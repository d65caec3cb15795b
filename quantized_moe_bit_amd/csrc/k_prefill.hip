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
// Work items: (expert or shared, 128-row tile, output tile), one per workgroup; all output
// tiles of a row tile run on the same XCD (workgroup i runs on XCD i % 8), so the row tile
// is fetched into one L2.
#include <type_traits>

#include "device_common.h"
#include "moe_internal.h"

namespace qmoe {
namespace {

constexpr int kPreWG = 256;

// LDS ring of the K loop: three stages, each an A tile (128 rows x 64 inputs, 16-bit, rows
// of 128 B with the 16-byte chunks XOR-swizzled), the four 1 KiB code tiles of the step and
// their scale/bias words (64 per wave, rows duplicated). Everything arrives by direct
// global->LDS loads, so no staging registers are needed.
constexpr int kStages = 3;
constexpr int kAStageBytes = kMT * 128;
constexpr int kBStageBytes = 4 * 1024;
constexpr int kSStageBytes = 4 * 256;
constexpr int kStageBytes = kAStageBytes + kBStageBytes + kSStageBytes;
constexpr int kSmemBytes = kStages * kStageBytes;
constexpr int kDmaPerStep = 6;   // per thread: 4 A chunks, 1 code chunk, 1 scale/bias word
// gate/up epilogue tiles (reusing the ring): u in fp32, then h in fp16
constexpr int kUPitch = 72;
constexpr int kHPitch = 72;
static_assert(kMT * kUPitch * 4 + kMT * kHPitch * 2 <= kSmemBytes, "epilogue tiles exceed the LDS ring");

// Physical 16-byte chunk of logical chunk c in A-tile row r is c ^ swz(r). 16 consecutive
// rows read at one logical chunk then hit 16 distinct 16-byte bank groups (and any 8
// consecutive rows 8 distinct ones), and swz depends on r mod 32 only, so the four 32-row
// subtiles of a lane share their offsets up to a constant.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 3); }

// Direct global->LDS load: every lane of the wave moves 16 (or 4) bytes from
// sbase + voff (sbase wave-uniform, voff a per-lane 32-bit byte offset) to lds_base +
// 16 lane (4 lane); lds_base is wave-uniform (both are read from lane 0). Issued as inline asm so that the compiler's
// wait insertion (which would wait for every outstanding direct load before any LDS read)
// stays out of the ring; the ring waits for them itself (ring_sync). M0 carries the LDS base
// and is restored afterwards.
__device__ __forceinline__ const void *uniform_ptr(const void *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const void *sbase, uint32_t voff, const uint8_t *lds_base) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    const void *sb = uniform_ptr(sbase);
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(voff), "s"(sb), "s"(m)
        : "memory");
}
__device__ __forceinline__ void dma4(const void *sbase, uint32_t voff, const uint8_t *lds_base) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    const void *sb = uniform_ptr(sbase);
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "global_load_lds_dword %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(voff), "s"(sb), "s"(m)
        : "memory");
}

// Ring barrier. Direct loads retire in issue order and are counted by vmcnt; every load of
// the ring goes through dma16/dma4 (six per thread per step), so "at most 6 outstanding"
// means every step but the last issued one has landed. The other vector loads of the
// workgroup are issued before the ring starts, so they only make the wait stricter.
// lgkmcnt(0): this wave's LDS reads of the stage about to be refilled are complete.
__device__ __forceinline__ void ring_sync(bool keep_one_step) {
    if (keep_one_step) asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
static_assert(kDmaPerStep == 6, "ring_sync encodes vmcnt(6)");

struct PreArgs {
    int T, d, k, I, Is, E;
    const uint16_t *x;          // gate/up A rows [T, d]
    const int32_t *perm, *offsets, *tile_off;
    const uint16_t *xsplit;     // [T, Ks_d]
    moe_qmat gate, up, sh_gate, sh_up, down, sh_down;
    uint16_t *h_r, *hsplit_r, *h_s, *hsplit_s;
    int Gp_d, Gp_I, Gp_Is;
    int Ks_d, Ks_I, Ks_Is;      // row strides of the split-sum buffers
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
    __shared__ __align__(16) uint8_t smem[kSmemBytes];
    __shared__ int32_t srow[kMT];   // A source row (-1: padding)
    __shared__ int32_t drow[kMT];   // destination row

    typedef typename OpT<MODE>::type op_t;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, half = lane >> 5;
    const int E = a.E;

    // A-fragment byte offsets within a stage: row 32 ms + n, logical chunk 2 s + half sits
    // at aoff[s] + 4096 ms.
    int aoff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) aoff[s] = n * 128 + 16 * ((2 * s + half) ^ swz(n));

    // Work item of this workgroup (one per workgroup). Shared-expert items come first, then
    // routed ones; within each part, 128-row tiles are dealt to the eight XCDs round-robin
    // (workgroup b runs on XCD b % 8, parts start at multiples of 8) and every output tile
    // of a row tile runs on the same XCD, so the row tile is fetched into one L2 only. The
    // routed part is sized for the worst case; workgroups past the real tiles exit at once.
    {
        const int Ms = cdiv(a.T, kMT), Ms8 = roundup(Ms, 8);
        const int NTs = MODE == 0 ? a.Is / 64 : a.d / 128;
        const int NTr = MODE == 0 ? a.I / 64 : a.d / 128;
        const int b = blockIdx.x, Gs = Ms8 * NTs;
        bool shared_item;
        int e = 0, mt, nt, count, rowbase;
        if (b < Gs) {
            const int j = b >> 3;
            shared_item = true;
            mt = 8 * (j / NTs) + (b & 7);
            nt = j % NTs;
            if (mt >= Ms) return;
            count = a.T;
            rowbase = 0;
        } else {
            const int i = b - Gs, j = i >> 3;
            shared_item = false;
            const int mg = 8 * (j / NTr) + (i & 7);
            nt = j % NTr;
            if (mg >= a.tile_off[E]) return;
            e = find_expert(a.tile_off, E, mg);
            mt = mg - a.tile_off[e];
            rowbase = a.offsets[e];
            count = a.offsets[e + 1] - rowbase;
        }
        const int K = MODE == 0 ? a.d : (shared_item ? a.Is : a.I);
        const int G = K / 64;
        const int Gp = MODE == 0 ? a.Gp_d : (shared_item ? a.Gp_Is : a.Gp_I);
        const int Ks = MODE == 0 ? a.Ks_d : (shared_item ? a.Ks_Is : a.Ks_I);
        const int nbs = 3 * Gp / 16;        // bias-term MFMA steps
        const int nbp = roundup(nbs, 12);   // ... padded with zero fragments in the table
        const int V = cdiv(nbs, 4);         // bias-term ring steps (64 K' columns each)
        const int S = V + G;                // ring steps of the item
        const uint16_t *Asrc = MODE == 0 ? a.x : (shared_item ? a.h_s : a.h_r);
        const uint16_t *Bsrc = MODE == 0 ? a.xsplit : (shared_item ? a.hsplit_s : a.hsplit_r);

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

        // Wave w owns one 32-row weight tile for all 128 token rows: gate/up -> gate blocks
        // 2nt, 2nt+1 (waves 0, 1) and up blocks 2nt, 2nt+1 (waves 2, 3); down -> block 4nt + w.
        const uint8_t *Bt;        // code tile of step 0 (wave-uniform); lane adds 16 lane
        const uint8_t *St;        // scale/bias words of step 0 (wave-uniform); lane adds 4 n
        const uint8_t *Tb;        // bias-term B' fragments, step 0, this lane
        {
            const moe_qmat *m = MODE == 0 ? (wave < 2 ? (shared_item ? &a.sh_gate : &a.gate)
                                                      : (shared_item ? &a.sh_up : &a.up))
                                          : (shared_item ? &a.sh_down : &a.down);
            const uint8_t *tb = MODE == 0 ? (wave < 2 ? (shared_item ? a.bt_sh_gate : a.bt_gate)
                                                      : (shared_item ? a.bt_sh_up : a.bt_up))
                                          : (shared_item ? a.bt_sh_down : a.bt_down);
            const int rows = MODE == 0 ? (shared_item ? a.Is : a.I) : a.d;
            const int rb = MODE == 0 ? 2 * nt + (wave & 1) : 4 * nt + wave;
            Bt = static_cast<const uint8_t *>(m->codes) + (size_t)e * rows * K / 2 + (size_t)rb * G * 1024;
            St = reinterpret_cast<const uint8_t *>(m->sb + (size_t)e * rows * G + (size_t)rb * G * 32);
            Bt = static_cast<const uint8_t *>(uniform_ptr(Bt));
            St = static_cast<const uint8_t *>(uniform_ptr(St));
            Tb = tb + (((size_t)e * (rows / 32) + rb) * 64 + lane) * nbp * 16;
        }
        const uint32_t boff = lane * 16, soff = n * 4;
        // A rows this thread moves: chunk i covers rows 8 (4 i + wave) .. +7, lane -> row
        // + lane/8 at physical chunk lane%8 (byte offsets from the buffer start). Padding rows
        // read the tile's first row (finite values; their results are discarded).
        uint32_t aro[4], apo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 8 * (4 * i + wave) + (lane >> 3);
            const int c = (lane & 7) ^ swz(r);
            int src = srow[r];
            if (src < 0) src = srow[0];
            aro[i] = ((uint32_t)src * K + 8 * c) * 2;
            apo[i] = ((uint32_t)src * Ks + 8 * c) * 2;
        }

        // stage of ring step t: real step g = t - V uses stage g % 3
        auto stage_of = [&](int t) { return (t - V + 3 * V) % 3; };
        auto issue = [&](int t) {
            uint8_t *sA = smem + stage_of(t) * kStageBytes;
            uint8_t *sB = sA + kAStageBytes;
            uint8_t *sS = sB + kBStageBytes;
            int g = 0;   // bias steps move step-0 codes too (unused)
            if (t < V) {
                const uint8_t *abase = reinterpret_cast<const uint8_t *>(Bsrc) + 128 * t;
#pragma unroll
                for (int i = 0; i < 4; ++i) dma16(abase, apo[i], sA + (4 * i + wave) * 1024);
            } else {
                g = t - V;
                const uint8_t *abase = reinterpret_cast<const uint8_t *>(Asrc) + 128 * g;
#pragma unroll
                for (int i = 0; i < 4; ++i) dma16(abase, aro[i], sA + (4 * i + wave) * 1024);
            }
            dma16(Bt + (size_t)g * 1024, boff, sB + wave * 1024);
            dma4(St + g * 128, soff, sS + wave * 256);
        };

        f32x16_t tot[4];
#pragma unroll
        for (int ms = 0; ms < 4; ++ms)
#pragma unroll
            for (int v = 0; v < 16; ++v) tot[ms][v] = 0.0f;
        const f32x16_t zero = tot[0];
        // 32-row subtiles holding at least one real row (uniform)
        const int live = count - mt * kMT;
        const int live_ms = live >= kMT ? 4 : (live + 31) >> 5;

        // The K loop, instantiated per number of live 32-row subtiles (1..4) so that padding
        // subtiles cost nothing and the MFMA sequence stays branch-free.
        auto kloop = [&](auto lms_c) {
            constexpr int LMS = decltype(lms_c)::value;
            // ---- bias term first: K' = 3 Gp, A' = [X_hi | X_lo | X_hi] rows of the split-sum
            // buffer, B' = [c_hi | c_hi | c_lo] (c = bias - 16 scale) from the table built at
            // layer creation; three ring steps (12 MFMA steps) of B' in registers at a time.
            for (int vc = 0; vc < V; vc += 3) {
                u32x4_t bp[12];
                const uint8_t *tb = Tb + (size_t)vc * 64;
#pragma unroll
                for (int j = 0; j < 12; ++j) bp[j] = ld16(tb + 16 * j);
                if (vc == 0) {
                    issue(0);
                    if (S > 1) issue(1);
                }
#pragma unroll
                for (int vv = 0; vv < 3; ++vv) {
                    const int t = vc + vv;
                    if (t < V) {
                        ring_sync(t + 1 < S);
                        if (t + 2 < S) issue(t + 2);
                        const uint8_t *sA = smem + stage_of(t) * kStageBytes;
                        const int nst = min(4, nbs - 4 * t);
#pragma unroll
                        for (int s = 0; s < 4; ++s) {
                            if (s < nst) {
                                const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bp[4 * vv + s]);
#pragma unroll
                                for (int ms = 0; ms < LMS; ++ms) {
                                    const bf16x8_t av =
                                        __builtin_bit_cast(bf16x8_t, ld16(sA + aoff[s] + 4096 * ms));
                                    tot[ms] = mfma32(av, b, tot[ms]);
                                }
                            }
                        }
                    }
                }
            }
            // ---- main loop: one 64-input group per ring step
            auto real_step = [&](int g, const uint8_t *sA) {
                const int t = V + g;
                ring_sync(t + 1 < S);
                if (t + 2 < S) issue(t + 2);
                const uint8_t *sB = sA + kAStageBytes;
                const uint8_t *sS = sB + kBStageBytes;
                const u32x4_t bw = ld16(sB + wave * 1024 + lane * 16);
                const uint32_t sbw = *reinterpret_cast<const uint32_t *>(sS + wave * 256 + lane * 4);
                f32x16_t acc[LMS];
                // A fragments of step s + 1 are read while step s multiplies
                u32x4_t af[2][LMS];
#pragma unroll
                for (int ms = 0; ms < LMS; ++ms) af[0][ms] = ld16(sA + aoff[0] + 4096 * ms);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (s < 3) {
#pragma unroll
                        for (int ms = 0; ms < LMS; ++ms) af[(s + 1) & 1][ms] = ld16(sA + aoff[s + 1] + 4096 * ms);
                    }
                    const op_t b = OpT<MODE>::frag(bw[s]);
#pragma unroll
                    for (int ms = 0; ms < LMS; ++ms)
                        acc[ms] = mfma32(__builtin_bit_cast(op_t, af[s & 1][ms]), b, s == 0 ? zero : acc[ms]);
                }
                const float s16 = 16.0f * bf16_to_f32(sbw & 0xFFFFu);
#pragma unroll
                for (int ms = 0; ms < LMS; ++ms)
#pragma unroll
                    for (int v = 0; v < 16; ++v) tot[ms][v] = fmaf(s16, acc[ms][v], tot[ms][v]);
            };
            if (V == 0) {   // no bias steps (only when Gp == 0, i.e. never for valid shapes)
                issue(0);
                if (S > 1) issue(1);
            }
            for (int g = 0; g < G; g += 3) {
                real_step(g, smem);
                if (g + 1 >= G) break;
                real_step(g + 1, smem + kStageBytes);
                if (g + 2 >= G) break;
                real_step(g + 2, smem + 2 * kStageBytes);
            }
        };
        switch (live_ms) {
            case 1: kloop(std::integral_constant<int, 1>{}); break;
            case 2: kloop(std::integral_constant<int, 2>{}); break;
            case 3: kloop(std::integral_constant<int, 3>{}); break;
            default: kloop(std::integral_constant<int, 4>{}); break;
        }
        __syncthreads();   // every wave is done with the ring (no loads are outstanding)

        // ---- epilogue. Accumulator element v of lane l in subtile ms: row 32 ms + 8 (v/4) +
        // 4 (l/32) + v%4, column l%32 of the wave's weight tile.
        if (MODE == 0) {
            // h = fp16(gelu(g) * u): the up waves hand u over through LDS, the gate waves form
            // h into an fp16 tile, then each row leaves as 16-byte stores and its 64-column
            // sum feeds the down projection's bias term
            const int J = shared_item ? a.Is : a.I;
            uint16_t *hout = shared_item ? a.h_s : a.h_r;
            float *U = reinterpret_cast<float *>(smem);
            uint16_t *Hs = reinterpret_cast<uint16_t *>(smem + kMT * kUPitch * 4);
            if (wave >= 2) {
#pragma unroll
                for (int ms = 0; ms < 4; ++ms)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = 32 * ms + 8 * (v >> 2) + 4 * half + (v & 3);
                        U[row * kUPitch + (wave - 2) * 32 + n] = tot[ms][v];
                    }
            }
            __syncthreads();
            if (wave < 2) {
#pragma unroll
                for (int ms = 0; ms < 4; ++ms)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = 32 * ms + 8 * (v >> 2) + 4 * half + (v & 3);
                        const float u = U[row * kUPitch + wave * 32 + n];
                        Hs[row * kHPitch + wave * 32 + n] = (uint16_t)f32_to_f16_sat(gelu_tanh_f32(tot[ms][v]) * u);
                    }
            }
            __syncthreads();
            const int row = tid >> 1, hh = tid & 1;
            const u32x4_t *src = reinterpret_cast<const u32x4_t *>(Hs + row * kHPitch + hh * 32);
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
                    const int Kso = shared_item ? a.Ks_Is : a.Ks_I;
                    uint16_t *hs = (shared_item ? a.hsplit_s : a.hsplit_r) + (size_t)dst * Kso;
                    const uint32_t hi = f32_to_bf16(H);
                    const uint32_t lo = f32_to_bf16(H - bf16_to_f32(hi));
                    hs[nt] = (uint16_t)hi;
                    hs[Gpo + nt] = (uint16_t)lo;
                    hs[2 * Gpo + nt] = (uint16_t)hi;
                }
            }
        } else {
            float *out = shared_item ? a.sh : a.r;
            const int c0 = (nt * 4 + wave) * 32 + n;
#pragma unroll
            for (int ms = 0; ms < 4; ++ms)
                if (ms < live_ms) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = 32 * ms + 8 * (v >> 2) + 4 * half + (v & 3);
                        const int dst = drow[row];
                        if (dst >= 0) out[(size_t)dst * a.d + c0] = tot[ms][v];
                    }
                }
        }
    }
}

// Bias-term B' fragments of one quantized matrix stack (n_mats x [rows, in]), laid out
// [matrix][32-row block rb][lane l][step st][8 bf16] with steps padded to a multiple of 12
// (zero fragments): the eight values for K' indices kk = 16 st + 8 (l / 32) + j, j = 0..7,
// of row rb*32 + l%32. With part = kk / Gp and g = kk % Gp, c = bias - 16 scale of group g,
// the value is c_hi (part 0, 1) or c_lo (part 2), and 0 for padding groups g >= G or part 3.
// grid: ceil(n_mats * rows/32 * 64 * steps_padded / 256); block 256
__global__ __launch_bounds__(256) void k_bias_table(const uint32_t *__restrict__ sb, int n_mats, int rows, int G,
                                                    int Gp, uint8_t *__restrict__ out) {
    const int steps = 3 * Gp / 16, sp = roundup(steps, 12);
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    const size_t total = (size_t)n_mats * (rows / 32) * 64 * sp;
    if (i >= total) return;
    const int st = (int)(i % sp);
    size_t r = i / sp;
    const int lane = (int)(r % 64);
    r /= 64;
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
            v2[h2] = (part < 3 && gg < G) ? bias_part(sbm[gg * 32], part) : 0u;
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
    a.Ks_d = L->Ks_d;
    a.Ks_I = L->Ks_I;
    a.Ks_Is = L->Ks_Is;
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

// Workgroups of one prefill GEMM launch: shared part (row tiles padded to a multiple of 8)
// plus the routed part sized for the worst case, cdiv(T k, 128) + min(E, T k) row tiles.
int pre_grid(const moe_layer *L, int T, int mode) {
    const moe_dims &D = L->dims;
    const int NTs = mode == 0 ? D.d_shared / 64 : D.d_model / 128;
    const int NTr = mode == 0 ? D.d_expert / 64 : D.d_model / 128;
    const int P = T * D.top_k;
    const int Mr = cdiv(P, kMT) + (D.n_experts < P ? D.n_experts : P);
    return roundup(cdiv(T, kMT), 8) * NTs + roundup(Mr, 8) * NTr;
}

}  // namespace

hipError_t launch_pre_gateup(const moe_layer *L, const uint16_t *x, int T, hipStream_t s) {
    launch(k_pre_gemm<0>, dim3(pre_grid(L, T, 0)), dim3(kPreWG), 0, s, make_args(L, x, T));
    return hipGetLastError();
}

hipError_t launch_pre_down(const moe_layer *L, int T, hipStream_t s) {
    launch(k_pre_gemm<1>, dim3(pre_grid(L, T, 1)), dim3(kPreWG), 0, s, make_args(L, nullptr, T));
    return hipGetLastError();
}

size_t bias_table_bytes(int n_mats, int rows, int in_dim) {
    const int Gp = roundup(in_dim / 64, 16);
    return (size_t)n_mats * (rows / 32) * 64 * roundup(3 * Gp / 16, 12) * 16;
}

hipError_t launch_bias_table(const moe_qmat &m, int n_mats, int rows, int in_dim, uint8_t *out, hipStream_t s) {
    const int G = in_dim / 64, Gp = roundup(G, 16);
    const size_t total = (size_t)n_mats * (rows / 32) * 64 * roundup(3 * Gp / 16, 12);
    launch(k_bias_table, dim3((unsigned)cdiv((int)total, 256)), dim3(256), 0, s, m.sb, n_mats, rows, G, Gp,
                       out);
    return hipGetLastError();
}

hipError_t launch_combine(const moe_layer *L, int T, float *y, hipStream_t s) {
    const int d = L->dims.d_model;
    launch(k_combine, dim3(cdiv(d, 1024), T), dim3(256), 0, s, d, L->dims.top_k, L->ws.sh, L->ws.r,
                       L->ws.pos, L->ws.wts, y);
    return hipGetLastError();
}

}  // namespace qmoe
