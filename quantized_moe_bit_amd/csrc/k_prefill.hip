// Prefill path: grouped GEMM over expert-bucketed token rows on gfx950 MFMA.
//
// Token/expert pairs of a chunk are grouped by expert (Mference system design,
// "Prefill"); each expert's rows then form one dense GEMM against its 4-bit
// group-64 affine weights. The Mference design unpacks an affine tile into bounded
// FP16 staging and hands it to a matrix unit ("Prefill"; "Metal execution"); here each
// wave turns its codes into fp16 MFMA operands in registers: with a power-of-two
// exponent m per matrix (chosen from the matrix's largest |scale|, see k_stage_shift), the
// staged weight is fp16(2^m (scale * q + bias)), formed by one packed fp16 fma per two
// weights (a single rounding of the exact value, 11 significant bits for scales of any
// magnitude), and the fp32 accumulators are scaled back by 2^-m (exact). The activations
// are fp16 too (x converted exactly from bf16 by the router; the hidden activation
// h = gelu(g) * u is carried in fp16), and v_mfma_f32_32x32x16_f16 accumulates in fp32
// across all groups. Q4_0 expert matrices (weight d (q - 8), one fp16 d per 32 inputs) take the
// same path with scale d and bias -8 d, the K-steps of a group's first 32 inputs using its
// first block's d and the last two K-steps its second block's. An 11-bit d times a 4-bit code
// does not fit fp16's 11 significant bits, so d is split into d_hi (its leading 8 bits) and
// d_lo = d - d_hi (at most 3 bits): both products are exact in fp16 (d_lo's down to the fp16
// subnormal quantum 2^-24 of the staged scale), and each K-step runs one MFMA per part into the
// same accumulator.
//
// Work items: (expert or shared, 128-row tile, output tile), one per workgroup, taken from the
// work list of the workgroup's XCD (workgroup b runs on XCD b % 8 and takes item b / 8 of its
// list; the lists are built with the grouping so that the XCDs get about the same work, the
// longest items first, and all output tiles of a routed row tile on one XCD, so its rows are
// fetched into one L2). Routed tiles with at most 32 live rows take a narrow workgroup tile
// (32 token rows x 512 weight rows) in the same launch.
#include <type_traits>

#include "device_common.h"
#include "moe_internal.h"

namespace qmoe {
namespace {

constexpr int kPreWG = 256;

// Workgroup tile: 128 token rows x 256 weight rows (down: output columns). Wave w owns 64
// weight rows as two 32-row code tiles for all 128 token rows: gate/up -> the gate and the up
// tile of hidden block 4 nt + w (32 hidden units), so GeGLU needs no exchange between waves;
// down -> row blocks 2 (4 nt + w) and 2 (4 nt + w) + 1 of the down matrix. acc is 4 x 2
// tiles of 32 x 32 fp32; two workgroups per compute unit.
//
// LDS rings of the K loop (one 64-input group per step). A ring: kAStages stages of the A
// tile (128 rows x 64 inputs, 16-bit, rows of 128 B with the 16-byte chunks XOR-swizzled),
// loaded one step ahead by all four waves together. B ring: kBStages stages of the eight
// 1 KiB code tiles and their scale/bias words (64 per tile, rows duplicated), each wave
// loading its own two tiles two steps ahead. Everything arrives by direct global->LDS loads,
// so no staging registers are needed. The K loop is unrolled by kUnroll steps, a multiple of
// both ring lengths, so every stage offset is a constant.
constexpr int kAStages = 2;
constexpr int kBStages = 4;
constexpr int kUnroll = 4;
constexpr int kADist = 1;   // steps the A loads run ahead
constexpr int kBDist = 2;   // steps the B loads run ahead
static_assert(kADist <= kBDist, "the prologue issues A no earlier than B");
static_assert(kADist < kAStages && kBDist < kBStages, "a stage is refilled only after its step");
static_assert(kUnroll % kAStages == 0 && kUnroll % kBStages == 0, "constant stages per unrolled step");
constexpr int kAStageBytes = kMT * 128;
constexpr int kBStageBytes = 4 * 2 * 1024;
constexpr int kSStageBytes = 4 * 2 * 256;
constexpr int kBRingOff = kAStages * kAStageBytes;
constexpr int kSRingOff = kBRingOff + kBStages * kBStageBytes;
constexpr int kSmemBytes = kSRingOff + kBStages * kSStageBytes;
static_assert(2 * kSmemBytes <= 159744, "two workgroups per compute unit");
constexpr int kDmaPerStep = 8;   // per thread: 4 A chunks, 2 code chunks, 2 scale/bias words
// Direct loads issued after the A chunks of step g up to the barrier of step g, and after the
// scale/bias words of step g + 1 up to their use at the end of step g (every step issues the
// same eight loads, the prologue the same pattern).
constexpr int kWaitA = 4 + kDmaPerStep * (kADist - 1);
constexpr int kWaitB = kDmaPerStep * (kBDist - 1);
// loads the prologue issues after the scale/bias words of step 0 (steps -kBDist + 1 .. -1: A when
// it has started, then B)
constexpr int prologue_after_b0() {
    int n = 0;
    for (int j = -kBDist + 1; j < 0; ++j) n += (j + kADist >= 0 ? 4 : 0) + 4;
    return n;
}
constexpr int kWaitB0 = prologue_after_b0();
// gate/up epilogue: each wave's h tile, 128 rows x 32 fp16 (rows 96 B apart: the two rows one
// 16-bit store instruction writes start 32 banks apart)
constexpr int kHPitch = 48;
constexpr int kHTile = kMT * kHPitch * 2;
static_assert(4 * kHTile <= kSmemBytes, "h tiles exceed the LDS rings");
// down epilogue: 64 rows x 256 fp32 per half (row pitch 264: the two rows one store
// instruction writes start 32 banks apart)
constexpr int kOPitch = 264;
static_assert(64 * kOPitch * 4 <= kSmemBytes, "down epilogue tile exceeds the LDS rings");

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
// Four direct loads of 16 bytes per lane from sbase + voff[i] to lds_base + 4096 i + 16 lane
// (the four 8-row A chunks of one wave), with one save and restore of M0. Each M0 write is
// followed by one wait state before the load that reads it.
__device__ __forceinline__ void dma16x4(const void *sbase, const uint32_t voff[4], const uint8_t *lds_base) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    const void *sb = uniform_ptr(sbase);
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %6\n\t"
        "s_add_u32 m0, m0, 0x1000\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %6\n\t"
        "s_add_u32 m0, m0, 0x1000\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %6\n\t"
        "s_add_u32 m0, m0, 0x1000\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %6\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(m), "s"(sb)
        : "memory", "scc");
}

// The wave's two code tiles (16 bytes per lane each, to lds_b and lds_b + 1024) and their
// scale/bias words (4 bytes per lane, to lds_s and lds_s + 256), one save and restore of M0.
__device__ __forceinline__ void dma_b(const void *sb0, const void *sb1, uint32_t voff_b, const uint8_t *lds_b,
                                      const void *ss0, const void *ss1, uint32_t voff_s, const uint8_t *lds_s) {
    const uint32_t mb = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_b);
    const uint32_t ms = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_s);
    const void *b0 = uniform_ptr(sb0), *b1 = uniform_ptr(sb1), *s0 = uniform_ptr(ss0), *s1 = uniform_ptr(ss1);
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %5\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %6\n\t"
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, %7\n\t"
        "s_add_u32 m0, m0, 0x100\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %2, %8\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(voff_b), "v"(voff_s), "s"(mb), "s"(ms), "s"(b0), "s"(b1), "s"(s0), "s"(s1)
        : "memory", "scc");
}

// All direct loads of one ring step with one save and restore of M0: the four A chunks
// (sbase_a + voff_a[i] -> lds_a + 4096 i + 16 lane), then the wave's two code tiles and
// their scale/bias words as in dma_b. Issue order is the one the counted waits assume.
__device__ __forceinline__ void dma_step(const void *sbase_a, const uint32_t voff_a[4], const uint8_t *lds_a,
                                         const void *sb0, const void *sb1, uint32_t voff_b, const uint8_t *lds_b,
                                         const void *ss0, const void *ss1, uint32_t voff_s, const uint8_t *lds_s) {
    const uint32_t ma = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_a);
    const uint32_t mb = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_b);
    const uint32_t ms = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_s);
    const void *sa = uniform_ptr(sbase_a);
    const void *b0 = uniform_ptr(sb0), *b1 = uniform_ptr(sb1), *s0 = uniform_ptr(ss0), *s1 = uniform_ptr(ss1);
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %7\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %10\n\t"
        "s_add_u32 m0, m0, 0x1000\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %10\n\t"
        "s_add_u32 m0, m0, 0x1000\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %3, %10\n\t"
        "s_add_u32 m0, m0, 0x1000\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %4, %10\n\t"
        "s_mov_b32 m0, %8\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %5, %11\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %5, %12\n\t"
        "s_mov_b32 m0, %9\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %6, %13\n\t"
        "s_add_u32 m0, m0, 0x100\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %6, %14\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(voff_a[0]), "v"(voff_a[1]), "v"(voff_a[2]), "v"(voff_a[3]), "v"(voff_b), "v"(voff_s), "s"(ma), "s"(mb),
          "s"(ms), "s"(sa), "s"(b0), "s"(b1), "s"(s0), "s"(s1)
        : "memory", "scc");
}

// Ring barrier of step g: step g's A tile has landed for this wave (direct loads retire in
// issue order and are counted by vmcnt) and for every wave (the barrier), which also frees
// the A stage about to be refilled; lgkmcnt(0): this wave's LDS reads of the stages about to
// be refilled are done.
__device__ __forceinline__ void ring_sync() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kWaitA) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// f(integral_constant<J>) for J = J0 .. N - 1, in order (the K loop's constant stage offsets)
template <int J0, int N, class F>
__device__ __forceinline__ void unroll_steps(F &&f) {
    if constexpr (J0 < N) {
        f(std::integral_constant<int, J0>{});
        unroll_steps<J0 + 1, N>(f);
    }
}

struct PreArgs {
    int T, d, k, I, Is, E;
    const uint16_t *x16;        // gate/up A rows [T, d], fp16
    const int32_t *perm;
    const int4 *list;           // [kXcds][cap] work items of this launch (Workspace::list)
    const int32_t *list_n;      // [kXcds] items in each XCD's list
    int cap;
    moe_qmat gate, up, sh_gate, sh_up, down, sh_down;
    uint16_t *h_r, *h_s;        // hidden activations (fp16): [T k, I] bucket order, [T, I_s]
    float *r, *sh;
    const int32_t *eslot;       // expert slots (null: expert e is matrix e of the routed arrays)
    int n_slots;
    int32_t *slot_faults;
    // expert tiles: routed items whose expert has no slot are skipped (not faults), and the
    // shared items run only with shared set
    int tile_mode, shared;
    const int32_t *shift;       // fp16 staging exponents: [kind * n_mats + matrix], shared at [3 n_mats + kind]
    int n_mats;
};

enum { kFmtAffine = 0, kFmtQ4_0 = 1 };

constexpr int kNMRows = 32;   // routed tiles with at most this many live rows run in the narrow-tile kernel

// Eight staged weights fp16(2^m (s q + b)) from one device-layout word (elements j = 0..7 of
// a K-step; element j in nibble j even ? j/2 : 4 + j/2, so pair p = elements 2p, 2p + 1 is
// nibbles p and 4 + p), given sc = {fp16(2^(24+m) s), fp16(2^(20+m) s)} and b2 = fp16(2^m b)
// in both halves. Each pair is masked out in place, as a pair of fp16 subnormals: pairs 0 and 1
// from the word, pairs 2 and 3 from the word shifted right by 8; nibbles at bits 0..3 / 16..19
// are q 2^-24 and take the 2^24 scale, nibbles at bits 4..7 / 20..23 are q 2^-20 and take the
// 2^20 scale (both exact), and one packed fma gives fp16(q s + b) times 2^m, rounded once: one
// shift, four ands and four fmas per eight weights. k_stage_shift chooses m so that
// 2^(24+m) |s| < 2^16 for every scale of the matrix (both fp16 scales are then exact, or for a
// scale below 2^-25 of the largest within 2^-24 of it).
__device__ __forceinline__ f16x8_t dequant_frag(uint32_t w, f16x2_t sc, f16x2_t b2) {
    const uint32_t lo = 0x000F000Fu, hi = 0x00F000F0u, w8 = w >> 8;
    const f16x2_t s24 = {sc[0], sc[0]}, s20 = {sc[1], sc[1]};
    u32x4_t r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, w & lo), s24, b2));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, w & hi), s20, b2));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, w8 & lo), s24, b2));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, w8 & hi), s20, b2));
    return __builtin_bit_cast(f16x8_t, r);
}

// fp16 staging exponent of one matrix. grid (n_mats + 1, 3): x = routed matrix (expert or
// slot, when routed is set, and for a layer with slots only a slot its table maps; x = n_mats:
// the shared expert, when shared is set), y = kind (gate, up, down);
// block 256. With e the bf16 exponent field of the matrix's largest |scale| (its value lies in
// [2^(e-127), 2^(e-126))), m = 118 - e puts that scale times 2^m in [2^-9, 2^-8): every scale
// times 2^(24+m) is then below 2^16 (an fp16 value), and every staged weight below
// 2^-4 + 2^m |bias|. A matrix whose scales are all zero takes m from its largest |bias|, placed
// in [2^14, 2^15). The matrix cannot be staged (m = 0, *faults += 1) if a scale or bias is NaN
// or infinite, m lies outside [-64, 64], or 2^m |bias| can reach 2^15.
// Q4_0 matrices (words d0 | d1 << 16, fp16): the same rule with the largest |d| as the
// largest scale; the biases -8 d then stay below 2^-5 after scaling, every finite fp16 d gives
// m in [-24, 15], and only a NaN or infinite d cannot be staged.
struct StageArgs {
    const uint32_t *sb[3];      // routed gate, up, down scale/bias words (n_mats matrices each)
    const uint32_t *sb_sh[3];   // shared gate, up, down
    int words[3], words_sh[3];  // words per matrix
    int n_mats, routed, shared;
    int32_t *shift, *faults;
    const int32_t *table;       // expert-to-slot table (layers with slots): only the slots it maps
    int E;                      // are read (others may be being filled)
    int q4_0;                   // Q4_0 expert matrices
};
__global__ __launch_bounds__(256) void k_stage_shift(StageArgs a) {
    const int kind = blockIdx.y, mat = blockIdx.x;
    const bool sh = mat == a.n_mats;
    if (sh ? !a.shared : !a.routed) return;
    if (!sh && a.table) {   // a slot the table does not map: no kernel of this call reads it
        __shared__ int mapped;
        if (threadIdx.x == 0) mapped = 0;
        __syncthreads();
        for (int e = threadIdx.x; e < a.E; e += 256)
            if (a.table[e] == mat) mapped = 1;
        __syncthreads();
        if (!mapped) return;
    }
    const int n = sh ? a.words_sh[kind] : a.words[kind];
    const uint32_t *w = sh ? a.sb_sh[kind] : a.sb[kind] + (size_t)mat * n;
    uint32_t smax = 0, bmax = 0;
    for (int i = threadIdx.x; i < n / 4; i += 256) {
        const u32x4_t v = ld16(w + 4 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (a.q4_0) {   // two fp16 scales; no biases
                smax = max(smax, max(v[j] & 0x7FFFu, (v[j] >> 16) & 0x7FFFu));
            } else {
                smax = max(smax, v[j] & 0x7FFFu);
                bmax = max(bmax, (v[j] >> 16) & 0x7FFFu);
            }
        }
    }
    for (int off = 32; off > 0; off >>= 1) {
        smax = max(smax, (uint32_t)__shfl_xor((int)smax, off));
        bmax = max(bmax, (uint32_t)__shfl_xor((int)bmax, off));
    }
    __shared__ uint32_t red[2][4];
    if ((threadIdx.x & 63) == 0) {
        red[0][threadIdx.x >> 6] = smax;
        red[1][threadIdx.x >> 6] = bmax;
    }
    __syncthreads();
    if (threadIdx.x != 0) return;
    smax = max(max(red[0][0], red[0][1]), max(red[0][2], red[0][3]));
    bmax = max(max(red[1][0], red[1][1]), max(red[1][2], red[1][3]));
    int m;
    bool bad;
    if (a.q4_0) {   // the fp32 exponent field of the largest |d| plays the bf16 one's part
        const int es = (int)((__builtin_bit_cast(uint32_t, f16_to_f32(smax)) >> 23) & 0xFF);
        m = smax ? 118 - es : 0;
        bad = smax >= 0x7C00u;
    } else {
        const int es = (int)(smax >> 7), eb = (int)(bmax >> 7);
        m = smax ? 118 - es : (bmax ? 141 - eb : 0);
        bad = smax >= 0x7F80u || bmax >= 0x7F80u || m < -64 || m > 64 || (bmax && eb + m > 141);
    }
    if (bad) {
        atomicAdd(a.faults, 1);
        m = 0;
    }
    a.shift[sh ? 3 * a.n_mats + kind : kind * a.n_mats + mat] = m;
}

// A 128-row work item of one GEMM launch (kind kItemShared or kItemWide; Workspace::list).
template <int MODE, int FMT>  // MODE 0: gate/up + GeGLU, 1: down; FMT: kFmtAffine / kFmtQ4_0
__device__ __forceinline__ void pre_gemm_wide(const PreArgs &a, uint8_t *smem, const int4 it) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, half = lane >> 5;

    // A-fragment byte offsets within a stage: row 32 ms + n, logical chunk 2 s + half sits
    // at aoff[s] + 4096 ms.
    int aoff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) aoff[s] = n * 128 + 16 * ((2 * s + half) ^ swz(n));

    // The work item: a row tile of the shared expert or of a routed expert with more than 32 live
    // rows, and its output tile nt
    const bool shared_item = (it.y >> 28) == kItemShared;
    const int nt = it.x >> 16, mt = it.y & 0xFFFFFFF;
    int e = 0, count, rowbase;
    if (shared_item) {
        if (!a.shared) return;
        count = a.T;
        rowbase = 0;
    } else {
        const int ex = it.x & 0xFFFF;
        if (a.tile_mode) {   // another tile's expert: its rows are computed by that tile's launch
            const int sl = a.eslot[ex];
            if (sl < 0 || sl >= a.n_slots) return;
        }
        e = expert_slot_of(a.eslot, a.n_slots, a.slot_faults, ex, MODE == 0 && nt == 0 && threadIdx.x == 0);
        rowbase = it.z;
        count = it.w;
    }
    const int K = MODE == 0 ? a.d : (shared_item ? a.Is : a.I);
    const int G = K / 64;   // ring steps: one 64-input group each
    const uint16_t *Asrc = MODE == 0 ? a.x16 : (shared_item ? a.h_s : a.h_r);

    // A source row of each tile row (-1: padding), staged at the start of the rings until every
    // wave has its load offsets
    int32_t *srow = reinterpret_cast<int32_t *>(smem);
    if (tid < kMT) {
        const int r = mt * kMT + tid;
        int src = -1;
        if (r < count) src = shared_item ? r : (MODE == 0 ? a.perm[rowbase + r] / a.k : rowbase + r);
        srow[tid] = src;
    }
    __syncthreads();
    // destination row of tile row r (-1: padding)
    auto drow = [&](int r) {
        const int rr = mt * kMT + r;
        return rr < count ? (shared_item ? 0 : rowbase) + rr : -1;
    };

    // The wave's block (gate/up: 32 hidden units; down: 64 output columns) and its two code
    // tiles. A wave past the end of the matrix (the last tile of a width that is not a multiple
    // of the tile) loads block 4 nt's tiles to keep the ring's load pattern and computes nothing.
    const int blk = 4 * nt + wave;
    const int J = MODE == 0 ? (shared_item ? a.Is : a.I) : a.d;   // rows of the weight matrices
    const bool live_w = MODE == 0 ? blk * 32 < J : blk * 64 < J;
    const uint8_t *Bt0, *Bt1;   // code tiles of step 0 (wave-uniform); lane adds 16 lane
    const uint8_t *St0, *St1;   // scale/bias words of step 0 (wave-uniform); lane adds 4 n
    {
        const int bl = live_w ? blk : 4 * nt;
        const moe_qmat *m0 = MODE == 0 ? (shared_item ? &a.sh_gate : &a.gate) : (shared_item ? &a.sh_down : &a.down);
        const moe_qmat *m1 = MODE == 0 ? (shared_item ? &a.sh_up : &a.up) : m0;
        const int rb0 = MODE == 0 ? bl : 2 * bl;
        const int rb1 = MODE == 0 ? bl : 2 * bl + 1;
        const size_t mat_bytes = (size_t)J * K / 2, mat_words = (size_t)J * G;
        Bt0 = static_cast<const uint8_t *>(m0->codes) + e * mat_bytes + (size_t)rb0 * G * 1024;
        Bt1 = static_cast<const uint8_t *>(m1->codes) + e * mat_bytes + (size_t)rb1 * G * 1024;
        St0 = reinterpret_cast<const uint8_t *>(m0->sb + e * mat_words + (size_t)rb0 * G * 32);
        St1 = reinterpret_cast<const uint8_t *>(m1->sb + e * mat_words + (size_t)rb1 * G * 32);
        Bt0 = static_cast<const uint8_t *>(uniform_ptr(Bt0));
        Bt1 = static_cast<const uint8_t *>(uniform_ptr(Bt1));
        St0 = static_cast<const uint8_t *>(uniform_ptr(St0));
        St1 = static_cast<const uint8_t *>(uniform_ptr(St1));
    }
    // fp16 staging exponents of the wave's two code tiles (gate/up: gate and up; down: down twice):
    // scales are multiplied by 2^(24+m) and 2^(20+m), biases by 2^m before the fp16 conversion,
    // the accumulators by 2^-m after the K loop
    float fS[2], fB[2], fR[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int kind = MODE == 0 ? t : 2;
        const int m = a.shift[shared_item ? 3 * a.n_mats + kind : kind * a.n_mats + e];
        fS[t] = __builtin_ldexpf(1.0f, 24 + m);
        fB[t] = __builtin_ldexpf(1.0f, m);
        fR[t] = __builtin_ldexpf(1.0f, -m);
    }
    const uint32_t boff = lane * 16, soff = n * 4;
    // A rows this thread moves: chunk i covers rows 8 (4 i + wave) .. +7, lane -> row
    // + lane/8 at physical chunk lane%8 (byte offsets from the buffer start). Padding rows
    // read the tile's first row (finite values; their results are discarded).
    uint32_t aro[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * (4 * i + wave) + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        int src = srow[r];
        if (src < 0) src = srow[0];
        aro[i] = ((uint32_t)src * K + 8 * c) * 2;
    }
    __syncthreads();   // srow is read; the ring loads may overwrite it

    // loads of the prologue: A chunks of step ga into A stage sa; the wave's code tiles and
    // scale/bias words of step gb into B stage sbi
    auto issue_a = [&](int ga, int sa) {
        dma16x4(reinterpret_cast<const uint8_t *>(Asrc) + 128 * ga, aro, smem + sa * kAStageBytes + wave * 1024);
    };
    auto issue_b = [&](int gb, int sbi) {
        dma_b(Bt0 + (size_t)gb * 1024, Bt1 + (size_t)gb * 1024, boff, smem + kBRingOff + sbi * kBStageBytes + wave * 2048,
              St0 + gb * 128, St1 + gb * 128, soff, smem + kSRingOff + sbi * kSStageBytes + wave * 512);
    };
    // raw code words and fp16 scale/bias pairs of the step whose tiles sit in B stage sbi:
    // [t][h] serves K-steps 2 h and 2 h + 1 (the same pair for both halves of an affine group;
    // Q4_0: block h of the group, scale d_h and bias -8 d_h, split into the parts hi, lo)
    auto load_w = [&](int sbi, u32x4_t (&bw)[2], f16x2_t (&s2)[2][2], f16x2_t (&b2)[2][2], f16x2_t (&s2l)[2][2],
                      f16x2_t (&b2l)[2][2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            bw[t] = ld16(smem + kBRingOff + sbi * kBStageBytes + wave * 2048 + t * 1024 + lane * 16);
            const uint32_t sbw =
                *reinterpret_cast<const uint32_t *>(smem + kSRingOff + sbi * kSStageBytes + wave * 512 + t * 256 + lane * 4);
            if constexpr (FMT == kFmtAffine) {
                const float sc = bf16_to_f32(sbw & 0xFFFFu) * fS[t], bi = bf16_to_f32(sbw >> 16) * fB[t];
                s2[t][0] = s2[t][1] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(sc, sc * 0.0625f));
                b2[t][0] = b2[t][1] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(bi, bi));
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float dh = f16_to_f32((sbw >> (16 * h)) & 0xFFFFu);
                    const float hi = __uint_as_float(__float_as_uint(dh) & 0xFFFF0000u), lo = dh - hi;   // exact
                    const float sc = hi * fS[t], bi = hi * (-8.0f * fB[t]);
                    const float scl = lo * fS[t], bil = lo * (-8.0f * fB[t]);
                    s2[t][h] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(sc, sc * 0.0625f));
                    b2[t][h] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(bi, bi));
                    s2l[t][h] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(scl, scl * 0.0625f));
                    b2l[t][h] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(bil, bil));
                }
            }
        }
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[ms][t][v] = 0.0f;
    // 32-row subtiles holding at least one real row (uniform)
    const int live = count - mt * kMT;
    const int live_ms = live >= kMT ? 4 : (live + 31) >> 5;

    // prologue, in the steady-state pattern of steps -kBDist .. -1
#pragma unroll
    for (int j = -kBDist; j < 0; ++j) {
        if (j + kADist >= 0) issue_a(min(j + kADist, G - 1), j + kADist);
        issue_b(min(j + kBDist, G - 1), j + kBDist);
    }

    // The K loop, instantiated per number of live 32-row subtiles (1..4) so that padding
    // subtiles cost nothing and the MFMA sequence stays branch-free. Within a step, K-step s
    // multiplies while the A fragments and the dequantized weights of K-step s + 1 are formed;
    // the code words of step g + 1 are read, and its K-step 0 dequantized, during K-step 3 of
    // step g.
    auto kloop = [&](auto lms_c) {
        constexpr int LMS = decltype(lms_c)::value;
        constexpr bool Q4 = FMT == kFmtQ4_0;
        u32x4_t bw[2];
        f16x2_t s2[2][2], b2[2][2], s2l[2][2], b2l[2][2];   // s2l, b2l: the d_lo part (Q4_0)
        f16x8_t bf0[2], bl0[2];   // K-step 0 of the next ring step, dequantized during K-step 3 of this one
        auto step = [&](auto j_c, int g) {
            constexpr int Ju = decltype(j_c)::value;
            constexpr int SA = Ju % kAStages, SAN = (Ju + kADist) % kAStages;
            constexpr int SB1 = (Ju + 1) % kBStages, SBN = (Ju + kBDist) % kBStages;
            ring_sync();
            {
                const int ga = min(g + kADist, G - 1), gb = min(g + kBDist, G - 1);
                dma_step(reinterpret_cast<const uint8_t *>(Asrc) + 128 * ga, aro, smem + SAN * kAStageBytes + wave * 1024,
                         Bt0 + (size_t)gb * 1024, Bt1 + (size_t)gb * 1024, boff,
                         smem + kBRingOff + SBN * kBStageBytes + wave * 2048, St0 + gb * 128, St1 + gb * 128, soff,
                         smem + kSRingOff + SBN * kSStageBytes + wave * 512);
            }
            // Scheduling: the LDS reads of K-step s + 1 (A fragments; in K-step 3 the next ring
            // step's code words and scale/bias words) are issued before the MFMAs of K-step s, so a
            // whole K-step of MFMAs covers their latency; the sched barriers keep the compiler from
            // sinking them next to their use. The dequantization VALU of K-step s + 1 interleaves
            // with the MFMAs of K-step s. K-loop note: the MFMA/dequantization phase of a K-step
            // runs at wave priority 1 (s_setprio), the LDS reads and ring barrier at 0, so of the two
            // waves sharing a SIMD (two workgroups per CU) the one with MFMAs ready issues first.
            if (live_w) {
                const uint8_t *sA = smem + SA * kAStageBytes;
                u32x4_t af[2][LMS];
                f16x8_t bf[2][2], bl[2][2];
#pragma unroll
                for (int ms = 0; ms < LMS; ++ms) af[0][ms] = ld16(sA + aoff[0] + 4096 * ms);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    bf[0][t] = bf0[t];
                    if constexpr (Q4) bl[0][t] = bl0[t];
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (s < 3) {
#pragma unroll
                        for (int ms = 0; ms < LMS; ++ms) af[(s + 1) & 1][ms] = ld16(sA + aoff[s + 1] + 4096 * ms);
                    } else {
                        // code words of step g + 1 (a past-the-end step reads a valid clamped stage);
                        // this K-step's fragments are already in registers
                        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWaitB) : "memory");
                        load_w(SB1, bw, s2, b2, s2l, b2l);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_setprio(1);   // MFMA phase first (see the K-loop note)
                    if (s < 3) {
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            const int hs = (s + 1) >> 1;
                            bf[(s + 1) & 1][t] = dequant_frag(bw[t][s + 1], s2[t][hs], b2[t][hs]);
                            if constexpr (Q4) bl[(s + 1) & 1][t] = dequant_frag(bw[t][s + 1], s2l[t][hs], b2l[t][hs]);
                        }
                    }
#pragma unroll
                    for (int ms = 0; ms < LMS; ++ms)
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            acc[ms][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                __builtin_bit_cast(f16x8_t, af[s & 1][ms]), bf[s & 1][t], acc[ms][t], 0, 0, 0);
                            if constexpr (Q4)
                                acc[ms][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                    __builtin_bit_cast(f16x8_t, af[s & 1][ms]), bl[s & 1][t], acc[ms][t], 0, 0, 0);
                        }
                    if (s == 3) {
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            bf0[t] = dequant_frag(bw[t][0], s2[t][0], b2[t][0]);
                            if constexpr (Q4) bl0[t] = dequant_frag(bw[t][0], s2l[t][0], b2l[t][0]);
                        }
                    }
                    __builtin_amdgcn_s_setprio(0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWaitB) : "memory");
            }
        };
        // B of step 0: issued first in the prologue
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kWaitB0) : "memory");
        if (live_w) {
            load_w(0, bw, s2, b2, s2l, b2l);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf0[t] = dequant_frag(bw[t][0], s2[t][0], b2[t][0]);
                if constexpr (Q4) bl0[t] = dequant_frag(bw[t][0], s2l[t][0], b2l[t][0]);
            }
        }
        int g = 0;
        for (; g + kUnroll <= G; g += kUnroll)
            unroll_steps<0, kUnroll>([&](auto j_c) { step(j_c, g + decltype(j_c)::value); });
        unroll_steps<0, kUnroll - 1>([&](auto j_c) {
            if (g + decltype(j_c)::value < G) step(j_c, g + decltype(j_c)::value);
        });
    };
    switch (live_ms) {
        case 1: kloop(std::integral_constant<int, 1>{}); break;
        case 2: kloop(std::integral_constant<int, 2>{}); break;
        case 3: kloop(std::integral_constant<int, 3>{}); break;
        default: kloop(std::integral_constant<int, 4>{}); break;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the clamped tail loads still land in the rings
    __syncthreads();   // every wave is done with the rings (no loads are outstanding)

    // ---- epilogue. Accumulator element v of lane l in tile (ms, t): token row 32 ms + 8 (v/4)
    // + 4 (l/32) + v%4, weight row l%32 of the wave's code tile t.
    if (MODE == 0) {
        // h = fp16(gelu(g) * u) in registers (tile 0: gate, tile 1: up, same hidden unit per
        // lane), staged through the wave's own LDS tile and written as 64-byte row pieces
        if (live_w) {
            uint16_t *hout = shared_item ? a.h_s : a.h_r;
            uint16_t *Hw = reinterpret_cast<uint16_t *>(smem + wave * kHTile);
#pragma unroll
            for (int ms = 0; ms < 4; ++ms) {
                if (ms < live_ms) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int row = 32 * ms + 8 * (v >> 2) + 4 * half + (v & 3);
                        Hw[row * kHPitch + n] =
                            (uint16_t)f32_to_f16(gelu_tanh_f32(acc[ms][0][v] * fR[0]) * (acc[ms][1][v] * fR[1]));
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            // lane -> row lane / 4 + 16 i, 16-byte chunk lane % 4
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int row = (lane >> 2) + 16 * i;
                const int dst = drow(row);
                if (row < 32 * live_ms && dst >= 0)
                    *reinterpret_cast<u32x4_t *>(hout + (size_t)dst * J + blk * 32 + 8 * (lane & 3)) =
                        *reinterpret_cast<const u32x4_t *>(Hw + row * kHPitch + 8 * (lane & 3));
            }
        }
    } else {
        // the 128 x 256 fp32 output tile leaves through LDS in two halves of 64 rows, each row
        // as one run of up to 1 KiB of 16-byte stores
        float *out = shared_item ? a.sh : a.r;
        float *O = reinterpret_cast<float *>(smem);
        const int c = tid & 63;   // 16-byte chunk of a row
        const bool col_ok = nt * 256 + 4 * c < a.d;
#pragma unroll
        for (int part = 0; part < 2; ++part) {
            if (2 * part < live_ms) {
                if (part) __syncthreads();   // the first half has left
                if (live_w) {
#pragma unroll
                    for (int mh = 0; mh < 2; ++mh)
#pragma unroll
                        for (int t = 0; t < 2; ++t)
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                const int row = 32 * mh + 8 * (v >> 2) + 4 * half + (v & 3);
                                O[row * kOPitch + wave * 64 + t * 32 + n] = acc[2 * part + mh][t][v] * fR[t];
                            }
                }
                __syncthreads();
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = (tid >> 6) + 4 * i;
                    const int dst = drow(64 * part + row);
                    if (col_ok && dst >= 0)
                        *reinterpret_cast<f32x4_t *>(out + (size_t)dst * a.d + nt * 256 + 4 * c) =
                            *reinterpret_cast<const f32x4_t *>(O + row * kOPitch + 4 * c);
                }
            }
        }
    }
}

// ----------------------------------------------------------------------------- narrow tiles
// Routed row tiles with at most 32 live rows (experts with few pairs, and the last tile of
// an expert whose pairs end just past a multiple of 128) run as narrow work items, after the
// 128-row ones in the same launch: 32 token rows x 512 weight rows per workgroup. In the 128-row kernel such a tile
// streams the weights of 256 weight rows and a 128-row A ring for a quarter of the MFMA work;
// here each weight is still dequantized once per tile, but the tile moves twice the weights
// per step behind one barrier, its A ring is a quarter of the size, and the weight ring runs
// two steps ahead with 16 KiB per wave in flight. Wave w owns four 32-row code tiles for the
// 32 token rows: gate/up -> gate and up of hidden blocks 8 nt + 2 w and 8 nt + 2 w + 1
// (tiles gate, up, gate, up); down -> row blocks 16 nt + 4 w .. 16 nt + 4 w + 3.
constexpr int kNM = kNMRows;                    // token rows per narrow tile
constexpr int kNStages = 3;                     // A and B ring stages (one step each)
constexpr int kNDist = 2;                       // steps the A and B loads run ahead
constexpr int kNUnroll = 3;
static_assert(kNDist < kNStages && kNUnroll % kNStages == 0, "narrow ring layout");
constexpr int kNAStageBytes = kNM * 128;        // 32 rows x 64 inputs, fp16, swizzled chunks
constexpr int kNBStageBytes = 4 * 4 * 1024;     // four waves x four code tiles
constexpr int kNSStageBytes = 4 * 4 * 256;      // their scale/bias words, rows duplicated
constexpr int kNBRingOff = kNStages * kNAStageBytes;
constexpr int kNSRingOff = kNBRingOff + kNStages * kNBStageBytes;
constexpr int kNSmemBytes = kNSRingOff + kNStages * kNSStageBytes;
static_assert(2 * kNSmemBytes <= 159744, "two narrow workgroups per compute unit");
constexpr int kNDmaPerStep = 9;                 // per thread: 1 A chunk, 4 code chunks, 4 scale/bias words
constexpr int kNWaitA = (kNDmaPerStep - 1) + kNDmaPerStep * (kNDist - 1);   // loads after step g's A chunk
constexpr int kNWaitB = kNDmaPerStep * (kNDist - 1);                        // loads after step g+1's words
constexpr int kNWaitB0 = 1 + 8;                 // prologue: A and B of step 1 follow step 0's words
constexpr int kNHPitch = 72;                    // gate/up epilogue: 32 rows x 64 fp16 per wave
constexpr int kNOPitch = 520;                   // down epilogue: 32 rows x 512 fp32
static_assert(4 * kNM * kNHPitch * 2 <= kNSmemBytes && kNM * kNOPitch * 4 <= kNSmemBytes, "narrow epilogue tiles");

// One ring step of a narrow tile with one save and restore of M0: the thread's A chunk
// (sbase_a + voff_a -> lds_a + 16 lane), the wave's four code tiles (b[t] + voff_b ->
// lds_b + 1024 t + 16 lane) and their scale/bias words (s[t] + voff_s -> lds_s + 256 t + 4 lane),
// in that order (the counted waits assume it).
__device__ __forceinline__ void dma_narrow(const void *sbase_a, uint32_t voff_a, const uint8_t *lds_a,
                                           const void *const b[4], uint32_t voff_b, const uint8_t *lds_b,
                                           const void *const sw[4], uint32_t voff_s, const uint8_t *lds_s) {
    const uint32_t ma = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_a);
    const uint32_t mb = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_b);
    const uint32_t ms = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_s);
    const void *sa = uniform_ptr(sbase_a);
    const void *b0 = uniform_ptr(b[0]), *b1 = uniform_ptr(b[1]), *b2 = uniform_ptr(b[2]), *b3 = uniform_ptr(b[3]);
    const void *s0 = uniform_ptr(sw[0]), *s1 = uniform_ptr(sw[1]), *s2 = uniform_ptr(sw[2]), *s3 = uniform_ptr(sw[3]);
    uint32_t save;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %7\n\t"
        "s_mov_b32 m0, %5\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %8\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %9\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %10\n\t"
        "s_add_u32 m0, m0, 0x400\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %11\n\t"
        "s_mov_b32 m0, %6\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %3, %12\n\t"
        "s_add_u32 m0, m0, 0x100\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %3, %13\n\t"
        "s_add_u32 m0, m0, 0x100\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %3, %14\n\t"
        "s_add_u32 m0, m0, 0x100\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %3, %15\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(save)
        : "v"(voff_a), "v"(voff_b), "v"(voff_s), "s"(ma), "s"(mb), "s"(ms), "s"(sa), "s"(b0), "s"(b1), "s"(b2), "s"(b3),
          "s"(s0), "s"(s1), "s"(s2), "s"(s3)
        : "memory", "scc");
}

__device__ __forceinline__ void ring_sync_narrow() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kNWaitA) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A narrow work item of one GEMM launch (kind kItemNarrow): a routed row tile with at most 32
// live rows and its output tile nt of 512 weight rows.
template <int MODE, int FMT>
__device__ __forceinline__ void pre_gemm_narrow(const PreArgs &a, uint8_t *smem, const int4 it) {
    constexpr bool Q4 = FMT == kFmtQ4_0;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, half = lane >> 5;

    const int ex = it.x & 0xFFFF, nt = it.x >> 16;
    const int mt = it.y & 0xFFFFFFF, rowbase = it.z, count = it.w;
    const int live = count - mt * kMT;   // 1 .. kNM (the list's class of the tile)
    if (a.tile_mode) {
        const int sl = a.eslot[ex];
        if (sl < 0 || sl >= a.n_slots) return;
    }
    const int e = expert_slot_of(a.eslot, a.n_slots, a.slot_faults, ex, MODE == 0 && nt == 0 && threadIdx.x == 0);
    const int K = MODE == 0 ? a.d : a.I;
    const int G = K / 64;
    const int J = MODE == 0 ? a.I : a.d;
    const uint16_t *Asrc = MODE == 0 ? a.x16 : a.h_r;

    // A row of this thread's chunk: tile row r = 8 wave + lane / 8 (padding rows read row 0)
    uint32_t aro;
    {
        const int r = 8 * wave + (lane >> 3);
        const int rr = r < live ? r : 0;
        const int src = MODE == 0 ? a.perm[rowbase + mt * kMT + rr] / a.k : rowbase + mt * kMT + rr;
        const int c = (lane & 7) ^ swz(r);
        aro = ((uint32_t)src * K + 8 * c) * 2;
    }
    int aoff[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) aoff[s] = n * 128 + 16 * ((2 * s + half) ^ swz(n));

    // the wave's four code tiles (a tile past the matrix reads tile 0 and is not stored)
    const void *Bt[4], *St[4];
    bool live_t[4];
    float fS[4], fB[4], fR[4];
    {
        const size_t mat_bytes = (size_t)J * K / 2, mat_words = (size_t)J * G;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const moe_qmat *m = MODE == 0 ? ((t & 1) ? &a.up : &a.gate) : &a.down;
            const int rb = MODE == 0 ? 8 * nt + 2 * wave + (t >> 1) : 16 * nt + 4 * wave + t;
            live_t[t] = rb * 32 < J;
            const int rbc = live_t[t] ? rb : 0;
            Bt[t] = uniform_ptr(static_cast<const uint8_t *>(m->codes) + e * mat_bytes + (size_t)rbc * G * 1024);
            St[t] = uniform_ptr(m->sb + e * mat_words + (size_t)rbc * G * 32);
            const int kind = MODE == 0 ? (t & 1) : 2;
            const int sh = a.shift[kind * a.n_mats + e];
            fS[t] = __builtin_ldexpf(1.0f, 24 + sh);
            fB[t] = __builtin_ldexpf(1.0f, sh);
            fR[t] = __builtin_ldexpf(1.0f, -sh);
        }
    }
    const bool live_w = live_t[0] || live_t[1] || live_t[2] || live_t[3];
    const uint32_t boff = lane * 16, soff = n * 4;
    auto issue = [&](int ga, int gb, int sa, int sbi) {
        const void *bs[4], *ss[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bs[t] = static_cast<const uint8_t *>(Bt[t]) + (size_t)gb * 1024;
            ss[t] = static_cast<const uint8_t *>(St[t]) + gb * 128;
        }
        dma_narrow(reinterpret_cast<const uint8_t *>(Asrc) + 128 * ga, aro, smem + sa * kNAStageBytes + wave * 1024, bs,
                   boff, smem + kNBRingOff + sbi * kNBStageBytes + wave * 4096, ss, soff,
                   smem + kNSRingOff + sbi * kNSStageBytes + wave * 1024);
    };
    // raw code words and fp16 scale/bias pairs of the step in B stage sbi ([t][h] as in k_pre_gemm)
    auto load_w = [&](int sbi, u32x4_t (&bw)[4], f16x2_t (&s2)[4][2], f16x2_t (&b2)[4][2], f16x2_t (&s2l)[4][2],
                      f16x2_t (&b2l)[4][2]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bw[t] = ld16(smem + kNBRingOff + sbi * kNBStageBytes + wave * 4096 + t * 1024 + lane * 16);
            const uint32_t sbw =
                *reinterpret_cast<const uint32_t *>(smem + kNSRingOff + sbi * kNSStageBytes + wave * 1024 + t * 256 + lane * 4);
            if constexpr (!Q4) {
                const float sc = bf16_to_f32(sbw & 0xFFFFu) * fS[t], bi = bf16_to_f32(sbw >> 16) * fB[t];
                s2[t][0] = s2[t][1] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(sc, sc * 0.0625f));
                b2[t][0] = b2[t][1] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(bi, bi));
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float dh = f16_to_f32((sbw >> (16 * h)) & 0xFFFFu);
                    const float hi = __uint_as_float(__float_as_uint(dh) & 0xFFFF0000u), lo = dh - hi;
                    const float sc = hi * fS[t], bi = hi * (-8.0f * fB[t]);
                    const float scl = lo * fS[t], bil = lo * (-8.0f * fB[t]);
                    s2[t][h] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(sc, sc * 0.0625f));
                    b2[t][h] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(bi, bi));
                    s2l[t][h] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(scl, scl * 0.0625f));
                    b2l[t][h] = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(bil, bil));
                }
            }
        }
    };

    f32x16_t acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[t][v] = 0.0f;

    // prologue: steps 0 .. kNDist - 1 into stages 0 .. kNDist - 1
#pragma unroll
    for (int p = 0; p < kNDist; ++p) issue(min(p, G - 1), min(p, G - 1), p, p);

    auto kloop = [&]() {
        u32x4_t bw[4];
        f16x2_t s2[4][2], b2[4][2], s2l[4][2], b2l[4][2];
        f16x8_t bf0[4], bl0[4];
        auto step = [&](auto j_c, int g) {
            constexpr int Ju = decltype(j_c)::value;
            constexpr int SA = Ju % kNStages, SN = (Ju + kNDist) % kNStages, SB1 = (Ju + 1) % kNStages;
            ring_sync_narrow();
            {
                const int gn = min(g + kNDist, G - 1);
                issue(gn, gn, SN, SN);
            }
            if (live_w) {
                const uint8_t *sA = smem + SA * kNAStageBytes;
                u32x4_t af[2];
                f16x8_t bf[2][4], bl[2][4];
                af[0] = ld16(sA + aoff[0]);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    bf[0][t] = bf0[t];
                    if constexpr (Q4) bl[0][t] = bl0[t];
                }
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (s < 3) {
                        af[(s + 1) & 1] = ld16(sA + aoff[s + 1]);
                    } else {
                        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kNWaitB) : "memory");
                        load_w(SB1, bw, s2, b2, s2l, b2l);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    __builtin_amdgcn_s_setprio(1);   // MFMA phase first (see the K-loop note)
                    if (s < 3) {
                        const int hs = (s + 1) >> 1;
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            bf[(s + 1) & 1][t] = dequant_frag(bw[t][s + 1], s2[t][hs], b2[t][hs]);
                            if constexpr (Q4) bl[(s + 1) & 1][t] = dequant_frag(bw[t][s + 1], s2l[t][hs], b2l[t][hs]);
                        }
                    }
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, af[s & 1]), bf[s & 1][t],
                                                                       acc[t], 0, 0, 0);
                        if constexpr (Q4)
                            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, af[s & 1]),
                                                                           bl[s & 1][t], acc[t], 0, 0, 0);
                    }
                    if (s == 3) {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            bf0[t] = dequant_frag(bw[t][0], s2[t][0], b2[t][0]);
                            if constexpr (Q4) bl0[t] = dequant_frag(bw[t][0], s2l[t][0], b2l[t][0]);
                        }
                    }
                    __builtin_amdgcn_s_setprio(0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kNWaitB) : "memory");
            }
        };
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kNWaitB0) : "memory");   // step 0's words
        if (live_w) {
            load_w(0, bw, s2, b2, s2l, b2l);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                bf0[t] = dequant_frag(bw[t][0], s2[t][0], b2[t][0]);
                if constexpr (Q4) bl0[t] = dequant_frag(bw[t][0], s2l[t][0], b2l[t][0]);
            }
        }
        int g = 0;
        for (; g + kNUnroll <= G; g += kNUnroll)
            unroll_steps<0, kNUnroll>([&](auto j_c) { step(j_c, g + decltype(j_c)::value); });
        unroll_steps<0, kNUnroll - 1>([&](auto j_c) {
            if (g + decltype(j_c)::value < G) step(j_c, g + decltype(j_c)::value);
        });
    };
    kloop();
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // ---- epilogue. Accumulator element v of lane l in tile t: token row 8 (v/4) + 4 (l/32) +
    // v%4, weight row l%32 of code tile t.
    auto drow = [&](int r) { return r < live ? rowbase + mt * kMT + r : -1; };
    if (MODE == 0) {
        // h = fp16(gelu(g) * u) of the wave's two hidden blocks, through its own LDS tile
        if (live_w) {
            uint16_t *Hw = reinterpret_cast<uint16_t *>(smem + wave * kNM * kNHPitch * 2);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = 8 * (v >> 2) + 4 * half + (v & 3);
                    Hw[row * kNHPitch + 32 * hb + n] = (uint16_t)f32_to_f16(
                        gelu_tanh_f32(acc[2 * hb][v] * fR[2 * hb]) * (acc[2 * hb + 1][v] * fR[2 * hb + 1]));
                }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            const int hb0 = 8 * nt + 2 * wave;
            // lane -> row lane / 8 + 8 i, 16-byte chunk lane % 8 of the 64 hidden units
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = (lane >> 3) + 8 * i, c = lane & 7;
                const int dst = drow(row);
                if (dst >= 0 && live_t[2 * (c >> 2)])
                    *reinterpret_cast<u32x4_t *>(a.h_r + (size_t)dst * J + 32 * hb0 + 8 * c) =
                        *reinterpret_cast<const u32x4_t *>(Hw + row * kNHPitch + 8 * c);
            }
        }
    } else {
        // the 32 x 512 fp32 output tile leaves through LDS, each row as one run of 16-byte stores
        float *O = reinterpret_cast<float *>(smem);
        if (live_w) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = 8 * (v >> 2) + 4 * half + (v & 3);
                    O[row * kNOPitch + wave * 128 + t * 32 + n] = acc[t][v] * fR[t];
                }
        }
        __syncthreads();
        const int c = tid & 127;   // 16-byte chunk of a row
        const bool col_ok = nt * 512 + 4 * c < a.d;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = (tid >> 7) + 2 * i;
            const int dst = drow(row);
            if (col_ok && dst >= 0)
                *reinterpret_cast<f32x4_t *>(a.r + (size_t)dst * a.d + nt * 512 + 4 * c) =
                    *reinterpret_cast<const f32x4_t *>(O + row * kNOPitch + 4 * c);
        }
    }
}

// One prefill GEMM launch: workgroup b takes item b / kXcds of XCD b % kXcds's list (past the
// list's items it exits), 128-row and narrow items side by side.
template <int MODE, int FMT>
__global__ __launch_bounds__(kPreWG, 2) void k_pre_gemm(PreArgs a) {
    static_assert(kNSmemBytes <= kSmemBytes, "one LDS buffer serves both tile kinds");
    __shared__ __align__(16) uint8_t smem[kSmemBytes];
    const int x = blockIdx.x % kXcds, q = blockIdx.x / kXcds;
    const int n = a.list_n[x];
    const int4 it = a.list[x * a.cap + q];   // in bounds: the grid is kXcds cap workgroups
    if (q >= n) return;
    if ((it.y >> 28) == kItemNarrow) pre_gemm_narrow<MODE, FMT>(a, smem, it);
    else pre_gemm_wide<MODE, FMT>(a, smem, it);
}

// y[t] = a_t sh[t] + sum_s w[t,s] * r[pos[t*k+s]] in slot order, a_t the shared-expert gate
// of token t from the fp16 copy of x (1 without a gate). grid (cdiv(d,1024), T); block 256
__global__ __launch_bounds__(kGlueWG) void k_combine(int d, int k, const float *__restrict__ sh,
                                                     const float *__restrict__ r, const int32_t *__restrict__ pos,
                                                     const float *__restrict__ wts, const uint16_t *__restrict__ x16,
                                                     const uint16_t *__restrict__ gvec, float *__restrict__ y) {
    __shared__ float gred[kGlueWG / 64];
    const int t = blockIdx.y;
    const int c = (blockIdx.x * kGlueWG + threadIdx.x) * 4;
    const float a = gvec ? shared_gate_token(x16 + (size_t)t * d, gvec, d, gred) : 1.0f;
    if (c >= d) return;
    f32x4_t acc = *reinterpret_cast<const f32x4_t *>(sh + (size_t)t * d + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= a;
    for (int s = 0; s < k; ++s) {
        const float w = wts[(size_t)t * k + s];
        // each routed output is read exactly once: non-temporal, so the stream does not evict
        // what the caches still hold for the other slots' rows
        const f32x4_t rv =
            __builtin_nontemporal_load(reinterpret_cast<const f32x4_t *>(r + (size_t)pos[(size_t)t * k + s] * d + c));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, rv[i], acc[i]);
    }
    st16_nt(y + (size_t)t * d + c, __builtin_bit_cast(u32x4_t, acc));
}

PreArgs make_args(const moe_layer *L, int T) {
    PreArgs a;
    const moe_dims &D = L->dims;
    a.T = T;
    a.d = D.d_model;
    a.k = D.top_k;
    a.I = D.d_expert;
    a.Is = D.d_shared;
    a.E = D.n_experts;
    a.x16 = L->ws.x16;
    a.perm = L->ws.perm;
    a.gate = L->w.gate;
    a.up = L->w.up;
    a.sh_gate = L->w.sh_gate;
    a.sh_up = L->w.sh_up;
    a.down = L->w.down;
    a.sh_down = L->w.sh_down;
    a.h_r = L->ws.h_r;
    a.h_s = L->ws.h_s;
    a.r = L->ws.r;
    a.sh = L->ws.sh;
    a.eslot = L->w.expert_slot;
    a.n_slots = L->w.n_slots;
    a.slot_faults = L->ws.slot_faults;
    a.tile_mode = 0;
    a.shared = 1;
    a.shift = L->ws.shift;
    a.n_mats = L->n_mats;
    return a;
}

// Workgroups of one prefill GEMM launch: kXcds lists of gemm_list_cap items.
int pre_grid(const moe_layer *L, int T, int mode) { return kXcds * gemm_list_cap(L->dims, T, mode); }

}  // namespace

hipError_t launch_stage_shift(const moe_layer *L, bool routed, bool shared, int32_t *faults, hipStream_t s) {
    const moe_dims &D = L->dims;
    const int d = D.d_model, I = D.d_expert, Is = D.d_shared;
    StageArgs a{};
    a.sb[0] = L->w.gate.sb;
    a.sb[1] = L->w.up.sb;
    a.sb[2] = L->w.down.sb;
    a.sb_sh[0] = L->w.sh_gate.sb;
    a.sb_sh[1] = L->w.sh_up.sb;
    a.sb_sh[2] = L->w.sh_down.sb;
    a.words[0] = a.words[1] = I * (d / 64);
    a.words[2] = d * (I / 64);
    a.words_sh[0] = a.words_sh[1] = Is * (d / 64);
    a.words_sh[2] = d * (Is / 64);
    a.n_mats = L->n_mats;
    a.routed = routed;
    a.shared = shared;
    a.shift = L->ws.shift;
    a.faults = faults;
    a.table = L->w.expert_slot;
    a.E = D.n_experts;
    a.q4_0 = D.expert_format == MOE_FORMAT_Q4_0;
    launch(k_stage_shift, dim3(L->n_mats + 1, 3), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pre_gateup(const moe_layer *L, const uint16_t *x, int T, hipStream_t s, int tile) {
    (void)x;   // the GEMM reads the fp16 copy of x the router wrote
    PreArgs a = make_args(L, T);
    a.tile_mode = tile >= 0;
    a.shared = tile <= 0;
    a.list = L->ws.list[0];
    a.list_n = L->ws.list_n;
    a.cap = gemm_list_cap(L->dims, T, 0);
    const dim3 grid(pre_grid(L, T, 0));
    if (L->dims.expert_format == MOE_FORMAT_Q4_0)
        launch(k_pre_gemm<0, kFmtQ4_0>, grid, dim3(kPreWG), 0, s, a);
    else
        launch(k_pre_gemm<0, kFmtAffine>, grid, dim3(kPreWG), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pre_down(const moe_layer *L, int T, hipStream_t s, int tile) {
    PreArgs a = make_args(L, T);
    a.tile_mode = tile >= 0;
    a.shared = tile <= 0;
    a.list = L->ws.list[1];
    a.list_n = L->ws.list_n + kXcds;
    a.cap = gemm_list_cap(L->dims, T, 1);
    const dim3 grid(pre_grid(L, T, 1));
    if (L->dims.expert_format == MOE_FORMAT_Q4_0)
        launch(k_pre_gemm<1, kFmtQ4_0>, grid, dim3(kPreWG), 0, s, a);
    else
        launch(k_pre_gemm<1, kFmtAffine>, grid, dim3(kPreWG), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_combine(const moe_layer *L, int T, float *y, hipStream_t s) {
    const int d = L->dims.d_model;
    launch(k_combine, dim3(cdiv(d, 4 * kGlueWG), T), dim3(kGlueWG), 0, s, d, L->dims.top_k, L->ws.sh, L->ws.r,
                       L->ws.pos, L->ws.wts, L->ws.x16, L->w.shared_gate, y);
    return hipGetLastError();
}

}  // namespace qmoe
