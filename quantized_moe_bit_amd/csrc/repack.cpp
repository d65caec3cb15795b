// Host-side lossless repack between the canonical weight layout and the device
// layout the gfx950 kernels stream. Codes are moved bit-for-bit, never
// re-quantized: the importer keeps source affine values unchanged and a layout
// change must be exactly invertible (Mference system design, "Source weights and
// bounded repack"; "Correctness and safety invariants").
//
// Device layout of a 4-bit matrix [out, in] (out % 32 == 0, in % 64 == 0):
//   tiles of 32 rows x 64 inputs, 1 KiB each, ordered (row block rb, group g);
//   inside a tile, lane l in 0..63 owns 16 bytes at l*16: row rb*32 + l%32 and,
//   for step s in 0..3, the u32 at l*16 + 4*s holds inputs 64g + 16s + 8*(l/32) + j,
//   j = 0..7, element j in nibble (j even ? j/2 : 4 + j/2).
// That is the operand order of one lane of a 32x32x16 MFMA B fragment, and the nibble
// order lets two bf16 values be built from one shift and one and-or per pair.
// Scale/bias words: (scale | bias << 16), ordered (rb, g, row in block).
//
// Device layout of an 8-bit matrix [out, in]: codes unchanged (row-major bytes),
// scale/bias words ordered (row, group).
//
// Q4_0 expert matrices (32 weights per 18-byte block: fp16 d, then byte j holding element j
// in its low and element j + 16 in its high nibble; Gem native architecture, "M4 Max operating
// assumptions") take the same code tiles, their codes unchanged, and one word per (row, group
// of 64) holding the d of the group's two blocks: d0 | d1 << 16.
#include <cstdint>
#include <cstring>

#include "moe.h"
#include "moe_internal.h"

namespace {

// Eight consecutive 4-bit elements j = 0..7 sit in nibble j of a canonical little-endian
// word; the device word holds element j in nibble (j even ? j/2 : 4 + j/2), i.e. the even
// elements in its low half and the odd ones in its high half.
inline uint32_t compact_nibbles(uint32_t v) {   // nibbles 0, 2, 4, 6 of v -> nibbles 0..3
    v &= 0x0F0F0F0Fu;
    v = (v | (v >> 4)) & 0x00FF00FFu;
    return (v | (v >> 8)) & 0x0000FFFFu;
}
inline uint32_t spread_nibbles(uint32_t v) {    // nibbles 0..3 of v -> nibbles 0, 2, 4, 6
    v &= 0x0000FFFFu;
    v = (v | (v << 8)) & 0x00FF00FFu;
    return (v | (v << 4)) & 0x0F0F0F0Fu;
}
inline uint32_t to_device_word(uint32_t c) { return compact_nibbles(c) | (compact_nibbles(c >> 4) << 16); }
inline uint32_t to_canonical_word(uint32_t w) { return spread_nibbles(w) | (spread_nibbles(w >> 16) << 4); }

moe_status check(int32_t bits, int32_t n_mats, int32_t out_dim, int32_t in_dim) {
    if (bits != 4 && bits != 8) return qmoe::fail(MOE_E_QUANT, "repack: bits must be 4 or 8, got %d", bits);
    if (n_mats < 1 || out_dim < 1 || in_dim < 64)
        return qmoe::fail(MOE_E_SHAPE, "repack: bad sizes n_mats=%d out=%d in=%d", n_mats, out_dim, in_dim);
    if (in_dim % 64) return qmoe::fail(MOE_E_SHAPE, "repack: in_dim %d not a multiple of 64", in_dim);
    if (bits == 4 && out_dim % 32)
        return qmoe::fail(MOE_E_SHAPE, "repack: 4-bit out_dim %d not a multiple of 32", out_dim);
    return MOE_OK;
}

}  // namespace

extern "C" size_t moe_packed_bytes(int32_t bits, int32_t n_mats, int32_t out_dim, int32_t in_dim,
                                   int32_t part) {
    if ((bits != 4 && bits != 8) || n_mats < 1 || out_dim < 1 || in_dim < 64 || in_dim % 64) return 0;
    if (bits == 4 && out_dim % 32) return 0;
    const size_t n = (size_t)n_mats * out_dim;
    if (part == 0) return n * (size_t)in_dim * bits / 8;
    if (part == 1) return n * (size_t)(in_dim / 64) * 4;
    return 0;
}

extern "C" moe_status moe_repack(int32_t bits, int32_t n_mats, int32_t out_dim, int32_t in_dim,
                                 const moe_host_qmat *src, void *codes_out, uint32_t *sb_out) {
    qmoe::clear_error();
    moe_status st = check(bits, n_mats, out_dim, in_dim);
    if (st != MOE_OK) return st;
    if (!src || !src->codes || !src->scales || !src->biases || !codes_out || !sb_out)
        return qmoe::fail(MOE_E_INVALID, "repack: null pointer");
    const int G = in_dim / 64;
    uint8_t *dst = static_cast<uint8_t *>(codes_out);
    if (bits == 8) {
        std::memcpy(dst, src->codes, (size_t)n_mats * out_dim * in_dim);
        for (size_t i = 0; i < (size_t)n_mats * out_dim * G; ++i)
            sb_out[i] = (uint32_t)src->scales[i] | ((uint32_t)src->biases[i] << 16);
        return MOE_OK;
    }
    const size_t row_bytes = (size_t)in_dim / 2;
    const int RB = out_dim / 32;
    for (int m = 0; m < n_mats; ++m) {
        const uint8_t *cm = src->codes + (size_t)m * out_dim * row_bytes;
        const uint16_t *sm = src->scales + (size_t)m * out_dim * G;
        const uint16_t *bm = src->biases + (size_t)m * out_dim * G;
        uint8_t *dm = dst + (size_t)m * out_dim * row_bytes;
        uint32_t *wm = sb_out + (size_t)m * out_dim * G;
        for (int rb = 0; rb < RB; ++rb)
            for (int g = 0; g < G; ++g) {
                uint8_t *tile = dm + ((size_t)rb * G + g) * 1024;
                for (int l = 0; l < 64; ++l) {
                    const int row = rb * 32 + (l & 31), half = l >> 5;
                    const uint8_t *crow = cm + (size_t)row * row_bytes;
                    for (int s = 0; s < 4; ++s) {
                        // elements 64 g + 16 s + 8 half + (0..7): one canonical word
                        uint32_t c;
                        std::memcpy(&c, crow + (64 * g + 16 * s + 8 * half) / 2, 4);
                        const uint32_t word = to_device_word(c);
                        std::memcpy(tile + l * 16 + s * 4, &word, 4);
                    }
                }
                for (int r = 0; r < 32; ++r) {
                    const size_t si = (size_t)(rb * 32 + r) * G + g;
                    wm[((size_t)rb * G + g) * 32 + r] = (uint32_t)sm[si] | ((uint32_t)bm[si] << 16);
                }
            }
    }
    return MOE_OK;
}

extern "C" moe_status moe_unrepack(int32_t bits, int32_t n_mats, int32_t out_dim, int32_t in_dim,
                                   const void *codes_in, const uint32_t *sb_in, uint8_t *codes,
                                   uint16_t *scales, uint16_t *biases) {
    qmoe::clear_error();
    moe_status st = check(bits, n_mats, out_dim, in_dim);
    if (st != MOE_OK) return st;
    if (!codes_in || !sb_in || !codes || !scales || !biases)
        return qmoe::fail(MOE_E_INVALID, "unrepack: null pointer");
    const int G = in_dim / 64;
    const uint8_t *srcb = static_cast<const uint8_t *>(codes_in);
    if (bits == 8) {
        std::memcpy(codes, srcb, (size_t)n_mats * out_dim * in_dim);
        for (size_t i = 0; i < (size_t)n_mats * out_dim * G; ++i) {
            scales[i] = (uint16_t)(sb_in[i] & 0xFFFFu);
            biases[i] = (uint16_t)(sb_in[i] >> 16);
        }
        return MOE_OK;
    }
    const size_t row_bytes = (size_t)in_dim / 2;
    const int RB = out_dim / 32;
    for (int m = 0; m < n_mats; ++m) {
        const uint8_t *sm_ = srcb + (size_t)m * out_dim * row_bytes;
        const uint32_t *wm = sb_in + (size_t)m * out_dim * G;
        uint8_t *cm = codes + (size_t)m * out_dim * row_bytes;
        uint16_t *scm = scales + (size_t)m * out_dim * G;
        uint16_t *bcm = biases + (size_t)m * out_dim * G;
        for (int rb = 0; rb < RB; ++rb)
            for (int g = 0; g < G; ++g) {
                const uint8_t *tile = sm_ + ((size_t)rb * G + g) * 1024;
                for (int l = 0; l < 64; ++l) {
                    const int row = rb * 32 + (l & 31), half = l >> 5;
                    uint8_t *crow = cm + (size_t)row * row_bytes;
                    for (int s = 0; s < 4; ++s) {
                        uint32_t word;
                        std::memcpy(&word, tile + l * 16 + s * 4, 4);
                        const uint32_t c = to_canonical_word(word);
                        std::memcpy(crow + (64 * g + 16 * s + 8 * half) / 2, &c, 4);
                    }
                }
                for (int r = 0; r < 32; ++r) {
                    const uint32_t v = wm[((size_t)rb * G + g) * 32 + r];
                    const size_t si = (size_t)(rb * 32 + r) * G + g;
                    scm[si] = (uint16_t)(v & 0xFFFFu);
                    bcm[si] = (uint16_t)(v >> 16);
                }
            }
    }
    return MOE_OK;
}

namespace {

moe_status check_q4_0(int32_t n_mats, int32_t out_dim, int32_t in_dim) {
    if (n_mats < 1 || out_dim < 1 || in_dim < 64)
        return qmoe::fail(MOE_E_SHAPE, "repack_q4_0: bad sizes n_mats=%d out=%d in=%d", n_mats, out_dim, in_dim);
    if (in_dim % 64) return qmoe::fail(MOE_E_SHAPE, "repack_q4_0: in_dim %d not a multiple of 64", in_dim);
    if (out_dim % 32) return qmoe::fail(MOE_E_SHAPE, "repack_q4_0: out_dim %d not a multiple of 32", out_dim);
    return MOE_OK;
}

// Block element i (0..31) sits in byte 2 + (i % 16) of its block, in the low nibble for
// i < 16 and the high nibble otherwise.
inline int q4_0_code(const uint8_t *blk, int i) { return (blk[2 + (i & 15)] >> (4 * (i >> 4))) & 0xF; }

}  // namespace

extern "C" moe_status moe_repack_q4_0(int32_t n_mats, int32_t out_dim, int32_t in_dim, const uint8_t *blocks,
                                      void *codes_out, uint32_t *sb_out) {
    qmoe::clear_error();
    moe_status st = check_q4_0(n_mats, out_dim, in_dim);
    if (st != MOE_OK) return st;
    if (!blocks || !codes_out || !sb_out) return qmoe::fail(MOE_E_INVALID, "repack_q4_0: null pointer");
    const int G = in_dim / 64, RB = out_dim / 32;
    const size_t row_blocks = (size_t)in_dim / 32;
    uint8_t *dst = static_cast<uint8_t *>(codes_out);
    for (int m = 0; m < n_mats; ++m) {
        const uint8_t *bm = blocks + (size_t)m * out_dim * row_blocks * 18;
        uint8_t *dm = dst + (size_t)m * out_dim * (in_dim / 2);
        uint32_t *wm = sb_out + (size_t)m * out_dim * G;
        for (int rb = 0; rb < RB; ++rb)
            for (int g = 0; g < G; ++g) {
                uint8_t *tile = dm + ((size_t)rb * G + g) * 1024;
                for (int l = 0; l < 64; ++l) {
                    const int row = rb * 32 + (l & 31), half = l >> 5;
                    const uint8_t *brow = bm + (size_t)row * row_blocks * 18;
                    for (int s = 0; s < 4; ++s) {
                        // elements 64 g + 16 s + 8 half + (0..7) as one canonical word (element j in nibble j)
                        uint32_t c = 0;
                        for (int j = 0; j < 8; ++j) {
                            const int e = 64 * g + 16 * s + 8 * half + j;
                            c |= (uint32_t)q4_0_code(brow + (size_t)(e / 32) * 18, e % 32) << (4 * j);
                        }
                        const uint32_t word = to_device_word(c);
                        std::memcpy(tile + l * 16 + s * 4, &word, 4);
                    }
                }
                for (int r = 0; r < 32; ++r) {
                    const uint8_t *b0 = bm + ((size_t)(rb * 32 + r) * row_blocks + 2 * g) * 18, *b1 = b0 + 18;
                    const uint32_t d0 = (uint32_t)b0[0] | ((uint32_t)b0[1] << 8);
                    const uint32_t d1 = (uint32_t)b1[0] | ((uint32_t)b1[1] << 8);
                    wm[((size_t)rb * G + g) * 32 + r] = d0 | (d1 << 16);
                }
            }
    }
    return MOE_OK;
}

extern "C" moe_status moe_unrepack_q4_0(int32_t n_mats, int32_t out_dim, int32_t in_dim, const void *codes_in,
                                        const uint32_t *sb_in, uint8_t *blocks) {
    qmoe::clear_error();
    moe_status st = check_q4_0(n_mats, out_dim, in_dim);
    if (st != MOE_OK) return st;
    if (!codes_in || !sb_in || !blocks) return qmoe::fail(MOE_E_INVALID, "unrepack_q4_0: null pointer");
    const int G = in_dim / 64, RB = out_dim / 32;
    const size_t row_blocks = (size_t)in_dim / 32;
    const uint8_t *src = static_cast<const uint8_t *>(codes_in);
    for (int m = 0; m < n_mats; ++m) {
        const uint8_t *sm_ = src + (size_t)m * out_dim * (in_dim / 2);
        const uint32_t *wm = sb_in + (size_t)m * out_dim * G;
        uint8_t *bm = blocks + (size_t)m * out_dim * row_blocks * 18;
        for (int rb = 0; rb < RB; ++rb)
            for (int g = 0; g < G; ++g) {
                const uint8_t *tile = sm_ + ((size_t)rb * G + g) * 1024;
                for (int r = 0; r < 32; ++r) {
                    const uint32_t v = wm[((size_t)rb * G + g) * 32 + r];
                    uint8_t *b0 = bm + ((size_t)(rb * 32 + r) * row_blocks + 2 * g) * 18, *b1 = b0 + 18;
                    b0[0] = (uint8_t)(v & 0xFF);
                    b0[1] = (uint8_t)((v >> 8) & 0xFF);
                    b1[0] = (uint8_t)((v >> 16) & 0xFF);
                    b1[1] = (uint8_t)(v >> 24);
                    std::memset(b0 + 2, 0, 16);
                    std::memset(b1 + 2, 0, 16);
                }
                for (int l = 0; l < 64; ++l) {
                    const int row = rb * 32 + (l & 31), half = l >> 5;
                    uint8_t *brow = bm + (size_t)row * row_blocks * 18;
                    for (int s = 0; s < 4; ++s) {
                        uint32_t word;
                        std::memcpy(&word, tile + l * 16 + s * 4, 4);
                        const uint32_t c = to_canonical_word(word);
                        for (int j = 0; j < 8; ++j) {
                            const int e = 64 * g + 16 * s + 8 * half + j, i = e % 32;
                            brow[(size_t)(e / 32) * 18 + 2 + (i & 15)] |= (uint8_t)(((c >> (4 * j)) & 0xF) << (4 * (i >> 4)));
                        }
                    }
                }
            }
    }
    return MOE_OK;
}
