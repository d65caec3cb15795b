/* The C ABI used from plain C99 (no C++, no Python): the host-side calls of include/moe.h,
 * which need no GPU. Exits 0 when every check holds, else prints the failed check and exits 1.
 *   - moe_packed_bytes against the device layout's sizes (1 KiB code tiles of 32 rows x 64
 *     inputs, one scale/bias word per row and group);
 *   - moe_repack / moe_unrepack of a 4-bit stack of matrices round-trip bit for bit;
 *   - argument errors are status codes with a message, and nothing is written;
 *   - moe_layer_create refuses bad dimensions before any device work. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe.h"

static int failures = 0;
#define CHECK(cond)                                                       \
    do {                                                                  \
        if (!(cond)) {                                                    \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++failures;                                                   \
        }                                                                 \
    } while (0)

static uint32_t rng_state = 12345u;
static uint32_t next_u32(void) {   /* xorshift32: test data only */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 17;
    rng_state ^= rng_state << 5;
    return rng_state;
}

int main(void) {
    const int32_t n = 3, out = 64, in = 192, G = in / 64;
    size_t i;

    CHECK(strcmp(moe_status_str(MOE_OK), "MOE_OK") == 0);
    CHECK(strcmp(moe_status_str(MOE_E_SHAPE), "MOE_E_SHAPE") == 0);
    CHECK(moe_build_id() != NULL && strlen(moe_build_id()) > 0);

    /* sizes: 4-bit codes (out / 32) * G tiles of 1 KiB per matrix; one word per (row, group) */
    CHECK(moe_packed_bytes(4, n, out, in, 0) == (size_t)n * (out / 32) * G * 1024);
    CHECK(moe_packed_bytes(4, n, out, in, 1) == (size_t)n * out * G * 4);
    CHECK(moe_packed_bytes(8, 1, out, in, 0) == (size_t)out * in);
    CHECK(moe_packed_bytes(4, n, 48, in, 0) == 0);   /* out not a multiple of 32 */

    {
        const size_t ncodes = (size_t)n * out * in / 2, nsb = (size_t)n * out * G;
        uint8_t *codes = malloc(ncodes), *codes_back = malloc(ncodes);
        uint16_t *scales = malloc(nsb * 2), *biases = malloc(nsb * 2);
        uint16_t *scales_back = malloc(nsb * 2), *biases_back = malloc(nsb * 2);
        uint8_t *dev_codes = malloc(moe_packed_bytes(4, n, out, in, 0));
        uint32_t *dev_sb = malloc(moe_packed_bytes(4, n, out, in, 1));
        moe_host_qmat m;
        if (!codes || !codes_back || !scales || !biases || !scales_back || !biases_back || !dev_codes || !dev_sb) {
            fprintf(stderr, "host allocation failed\n");
            return 1;
        }
        for (i = 0; i < ncodes; ++i) codes[i] = (uint8_t)next_u32();
        for (i = 0; i < nsb; ++i) {
            scales[i] = (uint16_t)next_u32();
            biases[i] = (uint16_t)next_u32();
        }
        m.codes = codes;
        m.scales = scales;
        m.biases = biases;
        CHECK(moe_repack(4, n, out, in, &m, dev_codes, dev_sb) == MOE_OK);
        /* one sb word: (bf16 scale) | (bf16 bias << 16), word 0 = row 0, group 0 of matrix 0 */
        CHECK(dev_sb[0] == ((uint32_t)scales[0] | ((uint32_t)biases[0] << 16)));
        CHECK(moe_unrepack(4, n, out, in, dev_codes, dev_sb, codes_back, scales_back, biases_back) == MOE_OK);
        CHECK(memcmp(codes, codes_back, ncodes) == 0);
        CHECK(memcmp(scales, scales_back, nsb * 2) == 0);
        CHECK(memcmp(biases, biases_back, nsb * 2) == 0);

        /* a bad shape is a status code with a message, and the outputs stay untouched */
        memset(dev_sb, 0xA5, moe_packed_bytes(4, n, out, in, 1));
        CHECK(moe_repack(4, n, 48, in, &m, dev_codes, dev_sb) == MOE_E_SHAPE);
        CHECK(strlen(moe_last_error()) > 0);
        CHECK(dev_sb[0] == 0xA5A5A5A5u);
        CHECK(moe_repack(4, n, out, in, NULL, dev_codes, dev_sb) == MOE_E_INVALID);

        free(codes);
        free(codes_back);
        free(scales);
        free(biases);
        free(scales_back);
        free(biases_back);
        free(dev_codes);
        free(dev_sb);
    }

    {   /* dimensions are checked before the weights or the device are touched */
        moe_dims d;
        moe_weights w;
        moe_layer *layer = NULL;
        memset(&d, 0, sizeof d);
        memset(&w, 0, sizeof w);
        d.d_model = 2816;
        d.n_experts = 128;
        d.top_k = 8;
        d.d_expert = 704;
        d.d_shared = 2112;
        d.group = 64;
        d.router_bits = 8;
        d.expert_bits = 4;
        d.max_tokens = 16;
        d.expert_format = MOE_FORMAT_AFFINE_G64;
        d.d_model = 2800;   /* not a multiple of 64 */
        CHECK(moe_layer_create(&d, &w, 0, &layer) == MOE_E_SHAPE && layer == NULL);
        d.d_model = 2816;
        d.top_k = 129;      /* more than the experts */
        CHECK(moe_layer_create(&d, &w, 0, &layer) == MOE_E_SHAPE && layer == NULL);
        d.top_k = 8;
        d.group = 32;
        CHECK(moe_layer_create(&d, &w, 0, &layer) == MOE_E_QUANT && layer == NULL);
        d.group = 64;
        CHECK(moe_layer_create(&d, &w, 0, &layer) == MOE_E_INVALID && layer == NULL);   /* NULL weights */
        CHECK(moe_layer_create(&d, &w, 0, NULL) == MOE_E_INVALID);
    }

    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("C ABI host checks passed\n");
    return 0;
}
