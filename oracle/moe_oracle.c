/*
 * CPU oracle for the quantized mixture-of-experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library calls, links or
 * loads this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do. It shares no code, header or table with the GPU path.
 *
 * What it computes, and where the pages define it:
 *
 *  - Affine group-64 dequantization: weight = scale * code + bias, BF16 scale and
 *    BF16 bias per 64 consecutive input elements, 8-bit router codes, 4-bit expert
 *    codes (Mference system design, "Why the runtime has this shape").
 *  - Q4_0 expert matrices, the alternative expert format: blocks of 32 elements in 18 bytes
 *    (Gem native architecture, "M4 Max operating assumptions"; "Ownership boundaries": the GGUF
 *    loader accepts Q4_0 matrices), read here as an fp16 scale d followed by 16 bytes of 4-bit
 *    codes, element j < 16 in the low nibble of byte j and element j + 16 in its high nibble,
 *    weight = d * (code - 8).
 *  - Router: one logit per expert from the 8-bit projection of the token, no
 *    softcap, top-8 by value, softmax over the selected logits (Mference,
 *    "Decode", the router listing; "Why the runtime has this shape" for the
 *    absent softcap). An optional per-expert logit bias models routing skew.
 *    Ties at the top-k boundary go to the lower expert index.
 *  - Token/expert grouping: the token/expert pairs of a chunk are grouped by
 *    expert (Mference, "Prefill").
 *  - Expert: a GELU-gated FFN (Gem architecture notes, "Ownership boundaries",
 *    the synthetic layer's GELU-gated FFN), gate and up projections, tanh-form
 *    GELU on the gate, product, down projection.
 *  - Shared expert: a dense branch on the same input, added without a routing
 *    weight (Mference, "Why the runtime has this shape"). Optionally gated per token
 *    (Mference system design, "Scope and limitations": the Qwen 3.6 layers have a gated
 *    shared expert): the branch is multiplied by sigmoid(g . x) for a learned bf16 vector
 *    g over the model dimension.
 *  - Combine: routed outputs reduced with the router weights and added to the
 *    shared branch (Mference, "Decode", the cb2 phase), in the fixed slot order
 *    (TinyTitan architecture, "Invariants": fp32-or-better accumulation in a fixed
 *    reduction order).
 *
 * Precision. The router logits decide integers (the top-k set), so they are
 * computed in the one fp32 order the GPU kernels also follow, written out in
 * orc_router_logits. Everything else is float64 and unrounded: dequantized
 * weights, the three projections, GELU, the expert hidden activation, routing
 * weights and the combine (the pages quantize weights, never the activation
 * between the gate/up and down projections).
 *
 * Pins: the tests under tests/ check each function here against hand-built
 * codec groups, exact integer arithmetic, a full sort, a dense brute force
 * written independently in NumPy, library GELU and closed forms, and the byte
 * accounting of the Mference expert blob.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ threads */
void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------ bf16 */
static float bf16_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static double bf16_f64(uint16_t b) { return (double)bf16_f32(b); }

/* Round a double straight to bf16 (8 significant bits), ties to even. */
uint16_t orc_f64_to_bf16(double v) {
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (isnan(a)) return (uint16_t)(sign | 0x7FC0u);
    int e;
    double m = frexp(a, &e);              /* a = m * 2^e, m in [0.5, 1) */
    /* value = (1.f) * 2^(e-1); normal bf16 needs e-1 >= -126 */
    if (e - 1 >= -126) {
        double r = nearbyint(ldexp(m, 8)); /* 8 significant bits, ties to even */
        if (r == 256.0) { r = 128.0; e += 1; }
        int ebits = (e - 1) + 127;
        if (ebits >= 255) return (uint16_t)(sign | 0x7F80u);
        return (uint16_t)(sign | (uint16_t)(ebits << 7) | (uint16_t)((int)r - 128));
    }
    /* subnormal: quantum 2^-133 */
    double r = nearbyint(ldexp(a, 133));
    return (uint16_t)(sign | (uint16_t)r); /* r == 128 carries into the exponent field */
}

/* ------------------------------------------------------------------ codec */
/* code of element i of a row in the canonical layout */
static inline int code_at(const uint8_t *row, int i, int bits) {
    if (bits == 8) return row[i];
    return (row[i >> 1] >> ((i & 1) * 4)) & 0xF;
}

/* Dequantize one row of K elements to float64: w_i = s[i/64] * q_i + b[i/64]. */
void orc_dequant_row(int bits, int K, const uint8_t *codes, const uint16_t *scales,
                     const uint16_t *biases, double *out) {
    for (int i = 0; i < K; ++i)
        out[i] = bf16_f64(scales[i / 64]) * (double)code_at(codes, i, bits) + bf16_f64(biases[i / 64]);
}

/* IEEE binary16 bits to float64, exactly (subnormals, infinities and NaN included). */
double orc_f16_to_f64(uint16_t h) {
    const int sign = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)m, -24);                      /* zero and subnormals: m 2^-24 */
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp(1024.0 + (double)m, e - 25);                 /* (1 + m/1024) 2^(e-15) */
    return sign ? -v : v;
}

/* Dequantize one row of K elements stored as K/32 Q4_0 blocks (18 bytes each: fp16 scale d,
 * little-endian, then 16 code bytes): element 32b + j is d_b * (q - 8) with q the low nibble of
 * code byte j (j < 16) or the high nibble of code byte j - 16 (j >= 16). */
void orc_dequant_q4_0_row(int K, const uint8_t *blocks, double *out) {
    for (int b = 0; b < K / 32; ++b) {
        const uint8_t *blk = blocks + (size_t)b * 18;
        const double d = orc_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
        for (int j = 0; j < 32; ++j) {
            const int q = j < 16 ? (blk[2 + j] & 0xF) : (blk[2 + j - 16] >> 4);
            out[32 * b + j] = d * (double)(q - 8);
        }
    }
}

/* ------------------------------------------------------------------ router */
/*
 * Router logits in the canonical fp32 order, for tokens t < T and experts e < E.
 * With x_j the token's bf16 activations (exact in fp32), q_j the 8-bit codes and s_g, b_g
 * the group's scale and bias:
 *
 *   w_j  = fma(s_g, q_j, b_g)                                         the dequantized weight, fp32
 *   A_g  = fma(x_{64g+63}, w_{64g+63}, ... fma(x_{64g}, w_{64g}, 0))   fp32 fma chain, ascending j
 *   L    = ((0 + A_0) + A_1) + ... + A_{G-1}                           fp32 adds, ascending g
 *   logit = L + bias_e   (only when a logit bias is given)
 *
 * This is the router projection W_r x of the affine-dequantized matrix with one fixed
 * rounding order, so that both sides reach the same fp32 logits and hence the same top-k.
 */
void orc_router_logits(int T, int d, int E, const uint16_t *x, const uint8_t *rq,
                       const uint16_t *rs, const uint16_t *rb, const float *logit_bias,
                       float *logits) {
    const int G = d / 64;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        float *xf = (float *)malloc(sizeof(float) * (size_t)d);
        for (int i = 0; i < d; ++i) xf[i] = bf16_f32(x[(size_t)t * d + i]);
        for (int e = 0; e < E; ++e) {
            const uint8_t *q = rq + (size_t)e * d;
            float L = 0.0f;
            for (int g = 0; g < G; ++g) {
                const float sg = bf16_f32(rs[(size_t)e * G + g]), bg = bf16_f32(rb[(size_t)e * G + g]);
                float A = 0.0f;
                for (int j = 0; j < 64; ++j) A = fmaf(xf[64 * g + j], fmaf(sg, (float)q[64 * g + j], bg), A);
                L = L + A;
            }
            logits[(size_t)t * E + e] = logit_bias ? L + logit_bias[e] : L;
        }
        free(xf);
    }
}

/*
 * Top-k of each row of logits: the k largest values, listed largest first; among equal
 * values the lower expert index comes first (and is the one kept at the k boundary).
 * Routing weights: softmax over the k selected logits, in float64, each multiplied by the
 * selected expert's per_expert_scale when one is given (Mference "Decode", router listing).
 */
void orc_topk(int T, int E, int k, const float *logits, const uint16_t *per_expert_scale, int32_t *idx,
              double *w) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float *l = logits + (size_t)t * E;
        unsigned char *taken = (unsigned char *)calloc((size_t)E, 1);
        int32_t *sel = idx + (size_t)t * k;
        for (int s = 0; s < k; ++s) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;   /* strict: earlier index wins ties */
            }
            taken[best] = 1;
            sel[s] = best;
        }
        double m = (double)l[sel[0]];
        double z = 0.0;
        for (int s = 0; s < k; ++s) z += exp((double)l[sel[s]] - m);
        for (int s = 0; s < k; ++s) {
            double v = exp((double)l[sel[s]] - m) / z;
            if (per_expert_scale) v *= bf16_f64(per_expert_scale[sel[s]]);   /* router epilogue */
            w[(size_t)t * k + s] = v;
        }
        free(taken);
    }
}

/*
 * Grouping of token/expert pairs by expert. Pair p = t*k + s is token t's slot s.
 *   counts[e]   = number of pairs routed to expert e
 *   offsets[e]  = sum of counts[0..e-1]  (E+1 entries)
 *   perm        = pair ids ordered by (expert, token)
 *   pos[p]      = position of pair p in perm
 */
void orc_bucket(int T, int E, int k, const int32_t *idx, int32_t *counts, int32_t *offsets,
                int32_t *perm, int32_t *pos) {
    const int P = T * k;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int p = 0; p < P; ++p) counts[idx[p]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int cursor = 0;
    for (int e = 0; e < E; ++e)
        for (int t = 0; t < T; ++t)
            for (int s = 0; s < k; ++s)
                if (idx[t * k + s] == e) perm[cursor++] = t * k + s;
    for (int i = 0; i < P; ++i) pos[perm[i]] = i;
}

/* ------------------------------------------------------------------ expert FFN */
double orc_gelu_tanh(double v) {
    const double c = 0.79788456080286535588; /* sqrt(2/pi) */
    return 0.5 * v * (1.0 + tanh(c * (v + 0.044715 * v * v * v)));
}

typedef struct {
    const uint8_t *codes;    /* affine: [out, in*bits/8]; Q4_0: blocks [out, in/32, 18 bytes] */
    const uint16_t *scales;  /* affine: [out, in/64]; Q4_0: unused */
    const uint16_t *biases;  /* affine: [out, in/64]; Q4_0: unused */
    int q4_0;                /* 1: Q4_0 blocks */
} orc_qmat;

static size_t qmat_row_bytes(const orc_qmat *W, int bits, int in_dim) {
    return W->q4_0 ? (size_t)in_dim / 32 * 18 : (size_t)in_dim * bits / 8;
}

/* y[out] = W x, W dequantized to float64 one row at a time. */
static void qmatvec(int bits, int out_dim, int in_dim, const orc_qmat *W, const double *x,
                    double *y, double *rowbuf) {
    const size_t row_bytes = qmat_row_bytes(W, bits, in_dim);
    const int G = in_dim / 64;
    for (int o = 0; o < out_dim; ++o) {
        if (W->q4_0)
            orc_dequant_q4_0_row(in_dim, W->codes + (size_t)o * row_bytes, rowbuf);
        else
            orc_dequant_row(bits, in_dim, W->codes + (size_t)o * row_bytes, W->scales + (size_t)o * G,
                            W->biases + (size_t)o * G, rowbuf);
        double acc = 0.0;
        for (int i = 0; i < in_dim; ++i) acc += rowbuf[i] * x[i];
        y[o] = acc;
    }
}

/*
 * One GELU-gated expert on one token:
 *   g = W_gate x,  u = W_up x,  h = gelu_tanh(g) * u,  r = W_down h.
 * x: float64 [d]; r: float64 [d]; I = expert width.
 */
void orc_ffn(int d, int I, const double *x, const orc_qmat *gate, const orc_qmat *up,
             const orc_qmat *down, double *r) {
    int n = d > I ? d : I;
    double *buf = (double *)malloc(sizeof(double) * (size_t)n);
    double *g = (double *)malloc(sizeof(double) * (size_t)I);
    double *u = (double *)malloc(sizeof(double) * (size_t)I);
    qmatvec(4, I, d, gate, x, g, buf);
    qmatvec(4, I, d, up, x, u, buf);
    for (int j = 0; j < I; ++j) g[j] = orc_gelu_tanh(g[j]) * u[j];
    qmatvec(4, d, I, down, g, r, buf);
    free(buf);
    free(g);
    free(u);
}

/* Expert e of a stack [E, out, ...] */
static orc_qmat expert_view(const orc_qmat *stack, int e, int out_dim, int in_dim) {
    orc_qmat m = *stack;
    size_t row_bytes = qmat_row_bytes(stack, 4, in_dim), G = (size_t)in_dim / 64;
    m.codes = stack->codes + (size_t)e * out_dim * row_bytes;
    if (!stack->q4_0) {
        m.scales = stack->scales + (size_t)e * out_dim * G;
        m.biases = stack->biases + (size_t)e * out_dim * G;
    }
    return m;
}

/*
 * Layer outputs for the listed tokens, given their routing:
 *   y_t = a_t * shared(x_t) + sum_{s=0..k-1} w[t,s] * expert_{idx[t,s]}(x_t)
 * accumulated in float64 in that order, with a_t = 1 / (1 + exp(-(g . x_t))) when the
 * shared-expert gate g (bf16 [d]) is given and a_t = 1 otherwise. Also returns the
 * (ungated) shared output, the per-slot outputs and a_t when the pointers are non-null
 * (sh: [n_tok, d], r: [n_tok, k, d], a: [n_tok]).
 */
void orc_layer_tokens(int d, int E, int k, int I, int Is, const uint16_t *x, int n_tok,
                      const int32_t *tokens, const int32_t *idx, const double *w,
                      const orc_qmat *gate, const orc_qmat *up, const orc_qmat *down,
                      const orc_qmat *sh_gate, const orc_qmat *sh_up, const orc_qmat *sh_down,
                      const uint16_t *shared_gate, double *y, double *sh_out, double *r_out, double *a_out) {
    (void)E;
#pragma omp parallel for schedule(dynamic, 1)
    for (int n = 0; n < n_tok; ++n) {
        const int t = tokens[n];
        double *xd = (double *)malloc(sizeof(double) * (size_t)d);
        double *sh = (double *)malloc(sizeof(double) * (size_t)d);
        double *r = (double *)malloc(sizeof(double) * (size_t)d);
        for (int i = 0; i < d; ++i) xd[i] = bf16_f64(x[(size_t)t * d + i]);
        orc_ffn(d, Is, xd, sh_gate, sh_up, sh_down, sh);
        double a = 1.0;
        if (shared_gate) {
            double z = 0.0;
            for (int i = 0; i < d; ++i) z += xd[i] * bf16_f64(shared_gate[i]);
            a = 1.0 / (1.0 + exp(-z));
        }
        if (a_out) a_out[n] = a;
        double *yt = y + (size_t)n * d;
        for (int i = 0; i < d; ++i) yt[i] = a * sh[i];
        if (sh_out)
            for (int i = 0; i < d; ++i) sh_out[(size_t)n * d + i] = sh[i];
        for (int s = 0; s < k; ++s) {
            const int e = idx[(size_t)t * k + s];
            orc_qmat G_ = expert_view(gate, e, I, d), U_ = expert_view(up, e, I, d),
                     D_ = expert_view(down, e, d, I);
            orc_ffn(d, I, xd, &G_, &U_, &D_, r);
            const double ws = w[(size_t)t * k + s];
            for (int i = 0; i < d; ++i) yt[i] += ws * r[i];
            if (r_out)
                for (int i = 0; i < d; ++i) r_out[((size_t)n * k + s) * d + i] = r[i];
        }
        free(xd);
        free(sh);
        free(r);
    }
}

/* ------------------------------------------------------------------ router prologue */
/*
 * Router input from the layer input (Mference "Decode", router listing): the input is
 * normalized without a learned scale, multiplied by the router scale and by 1/sqrt(d):
 *   v = x / sqrt(mean(x^2) + eps)          (sum of squares ascending, float64)
 *   u = bf16(((v * router_scale) / sqrt(d)))   (float64, rounded once)
 * x, u: bf16 bits [T, d]; router_scale: bf16 bits [d].
 */
void orc_router_prologue(int T, int d, const uint16_t *x, const uint16_t *router_scale, double eps,
                         uint16_t *u) {
    for (int t = 0; t < T; ++t) {
        const uint16_t *xt = x + (size_t)t * d;
        double ss = 0.0;
        for (int i = 0; i < d; ++i) {
            const double v = bf16_f64(xt[i]);
            ss += v * v;
        }
        const double inv = 1.0 / sqrt(ss / d + eps);
        const double sd = sqrt((double)d);
        for (int i = 0; i < d; ++i)
            u[(size_t)t * d + i] = orc_f64_to_bf16(((bf16_f64(xt[i]) * inv) * bf16_f64(router_scale[i])) / sd);
    }
}

/* ------------------------------------------------------------------ layer stack glue */
/*
 * Residual stream between layers of the decode stack, with the layer tail (Mference system
 * design, "Decode", cb2: post-FFN norm, residual, layer scalar):
 *   z      = y / sqrt(mean(y^2) + eps) * post          (only when post is given; else z = y)
 *   h_next = bf16((h + z) * scalar)
 *   x_next = bf16(h_next / sqrt(mean(h_next^2) + eps))  (norm without a learned scale)
 * float64 throughout, sums of squares ascending. h, h_next, x_next: bf16 bits [T, d];
 * y: float64 [T, d] (NULL: no layer output yet, h_next = h); post: bf16 bits [d] or NULL.
 */
void orc_stack_glue(int T, int d, const uint16_t *h, const double *y, const uint16_t *post, double scalar,
                    double eps, uint16_t *h_next, uint16_t *x_next) {
    for (int t = 0; t < T; ++t) {
        const double *yt = y ? y + (size_t)t * d : NULL;
        double inv_y = 1.0;
        if (yt && post) {
            double sy = 0.0;
            for (int i = 0; i < d; ++i) sy += yt[i] * yt[i];
            inv_y = 1.0 / sqrt(sy / d + eps);
        }
        double ss = 0.0;
        for (int i = 0; i < d; ++i) {
            size_t o = (size_t)t * d + i;
            double v = bf16_f64(h[o]);
            if (yt) {
                const double z = post ? (yt[i] * inv_y) * bf16_f64(post[i]) : yt[i];
                v = (v + z) * scalar;
            }
            h_next[o] = orc_f64_to_bf16(v);
            const double r = bf16_f64(h_next[o]);
            ss += r * r;
        }
        double inv = 1.0 / sqrt(ss / d + eps);
        for (int i = 0; i < d; ++i) {
            size_t o = (size_t)t * d + i;
            x_next[o] = orc_f64_to_bf16(bf16_f64(h_next[o]) * inv);
        }
    }
}
