/*
 * moe_oracle.c -- plain, slow CPU definition of the fused mixture-of-experts
 * FFN forward.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the HIP library; it is the yardstick the HIP
 * path is measured against, never a fallback for it.
 *
 * What it computes (sources are the five pages on fused MoE):
 *   - routed-item form, FlagGems "fused_moe.py" walkthrough, sec. 1.2
 *     (h_r = W1^T x + b1, z_r = phi(h_r), o_r = W2^T z_r + b2,
 *      y_t = sum_{r: t(r)=t} a(r) o_r), with the gated SiLU phi that the
 *     fused gate/up weight of the MindIE-SD "Fused MoE" page (parameter
 *     table, w13_weight [E, H, 2I]) implies: phi(h) = SiLU(h[:I]) * h[I:];
 *   - routing: MindIE-SD "Fused MoE" page, "routing selection" section and
 *     parameter table (softmax | sigmoid, grouped selection by group max or
 *     top-2 sum, renormalize, routed_scaling_factor); its custom routing
 *     example (softmax -> top-k -> optional divide by the sum);
 *   - align: FlagGems walkthrough, "moe_align_block_size" section (sort
 *     routed items by expert, pad each expert to BLOCK_SIZE_M), stable in
 *     the sense of the MoonEP page's build_permutation (a stable argsort);
 *   - WNA16: FlagGems walkthrough, "WNA16" section (int8_w8a16 and
 *     int4_w4a16 weights with group scales and zero points; activations stay
 *     16-bit): w = (q - z) * s, one (s, z) per group of K rows and column;
 *   - fp8: FlagGems walkthrough, "FP8 W8A8" section (per-channel or
 *     block-wise weight scales, per-token or block-wise activation scales;
 *     a block-wise product is the sum over K blocks of dot(qA, qB) times the
 *     two blocks' scales, which is the product of the dequantised operands).
 *
 * Precision: every value-path sum and product is taken in double from the
 * exactly-upcast inputs (bf16 and fp8 codes convert to double exactly).
 * Where a float decides an integer (an fp8 code, the grouped-routing key),
 * the decision is made in float32, the precision the device kernels use.
 * Expert selection compares logits, which is exact because softmax and the
 * sigmoid are strictly increasing.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8 = 2, OR_U8 = 3, OR_U4 = 4 };
enum { OR_SOFTMAX = 0, OR_SIGMOID = 1 };

/* ------------------------------------------------------------------ */
/* scalar formats                                                      */
/* ------------------------------------------------------------------ */

static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16; /* bf16 is the top half of a float32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP 8-bit float E4M3FN: sign, 4 exponent bits (bias 7), 3 mantissa bits,
 * no infinities, S.1111.111 is NaN, largest finite magnitude 448. */
double oracle_fp8_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);          /* (m/8) * 2^-6          */
    else
        v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7)   */
    return s ? -v : v;
}

/* Round-to-nearest-even onto E4M3FN, saturating at +-448.  Done the plain
 * way: scan the 127 non-negative finite codes for the nearest value; on an
 * exact tie take the code with an even mantissa (its lowest bit clear). */
uint8_t oracle_fp8_encode(float x)
{
    uint8_t sign, best = 0;
    double a, bestd = INFINITY;
    if (isnan(x))
        return 0x7F;
    sign = signbit(x) ? 0x80 : 0x00;
    a = fabs((double)x);
    if (a >= 448.0)
        return sign | 0x7E;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(oracle_fp8_decode((uint8_t)c) - a);
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            bestd = d;
            best = (uint8_t)c;
        }
    }
    return sign | best;
}

static double fp8_table[256];
static int fp8_table_ready = 0;

static void fp8_table_init(void)
{
    if (fp8_table_ready)
        return;
    for (int c = 0; c < 256; ++c)
        fp8_table[c] = oracle_fp8_decode((uint8_t)c);
    fp8_table_ready = 1;
}

/* Dynamic per-row fp8 quantisation (FlagGems walkthrough, "FP8 W8A8":
 * activations are quantised before each expert GEMM).  Decision precision
 * float32: scale = amax / 448 (1 when the row is all zero), code =
 * RNE(x / scale). */
void oracle_quant_row_fp8(const float* x, int64_t n, uint8_t* q, float* scale_out)
{
    float amax = 0.0f, scale;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    scale = (amax > 0.0f) ? amax / 448.0f : 1.0f;
    for (int64_t i = 0; i < n; ++i)
        q[i] = oracle_fp8_encode(x[i] / scale);
    *scale_out = scale;
}

/* Block-wise dynamic quantisation of one row (FlagGems walkthrough, "FP8
 * W8A8", block-wise granularity): every group of `block` columns (the last
 * one may be shorter) is quantised on its own, as oracle_quant_row_fp8 does
 * for a whole row; scale_out[g] is group g's scale. */
void oracle_quant_row_fp8_groups(const float* x, int64_t n, int64_t block, uint8_t* q,
                                 float* scale_out)
{
    for (int64_t g0 = 0, g = 0; g0 < n; g0 += block, ++g) {
        const int64_t len = (n - g0 < block) ? n - g0 : block;
        oracle_quant_row_fp8(x + g0, len, q + g0, scale_out + g);
    }
}

/* ------------------------------------------------------------------ */
/* routing                                                             */
/* ------------------------------------------------------------------ */

typedef struct {
    int32_t E, top_k;
    int32_t scoring;           /* OR_SOFTMAX or OR_SIGMOID               */
    int32_t renormalize;       /* softmax only; sigmoid always normalises */
    int32_t group_count;       /* 1 = no grouped selection               */
    int32_t k_group;
    int32_t group_select_mode; /* 0 group max, 1 sum of the group top-2  */
    int32_t logits_dtype;      /* OR_F32 or OR_BF16                      */
    double routed_scaling_factor;
} oracle_routing;

static double logit_at(const oracle_routing* R, const void* logits, int64_t t, int e)
{
    int64_t idx = t * (int64_t)R->E + e;
    if (R->logits_dtype == OR_BF16)
        return bf16_bits_to_double(((const uint16_t*)logits)[idx]);
    return (double)((const float*)logits)[idx];
}

/* Grouped-routing key of mode 1 for one expert logit v: the expert's score
 * up to a positive factor shared by the whole token (softmax: exp(v - max),
 * sigmoid: 1/(1+exp(-v))), evaluated in double and rounded to float32. */
static float group_score_f32(int scoring, double v, double vmax)
{
    if (scoring == OR_SIGMOID)
        return (float)(1.0 / (1.0 + exp(-v)));
    return (float)exp(v - vmax);
}

/* Routes one token.  ids[k] in selection order, w[k] in double. */
static void route_token(const oracle_routing* R, const double* s, int32_t* ids, double* w,
                        unsigned char* cand, unsigned char* taken, double* p)
{
    const int E = R->E, K = R->top_k;
    double vmax = s[0], sum;

    for (int e = 1; e < E; ++e)
        if (s[e] > vmax)
            vmax = s[e];

    /* scores p_t (FlagGems sec. 1.1 softmax; MindIE routing: sigmoid) */
    if (R->scoring == OR_SOFTMAX) {
        sum = 0.0;
        for (int e = 0; e < E; ++e) {
            p[e] = exp(s[e] - vmax);
            sum += p[e];
        }
        for (int e = 0; e < E; ++e)
            p[e] /= sum;
    } else {
        for (int e = 0; e < E; ++e)
            p[e] = 1.0 / (1.0 + exp(-s[e]));
    }

    /* candidate experts: all, or those of the k_group best groups */
    if (R->group_count > 1) {
        const int G = R->group_count, per = E / G;
        double key[1024];
        unsigned char gtaken[1024];
        for (int g = 0; g < G; ++g) {
            const double* sg = s + g * per;
            gtaken[g] = 0;
            if (R->group_select_mode == 0) {
                double m = sg[0];
                for (int i = 1; i < per; ++i)
                    if (sg[i] > m)
                        m = sg[i];
                key[g] = m; /* the group max score, compared through its logit */
            } else {
                /* the two largest logits of the group */
                int a = 0;
                for (int i = 1; i < per; ++i)
                    if (sg[i] > sg[a])
                        a = i;
                int b = (a == 0) ? 1 : 0;
                for (int i = 0; i < per; ++i)
                    if (i != a && sg[i] > sg[b])
                        b = i;
                float ka = group_score_f32(R->scoring, sg[a], vmax);
                float kb = group_score_f32(R->scoring, sg[b], vmax);
                float k2 = ka + kb; /* float32 addition */
                key[g] = (double)k2;
            }
        }
        for (int e = 0; e < E; ++e)
            cand[e] = 0;
        for (int round = 0; round < R->k_group; ++round) {
            int best = -1;
            for (int g = 0; g < G; ++g)
                if (!gtaken[g] && (best < 0 || key[g] > key[best]))
                    best = g; /* strict '>' keeps the lower index on ties */
            gtaken[best] = 1;
            for (int i = 0; i < per; ++i)
                cand[best * per + i] = 1;
        }
    } else {
        for (int e = 0; e < E; ++e)
            cand[e] = 1;
    }

    /* top-k over the candidates by (logit desc, index asc) */
    for (int e = 0; e < E; ++e)
        taken[e] = 0;
    for (int j = 0; j < K; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e)
            if (cand[e] && !taken[e] && (best < 0 || s[e] > s[best]))
                best = e;
        taken[best] = 1;
        ids[j] = best;
        w[j] = p[best];
    }

    /* renormalise (softmax when asked; sigmoid always), then scale */
    if ((R->scoring == OR_SOFTMAX && R->renormalize) || R->scoring == OR_SIGMOID) {
        double tot = 0.0;
        for (int j = 0; j < K; ++j)
            tot += w[j];
        for (int j = 0; j < K; ++j)
            w[j] /= tot;
    }
    for (int j = 0; j < K; ++j)
        w[j] *= R->routed_scaling_factor;
}

/* Routes tokens [0, M).  topk_ids [M, top_k], topk_w [M, top_k] (double). */
int oracle_route(const oracle_routing* R, const void* logits, int64_t M, int32_t* topk_ids,
                 double* topk_w)
{
    const int E = R->E, K = R->top_k;
    if (E < 1 || E > 1024 || K < 1 || K > E)
        return -1;
    if (R->group_count > 1) {
        if (E % R->group_count || R->k_group < 1 || R->k_group > R->group_count)
            return -1;
        if (K > R->k_group * (E / R->group_count))
            return -1;
        if (R->group_select_mode == 1 && E / R->group_count < 2)
            return -1;
    }
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * E);
        double* p = (double*)malloc(sizeof(double) * E);
        unsigned char* cand = (unsigned char*)malloc(E);
        unsigned char* taken = (unsigned char*)malloc(E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < M; ++t) {
            for (int e = 0; e < E; ++e)
                s[e] = logit_at(R, logits, t, e);
            route_token(R, s, topk_ids + t * K, topk_w + t * K, cand, taken, p);
        }
        free(s);
        free(p);
        free(cand);
        free(taken);
    }
    return 0;
}

/* Group keys as float32 for tests that inspect near-ties: keys[M, G].
 * Mode 0 keys are the group's largest logit. */
int oracle_group_keys(const oracle_routing* R, const void* logits, int64_t M, float* keys)
{
    const int E = R->E, G = R->group_count, per = E / G;
    for (int64_t t = 0; t < M; ++t) {
        double vmax = logit_at(R, logits, t, 0);
        for (int e = 1; e < E; ++e) {
            double v = logit_at(R, logits, t, e);
            if (v > vmax)
                vmax = v;
        }
        for (int g = 0; g < G; ++g) {
            double a = -INFINITY, b = -INFINITY;
            for (int i = 0; i < per; ++i) {
                double v = logit_at(R, logits, t, g * per + i);
                if (v > a) {
                    b = a;
                    a = v;
                } else if (v > b) {
                    b = v;
                }
            }
            if (R->group_select_mode == 0)
                keys[t * G + g] = (float)a;
            else
                keys[t * G + g] = group_score_f32(R->scoring, a, vmax) +
                                  group_score_f32(R->scoring, b, vmax);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* align (permute metadata)                                            */
/* ------------------------------------------------------------------ */

/* Stable sort of the Mk routed items r = t*top_k + j by expert, each
 * expert's run padded up to a multiple of BM with the sentinel Mk.
 *   counts[E], sorted_ids[>= num_post_padded], expert_ids[num_post_padded/BM],
 *   *num_post_padded.  An id of -1 marks an item whose expert is held by
 *   another expert-parallel rank (the walkthrough's expert_id == -1): it gets
 *   no row.  Returns 0, or -1 when an id is out of [-1, E) or the output
 *   capacity is too small. */
int oracle_align(const int32_t* ids, int64_t Mk, int32_t E, int32_t BM, int32_t* counts,
                 int32_t* sorted_ids, int64_t sorted_cap, int32_t* expert_ids, int64_t blocks_cap,
                 int32_t* num_post_padded)
{
    int64_t pos = 0;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t r = 0; r < Mk; ++r) {
        if (ids[r] == -1)
            continue;
        if (ids[r] < 0 || ids[r] >= E)
            return -1;
        counts[ids[r]]++;
    }
    for (int e = 0; e < E; ++e) {
        int64_t start = pos, padded = ((int64_t)counts[e] + BM - 1) / BM * BM;
        if (start + padded > sorted_cap || (start + padded) / BM > blocks_cap)
            return -1;
        for (int64_t r = 0; r < Mk; ++r)
            if (ids[r] == e)
                sorted_ids[pos++] = (int32_t)r;
        while (pos < start + padded)
            sorted_ids[pos++] = (int32_t)Mk;
        for (int64_t b = start / BM; b < (start + padded) / BM; ++b)
            expert_ids[b] = e;
    }
    *num_post_padded = (int32_t)pos;
    return 0;
}

/* ------------------------------------------------------------------ */
/* expert FFN                                                          */
/* ------------------------------------------------------------------ */

typedef struct {
    int32_t H, I, E;
    int32_t w_dtype;          /* OR_F32, OR_BF16, OR_FP8                      */
    const void* w13;          /* [E][H][2I]; gate = columns [0,I), up = [I,2I) */
    const void* w2;           /* [E][I][H]                                     */
    const float* w13_scale;   /* OR_FP8: per output channel [E][2I], or with  */
                              /*   block B: [E][ceil(2I/B)][ceil(H/B)]         */
    const float* w2_scale;    /* OR_FP8: per output channel [E][H], or with   */
                              /*   block B: [E][ceil(H/B)][ceil(I/B)]          */
    int32_t bias_dtype;       /* OR_F32 or OR_BF16                             */
    const void* w13_bias;     /* [E][2I] or NULL                               */
    const void* w2_bias;      /* [E][H] or NULL                                */
    int32_t requant_z;        /* 1: z is requantised to fp8 per (row, 128 cols) */
    int32_t block;            /* OR_FP8: 0 per-channel scales; B > 0: one scale */
                              /*   per B x B block (output columns x K rows)   */
    int32_t group;            /* OR_U8 / OR_U4: K rows per scale group          */
    const uint8_t* w13_zero;  /* OR_U8 / OR_U4: [E][ceil(H/group)][2I] or NULL  */
    const uint8_t* w2_zero;   /*   [E][ceil(I/group)][H] or NULL (2^(bits-1))   */
    int32_t wq_bf16;          /* OR_U8 / OR_U4: 0 the exact weight (q - z) s;   */
                              /*   1 that weight formed in float32, then rounded */
                              /*   to bf16 (the compute type)                    */
    int32_t z_bf16;           /* 1: z is held in bf16 (the compute type) before */
                              /*   the second GEMM (without requant_z)          */
} oracle_experts;

/* WNA16 weight codes: OR_U8 one unsigned byte per weight, [E][K][N];
 * OR_U4 two per byte along N, [E][K][N/2], the even column in the low
 * nibble.  The scales are [E][ceil(K/group)][N] floats (w13_scale / w2_scale). */
static int wq_code(const oracle_experts* W, const void* w, int64_t row, int64_t N, int64_t n)
{
    if (W->w_dtype == OR_U8)
        return ((const uint8_t*)w)[row * N + n];
    const uint8_t b = ((const uint8_t*)w)[row * (N / 2) + n / 2];
    return (n & 1) ? (b >> 4) : (b & 15);
}

/* Dequantised WNA16 weight (k, n) of expert e: (q - z) * s of its K group. */
/* x rounded to the nearest bf16, ties to even (finite x). */
static double round_bf16(float x)
{
    uint32_t b;
    memcpy(&b, &x, 4);
    b = (b + 0x7fffu + ((b >> 16) & 1u)) & 0xffff0000u;
    memcpy(&x, &b, 4);
    return (double)x;
}

/* Dequantised WNA16 weight (FlagGems walkthrough, "WNA16" section: group
 * scales and zero points; its "fused_experts_impl" section, special
 * quantisation formats: the public entry dequantises the codes to
 * hidden_states.dtype before the generic kernel runs).  wq_bf16 selects that
 * reading, (q - z) s in float32 rounded to bf16; without it the weight is
 * exact. */
static double wq_weight(const oracle_experts* W, const void* w, const float* scale,
                        const uint8_t* zero, int e, int64_t K, int64_t N, int64_t k, int64_t n)
{
    const int64_t G = W->group, ng = (K + G - 1) / G;
    const int64_t gi = ((int64_t)e * ng + k / G) * N + n;
    const int z = zero ? zero[gi] : (W->w_dtype == OR_U8 ? 128 : 8);
    const int q = wq_code(W, w, (int64_t)e * K + k, N, n);
    if (W->wq_bf16)
        return round_bf16((float)(q - z) * scale[gi]);
    return (double)(q - z) * (double)scale[gi];
}

/* GPTQ and AWQ checkpoints ship WNA16 codes packed into int32 words
 * (FlagGems walkthrough, "WNA16" section, which names both layouts without
 * giving their bit order).  The reading taken here, per K x N weight of one
 * expert (per = 32 / bits codes a word, the code at word bits
 * [bits * i, bits * (i + 1))):
 *   GPTQ   qweight [K / per][N]: word (r, n), slot i = row per * r + i of
 *          column n (rows packed along K);
 *          qzeros [ng][N / per]: word (g, c), slot i = the zero point of
 *          column per * c + i in group g (packed along N in order);
 *   AWQ    (4-bit) qweight [K][N / 8]: word (k, c), slot i = column
 *          8 c + AWQ_ORDER[i] of row k, AWQ_ORDER = {0, 2, 4, 6, 1, 3, 5, 7};
 *          qzeros [ng][N / 8] the same way.
 * zero_adjust is added to every stored zero point (checkpoints of the
 * earlier GPTQ format store z - 1).
 * Output: the oracle's plain codes (OR_U8: one byte a code, [K][N]; OR_U4:
 * two a byte along N, even column in the low nibble, [K][N / 2]) and the
 * zero points as one byte per group and column [ng][N] (when qzeros is
 * given).  Returns 0, or -1 for an unsupported combination. */
enum { OR_GPTQ = 1, OR_AWQ = 2 };

static int packed_slot(const int32_t* words, int64_t idx, int bits, int slot)
{
    const uint32_t w = (uint32_t)words[idx];
    return (int)((w >> (bits * slot)) & ((1u << bits) - 1u));
}

int oracle_unpack_wq(int32_t format, int32_t bits, int64_t E, int64_t K, int64_t N, int64_t group,
                     const int32_t* qweight, const int32_t* qzeros, int32_t zero_adjust,
                     uint8_t* codes, uint8_t* zeros)
{
    static const int awq_order[8] = {0, 2, 4, 6, 1, 3, 5, 7};
    const int per = 32 / bits;
    const int64_t ng = (K + group - 1) / group;
    if ((bits != 4 && bits != 8) || (format != OR_GPTQ && format != OR_AWQ) || group < 1)
        return -1;
    if (format == OR_AWQ && bits != 4)
        return -1;
    if ((format == OR_GPTQ && K % per) || (format == OR_AWQ && N % 8) ||
        (qzeros && N % per) || (bits == 4 && N % 2))
        return -1;
    for (int64_t e = 0; e < E; ++e) {
        for (int64_t k = 0; k < K; ++k) {
            for (int64_t n = 0; n < N; ++n) {
                int q;
                if (format == OR_GPTQ) {
                    const int64_t idx = (e * (K / per) + k / per) * N + n;
                    q = packed_slot(qweight, idx, bits, (int)(k % per));
                } else {
                    /* column n sits in word n / 8 at the slot whose order entry is n % 8 */
                    int slot = 0;
                    while (awq_order[slot] != (int)(n % 8))
                        ++slot;
                    q = packed_slot(qweight, (e * K + k) * (N / 8) + n / 8, bits, slot);
                }
                if (bits == 8) {
                    codes[(e * K + k) * N + n] = (uint8_t)q;
                } else {
                    uint8_t* b = codes + (e * K + k) * (N / 2) + n / 2;
                    if (n % 2 == 0)
                        *b = (uint8_t)((*b & 0xF0) | q);
                    else
                        *b = (uint8_t)((*b & 0x0F) | (q << 4));
                }
            }
        }
        if (!qzeros || !zeros)
            continue;
        for (int64_t g = 0; g < ng; ++g) {
            for (int64_t n = 0; n < N; ++n) {
                int z;
                if (format == OR_GPTQ) {
                    z = packed_slot(qzeros, (e * ng + g) * (N / per) + n / per, bits,
                                    (int)(n % per));
                } else {
                    int slot = 0;
                    while (awq_order[slot] != (int)(n % 8))
                        ++slot;
                    z = packed_slot(qzeros, (e * ng + g) * (N / 8) + n / 8, bits, slot);
                }
                zeros[(e * ng + g) * N + n] = (uint8_t)((z + zero_adjust) & ((1 << bits) - 1));
            }
        }
    }
    return 0;
}

typedef struct {
    int32_t dtype;            /* OR_F32, OR_BF16, OR_FP8 (codes + per-row scale) */
    const void* data;         /* [rows][H]                                       */
    const float* scale;       /* OR_FP8: [rows], or with block B: [rows][ceil(H/B)] */
    int32_t quantize;         /* 1: quantise the f32/bf16 row to fp8 first      */
    int32_t block;            /* 0: one scale per row; B > 0: per B columns     */
} oracle_acts;

static double bias_at(const oracle_experts* W, const void* b, int64_t idx)
{
    if (W->bias_dtype == OR_BF16)
        return bf16_bits_to_double(((const uint16_t*)b)[idx]);
    return (double)((const float*)b)[idx];
}

/* x = one activation row as double (dequantised where it is fp8). */
static void load_row(const oracle_acts* A, int64_t H, int64_t row, double* x, float* xf,
                     uint8_t* q)
{
    if (A->dtype == OR_FP8) {
        const uint8_t* c = (const uint8_t*)A->data + row * H;
        if (A->block > 0) {
            const int64_t B = A->block, ng = (H + B - 1) / B;
            for (int64_t k = 0; k < H; ++k)
                x[k] = fp8_table[c[k]] * (double)A->scale[row * ng + k / B];
            return;
        }
        double sc = (double)A->scale[row];
        for (int64_t k = 0; k < H; ++k)
            x[k] = fp8_table[c[k]] * sc;
        return;
    }
    for (int64_t k = 0; k < H; ++k)
        x[k] = (A->dtype == OR_BF16) ? bf16_bits_to_double(((const uint16_t*)A->data)[row * H + k])
                                     : (double)((const float*)A->data)[row * H + k];
    if (A->quantize) {
        const int64_t B = (A->block > 0) ? A->block : H;
        float* sc = (float*)malloc(sizeof(float) * (size_t)((H + B - 1) / B));
        for (int64_t k = 0; k < H; ++k)
            xf[k] = (float)x[k];
        oracle_quant_row_fp8_groups(xf, H, B, q, sc);
        for (int64_t k = 0; k < H; ++k)
            x[k] = fp8_table[q[k]] * (double)sc[k / B];
        free(sc);
    }
}

/* Codes decided near a rounding tie, for the re-quantisation of the
 * intermediate z on the fp8 path (FlagGems walkthrough, "FP8 W8A8").
 * Whoever computes t = z / scale in a different order, or with a different
 * exp / reciprocal, gets a t that differs in its last bits, and where t lies
 * that close to the midpoint between two fp8 values both roundings are
 * correct answers.  Returns the code that t * (1 + window) or
 * t * (1 - window) rounds to when it differs from t's own code (the
 * neighbour across the nearby midpoint), else -1. */
int oracle_fp8_tie_alt(float t, float window)
{
    const uint8_t c = oracle_fp8_encode(t);
    const uint8_t up = oracle_fp8_encode(t * (1.0f + window));
    const uint8_t dn = oracle_fp8_encode(t * (1.0f - window));
    if (up != c)
        return up;
    if (dn != c)
        return dn;
    return -1;
}

/* Near-tie z codes of one expert row: where each sits in z and how much the
 * dequantised z value changes (alternative minus chosen) if the other code is
 * taken.  n counts every near-tie code, also past ORACLE_MAX_TIES. */
#define ORACLE_MAX_TIES 8
typedef struct {
    int32_t n;
    int64_t k[ORACLE_MAX_TIES];
    double dz[ORACLE_MAX_TIES];
} tie_rec;

/* Codes of one 128-column group of z (n <= 128 values) on the fp8 path: the
 * group's scale *sc = amax / 448 (1 for an all-zero group) and each code
 * decided in float32 as the device does, RNE(z / scale).  alt (may be NULL):
 * with window > 0 the other code of a near-tie code (oracle_fp8_tie_alt),
 * else -1. */
static void z_group_codes(const double* z, int64_t n, float window, uint8_t* codes, float* sc,
                          int16_t* alt)
{
    float zf[128], amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        zf[i] = (float)z[i];
        if (fabsf(zf[i]) > amax)
            amax = fabsf(zf[i]);
    }
    *sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;
    for (int64_t i = 0; i < n; ++i) {
        codes[i] = oracle_fp8_encode(zf[i] / *sc);
        if (alt)
            alt[i] = (int16_t)((window > 0.0f) ? oracle_fp8_tie_alt(zf[i] / *sc, window) : -1);
    }
}

/* z requantisation for the fp8 path: each 128-column group of a row gets
 * its own scale (the block-wise granularity of the "FP8 W8A8" section);
 * z is replaced by its dequantised codes.  With window > 0 the codes within
 * that relative distance of a rounding tie go into tr. */
static void requant_z(double* z, int64_t I, float window, tie_rec* tr)
{
    for (int64_t g0 = 0; g0 < I; g0 += 128) {
        const int64_t n = (I - g0 < 128) ? I - g0 : 128;
        uint8_t c[128];
        int16_t alt[128];
        float sc;
        z_group_codes(z + g0, n, (tr ? window : 0.0f), c, &sc, alt);
        for (int64_t i = 0; i < n; ++i) {
            z[g0 + i] = fp8_table[c[i]] * (double)sc;
            if (alt[i] >= 0) {
                if (tr->n < ORACLE_MAX_TIES) {
                    tr->k[tr->n] = g0 + i;
                    tr->dz[tr->n] = (fp8_table[alt[i]] - fp8_table[c[i]]) * (double)sc;
                }
                tr->n++;
            }
        }
    }
}

/* o += zi * (row i of expert e's dequantised W2). */
static void add_w2_row(const oracle_experts* W, int e, int64_t i, double zi, double* o)
{
    const int64_t H = W->H, I = W->I;
    const int64_t base = ((int64_t)e * I + i) * H;
    if (W->w_dtype == OR_F32) {
        const float* w = (const float*)W->w2 + base;
        for (int64_t c = 0; c < H; ++c)
            o[c] += zi * (double)w[c];
    } else if (W->w_dtype == OR_BF16) {
        const uint16_t* w = (const uint16_t*)W->w2 + base;
        for (int64_t c = 0; c < H; ++c)
            o[c] += zi * bf16_bits_to_double(w[c]);
    } else if (W->w_dtype == OR_U8 || W->w_dtype == OR_U4) {
        for (int64_t c = 0; c < H; ++c)
            o[c] += zi * wq_weight(W, W->w2, W->w2_scale, W->w2_zero, e, I, H, i, c);
    } else if (W->block > 0) {
        /* scale of weight (i, c): block (c / B, i / B) of expert e */
        const int64_t B = W->block, nbn = (H + B - 1) / B, nbk = (I + B - 1) / B;
        const uint8_t* w = (const uint8_t*)W->w2 + base;
        const float* sc = W->w2_scale + (int64_t)e * nbn * nbk + i / B;
        for (int64_t c = 0; c < H; ++c)
            o[c] += zi * (fp8_table[w[c]] * (double)sc[(c / B) * nbk]);
    } else {
        const uint8_t* w = (const uint8_t*)W->w2 + base;
        const float* sc = W->w2_scale + (int64_t)e * H;
        for (int64_t c = 0; c < H; ++c)
            o[c] += zi * (fp8_table[w[c]] * (double)sc[c]);
    }
}

/* h = W13_e^T x + b13_e and z = a * SiLU(h[:I]) * h[I:] of one expert row,
 * before any requantisation.  a = zscale: 1, or the routing weight when it
 * is applied to the first layer's output (the walkthrough's
 * apply_router_weight_on_input, sec. 1.2).  h[2I], z[I]. */
static void expert_hz(const oracle_experts* W, int e, const double* x, double* h, double* z,
                      double zscale)
{
    const int64_t H = W->H, I = W->I, N = 2 * (int64_t)W->I;

    for (int64_t n = 0; n < N; ++n)
        h[n] = 0.0;
    for (int64_t k = 0; k < H; ++k) {
        const double xk = x[k];
        const int64_t base = ((int64_t)e * H + k) * N;
        if (W->w_dtype == OR_F32) {
            const float* w = (const float*)W->w13 + base;
            for (int64_t n = 0; n < N; ++n)
                h[n] += xk * (double)w[n];
        } else if (W->w_dtype == OR_BF16) {
            const uint16_t* w = (const uint16_t*)W->w13 + base;
            for (int64_t n = 0; n < N; ++n)
                h[n] += xk * bf16_bits_to_double(w[n]);
        } else if (W->w_dtype == OR_U8 || W->w_dtype == OR_U4) {
            for (int64_t n = 0; n < N; ++n)
                h[n] += xk * wq_weight(W, W->w13, W->w13_scale, W->w13_zero, e, H, N, k, n);
        } else if (W->block > 0) {
            /* scale of weight (k, n): block (n / B, k / B) of expert e */
            const int64_t B = W->block, nbn = (N + B - 1) / B, nbk = (H + B - 1) / B;
            const uint8_t* w = (const uint8_t*)W->w13 + base;
            const float* sc = W->w13_scale + (int64_t)e * nbn * nbk + k / B;
            for (int64_t n = 0; n < N; ++n)
                h[n] += xk * (fp8_table[w[n]] * (double)sc[(n / B) * nbk]);
        } else {
            const uint8_t* w = (const uint8_t*)W->w13 + base;
            const float* sc = W->w13_scale + (int64_t)e * N;
            for (int64_t n = 0; n < N; ++n)
                h[n] += xk * (fp8_table[w[n]] * (double)sc[n]);
        }
    }
    if (W->w13_bias)
        for (int64_t n = 0; n < N; ++n)
            h[n] += bias_at(W, W->w13_bias, (int64_t)e * N + n);

    for (int64_t i = 0; i < I; ++i) {
        const double g = h[i], u = h[I + i];
        z[i] = zscale * (g / (1.0 + exp(-g)) * u); /* SiLU(g) = g * sigmoid(g) */
    }
}

/* o = f_e(x): h and z as expert_hz; on the fp8 path z re-quantised
 * (requant_z), with z_bf16 z held in bf16 (the walkthrough's
 * "fused_experts_impl" keeps the activation output, intermediate_cache2, in
 * the compute type); o = W2_e^T z + b2_e.  scratch: h[2I], z[I].  window / tr:
 * near-tie z codes (fp8 path), see requant_z. */
static void expert_ffn(const oracle_experts* W, int e, const double* x, double* h, double* z,
                       double* o, double zscale, float window, tie_rec* tr)
{
    const int64_t H = W->H, I = W->I;

    expert_hz(W, e, x, h, z, zscale);
    if (W->requant_z)
        requant_z(z, I, window, tr);
    else if (W->z_bf16)
        for (int64_t i = 0; i < I; ++i)
            z[i] = round_bf16((float)z[i]);

    for (int64_t c = 0; c < H; ++c)
        o[c] = 0.0;
    for (int64_t i = 0; i < I; ++i)
        add_w2_row(W, e, i, z[i], o);
    if (W->w2_bias)
        for (int64_t c = 0; c < H; ++c)
            o[c] += bias_at(W, W->w2_bias, (int64_t)e * H + c);
}

/* Contiguous format.  For each listed token t: y[t] = sum_j w[t,j] f_{id[t,j]}(x_t),
 * j ascending, with (ids, weights) from oracle_route (or given).
 * tokens[n_tokens] index rows of the activations; y is [n_tokens][H] double.
 * expert_map (may be NULL): global expert id -> index into W's experts, -1 for
 * an expert held by another expert-parallel rank, whose items are left out
 * (y is then this rank's partial sum).  weight_on_input: the routing weight
 * scales z_r and the expert outputs are summed unweighted.
 * nthreads <= 0 keeps the OpenMP default.  Returns the thread count used. */
/* Near-tie deltas of one output row: each recorded tie t of an expert row
 * (scaled by `scale`, the routing weight the row enters the output with)
 * becomes delta slot *used (while there is one): scale * dz_t * W2_e row k_t,
 * the change of the output if that code were rounded the other way. */
static void tie_deltas(const oracle_experts* W, int e, const tie_rec* tr, double scale,
                       double* delta, int32_t* used)
{
    const int64_t H = W->H;
    const int n = tr->n < ORACLE_MAX_TIES ? tr->n : ORACLE_MAX_TIES;
    for (int t = 0; t < n && *used < ORACLE_MAX_TIES; ++t) {
        double* d = delta + (int64_t)(*used) * H;
        for (int64_t c = 0; c < H; ++c)
            d[c] = 0.0;
        add_w2_row(W, e, tr->k[t], scale * tr->dz[t], d);
        ++*used;
    }
}

static int forward_tokens(const oracle_experts* W, const oracle_acts* A, int32_t top_k,
                          const int32_t* topk_ids, const double* topk_w, const int64_t* tokens,
                          int64_t n_tokens, double* y, int32_t nthreads,
                          const int32_t* expert_map, int32_t weight_on_input, float window,
                          int32_t* tie_count, double* tie_delta)
{
    int used = 1;
    fp8_table_init();
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        const int64_t H = W->H, I = W->I;
        double* x = (double*)malloc(sizeof(double) * H);
        float* xf = (float*)malloc(sizeof(float) * H);
        uint8_t* q = (uint8_t*)malloc(H);
        double* h = (double*)malloc(sizeof(double) * 2 * I);
        double* z = (double*)malloc(sizeof(double) * I);
        double* o = (double*)malloc(sizeof(double) * H);
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_tokens; ++n) {
            const int64_t t = tokens[n];
            double* yt = y + n * H;
            int32_t ties = 0, used = 0;
            load_row(A, H, t, x, xf, q);
            for (int64_t c = 0; c < H; ++c)
                yt[c] = 0.0;
            for (int j = 0; j < top_k; ++j) {
                const int g = topk_ids[t * top_k + j];
                const int e = expert_map ? expert_map[g] : g;
                const double wj = topk_w[t * top_k + j];
                tie_rec tr = {0};
                if (e < 0)
                    continue;                       /* held by another rank */
                if (weight_on_input) {
                    expert_ffn(W, e, x, h, z, o, wj, window, &tr);
                    for (int64_t c = 0; c < H; ++c)
                        yt[c] += o[c];
                } else {
                    expert_ffn(W, e, x, h, z, o, 1.0, window, &tr);
                    for (int64_t c = 0; c < H; ++c)
                        yt[c] += wj * o[c];
                }
                if (tie_count) {
                    ties += tr.n;
                    tie_deltas(W, e, &tr, weight_on_input ? 1.0 : wj,
                               tie_delta + n * ORACLE_MAX_TIES * H, &used);
                }
            }
            if (tie_count)
                tie_count[n] = ties;
        }
        free(x);
        free(xf);
        free(q);
        free(h);
        free(z);
        free(o);
    }
    return used;
}

int oracle_forward_tokens(const oracle_experts* W, const oracle_acts* A, int32_t top_k,
                          const int32_t* topk_ids, const double* topk_w, const int64_t* tokens,
                          int64_t n_tokens, double* y, int32_t nthreads,
                          const int32_t* expert_map, int32_t weight_on_input)
{
    return forward_tokens(W, A, top_k, topk_ids, topk_w, tokens, n_tokens, y, nthreads,
                          expert_map, weight_on_input, 0.0f, NULL, NULL);
}

/* oracle_forward_tokens that also reports the fp8 z codes decided within a
 * relative `window` of a rounding tie (see oracle_fp8_tie_alt): tie_count[n]
 * is the number of such codes behind token n's output, and tie_delta
 * [n_tokens][ORACLE_MAX_TIES][H] the change of y[n] if the i-th of them were
 * rounded the other way (the first ORACLE_MAX_TIES; any subset of them gives
 * an equally correct output, since GEMM2 and the reduction are linear in z). */
int oracle_forward_tokens_ties(const oracle_experts* W, const oracle_acts* A, int32_t top_k,
                               const int32_t* topk_ids, const double* topk_w,
                               const int64_t* tokens, int64_t n_tokens, double* y,
                               int32_t nthreads, const int32_t* expert_map,
                               int32_t weight_on_input, float window, int32_t* tie_count,
                               double* tie_delta)
{
    return forward_tokens(W, A, top_k, topk_ids, topk_w, tokens, n_tokens, y, nthreads,
                          expert_map, weight_on_input, window, tie_count, tie_delta);
}

int oracle_max_ties(void) { return ORACLE_MAX_TIES; }

static int expert_rows(const oracle_experts* W, const oracle_acts* A, const int64_t* rows,
                       const int32_t* experts, int64_t n_rows, double* out, int32_t nthreads,
                       float window, int32_t* tie_count, double* tie_delta);

/* Any list of (activation row, expert) pairs: out[n][H] = f_{experts[n]}(row rows[n]).
 * Serves the batched format, where row = e * max_tokens + i for i < count_e. */
int oracle_expert_rows(const oracle_experts* W, const oracle_acts* A, const int64_t* rows,
                       const int32_t* experts, int64_t n_rows, double* out, int32_t nthreads)
{
    return expert_rows(W, A, rows, experts, n_rows, out, nthreads, 0.0f, NULL, NULL);
}

/* oracle_expert_rows with the near-tie report of oracle_forward_tokens_ties. */
int oracle_expert_rows_ties(const oracle_experts* W, const oracle_acts* A, const int64_t* rows,
                            const int32_t* experts, int64_t n_rows, double* out,
                            int32_t nthreads, float window, int32_t* tie_count,
                            double* tie_delta)
{
    return expert_rows(W, A, rows, experts, n_rows, out, nthreads, window, tie_count, tie_delta);
}

static int expert_rows(const oracle_experts* W, const oracle_acts* A, const int64_t* rows,
                       const int32_t* experts, int64_t n_rows, double* out, int32_t nthreads,
                       float window, int32_t* tie_count, double* tie_delta)
{
    int used = 1;
    fp8_table_init();
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        const int64_t H = W->H, I = W->I;
        double* x = (double*)malloc(sizeof(double) * H);
        float* xf = (float*)malloc(sizeof(float) * H);
        uint8_t* q = (uint8_t*)malloc(H);
        double* h = (double*)malloc(sizeof(double) * 2 * I);
        double* z = (double*)malloc(sizeof(double) * I);
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_rows; ++n) {
            tie_rec tr = {0};
            int32_t used = 0;
            load_row(A, H, rows[n], x, xf, q);
            expert_ffn(W, experts[n], x, h, z, out + n * H, 1.0, window, &tr);
            if (tie_count) {
                tie_count[n] = tr.n;
                tie_deltas(W, experts[n], &tr, 1.0, tie_delta + n * ORACLE_MAX_TIES * H, &used);
            }
        }
        free(x);
        free(xf);
        free(q);
        free(h);
        free(z);
    }
    return used;
}

/* The fp8 path's re-quantised intermediate for any list of (activation row,
 * expert) pairs (the "FP8 W8A8" section's per-group codes of z): codes[n][I]
 * and scales[n][ceil(I/128)] as requant_z decides them, and alt[n][I] the
 * other code of each near-tie code (relative window, oracle_fp8_tie_alt),
 * else -1.  Returns the thread count used. */
int oracle_expert_z_codes(const oracle_experts* W, const oracle_acts* A, const int64_t* rows,
                          const int32_t* experts, int64_t n_rows, float window, uint8_t* codes,
                          float* scales, int16_t* alt, int32_t nthreads)
{
    int used = 1;
    fp8_table_init();
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        const int64_t H = W->H, I = W->I, G = (I + 127) / 128;
        double* x = (double*)malloc(sizeof(double) * H);
        float* xf = (float*)malloc(sizeof(float) * H);
        uint8_t* q = (uint8_t*)malloc(H);
        double* h = (double*)malloc(sizeof(double) * 2 * I);
        double* z = (double*)malloc(sizeof(double) * I);
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_rows; ++n) {
            load_row(A, H, rows[n], x, xf, q);
            expert_hz(W, experts[n], x, h, z, 1.0);
            for (int64_t g = 0; g < G; ++g) {
                const int64_t g0 = g * 128, m = (I - g0 < 128) ? I - g0 : 128;
                z_group_codes(z + g0, m, window, codes + n * I + g0, scales + n * G + g,
                              alt + n * I + g0);
            }
        }
        free(x);
        free(xf);
        free(q);
        free(h);
        free(z);
    }
    return used;
}

/* z = a * SiLU(h[:I]) * h[I:] (a = 1) of any list of (activation row,
 * expert) pairs, before any requantisation: z[n][I].  Returns the thread
 * count used. */
int oracle_expert_z(const oracle_experts* W, const oracle_acts* A, const int64_t* rows,
                    const int32_t* experts, int64_t n_rows, double* zout, int32_t nthreads)
{
    int used = 1;
    fp8_table_init();
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#endif
#pragma omp parallel
    {
        const int64_t H = W->H, I = W->I;
        double* x = (double*)malloc(sizeof(double) * H);
        float* xf = (float*)malloc(sizeof(float) * H);
        uint8_t* q = (uint8_t*)malloc(H);
        double* h = (double*)malloc(sizeof(double) * 2 * I);
#ifdef _OPENMP
#pragma omp single
        used = omp_get_num_threads();
#endif
#pragma omp for schedule(dynamic, 1)
        for (int64_t n = 0; n < n_rows; ++n) {
            load_row(A, H, rows[n], x, xf, q);
            expert_hz(W, experts[n], x, h, zout + n * I, 1.0);
        }
        free(x);
        free(xf);
        free(q);
        free(h);
    }
    return used;
}
