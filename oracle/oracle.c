/*
 * CPU oracle for the fused MoE router — TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, the smoke check and the benchmark's CPU-baseline leg may load
 * this.  It is deliberately plain: one row at a time, fp64 throughout, no
 * blocking, no fusion, no reordering beyond what each step's definition says.
 * It shares no code with the HIP path.
 *
 * Sources (pages on the fused MoE router):
 *  - qwisp issue #145, "Observation"/"Change": the gate matvec postNorm[H] ->
 *    gateLogits[E=256] followed by a top-8 producing inds and scores.
 *  - qwisp issue #145, "Bit-exactness": the tie order of the top-k selection is
 *    part of the contract.  Here: keys descending, equal keys to the lower
 *    expert index, emitted in that order.
 *  - dense_router_decode commit notes ("DenseRouterDecodeKernel"): score is
 *    sqrt(softplus(logit)) with the stable softplus max(x,0)+log(1+exp(-|x|));
 *    selection is on score plus a per-expert bias; the heap carries the
 *    unbiased activation beside the selection key, and the winners'
 *    unbiased values are renormalised.
 *  - b70 lab MTP1 note, "Unique-route router screen": the M=2 table of
 *    encounter-ordered unique experts, per-expert token masks, slot-to-unique
 *    map and unique count, leaving ids and weights untouched.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - logits are fp32: the exact dot product of the bf16 operands (summed in
 *    double, in index order) rounded once to fp32;
 *  - scores are computed in double from the fp32 logit and rounded once to
 *    fp32 where they form a key; softplus uses log1p;
 *  - with no bias the selection key is the logit itself (both scorings are
 *    strictly increasing in it); with a bias the key is fl32(fl32(score)+bias),
 *    the score being the softmax probability or the sqrt-softplus value;
 *  - -0 and +0 are the same key;
 *  - renormalised weight j = u_j / sum of the winners' u in rank order, with u
 *    = exp(l - max l) for softmax and the sqrt-softplus value otherwise; without
 *    renormalisation the weight is the full-row probability (softmax) or the
 *    sqrt-softplus value; the bias never enters a weight;
 *  - table: slots walked token-major then rank; an expert's position is the
 *    order of its first appearance; mask bit t set when token t picked it;
 *    unused ids are -1 and unused masks 0;
 *  - block-scaled gate (the notes' NVFP4 gate, in the MX form gfx950 reads
 *    natively): OCP MXFP4, E2M1 codes two per byte (even element low), one
 *    E8M0 scale per 32 elements of a row; scales in [2, 252], so every
 *    dequantised weight is zero or a normal bf16 value and the logits are
 *    the exact dot product with those values, as for bf16 weights.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_logits(const uint16_t* x, const uint16_t* w, int64_t M, int64_t H, int64_t E,
                  float* logits, double* absdot)
{
    if (M < 0 || H < 1 || E < 1 || (M > 0 && (!x || !w || !logits))) return ORACLE_EINVAL;
    for (int64_t t = 0; t < M; ++t) {
        const uint16_t* xr = x + t * H;
        for (int64_t e = 0; e < E; ++e) {
            const uint16_t* wr = w + e * H;
            double acc = 0.0, mag = 0.0;
            for (int64_t i = 0; i < H; ++i) {
                /* a product of two bf16 values is exact in double */
                double p = bf16_value(xr[i]) * bf16_value(wr[i]);
                acc += p;
                mag += fabs(p);
            }
            logits[t * E + e] = (float)acc;
            if (absdot) absdot[t * E + e] = mag;
        }
    }
    return 0;
}

int oracle_row_scores(const float* l, int64_t E, int scoring, double* score, double* unbiased)
{
    if (E < 1 || !l || !score || !unbiased) return ORACLE_EINVAL;
    if (scoring == ORACLE_SOFTMAX) {
        double m = (double)l[0];
        for (int64_t e = 1; e < E; ++e)
            if ((double)l[e] > m) m = (double)l[e];
        double Z = 0.0;
        for (int64_t e = 0; e < E; ++e) {
            unbiased[e] = exp((double)l[e] - m);
            Z += unbiased[e];
        }
        for (int64_t e = 0; e < E; ++e) score[e] = unbiased[e] / Z;
    } else if (scoring == ORACLE_SQRT_SOFTPLUS) {
        for (int64_t e = 0; e < E; ++e) {
            double v = (double)l[e];
            double softplus = fmax(v, 0.0) + log1p(exp(-fabs(v)));
            score[e] = sqrt(softplus);
            unbiased[e] = score[e];
        }
    } else {
        return ORACLE_EINVAL;
    }
    return 0;
}

/* Does expert a (key ka) come before expert b (key kb) in the selection order? */
static int precedes(float ka, int32_t a, float kb, int32_t b)
{
    if (ka > kb) return 1;
    if (ka < kb) return 0;
    return a < b;
}

int oracle_topk_from_logits(const float* logits, const float* bias, int64_t M, int64_t E,
                            int k, int scoring, int renorm, int32_t* inds, float* weights)
{
    if (M < 0 || E < 1 || k < 1 || k > E) return ORACLE_EINVAL;
    if (scoring != ORACLE_SOFTMAX && scoring != ORACLE_SQRT_SOFTPLUS) return ORACLE_EINVAL;
    if (M > 0 && (!logits || !inds || !weights)) return ORACLE_EINVAL;

    double* score = (double*)malloc((size_t)E * sizeof(double));
    double* unb = (double*)malloc((size_t)E * sizeof(double));
    float* key = (float*)malloc((size_t)E * sizeof(float));
    float* top_key = (float*)malloc((size_t)k * sizeof(float));
    int32_t* top_idx = (int32_t*)malloc((size_t)k * sizeof(int32_t));
    int rc = 0;
    if (!score || !unb || !key || !top_key || !top_idx) {
        rc = ORACLE_ENOMEM;
        goto done;
    }

    for (int64_t t = 0; t < M; ++t) {
        const float* l = logits + t * E;
        rc = oracle_row_scores(l, E, scoring, score, unb);
        if (rc) goto done;

        /* selection key */
        for (int64_t e = 0; e < E; ++e) {
            float kv;
            if (bias) {
                float s32 = (float)score[e];
                kv = s32 + bias[e]; /* one fp32 addition, round to nearest */
            } else {
                kv = l[e];
            }
            if (!isfinite(kv)) {
                rc = ORACLE_ENONFINITE;
                goto done;
            }
            if (kv == 0.0f) kv = 0.0f; /* -0 and +0 are one key */
            key[e] = kv;
        }

        /* top-k by insertion into a ranked list */
        int filled = 0;
        for (int64_t e = 0; e < E; ++e) {
            int32_t idx = (int32_t)e;
            float kv = key[e];
            if (filled == k && !precedes(kv, idx, top_key[k - 1], top_idx[k - 1])) continue;
            int pos = (filled < k) ? filled : k - 1;
            /* walk up while the new entry precedes the one above it */
            while (pos > 0 && precedes(kv, idx, top_key[pos - 1], top_idx[pos - 1])) {
                top_key[pos] = top_key[pos - 1];
                top_idx[pos] = top_idx[pos - 1];
                --pos;
            }
            top_key[pos] = kv;
            top_idx[pos] = idx;
            if (filled < k) ++filled;
        }

        /* weights of the winners: unbiased values, optionally renormalised */
        double total = 0.0;
        for (int j = 0; j < k; ++j) total += unb[top_idx[j]];
        for (int j = 0; j < k; ++j) {
            int32_t e = top_idx[j];
            double wgt;
            if (renorm)
                wgt = unb[e] / total;
            else
                wgt = score[e];
            inds[t * k + j] = e;
            weights[t * k + j] = (float)wgt;
        }
    }

done:
    free(score);
    free(unb);
    free(key);
    free(top_key);
    free(top_idx);
    return rc;
}

/* MXFP4 gate weights (OCP Microscaling Formats v1.0; the gfx950 counterpart of
 * the NVFP4 gate of the dense_router_decode notes, "NVFP4 gate"): element FP4
 * E2M1 = sign, two exponent bits (bias 1), one mantissa bit, no inf/NaN; a
 * shared E8M0 scale 2^(s-127) per 32 consecutive elements of a row. */
double oracle_e2m1_value(int code)
{
    int sign = (code >> 3) & 1, ex = (code >> 1) & 3, man = code & 1;
    double mag = ex == 0 ? 0.5 * man                     /* subnormal: 0 or 0.5 */
                         : ldexp(1.0 + 0.5 * man, ex - 1);
    return sign ? -mag : mag;
}

int oracle_dequant_mxfp4(const uint8_t* elems, const uint8_t* scales, int64_t E, int64_t H,
                         double* w)
{
    if (E < 1 || H < 32 || H % 32 != 0 || !elems || !scales || !w) return ORACLE_EINVAL;
    for (int64_t e = 0; e < E; ++e)
        for (int64_t col = 0; col < H; ++col) {
            int sc = scales[e * (H / 32) + col / 32];
            if (sc < ORACLE_MX_SCALE_MIN || sc > ORACLE_MX_SCALE_MAX) return ORACLE_EINVAL;
            int byte = elems[e * (H / 2) + col / 2];
            int code = (col % 2 == 0) ? (byte & 15) : (byte >> 4); /* even element: low nibble */
            w[e * H + col] = ldexp(oracle_e2m1_value(code), sc - 127);
        }
    return 0;
}

/* The router on dequantised block-scaled weights w [E, H] (doubles): exact
 * dot products with the bf16 activations, then the router's selection. */
static int router_on_dequantised(const uint16_t* x, const double* w, const float* bias, int64_t M,
                                 int64_t H, int64_t E, int k, int scoring, int renorm,
                                 int32_t* inds, float* weights, float* logits_out,
                                 double* absdot_out)
{
    float* l = logits_out ? logits_out : (float*)calloc((size_t)(M * E), sizeof(float));
    if (!l) return ORACLE_ENOMEM;
    for (int64_t t = 0; t < M; ++t)
        for (int64_t e = 0; e < E; ++e) {
            double acc = 0.0, absacc = 0.0;
            for (int64_t col = 0; col < H; ++col) {
                /* bf16 times a block-scaled FP4/FP8 value: exact in double */
                double p = bf16_value(x[t * H + col]) * w[e * H + col];
                acc += p;
                absacc += fabs(p);
            }
            l[t * E + e] = (float)acc;
            if (absdot_out) absdot_out[t * E + e] = absacc;
        }
    int rc = oracle_topk_from_logits(l, bias, M, E, k, scoring, renorm, inds, weights);
    if (!logits_out) free(l);
    return rc;
}

int oracle_router_mxfp4(const uint16_t* x, const uint8_t* elems, const uint8_t* scales,
                        const float* bias, int64_t M, int64_t H, int64_t E, int k, int scoring,
                        int renorm, int32_t* inds, float* weights, float* logits_out,
                        double* absdot_out)
{
    if (M < 0 || H < 32 || E < 1 || k < 1 || k > E) return ORACLE_EINVAL;
    if (M == 0) return 0;
    if (!x) return ORACLE_EINVAL;
    double* w = (double*)malloc((size_t)(E * H) * sizeof(double));
    if (!w) return ORACLE_ENOMEM;
    int rc = oracle_dequant_mxfp4(elems, scales, E, H, w);
    if (!rc)
        rc = router_on_dequantised(x, w, bias, M, H, E, k, scoring, renorm, inds, weights, logits_out,
                                   absdot_out);
    free(w);
    return rc;
}

/* OCP FP8 E4M3 (OCP 8-bit Floating Point Specification; Microscaling
 * Formats v1.0 element type): sign bit 7, exponent bits 6..3 with bias 7,
 * mantissa bits 2..0; exponent field 0 is subnormal, frac/8 * 2^-6; the
 * pattern S.1111.111 is NaN; there are no infinities (largest value 448). */
double oracle_e4m3_value(int code)
{
    const int negative = (code >> 7) & 1, biased = (code >> 3) & 15, frac = code & 7;
    if (biased == 15 && frac == 7) return NAN;
    const double magnitude = biased == 0 ? ldexp(frac / 8.0, -6) : ldexp(1.0 + frac / 8.0, biased - 7);
    return negative ? -magnitude : magnitude;
}

int oracle_dequant_mxfp8(const uint8_t* elems, const uint8_t* scales, int64_t E, int64_t H,
                         double* w)
{
    if (E < 1 || H < 32 || H % 32 != 0 || !elems || !scales || !w) return ORACLE_EINVAL;
    for (int64_t row = 0; row < E; ++row)
        for (int64_t idx = 0; idx < H; ++idx) {
            const int s8 = scales[row * (H / 32) + idx / 32];
            if (s8 < ORACLE_MX8_SCALE_MIN || s8 > ORACLE_MX8_SCALE_MAX) return ORACLE_EINVAL;
            const double v = oracle_e4m3_value(elems[row * H + idx]);  /* one code per byte */
            if (isnan(v)) return ORACLE_EINVAL;
            w[row * H + idx] = ldexp(v, s8 - 127);
        }
    return 0;
}

int oracle_router_mxfp8(const uint16_t* x, const uint8_t* elems, const uint8_t* scales,
                        const float* bias, int64_t M, int64_t H, int64_t E, int k, int scoring,
                        int renorm, int32_t* inds, float* weights, float* logits_out,
                        double* absdot_out)
{
    if (M < 0 || H < 32 || E < 1 || k < 1 || k > E) return ORACLE_EINVAL;
    if (M == 0) return 0;
    if (!x) return ORACLE_EINVAL;
    double* w8 = (double*)malloc((size_t)(E * H) * sizeof(double));
    if (!w8) return ORACLE_ENOMEM;
    int rc = oracle_dequant_mxfp8(elems, scales, E, H, w8);
    if (!rc)
        rc = router_on_dequantised(x, w8, bias, M, H, E, k, scoring, renorm, inds, weights,
                                   logits_out, absdot_out);
    free(w8);
    return rc;
}

int oracle_router(const uint16_t* x, const uint16_t* w, const float* bias, int64_t M,
                  int64_t H, int64_t E, int k, int scoring, int renorm, int32_t* inds,
                  float* weights, float* logits_out, double* absdot_out)
{
    if (M < 0 || H < 1 || E < 1 || k < 1 || k > E) return ORACLE_EINVAL;
    if (M == 0) return 0;
    float* l = logits_out ? logits_out : (float*)malloc((size_t)(M * E) * sizeof(float));
    if (!l) return ORACLE_ENOMEM;
    int rc = oracle_logits(x, w, M, H, E, l, absdot_out);
    if (!rc) rc = oracle_topk_from_logits(l, bias, M, E, k, scoring, renorm, inds, weights);
    if (!logits_out) free(l);
    return rc;
}

int oracle_route_table(const int32_t* inds, int M, int k, int32_t* ids, int32_t* token_mask,
                       int32_t* slot_to_unique, int32_t* count)
{
    if (M < 1 || M > 31 || k < 1 || !inds || !ids || !token_mask || !slot_to_unique || !count)
        return ORACLE_EINVAL;
    int n = M * k;
    int u = 0;
    for (int i = 0; i < n; ++i) {
        ids[i] = -1;
        token_mask[i] = 0;
    }
    for (int s = 0; s < n; ++s) {
        int token = s / k;
        int pos = -1;
        for (int q = 0; q < u; ++q)
            if (ids[q] == inds[s]) {
                pos = q;
                break;
            }
        if (pos < 0) {
            pos = u;
            ids[u++] = inds[s];
        }
        slot_to_unique[s] = pos;
        token_mask[pos] |= 1 << token;
    }
    *count = u;
    return 0;
}

int oracle_route_table_m2(const int32_t* inds, int k, int32_t* ids, int32_t* token_mask,
                          int32_t* slot_to_unique, int32_t* count)
{
    return oracle_route_table(inds, 2, k, ids, token_mask, slot_to_unique, count);
}

/* ------------------------------------------------------------------------
 * Routed gather + shared-expert add (B70 note, "Exact arithmetic": the
 * routed outputs are accumulated in FP32, that sum is rounded to BF16, the
 * shared expert's BF16 output is added, and the result is rounded to BF16).
 * Readings where the note is silent: token t takes its slots j = 0..k-1 in
 * order; a slot with row r >= 0 adds the fp32 product fl32(w[t,j] * y[r,d])
 * to an fp32 accumulator that starts at +0 (the product and the sum each
 * round once: no fused multiply-add); a slot with row -1 (an expert with no
 * local output row) adds nothing; the BF16 + BF16 addition is an fp32
 * addition rounded once to BF16; every rounding to BF16 is to nearest, ties
 * to even.
 * ------------------------------------------------------------------------ */
static float bf16_to_float(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_bf16_round(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if (isnan(f)) return (uint16_t)(sign | 0x7fc0u);
    if (isinf(f)) return (uint16_t)(sign | 0x7f80u);
    /* the two BF16 neighbours of |f|: its truncation and the next magnitude up */
    const uint16_t lo = (uint16_t)((u >> 16) & 0x7fffu);
    const uint16_t hi = (uint16_t)(lo + 1u);
    const double a = fabs((double)f);
    const double vlo = (double)bf16_to_float(lo);
    /* past the largest finite value the next step up is 2^128 (infinity) */
    const double vhi = hi >= 0x7f80u ? ldexp(1.0, 128) : (double)bf16_to_float(hi);
    uint16_t mag;
    if (a - vlo < vhi - a)
        mag = lo;
    else if (vhi - a < a - vlo)
        mag = hi;
    else
        mag = (lo & 1u) ? hi : lo;  /* tie: the even neighbour */
    return (uint16_t)(sign | mag);
}

int oracle_gather_shared_add(const uint16_t* y, int64_t y_rows, int64_t D, const int32_t* slot_rows,
                             const float* weights, const uint16_t* shared, int64_t M, int k,
                             uint16_t* out)
{
    if (M < 0 || k < 1 || D < 1 || y_rows < 0) return ORACLE_EINVAL;
    for (int64_t s = 0; s < M * k; ++s)
        if (slot_rows[s] < -1 || slot_rows[s] >= y_rows) return ORACLE_EINVAL;
    for (int64_t t = 0; t < M; ++t) {
        for (int64_t d = 0; d < D; ++d) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                int64_t r = slot_rows[t * k + j];
                if (r < 0) continue;
                const float p = weights[t * k + j] * bf16_to_float(y[r * D + d]);
                acc = acc + p;
            }
            const float routed = bf16_to_float(oracle_bf16_round(acc));
            const float sum = routed + bf16_to_float(shared[t * D + d]);
            out[t * D + d] = oracle_bf16_round(sum);
        }
    }
    return 0;
}

/* Rows of the compact expert-output layout the unique-route table implies
 * (B70 note, "Why literal source-direct GEMM1 is not funded": each unique
 * expert computes only its tokens' rows, [token0], [token1] or
 * [token0, token1]).  Reading: the experts' row blocks follow the table's
 * order, and inside a block the tokens come in token order, so slot
 * s = t*k + j (expert u = slot_to_unique[s]) reads row
 *   sum over v < u of popcount(token_mask[v])  +  the number of tokens
 *   below t in token_mask[u].
 * Fails if the table is inconsistent (u out of range, or bit t of
 * token_mask[u] clear). */
int oracle_table_rows(const int32_t* token_mask, const int32_t* slot_to_unique, int count, int M,
                      int k, int32_t* slot_rows)
{
    if (M < 1 || M > 31 || k < 1 || count < 0 || count > M * k) return ORACLE_EINVAL;
    for (int s = 0; s < M * k; ++s) {
        const int t = s / k;
        const int u = slot_to_unique[s];
        if (u < 0 || u >= count) return ORACLE_EINVAL;
        if (((token_mask[u] >> t) & 1) == 0) return ORACLE_EINVAL;
        int before = 0;
        for (int v = 0; v < u; ++v)
            for (int q = 0; q < M; ++q) before += (token_mask[v] >> q) & 1;
        int within = 0;
        for (int q = 0; q < t; ++q) within += (token_mask[u] >> q) & 1;
        slot_rows[s] = before + within;
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Expert GEMM1 on the unique-route table (B70 note, "Why literal
 * source-direct GEMM1 is not funded": once identical (token, expert) routes
 * are deduplicated upstream, each expert has the affine rows [token0],
 * [token1] or [token0, token1]; the table is consumed by the GEMMs).
 * Reading: unique expert u (expert id unique_ids[u]) multiplies the rows of
 * the tokens in token_mask[u] by its GEMM1 weights w1[id] ([F, D], one
 * output feature per row); the product of token t lands in the compact row
 * oracle_table_rows gives (unique experts in table order, tokens in token
 * order).  The exact dot products are returned in double, with the sums of
 * absolute products for the tolerance; the kernel rounds to BF16.
 * ------------------------------------------------------------------------ */
int oracle_expert_gemm1_table(const uint16_t* x, const uint16_t* w1, int64_t E, int64_t F, int64_t D,
                              const int32_t* unique_ids, const int32_t* token_mask, int count, int M,
                              double* out, double* absdot)
{
    if (M < 1 || M > 31 || E < 1 || F < 1 || D < 1 || count < 0) return ORACLE_EINVAL;
    int row = 0;
    for (int u = 0; u < count; ++u) {
        const int64_t id = unique_ids[u];
        if (id < 0 || id >= E) return ORACLE_EINVAL;
        const uint16_t* wexp = w1 + id * F * D;
        for (int t = 0; t < M; ++t) {
            if (((token_mask[u] >> t) & 1) == 0) continue;
            const uint16_t* xr = x + (int64_t)t * D;
            for (int64_t f = 0; f < F; ++f) {
                const uint16_t* wrow = wexp + f * D;
                double dot = 0.0, amag = 0.0;
                for (int64_t d = 0; d < D; ++d) {
                    const double prod = bf16_value(xr[d]) * bf16_value(wrow[d]);
                    dot += prod;
                    amag += fabs(prod);
                }
                out[(int64_t)row * F + f] = dot;
                if (absdot) absdot[(int64_t)row * F + f] = amag;
            }
            ++row;  /* rows follow the table's compact layout */
        }
    }
    return row;  /* number of rows written */
}
