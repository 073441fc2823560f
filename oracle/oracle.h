/*
 * CPU oracle for the fused MoE router — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, single-threaded C99 in fp64.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the product path
 * (librouter and its Python binding) never does.  It shares no source with
 * the HIP path.
 *
 * What it computes is the plain definition of the router, taken from the
 * pages on the fused route kernel (qwisp issue #145: the gate matvec
 * postNorm[H] -> gateLogits[E] followed by a top-8 whose tie order is part of
 * the contract), the dense-router decode notes (sqrt(softplus) activation,
 * selection on score plus bias with unbiased weights kept beside the key,
 * renormalised winners) and the B70 MTP1 M=2 note (the unique-route table,
 * and the routed gather + shared-expert add that consumes the routes, whose
 * FP32 -> BF16 -> + BF16 -> BF16 chain fixes its precision, so that part
 * works in fp32 and BF16 as the note states rather than in fp64).
 *
 * All functions return 0 on success and a negative value on bad arguments.
 */
#ifndef ROUTER_ORACLE_H
#define ROUTER_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_SOFTMAX 0
#define ORACLE_SQRT_SOFTPLUS 1

#define ORACLE_EINVAL (-1)
#define ORACLE_ENONFINITE (-2)
#define ORACLE_ENOMEM (-3)

/* logits[t,e] = fl32( sum_i x[t,i] * w[e,i] ), summed in i order in double;
 * absdot[t,e] = sum_i |x[t,i] * w[e,i]| in double (may be NULL).
 * x: bf16 bits [M,H]; w: bf16 bits [E,H]; both row-major. */
int oracle_logits(const uint16_t* x, const uint16_t* w, int64_t M, int64_t H, int64_t E,
                  float* logits, double* absdot);

/* Scoring, key, top-k selection and weights on fp32 logits [M,E].
 * bias: fp32 [E] or NULL (NULL selects on the logit itself).
 * inds: int32 [M,k]; weights: fp32 [M,k]. */
int oracle_topk_from_logits(const float* logits, const float* bias, int64_t M, int64_t E,
                            int k, int scoring, int renorm, int32_t* inds, float* weights);

/* MXFP4 gate weights (OCP Microscaling Formats v1.0).  elems: uint8 [E, H/2],
 * element i of a row in byte i/2, even i in the low nibble, each an FP4 E2M1
 * code; scales: uint8 [E, H/32], E8M0: element i of row e is
 * e2m1(code) * 2^(scales[e, i/32] - 127).  Scales outside
 * [ORACLE_MX_SCALE_MIN, ORACLE_MX_SCALE_MAX] (every dequantised weight then
 * is a normal bf16 value, or zero) are refused, as is H % 32 != 0. */
#define ORACLE_MX_SCALE_MIN 2
#define ORACLE_MX_SCALE_MAX 252
double oracle_e2m1_value(int code);
/* w: [E, H] doubles. */
int oracle_dequant_mxfp4(const uint8_t* elems, const uint8_t* scales, int64_t E, int64_t H,
                         double* w);
/* The router on MXFP4 gate weights: logits[t,e] = fl32(sum_i x[t,i] * w[e,i])
 * with the dequantised w, then oracle_topk_from_logits. */
int oracle_router_mxfp4(const uint16_t* x, const uint8_t* elems, const uint8_t* scales,
                        const float* bias, int64_t M, int64_t H, int64_t E, int k, int scoring,
                        int renorm, int32_t* inds, float* weights, float* logits_out,
                        double* absdot_out);

/* MXFP8 gate weights (OCP Microscaling Formats v1.0, FP8 E4M3 elements):
 * elems: uint8 [E, H], one E4M3 code per element; scales: uint8 [E, H/32],
 * E8M0: element i of row e is e4m3(code) * 2^(scales[e, i/32] - 127).
 * Scales outside [ORACLE_MX8_SCALE_MIN, ORACLE_MX8_SCALE_MAX] or NaN codes
 * are refused (inside, every dequantised weight is zero or a normal bf16
 * value: the smallest E4M3 magnitude is 2^-9, the largest 448). */
#define ORACLE_MX8_SCALE_MIN 10
#define ORACLE_MX8_SCALE_MAX 246
double oracle_e4m3_value(int code);
int oracle_dequant_mxfp8(const uint8_t* elems, const uint8_t* scales, int64_t E, int64_t H,
                         double* w);
/* The router on MXFP8 gate weights (as oracle_router_mxfp4). */
int oracle_router_mxfp8(const uint16_t* x, const uint8_t* elems, const uint8_t* scales,
                        const float* bias, int64_t M, int64_t H, int64_t E, int k, int scoring,
                        int renorm, int32_t* inds, float* weights, float* logits_out,
                        double* absdot_out);

/* The whole router: logits then oracle_topk_from_logits.  logits_out [M,E]
 * and absdot_out [M,E] are optional (NULL). */
int oracle_router(const uint16_t* x, const uint16_t* w, const float* bias, int64_t M,
                  int64_t H, int64_t E, int k, int scoring, int renorm, int32_t* inds,
                  float* weights, float* logits_out, double* absdot_out);

/* Unique-route table of M tokens (1 <= M <= 31).  inds: [M,k] as produced by
 * the router; slots s = t*k + j are walked token-major, then rank.
 * ids [M*k]: distinct experts in order of first appearance, -1 after count;
 * token_mask [M*k]: bit t set iff token t selected ids[q], 0 after count;
 * slot_to_unique [M*k]: position of slot s's expert in ids; count [1].
 * (The B70 note defines the table for the MTP1 pair, M=2; the same walk
 * gives it at every verify width.) */
int oracle_route_table(const int32_t* inds, int M, int k, int32_t* ids, int32_t* token_mask,
                       int32_t* slot_to_unique, int32_t* count);

/* The M=2 table (oracle_route_table with M=2). */
int oracle_route_table_m2(const int32_t* inds, int k, int32_t* ids, int32_t* token_mask,
                          int32_t* slot_to_unique, int32_t* count);

/* Per-row scores in double, as used by the key and the weights (exposed for
 * the self-checks).  score[e]: softmax probability or sqrt-softplus value;
 * unbiased[e]: the quantity renormalisation divides (exp(l-max) for softmax,
 * the sqrt-softplus value otherwise). */
int oracle_row_scores(const float* logits_row, int64_t E, int scoring, double* score,
                      double* unbiased);

/* Round an fp32 value to BF16 bits: to nearest, ties to even; overflow to
 * infinity; NaN stays a (quiet) NaN. */
uint16_t oracle_bf16_round(float f);

/* Routed gather + shared-expert add (B70 note, "Exact arithmetic"):
 *   out[t,d] = bf16( bf16( acc ) + shared[t,d] ),
 *   acc = fp32 sum over slots j in order of fl32(weights[t,j] * y[r,d]),
 *         r = slot_rows[t*k + j], slots with r == -1 skipped.
 * y: bf16 bits [y_rows, D]; slot_rows: int32 [M*k], each in [-1, y_rows);
 * weights: fp32 [M*k]; shared, out: bf16 bits [M, D]. */
int oracle_gather_shared_add(const uint16_t* y, int64_t y_rows, int64_t D, const int32_t* slot_rows,
                             const float* weights, const uint16_t* shared, int64_t M, int k,
                             uint16_t* out);

/* slot_rows [M*k] of the compact expert-output layout that the unique-route
 * table (token_mask, slot_to_unique, count) implies: unique experts in table
 * order, each with the rows of its tokens in token order (1 <= M <= 31). */
int oracle_table_rows(const int32_t* token_mask, const int32_t* slot_to_unique, int count, int M,
                      int k, int32_t* slot_rows);

/* Expert GEMM1 on the table's compact rows: for unique expert u < count
 * (expert unique_ids[u]) and each token t of token_mask[u], in table order
 * then token order, out[row, f] = sum_d x[t,d] * w1[unique_ids[u], f, d]
 * exactly in double (absdot: the sum of |products|, may be NULL).
 * x: bf16 bits [M, D]; w1: bf16 bits [E, F, D]; out, absdot: [rows, F].
 * Returns the number of rows written (>= 0) or a negative error. */
int oracle_expert_gemm1_table(const uint16_t* x, const uint16_t* w1, int64_t E, int64_t F, int64_t D,
                              const int32_t* unique_ids, const int32_t* token_mask, int count, int M,
                              double* out, double* absdot);

#ifdef __cplusplus
}
#endif

#endif
