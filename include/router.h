/*
 * librouter — fused MoE router for AMD MI355X (gfx950).
 *
 * C ABI.  Every entry point takes plain pointers and sizes; device pointers
 * are owned by the caller and are never freed or retained by the library.
 * All calls are asynchronous on `stream`: they enqueue HIP kernels and
 * return without synchronising.  After router_init() on a device no call
 * allocates memory, so calls may be captured into a HIP graph (router_status
 * excepted, which synchronises).
 *
 * What is computed (pages on the fused MoE router):
 *   - qwisp issue #145 "Observation" and "Change": the gate matvec
 *     postNorm[H] -> gateLogits[E] and the top-8 producing inds/scores, fused
 *     into one kernel whose E logits stay on chip;
 *   - qwisp issue #145 "Bit-exactness": the tie order of the selection is
 *     part of the contract — keys descending, equal keys to the lower expert
 *     index, results emitted in that order;
 *   - dense_router_decode commit notes, "DenseRouterDecodeKernel": scoring by
 *     sqrt(softplus(logit)) with the stable softplus, selection on score plus
 *     a per-expert bias, unbiased winners' scores renormalised; the BF16 GEMM
 *     with FP32 accumulation and the row-level top-k epilogue;
 *   - dense_router_decode commit notes, the fused NVFP4 router: the gate
 *     projection on block-scaled low-precision weights (here OCP MXFP4, and
 *     MXFP8 with FP8 E4M3 elements);
 *   - b70 lab MTP1 M=2 note, "Outcome" and "Exact arithmetic": the routed
 *     gather fused with the shared-expert BF16 add that follows the router;
 *   - b70 lab MTP1 M=2 note, "Why literal source-direct GEMM1 is not
 *     funded": the expert GEMM1 that consumes the unique-route table;
 *   - b70 lab MTP1 M=2 note, "Unique-route router screen": the optional M=2
 *     unique-route table produced inside the router launch (here also at the
 *     other verify widths of qwisp issue #145, "Observation").
 *
 * Precise definition (shared by every entry point):
 *   logit[t,e]  = sum_i x[t,i]*w[e,i], bf16 operands, fp32 accumulation
 *                 (order of the fp32 sum is the kernel's, fixed per call shape
 *                 and identical for every expert);
 *   scores      = softmax over the row (p_e), or s_e = sqrt(max(l,0) +
 *                 log1p(exp(-|l|))); computed in double from the fp32 logit;
 *   key[e]      = logit[e] when bias == NULL (both scorings are increasing in
 *                 the logit, so this is the exact score order);
 *               = fl32( fl32(score[e]) + bias[e] ) otherwise;
 *                 -0 and +0 are the same key;
 *   inds[t,:]   = the first k experts in (key descending, index ascending)
 *                 order, in that order;
 *   weights     = renorm: u_j / sum_{winners} u, with u = exp(l - max l)
 *                 (softmax) or s (sqrt-softplus), in double (the sum over
 *                 the winners in a fixed pairwise order), rounded once to
 *                 fp32;
 *                 no renorm: the full-row probability p_j (softmax) or s_j;
 *                 the bias never enters a weight.
 *
 * Layouts: row-major, innermost dimension contiguous.
 *   x        bf16 [M, H]    (16-byte aligned; H % 8 == 0)
 *   w        bf16 [E, H]    (W_gate, one row per expert; 16-byte aligned)
 *   bias     fp32 [E]       or NULL
 *   logits   fp32 [M, E]
 *   inds     int32 [M, k]
 *   weights  fp32 [M, k]
 *
 * Limits: 1 <= E <= 256, 1 <= k <= min(E, 16), H >= 8, H % 8 == 0, M >= 0
 * (M == 0 is a no-op).  Inputs must not alias outputs.
 *
 * Errors: arguments are validated on the host before anything is enqueued;
 * on any error nothing is launched and no output byte changes.  The return
 * value is ROUTER_OK or one of the codes below; router_strerror() names it.
 *
 * Concurrency: the fused router entry points (router_fwd*) need a
 * workspace (partial sums, tagged logit slots, arrival counters, a status
 * word).  router_init allocates ROUTER_MAX_STREAMS of them per device, and
 * each stream that calls a fused entry point takes one for itself on its
 * first call and keeps it (router_release_stream gives it back).  Calls on
 * one stream are ordered by the stream, so calls on different streams may
 * overlap freely.  A call from one more stream than that gets
 * ROUTER_ERR_BUSY, nothing launched.  A captured graph keeps the workspace
 * of the stream it was captured on: replays of it must not overlap each
 * other or calls on that stream.  router_fwd_noalloc is the exception: its
 * workspace is one static array per device, so its calls must be ordered
 * with each other (see there).  The other entry points use no workspace.
 */
#ifndef GATE_PROJECTION_TOP_ROUTER_H
#define GATE_PROJECTION_TOP_ROUTER_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ROUTER_MAX_E 256
#define ROUTER_MAX_K 16
/* router_fwd runs a decode kernel up to this many tokens (one workgroup per
 * gate row up to 4 tokens, row blocks x expert blocks x H-splits from 5) and
 * the MFMA GEMM-with-epilogue prefill kernel above it. */
#define ROUTER_DECODE_MAX_M 256
/* router_fwd_route_table: at most this many tokens, and at most
 * ROUTER_TABLE_MAX_SLOTS = M*k slots (one wavefront builds the table). */
#define ROUTER_TABLE_MAX_M 16
#define ROUTER_TABLE_MAX_SLOTS 64

typedef enum {
    ROUTER_SCORING_SOFTMAX = 0,
    ROUTER_SCORING_SQRT_SOFTPLUS = 1
} router_scoring_t;

enum {
    ROUTER_OK = 0,
    ROUTER_ERR_INVALID_ARGUMENT = 1, /* NULL required pointer, bad enum, M < 0 */
    ROUTER_ERR_UNSUPPORTED = 2,      /* shape outside the limits above */
    ROUTER_ERR_MISALIGNED = 3,       /* x or the gate weights not aligned as stated */
    ROUTER_ERR_HIP = 4,              /* a HIP runtime call failed */
    ROUTER_ERR_NO_WORKSPACE = 5,     /* workspace could not be allocated */
    ROUTER_ERR_BUSY = 6,             /* every workspace of the device is held by other streams */
    ROUTER_ERR_NOT_INITIALIZED = 7   /* first fused call on a device made under stream capture */
};

/* Streams per device that can hold a fused-router workspace at once. */
#define ROUTER_MAX_STREAMS 8

/* Allocates the ROUTER_MAX_STREAMS workspaces of `device` (or of the
 * current device when device < 0; about 34 MiB each) and zeroes what must
 * start at zero, then waits for the device.  Idempotent and thread-safe.
 * Call it before capturing a fused call into a graph: a first fused call on
 * a device that is made under stream capture cannot allocate and returns
 * ROUTER_ERR_NOT_INITIALIZED; otherwise the first fused call runs it.  The
 * workspaces live until process exit. */
int router_init(int device);

/* Gives back the workspace that `stream` holds on the current device, if
 * any, for another stream to take.  Call it only once the stream's router
 * work has finished (e.g. after synchronising the stream): a later stream
 * may otherwise race with it.  A released stream that calls again takes a
 * workspace again.  Always ROUTER_OK unless the runtime fails. */
int router_release_stream(hipStream_t stream);

/* Fused router (gate projection + scoring + top-k + renorm in one launch).
 * Decode (M <= ROUTER_DECODE_MAX_M): the gate rows (and, from 5 tokens, H)
 * are split across workgroups, which publish their logits as tagged slots;
 * a finisher workgroup picked by an arrival ticket gathers a row's E logits
 * and runs the selection.  Prefill (larger M): one MFMA GEMM whose epilogue
 * does the selection from LDS.  Logits reach HBM only when
 * opt_out_logits is non-NULL, and writing them never changes inds/weights.
 *   x, w, bias, inds, weights, opt_out_logits: device pointers (see layouts);
 *   scoring: router_scoring_t; renorm: 0 or 1. */
int router_fwd(const void* x, const void* w, const float* bias, int64_t M, int H, int E, int k,
               int scoring, int renorm, int32_t* out_inds, float* out_weights,
               float* opt_out_logits, hipStream_t stream);

/* router_fwd for exactly two tokens that also emits the unique-route table
 * in the same launch (b70 lab MTP1 note, "Unique-route router screen"):
 *   out_unique_ids      int32 [2k]: distinct experts in order of first
 *                       appearance over the slots (token 0 ranks 0..k-1,
 *                       then token 1); unused tail entries are -1;
 *   out_token_mask      int32 [2k]: bit t set iff token t selected that
 *                       unique expert; unused tail entries are 0;
 *   out_slot_to_unique  int32 [2k]: for slot s = t*k + j, the position of
 *                       inds[t,j] in out_unique_ids;
 *   out_unique_count    int32 [1]:  number of distinct experts (k..2k).
 * inds/weights are bit-identical to router_fwd's on the same inputs. */
int router_fwd_m2_table(const void* x, const void* w, const float* bias, int H, int E, int k,
                        int scoring, int renorm, int32_t* out_inds, float* out_weights,
                        float* opt_out_logits, int32_t* out_unique_ids,
                        int32_t* out_token_mask, int32_t* out_slot_to_unique,
                        int32_t* out_unique_count, hipStream_t stream);

/* router_fwd plus the unique-route table at any verify width: the table of
 * router_fwd_m2_table extended from the MTP1 pair to M tokens (qwisp issue
 * #145, "Observation": the router runs at every verify width), in the same
 * launch.  Slots s = t*k + j are walked token-major, then rank:
 *   out_unique_ids      int32 [M*k]: distinct experts in order of first
 *                       appearance; unused tail entries are -1;
 *   out_token_mask      int32 [M*k]: bit t set iff token t selected that
 *                       unique expert; unused tail entries are 0;
 *   out_slot_to_unique  int32 [M*k]: position of inds[t,j] in out_unique_ids;
 *   out_unique_count    int32 [1]:   number of distinct experts (k..M*k).
 * Limits: 1 <= M <= ROUTER_TABLE_MAX_M and M*k <= ROUTER_TABLE_MAX_SLOTS,
 * else ROUTER_ERR_UNSUPPORTED (nothing launched); the rest as router_fwd.
 * inds/weights are bit-identical to router_fwd's on the same inputs; with
 * M = 2 the call is router_fwd_m2_table. */
int router_fwd_route_table(const void* x, const void* w, const float* bias, int M, int H, int E,
                           int k, int scoring, int renorm, int32_t* out_inds, float* out_weights,
                           float* opt_out_logits, int32_t* out_unique_ids,
                           int32_t* out_token_mask, int32_t* out_slot_to_unique,
                           int32_t* out_unique_count, hipStream_t stream);

/* router_fwd with a block-scaled FP4 gate (dense_router_decode commit notes,
 * the fused NVFP4 block-scaled gate GEMM with the router epilogue; here in
 * the OCP MXFP4 encoding that gfx950 converts natively):
 *   w_fp4    uint8 [E, H/2]: FP4 E2M1 codes, element i of a row in byte
 *            i/2, even i in the low nibble (16-byte aligned);
 *   w_scale  uint8 [E, H/32]: E8M0 scales; element i of row e is
 *            e2m1(code) * 2^(w_scale[e, i/32] - 127) (4-byte aligned when
 *            M > ROUTER_DECODE_MAX_M, else ROUTER_ERR_MISALIGNED).
 * Scales must lie in [2, 252], so that every dequantised weight is zero or
 * a normal bf16 value; other scales give unspecified (but finite-time and
 * in-bounds) results.  The logits are then sums of exact bf16 products
 * accumulated in fp32, as router_fwd's are (in this kernel's own order, so
 * not bit-identical to router_fwd on the dequantised gate), and everything
 * after them is the same device routine.
 * Limits: H % 32 == 0, and H % 128 == 0 when M > ROUTER_DECODE_MAX_M (the
 * prefill kernel), else ROUTER_ERR_UNSUPPORTED; the rest as router_fwd.
 * The decode/prefill split is router_fwd's. */
int router_fwd_mxfp4(const void* x, const uint8_t* w_fp4, const uint8_t* w_scale,
                     const float* bias, int64_t M, int H, int E, int k, int scoring, int renorm,
                     int32_t* out_inds, float* out_weights, float* opt_out_logits,
                     hipStream_t stream);

/* router_fwd with a block-scaled FP8 gate: the same low-precision gate
 * projection (dense_router_decode commit notes, block-scaled gate GEMM with
 * the router epilogue) in the OCP MXFP8 encoding, 8-bit elements with the
 * same E8M0 block scale per 32 elements:
 *   w_fp8    uint8 [E, H]: FP8 E4M3 codes (bias 7, no infinities, NaN only
 *            at S.1111.111, largest magnitude 448), one per byte
 *            (16-byte aligned);
 *   w_scale  uint8 [E, H/32]: E8M0 scales; element i of row e is
 *            e4m3(code) * 2^(w_scale[e, i/32] - 127) (4-byte aligned when
 *            M > ROUTER_DECODE_MAX_M, else ROUTER_ERR_MISALIGNED).
 * Scales must lie in [10, 246] and codes must not be NaN, so that every
 * dequantised weight is zero or a normal bf16 value; other inputs give
 * unspecified (but finite-time and in-bounds) results.  The logits are sums
 * of exact bf16 products accumulated in fp32, in this kernel's own order,
 * and everything after them is router_fwd's device routine.
 * Limits as router_fwd_mxfp4: H % 32 == 0, and H % 128 == 0 when
 * M > ROUTER_DECODE_MAX_M, else ROUTER_ERR_UNSUPPORTED. */
int router_fwd_mxfp8(const void* x, const uint8_t* w_fp8, const uint8_t* w_scale,
                     const float* bias, int64_t M, int H, int E, int k, int scoring, int renorm,
                     int32_t* out_inds, float* out_weights, float* opt_out_logits,
                     hipStream_t stream);

/* The step after the router: routed gather fused with the shared-expert
 * add (b70 lab MTP1 M=2 note, "Outcome"), with the note's rounding chain
 * ("Exact arithmetic": FP32 routed accumulation -> BF16 -> add shared BF16
 * -> BF16):
 *   out[t,d] = bf16( bf16(acc) + shared[t,d] ),
 *   acc      = fp32 sum over slots j = 0..k-1 of token t, in order, of
 *              fl32(weights[t,j] * y[r,d]), r = slot_rows[t,j]; the product
 *              and each addition round separately (no fused multiply-add);
 *   bf16()   = round to nearest, ties to even (NaN stays NaN).
 * A slot whose row is -1 (its expert has no local output row) adds
 * nothing; so does a row outside [0, y_rows), which is a caller error the
 * kernel cannot report.  With no row in any slot, out = bf16(0 + shared).
 *   y          bf16 [y_rows, D]  expert output rows (16-byte aligned)
 *   slot_rows  int32 [M, k]      row of y per slot, or -1
 *   weights    fp32 [M, k]       the router's weights (router_fwd's out_weights)
 *   shared     bf16 [M, D]       shared-expert output (16-byte aligned)
 *   out        bf16 [M, D]       may be `shared` (in place); must not overlap y
 * Limits: 1 <= k <= ROUTER_MAX_K, D % 8 == 0, M >= 0 (M == 0 is a no-op).
 * Uses no workspace. */
int router_gather_shared_add(const void* y, int64_t y_rows, const int32_t* slot_rows,
                             const float* weights, const void* shared, int64_t M, int k, int D,
                             void* out, hipStream_t stream);

/* router_gather_shared_add with the rows taken from a unique-route table
 * (router_fwd_route_table's token_mask, slot_to_unique and unique_count,
 * read on the device).  The expert outputs are in the compact layout the
 * table implies (same note, "Why literal source-direct GEMM1 is not
 * funded": each unique expert computes only its tokens' rows): unique
 * experts in table order, each with one row per token of its mask in token
 * order, so slot (t, j) of expert u reads row
 *   sum over unique v < u of popcount(token_mask[v])
 *   + popcount(token_mask[u] & ((1 << t) - 1)).
 * y must hold M*k rows (the most the layout can use).  Limits as
 * router_fwd_route_table (1 <= M <= ROUTER_TABLE_MAX_M, M*k <=
 * ROUTER_TABLE_MAX_SLOTS) and as router_gather_shared_add. */
int router_gather_shared_add_table(const void* y, const int32_t* token_mask,
                                   const int32_t* slot_to_unique, const int32_t* unique_count,
                                   const float* weights, const void* shared, int M, int k, int D,
                                   void* out, hipStream_t stream);

/* Expert GEMM1 consuming the unique-route table (b70 lab MTP1 M=2 note,
 * "Why literal source-direct GEMM1 is not funded": after deduplicating
 * identical (token, expert) routes, each expert has the rows [token0],
 * [token1] or [token0, token1]).  For each unique expert u < unique_count
 * (expert unique_ids[u]) and each token t of token_mask[u]:
 *   out[row, f] = bf16( sum over d of x[t,d] * w1[unique_ids[u], f, d] ),
 * accumulated in fp32 (order of the fp32 sum is the kernel's), rounded once
 * to nearest-even BF16, with row = the compact row router_gather_shared_add_table
 * reads (unique experts in table order, each with its tokens in token order).
 * Each expert's weights are read once per call, however many tokens use it.
 *   x           bf16 [M, D]       token activations (16-byte aligned)
 *   w1          bf16 [E, F, D]    every expert's GEMM1 weights (16-byte aligned)
 *   unique_ids, token_mask, unique_count: router_fwd_route_table's outputs
 *   out         bf16 [M*k, F]     rows past the layout's last are not written
 * A unique id outside [0, E) writes nothing for that expert.
 * Limits: 1 <= M <= ROUTER_TABLE_MAX_M, M*k <= ROUTER_TABLE_MAX_SLOTS,
 * 1 <= k <= ROUTER_MAX_K, D % 8 == 0.  Uses no workspace. */
int router_expert_gemm1_table(const void* x, const void* w1, int E, int64_t F, int D,
                              const int32_t* unique_ids, const int32_t* token_mask,
                              const int32_t* unique_count, int M, int k, void* out,
                              hipStream_t stream);

/* Scoring, selection and weights on logits already in HBM (the standalone
 * logits-to-top-k of the unfused pair; dense_router_decode notes, "Current
 * working path").  One wavefront per row; uses the same device routine as
 * the fused kernels, so fused and unfused results are bit-identical.
 *   logits: fp32 [M, E] device pointer (16-byte aligned rows are read as
 *   vectors when E % 4 == 0, otherwise element by element). */
int router_topk_from_logits(const float* logits, const float* bias, int64_t M, int E, int k,
                            int scoring, int renorm, int32_t* out_inds, float* out_weights,
                            hipStream_t stream);

/* Bounded wait, in microseconds, that a prefill K-split workgroup spends
 * waiting for its sibling splits before it hands its rows to whichever split
 * finishes last (default 200).  Results do not depend on it: both paths sum
 * the same partials in the same order.  0 makes every split that is not the
 * last to arrive hand over at once (used by the tests to exercise that path).
 * Process-wide; applies to calls enqueued after it returns.  Negative values
 * are rejected with ROUTER_ERR_INVALID_ARGUMENT. */
int router_set_exchange_timeout_us(int microseconds);

/* router_fwd for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * one-gate-row-per-workgroup decode kernel, bit-identical results, with its
 * workspace (tagged logit slots, arrival words, a status word: 9,536 bytes)
 * in a statically allocated device array that each GPU holds until the
 * process ends, instead of router_init's workspace.  The call allocates
 * nothing, on the host or the device; router_init (or the first call on a
 * device) resolves that device's copy of the array once.  Every call on a
 * GPU shares its copy: overlapping calls on one device race (order them on
 * one stream).  Limits: 1 <= M <= ROUTER_NOALLOC_MAX_M (M == 0 is a no-op),
 * else ROUTER_ERR_UNSUPPORTED, nothing launched; bf16 gate; the rest as
 * router_fwd.  A row given up at the decode wait limit sets the status bit
 * router_status reports. */
#define ROUTER_NOALLOC_MAX_M 4
int router_fwd_noalloc(const void* x, const void* w, const float* bias, int64_t M, int H, int E, int k,
                       int scoring, int renorm, int32_t* out_inds, float* out_weights,
                       float* opt_out_logits, hipStream_t stream);

/* Bound, in microseconds, on how long a decode finisher (the workgroup that
 * routes the rows) waits for the other workgroups' published logits before
 * it gives a row up (default 100000 = 100 ms; every real wait ends in
 * microseconds).  A row given up comes out as index -1 with a NaN weight in
 * each of its k places, and ROUTER_STATUS_WAIT_LIMIT is set in the device's
 * sticky status word (router_status).  The workspace stays valid: values
 * published after the finisher stopped waiting carry an older launch's tag
 * and are never taken for a later launch's.  0 gives every row up unless its
 * logits are already in place at the first look (used by the tests to
 * exercise that path from the host).  Process-wide; applies to calls
 * enqueued after it returns.  Negative values: ROUTER_ERR_INVALID_ARGUMENT. */
int router_set_decode_wait_limit_us(int microseconds);

/* Sticky status bits of a device's workspaces (all streams' and the
 * allocation-free entry point's, read together). */
#define ROUTER_STATUS_WAIT_LIMIT 1u /* a decode finisher gave a row up */

/* Waits for the device to finish all enqueued work (hipDeviceSynchronize),
 * then reads the device's sticky status bits into *out_flags (0 when the
 * workspace was never allocated); clear != 0 also resets them to 0.
 * device < 0 means the current device.  Synchronising: not for use inside
 * graph capture. */
int router_status(int device, int clear, uint32_t* out_flags);

/* Static, human-readable name of a return code. */
const char* router_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif
