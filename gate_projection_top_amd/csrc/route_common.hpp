// Device-side routing of one row: scoring, selection key, top-k under the
// tie contract, weights, and the M=2 unique-route table.
//
// Every kernel (decode, prefill, standalone top-k) routes a row through
// route_row(), so fused and unfused paths give bit-identical results on
// identical logits (qwisp issue #145, gate G-A: fused vs unfused must agree
// bit for bit, including exact and near ties at the top-8 cut).
//
// Layout contract: one 64-lane wavefront per row, lane L holding the logits of
// experts 4L..4L+3 (E <= 256).  Because lanes are in expert order, the lowest
// lane holding the maximum key also holds the lowest expert index among the
// tied maxima, which is how ties go to the lower index without a 64-bit key.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "softmax_exp.hpp"

namespace gpt {

constexpr int kWave = 64;
constexpr int kMaxE = 256;
constexpr int kMaxK = 16;
constexpr int kPerLane = kMaxE / kWave;  // 4 experts per lane

enum : int { kSoftmax = 0, kSqrtSoftplus = 1 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// cross-lane primitives (full wavefront active)
// ---------------------------------------------------------------------------
// DPP controls: quad_perm [1,0,3,2] = 0xB1, quad_perm [2,3,0,1] = 0x4E,
// row_ror:4 = 0x124, row_ror:8 = 0x128, row_mirror = 0x140 and
// row_half_mirror = 0x141 (each moves data only inside a 16-lane row);
// row_bcast:15 = 0x142 and row_bcast:31 = 0x143 carry a row's value into
// the rows above it.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane)
{
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

__device__ __forceinline__ double readlane_f64(double v, int lane)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = readlane_u32((uint32_t)u, lane);
    const uint32_t hi = readlane_u32((uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = dpp_u32<CTRL>((uint32_t)u);
    const uint32_t hi = dpp_u32<CTRL>((uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// One butterfly step of an unsigned max against the DPP source lane's value;
// the old value 0 (the identity of max) lets the compiler fold the move into
// a single v_max_u32_dpp.
template <int CTRL>
__device__ __forceinline__ uint32_t max_step_u32(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false));
}

// Wave-wide max in a scalar register: the butterfly inside each 16-lane row,
// then DPP row_bcast:15 (rows 1 and 3 take lane 15 of the row below) and
// row_bcast:31 (rows 2 and 3 take lane 31), which leaves the maximum of all
// 64 lanes in lane 63, and one readlane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max_step_u32<0xB1>(v);
    v = max_step_u32<0x4E>(v);
    v = max_step_u32<0x124>(v);
    v = max_step_u32<0x128>(v);
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
    return readlane_u32(v, 63);
}

// Wave-wide max delivered to every lane: the butterfly inside each 16-lane
// row (quad_perm xor 1 and xor 2, row_half_mirror, then row_mirror and
// row_ror:8 into two registers, which both end with the row max), then
// gfx950's permlane16 and permlane32 swaps across rows.  Every lane can then
// compare against the max without a readlane into a scalar register.
__device__ __forceinline__ uint32_t wave_max_all_u32(uint32_t v)
{
    v = max_step_u32<0xB1>(v);
    v = max_step_u32<0x4E>(v);
    v = max_step_u32<0x141>(v);
    const uint32_t a = max_step_u32<0x140>(v);
    const uint32_t b = max_step_u32<0x128>(v);
    const auto p = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    const uint32_t x = max((uint32_t)p[0], (uint32_t)p[1]);
    const auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max((uint32_t)q[0], (uint32_t)q[1]);
}

// Sum over the wavefront in a fixed association: the 16-lane row sums are
// read from lanes 0, 16, 32, 48 and added in that order, so the result is a
// deterministic function of the 64 inputs.
__device__ __forceinline__ double wave_sum_f64(double v)
{
    v = v + dpp_f64<0xB1>(v);
    v = v + dpp_f64<0x4E>(v);
    v = v + dpp_f64<0x124>(v);
    v = v + dpp_f64<0x128>(v);
    const double a = readlane_f64(v, 0), b = readlane_f64(v, 16);
    const double c = readlane_f64(v, 32), d = readlane_f64(v, 48);
    return ((a + b) + c) + d;
}

// ---------------------------------------------------------------------------
// scoring and keys
// ---------------------------------------------------------------------------
// Monotone map from a finite fp32 key to uint32 (larger key -> larger code),
// with -0 folded onto +0.  Code 0 is below every finite key and marks an
// entry that is absent or already selected.  Adding +0 turns -0 into +0
// (round to nearest) and leaves every other finite value unchanged; then a
// negative key has all its bits flipped and a non-negative one its sign bit.
__device__ __forceinline__ uint32_t order_code(float f)
{
    const uint32_t u = __float_as_uint(f + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// Inverse of order_code (a folded -0 comes back as +0).
__device__ __forceinline__ float order_value(uint32_t c)
{
    return __uint_as_float((c & 0x80000000u) ? (c & 0x7FFFFFFFu) : ~c);
}

// sqrt(softplus(l)) with the stable softplus max(l,0) + log1p(exp(-|l|))
// (dense_router_decode notes, "Numerically stable softplus"), in double.
__device__ __forceinline__ double sqrt_softplus(float l)
{
    const double v = (double)l;
    return sqrt(fmax(v, 0.0) + log1p(exp(-fabs(v))));
}

struct RowSpec {
    int E;
    int k;
    int scoring;
    int renorm;
    int has_bias;
};

struct RowResult {
    int idx;    // lane j < k: expert of rank j
    float w;    // lane j < k: its weight
};

// Compare-exchange of two (code, slot) entries so that the first one is the
// earlier in selection order: larger code, or equal code and lower slot.
__device__ __forceinline__ void order_pair(uint32_t& ca, int& ia, uint32_t& cb, int& ib)
{
    const bool swap = cb > ca || (cb == ca && ib < ia);
    const uint32_t c = swap ? cb : ca;
    const int i = swap ? ib : ia;
    cb = swap ? ca : cb;
    ib = swap ? ia : ib;
    ca = c;
    ia = i;
}

// One selection round's pop: the lane whose head equals the round's maximum
// and that no lower lane matches.  mask: the lanes whose head equals it.
__device__ __forceinline__ bool round_pop(uint32_t head, uint32_t top, uint64_t& mask)
{
    const bool eq = head == top;
    mask = __builtin_amdgcn_ballot_w64(eq);
    const uint32_t below =
        __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    return (eq ? below : 1u) == 0u;
}

// After the rounds: rank `lane` went to the lowest lane L of that round's
// mask.  L's pops follow its selection order, so the position of the rank in
// L's list of won ranks (`wins`, rank + 1 in 5-bit fields, pop order) picks
// the slot out of L's selection order (`order`, 2-bit slots).
__device__ __forceinline__ int round_winner(uint64_t my_mask, uint32_t wins, uint32_t order)
{
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t lo = (uint32_t)my_mask, hi = (uint32_t)(my_mask >> 32);
    const int L = lo ? __builtin_ctz(lo) : (hi ? 32 + __builtin_ctz(hi) : 0);
    const uint32_t info = (uint32_t)__builtin_amdgcn_ds_bpermute(L << 2, (int)(wins | (order << 20)));
    const uint32_t want = (uint32_t)lane + 1u;
    uint32_t w = 0u;
#pragma unroll
    for (int q = 1; q < kPerLane; ++q) w = (((info >> (5 * q)) & 31u) == want) ? (uint32_t)q : w;
    return L * kPerLane + (int)((info >> (20 + 2 * w)) & 3u);
}

// Sum of u over lanes 0..k-1 (k <= 16; lanes k.. hold +0) as a fixed tree
// inside the first 16-lane row: partners xor 1, xor 2, then the mirrored
// quad and the mirrored half.  Each step adds the same two values in both
// partner lanes, so every lane of the row ends with the same bits.
__device__ __forceinline__ double rank_sum(double u)
{
    u = u + dpp_f64<0xB1>(u);
    u = u + dpp_f64<0x4E>(u);
    u = u + dpp_f64<0x141>(u);
    return u + dpp_f64<0x140>(u);
}

// Two ways to run the k selection rounds; they give bit-identical results.
//   kRoundsLane: each round's maximum reaches every lane (wave_max_all_u32),
//     the pop is decided with vector instructions only, and the winners'
//     indices are resolved once after the last round.  The shortest chain of
//     dependent steps per round: for a routing wave with a SIMD to itself.
//   kRoundsScalar: the maximum and the winning lane pass through scalar
//     registers (readlane, find-first-set).  Fewer vector instructions per
//     round: for routing waves that share a SIMD.
//   kFilter: no rounds where a threshold leaves between k and kFilterCap
//     candidates (select_filter above): they are ranked by counting; the
//     lane rounds otherwise.  Needs kFilterSlots 8-byte LDS entries per row.
enum RoundStyle : int { kRoundsLane = 0, kRoundsScalar = 1, kFilter = 2 };

template <RoundStyle kStyle>
__device__ __forceinline__ uint32_t max_code(uint32_t v)
{
    if constexpr (kStyle == kRoundsLane)
        return wave_max_all_u32(v);
    else
        return wave_max_u32(v);
}

// Filtered selection of one row (the lane's four codes in any order, their
// slots in `order`, two bits each).
//
// A threshold T below the row maximum is chosen so that at least k and at
// most kFilterCap codes reach it: T = top - D in code space (codes are
// monotone in the key; top is the largest first-slot code, any reference
// below the maximum works), D moved by doubling, halving and bisection, each
// try costing one ballot and population count per code slot.  Every winner
// is at or above T (at least k codes are), so the winners are the first k of
// the candidates under the contract's precedence.  Each candidate goes to
// LDS as one 64-bit word, code above (0xFFFF - expert) below, so that one
// unsigned comparison is that precedence (larger key first, equal keys by
// lower index); a candidate's rank is the number of candidate words above
// its own, and the first k are re-read in rank order.  Lane j < k ends with
// the index and the code of rank j.  Rows where no such T exists within the
// try budget (many equal or nearly equal codes near the top) return false
// and leave the outputs untouched; the caller runs the rounds instead.
// The budget covers biased softmax keys too, whose k-th largest can sit
// several binades below the top when a peaked probability leads a tail that
// the bias spreads (logits of standard deviation 4: up to 9 tries, 6 on
// average, where plain logits need 1-2).
// `lds`: kFilterSlots entries owned by this wave.
constexpr int kFilterCap = 32;
constexpr int kFilterSlots = kFilterCap + 2;  // + a discard slot, rows kept 16-byte aligned
constexpr int kFilterTries = 12;
constexpr int kFilterTriesUnrolled = 6;  // most rows need one to three

// m[j]: the lanes whose code in slot j is at least T (the whole wavefront
// active).  The four compares write four scalar pairs back to back, so none
// waits for the previous one's mask to be read (a compare into VCC would);
// the trailing wait states cover a vector instruction reading the masks.
__device__ __forceinline__ void masks_at_least(const uint32_t (&c)[kPerLane], uint32_t T, uint64_t (&m)[kPerLane])
{
    asm("v_cmp_le_u32_e64 %0, %4, %5\n\t"
        "v_cmp_le_u32_e64 %1, %4, %6\n\t"
        "v_cmp_le_u32_e64 %2, %4, %7\n\t"
        "v_cmp_le_u32_e64 %3, %4, %8\n\t"
        "s_nop 4"
        : "=&s"(m[0]), "=&s"(m[1]), "=&s"(m[2]), "=&s"(m[3])
        : "s"(T), "v"(c[0]), "v"(c[1]), "v"(c[2]), "v"(c[3]));
}

__device__ __forceinline__ int count_masks(const uint64_t (&m)[kPerLane])
{
    return (__builtin_popcountll(m[0]) + __builtin_popcountll(m[1])) +
           (__builtin_popcountll(m[2]) + __builtin_popcountll(m[3]));
}


// The filter's threshold: T = top - D in code space with k <= n <= cap
// codes at or above it (n returned), D moved by doubling, halving and
// bisection; false when no try within the budget finds one.  top: the
// largest code of the row (returned); m: the masks of T (masks_at_least).
// The first tries are unrolled; rows of peaked keys that need more continue
// in a loop.
__device__ __forceinline__ bool filter_threshold(const uint32_t (&c)[kPerLane], int k, uint32_t& T, int& n,
                                                 uint32_t& top, uint64_t (&m)[kPerLane])
{
    top = wave_max_u32(max(max(c[0], c[1]), max(c[2], c[3])));
    // distances in code space: dlo gave fewer than k codes, dhi more than the cap
    uint32_t D = 3u << 21, dlo = 0u, dhi = 0u;
    T = 1u;
    n = 0;
    bool open = true;  // no try has settled the row yet
#pragma unroll
    for (int t = 0; t < kFilterTriesUnrolled; ++t) {
        T = top > D ? top - D : 1u;  // valid codes are >= 1; absent entries are 0
        masks_at_least(c, T, m);
        n = count_masks(m);
        if (n >= k && n <= kFilterCap) return true;
        if (n < k) {
            if (T == 1u) { open = false; break; }  // fewer than k valid codes cannot happen; stop
            dlo = D;
            D = dhi ? dlo + ((dhi - dlo) >> 1) : (D > 0x7fffffffu ? 0xffffffffu : 2u * D);
        } else {
            dhi = D;
            D = dlo + ((dhi - dlo) >> 1);
        }
        if (dhi && dhi - dlo <= 1u) { open = false; break; }  // no threshold separates k..cap codes
    }
    if (open) {
#pragma nounroll
        for (int t = kFilterTriesUnrolled; t < kFilterTries; ++t) {
            T = top > D ? top - D : 1u;
            masks_at_least(c, T, m);
            n = count_masks(m);
            if (n >= k && n <= kFilterCap) return true;
            if (n < k) {
                if (T == 1u) break;
                dlo = D;
                D = dhi ? dlo + ((dhi - dlo) >> 1) : (D > 0x7fffffffu ? 0xffffffffu : 2u * D);
            } else {
                dhi = D;
                D = dlo + ((dhi - dlo) >> 1);
            }
            if (dhi && dhi - dlo <= 1u) break;
        }
    }
    return false;
}

// Rank of each candidate word among the n (k <= n <= kFilterCap) words of
// `table` (entries n .. kFilterCap-1 zero, below every word): the number of
// words above it.  With span = 16 when n <= 16, else 32, lane L holds
// candidate L mod span (`mine`), and the 64/span lanes holding the same
// candidate each compare it with their own slice of the table (4 or 16
// entries, one round of reads), their counts summed across the wave's rows
// with the permlane swaps; every lane ends with its candidate's rank.
// `between(mine)` runs while the reads are in flight (the scheduling
// barriers keep it there).
template <class F>
__device__ __forceinline__ int filter_rank(const uint64_t* table, int n, uint64_t& mine, F&& between)
{
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t part = 0u;
    if (n <= 16) {
        const int p = lane >> 4;
        mine = table[lane & 15];
        uint64_t q[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = table[4 * p + i];
        between(mine);
#pragma unroll
        for (int i = 0; i < 4; ++i) part += q[i] > mine ? 1u : 0u;
        const auto r = __builtin_amdgcn_permlane16_swap(part, part, false, false);  // rows 0+1, 2+3
        part = r[0] + r[1];
    } else {
        const int p = lane >> 5;
        mine = table[lane & 31];
        uint64_t q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = table[16 * p + i];
        between(mine);
#pragma unroll
        for (int i = 0; i < 8; ++i) part += q[i] > mine ? 1u : 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = table[16 * p + 8 + i];
#pragma unroll
        for (int i = 0; i < 8; ++i) part += q[i] > mine ? 1u : 0u;
    }
    const auto h = __builtin_amdgcn_permlane32_swap(part, part, false, false);  // halves 0+1
    return (int)(h[0] + h[1]);
}

// The first k candidates to lanes 0 .. k-1 by rank: lane L < n (which holds
// candidate L, L < span) with rank r < k sends its value to lane r through
// the LDS crossbar (ds_permute, no LDS memory); every other lane sends to
// lane 63, which no rank reaches (k <= 16).
__device__ __forceinline__ uint32_t push_by_rank(int dst, uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_ds_permute(dst << 2, (int)v);
}

__device__ __forceinline__ uint64_t push_by_rank64(int dst, uint64_t v)
{
    const uint32_t lo = push_by_rank(dst, (uint32_t)v), hi = push_by_rank(dst, (uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// kScore (rows with no bias, so that a candidate's key is its logit):
// kSoftmax or kSqrtSoftplus has each candidate's unbiased score computed too,
// exp(l - max l) in double or sqrt(softplus(l)), while the ranking's reads
// are in flight; it travels with the candidate to its rank (my_u; 0 past
// rank k-1), so the winners' scores cost no time after the selection.
// kScore < 0: no scores.
template <int kScore>
__device__ __forceinline__ bool select_filter_impl(const uint32_t (&c)[kPerLane], uint32_t order, int k,
                                                   uint64_t* lds, int& my_idx, uint32_t& my_code, double& my_u,
                                                   const Exp2Lane& et)
{
    constexpr bool kScored = kScore >= 0;
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t T = 1u, top = 0u;
    int n = 0;
    uint64_t m[kPerLane];
    const bool found = filter_threshold(c, k, T, n, top, m);
    if (!found) return false;
    // compaction: lane L's candidates go to [at, ...), at counting the
    // candidates of the lower lanes (from the threshold's masks), in slot
    // order; its other entries go to the discard slot, and lanes n .. cap-1
    // zero the unused tail, so that entries 0 .. cap-1 hold the n candidates
    // and then zeros (below every candidate word).  No write needs a lane mask.
    uint32_t at = 0u;
    bool take[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        take[j] = c[j] >= T;
        at += __builtin_amdgcn_mbcnt_hi((uint32_t)(m[j] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[j], 0u));
    }
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const uint32_t idx = (uint32_t)(lane * kPerLane) + ((order >> (2 * j)) & 3u);
        lds[take[j] ? at : (uint32_t)kFilterCap] = ((uint64_t)c[j] << 32) | (0xFFFFu - idx);
        at += take[j] ? 1u : 0u;
    }
    lds[(lane >= n && lane < kFilterCap) ? lane : kFilterCap] = 0ull;
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    double u = 0.0;
    uint64_t mine = 0ull;
    const int rank = filter_rank(lds, n, mine, [&](uint64_t w) {
        if constexpr (kScored) {
            __builtin_amdgcn_sched_barrier(0);
            const float l = order_value((uint32_t)(w >> 32));
            if constexpr (kScore == kSoftmax)
                u = softmax_exp((double)l - (double)order_value(top), et);
            else
                u = sqrt_softplus(l);
            asm volatile("" ::"v"(u));  // computed here, not where it is used
            __builtin_amdgcn_sched_barrier(0);
        }
    });
    const int dst = (lane < n && rank < k) ? rank : kWave - 1;
    const uint64_t got = push_by_rank64(dst, mine);
    if constexpr (kScored) {
        const uint64_t ub = push_by_rank64(dst, __builtin_bit_cast(uint64_t, u));
        my_u = lane < k ? __builtin_bit_cast(double, ub) : 0.0;
    }
    my_code = lane < k ? (uint32_t)(got >> 32) : 0u;
    my_idx = lane < k ? (int)(0xFFFFu - (uint32_t)got) : 0;
    // the table is rewritten by the next selection on this wave's entries:
    // LDS operations of one wave complete in order
    return true;
}

__device__ __forceinline__ bool select_filter(const uint32_t (&c)[kPerLane], uint32_t order, int k,
                                              uint64_t* lds, int& my_idx, uint32_t& my_code)
{
    double unused = 0.0;
    return select_filter_impl<-1>(c, order, k, lds, my_idx, my_code, unused, Exp2Lane{0.0, 0.0});
}

// Sqrt-softplus scores with a bias, decided with as little double precision
// as the result allows.  Every key fl32(fl32(s) + b) is first bracketed from
// an fp32 evaluation of s (hardware exp, log and square root; a series for
// log1p of small arguments), whose relative error stays below 2^-17 for
// |logit| <= 40, bracketed at 2^-13, plus one code of slack each way.  A
// threshold T on the lower ends with at least k of them at or above it (the
// filter's search) makes T a lower bound on the k-th largest exact key, so
// only experts whose upper end reaches T can win.  Those candidates (at most
// kFilterCap, one per lane after compaction) get their exact double score
// and key, exactly as the all-double path computes them, and are ranked by
// the filter's counting; lane j < k ends with the winner of rank j, its code
// and its double score.  Results are bit-identical to the all-double path.
// Returns false (outputs untouched) for rows with a logit beyond +-40 or too
// many candidates; the caller then scores every expert in double.
// `lds`: kRefineSlots 8-byte entries owned by this wave.
constexpr int kRefineSlots = 3 * kFilterSlots;

__device__ __forceinline__ bool select_refined_softplus(const float (&v)[kPerLane], const float (&bv)[kPerLane],
                                                        const bool (&valid)[kPerLane], int k, uint64_t* lds,
                                                        int& my_idx, uint32_t& my_code, double& my_u)
{
    const int lane = threadIdx.x & (kWave - 1);
    bool far = false;
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) far |= valid[j] && !(fabsf(v[j]) <= 40.0f);
    if (__builtin_amdgcn_ballot_w64(far) != 0) return false;
    uint32_t clo[kPerLane], chi[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const float l = v[j];
        const float a = __expf(-fabsf(l));
        // log1p(a): a - a^2/2 + a^3/3 - a^4/4 below 1/32 (truncation < a^5/5),
        // log(1 + a) above
        const float lp = a < 0.03125f ? a * (1.0f - a * (0.5f - a * (0.33333334f - a * 0.25f))) : __logf(1.0f + a);
        const float sq = sqrtf(fmaxf(l, 0.0f) + lp);
        const uint32_t lo = order_code(sq * (1.0f - 0x1p-13f) + bv[j]);
        const uint32_t hi = order_code(sq * (1.0f + 0x1p-13f) + bv[j]);
        clo[j] = valid[j] ? (lo > 1u ? lo - 1u : 1u) : 0u;
        chi[j] = valid[j] ? hi + 1u : 0u;
    }
    uint32_t T = 1u, top = 0u;
    int n = 0;
    uint64_t mlo[kPerLane];
    if (!filter_threshold(clo, k, T, n, top, mlo)) return false;
    uint64_t m[kPerLane];
    masks_at_least(chi, T, m);
    const int nc = count_masks(m);
    if (nc > kFilterCap) return false;

    uint64_t* cand = lds;                      // (logit bits, bias bits) of candidate i
    uint64_t* cidx = lds + kFilterSlots;       // its expert index
    uint64_t* table = lds + 2 * kFilterSlots;  // ranking words
    uint32_t at = 0u;
    bool take[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        take[j] = chi[j] >= T;
        at += __builtin_amdgcn_mbcnt_hi((uint32_t)(m[j] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m[j], 0u));
    }
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        const uint32_t pos = take[j] ? at : (uint32_t)kFilterCap;
        cand[pos] = ((uint64_t)__float_as_uint(v[j]) << 32) | __float_as_uint(bv[j]);
        cidx[pos] = (uint64_t)(lane * kPerLane + j);
        at += take[j] ? 1u : 0u;
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    uint64_t word = 0ull;
    double u = 0.0;
    if (lane < nc) {
        const uint64_t e = cand[lane];
        const uint32_t id = (uint32_t)cidx[lane];
        u = sqrt_softplus(__uint_as_float((uint32_t)(e >> 32)));
        const float key = (float)u + __uint_as_float((uint32_t)e);
        word = ((uint64_t)order_code(key) << 32) | (0xFFFFu - id);
    }
    table[(lane < kFilterCap) ? lane : kFilterCap] = word;  // zeros past the candidates
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    // lane j < nc holds candidate j and its score (nc <= the ranking's span)
    uint64_t mine = 0ull;
    const int rank = filter_rank(table, nc, mine, [](uint64_t) {});
    const int dst = (lane < nc && rank < k) ? rank : kWave - 1;
    const uint64_t got = push_by_rank64(dst, mine);
    const uint64_t ub = push_by_rank64(dst, __builtin_bit_cast(uint64_t, u));
    my_u = lane < k ? __builtin_bit_cast(double, ub) : 0.0;
    my_code = lane < k ? (uint32_t)(got >> 32) : 0u;
    my_idx = lane < k ? (int)(0xFFFFu - (uint32_t)got) : 0;
    return true;
}

// k rounds over N rows: the wave-wide largest head wins; among equal heads
// the lowest lane, whose head is its lowest-slot entry of that code, i.e. the
// lowest expert index.  The winning lane pops its head.  c[n]: the lane's
// four codes in selection order; order[n]: their slots, two bits each, head
// in the low bits.  Lane j < k ends with the index and code of rank j.
template <int N, RoundStyle kStyle>
__device__ __forceinline__ void select_rounds(uint32_t (&c)[N][kPerLane], const uint32_t (&order)[N],
                                              int k, int (&my_idx)[N], uint32_t (&my_code)[N],
                                              uint64_t* lds)
{
    const int lane = threadIdx.x & (kWave - 1);
    static_assert(kStyle != kFilter, "the filter is tried by the callers; select_rounds runs the rounds");
    if constexpr (kStyle == kRoundsLane) {
        // lane `it` keeps round it's mask; each lane lists the ranks it won
        uint64_t my_mask[N];
        uint32_t wins[N], wshift[N];
#pragma unroll
        for (int n = 0; n < N; ++n) {
            my_mask[n] = 0u;
            my_code[n] = 0u;
            wins[n] = 0u;
            wshift[n] = 0u;
        }
        for (int it = 0; it < k; ++it) {
            uint32_t top[N];
#pragma unroll
            for (int n = 0; n < N; ++n) top[n] = wave_max_all_u32(c[n][0]);
#pragma unroll
            for (int n = 0; n < N; ++n) {
                uint64_t m;
                const bool pop = round_pop(c[n][0], top[n], m);
                c[n][0] = pop ? c[n][1] : c[n][0];
                c[n][1] = pop ? c[n][2] : c[n][1];
                c[n][2] = pop ? c[n][3] : c[n][2];
                c[n][3] = pop ? 0u : c[n][3];
                wins[n] = pop ? wins[n] | ((uint32_t)(it + 1) << wshift[n]) : wins[n];
                wshift[n] = pop ? wshift[n] + 5u : wshift[n];
                if (lane == it) {
                    my_mask[n] = m;
                    my_code[n] = top[n];
                }
            }
        }
#pragma unroll
        for (int n = 0; n < N; ++n) my_idx[n] = round_winner(my_mask[n], wins[n], order[n]);
    } else {
        uint32_t slots[N];
#pragma unroll
        for (int n = 0; n < N; ++n) {
            slots[n] = order[n];
            my_idx[n] = 0;
            my_code[n] = 0u;
        }
        for (int it = 0; it < k; ++it) {
            uint32_t top[N];
#pragma unroll
            for (int n = 0; n < N; ++n) top[n] = wave_max_u32(c[n][0]);
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const uint64_t hit = __builtin_amdgcn_ballot_w64(c[n][0] == top[n]);
                const int L = (int)__builtin_ctzll(hit);
                const int wslot = (int)(readlane_u32(slots[n], L) & 3u);
                if (lane == it) {
                    my_idx[n] = L * kPerLane + wslot;
                    my_code[n] = top[n];
                }
                const bool pop = lane == L;
                c[n][0] = pop ? c[n][1] : c[n][0];
                c[n][1] = pop ? c[n][2] : c[n][1];
                c[n][2] = pop ? c[n][3] : c[n][2];
                c[n][3] = pop ? 0u : c[n][3];
                slots[n] = pop ? slots[n] >> 2 : slots[n];
            }
        }
    }
}

// Route one row.  v[j]: logit of expert 4*lane+j (ignored when >= E);
// bv[j]: its selection bias (used only when s.has_bias).
// Routes N rows at once, in lockstep: every step below runs for each row in
// turn, so the N rows' dependency chains (DPP reductions, readlanes, f64
// arithmetic) interleave and a wave issues instructions while one row waits.
// kNeedAll: scores for every expert are needed (they form the key, or a
// softmax weight is the full-row probability); the two cases compile apart.
template <int N, bool kNeedAll, RoundStyle kStyle>
__device__ __forceinline__ void route_rows_impl(const float (&v)[N][kPerLane],
                                                const float (&bv)[kPerLane], const RowSpec& s,
                                                RowResult (&out)[N], uint64_t* lds, const Exp2Lane& et)
{
    const int lane = threadIdx.x & (kWave - 1);
    bool valid[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) valid[j] = (lane * kPerLane + j) < s.E;

    const bool softmax = s.scoring == kSoftmax;
    constexpr bool need_all = kNeedAll;

    float mx[N];                 // softmax shift: the row's largest logit
    double Z[N];
    double sc[N][kPerLane];      // scores: the key's first term
    double un[N][kPerLane];      // unbiased scores: the weights' terms
#pragma unroll
    for (int n = 0; n < N; ++n) {
        mx[n] = 0.0f;
        Z[n] = 1.0;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) sc[n][j] = un[n][j] = 0.0;
    }
    if constexpr (need_all) {
        if (softmax) {
            // the row max through order codes (a max of -0 comes back as
            // +0, which shifts every exponent by exactly the same zero)
            uint32_t m[N];
#pragma unroll
            for (int n = 0; n < N; ++n) {
                m[n] = 0u;
#pragma unroll
                for (int j = 0; j < kPerLane; ++j)
                    if (valid[j]) m[n] = max(m[n], order_code(v[n][j]));
            }
#pragma unroll
            for (int n = 0; n < N; ++n) mx[n] = order_value(max_code<kStyle>(m[n]));
#pragma unroll
            for (int n = 0; n < N; ++n)
#pragma unroll
                for (int j = 0; j < kPerLane; ++j) {
                    const double e = softmax_exp((double)v[n][j] - (double)mx[n], et);  // whole wave
                    un[n][j] = valid[j] ? e : 0.0;
                }
#pragma unroll
            for (int n = 0; n < N; ++n)
                Z[n] = wave_sum_f64(((un[n][0] + un[n][1]) + un[n][2]) + un[n][3]);
            // z * (1/Z): within an ulp of z / Z in double, so its rounding
            // to fp32 (all the key keeps) agrees but for ~1e-8 of values
#pragma unroll
            for (int n = 0; n < N; ++n) {
                const double rZ = 1.0 / Z[n];
#pragma unroll
                for (int j = 0; j < kPerLane; ++j) sc[n][j] = un[n][j] * rZ;
            }
        } else {
#pragma unroll
            for (int n = 0; n < N; ++n)
#pragma unroll
                for (int j = 0; j < kPerLane; ++j) {
                    sc[n][j] = valid[j] ? sqrt_softplus(v[n][j]) : 0.0;
                    un[n][j] = sc[n][j];
                }
        }
    }

    // Selection codes (lane-local order: the filter needs none, the rounds
    // sort each lane's four entries first).
    uint32_t c[N][kPerLane];
#pragma unroll
    for (int n = 0; n < N; ++n) {
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            float key = v[n][j];
            if (s.has_bias) {
                const float s32 = (float)sc[n][j];
                key = s32 + bv[j];
            }
            c[n][j] = valid[j] ? order_code(key) : 0u;
        }
    }
    int my_idx[N];
    uint32_t my_code[N];
    bool selected = false;
    if constexpr (kStyle == kFilter) {
        selected = true;
#pragma unroll
        for (int n = 0; n < N; ++n)
            selected &= select_filter(c[n], 0xE4u, s.k, lds + n * kFilterSlots, my_idx[n], my_code[n]);
    }
    if (!selected) {
        uint32_t slots[N];  // the four slots in selection order, two bits each, head lowest
#pragma unroll
        for (int n = 0; n < N; ++n) {
            int slot[kPerLane] = {0, 1, 2, 3};
            order_pair(c[n][0], slot[0], c[n][1], slot[1]);
            order_pair(c[n][2], slot[2], c[n][3], slot[3]);
            order_pair(c[n][0], slot[0], c[n][2], slot[2]);
            order_pair(c[n][1], slot[1], c[n][3], slot[3]);
            order_pair(c[n][1], slot[1], c[n][2], slot[2]);
            slots[n] = (uint32_t)slot[0] | ((uint32_t)slot[1] << 2) | ((uint32_t)slot[2] << 4) |
                       ((uint32_t)slot[3] << 6);
        }
        constexpr RoundStyle kRounds = kStyle == kFilter ? kRoundsScalar : kStyle;
        select_rounds<N, kRounds>(c, slots, s.k, my_idx, my_code, lds);
    }

    // The winners' unbiased scores.  When every score was computed above,
    // fetch the winner's from the lane that holds it; otherwise compute it
    // from the winner's logit (the key itself, since there is no bias).
    double u[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        u[n] = 0.0;
        if constexpr (need_all) {
            const int src = (my_idx[n] >> 2) << 2;  // byte address of the owning lane
            const int j = my_idx[n] & 3;
            double got[kPerLane];
#pragma unroll
            for (int q = 0; q < kPerLane; ++q) {
                const uint64_t bits = __builtin_bit_cast(uint64_t, un[n][q]);
                const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)bits);
                const uint32_t hi =
                    (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(bits >> 32));
                got[q] = __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
            }
            u[n] = j == 0 ? got[0] : (j == 1 ? got[1] : (j == 2 ? got[2] : got[3]));
            if (lane >= s.k) u[n] = 0.0;
        } else {
            const float my_logit = order_value(my_code[n]);
            if (softmax) {
                mx[n] = order_value(readlane_u32(my_code[n], 0));  // rank 0 holds the max
                const double e = softmax_exp((double)my_logit - (double)mx[n], et);  // whole wave
                u[n] = lane < s.k ? e : 0.0;
            } else if (lane < s.k) {
                u[n] = sqrt_softplus(my_logit);
            }
        }
    }
    // The bias never enters the weights.
#pragma unroll
    for (int n = 0; n < N; ++n) {
        float w;
        if (s.renorm) {
            w = (float)(u[n] / rank_sum(u[n]));
        } else {
            w = softmax ? (float)(u[n] / Z[n]) : (float)u[n];
        }
        out[n] = RowResult{my_idx[n], w};
    }
}

// N rows in lockstep (same spec); rows n carry logits v[n] and get out[n].
// lds: N * kFilterSlots entries owned by this wave (kFilter only); et: the
// wave's exp table (load_exp2_lane).
template <int N, RoundStyle kStyle = kRoundsScalar>
__device__ __forceinline__ void route_rows(const float (&v)[N][kPerLane], const float (&bv)[kPerLane],
                                           const RowSpec& s, RowResult (&out)[N], uint64_t* lds,
                                           const Exp2Lane& et)
{
    const bool need_all = s.has_bias || (s.scoring == kSoftmax && !s.renorm);
    if (need_all)
        route_rows_impl<N, true, kStyle>(v, bv, s, out, lds, et);
    else
        route_rows_impl<N, false, kStyle>(v, bv, s, out, lds, et);
}

// One row: the same steps as route_rows, written for a single row (the
// generic form costs the single-row decode path ~0.3 us of latency).  The
// two give bit-identical results on identical inputs.  Without a bias the
// filter also scores its candidates (select_filter_impl<true>), which takes
// the winners' scores off the end of the routing.
template <bool kNeedAll, RoundStyle kStyle>
__device__ __forceinline__ RowResult route_row_impl(const float (&v)[kPerLane],
                                                    const float (&bv)[kPerLane], const RowSpec& s,
                                                    uint64_t* lds, const Exp2Lane& et)
{
    const int lane = threadIdx.x & (kWave - 1);
    bool valid[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) valid[j] = (lane * kPerLane + j) < s.E;

    const bool softmax = s.scoring == kSoftmax;
    constexpr bool need_all = kNeedAll;

    if constexpr (need_all && kStyle == kFilter) {
        // sqrt-softplus with a bias: exact keys only where they can decide
        if (!softmax) {
            int ridx = 0;
            uint32_t rcode = 0u;
            double ru = 0.0;
            if (select_refined_softplus(v, bv, valid, s.k, lds, ridx, rcode, ru)) {
                const float w = s.renorm ? (float)(ru / rank_sum(ru)) : (float)ru;
                return RowResult{ridx, w};
            }
        }
    }

    float mx = 0.0f;  // softmax shift: the row's largest logit
    double Z = 1.0;
    double sc[kPerLane] = {0.0, 0.0, 0.0, 0.0};  // scores: the key's first term
    double un[kPerLane] = {0.0, 0.0, 0.0, 0.0};  // unbiased scores: the weights' terms
    if constexpr (need_all) {
        if (softmax) {
            // the row max through order codes (a max of -0 comes back as
            // +0, which shifts every exponent by exactly the same zero)
            uint32_t m = 0u;
#pragma unroll
            for (int j = 0; j < kPerLane; ++j)
                if (valid[j]) m = max(m, order_code(v[j]));
            mx = order_value(max_code<kStyle>(m));
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) {
                const double e = softmax_exp((double)v[j] - (double)mx, et);  // whole wave
                un[j] = valid[j] ? e : 0.0;
            }
            Z = wave_sum_f64(((un[0] + un[1]) + un[2]) + un[3]);
            // z * (1/Z): within an ulp of z / Z in double, so its rounding
            // to fp32 (all the key keeps) agrees but for ~1e-8 of values
            const double rZ = 1.0 / Z;
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) sc[j] = un[j] * rZ;
        } else {
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) sc[j] = valid[j] ? sqrt_softplus(v[j]) : 0.0;
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) un[j] = sc[j];
        }
    }

    // Selection codes, then each lane's four entries in selection order.
    uint32_t c[kPerLane];
    int slot[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) {
        float key = v[j];
        if (s.has_bias) {
            const float s32 = (float)sc[j];
            key = s32 + bv[j];
        }
        c[j] = valid[j] ? order_code(key) : 0u;
        slot[j] = j;
    }
    int my_idx = 0;
    uint32_t my_code = 0u;
    // the filter needs no order inside a lane (its words carry the index);
    // the lane's entries are sorted only for the rounds
    bool selected = false;
    if constexpr (kStyle == kFilter) {
        double su = 0.0;  // the winner's unbiased score, when the filter scored its candidates
        if constexpr (need_all) {
            selected = select_filter_impl<-1>(c, 0xE4u, s.k, lds, my_idx, my_code, su, et);
        } else {
            // no bias: softmax with renorm, or sqrt-softplus
            selected = softmax ? select_filter_impl<kSoftmax>(c, 0xE4u, s.k, lds, my_idx, my_code, su, et)
                               : select_filter_impl<kSqrtSoftplus>(c, 0xE4u, s.k, lds, my_idx, my_code, su, et);
            if (selected) return RowResult{my_idx, s.renorm ? (float)(su / rank_sum(su)) : (float)su};
        }
    }
    if (!selected) {
        order_pair(c[0], slot[0], c[1], slot[1]);
        order_pair(c[2], slot[2], c[3], slot[3]);
        order_pair(c[0], slot[0], c[2], slot[2]);
        order_pair(c[1], slot[1], c[3], slot[3]);
        order_pair(c[1], slot[1], c[2], slot[2]);
        // the four slots in selection order, two bits each, head in the low bits
        uint32_t slots = (uint32_t)slot[0] | ((uint32_t)slot[1] << 2) | ((uint32_t)slot[2] << 4) |
                         ((uint32_t)slot[3] << 6);
        uint32_t cc[1][kPerLane] = {{c[0], c[1], c[2], c[3]}};
        const uint32_t ord[1] = {slots};
        int idx1[1];
        uint32_t code1[1];
        constexpr RoundStyle kRounds = kStyle == kFilter ? kRoundsLane : kStyle;
        select_rounds<1, kRounds>(cc, ord, s.k, idx1, code1, lds);
        my_idx = idx1[0];
        my_code = code1[0];
    }

    // The winners' unbiased scores.  When every score was computed above,
    // fetch the winner's from the lane that holds it; otherwise compute it
    // from the winner's logit (the key itself, since there is no bias).
    double u = 0.0;
    if constexpr (need_all) {
        const int src = (my_idx >> 2) << 2;  // byte address of the owning lane
        const int j = my_idx & 3;
        double got[kPerLane];
#pragma unroll
        for (int q = 0; q < kPerLane; ++q) {
            const uint64_t bits = __builtin_bit_cast(uint64_t, un[q]);
            const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)bits);
            const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)(uint32_t)(bits >> 32));
            got[q] = __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
        }
        u = j == 0 ? got[0] : (j == 1 ? got[1] : (j == 2 ? got[2] : got[3]));
        if (lane >= s.k) u = 0.0;
    } else {
        const float my_logit = order_value(my_code);
        if (softmax) {
            mx = order_value(readlane_u32(my_code, 0));  // rank 0 holds the max
            const double e = softmax_exp((double)my_logit - (double)mx, et);  // whole wave
            u = lane < s.k ? e : 0.0;
        } else if (lane < s.k) {
            u = sqrt_softplus(my_logit);
        }
    }
    // The bias never enters the weights.
    float w;
    if (s.renorm) {
        w = (float)(u / rank_sum(u));
    } else {
        w = softmax ? (float)(u / Z) : (float)u;
    }
    return RowResult{my_idx, w};
}

// lds: kRefineSlots entries owned by this wave (kFilter only); et: the
// wave's exp table (load_exp2_lane).
template <RoundStyle kStyle = kRoundsLane>
__device__ __forceinline__ RowResult route_row(const float (&v)[kPerLane],
                                               const float (&bv)[kPerLane], const RowSpec& s,
                                               uint64_t* lds, const Exp2Lane& et)
{
    const bool need_all = s.has_bias || (s.scoring == kSoftmax && !s.renorm);
    return need_all ? route_row_impl<true, kStyle>(v, bv, s, lds, et)
                    : route_row_impl<false, kStyle>(v, bv, s, lds, et);
}

// ---------------------------------------------------------------------------
// unique-route table (b70 lab MTP1 note, "Unique-route router screen", for
// the MTP1 pair; qwisp issue #145, "Observation", for the other verify widths)
// ---------------------------------------------------------------------------
// One wavefront; slot s = t*k + j holds inds[t][j] for M tokens (M*k <= 64
// slots).  Per expert, two LDS cells (first_of, mask_of: kMaxE + 1 entries
// each, the last one shared by any id outside 0..kMaxE-1) collect, with LDS
// min and or atomics, the expert's first slot and its token mask (bit t =
// token t); the first appearances, ranked by a prefix count over a ballot,
// give the unique list in encounter order.
__device__ __forceinline__ void emit_route_table(const int32_t* slot_ids, int M, int k,
                                                 int32_t* first_of, int32_t* mask_of,
                                                 int32_t* ids, int32_t* mask,
                                                 int32_t* slot_to_unique, int32_t* count)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int n = M * k;
    const bool active = lane < n;
    const int id = active ? slot_ids[lane] : 0;
    const int cell = (id >= 0 && id < kMaxE) ? id : kMaxE;
    if (active) {
        first_of[cell] = kWave;
        mask_of[cell] = 0;
    }
    if (active) {
        __hip_atomic_fetch_min(&first_of[cell], lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_or(&mask_of[cell], 1 << (lane / k), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    const int first = active ? __hip_atomic_load(&first_of[cell], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_WORKGROUP)
                             : -1;
    const uint64_t firsts = __builtin_amdgcn_ballot_w64(active && first == lane);
    const int unique = __builtin_popcountll(firsts);
    const int rank = active ? __builtin_popcountll(firsts & ((1ull << first) - 1ull)) : 0;

    if (active) {
        slot_to_unique[lane] = rank;
        if (first == lane) {
            ids[rank] = id;
            mask[rank] = __hip_atomic_load(&mask_of[cell], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (lane >= unique) {
            ids[lane] = -1;
            mask[lane] = 0;
        }
    }
    if (lane == 0) count[0] = unique;
}

// 16-byte load of 8 bf16 values.
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p)
{
    return *reinterpret_cast<const bf16x8*>(p);
}

// Eight E2M1 codes (one dword, element 0 in the low nibble of byte 0) times a
// power-of-two scale, as eight bf16 values: gfx950's scaled fp4 -> bf16
// conversion, two elements per instruction.  Exact for the contract's scales.
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t codes, float scale)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Eight FP8 E4M3 codes (two dwords, element 0 in the low byte of lo) times a
// power-of-two scale, as eight bf16 values: gfx950's scaled fp8 -> bf16
// conversion, two elements (one 16-bit word) per instruction.  Exact for
// the contract's scales (E4M3 has four significant bits).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi, float scale)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

}  // namespace gpt
