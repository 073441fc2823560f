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
// row_ror:4 = 0x124, row_ror:8 = 0x128 (after these four steps every lane
// holds the reduction over its 16-lane row), row_bcast:15 = 0x142 and
// row_bcast:31 = 0x143 (carry a row's result into the rows above it).
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

// One butterfly step of an unsigned max: the DPP source lane's value, with 0
// (the identity of max) where the pattern leaves a lane unwritten, so the
// compiler folds the move into a single v_max_u32_dpp.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t max_step_u32(uint32_t v)
{
    return max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false));
}

// Wave-wide max: butterfly inside each 16-lane row, then DPP row_bcast:15
// (rows 1 and 3 take lane 15 of the row below) and row_bcast:31 (rows 2 and 3
// take lane 31), which leaves the maximum of all 64 lanes in lane 63; one
// readlane makes it wave-uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max_step_u32<0xB1>(v);
    v = max_step_u32<0x4E>(v);
    v = max_step_u32<0x124>(v);
    v = max_step_u32<0x128>(v);
    v = max_step_u32<0x142, 0xA>(v);
    v = max_step_u32<0x143, 0xC>(v);
    return readlane_u32(v, 63);
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
// entry that is absent or already selected.
__device__ __forceinline__ uint32_t order_code(float f)
{
    uint32_t u = __float_as_uint(f);
    u = (f == 0.0f) ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
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

// Route one row.  v[j]: logit of expert 4*lane+j (ignored when >= E);
// bv[j]: its selection bias (used only when s.has_bias).
// Routes N rows at once, in lockstep: every step below runs for each row in
// turn, so the N rows' dependency chains (DPP reductions, readlanes, f64
// arithmetic) interleave and a wave issues instructions while one row waits.
// kNeedAll: scores for every expert are needed (they form the key, or a
// softmax weight is the full-row probability); the two cases compile apart.
template <int N, bool kNeedAll>
__device__ __forceinline__ void route_rows_impl(const float (&v)[N][kPerLane],
                                                const float (&bv)[kPerLane], const RowSpec& s,
                                                RowResult (&out)[N])
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
            for (int n = 0; n < N; ++n) mx[n] = order_value(wave_max_u32(m[n]));
#pragma unroll
            for (int n = 0; n < N; ++n)
#pragma unroll
                for (int j = 0; j < kPerLane; ++j)
                    un[n][j] = valid[j] ? exp((double)v[n][j] - (double)mx[n]) : 0.0;
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

    // Selection codes, then each lane's four entries in selection order.
    uint32_t c[N][kPerLane];
    uint32_t slots[N];  // the four slots in selection order, two bits each, head lowest
#pragma unroll
    for (int n = 0; n < N; ++n) {
        int slot[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            float key = v[n][j];
            if (s.has_bias) {
                const float s32 = (float)sc[n][j];
                key = s32 + bv[j];
            }
            c[n][j] = valid[j] ? order_code(key) : 0u;
            slot[j] = j;
        }
        order_pair(c[n][0], slot[0], c[n][1], slot[1]);
        order_pair(c[n][2], slot[2], c[n][3], slot[3]);
        order_pair(c[n][0], slot[0], c[n][2], slot[2]);
        order_pair(c[n][1], slot[1], c[n][3], slot[3]);
        order_pair(c[n][1], slot[1], c[n][2], slot[2]);
        slots[n] = (uint32_t)slot[0] | ((uint32_t)slot[1] << 2) | ((uint32_t)slot[2] << 4) |
                   ((uint32_t)slot[3] << 6);
    }

    // k rounds: the wave-wide largest head wins; among equal heads the lowest
    // lane, whose head is its lowest-slot entry of that code, i.e. the lowest
    // expert index.  The winning lane pops its head.
    int my_idx[N];
    uint32_t my_code[N];
#pragma unroll
    for (int n = 0; n < N; ++n) {
        my_idx[n] = 0;
        my_code[n] = 0u;
    }
    for (int it = 0; it < s.k; ++it) {
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
            if (softmax) mx[n] = order_value(readlane_u32(my_code[n], 0));  // rank 0 holds the max
            if (lane < s.k) {
                const float my_logit = order_value(my_code[n]);
                u[n] = softmax ? exp((double)my_logit - (double)mx[n]) : sqrt_softplus(my_logit);
            }
        }
    }
    // The bias never enters the weights.
#pragma unroll
    for (int n = 0; n < N; ++n) {
        float w;
        if (s.renorm) {
            double total = 0.0;
            for (int j = 0; j < s.k; ++j) total += readlane_f64(u[n], j);
            w = (float)(u[n] / total);
        } else {
            w = softmax ? (float)(u[n] / Z[n]) : (float)u[n];
        }
        out[n] = RowResult{my_idx[n], w};
    }
}

// N rows in lockstep (same spec); rows n carry logits v[n] and get out[n].
template <int N>
__device__ __forceinline__ void route_rows(const float (&v)[N][kPerLane], const float (&bv)[kPerLane],
                                           const RowSpec& s, RowResult (&out)[N])
{
    const bool need_all = s.has_bias || (s.scoring == kSoftmax && !s.renorm);
    if (need_all)
        route_rows_impl<N, true>(v, bv, s, out);
    else
        route_rows_impl<N, false>(v, bv, s, out);
}

// One row: the same steps as route_rows, written for a single row (the
// generic form costs the single-row decode path ~0.3 us of latency).  The
// two give bit-identical results on identical inputs.
template <bool kNeedAll>
__device__ __forceinline__ RowResult route_row_impl(const float (&v)[kPerLane],
                                                    const float (&bv)[kPerLane], const RowSpec& s)
{
    const int lane = threadIdx.x & (kWave - 1);
    bool valid[kPerLane];
#pragma unroll
    for (int j = 0; j < kPerLane; ++j) valid[j] = (lane * kPerLane + j) < s.E;

    const bool softmax = s.scoring == kSoftmax;
    constexpr bool need_all = kNeedAll;

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
            mx = order_value(wave_max_u32(m));
#pragma unroll
            for (int j = 0; j < kPerLane; ++j)
                un[j] = valid[j] ? exp((double)v[j] - (double)mx) : 0.0;
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
    order_pair(c[0], slot[0], c[1], slot[1]);
    order_pair(c[2], slot[2], c[3], slot[3]);
    order_pair(c[0], slot[0], c[2], slot[2]);
    order_pair(c[1], slot[1], c[3], slot[3]);
    order_pair(c[1], slot[1], c[2], slot[2]);
    // the four slots in selection order, two bits each, head in the low bits
    uint32_t slots = (uint32_t)slot[0] | ((uint32_t)slot[1] << 2) | ((uint32_t)slot[2] << 4) |
                     ((uint32_t)slot[3] << 6);

    // k rounds: the wave-wide largest head wins; among equal heads the lowest
    // lane, whose head is its lowest-slot entry of that code, i.e. the lowest
    // expert index.  The winning lane pops its head.
    int my_idx = 0;
    uint32_t my_code = 0u;
    for (int it = 0; it < s.k; ++it) {
        const uint32_t top = wave_max_u32(c[0]);
        const uint64_t hit = __builtin_amdgcn_ballot_w64(c[0] == top);
        const int L = (int)__builtin_ctzll(hit);
        const int wslot = (int)(readlane_u32(slots, L) & 3u);
        if (lane == it) {
            my_idx = L * kPerLane + wslot;
            my_code = top;
        }
        const bool pop = lane == L;
        c[0] = pop ? c[1] : c[0];
        c[1] = pop ? c[2] : c[1];
        c[2] = pop ? c[3] : c[2];
        c[3] = pop ? 0u : c[3];
        slots = pop ? slots >> 2 : slots;
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
        if (softmax) mx = order_value(readlane_u32(my_code, 0));  // rank 0 holds the max
        if (lane < s.k) {
            const float my_logit = order_value(my_code);
            u = softmax ? exp((double)my_logit - (double)mx) : sqrt_softplus(my_logit);
        }
    }
    // The bias never enters the weights.
    float w;
    if (s.renorm) {
        double total = 0.0;
        for (int j = 0; j < s.k; ++j) total += readlane_f64(u, j);
        w = (float)(u / total);
    } else {
        w = softmax ? (float)(u / Z) : (float)u;
    }
    return RowResult{my_idx, w};
}

__device__ __forceinline__ RowResult route_row(const float (&v)[kPerLane],
                                               const float (&bv)[kPerLane], const RowSpec& s)
{
    const bool need_all = s.has_bias || (s.scoring == kSoftmax && !s.renorm);
    return need_all ? route_row_impl<true>(v, bv, s) : route_row_impl<false>(v, bv, s);
}

// ---------------------------------------------------------------------------
// M=2 unique-route table (b70 lab MTP1 note, "Unique-route router screen")
// ---------------------------------------------------------------------------
// One wavefront; slot s = t*k + j holds inds[t][j] (2k <= 64 slots).  Stable
// de-duplication by first appearance, ranks by a prefix count of first
// appearances, token masks gathered onto each first appearance.
__device__ __forceinline__ void emit_route_table_m2(const int32_t* slot_ids, int k,
                                                    int32_t* ids, int32_t* mask,
                                                    int32_t* slot_to_unique, int32_t* count)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int n = 2 * k;
    const bool active = lane < n;
    const int id = active ? slot_ids[lane] : -1 - lane;  // inactive lanes never match

    int first = -1;
    for (int j = 0; j < n; ++j) {
        const int idj = __builtin_amdgcn_readlane(id, j);
        if (first < 0 && idj == id) first = j;
    }
    const uint64_t firsts = __builtin_amdgcn_ballot_w64(active && first == lane);
    const int unique = __builtin_popcountll(firsts);
    const int rank = active ? __builtin_popcountll(firsts & ((1ull << first) - 1ull)) : 0;

    int token_bits = 0;
    for (int j = 0; j < n; ++j) {
        const int fj = __builtin_amdgcn_readlane(first, j);
        if (lane == fj) token_bits |= 1 << (j / k);
    }

    if (active) {
        slot_to_unique[lane] = rank;
        if (first == lane) {
            ids[rank] = id;
            mask[rank] = token_bits;
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

}  // namespace gpt
