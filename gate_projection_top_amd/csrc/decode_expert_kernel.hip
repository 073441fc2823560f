// Fused decode router for a few tokens (M <= kExpertMaxRows): gate
// projection, scoring, top-k and renormalisation in ONE launch (qwisp issue
// #145, "Change": one kernel from postNorm to inds/scores, the E logits
// held on chip).
//
// The page leaves open how a matvec spread over many workgroups meets a
// top-k that needs the whole logit row in one place.  Here each workgroup
// owns ONE expert: it streams that expert's whole gate row (H bf16 values,
// 14 KiB at H = 7168, contiguous) and forms the complete logit of every
// token, so the hand-off to the routing workgroup carries finished logits
// (one 8-byte slot per token and expert, 1 KiB + tags per row) rather than
// partial sums.
//
//   grid = E workgroups of four load waves (eight above four tokens), one
//   control wave and one warm-up wave.
//   Control wave: draws the arrival ticket at kernel start, in two levels
//     (groups of 16 workgroups, then the groups), so no counter sees more
//     than 16 arrivals.  A group's counter word also carries the epoch of
//     the launch in its upper bits: every workgroup learns the epoch from its
//     own ticket, tags its published logits with it, and the last arrival of
//     a group moves the group's epoch on while clearing its count.  The
//     workgroup drawing the last group ticket is the finisher; every other
//     workgroup has drawn a ticket by then, so all of them have started and
//     none of them waits on anything: the finisher's wait below always ends.
//   Phase 1 (load waves): thread t takes 16-byte units t, t + 256, ... of the
//     gate row and the same units of each token's activation row, all of a
//     batch's loads issued before the first product; fp32 fused multiply-adds
//     in a fixed order; the waves' sums meet in LDS and are added in wave
//     order.  Every expert's logit is therefore formed by the same sequence
//     of operations, so equal gate rows give bitwise-equal logits (the
//     contract's ties).
//   Publish: one device-coherent 8-byte store (logit, tag) per token.
//   Phase 2 (finisher): wave t routes token t; lane L polls the slots of
//     experts 4L..4L+3 (two 16-byte loads; several polls in flight) until all
//     four carry this launch's tag, clears them (tag 0, which no launch uses),
//     and routes the row; a spare wave runs the routing code once on a dummy
//     row first, so the finisher's CU has it in its instruction cache.  The
//     unique-route table, when asked for, follows.
//
// Tags make the hand-off robust: a slot published by an earlier launch (for
// instance after a finisher stopped waiting at the time limit and a publish
// landed later) carries an older tag and is never taken for this launch's.
// A finisher that reaches the limit writes index -1 and a NaN weight for the
// row and sets kStatusWaitLimit in the workspace's sticky status word.
#include <mutex>

#include "coherent.hpp"
#include "launch.hpp"
#include "route_common.hpp"

namespace gpt {

namespace {

// Load waves per workgroup: four for up to four tokens, eight (one routing
// wave per token) for more; 16-byte gate loads per thread issued together.
template <int kRows> constexpr int kLoadWavesOf = kRows <= 4 ? 4 : 8;
template <int kRows> constexpr int kBatchOf = kRows <= 4 ? 4 : 2;
constexpr int kPollsInFlight = 3;
constexpr int kPollGap = 2;       // s_sleep units (64 clocks) between polls

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Sum over the wavefront in a fixed association (butterfly inside each
// 16-lane row, then rows 0..3 in order); every lane gets the same bits.
__device__ __forceinline__ float wave_sum_f32(float v)
{
    v = v + __builtin_bit_cast(float, dpp_u32<0xB1>(__builtin_bit_cast(uint32_t, v)));
    v = v + __builtin_bit_cast(float, dpp_u32<0x4E>(__builtin_bit_cast(uint32_t, v)));
    v = v + __builtin_bit_cast(float, dpp_u32<0x124>(__builtin_bit_cast(uint32_t, v)));
    v = v + __builtin_bit_cast(float, dpp_u32<0x128>(__builtin_bit_cast(uint32_t, v)));
    const float a = __builtin_bit_cast(float, readlane_u32(__builtin_bit_cast(uint32_t, v), 0));
    const float b = __builtin_bit_cast(float, readlane_u32(__builtin_bit_cast(uint32_t, v), 16));
    const float c = __builtin_bit_cast(float, readlane_u32(__builtin_bit_cast(uint32_t, v), 32));
    const float d = __builtin_bit_cast(float, readlane_u32(__builtin_bit_cast(uint32_t, v), 48));
    return ((a + b) + c) + d;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// acc + sum over the 8 products of two 16-byte bf16 units, in element order.
__device__ __forceinline__ float dot8(u32x4v x, u32x4v w, float acc)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc = __builtin_fmaf(bf16_lo(x[q]), bf16_lo(w[q]), acc);
        acc = __builtin_fmaf(bf16_hi(x[q]), bf16_hi(w[q]), acc);
    }
    return acc;
}

// acc + sum over 8 products of a 16-byte bf16 activation unit and eight gate
// values already in fp32 (g[0..7]), in element order.
__device__ __forceinline__ float dot8f(u32x4v x, const float (&g)[8], float acc)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc = __builtin_fmaf(bf16_lo(x[q]), g[2 * q], acc);
        acc = __builtin_fmaf(bf16_hi(x[q]), g[2 * q + 1], acc);
    }
    return acc;
}

__device__ __forceinline__ u32x4v load16(const void* p) { return *reinterpret_cast<const u32x4v*>(p); }

// A launch's tag: odd, so never the cleared value 0.
__device__ __forceinline__ uint32_t tag_of(uint64_t epoch) { return ((uint32_t)epoch << 1) | 1u; }

// Waves of a workgroup: the load waves, then the control wave, then the
// warm-up wave.
template <int kRows> constexpr int kBlockOf = (kLoadWavesOf<kRows> + 2) * kWave;

// Waits (sleeping) until the workgroup-shared word reaches `want`.
__device__ __forceinline__ void wait_lds_at_least(int* w, int want)
{
    while (__hip_atomic_load(w, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < want) __builtin_amdgcn_s_sleep(1);
}

template <int kRows, int kFmt>
__global__ __launch_bounds__(kBlockOf<kRows>) void decode_expert_kernel(DecodeLaunch a)
{
    constexpr int kLoadWaves = kLoadWavesOf<kRows>;
    constexpr int kThreads = kLoadWaves * kWave;
    constexpr int kBatch = kBatchOf<kRows>;
    constexpr int kControlWave = kLoadWaves;
    constexpr int kWarmWave = kLoadWaves + 1;
    __shared__ float red[kLoadWaves][kRows];
    __shared__ uint64_t sel[kWarmWave + 1][kRefineSlots];  // selection scratch, one per routing wave
    __shared__ int32_t slots[kWave];                      // route table: M*k <= 64 slots
    __shared__ int32_t tab_first[kMaxE + 1], tab_mask[kMaxE + 1];
    __shared__ uint32_t s_tag;
    __shared__ int s_loaded;  // load waves whose sums are in `red`
    __shared__ int s_ctl;     // 1: s_tag written; 2: s_role written too
    __shared__ int s_role;    // 0: publisher, 1: finisher
    __shared__ double s_exp2[kWave][2];  // the exp table (load_exp2_lane), for the routing waves
    __shared__ float s_bias[kMaxE];      // the selection bias (0 past E and without one)
    __shared__ int s_aux;                // 1: s_exp2 and s_bias written

    const int e = blockIdx.x;  // this workgroup's expert
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int M = a.M;
    const RowSpec spec{a.E, a.k, a.scoring, a.renorm, a.bias != nullptr};

    if (tid == 0) {
        s_loaded = 0;
        s_ctl = 0;
        s_aux = 0;
    }
    __syncthreads();  // the only barrier before the routing: the warm-up wave never waits

    if (wave == kWarmWave) {
        // Fetches the routing waves' exp table and selection bias into LDS
        // (fetched by a routing wave, a cold line would hold up its poll or
        // its loads: loads complete in order), then runs the routing code
        // once on a dummy row: whichever workgroup turns out to be the
        // finisher then finds that code in its CU's instruction cache when
        // its rows' logits arrive, instead of fetching it instruction block
        // by block while the row waits.
        const Exp2Lane et = load_exp2_lane();
        const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(a.bias), 0, a.bias ? a.E * 4 : 0, 0x00020000);
        float v[kPerLane], bv[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j)  // bias past E reads as 0 (out-of-range loads return zero)
            bv[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  brs, (lane * kPerLane + j) * 4, 0, 0));
        s_exp2[lane][0] = et.hi;
        s_exp2[lane][1] = et.lo;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            s_bias[lane * kPerLane + j] = bv[j];
            v[j] = 0.0625f * (float)(lane * kPerLane + j);
            bv[j] = 0.f;
        }
        __hip_atomic_store(&s_aux, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        const RowResult res = route_row<kFilter>(v, bv, spec, sel[kWarmWave], et);
        asm volatile("; warm-up row %0 %1" ::"v"(res.idx), "v"(res.w));  // keep the pass
        return;
    }

    if (wave == kControlWave) {
        // ---- control wave: ticket and epoch
        int role = 0;
        if (lane == 0) {
            const int g = e / kExpertGroup;
            const int ng = min(kExpertGroup, a.E - kExpertGroup * g);
            const int B = (a.E + kExpertGroup - 1) / kExpertGroup;
            uint64_t* gw = a.xcounters + kExpertCounterStride * g;
            const uint64_t old = __hip_atomic_fetch_add(gw, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t epoch = old >> 8;
            s_tag = tag_of(epoch);
            __hip_atomic_store(&s_ctl, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            if ((int)(old & 0xffu) == ng - 1) {
                // last of the group: next epoch, count back to zero
                __hip_atomic_fetch_add(gw, (1ull << 8) - (uint64_t)ng, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                uint64_t* top = a.xcounters + kExpertCounterStride * kExpertGroups;
                const uint64_t t = __hip_atomic_fetch_add(top, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((int)t == B - 1) {
                    __hip_atomic_store(top, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    // groups this launch does not use move on too, so that every
                    // group word carries the same epoch at the next launch
                    for (int u = B; u < kExpertGroups; ++u)
                        __hip_atomic_fetch_add(a.xcounters + kExpertCounterStride * u, 1ull << 8, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                    role = 1;
                }
            }
            s_role = role;
            __hip_atomic_store(&s_ctl, 2, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        return;
    }

    // ---- phase 1 (load waves): this expert's logit for every token
    {
        float acc[kRows];
#pragma unroll
        for (int t = 0; t < kRows; ++t) acc[t] = 0.f;
        if constexpr (kFmt == kGateBf16) {
            const int nu = a.H >> 3;  // 16-byte units per row
            const uint16_t* wrow = a.w + (int64_t)e * a.H;
            for (int base = 0; base < nu; base += kThreads * kBatch) {
                u32x4v wv[kBatch];
                u32x4v xv[kBatch][kRows];
#pragma unroll
                for (int i = 0; i < kBatch; ++i) {
                    const int u = base + i * kThreads + tid;
                    const bool in = u < nu;
                    wv[i] = in ? load16(wrow + 8 * u) : u32x4v{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int t = 0; t < kRows; ++t)
                        xv[i][t] = (in && t < M) ? load16(a.x + (int64_t)t * a.H + 8 * u) : u32x4v{0u, 0u, 0u, 0u};
                }
#pragma unroll
                for (int i = 0; i < kBatch; ++i)
#pragma unroll
                    for (int t = 0; t < kRows; ++t) acc[t] = dot8(xv[i][t], wv[i], acc[t]);
            }
        } else {
            // block-scaled gate: unit u = 32 codes (16 bytes of E2M1, 32 of
            // E4M3) and their block's E8M0 scale; the activation's 32 values
            // are four 16-byte units.  Codes convert to fp32 exactly
            // (2^(s-127) times the code's value).
            const int nu = a.H >> 5;
            constexpr int kRowDiv = kFmt == kGateMxfp8 ? 1 : 2;
            const uint8_t* crow = a.w_codes + (int64_t)e * (a.H / kRowDiv);
            const uint8_t* srow = a.w_scale + (int64_t)e * (a.H / 32);
            for (int base = 0; base < nu; base += kThreads) {
                const int u = base + tid;
                const bool in = u < nu;
                const int uc = in ? u : 0;  // a lane past the row reads unit 0 (in bounds) and adds nothing
                u32x4v cv[2];
                cv[0] = load16(crow + (32 / kRowDiv) * uc);
                cv[1] = kFmt == kGateMxfp8 ? load16(crow + 32 * uc + 16) : u32x4v{0u, 0u, 0u, 0u};
                const uint32_t sb = srow[uc];
                u32x4v xv[kRows][4];
#pragma unroll
                for (int t = 0; t < kRows; ++t)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        xv[t][j] = (in && t < M) ? load16(a.x + (int64_t)t * a.H + 32 * u + 8 * j)
                                                 : u32x4v{0u, 0u, 0u, 0u};
                const float scale = in ? __uint_as_float(sb << 23) : 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float gv[8];
                    if constexpr (kFmt == kGateMxfp8) {
                        const uint32_t lo = cv[j / 2][(2 * j) % 4], hi = cv[j / 2][(2 * j + 1) % 4];
                        const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, scale, false);
                        const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(lo, scale, true);
                        const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, scale, false);
                        const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi, scale, true);
                        gv[0] = p0[0]; gv[1] = p0[1]; gv[2] = p1[0]; gv[3] = p1[1];
                        gv[4] = p2[0]; gv[5] = p2[1]; gv[6] = p3[0]; gv[7] = p3[1];
                    } else {
                        const uint32_t d = cv[0][j];
                        const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, scale, 0);
                        const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, scale, 1);
                        const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, scale, 2);
                        const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, scale, 3);
                        gv[0] = p0[0]; gv[1] = p0[1]; gv[2] = p1[0]; gv[3] = p1[1];
                        gv[4] = p2[0]; gv[5] = p2[1]; gv[6] = p3[0]; gv[7] = p3[1];
                    }
#pragma unroll
                    for (int t = 0; t < kRows; ++t) acc[t] = dot8f(xv[t][j], gv, acc[t]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < kRows; ++t) {
            const float s = wave_sum_f32(acc[t]);
            if (lane == 0) red[wave][t] = s;
        }
        if (lane == 0) __hip_atomic_fetch_add(&s_loaded, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }

    // ---- publish: lane t of wave 0 stores (logit, tag) of token t
    const __amdgpu_buffer_rsrc_t srs =
        __builtin_amdgcn_make_buffer_rsrc(a.xslots, 0, M * kMaxE * 8, 0x00020000);
    if (wave == 0) {
        wait_lds_at_least(&s_loaded, kLoadWaves);
        wait_lds_at_least(&s_ctl, 1);
        const uint32_t tag0 = s_tag;
        if (lane < M) {
            float l = red[0][lane];
#pragma unroll
            for (int w = 1; w < kLoadWaves; ++w) l += red[w][lane];
            const u32x2 v = {__float_as_uint(l), tag0};
            __builtin_amdgcn_raw_buffer_store_b64(v, srs, (lane * kMaxE + e) * 8, 0, kCoherent);
        }
    }
    wait_lds_at_least(&s_ctl, 2);
    if (s_role == 0) return;

    // ---- phase 2 (finisher): load wave t routes token t
    const uint32_t tag = s_tag;
    if (wave < M) {
        const int t = wave;
        // the warm-up wave's table and bias (in LDS before the poll starts)
        wait_lds_at_least(&s_aux, 1);
        const Exp2Lane et{s_exp2[lane][0], s_exp2[lane][1]};
        float bv[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) bv[j] = s_bias[lane * kPerLane + j];
        float v[kPerLane];
        bool gave_up = false;
        const int off = (t * kMaxE + lane * kPerLane) * 8;
        // valid[j]: expert 4L+j exists (slots past E are never published)
        const bool v0 = lane * kPerLane + 0 < a.E, v1 = lane * kPerLane + 1 < a.E;
        const bool v2 = lane * kPerLane + 2 < a.E, v3 = lane * kPerLane + 3 < a.E;
        u32x4v p[kPollsInFlight][2];
        auto issue = [&](int i) {
            asm volatile("" ::: "memory");
            p[i][0] = __builtin_amdgcn_raw_buffer_load_b128(srs, off, 0, kCoherent);
            p[i][1] = __builtin_amdgcn_raw_buffer_load_b128(srs, off + 16, 0, kCoherent);
        };
        auto ready = [&](int i) {
            // bitwise, not short-circuit: no branch per slot
            const int ok = ((int)!v0 | (int)(p[i][0][1] == tag)) & ((int)!v1 | (int)(p[i][0][3] == tag)) &
                           ((int)!v2 | (int)(p[i][1][1] == tag)) & ((int)!v3 | (int)(p[i][1][3] == tag));
            return __builtin_amdgcn_ballot_w64(ok == 0) == 0;
        };
        const uint64_t t_poll = __builtin_amdgcn_s_memrealtime();
        int got = -1;
#pragma unroll
        for (int i = 0; i < kPollsInFlight - 1; ++i) {
            issue(i);
            __builtin_amdgcn_s_sleep(kPollGap);
        }
        for (;;) {
            // the newest poll goes out before the oldest is examined
            issue(kPollsInFlight - 1);
            if (ready(0)) { got = 0; break; }
            __builtin_amdgcn_s_sleep(kPollGap);
            issue(0);
            if (ready(1)) { got = 1; break; }
            __builtin_amdgcn_s_sleep(kPollGap);
            issue(1);
            if (ready(2)) { got = 2; break; }
            if (__builtin_amdgcn_s_memrealtime() - t_poll > a.wait_ticks) {
                gave_up = true;
                break;
            }
            __builtin_amdgcn_s_sleep(kPollGap);
        }
        static_assert(kPollsInFlight == 3, "the polling loop above is written for three polls");
        if (gave_up) {
            if (lane == 0)
                __hip_atomic_fetch_or(a.status, kStatusWaitLimit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            if (lane < a.k) {
                const int64_t o = (int64_t)t * a.k + lane;
                a.inds[o] = -1;
                a.weights[o] = __builtin_nanf("");
                if (a.table_ids) slots[t * a.k + lane] = -1;
            }
        } else {
            const u32x4v q0 = got == 0 ? p[0][0] : (got == 1 ? p[1][0] : p[2][0]);
            const u32x4v q1 = got == 0 ? p[0][1] : (got == 1 ? p[1][1] : p[2][1]);
            v[0] = v0 ? __uint_as_float(q0[0]) : 0.f;
            v[1] = v1 ? __uint_as_float(q0[2]) : 0.f;
            v[2] = v2 ? __uint_as_float(q1[0]) : 0.f;
            v[3] = v3 ? __uint_as_float(q1[2]) : 0.f;
            // the slots are consumed: tag 0 until the next publish
            const u32x4v zero = {0u, 0u, 0u, 0u};
            __builtin_amdgcn_raw_buffer_store_b128(zero, srs, off, 0, kCoherent);
            __builtin_amdgcn_raw_buffer_store_b128(zero, srs, off + 16, 0, kCoherent);
            if (a.logits_out) {
                float* lo = a.logits_out + (int64_t)t * a.E + lane * kPerLane;
#pragma unroll
                for (int j = 0; j < kPerLane; ++j)
                    if (lane * kPerLane + j < a.E) lo[j] = v[j];
            }
            const RowResult res = route_row<kFilter>(v, bv, spec, sel[wave], et);
            if (lane < a.k) {
                const int64_t o = (int64_t)t * a.k + lane;
                a.inds[o] = res.idx;
                a.weights[o] = res.w;
                if (a.table_ids) slots[t * a.k + lane] = res.idx;  // M*k <= 64
            }
        }
    }

    if (a.table_ids) {
        // every routing wave has written its row's slots (waves that route
        // nothing arrive at once; the warm-up wave has exited or ends
        // without waiting)
        __syncthreads();
        if (wave == 0)
            emit_route_table(slots, M, a.k, tab_first, tab_mask, a.table_ids, a.table_mask, a.table_s2u,
                             a.table_count);
    }
}

}  // namespace

hipError_t launch_decode_expert(const DecodeLaunch& a, hipStream_t stream)
{
    if (a.M < 1 || a.M > kExpertMaxRows || a.E < 1 || a.E > kMaxE) return hipErrorInvalidValue;
    const dim3 grid(a.E);
#define GPT_EXPERT_LAUNCH(ROWS, FMT) \
    hipLaunchKernelGGL((decode_expert_kernel<ROWS, FMT>), grid, dim3(kBlockOf<ROWS>), 0, stream, a)
#define GPT_EXPERT_FORMATS(ROWS)                                                \
    if (a.w_format == kGateBf16) GPT_EXPERT_LAUNCH(ROWS, kGateBf16);            \
    else if (a.w_format == kGateMxfp4) GPT_EXPERT_LAUNCH(ROWS, kGateMxfp4);     \
    else if (a.w_format == kGateMxfp8) GPT_EXPERT_LAUNCH(ROWS, kGateMxfp8);     \
    else return hipErrorInvalidValue;
    if (a.M == 1) {
        GPT_EXPERT_FORMATS(1)
    } else if (a.M == 2) {
        GPT_EXPERT_FORMATS(2)
    } else if (a.M <= 4) {
        GPT_EXPERT_FORMATS(4)
    } else {
        GPT_EXPERT_FORMATS(8)
    }
#undef GPT_EXPERT_FORMATS
#undef GPT_EXPERT_LAUNCH
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// allocation-free entry: the kernel's workspace in static device memory
// ---------------------------------------------------------------------------
// Tagged logit slots, arrival words and the status word of the one-expert
// kernel for up to kNoAllocMaxRows tokens, in one array per device that the
// code object defines (zero when the library loads, which is the kernel's
// starting state: tag 0 is no launch's, every counter at zero).  Host code
// never uses the array's name as an address: each device's copy is resolved
// once with hipGetSymbolAddress (with that device current) and that pointer
// is what the kernel gets.  The array persists until the process ends; every
// call on a device shares it (overlapping calls on one device race).
constexpr size_t kNoAllocSlotBytes = (size_t)kNoAllocMaxRows * kMaxE * 8;
constexpr size_t kNoAllocCounterBytes = (size_t)kExpertCounterWords * 8;
constexpr size_t kNoAllocBytes = kNoAllocSlotBytes + kNoAllocCounterBytes + 256;  // + the status word
static_assert(kNoAllocSlotBytes % 256 == 0 && kNoAllocCounterBytes % 8 == 0, "scratch layout alignment");

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {
constexpr int kNoAllocDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kNoAllocDevices] = {};
}  // namespace

size_t noalloc_scratch_bytes() { return kNoAllocBytes; }

hipError_t noalloc_scratch(int device, void** out)
{
    if (device < 0 || device >= kNoAllocDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_scratch_mutex);
    if (!g_scratch_ptr[device]) {
        int prev = -1;
        hipError_t e = hipGetDevice(&prev);
        if (e != hipSuccess) return e;
        if (prev != device && (e = hipSetDevice(device)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (prev != device) (void)hipSetDevice(prev);
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = p;
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

hipError_t launch_decode_expert_noalloc(DecodeLaunch a, hipStream_t stream)
{
    if (a.M < 1 || a.M > kNoAllocMaxRows || a.table_ids) return hipErrorInvalidValue;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    void* base = nullptr;
    if ((e = noalloc_scratch(dev, &base)) != hipSuccess) return e;
    unsigned char* b = static_cast<unsigned char*>(base);
    a.xslots = reinterpret_cast<uint32_t*>(b);
    a.xcounters = reinterpret_cast<uint64_t*>(b + kNoAllocSlotBytes);
    a.status = reinterpret_cast<uint32_t*>(b + kNoAllocSlotBytes + kNoAllocCounterBytes);
    return launch_decode_expert(a, stream);
}

}  // namespace gpt
