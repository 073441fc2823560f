// Fused decode router (M <= 64 tokens): gate projection, scoring, top-k and
// renormalisation in ONE launch (qwisp issue #145, "Change": one kernel from
// postNorm to inds/scores with the E logits held on chip).
//
// The page leaves open how a matvec spread over many workgroups meets a top-k
// that needs the whole logit row in one place (serialise the matvec into one
// threadgroup, or reduce across threadgroups).  Here: reduce across
// workgroups, because one CU cannot pull the 2-3.5 MiB gate matrix from HBM
// fast enough on its own.
//
//   grid = R row blocks x B expert blocks x S H-splits; each workgroup has
//   kDecodeWaves load waves and one control wave.
//   Start: the control wave draws an arrival ticket on the row block's
//     counter.  The workgroups that draw the last F tickets are the row
//     block's finishers (F > 1 when the block has more rows than a
//     workgroup has waves to spare, each finisher taking every F-th row).
//     No workgroup but a finisher ever waits, and the grid (at most 256
//     workgroups) is resident at once, so the finishers' waits below always
//     end.  The ticket's round trip overlaps the loads of phase 1.
//   Phase 1 (every workgroup): the 16x16 (tokens x experts) partial dot
//     products over its H-split, one bf16 MFMA 16x16x32 per 32-wide k-step,
//     every wave's loads issued before its first MFMA; the waves' partials
//     summed in LDS in wave order and published with device-coherent 16-byte
//     stores.  Non-finishers are then done: no wait for the stores.
//   Phase 2 (finisher): every partial slot holds a signalling-NaN sentinel
//     between launches, and arithmetic never produces that bit pattern, so
//     a slot holding anything else has been published.  Each wave takes rows
//     of the block; lane L polls the S partials of experts 4L..4L+3 (the
//     routing layout itself) until none is the sentinel, resets those slots
//     to the sentinel, adds the partials in split order and routes the row
//     with route_row(); the unique-route table, when asked for, follows.  The finisher
//     also resets the counter, so the kernel replays inside a HIP graph.
//
// Every logit is accumulated in the same order regardless of its expert
// index, so two experts with identical gate rows get bitwise-equal logits and
// the tie goes to the lower index, as the contract requires.
#include "coherent.hpp"
#include "launch.hpp"
#include "route_common.hpp"

namespace gpt {

namespace {

constexpr int kChunk = 8;      // k-steps whose loads a wave issues before its MFMAs
constexpr int kPollGap = 16;   // s_sleep units (64 clocks) between the two polls in flight

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float not_sentinel(float v)
{
    // a quiet NaN stands in for the (never produced) sentinel pattern
    return __float_as_uint(v) == kPartialSentinel ? __uint_as_float(0x7fc00000u) : v;
}

__device__ __forceinline__ bool published(f32x4 v)
{
    // bitwise, not short-circuit: one compare per value, no branches
    const int p0 = __float_as_uint(v[0]) != kPartialSentinel, p1 = __float_as_uint(v[1]) != kPartialSentinel;
    const int p2 = __float_as_uint(v[2]) != kPartialSentinel, p3 = __float_as_uint(v[3]) != kPartialSentinel;
    return (p0 & p1 & p2 & p3) != 0;
}

// One poll: every split's slot of this lane's four experts.  Splits q >= S
// lie past the end of the buffer range, so their loads return zeros without
// touching memory.  The empty asm keeps the loads from being hoisted out of
// the polling loop.
template <int kMaxS>
__device__ __forceinline__ void poll_issue(f32x4 (&p)[kMaxS], __amdgpu_buffer_rsrc_t prs, int off,
                                           int qstride)
{
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < kMaxS; ++q) p[q] = fetch4(prs, off + q * qstride);
}

// True when no lane that owns published slots still sees the sentinel.
template <int kMaxS>
__device__ __forceinline__ bool poll_ready(const f32x4 (&p)[kMaxS], bool mine)
{
    bool ok = true;
#pragma unroll
    for (int q = 0; q < kMaxS; ++q) ok &= published(p[q]);
    return __builtin_amdgcn_ballot_w64(mine && !ok) == 0;
}

// The logit: partials added in split order (zeros past S change nothing).
template <int kMaxS>
__device__ __forceinline__ f32x4 poll_sum(const f32x4 (&p)[kMaxS])
{
    f32x4 sum = p[0];
#pragma unroll
    for (int q = 1; q < kMaxS; ++q) sum += p[q];
    return sum;
}

constexpr int kMxChunk = 2;  // block-scaled gate: 128-wide k blocks whose loads a wave issues together

template <int kLoadWaves, int kMaxS, int kFmt>
__global__ __launch_bounds__((kLoadWaves + 1) * kWave) void decode_router_kernel(DecodeLaunch a)
{
    constexpr int kWaves = kLoadWaves + 1;  // + the control wave

    __shared__ float red[kLoadWaves][kDecodeTile][kDecodeTile + 1];
    __shared__ int32_t slots[kWave];  // route table: M*k <= 64 slots
    __shared__ int32_t tab_first[kMaxE + 1], tab_mask[kMaxE + 1];
    __shared__ int polled[kDecodeTile];  // finisher: 1 = row's partials read, 2 = row gave up
    __shared__ int fin_index;  // this workgroup's finisher index, -1: not a finisher
    __shared__ uint64_t sel[kWaves][kFilterCap];  // selection scratch, one per routing wave

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int B = (a.E + kDecodeTile - 1) / kDecodeTile;

    // Block-scaled gates: the hardware deals consecutive workgroup ids to the
    // 8 XCDs in turn; renumber so that each XCD holds a contiguous range of
    // logical ids (whole expert blocks with all their splits), whose shared
    // scale lines its L2 then fetches once (measured: 14 % less fabric
    // traffic and a slightly shorter launch at M=1; the bf16 gate shares no
    // lines between splits but the token row, and measured slower this way).
    int bid = blockIdx.x;
    if constexpr (kFmt != kGateBf16)
        if (gridDim.x % 8u == 0u) bid = (bid % 8) * (int)(gridDim.x / 8u) + bid / 8;
    const int s = bid % a.S;
    bid /= a.S;
    const int b = bid % B;
    const int r = bid / B;

    // Finishers per row block: the last nfin workgroups to draw a ticket on
    // the block's row counter each route every nfin-th row, so that no wave
    // of a finisher routes more than one row.  (The route table needs all
    // rows in one workgroup: one finisher then.)
    const int t0 = r * kDecodeTile;
    const int rows_here = min(kDecodeTile, a.M - t0);
    const int nfin = a.table_ids ? 1 : min(B, max(1, (rows_here + kWaves - 2) / (kWaves - 1)));

    if (tid < kDecodeTile) polled[tid] = 0;
    if (wave == kLoadWaves) {
        // ---- control wave: the arrival ticket, in two levels so that no
        // counter sees more than max(S, B) arrivals: the last of an expert
        // block's S workgroups goes on to the row block's counter, and the
        // last of those B is the finisher.  The control wave's waits stall no
        // load wave.  Each counter is reset by the workgroup that drew its
        // last ticket, when every ticket on it has been drawn.
        if (lane == 0) {
            uint32_t* block_ctr = a.counters + kDecodeCounterStride * (r * kDecodeMaxBlocks + b);
            uint32_t* row_ctr = a.counters + kDecodeCounterStride * (kDecodeMaxRowBlocks * kDecodeMaxBlocks + r);
            int fin = -1;
            if (__hip_atomic_fetch_add(block_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)a.S - 1u) {
                __hip_atomic_store(block_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const uint32_t rt = __hip_atomic_fetch_add(row_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (rt == (uint32_t)B - 1u)
                    __hip_atomic_store(row_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (rt >= (uint32_t)(B - nfin)) fin = (int)rt - (B - nfin);
            }
            fin_index = fin;
        }
    } else {
        // ---- phase 1: partial logits of 16 tokens x 16 experts over one H-split
        const int arow = r * kDecodeTile + (lane & 15);  // MFMA A row  = token
        const int bcol = b * kDecodeTile + (lane & 15);  // MFMA B col  = expert
        const bool arow_ok = arow < a.M;
        const bool bcol_ok = bcol < a.E;
        const bf16x8 zero = __builtin_bit_cast(bf16x8, i32x4{0, 0, 0, 0});
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kFmt == kGateBf16) {
            const int kq = (lane >> 4) * 8;  // this lane's 8 of the 32 k
            const uint16_t* xp = a.x + (int64_t)(arow_ok ? arow : 0) * a.H + kq;
            const uint16_t* wp = a.w + (int64_t)(bcol_ok ? bcol : 0) * a.H + kq;

            const int KS = (a.H + 31) >> 5;
            const int ks0 = s * a.ks_per_split;
            const int ks1 = min(KS, ks0 + a.ks_per_split);

            for (int base = ks0 + wave; base < ks1; base += kLoadWaves * kChunk) {
                bf16x8 av[kChunk], bv[kChunk];
#pragma unroll
                for (int c = 0; c < kChunk; ++c) {
                    const int ks = base + c * kLoadWaves;
                    const int k0 = ks * 32;
                    const bool in = ks < ks1 && (k0 + kq) < a.H;
                    av[c] = (in && arow_ok) ? load_bf16x8(xp + k0) : zero;
                    bv[c] = (in && bcol_ok) ? load_bf16x8(wp + k0) : zero;
                }
#pragma unroll
                for (int c = 0; c < kChunk; ++c)
                    if (base + c * kLoadWaves < ks1)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[c], bv[c], acc, 0, 0, 0);
            }
        } else {
            // Block-scaled gate, in 128-wide k blocks.  Lane (expert, g) loads
            // the 32 codes of k in [128 kb + 32 g, +32) (16 bytes of MXFP4, 32
            // of MXFP8) and their block's scale; MFMA step j of the block gives
            // k-slots 8g..8g+7 the k values 128 kb + 32 g + 8 j + (0..7), for X
            // as for W, so every k is counted once.  (H % 32 == 0: a lane's 32
            // codes are in or out.)
            constexpr int kCodeBytes = kFmt == kGateMxfp8 ? 2 : 1;  // MXFP8: 2x16 bytes per 32 codes
            constexpr int kRowDiv = kFmt == kGateMxfp8 ? 1 : 2;     // code bytes per row = H / kRowDiv
            const int g = lane >> 4;
            const uint16_t* xrow = a.x + (int64_t)(arow_ok ? arow : 0) * a.H;
            const uint8_t* wrow = a.w_codes + (int64_t)(bcol_ok ? bcol : 0) * (a.H / kRowDiv);
            const uint8_t* srow = a.w_scale + (int64_t)(bcol_ok ? bcol : 0) * (a.H / 32);
            const int KB = (a.H + 127) >> 7;
            const int kb0 = s * a.ks_per_split;
            const int kb1 = min(KB, kb0 + a.ks_per_split);
            const int wave_u = __builtin_amdgcn_readfirstlane(wave);
            for (int base = kb0 + wave_u; base < kb1; base += kLoadWaves * kMxChunk) {
                u32x4 wv[kMxChunk][kCodeBytes];
                uint32_t sv[kMxChunk];
                bool wok[kMxChunk];
                bf16x8 xv[kMxChunk][4];
                // A block past the split is skipped by a wave-uniform branch.
                // Inside one, the gate codes and scale are loaded by every
                // lane (a lane past E or H reads its clamped row's first 32 k
                // of the block, always in bounds) and masked after the batch,
                // through a zero scale: a byte load under a per-lane branch,
                // or a select on a loaded value ahead of the next loads, makes
                // the compiler wait for the load there.  Activation rows past
                // M stay masked off (their lanes would break up the
                // coalescing of the real rows' loads).  The empty asm keeps
                // every load of the batch ahead of the first MFMA.
#pragma unroll
                for (int c = 0; c < kMxChunk; ++c) {
                    const int kb = base + c * kLoadWaves;
#pragma unroll
                    for (int h = 0; h < kCodeBytes; ++h) wv[c][h] = u32x4{0u, 0u, 0u, 0u};
                    sv[c] = 0u;
                    wok[c] = false;
#pragma unroll
                    for (int j = 0; j < 4; ++j) xv[c][j] = zero;
                    if (kb < kb1) {
                        const int k0 = kb * 128 + 32 * g;
                        const bool in = k0 < a.H;
                        const int kc = in ? k0 : kb * 128;
#pragma unroll
                        for (int h = 0; h < kCodeBytes; ++h)
                            wv[c][h] = *reinterpret_cast<const u32x4*>(wrow + kc / kRowDiv + 16 * h);
                        sv[c] = srow[kc / 32];
                        wok[c] = in && bcol_ok;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (in && arow_ok) xv[c][j] = load_bf16x8(xrow + k0 + 8 * j);
                    }
                }
                asm volatile("" ::: "memory");
#pragma unroll
                for (int c = 0; c < kMxChunk; ++c) {
                    if (base + c * kLoadWaves >= kb1) continue;
                    // 2^(s - 127); zero for a lane outside the gate
                    const float scale = wok[c] ? __uint_as_float(sv[c] << 23) : 0.0f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        bf16x8 wj;
                        if constexpr (kFmt == kGateMxfp8)  // codes 8j..8j+7: dwords 2j, 2j+1
                            wj = fp8x8_to_bf16x8(wv[c][j / 2][(2 * j) % 4], wv[c][j / 2][(2 * j + 1) % 4], scale);
                        else
                            wj = fp4x8_to_bf16x8(wv[c][0][j], scale);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv[c][j], wj, acc, 0, 0, 0);
                    }
                }
            }
        }
        // MFMA 16x16 result layout: lane holds rows 4*(lane/16)+i, column lane%16.
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][4 * (lane >> 4) + i][lane & 15] = acc[i];
    }
    __syncthreads();

    // ---- publish: wave 0 sums the load waves' partials (wave order) and
    // stores them device-coherently (lane l: token row l/4, experts
    // 4(l%4)..+3 of the block).  Layout [S][M][256] fp32.
    const int qstride = a.M * kMaxE * 4;  // bytes per split
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(a.partials, 0, a.S * qstride, 0x00020000);
    if (wave == 0) {
        const int rr = lane >> 2, cc = (lane & 3) * 4;
        f32x4 sum;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v = red[0][rr][cc + j];
#pragma unroll
            for (int w = 1; w < kLoadWaves; ++w) v += red[w][rr][cc + j];
            sum[j] = not_sentinel(v);
        }
        const int row = r * kDecodeTile + rr;
        if (row < a.M) publish4(prs, s * qstride + (row * kMaxE + b * kDecodeTile + cc) * 4, sum);
    }
    const int f = fin_index;  // written by the control wave before the barrier
    if (f < 0) return;

    // ---- phase 2 (finisher f): rows t = f + nfin*i of the row block, one
    // wave per row; lane L owns experts 4L..4L+3.
    const int nrows = (rows_here - f + nfin - 1) / nfin;  // this finisher's rows
    const RowSpec spec{a.E, a.k, a.scoring, a.renorm, a.bias != nullptr};
    const bool mine = lane < 4 * B;  // the lane's expert group lies in a published block
    const f32x4 sentinel4 = __builtin_bit_cast(f32x4, u32x4{kPartialSentinel, kPartialSentinel,
                                                            kPartialSentinel, kPartialSentinel});
    // bias beyond E reads as 0 (out-of-range buffer loads return zero)
    const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.bias), 0, a.bias ? a.E * 4 : 0, 0x00020000);

    // Rows go to the waves in turn starting at wave 1 (wave 0 has just spent
    // its time on the publish, and the others reach this point first).
    // The first wave with no row of its own takes one pass over a dummy row
    // through the same code: the finisher runs on a different CU from call
    // to call, so its routing code is usually not in that CU's instruction
    // cache, and this wave, running ahead, fetches it while the row waves
    // are still polling.  (One wave only: dummy passes share SIMDs with the
    // real rows.)  The next free wave, if there is one, puts the sentinel
    // back into each row's slots once the row's wave has read them, so the
    // row waves go straight from their poll to routing.
    const int slot_of_wave = (wave + kWaves - 1) % kWaves;  // row t goes to wave (t + 1) % kWaves
    const int my_rows = slot_of_wave < nrows ? (nrows - slot_of_wave + kWaves - 1) / kWaves : 0;
    const int passes = my_rows > 0 ? my_rows : (slot_of_wave == nrows ? 1 : 0);
    const bool has_helper = nrows + 1 < kWaves;
    if (has_helper && slot_of_wave == nrows + 1) {
        const uint64_t t_wait = __builtin_amdgcn_s_memrealtime();
        for (int t = 0; t < nrows; ++t) {
            int st;
            // the row waves' own poll limit bounds this wait; the doubled
            // limit here is only a guard
            while ((st = __hip_atomic_load(&polled[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) == 0 &&
                   __builtin_amdgcn_s_memrealtime() - t_wait < 2 * kDecodePollLimitTicks)
                __builtin_amdgcn_s_sleep(1);
            if (st == 1 && mine) {
                const int off = ((t0 + f + nfin * t) * kMaxE + lane * kPerLane) * 4;
#pragma unroll
                for (int q = 0; q < kMaxS; ++q) publish4(prs, off + q * qstride, sentinel4);
            }
        }
    }
    for (int it = 0; it < passes; ++it) {
        const int i = slot_of_wave + it * kWaves;  // the finisher's i-th row
        const bool real = i < nrows;               // wave-uniform
        const int t = f + nfin * i;                // its row in the block
        float v[kPerLane];
        float bv[kPerLane] = {0.f, 0.f, 0.f, 0.f};
        if (real) {
            const int off = ((t0 + t) * kMaxE + lane * kPerLane) * 4;
            // Splits q >= S lie past the end of the buffer range: their loads
            // return zeros and their stores are dropped, so no branch on S.
            // The wait ends once the publishers' stores land; the time limit is
            // only a guard so that no wave can spin forever: a row that hits it
            // is reported as index -1 with a NaN weight.
            f32x4 sum;
            const uint64_t t_poll = __builtin_amdgcn_s_memrealtime();
            bool gave_up = false;
            if constexpr (kMaxS <= 8) {
                // Two polls stay in flight, half a round trip apart, so a
                // partial that lands is seen about a quarter round trip
                // sooner on average.  (At 16 splits the second poll's
                // registers would spill.)
                f32x4 p0[kMaxS], p1[kMaxS];
                poll_issue<kMaxS>(p0, prs, off, qstride);
                __builtin_amdgcn_s_sleep(kPollGap);
                for (;;) {
                    poll_issue<kMaxS>(p1, prs, off, qstride);
                    if (poll_ready<kMaxS>(p0, mine)) {
                        sum = poll_sum<kMaxS>(p0);
                        break;
                    }
                    poll_issue<kMaxS>(p0, prs, off, qstride);
                    if (poll_ready<kMaxS>(p1, mine)) {
                        sum = poll_sum<kMaxS>(p1);
                        break;
                    }
                    if (__builtin_amdgcn_s_memrealtime() - t_poll > kDecodePollLimitTicks) {
                        gave_up = true;
                        break;
                    }
                }
            } else {
                f32x4 p0[kMaxS];
                for (;;) {
                    poll_issue<kMaxS>(p0, prs, off, qstride);
                    if (poll_ready<kMaxS>(p0, mine)) {
                        sum = poll_sum<kMaxS>(p0);
                        break;
                    }
                    if (__builtin_amdgcn_s_memrealtime() - t_poll > kDecodePollLimitTicks) {
                        gave_up = true;
                        break;
                    }
                }
            }
            if (gave_up) {
                if (lane == 0) __hip_atomic_store(&polled[i], 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                if (lane < a.k) {
                    const int64_t o = (int64_t)(t0 + t) * a.k + lane;
                    a.inds[o] = -1;
                    a.weights[o] = __builtin_nanf("");
                    if (a.table_ids) slots[t * a.k + lane] = -1;
                }
                continue;
            }
            if (has_helper) {
                if (lane == 0) __hip_atomic_store(&polled[i], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            } else if (mine) {
#pragma unroll
                for (int q = 0; q < kMaxS; ++q) publish4(prs, off + q * qstride, sentinel4);
            }
#pragma unroll
            for (int j = 0; j < kPerLane; ++j)
                bv[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                      brs, (lane * kPerLane + j) * 4, 0, 0));
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) v[j] = (lane * kPerLane + j < a.E) ? sum[j] : 0.f;
            if (a.logits_out) {
                float* lo = a.logits_out + (int64_t)(t0 + t) * a.E + lane * kPerLane;
#pragma unroll
                for (int j = 0; j < kPerLane; ++j)
                    if (lane * kPerLane + j < a.E) lo[j] = v[j];
            }
        } else {
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) v[j] = 0.0625f * (float)(lane * kPerLane + j);
        }
        // a routing wave has a SIMD to itself in the narrow geometry; the
        // wide one puts two or three waves on each SIMD
        const RowResult res = route_row<kFilter>(v, bv, spec, sel[wave]);
        if (!real) {
            asm volatile("; dummy row %0 %1" :: "v"(res.idx), "v"(res.w));  // keep the pass
            continue;
        }
        if (lane < a.k) {
            const int64_t o = (int64_t)(t0 + t) * a.k + lane;
            a.inds[o] = res.idx;
            a.weights[o] = res.w;
            if (a.table_ids) slots[t * a.k + lane] = res.idx;  // table: M*k <= 64
        }
    }

    if (a.table_ids) {  // table: M <= 16, so every row is in this row block
        __syncthreads();
        if (wave == 0)
            emit_route_table(slots, a.M, a.k, tab_first, tab_mask, a.table_ids, a.table_mask,
                             a.table_s2u, a.table_count);
    }
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream)
{
    const int R = (a.M + kDecodeTile - 1) / kDecodeTile;
    const int B = (a.E + kDecodeTile - 1) / kDecodeTile;
    const int grid = R * B * a.S;
    const bool narrow = a.load_waves == kDecodeNarrow.load_waves && a.S <= kDecodeNarrow.max_splits;
    const bool wide = a.load_waves == kDecodeWide.load_waves && a.S <= kDecodeWide.max_splits;
    const dim3 nb((kDecodeNarrow.load_waves + 1) * kWave), wb((kDecodeWide.load_waves + 1) * kWave);
#define GPT_DECODE_LAUNCH(GEO, FMT, BLOCK)                                                           \
    hipLaunchKernelGGL((decode_router_kernel<GEO.load_waves, GEO.max_splits, FMT>), dim3(grid), BLOCK, 0, \
                       stream, a)
    if (narrow && a.w_format == kGateBf16) GPT_DECODE_LAUNCH(kDecodeNarrow, kGateBf16, nb);
    else if (narrow && a.w_format == kGateMxfp4) GPT_DECODE_LAUNCH(kDecodeNarrow, kGateMxfp4, nb);
    else if (narrow && a.w_format == kGateMxfp8) GPT_DECODE_LAUNCH(kDecodeNarrow, kGateMxfp8, nb);
    else if (wide && a.w_format == kGateBf16) GPT_DECODE_LAUNCH(kDecodeWide, kGateBf16, wb);
    else if (wide && a.w_format == kGateMxfp4) GPT_DECODE_LAUNCH(kDecodeWide, kGateMxfp4, wb);
    else if (wide && a.w_format == kGateMxfp8) GPT_DECODE_LAUNCH(kDecodeWide, kGateMxfp8, wb);
    else return hipErrorInvalidValue;
#undef GPT_DECODE_LAUNCH
    return hipGetLastError();
}

}  // namespace gpt
