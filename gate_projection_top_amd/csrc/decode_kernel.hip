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
//   kLoadWaves load waves and one control wave.  (Up to kExpertMaxRows
//   tokens take the one-expert-per-workgroup kernel instead.)
//   Start: the control wave draws an arrival ticket, in two levels: on its
//     expert block's word (S arrivals), then, for the last of those, on the
//     row block's word (B arrivals).  The workgroups that draw the last F row
//     tickets are the row block's finishers (F > 1 when the block has more
//     rows than a workgroup has waves to spare, each finisher taking every
//     F-th row).  An expert block's word also carries the row block's epoch
//     in its upper bits: every workgroup learns it from its own ticket and
//     tags the partials it publishes with it; the last arrival on a block
//     word moves its epoch on while clearing its count, and the last finisher
//     moves on the words of blocks this launch does not use, so all of a row
//     block's words keep one epoch.  The ticket's round trip overlaps the
//     loads of phase 1.
//   Phase 1 (every workgroup): the 16x16 (tokens x experts) partial dot
//     products over its H-split, one bf16 MFMA 16x16x32 per 32-wide k-step,
//     every wave's loads issued before its first MFMA; the waves' partials
//     summed in LDS in wave order and published as (value, tag) pairs with
//     device-coherent stores.  Non-finishers are then done.
//   Phase 2 (finisher): each wave takes rows of the block; lane L polls the
//     S partials of experts 4L..4L+3 (the routing layout itself) until all
//     carry this launch's tag, adds them in split order and routes the row
//     with route_row(); a helper wave clears the slots' tags afterwards (tag
//     0, which no launch uses); the unique-route table, when asked for,
//     follows.  Counters return to zero and epochs move on, so the kernel
//     replays inside a HIP graph.
//   The last finisher's wait always ends (every workgroup of its row block
//     has drawn a ticket, so all have started, and none waits).  A finisher
//     that is not the last waits for workgroups that may not have started
//     yet; they start as soon as any CU frees a slot, since no workgroup of
//     this kernel but the finishers ever waits.  Every wait is bounded all
//     the same (wait_ticks): a row given up comes out as index -1 with a NaN
//     weight and sets kStatusWaitLimit, and the slots it leaves behind carry
//     an older tag, so no later launch takes them for its own.
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

typedef int i32x4 __attribute__((ext_vector_type(4)));

// A launch's tag: odd, so never the cleared value 0.
__device__ __forceinline__ uint32_t partial_tag(uint64_t epoch) { return ((uint32_t)epoch << 1) | 1u; }

// One poll: every split's (value, tag) pairs of this lane's four experts, two
// 16-byte loads per split.  Splits q >= S lie past the end of the buffer
// range: their loads return zeros without touching memory.  The empty asm
// keeps the loads from being hoisted out of the polling loop.
template <int kMaxS>
__device__ __forceinline__ void poll_issue(u32x4 (&p)[kMaxS][2], __amdgpu_buffer_rsrc_t prs, int off,
                                           int qstride)
{
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < kMaxS; ++q) {
        p[q][0] = __builtin_amdgcn_raw_buffer_load_b128(prs, off + q * qstride, 0, kCoherent);
        p[q][1] = __builtin_amdgcn_raw_buffer_load_b128(prs, off + q * qstride + 16, 0, kCoherent);
    }
}

// True when every lane that owns published slots sees this launch's tag in
// all of them (splits q < S).
template <int kMaxS>
__device__ __forceinline__ bool poll_ready(const u32x4 (&p)[kMaxS][2], bool mine, int S, uint32_t tag)
{
    int ok = 1;  // bitwise, not short-circuit: no branch per slot
#pragma unroll
    for (int q = 0; q < kMaxS; ++q)
        ok &= (int)(q >= S) | ((int)(p[q][0][1] == tag) & (int)(p[q][0][3] == tag) & (int)(p[q][1][1] == tag) &
                               (int)(p[q][1][3] == tag));
    return __builtin_amdgcn_ballot_w64(mine && ok == 0) == 0;
}

// The logit: partials added in split order (zeros past S change nothing).
template <int kMaxS>
__device__ __forceinline__ f32x4 poll_sum(const u32x4 (&p)[kMaxS][2])
{
    f32x4 sum = {__uint_as_float(p[0][0][0]), __uint_as_float(p[0][0][2]), __uint_as_float(p[0][1][0]),
                 __uint_as_float(p[0][1][2])};
#pragma unroll
    for (int q = 1; q < kMaxS; ++q)
        sum += f32x4{__uint_as_float(p[q][0][0]), __uint_as_float(p[q][0][2]), __uint_as_float(p[q][1][0]),
                     __uint_as_float(p[q][1][2])};
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
    __shared__ uint32_t s_tag;  // this launch's tag (row block epoch)
    __shared__ uint64_t sel[kWaves][kRefineSlots];  // selection scratch, one per routing wave
    __shared__ double exp2_tab[kWave][2];  // the exp table (load_exp2_lane), for the routing waves
    __shared__ float bias_tab[kMaxE];       // the selection bias (0 past E and without one)

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
    // of a finisher routes more than one row.  With the route table, every
    // routing wave also publishes its row's indices as (index, tag) slots,
    // and the last finisher collects them and builds the table.
    const int t0 = r * kDecodeTile;
    const int rows_here = min(kDecodeTile, a.M - t0);
    const int nfin = min(B, rows_here);

    if (tid < kDecodeTile) polled[tid] = 0;
    if (wave == kLoadWaves) {
        // ---- control wave: the arrival ticket, in two levels so that no
        // counter sees more than max(S, B) arrivals: the last of an expert
        // block's S workgroups goes on to the row block's counter, and the
        // last of those B is the finisher.  The control wave's waits stall no
        // load wave.  Each counter is reset by the workgroup that drew its
        // last ticket, when every ticket on it has been drawn.
        if (lane == 0) {
            // 8-byte words, one 64-byte line apart: (epoch << 8 | count) per
            // (row block, expert block), then a count per row block
            uint64_t* words = reinterpret_cast<uint64_t*>(a.counters);
            constexpr int kW = kDecodeCounterStride / 2;
            uint64_t* block_w = words + kW * (r * kDecodeMaxBlocks + b);
            uint64_t* row_w = words + kW * (kDecodeMaxRowBlocks * kDecodeMaxBlocks + r);
            int fin = -1;
            const uint64_t old = __hip_atomic_fetch_add(block_w, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_tag = partial_tag(old >> 8);
            if ((int)(old & 0xffu) == a.S - 1) {
                // last of the block: next epoch, count back to zero
                __hip_atomic_fetch_add(block_w, (1ull << 8) - (uint64_t)a.S, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t rt = __hip_atomic_fetch_add(row_w, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if ((int)rt == B - 1) {
                    __hip_atomic_store(row_w, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    for (int u = B; u < kDecodeMaxBlocks; ++u)
                        __hip_atomic_fetch_add(words + kW * (r * kDecodeMaxBlocks + u), 1ull << 8, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                }
                if ((int)rt >= B - nfin) fin = (int)rt - (B - nfin);
            }
            fin_index = fin;
        }
        // The routing waves' exp table and selection bias (past E, and with
        // no bias, out-of-range buffer loads return 0), fetched here after the
        // ticket (fetched before it, they would hold up its atomics: loads
        // complete in order), during the load waves' loads, and handed over
        // in LDS at the barrier: fetched by a routing wave after the barrier,
        // a cold line would hold up its poll.
        const Exp2Lane t = load_exp2_lane();
        float tb[kPerLane];
        {
            const __amdgpu_buffer_rsrc_t brs0 = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(a.bias), 0, a.bias ? a.E * 4 : 0, 0x00020000);
#pragma unroll
            for (int j = 0; j < kPerLane; ++j)
                tb[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                      brs0, (lane * kPerLane + j) * 4, 0, 0));
        }
        exp2_tab[lane][0] = t.hi;
        exp2_tab[lane][1] = t.lo;
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) bias_tab[lane * kPerLane + j] = tb[j];
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
    // stores them with the tag, device-coherently (lane l: token row l/4,
    // experts 4(l%4)..+3 of the block).  Layout [S][M][256] (value, tag).
    const int qstride = a.M * kMaxE * 8;  // bytes per split
    const __amdgpu_buffer_rsrc_t prs =
        __builtin_amdgcn_make_buffer_rsrc(a.partials, 0, a.S * qstride, 0x00020000);
    const uint32_t tag = s_tag;  // written by the control wave before the barrier
    if (wave == 0) {
        const int rr = lane >> 2, cc = (lane & 3) * 4;
        float sum[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v = red[0][rr][cc + j];
#pragma unroll
            for (int w = 1; w < kLoadWaves; ++w) v += red[w][rr][cc + j];
            sum[j] = v;
        }
        const int row = r * kDecodeTile + rr;
        if (row < a.M) {
            const int off = s * qstride + (row * kMaxE + b * kDecodeTile + cc) * 8;
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(sum[0]), tag, __float_as_uint(sum[1]), tag},
                                                   prs, off, 0, kCoherent);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{__float_as_uint(sum[2]), tag, __float_as_uint(sum[3]), tag},
                                                   prs, off + 16, 0, kCoherent);
        }
    }
    const int f = fin_index;  // written by the control wave before the barrier
    if (f < 0) return;

    // ---- phase 2 (finisher f): rows t = f + nfin*i of the row block, one
    // wave per row; lane L owns experts 4L..4L+3.
    const int nrows = (rows_here - f + nfin - 1) / nfin;  // this finisher's rows
    const RowSpec spec{a.E, a.k, a.scoring, a.renorm, a.bias != nullptr};
    const bool mine = lane < 4 * B;  // the lane's expert group lies in a published block
    const u32x4 cleared = {0u, 0u, 0u, 0u};
    // the table's (index, tag) slots (routed slot s = t*k + j of the block)
    const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
        a.counters + kDecodeTableSlotWord, 0, a.table_ids ? 64 * 8 : 0, 0x00020000);

    // Rows go to the waves in turn starting at wave 1 (wave 0 has just spent
    // its time on the publish, and the others reach this point first).
    // The first wave with no row of its own takes one pass over a dummy row
    // through the same code: the finisher runs on a different CU from call
    // to call, so its routing code is usually not in that CU's instruction
    // cache, and this wave, running ahead, fetches it while the row waves
    // are still polling.  (One wave only: dummy passes share SIMDs with the
    // real rows.)  The next free wave, if there is one, clears the tags of
    // each row's slots once the row's wave has read them, so the row waves
    // go straight from their poll to routing.
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
                   __builtin_amdgcn_s_memrealtime() - t_wait < 2ull * a.wait_ticks)
                __builtin_amdgcn_s_sleep(1);
            if (st == 1 && mine) {
                const int off = ((t0 + f + nfin * t) * kMaxE + lane * kPerLane) * 8;
#pragma unroll
                for (int q = 0; q < kMaxS; ++q) {
                    __builtin_amdgcn_raw_buffer_store_b128(cleared, prs, off + q * qstride, 0, kCoherent);
                    __builtin_amdgcn_raw_buffer_store_b128(cleared, prs, off + q * qstride + 16, 0, kCoherent);
                }
            }
        }
    }
    const Exp2Lane et{exp2_tab[lane][0], exp2_tab[lane][1]};
    for (int it = 0; it < passes; ++it) {
        const int i = slot_of_wave + it * kWaves;  // the finisher's i-th row
        const bool real = i < nrows;               // wave-uniform
        const int t = f + nfin * i;                // its row in the block
        float v[kPerLane];
        float bv[kPerLane] = {0.f, 0.f, 0.f, 0.f};
        if (real) {
            const int off = ((t0 + t) * kMaxE + lane * kPerLane) * 8;
            // Splits q >= S lie past the end of the buffer range: their loads
            // return zeros (and are not examined) and their stores are
            // dropped.  The wait ends once the publishers' stores land; the
            // time limit only bounds it: a row that reaches it is reported as
            // index -1 with a NaN weight.
            f32x4 sum;
            const uint64_t t_poll = __builtin_amdgcn_s_memrealtime();
            bool gave_up = false;
            u32x4 p0[kMaxS][2];
            for (;;) {
                poll_issue<kMaxS>(p0, prs, off, qstride);
                if (poll_ready<kMaxS>(p0, mine, a.S, tag)) {
                    sum = poll_sum<kMaxS>(p0);
                    break;
                }
                if (__builtin_amdgcn_s_memrealtime() - t_poll > a.wait_ticks) {
                    gave_up = true;
                    break;
                }
            }
            if (gave_up) {
                if (lane == 0) {
                    __hip_atomic_store(&polled[i], 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                    __hip_atomic_fetch_or(a.status, kStatusWaitLimit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                }
                if (lane < a.k) {
                    const int64_t o = (int64_t)(t0 + t) * a.k + lane;
                    a.inds[o] = -1;
                    a.weights[o] = __builtin_nanf("");
                    if (a.table_ids) {
                        const u32x2 sv = {0xffffffffu, tag};
                        __builtin_amdgcn_raw_buffer_store_b64(sv, trs, (t * a.k + lane) * 8, 0, kCoherent);
                    }
                }
                continue;
            }
            if (has_helper) {
                if (lane == 0) __hip_atomic_store(&polled[i], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            } else if (mine) {
#pragma unroll
                for (int q = 0; q < kMaxS; ++q) {
                    __builtin_amdgcn_raw_buffer_store_b128(cleared, prs, off + q * qstride, 0, kCoherent);
                    __builtin_amdgcn_raw_buffer_store_b128(cleared, prs, off + q * qstride + 16, 0, kCoherent);
                }
            }
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) bv[j] = bias_tab[lane * kPerLane + j];
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
        const RowResult res = route_row<kFilter>(v, bv, spec, sel[wave], et);
        if (!real) {
            asm volatile("; dummy row %0 %1" :: "v"(res.idx), "v"(res.w));  // keep the pass
            continue;
        }
        if (lane < a.k) {
            const int64_t o = (int64_t)(t0 + t) * a.k + lane;
            a.inds[o] = res.idx;
            a.weights[o] = res.w;
            if (a.table_ids) {
                const u32x2 sv = {(uint32_t)res.idx, tag};
                __builtin_amdgcn_raw_buffer_store_b64(sv, trs, (t * a.k + lane) * 8, 0, kCoherent);
            }
        }
    }

    if (a.table_ids && f == nfin - 1 && wave == 0) {
        // Table (M <= 16: one row block): wave 0 of the last finisher (the
        // last workgroup to draw a ticket, so every routing wave it waits on
        // has started) waits until every routed slot carries this launch's
        // tag (lane s: slot s), then builds the table.
        const int nslots = a.M * a.k;
        const uint64_t t_wait = __builtin_amdgcn_s_memrealtime();
        int32_t id = -1;
        for (;;) {
            asm volatile("" ::: "memory");
            const u32x2 sv = __builtin_amdgcn_raw_buffer_load_b64(trs, lane * 8, 0, kCoherent);
            const bool ok = lane >= nslots || sv[1] == tag;
            if (__builtin_amdgcn_ballot_w64(!ok) == 0) {
                id = (int32_t)sv[0];
                break;
            }
            if (__builtin_amdgcn_s_memrealtime() - t_wait > a.wait_ticks) {
                // a row never arrived: its slots read -1, as a given-up row's do
                if (lane == 0)
                    __hip_atomic_fetch_or(a.status, kStatusWaitLimit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
                id = ok ? (int32_t)sv[0] : -1;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        slots[lane] = id;
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        emit_route_table(slots, a.M, a.k, tab_first, tab_mask, a.table_ids, a.table_mask, a.table_s2u,
                         a.table_count);
    }
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream)
{
    const int R = (a.M + kDecodeTile - 1) / kDecodeTile;
    const int B = (a.E + kDecodeTile - 1) / kDecodeTile;
    const int grid = R * B * a.S;
    if (a.load_waves != kDecodeWide.load_waves || a.S > kDecodeWide.max_splits || a.S < 1)
        return hipErrorInvalidValue;
    const dim3 wb((kDecodeWide.load_waves + 1) * kWave);
#define GPT_DECODE_LAUNCH(FMT)                                                                           \
    hipLaunchKernelGGL((decode_router_kernel<kDecodeWide.load_waves, kDecodeWide.max_splits, FMT>), dim3(grid), \
                       wb, 0, stream, a)
    if (a.w_format == kGateBf16) GPT_DECODE_LAUNCH(kGateBf16);
    else if (a.w_format == kGateMxfp4) GPT_DECODE_LAUNCH(kGateMxfp4);
    else if (a.w_format == kGateMxfp8) GPT_DECODE_LAUNCH(kGateMxfp8);
    else return hipErrorInvalidValue;
#undef GPT_DECODE_LAUNCH
    return hipGetLastError();
}

}  // namespace gpt
