// Fused prefill router (M > 64 tokens): a bf16 MFMA GEMM whose epilogue does
// scoring, top-k and renormalisation per row from LDS, so the [M, E] logits
// never travel to HBM (dense_router_decode notes, "DenseRouterDecodeKernel":
// BF16 GEMM with FP32 accumulation and a row-level top-k epilogue rather than
// a per-element one; its TMA/TMEM warp roles have no gfx950 counterpart).
//
// Tiling.  A tile is 128 complete rows x all E <= 256 experts, so a row's
// logits meet in one workgroup.  With E = 256 columns only, a 32-row tile
// would re-read the whole gate matrix from L2 for every 32 tokens; 128-row
// tiles cut that traffic 4x.  To still occupy every CU, the K (= H) range of
// a tile is split S ways (S = 16, 8, 4 or 2: as many as the exchange buffer's
// 256 (tile, split) pairs allow for the tile count): S workgroups of 8 waves
// each compute the tile's 128 x 256 partial over their K slice.  The waves
// split the work by role: four producers issue every load of the LDS rings,
// so that only they ever queue on the memory pipeline, and four compute
// waves, each owning a 64 x 128 block as 4 x 8 MFMA 16x16x32 accumulators,
// only read fragments and multiply.  K is staged through the rings in
// 64-wide steps by direct-to-LDS buffer loads (no staging registers; 8
// consecutive lanes read one row's 128 contiguous bytes): X, streamed from
// HBM, three steps ahead; W, which every tile re-reads and L2 mostly holds,
// two steps ahead.  The MFMA operands are read back from LDS through XOR
// slot swizzles, measured free of bank conflicts for these reads.
//
// Split exchange.  Split s owns rows [s*128/S, (s+1)*128/S) for the
// epilogue.  It publishes the rows it does not own (device-coherent stores),
// takes a ticket on the tile's arrival counter, waits a bounded time for all
// S tickets, then sums the S partials of its rows in split order (its own
// from LDS) and routes them, reading the next rows' partials while routing
// the current ones.  If the wait times out (other splits not resident), it
// publishes its own rows, marks them abandoned and leaves; the split that
// takes the last ticket on the tile's completion counter routes every
// abandoned row set and resets the counters.  No workgroup ever waits
// without a bound, and every logit is summed in the same split order
// whichever path produces it.
#include "launch.hpp"
#include "route_common.hpp"
#include "coherent.hpp"

namespace gpt {

namespace {

constexpr int kBM = kPrefillTileRows;
constexpr int kXcds = 8;                    // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kBN = kMaxE;                  // 256
constexpr int kBK = 64;                     // k per stage: one 128-byte segment per row
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;    // 512
// LDS rings: X (from HBM) runs three stages ahead in a four-slot ring, W
// (re-read by every tile, so mostly served from L2) two stages ahead in a
// three-slot ring: 4 x 16 + 3 x 32 KiB = 160 KiB, all of the CU's LDS.
constexpr int kXSlots = 4;
constexpr int kWSlots = 3;
constexpr int kRowBytes = kBK * 2;
constexpr int kXStageBytes = kBM * kRowBytes;             // 16 KiB
constexpr int kWStageBytes = kBN * kRowBytes;             // 32 KiB
constexpr int kWRingOffset = kXSlots * kXStageBytes;      // 64 KiB
constexpr int kTileStride = kBN + 4;        // fp32 per row of the epilogue tile
constexpr int kTileBytes = kBM * kTileStride * 4;
constexpr int kRingBytes = kWRingOffset + kWSlots * kWStageBytes;
constexpr int kLdsBytes = kRingBytes;
constexpr int kFlagOffset = kLdsBytes - 16;  // one int after the ring's last use
// epilogue: each wave's selection scratch (route_rows' filter), past the row tile
constexpr int kSelOffset = ((kBM * (kBN + 4) * 4) + 255) & ~255;
// Block-scaled gate: a W stage holds 256 rows of 64 k codes (32 bytes of
// MXFP4, 64 of MXFP8) and a scale stage one dword per expert (the aligned
// dword holding the stage's two block scales); the X ring is unchanged.
template <int kFmt> constexpr int kCodeRowBytes = kFmt == kGateMxfp8 ? kBK : kBK / 2;
template <int kFmt> constexpr int kWStageBytesOf = kFmt == kGateBf16 ? kWStageBytes : kBN * kCodeRowBytes<kFmt>;
constexpr int kSStageBytes = kBN * 4;                            // 1 KiB
constexpr int kSRingOffset = kWRingOffset + kWSlots * kWStageBytesOf<kGateMxfp8>;
static_assert(kSRingOffset + kWSlots * kSStageBytes <= kRingBytes, "block-scaled rings fit the LDS ring");
static_assert(kTileBytes <= kFlagOffset, "row tile and flag overlap");
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------------------
// LDS ring: direct-to-LDS loads
// ---------------------------------------------------------------------------
// Staged rows hold 8 chunks of 16 bytes (8 bf16 of k).  Chunk c of row R sits
// in slot c ^ (R mod 8).  Measured on gfx950 with the fragment reads of the
// main loop (16 consecutive rows x 4 chunks per ds_read_b128): this layout
// reads at the LDS's full 256 bytes per clock with no bank conflicts, where
// the swizzle c ^ ((R ^ R/8) mod 8) took 1.7x as long.
__device__ __forceinline__ int slot_swizzle(int R) { return R & 7; }

// The block-scaled gates read X with the k order of their B fragments (lane
// group g takes k = 16 g + 8 kk + 0..7 in MFMA step kk, so that its codes for
// both steps are contiguous): A chunk 2 g + kk instead of 4 kk + g.  For that
// pattern c ^ ((R ^ R/8) mod 8) is the conflict-free slot (measured, as above).
template <int kFmt>
__device__ __forceinline__ int x_swizzle(int R) { return kFmt == kGateBf16 ? slot_swizzle(R) : (R ^ (R >> 3)) & 7; }

constexpr int kOutOfRange = 0x7ffffff0;  // past every descriptor limit: loads read zeros

// Code rows hold 16-byte chunks: MXFP4 two (one 32-block each), MXFP8 four
// (16 k each).  Chunk c of row R sits in physical chunk c ^ sw(R); the swizzles
// are the ones measured fastest for the fragment reads below (one ds_read_b64
// of 16 MXFP4 codes, one ds_read_b128 of 16 MXFP8 codes, per expert row and
// stage): 7.1 and 3.9 clocks per read per CU.
__device__ __forceinline__ int half_swizzle(int R) { return (R >> 3) & 1; }     // MXFP4, 32-byte rows
__device__ __forceinline__ int quarter_swizzle(int R) { return (R >> 1) & 3; }  // MXFP8, 64-byte rows

// A lane's block-scaled codes for one stage: MXFP4 16 codes in two dwords,
// MXFP8 16 codes in four (unused for bf16).
template <int kFmt> struct BStage { using type = u32x4; };
template <> struct BStage<kGateMxfp4> { using type = u32x2; };

// A 1 KiB direct-to-LDS block b of a bf16 stage fills row R = 8b + i/8 with
// lane i, at slot i%8, so lane i fetches chunk (i%8) ^ sw(R) of that row;
// code blocks hold 32 (MXFP4) or 16 (MXFP8) rows the same way.  Chunks at or
// past H take the out-of-range offset and land as zeros; so do rows at or past
// M (X limit) and E (W limit).
//
// One 1 KiB direct-to-LDS load (lane i's 16 bytes to lds + 16 i).  Written as
// inline asm so that the compiler does not track it: its waitcnt pass would
// otherwise wait for every such load in flight before any LDS read, since it
// cannot tell the ring stages apart.  The ring waits for these loads itself
// (explicit vmcnt) before the barrier that publishes a stage.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int byte_off, unsigned char* lds)
{
    const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_void*)lds);
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(byte_off), "s"(r), "{m0}"(m0) : "memory");
}

// One 256-byte direct-to-LDS dword load (lane i's 4 bytes to lds + 4 i).
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, int byte_off, unsigned char* lds)
{
    const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_void*)lds);
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(byte_off), "s"(r), "{m0}"(m0) : "memory");
}

// Workgroup barrier for the LDS ring.  Each wave has already waited (vmcnt)
// for its own loads of the stage about to be read, and its MFMAs have
// consumed every LDS read of the previous stage, so the hardware barrier is
// all that is needed; the empty asm statements stop the compiler from moving
// memory accesses across it.  (A __syncthreads() here would also wait for the
// loads still in flight for the next stages.)
__device__ __forceinline__ void ring_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Byte offset of the published partial of split s, tile-local row r, column
// e: layout [tile][s][row][256] fp32 (at most 32 MiB).
__device__ __forceinline__ int partial_off(const PrefillLaunch& p, int tile, int s, int r, int e)
{
    return ((((tile * p.S + s) * kBM + r) * kBN) + e) * 4;
}

constexpr int kRowGroup = 4;  // rows a wave routes in lockstep (route_rows)
static_assert(kSelOffset + kWaves * kRowGroup * kFilterSlots * 8 <= kFlagOffset, "selection scratch and flag overlap");

// Route rows [r_begin, r_end) of the LDS tile (local row indices): wave w
// takes rows w, w+8, ... in groups of kRowGroup routed together.
__device__ __forceinline__ uint64_t* wave_sel(float* tile_f, int wave)
{
    return reinterpret_cast<uint64_t*>(reinterpret_cast<unsigned char*>(tile_f) + kSelOffset) +
           wave * kRowGroup * kFilterSlots;
}

__device__ __forceinline__ void route_tile_rows(const PrefillLaunch& p, float* tile,
                                                int64_t row0, int r_begin, int r_end, int wave,
                                                int lane, const float (&bv)[kPerLane], const Exp2Lane& et)
{
    const RowSpec spec{p.E, p.k, p.scoring, p.renorm, p.bias != nullptr};
    const int col = lane * kPerLane;
    for (int t0 = r_begin + wave; t0 < r_end && row0 + t0 < p.M; t0 += kWaves * kRowGroup) {
        float v[kRowGroup][kPerLane];
#pragma unroll
        for (int g = 0; g < kRowGroup; ++g) {
            const int t = t0 + g * kWaves;
#pragma unroll
            for (int j = 0; j < kPerLane; ++j)
                v[g][j] = (t < r_end && col + j < p.E) ? tile[t * kTileStride + col + j] : 0.f;
        }
        RowResult res[kRowGroup];
        route_rows<kRowGroup, kFilter>(v, bv, spec, res, wave_sel(tile, wave), et);
#pragma unroll
        for (int g = 0; g < kRowGroup; ++g) {
            const int t = t0 + g * kWaves;
            if (t >= r_end || row0 + t >= p.M) continue;
            if (lane < p.k) {
                p.inds[(row0 + t) * p.k + lane] = res[g].idx;
                p.weights[(row0 + t) * p.k + lane] = res[g].w;
            }
            if (p.logits_out) {
#pragma unroll
                for (int j = 0; j < kPerLane; ++j)
                    if (col + j < p.E) p.logits_out[(row0 + t) * p.E + col + j] = v[g][j];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// split exchange (S = 2, 4, 8 or 16 splits of one 128-row tile)
// ---------------------------------------------------------------------------
// Sum every split's partial of tile-local rows [r0, r0 + rows) in split order
// into the LDS tile (hand-over path: all splits published these rows).
template <int S>
__device__ __forceinline__ void pf_gather_rows(const PrefillLaunch& p, float* tile_f, int tile, int r0,
                                               int rows, int tid)
{
    constexpr int kVecPerRow = kBN / 4;
    const __amdgpu_buffer_rsrc_t prs = coherent_rsrc(p.partials);
    for (int it = tid; it < rows * kVecPerRow; it += kThreads) {
        const int r = r0 + it / kVecPerRow, col = (it % kVecPerRow) * 4;
        f32x4 part[S];
#pragma unroll
        for (int q = 0; q < S; ++q) part[q] = fetch4(prs, partial_off(p, tile, q, r, col));
        f32x4 sum = part[0];
#pragma unroll
        for (int q = 1; q < S; ++q) sum += part[q];
        *reinterpret_cast<f32x4*>(&tile_f[r * kTileStride + col]) = sum;
    }
}

// Route own rows from the exchange: wave w takes rows w, w+8, ... of
// [r0, r0 + rows) in groups of four (at S = 4 a split owns 32 rows, one group
// per wave; with more, the next group's loads are issued before the current
// one is routed, so the reads overlap routing); lane L reads the other
// splits' partials of experts 4L..4L+3 of the group's rows, adds them to its
// own partials from LDS in split order, and the group is routed in lockstep.
// Every split's partials are complete (each waited for its stores before
// counting itself in).
template <int S>
__device__ __forceinline__ void pf_route_own_rows(const PrefillLaunch& p, float* tile_f, int tile,
                                                  int s, int64_t row0, int r0, int rows, int wave,
                                                  int lane, const float (&bv)[kPerLane], const Exp2Lane& et)
{
    const __amdgpu_buffer_rsrc_t prs = coherent_rsrc(p.partials);
    const RowSpec spec{p.E, p.k, p.scoring, p.renorm, p.bias != nullptr};
    const int col = lane * kPerLane;
    const int r_end = r0 + rows;
    if constexpr (S >= 8) {
        // 16 or 8 own rows: wave w takes rows w and w + 8 (two in lockstep)
        // or w alone, every other split's partial of them loaded at once
        constexpr int G = kBM / S / kWaves;
        static_assert(G >= 1 && G <= kRowGroup, "rows per wave");
        f32x4 part[G][S];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int t = r0 + wave + g * kWaves;
#pragma unroll
            for (int q = 0; q < S; ++q)
                if (q != s && t < r_end) part[g][q] = fetch4(prs, partial_off(p, tile, q, t, col));
        }
        float v[G][kPerLane];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int t = r0 + wave + g * kWaves;
            if (t >= r_end) {
#pragma unroll
                for (int j = 0; j < kPerLane; ++j) v[g][j] = 0.f;
                continue;
            }
            const f32x4 mine = *reinterpret_cast<const f32x4*>(&tile_f[t * kTileStride + col]);
            f32x4 sum = (s == 0) ? mine : part[g][0];
#pragma unroll
            for (int q = 1; q < S; ++q) sum += (q == s) ? mine : part[g][q];
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) v[g][j] = col + j < p.E ? sum[j] : 0.f;
            if (p.logits_out && row0 + t < p.M) {
#pragma unroll
                for (int j = 0; j < kPerLane; ++j)
                    if (col + j < p.E) p.logits_out[(row0 + t) * p.E + col + j] = v[g][j];
            }
        }
        RowResult res[G];
        route_rows<G, kFilter>(v, bv, spec, res, wave_sel(tile_f, wave), et);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int t = r0 + wave + g * kWaves;
            if (t >= r_end || row0 + t >= p.M || lane >= p.k) continue;
            p.inds[(row0 + t) * p.k + lane] = res[g].idx;
            p.weights[(row0 + t) * p.k + lane] = res[g].w;
        }
        return;
    }
    constexpr int G = 4;
    f32x4 cur[G][S], nxt[G][S];
    auto issue = [&](int t0, f32x4 (&dst)[G][S]) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int t = t0 + g * kWaves;
#pragma unroll
            for (int q = 0; q < S; ++q)
                if (q != s && t < r_end) dst[g][q] = fetch4(prs, partial_off(p, tile, q, t, col));
        }
    };
    if (r0 + wave < r_end) issue(r0 + wave, cur);
    for (int t0 = r0 + wave; t0 < r_end; t0 += kWaves * G) {
        if (t0 + kWaves * G < r_end) issue(t0 + kWaves * G, nxt);
        float v[G][kPerLane];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int t = t0 + g * kWaves;
            if (t >= r_end) {
#pragma unroll
                for (int j = 0; j < kPerLane; ++j) v[g][j] = 0.f;
                continue;
            }
            const f32x4 mine = *reinterpret_cast<const f32x4*>(&tile_f[t * kTileStride + col]);
            f32x4 sum = (s == 0) ? mine : cur[g][0];
#pragma unroll
            for (int q = 1; q < S; ++q) sum += (q == s) ? mine : cur[g][q];
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) v[g][j] = col + j < p.E ? sum[j] : 0.f;
            if (p.logits_out && row0 + t < p.M) {
#pragma unroll
                for (int j = 0; j < kPerLane; ++j)
                    if (col + j < p.E) p.logits_out[(row0 + t) * p.E + col + j] = v[g][j];
            }
        }
        RowResult res[G];
        static_assert(G == kRowGroup, "selection scratch holds kRowGroup rows per wave");
        route_rows<G, kFilter>(v, bv, spec, res, wave_sel(tile_f, wave), et);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int t = t0 + g * kWaves;
            if (t >= r_end || row0 + t >= p.M || lane >= p.k) continue;
            p.inds[(row0 + t) * p.k + lane] = res[g].idx;
            p.weights[(row0 + t) * p.k + lane] = res[g].w;
        }
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int q = 0; q < S; ++q) cur[g][q] = nxt[g][q];
    }
}

// Split s owns tile rows [s*128/S, (s+1)*128/S).  It publishes every other
// row of its partial tile (device-coherent stores, all issued before the
// wait for them), takes a ticket on the tile's arrival counter and waits a
// bounded time for all S tickets; its own rows' partials are then complete
// and it routes them straight from the exchange (pf_route_own_rows).  If
// the wait times out (a sibling not resident yet), it publishes its own rows
// too, flags them abandoned and moves on; the split that draws the last
// ticket on the tile's done counter routes every abandoned row set and
// resets the counters.  No workgroup waits without a bound, and every logit
// is summed in the same split order whichever path produces it.
template <int S>
__device__ __forceinline__ void exchange_and_route(const PrefillLaunch& p, float* tile_f, int& flag,
                                                   int tile, int s, int64_t row0, int tid, int wave,
                                                   int lane, const float (&bv)[kPerLane], const Exp2Lane& et)
{
    constexpr int kRowsPer = kBM / S;
    constexpr int kVecPerRow = kBN / 4;
    constexpr int kPubCells = (kBM - kRowsPer) * kVecPerRow / kThreads;  // 8, 12, 14, 15 (S = 2..16)
    static_assert((kBM - kRowsPer) * kVecPerRow % kThreads == 0, "published cells per thread");
    const int my_r0 = s * kRowsPer;
    uint32_t* arrive = p.counters + tile * kPrefillCountersPerTile;
    uint32_t* done = arrive + 1;
    uint32_t* abandoned = arrive + 2;  // one flag per split
    const __amdgpu_buffer_rsrc_t prs = coherent_rsrc(p.partials);

    // publish the rows the other splits own (LDS reads first, then stores)
    {
        f32x4 val[kPubCells];
        int off[kPubCells];
#pragma unroll
        for (int c = 0; c < kPubCells; ++c) {
            const int it = tid + c * kThreads;
            const int rn = it / kVecPerRow, col = (it % kVecPerRow) * 4;
            const int r = rn < my_r0 ? rn : rn + kRowsPer;
            val[c] = *reinterpret_cast<const f32x4*>(&tile_f[r * kTileStride + col]);
            off[c] = partial_off(p, tile, s, r, col);
        }
#pragma unroll
        for (int c = 0; c < kPubCells; ++c) publish4(prs, off[c], val[c]);
    }
    __builtin_amdgcn_s_waitcnt(0);  // every published store has completed
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int ok = 1;
        if (prev != (uint32_t)S - 1u) {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (__hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)S) {
                if (__builtin_amdgcn_s_memrealtime() - t0 >= (uint64_t)p.spin_ticks) {
                    ok = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        flag = ok;
    }
    __syncthreads();
    const bool ok = flag != 0;
    __syncthreads();
    if (!ok) {
        // give up: publish my own rows too and mark them abandoned
        for (int it = tid; it < kRowsPer * kVecPerRow; it += kThreads) {
            const int r = my_r0 + it / kVecPerRow, col = (it % kVecPerRow) * 4;
            publish4(prs, partial_off(p, tile, s, r, col),
                     *reinterpret_cast<const f32x4*>(&tile_f[r * kTileStride + col]));
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            __hip_atomic_store(abandoned + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(0);  // the flag is visible before the done ticket
        }
    }

    // The done ticket is drawn before routing; its result is needed only after.
    uint32_t prev = 0;
    if (tid == 0) prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (ok) pf_route_own_rows<S>(p, tile_f, tile, s, row0, my_r0, kRowsPer, wave, lane, bv, et);
    __syncthreads();
    if (tid == 0) flag = (prev == (uint32_t)S - 1u);
    __syncthreads();
    if (!flag) return;

    // ---- last split: every split has published all it will, with its
    // stores complete; route every abandoned row set, then reset the counters
    for (int q = 0; q < S; ++q) {
        if (__hip_atomic_load(abandoned + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) continue;
        __syncthreads();
        pf_gather_rows<S>(p, tile_f, tile, q * kRowsPer, kRowsPer, tid);
        __syncthreads();
        route_tile_rows(p, tile_f, row0, q * kRowsPer, (q + 1) * kRowsPer, wave, lane, bv, et);
        if (tid == 0) __hip_atomic_store(abandoned + q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) {
        __hip_atomic_store(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Role-split GEMM: waves 4..7 only issue the ring's direct-to-LDS loads (and
// wait for them), so that only they ever queue on the memory pipeline; waves
// 0..3 only read fragments and multiply, each a 64 x 128 block (4 x 8 MFMA
// 16x16 accumulators).  The epilogue is the one above.
template <int kFmt>
__global__ __launch_bounds__(kThreads) void prefill_router_kernel(PrefillLaunch p)
{
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
    int& flag = *reinterpret_cast<int*>(lds + kFlagOffset);
    float* tile_f = reinterpret_cast<float*>(lds);

    constexpr bool kMx = kFmt != kGateBf16;
    constexpr int kWStage = kWStageBytesOf<kFmt>;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const bool producer = wave >= 4;
    const int cw = wave & 3;
    const int wm = cw >> 1;  // compute: 64-row half
    const int wn = cw & 1;   // compute: 128-expert half

    const int xcd = blockIdx.x % kXcds;
    const int q8 = blockIdx.x / kXcds;
    const int s = q8 % p.S;
    const int tile = xcd + kXcds * (q8 / p.S);
    const int64_t row0 = (int64_t)tile * kBM;
    if (row0 >= p.M) return;

    const int k_begin = s * p.k_per_split;
    const int k_end = min(p.H, k_begin + p.k_per_split);
    const int nstages = k_end > k_begin ? (k_end - k_begin + kBK - 1) / kBK : 0;

    unsigned char* const xring = lds;
    unsigned char* const wring = lds + kWRingOffset;
    unsigned char* const sring = lds + kSRingOffset;
    const int fr = lane & 15;
    const int g = lane >> 4;

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (producer) {
        // Producer pi fills 1 KiB blocks pi*4 .. pi*4+3 of an X stage and a
        // quarter of each W stage: bf16 blocks pi*8 .. +7; codes blocks
        // pi*2 .. +1 (MXFP4: 32 rows each) or pi*4 .. +3 (MXFP8: 16 rows
        // each), plus the scale dwords of experts 64 pi .. 64 pi + 63.
        constexpr int kPA = 4;
        constexpr int kPB = kFmt == kGateBf16 ? 8 : (kFmt == kGateMxfp4 ? 2 : 4);
        constexpr int kPW = kPB + (kMx ? 1 : 0);  // W-side loads per stage
        constexpr int kPLoads = kPA + kPW;
        const int pi = wave - 4;
        const int64_t rows_here = min((int64_t)kBM, p.M - row0);
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(p.x + row0 * p.H), 0, (int)(rows_here * p.H * 2), 0x00020000);
        __amdgpu_buffer_rsrc_t wr, sr;
        if constexpr (kFmt == kGateBf16)
            wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.w), 0, p.E * p.H * 2, 0x00020000);
        else
            wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.w_codes), 0,
                                                   p.E * (kFmt == kGateMxfp8 ? p.H : p.H / 2), 0x00020000);
        if constexpr (kMx)
            sr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.w_scale), 0, p.E * (p.H / 32), 0x00020000);
        const int li = lane >> 3, ls = lane & 7;
        int a_off[kPA], a_k[kPA], b_off[kPB], b_k[kPB];
#pragma unroll
        for (int j = 0; j < kPA; ++j) {
            const int R = (pi * kPA + j) * 8 + li;
            a_k[j] = (ls ^ x_swizzle<kFmt>(R)) * 8;
            a_off[j] = (R * p.H + a_k[j]) * 2;
        }
#pragma unroll
        for (int j = 0; j < kPB; ++j) {
            const int blk = pi * kPB + j;
            if constexpr (kFmt == kGateBf16) {
                const int R = blk * 8 + li;
                b_k[j] = (ls ^ slot_swizzle(R)) * 8;
                b_off[j] = (R * p.H + b_k[j]) * 2;
            } else if constexpr (kFmt == kGateMxfp4) {
                const int R = blk * 32 + (lane >> 1);
                b_k[j] = ((lane & 1) ^ half_swizzle(R)) * 32;
                b_off[j] = R * (p.H / 2) + b_k[j] / 2;
            } else {
                const int R = blk * 16 + (lane >> 2);
                b_k[j] = ((lane & 3) ^ quarter_swizzle(R)) * 16;
                b_off[j] = R * p.H + b_k[j];
            }
        }
        const int s_off = (pi * 64 + lane) * (p.H / 32);
        auto issue = [&](int j) {
            if (j + 3 >= 0 && j + 3 < nstages) {
                const int k0 = k_begin + (j + 3) * kBK;
                unsigned char* slot = xring + ((j + 3) % kXSlots) * kXStageBytes;
#pragma unroll
                for (int q = 0; q < kPA; ++q)
                    dma16(xr, (k0 + a_k[q] < p.H) ? a_off[q] + k0 * 2 : kOutOfRange, slot + (pi * kPA + q) * 1024);
            }
            if (j + 2 >= 0 && j + 2 < nstages) {
                const int k0 = k_begin + (j + 2) * kBK;
                unsigned char* slot = wring + ((j + 2) % kWSlots) * kWStage;
                constexpr int kDiv = kFmt == kGateBf16 ? 0 : (kFmt == kGateMxfp4 ? 2 : 1);
#pragma unroll
                for (int q = 0; q < kPB; ++q) {
                    int off;
                    if constexpr (kFmt == kGateBf16)
                        off = (k0 + b_k[q] < p.H) ? b_off[q] + k0 * 2 : kOutOfRange;
                    else
                        off = (k0 + b_k[q] < p.H) ? b_off[q] + k0 / kDiv : kOutOfRange;
                    dma16(wr, off, slot + (pi * kPB + q) * 1024);
                }
                if constexpr (kMx)  // the stage's two scales lie in the aligned dword at k0 / 32 & ~3
                    dma4(sr, s_off + ((k0 >> 5) & ~3), sring + ((j + 2) % kWSlots) * kSStageBytes + pi * 256);
            }
        };
        issue(-3);
        issue(-2);
        issue(-1);
        for (int ks = 0; ks < nstages; ++ks) {
            if (ks + 2 < nstages)
                __builtin_amdgcn_s_waitcnt(0x0F70 | kPLoads);  // iteration ks-1's loads may be in flight
            else if (ks + 1 < nstages)
                __builtin_amdgcn_s_waitcnt(0x0F70 | kPW);      // only W[ks+1] after W[ks]
            else
                __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0)
            ring_barrier();
            issue(ks);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);
    } else {
        int a_row[4], b_row[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) a_row[i] = wm * 64 + i * 16 + fr;
#pragma unroll
        for (int j = 0; j < 8; ++j) b_row[j] = wn * 128 + j * 16 + fr;
        for (int ks = 0; ks < nstages; ++ks) {
            ring_barrier();
            const unsigned char* xs = xring + (ks % kXSlots) * kXStageBytes;
            const unsigned char* ws = wring + (ks % kWSlots) * kWStage;
            if constexpr (!kMx) {
                bf16x8 af[2][4], bf[2][8];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int c = kk * 4 + g;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        af[kk][i] = *reinterpret_cast<const bf16x8*>(xs + a_row[i] * kRowBytes +
                                                                     ((c ^ slot_swizzle(a_row[i])) << 4));
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        bf[kk][j] = *reinterpret_cast<const bf16x8*>(ws + b_row[j] * kRowBytes +
                                                                     ((c ^ slot_swizzle(b_row[j])) << 4));
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kk][i], bf[kk][j], acc[i][j], 0, 0, 0);
            } else {
                // block-scaled: k of lane group g in step kk is 16 g + 8 kk + 0..7
                // (both operands); a row's 16 codes of the stage are read once
                const unsigned char* ss =
                    sring + (ks % kWSlots) * kSStageBytes + (((k_begin + ks * kBK) >> 5) & 3);
                typename BStage<kFmt>::type braw[8];
                float bscale[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if constexpr (kFmt == kGateMxfp4)
                        braw[j] = *reinterpret_cast<const u32x2*>(ws + b_row[j] * (kBK / 2) +
                                                                  (((g >> 1) ^ half_swizzle(b_row[j])) << 4) + 8 * (g & 1));
                    else
                        braw[j] = *reinterpret_cast<const u32x4*>(ws + b_row[j] * kBK +
                                                                  ((g ^ quarter_swizzle(b_row[j])) << 4));
                    bscale[j] = __uint_as_float((uint32_t)ss[b_row[j] * 4 + (g >> 1)] << 23);
                }
                bf16x8 af[2][4];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        af[kk][i] = *reinterpret_cast<const bf16x8*>(xs + a_row[i] * kRowBytes +
                                                                     (((2 * g + kk) ^ x_swizzle<kFmt>(a_row[i])) << 4));
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        bf16x8 b;
                        if constexpr (kFmt == kGateMxfp4)
                            b = fp4x8_to_bf16x8(braw[j][kk], bscale[j]);
                        else
                            b = fp8x8_to_bf16x8(braw[j][2 * kk], braw[j][2 * kk + 1], bscale[j]);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kk][i], b, acc[i][j], 0, 0, 0);
                    }
                }
            }
        }
    }
    __syncthreads();  // every wave is done with the ring before it becomes the row tile

    if (!producer) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    tile_f[(wm * 64 + i * 16 + 4 * g + q) * kTileStride + wn * 128 + j * 16 + fr] = acc[i][j][q];
    }
    __syncthreads();

    float bv[kPerLane] = {0.f, 0.f, 0.f, 0.f};
    if (p.bias) {
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane * kPerLane + j;
            if (e < p.E) bv[j] = p.bias[e];
        }
    }
    const Exp2Lane et = load_exp2_lane();
    if (p.S == 1) {
        route_tile_rows(p, tile_f, row0, 0, kBM, wave, lane, bv, et);
        return;
    }
    if (p.S == 16)
        exchange_and_route<16>(p, tile_f, flag, tile, s, row0, tid, wave, lane, bv, et);
    else if (p.S == 8)
        exchange_and_route<8>(p, tile_f, flag, tile, s, row0, tid, wave, lane, bv, et);
    else if (p.S == 4)
        exchange_and_route<4>(p, tile_f, flag, tile, s, row0, tid, wave, lane, bv, et);
    else
        exchange_and_route<2>(p, tile_f, flag, tile, s, row0, tid, wave, lane, bv, et);
}

}  // namespace

// K splits per tile: as many as keep (tiles, padded to the 8 XCDs) x splits
// within the 256 (tile, split) pairs of the exchange buffer, so few tiles
// still fill the CUs.
int prefill_splits(int64_t M)
{
    const int64_t tiles = (M + kBM - 1) / kBM;
    const int64_t padded = (tiles + kXcds - 1) / kXcds * kXcds;
    for (int S = 16; S >= 2; S /= 2)
        if (padded * S <= kPrefillMaxPairs) return S;
    return 1;
}

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream)
{
    if (a.M <= 0) return hipSuccess;
    const int64_t tiles = (a.M + kBM - 1) / kBM;
    const int64_t padded = (tiles + kXcds - 1) / kXcds * kXcds;
    const int64_t blocks = padded * a.S;
    if (a.w_format == kGateMxfp4)
        hipLaunchKernelGGL(prefill_router_kernel<kGateMxfp4>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    else if (a.w_format == kGateMxfp8)
        hipLaunchKernelGGL(prefill_router_kernel<kGateMxfp8>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    else if (a.w_format == kGateBf16)
        hipLaunchKernelGGL(prefill_router_kernel<kGateBf16>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace gpt
