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
// a tile is split S ways (S = 4 for <= 64 tiles): S workgroups of 8 waves
// each compute the tile's 128 x 256 partial over their K slice.  Each wave
// owns a 64 x 64 block as 4 x 4 MFMA 16x16x32 accumulators.  K is staged
// through a three-deep LDS ring in 64-wide steps by direct-to-LDS buffer
// loads (no staging registers; 8 consecutive lanes read one row's 128
// contiguous bytes), and the MFMA operands are read back from LDS through an
// XOR slot swizzle that keeps fragment reads free of bank conflicts.
//
// Split exchange.  Split s owns rows [s*128/S, (s+1)*128/S) for the
// epilogue.  It publishes the rows it does not own (device-coherent stores),
// takes a ticket on the tile's arrival counter, waits a bounded time for all
// S tickets, then sums the S partials of its rows in split order (its own from
// LDS) and routes them.  If the wait times out (other splits not resident),
// it publishes its own rows, marks them abandoned and leaves; the split that
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
constexpr int kBN = kMaxE;                  // 256
constexpr int kBK = 64;                     // k per stage: one 128-byte segment per row
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;    // 512
constexpr int kNStage = 3;                  // LDS ring depth (two stages in flight)
constexpr int kRowBytes = kBK * 2;
constexpr int kStageABytes = kBM * kRowBytes;             // 16 KiB
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;      // 48 KiB
constexpr int kDmaA = kBM / 8 / kWaves;                   // 1 KiB DMA blocks per wave: 2
constexpr int kDmaB = kBN / 8 / kWaves;                   // 4
constexpr int kTileStride = kBN + 4;        // fp32 per row of the epilogue tile
constexpr int kTileBytes = kBM * kTileStride * 4;
constexpr int kRingBytes = kNStage * kStageBytes;
constexpr int kLdsBytes = kRingBytes > kTileBytes ? kRingBytes : kTileBytes;

typedef __attribute__((address_space(3))) void lds_void;

// ---------------------------------------------------------------------------
// LDS ring: direct-to-LDS loads
// ---------------------------------------------------------------------------
// Staged rows hold 8 chunks of 16 bytes (8 bf16 of k).  Chunk c of row R sits
// in slot c ^ sw(R): rows 8 apart and rows 1 apart land on different bank
// groups, so the 16 rows an MFMA fragment read touches at one k never collide.
__device__ __forceinline__ int slot_swizzle(int R) { return (R ^ (R >> 3)) & 7; }

constexpr int kOutOfRange = 0x7ffffff0;  // past every descriptor limit: loads read zeros

// Lane i of a 1 KiB block b fills row R = 8b + i/8, slot i%8, so it fetches
// chunk (i%8) ^ sw(R) of that row.  Chunks at or past H take the
// out-of-range offset and land as zeros; so do rows at or past M (X limit)
// and E (W limit).
struct DmaPlan {
    __amdgpu_buffer_rsrc_t x;  // this tile's rows of X
    __amdgpu_buffer_rsrc_t w;  // all of W
    int a_off[kDmaA], a_k[kDmaA];
    int b_off[kDmaB], b_k[kDmaB];
};

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

__device__ __forceinline__ void issue_stage(const DmaPlan& d, unsigned char* stage, int k0, int H,
                                            int wave)
{
#pragma unroll
    for (int j = 0; j < kDmaA; ++j) {
        const int off = (k0 + d.a_k[j] < H) ? d.a_off[j] + k0 * 2 : kOutOfRange;
        dma16(d.x, off, stage + (wave * kDmaA + j) * 1024);
    }
#pragma unroll
    for (int j = 0; j < kDmaB; ++j) {
        const int off = (k0 + d.b_k[j] < H) ? d.b_off[j] + k0 * 2 : kOutOfRange;
        dma16(d.w, off, stage + kStageABytes + (wave * kDmaB + j) * 1024);
    }
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

// Route rows [r_begin, r_end) of the LDS tile (local row indices); one wave per row.
__device__ __forceinline__ void route_tile_rows(const PrefillLaunch& p, const float* tile,
                                                int64_t row0, int r_begin, int r_end, int wave,
                                                int lane, const float (&bv)[kPerLane])
{
    const RowSpec spec{p.E, p.k, p.scoring, p.renorm, p.bias != nullptr};
    for (int t = r_begin + wave; t < r_end; t += kWaves) {
        if (row0 + t >= p.M) break;
        float v[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane * kPerLane + j;
            v[j] = e < p.E ? tile[t * kTileStride + e] : 0.f;
        }
        const RowResult res = route_row(v, bv, spec);
        if (lane < p.k) {
            const int64_t o = (row0 + t) * p.k + lane;
            p.inds[o] = res.idx;
            p.weights[o] = res.w;
        }
        if (p.logits_out) {
#pragma unroll
            for (int j = 0; j < kPerLane; ++j) {
                const int e = lane * kPerLane + j;
                if (e < p.E) p.logits_out[(row0 + t) * p.E + e] = v[j];
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void prefill_router_kernel(PrefillLaunch p)
{
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsBytes];
    __shared__ int flag;

    float* tile_f = reinterpret_cast<float*>(lds);

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wm = wave >> 2;  // 0..1: 64-row half of the tile
    const int wn = wave & 3;   // 0..3: 64-expert quarter

    const int s = blockIdx.x % p.S;
    const int tile = blockIdx.x / p.S;
    const int64_t row0 = (int64_t)tile * kBM;

    const int k_begin = s * p.k_per_split;
    const int k_end = min(p.H, k_begin + p.k_per_split);
    const int nstages = k_end > k_begin ? (k_end - k_begin + kBK - 1) / kBK : 0;

    // ---- GEMM over this split's K range
    f32x4 acc[4][4];  // wave tile 64 x 64: 4 x 4 MFMA 16x16 blocks
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int fr = lane & 15;  // fragment row / column
    const int g = lane >> 4;   // this lane's 16-byte chunk inside a 32-wide k step

    DmaPlan d;
    {
        const int64_t rows_here = min((int64_t)kBM, p.M - row0);
        d.x = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.x + row0 * p.H), 0,
                                                (int)(rows_here * p.H * 2), 0x00020000);
        d.w = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.w), 0, p.E * p.H * 2, 0x00020000);
        const int li = lane >> 3, ls = lane & 7;
#pragma unroll
        for (int j = 0; j < kDmaA; ++j) {
            const int R = (wave * kDmaA + j) * 8 + li;
            d.a_k[j] = (ls ^ slot_swizzle(R)) * 8;
            d.a_off[j] = (R * p.H + d.a_k[j]) * 2;
        }
#pragma unroll
        for (int j = 0; j < kDmaB; ++j) {
            const int R = (wave * kDmaB + j) * 8 + li;
            d.b_k[j] = (ls ^ slot_swizzle(R)) * 8;
            d.b_off[j] = (R * p.H + d.b_k[j]) * 2;
        }
    }
    // Fragment read addresses: row R, chunk c -> R * 128 + (c ^ sw(R)) * 16.
    int a_row[4], b_row[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a_row[i] = wm * 64 + i * 16 + fr;
        b_row[i] = wn * 64 + i * 16 + fr;
    }

    // Three-stage ring: while stage ks is multiplied, stages ks+1 and ks+2
    // are in flight.
    if (nstages > 0) issue_stage(d, lds, k_begin, p.H, wave);
    if (nstages > 1) issue_stage(d, lds + kStageBytes, k_begin + kBK, p.H, wave);
    for (int ks = 0; ks < nstages; ++ks) {
        // stage ks has landed once at most the next stage's loads are outstanding
        if (ks + 1 < nstages)
            __builtin_amdgcn_s_waitcnt(0x0F70 | (kDmaA + kDmaB));  // vmcnt(6)
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);                    // vmcnt(0)
        ring_barrier();
        if (ks + 2 < nstages)
            issue_stage(d, lds + ((ks + 2) % kNStage) * kStageBytes, k_begin + (ks + 2) * kBK, p.H, wave);
        const unsigned char* cur = lds + (ks % kNStage) * kStageBytes;
#pragma unroll
        for (int kk = 0; kk < kBK / 32; ++kk) {
            const int c = kk * 4 + g;
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(cur + a_row[i] * kRowBytes +
                                                          ((c ^ slot_swizzle(a_row[i])) << 4));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(cur + kStageABytes + b_row[j] * kRowBytes +
                                                           ((c ^ slot_swizzle(b_row[j])) << 4));
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no ring load still in flight
    __syncthreads();  // every wave is done with the ring before it becomes the row tile

    // ---- accumulators -> fp32 row tile in LDS (reuses the ring)
    // MFMA 16x16 layout: lane holds rows 4*(lane/16)+q of the tile, column lane%16.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                tile_f[(wm * 64 + i * 16 + 4 * g + q) * kTileStride + wn * 64 + j * 16 + fr] = acc[i][j][q];
    __syncthreads();

    float bv[kPerLane] = {0.f, 0.f, 0.f, 0.f};
    if (p.bias) {
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane * kPerLane + j;
            if (e < p.E) bv[j] = p.bias[e];
        }
    }

    if (p.S == 1) {
        route_tile_rows(p, tile_f, row0, 0, kBM, wave, lane, bv);
        return;
    }

    // ---- split exchange
    const int rows_per = kBM / p.S;
    const int my_r0 = s * rows_per;
    uint32_t* arrive = p.counters + tile * kPrefillCountersPerTile;
    uint32_t* done = arrive + 1;
    uint32_t* abandoned = arrive + 2;  // one flag per split
    const __amdgpu_buffer_rsrc_t prs = coherent_rsrc(p.partials);
    constexpr int kVecPerRow = kBN / 4;  // 64 float4 per row

    // publish the rows owned by the other splits
    for (int it = tid; it < kBM * kVecPerRow; it += kThreads) {
        const int r = it / kVecPerRow;
        const int c = (it % kVecPerRow) * 4;
        if (r >= my_r0 && r < my_r0 + rows_per) continue;
        publish4(prs, partial_off(p, tile, s, r, c), *reinterpret_cast<const f32x4*>(&tile_f[r * kTileStride + c]));
    }
    __builtin_amdgcn_s_waitcnt(0);  // every published store has completed
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        int ok = 1;
        if (prev != (uint32_t)p.S - 1u) {
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (__hip_atomic_load(arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)p.S) {
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

    if (flag) {
        // sum the S partials of my rows in split order (mine from LDS)
        constexpr int kItems = 4;  // float4 cells per thread per batch
        const int items = rows_per * kVecPerRow;
        for (int base = tid; base < items; base += kThreads * kItems) {
            f32x4 part[kItems][4];
#pragma unroll
            for (int u = 0; u < kItems; ++u) {
                const int it = base + u * kThreads;
                const int r = my_r0 + it / kVecPerRow;
                const int c = (it % kVecPerRow) * 4;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    part[u][q] = f32x4{0.f, 0.f, 0.f, 0.f};
                    if (it < items && q < p.S && q != s) part[u][q] = fetch4(prs, partial_off(p, tile, q, r, c));
                }
            }
#pragma unroll
            for (int u = 0; u < kItems; ++u) {
                const int it = base + u * kThreads;
                if (it < items) {
                    const int r = my_r0 + it / kVecPerRow;
                    const int c = (it % kVecPerRow) * 4;
                    f32x4* cell = reinterpret_cast<f32x4*>(&tile_f[r * kTileStride + c]);
                    const f32x4 mine = *cell;
                    f32x4 sum = (s == 0) ? mine : part[u][0];
#pragma unroll
                    for (int q = 1; q < 4; ++q)
                        if (q < p.S) sum += (q == s) ? mine : part[u][q];
                    *cell = sum;
                }
            }
        }
        __syncthreads();
        route_tile_rows(p, tile_f, row0, my_r0, my_r0 + rows_per, wave, lane, bv);
    } else {
        // give up: publish my own rows too and mark them abandoned
        for (int it = tid; it < rows_per * kVecPerRow; it += kThreads) {
            const int r = my_r0 + it / kVecPerRow;
            const int c = (it % kVecPerRow) * 4;
            publish4(prs, partial_off(p, tile, s, r, c), *reinterpret_cast<const f32x4*>(&tile_f[r * kTileStride + c]));
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0) {
            __hip_atomic_store(abandoned + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(0);
        }
    }

    // ---- completion: the last split routes abandoned row sets and resets
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        flag = (prev == (uint32_t)p.S - 1u);
    }
    __syncthreads();
    if (!flag) return;
    for (int q = 0; q < p.S; ++q) {
        if (__hip_atomic_load(abandoned + q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) continue;
        const int q_r0 = q * rows_per;
        __syncthreads();
        for (int it = tid; it < rows_per * kVecPerRow; it += kThreads) {
            const int r = q_r0 + it / kVecPerRow;
            const int c = (it % kVecPerRow) * 4;
            f32x4 sum = fetch4(prs, partial_off(p, tile, 0, r, c));
            for (int u = 1; u < p.S; ++u) sum += fetch4(prs, partial_off(p, tile, u, r, c));
            *reinterpret_cast<f32x4*>(&tile_f[r * kTileStride + c]) = sum;
        }
        __syncthreads();
        route_tile_rows(p, tile_f, row0, q_r0, q_r0 + rows_per, wave, lane, bv);
        if (tid == 0) __hip_atomic_store(abandoned + q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (tid == 0) {
        __hip_atomic_store(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

}  // namespace

int prefill_splits(int64_t M)
{
    const int64_t tiles = (M + kBM - 1) / kBM;
    if (tiles <= kPrefillMaxPairs / 4) return 4;
    if (tiles <= kPrefillMaxPairs / 2) return 2;
    return 1;
}

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream)
{
    if (a.M <= 0) return hipSuccess;
    const int64_t tiles = (a.M + kBM - 1) / kBM;
    const int64_t blocks = tiles * a.S;
    hipLaunchKernelGGL(prefill_router_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gpt
