// Fused prefill router (M > 64 tokens): a bf16 MFMA GEMM whose epilogue does
// scoring, top-k and renormalisation per row from LDS, so the [M, E] logits
// never travel to HBM (dense_router_decode notes, "DenseRouterDecodeKernel":
// BF16 GEMM with FP32 accumulation and a row-level top-k epilogue rather than
// a per-element one; its TMA/TMEM warp roles have no gfx950 counterpart and
// are not reproduced).
//
// Each workgroup owns 32 complete rows (all E <= 256 experts), so the
// epilogue needs no cross-workgroup exchange.  Four waves; wave w computes the
// 32 x 64 block of experts [64w, 64w+64) as 2 x 4 MFMA 16x16x32 tiles, with
// operands loaded straight from global memory (X rows are shared by the four
// waves through L1, gate rows are each read by one wave) and the next k-steps
// prefetched while the current ones are multiplied.  The accumulators are
// dropped into an LDS row tile and every wave routes 8 rows with the shared
// route_row().
#include "launch.hpp"
#include "route_common.hpp"

namespace gpt {

namespace {

constexpr int kRows = 32;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kChunk = 2;  // k-steps per prefetch batch
constexpr int kRowTiles = kRows / 16;            // 2
constexpr int kColTiles = kMaxE / kWaves / 16;   // 4 tiles of 16 experts per wave
constexpr int kTileStride = kMaxE + 4;           // LDS row stride (floats)

typedef int i32x4 __attribute__((ext_vector_type(4)));

struct Operands {
    bf16x8 a[kChunk][kRowTiles];
    bf16x8 b[kChunk][kColTiles];
};

__device__ __forceinline__ void load_operands(Operands& o, int ks, int KS, int H, int kq,
                                              const uint16_t* const (&xp)[kRowTiles],
                                              const bool (&xok)[kRowTiles],
                                              const uint16_t* const (&wp)[kColTiles],
                                              const bool (&wok)[kColTiles])
{
    const bf16x8 zero = __builtin_bit_cast(bf16x8, i32x4{0, 0, 0, 0});
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
        const int k0 = (ks + c) * 32;
        const bool in = (ks + c) < KS && (k0 + kq) < H;
#pragma unroll
        for (int i = 0; i < kRowTiles; ++i) o.a[c][i] = (in && xok[i]) ? load_bf16x8(xp[i] + k0) : zero;
#pragma unroll
        for (int j = 0; j < kColTiles; ++j) o.b[c][j] = (in && wok[j]) ? load_bf16x8(wp[j] + k0) : zero;
    }
}

__global__ __launch_bounds__(kThreads) void prefill_router_kernel(PrefillLaunch a)
{
    __shared__ float tile[kRows * kTileStride];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int64_t row0 = (int64_t)blockIdx.x * kRows;
    const int kq = (lane >> 4) * 8;

    const uint16_t* xp[kRowTiles];
    bool xok[kRowTiles];
#pragma unroll
    for (int i = 0; i < kRowTiles; ++i) {
        const int64_t row = row0 + i * 16 + (lane & 15);
        xok[i] = row < a.M;
        xp[i] = a.x + (xok[i] ? row : 0) * a.H + kq;
    }
    const uint16_t* wp[kColTiles];
    bool wok[kColTiles];
#pragma unroll
    for (int j = 0; j < kColTiles; ++j) {
        const int e = wave * 64 + j * 16 + (lane & 15);
        wok[j] = e < a.E;
        wp[j] = a.w + (int64_t)(wok[j] ? e : 0) * a.H + kq;
    }

    f32x4 acc[kRowTiles][kColTiles];
#pragma unroll
    for (int i = 0; i < kRowTiles; ++i)
#pragma unroll
        for (int j = 0; j < kColTiles; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KS = (a.H + 31) >> 5;
    Operands cur, nxt;
    load_operands(cur, 0, KS, a.H, kq, xp, xok, wp, wok);
    for (int ks = 0; ks < KS; ks += kChunk) {
        if (ks + kChunk < KS) load_operands(nxt, ks + kChunk, KS, a.H, kq, xp, xok, wp, wok);
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
            if (ks + c < KS) {
#pragma unroll
                for (int i = 0; i < kRowTiles; ++i)
#pragma unroll
                    for (int j = 0; j < kColTiles; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.a[c][i], cur.b[c][j],
                                                                            acc[i][j], 0, 0, 0);
            }
        }
        cur = nxt;
    }

    // accumulators -> LDS row tile: lane holds rows 4*(lane/16)+q, column lane%16
#pragma unroll
    for (int i = 0; i < kRowTiles; ++i)
#pragma unroll
        for (int j = 0; j < kColTiles; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                tile[(i * 16 + 4 * (lane >> 4) + q) * kTileStride + wave * 64 + j * 16 + (lane & 15)] =
                    acc[i][j][q];
    __syncthreads();

    if (a.logits_out) {
        for (int it = tid; it < kRows * a.E; it += kThreads) {
            const int t = it / a.E;
            const int e = it - t * a.E;
            if (row0 + t < a.M) a.logits_out[(row0 + t) * a.E + e] = tile[t * kTileStride + e];
        }
    }

    const RowSpec spec{a.E, a.k, a.scoring, a.renorm, a.bias != nullptr};
    float bv[kPerLane] = {0.f, 0.f, 0.f, 0.f};
    if (a.bias) {
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane * kPerLane + j;
            if (e < a.E) bv[j] = a.bias[e];
        }
    }
    for (int t = wave; t < kRows; t += kWaves) {
        if (row0 + t >= a.M) break;
        float v[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane * kPerLane + j;
            v[j] = e < a.E ? tile[t * kTileStride + e] : 0.f;
        }
        const RowResult res = route_row(v, bv, spec);
        if (lane < a.k) {
            const int64_t o = (row0 + t) * a.k + lane;
            a.inds[o] = res.idx;
            a.weights[o] = res.w;
        }
    }
}

}  // namespace

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream)
{
    if (a.M <= 0) return hipSuccess;
    const int64_t blocks = (a.M + kRows - 1) / kRows;
    hipLaunchKernelGGL(prefill_router_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gpt
