// Fused decode router (M <= 64 tokens): gate projection, scoring, top-k and
// renormalisation in ONE launch (qwisp issue #145, "Change": one kernel from
// postNorm to inds/scores with the E logits held on chip).
//
// The page leaves open how a matvec spread over many workgroups meets a top-k
// that needs the whole logit row in one place (serialise the matvec into one
// threadgroup, or reduce across threadgroups).  Here: reduce across
// workgroups with a last-arriver hand-off, because one CU cannot pull the
// 2-3.5 MiB gate matrix from HBM fast enough on its own.
//
//   grid = R row blocks x B expert blocks x S H-splits, 4 waves each.
//   Phase 1 (every workgroup): the 16x16 (tokens x experts) partial dot
//     products over its H-split, one bf16 MFMA 16x16x32 per 32-wide k-step,
//     the four waves' partials summed in LDS in a fixed order and published
//     with device-coherent stores; then an agent-scope arrival count per row
//     block.
//   Phase 2 (the last workgroup of a row block): sum the S partials
//     of each logit in split order into an LDS row tile (the only place the
//     logits live unless the caller asks for them), route each row with the
//     shared route_row(), and at M=2 emit the unique-route table.  It resets
//     the counter, so the kernel is replayable inside a HIP graph.
//
// Every logit is accumulated in the same order regardless of its expert
// index, so two experts with identical gate rows get bitwise-equal logits and
// the tie goes to the lower index, as the contract requires.
#include "launch.hpp"
#include "route_common.hpp"

namespace gpt {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kChunk = 4;  // k-steps loaded per wave before its MFMAs
constexpr int kItemsPerThread = 4;  // logits gathered per thread per batch in phase 2

typedef int i32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void decode_router_kernel(DecodeLaunch a)
{
    __shared__ float red[kWaves][kDecodeTile][kDecodeTile + 1];
    __shared__ float lrow[kDecodeTile][kMaxE];
    __shared__ int32_t slots[2 * kMaxK];
    __shared__ int is_last;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int B = (a.E + kDecodeTile - 1) / kDecodeTile;

    int bid = blockIdx.x;
    const int s = bid % a.S;
    bid /= a.S;
    const int b = bid % B;
    const int r = bid / B;

    // ---- phase 1: partial logits of 16 tokens x 16 experts over one H-split
    const int arow = r * kDecodeTile + (lane & 15);  // MFMA A row  = token
    const int bcol = b * kDecodeTile + (lane & 15);  // MFMA B col  = expert
    const int kq = (lane >> 4) * 8;                  // this lane's 8 of the 32 k
    const bool arow_ok = arow < a.M;
    const bool bcol_ok = bcol < a.E;
    const uint16_t* xp = a.x + (int64_t)(arow_ok ? arow : 0) * a.H + kq;
    const uint16_t* wp = a.w + (int64_t)(bcol_ok ? bcol : 0) * a.H + kq;

    const int KS = (a.H + 31) >> 5;
    const int ks0 = s * a.ks_per_split;
    const int ks1 = min(KS, ks0 + a.ks_per_split);
    const bf16x8 zero = __builtin_bit_cast(bf16x8, i32x4{0, 0, 0, 0});

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int base = ks0 + wave; base < ks1; base += kWaves * kChunk) {
        bf16x8 av[kChunk], bv[kChunk];
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
            const int ks = base + c * kWaves;
            const int k0 = ks * 32;
            const bool in = ks < ks1 && (k0 + kq) < a.H;
            av[c] = (in && arow_ok) ? load_bf16x8(xp + k0) : zero;
            bv[c] = (in && bcol_ok) ? load_bf16x8(wp + k0) : zero;
        }
#pragma unroll
        for (int c = 0; c < kChunk; ++c)
            if (base + c * kWaves < ks1)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[c], bv[c], acc, 0, 0, 0);
    }

    // MFMA 16x16 result layout: lane holds rows 4*(lane/16)+i, column lane%16.
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * (lane >> 4) + i][lane & 15] = acc[i];
    __syncthreads();

    // ---- hand-off.  Wave 0 alone publishes the workgroup's 16x16 partials
    // with device-coherent (agent-scope) stores, waits until they have
    // completed, then takes a ticket on the row block's arrival counter.  The
    // workgroup that draws the last ticket reads every partial back with
    // device-coherent loads.  No cache-wide writeback or invalidate is needed
    // because the published data never sits in a non-coherent cache line.
    if (wave == 0) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int idx = h * kWave + lane;
            const int rr = idx >> 4, cc = idx & 15;
            const float sum = ((red[0][rr][cc] + red[1][rr][cc]) + red[2][rr][cc]) + red[3][rr][cc];
            const int row = r * kDecodeTile + rr;
            const int e = b * kDecodeTile + cc;
            if (row < a.M && e < a.E)
                __hip_atomic_store(&a.partials[((int64_t)s * a.M + row) * a.E + e], sum,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0);  // every partial store has completed
        if (lane == 0) {
            const uint32_t arrivals = (uint32_t)(B * a.S);
            const uint32_t prev = __hip_atomic_fetch_add(&a.counters[r], 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            is_last = (prev == arrivals - 1u);
        }
    }
    __syncthreads();
    if (!is_last) return;
    if (tid == 0) __hip_atomic_store(&a.counters[r], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // ---- phase 2: full logits of the row block into LDS, then route rows
    // All of a thread's partial loads are issued before any is consumed (one
    // memory round trip per batch instead of one per split); the sum itself
    // runs in split order.
    const int t0 = r * kDecodeTile;
    const int nrows = min(kDecodeTile, a.M - t0);
    const int items = nrows * a.E;
    const int64_t split_stride = (int64_t)a.M * a.E;
    const float* pbase = a.partials + (int64_t)t0 * a.E;
    for (int base = tid; base < items; base += kThreads * kItemsPerThread) {
        float part[kItemsPerThread][kDecodeMaxSplits];
#pragma unroll
        for (int u = 0; u < kItemsPerThread; ++u) {
            const int it = base + u * kThreads;
#pragma unroll
            for (int q = 0; q < kDecodeMaxSplits; ++q)
                part[u][q] = (it < items && q < a.S)
                                 ? __hip_atomic_load(pbase + q * split_stride + it, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                                 : 0.f;
        }
#pragma unroll
        for (int u = 0; u < kItemsPerThread; ++u) {
            const int it = base + u * kThreads;
            if (it < items) {
                float sum = part[u][0];
#pragma unroll
                for (int q = 1; q < kDecodeMaxSplits; ++q)
                    if (q < a.S) sum += part[u][q];
                const int t = it / a.E;
                const int e = it - t * a.E;
                lrow[t][e] = sum;
                if (a.logits_out) a.logits_out[(int64_t)(t0 + t) * a.E + e] = sum;
            }
        }
    }
    __syncthreads();

    const RowSpec spec{a.E, a.k, a.scoring, a.renorm, a.bias != nullptr};
    float bv[kPerLane] = {0.f, 0.f, 0.f, 0.f};
    if (a.bias) {
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane * kPerLane + j;
            if (e < a.E) bv[j] = a.bias[e];
        }
    }
    for (int t = wave; t < nrows; t += kWaves) {
        float v[kPerLane];
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane * kPerLane + j;
            v[j] = e < a.E ? lrow[t][e] : 0.f;
        }
        const RowResult res = route_row(v, bv, spec);
        if (lane < a.k) {
            const int64_t o = (int64_t)(t0 + t) * a.k + lane;
            a.inds[o] = res.idx;
            a.weights[o] = res.w;
            if (a.table_ids) slots[t * a.k + lane] = res.idx;  // M == 2: t < 2, k <= 16
        }
    }

    if (a.table_ids) {  // M == 2: both rows are in this row block
        __syncthreads();
        if (wave == 0)
            emit_route_table_m2(slots, a.k, a.table_ids, a.table_mask, a.table_s2u, a.table_count);
    }
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream)
{
    const int R = (a.M + kDecodeTile - 1) / kDecodeTile;
    const int B = (a.E + kDecodeTile - 1) / kDecodeTile;
    const int grid = R * B * a.S;
    hipLaunchKernelGGL(decode_router_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gpt
