// Standalone logits -> top-k (the unfused second half: dense_router_decode
// notes, "Current working path", and qwisp issue #145's route_top8_rows).
//
// One wavefront per row, one launch covering every row.  Lane L reads logits
// 4L..4L+3 (one 16-byte load when rows are aligned), so a 256-expert row is
// one fully coalesced 1 KiB read; then the shared route_row() does scoring,
// key, selection and weights.
#include "launch.hpp"
#include "route_common.hpp"

namespace gpt {

namespace {

constexpr int kTopkWaves = 4;

__global__ __launch_bounds__(kTopkWaves * kWave) void topk_from_logits_kernel(TopkLaunch a)
{
    __shared__ uint64_t sel[kTopkWaves][kRefineSlots];  // selection scratch, one per wave
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const RowSpec spec{a.E, a.k, a.scoring, a.renorm, a.bias != nullptr};

    float bv[kPerLane] = {0.f, 0.f, 0.f, 0.f};
    if (a.bias) {
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane * kPerLane + j;
            if (e < a.E) bv[j] = a.bias[e];
        }
    }

    // one row per wave: no loop, so that nothing is held across rows
    const int64_t row = (int64_t)blockIdx.x * kTopkWaves + wave;
    if (row >= a.M) return;
    const Exp2Lane et = load_exp2_lane();
    const float* r = a.logits + row * a.E;
    float v[kPerLane] = {0.f, 0.f, 0.f, 0.f};
    if (a.vector_rows) {
        if (lane * kPerLane < a.E) {
            const float4 q = *reinterpret_cast<const float4*>(r + lane * kPerLane);
            v[0] = q.x;
            v[1] = q.y;
            v[2] = q.z;
            v[3] = q.w;
        }
    } else {
#pragma unroll
        for (int j = 0; j < kPerLane; ++j) {
            const int e = lane * kPerLane + j;
            if (e < a.E) v[j] = r[e];
        }
    }
    const RowResult res = route_row<kFilter>(v, bv, spec, sel[wave], et);
    if (lane < a.k) {
        a.inds[row * a.k + lane] = res.idx;
        a.weights[row * a.k + lane] = res.w;
    }
}

}  // namespace

hipError_t launch_topk(const TopkLaunch& a, hipStream_t stream)
{
    if (a.M <= 0) return hipSuccess;
    const int64_t blocks = (a.M + kTopkWaves - 1) / kTopkWaves;  // one wave per row
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(topk_from_logits_kernel, dim3((unsigned)blocks), dim3(kTopkWaves * kWave), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gpt
