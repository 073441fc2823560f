// Routed gather + shared-expert add, the step after the router.  One launch
// does both the weighted gather of the routed experts' rows and the add of
// the shared expert's row (b70 lab MTP1 M=2 note, "Outcome"), with the
// rounding chain of that note's "Exact arithmetic" section: the routed sum
// in FP32, rounded to BF16, then the BF16 shared row added and rounded to
// BF16 again.
//
//   out[t, d] = bf16( bf16(acc) + shared[t, d] ),
//   acc = fp32 sum over the slots j = 0..k-1 of token t, in order, of
//         fl32(w[t, j] * y[row(t, j), d]) (product and sum rounded
//         separately; the library is built without FP contraction),
//
// with row(t, j) = -1 for a slot whose expert has no local output row (it
// adds nothing).  The rows come either from an explicit [M, k] map or from
// the unique-route table (same note, "Why literal source-direct GEMM1 is not
// funded": each unique expert computes only the rows of its tokens, so slot
// (t, j) reads the compact row  sum over earlier unique experts of their
// token counts  +  the number of its expert's tokens below t).
//
// Layout: one thread per 8 consecutive elements of one token's row (16-byte
// loads and stores); a workgroup covers 1024 elements of one token, so the
// token, its k rows and its k weights are uniform across the workgroup.
// Every row load of a thread is issued before the first product is formed.
// The work is a few loads per output: the kernel is bound by memory latency
// at decode sizes and by HBM bandwidth at large M.
#include "launch.hpp"
#include "route_common.hpp"

namespace gpt {
namespace {

constexpr int kGatherThreads = 128;
constexpr int kGatherChunk = kGatherThreads * 8;  // elements of D per workgroup
constexpr int kGatherMaxK = 16;

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_value(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> BF16, to nearest, ties to even
__device__ __forceinline__ uint16_t to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// kMaxK: k rounded up to 4, 6, 8 or 16 (the unrolled slot count; a slot
// past k costs a load, so the common k = 6 and k = 8 have their own).
// kStream: the expert rows are loaded non-temporally (streaming replacement
// in the caches), for calls large enough to be bound by HBM bandwidth.
template <bool kTable, int kMaxK, bool kStream>
__global__ __launch_bounds__(kGatherThreads) void gather_shared_add_kernel(GatherLaunch a)
{
    __shared__ int32_t table_rows[kGatherMaxK];
    const int chunks = (a.D + kGatherChunk - 1) / kGatherChunk;
    const int64_t t = blockIdx.x / chunks;
    const int d0 = (blockIdx.x % chunks) * kGatherChunk + threadIdx.x * 8;
    const int k = a.k;

    if constexpr (kTable) {
        // wave 0: this token's k rows of the compact layout
        if (threadIdx.x < kWave) {
            const int lane = threadIdx.x;
            const int slots = (int)a.M * k;  // <= 64
            int n = *a.unique_count;
            n = n < 0 ? 0 : (n > slots ? slots : n);
            const uint32_t mask = lane < n ? (uint32_t)a.token_mask[lane] : 0u;
            const int count = __builtin_popcount(mask);
            int incl = count;  // inclusive prefix sum of the token counts over unique experts
#pragma unroll
            for (int off = 1; off < kWave; off <<= 1) {
                const int v = __shfl_up(incl, off);
                if (lane >= off) incl += v;
            }
            const int base = incl - count;
            const int u = lane < k ? a.slot_to_unique[t * k + lane] : 0;
            const bool u_ok = u >= 0 && u < n;
            const int src = u_ok ? u : 0;
            const int base_u = __shfl(base, src);
            const uint32_t mask_u = (uint32_t)__shfl((int)mask, src);
            const bool picked = u_ok && ((mask_u >> t) & 1u);
            if (lane < k)
                table_rows[lane] = picked ? base_u + __builtin_popcount(mask_u & ((1u << t) - 1u)) : -1;
        }
        __syncthreads();
    }
    // The token's rows and weights: lane j of each wave loads slot j's (one
    // round trip for all of them), then each is broadcast to a scalar.  Every
    // lane stays until the broadcasts are done (a lane past D still lends
    // its slot), and only then do lanes past D drop out.
    const int lane = threadIdx.x & (kWave - 1);
    int my_row = -1;
    float my_w = 0.f;
    if (lane < k) {
        my_row = kTable ? table_rows[lane] : a.slot_rows[t * k + lane];
        my_w = a.weights[t * k + lane];
    }
    // (lanes past k hold row -1 and weight 0, so every broadcast is valid;
    // all of them come before the first row load, so that no wait for a
    // row load is placed between two of them)
    int64_t rows[kMaxK];
    float wv[kMaxK];
    bool live[kMaxK];
    bool any = false;
    int64_t first = 0;
#pragma unroll
    for (int j = kMaxK - 1; j >= 0; --j) {
        rows[j] = __builtin_amdgcn_readlane(my_row, j);
        wv[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_w), j));
        live[j] = rows[j] >= 0 && rows[j] < a.y_rows;  // wave-uniform
        any |= live[j];
        first = live[j] ? rows[j] : first;
    }
    if (d0 >= a.D) return;
    // Straight-line loads (a load under a per-slot branch made the compiler
    // wait for each in turn): a slot with no row reads the first live row
    // again, a line this thread fetches anyway, and adds nothing.  With no
    // live slot at all, nothing is loaded.  Each expert row is read once:
    // at bandwidth-bound sizes the loads are non-temporal (M=4096, k=8: the
    // launch sustains ~6.2 TB/s instead of ~5.1).
    u16x8 yv[kMaxK];
    if (any) {
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            const u16x8* p = reinterpret_cast<const u16x8*>(a.y + (live[j] ? rows[j] : first) * a.D + d0);
            if constexpr (kStream)
                yv[j] = __builtin_bit_cast(u16x8, __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p)));
            else
                yv[j] = *p;
        }
    }
    const u16x8 sv = *reinterpret_cast<const u16x8*>(a.shared + t * a.D + d0);

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
        if (!live[j]) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = wv[j] * bf16_value(yv[j][e]);
            acc[e] = acc[e] + p;
        }
    }
    u16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float routed = bf16_value(to_bf16(acc[e]));
        o[e] = to_bf16(routed + bf16_value(sv[e]));
    }
    *reinterpret_cast<u16x8*>(a.out + t * a.D + d0) = o;
}

// Calls reading at least this many expert rows take the streaming loads.
constexpr int64_t kGatherStreamRows = 256;

template <bool kTable, int kMaxK>
void launch_gather_k(const GatherLaunch& a, dim3 grid, dim3 block, hipStream_t stream)
{
    if ((int64_t)a.M * a.k >= kGatherStreamRows)
        hipLaunchKernelGGL((gather_shared_add_kernel<kTable, kMaxK, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((gather_shared_add_kernel<kTable, kMaxK, false>), grid, block, 0, stream, a);
}

template <bool kTable>
hipError_t launch_gather_t(const GatherLaunch& a, dim3 grid, dim3 block, hipStream_t stream)
{
    if (a.k <= 4)
        launch_gather_k<kTable, 4>(a, grid, block, stream);
    else if (a.k <= 6)
        launch_gather_k<kTable, 6>(a, grid, block, stream);
    else if (a.k <= 8)
        launch_gather_k<kTable, 8>(a, grid, block, stream);
    else if (a.k <= kGatherMaxK)
        launch_gather_k<kTable, 16>(a, grid, block, stream);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gather(const GatherLaunch& a, hipStream_t stream)
{
    if (a.M <= 0) return hipSuccess;
    const int64_t chunks = (a.D + kGatherChunk - 1) / kGatherChunk;
    const dim3 grid((unsigned)(a.M * chunks)), block(kGatherThreads);
    return a.slot_rows == nullptr ? launch_gather_t<true>(a, grid, block, stream)
                                  : launch_gather_t<false>(a, grid, block, stream);
}

}  // namespace gpt
