// Prefill main-loop stream probe: the load streams of the prefill kernel's
// main loop taken apart.  Measurement only: built into the probe library
// (libfloorprobes.so) that the benchmark loads; the router never calls it.
//
// Geometry of the prefill at four K splits: 128-row tiles x 4 splits, one
// workgroup of 8 waves per (tile, split), K staged 64 wide.  Waves 4..7 issue
// the direct-to-LDS loads of two rings exactly as the prefill does (X three
// stages ahead in a four-slot ring, W two stages ahead in a three-slot ring,
// chunk c of row R in 16-byte slot c ^ (R mod 8)), waiting for a stage's
// loads before its barrier; waves 0..3 pass the same barriers and, in the
// last mode, read the MFMA fragments of each stage and multiply.  Modes:
//   0  X and W streams, no compute;
//   1  X stream only;
//   2  W stream only;
//   3  X and W, every W stage the same 32 KiB (W always hits the caches);
//   4  X and W with the fragment reads and MFMAs (the main loop without the
//      row tile, exchange and routing).
// Each workgroup writes one float (its accumulators' sum) to out.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kBM = 128, kBK = 64, kSplits = 4, kWaves = 8, kThreads = kWaves * 64;
constexpr int kXSlots = 4, kWSlots = 3;                    // X three ahead, W two ahead
constexpr int kXStage = kBM * kBK * 2, kWStage = 256 * kBK * 2;  // 16 and 32 KiB
constexpr int kXAhead = kXSlots - 1, kWAhead = kWSlots - 1;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ int swz(int R) { return R & 7; }

// one 1 KiB direct-to-LDS load (lane i's 16 bytes to lds + 16 i); untracked
// by the compiler, waited for with explicit vmcnt below
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int off, unsigned char* lds)
{
    const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_void*)lds);
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(m0) : "memory");
}

__device__ __forceinline__ void raw_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm()
{
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// wait until at most n (a multiple of 4 up to 24) loads are in flight
__device__ __forceinline__ void wait_vm_rt(int n)
{
    switch (n) {
    case 0: wait_vm<0>(); break;
    case 4: wait_vm<4>(); break;
    case 8: wait_vm<8>(); break;
    case 12: wait_vm<12>(); break;
    case 16: wait_vm<16>(); break;
    case 20: wait_vm<20>(); break;
    case 24: wait_vm<24>(); break;
    default: wait_vm<0>(); break;
    }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void pf_stream_kernel(const uint16_t* x, const uint16_t* w, int H, float* out)
{
    __shared__ __attribute__((aligned(16))) unsigned char lds[kXSlots * kXStage + kWSlots * kWStage];
    constexpr bool kX = MODE != 2, kW = MODE != 1, kWHot = MODE == 3, kMfma = MODE == 4;
    unsigned char* xring = lds;
    unsigned char* wring = lds + kXSlots * kXStage;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // workgroup -> (tile, split) as in the prefill: the splits of a tile on one XCD
    const int xcd = blockIdx.x % 8, q8 = blockIdx.x / 8, s = q8 % kSplits, tile = xcd + 8 * (q8 / kSplits);
    const int kps = H / kSplits, nst = kps / kBK, kb = s * kps;
    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (wave >= 4) {
        const int pi = wave - 4, li = lane >> 3, ls = lane & 7;
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint16_t*>(x + (int64_t)tile * kBM * H), 0, kBM * H * 2, 0x00020000);
        const __amdgpu_buffer_rsrc_t wr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(w), 0, 256 * H * 2, 0x00020000);
        int a_off[4], b_off[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int R = (pi * 4 + j) * 8 + li;
            a_off[j] = (R * H + (ls ^ swz(R)) * 8) * 2;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int R = (pi * 8 + j) * 8 + li;
            b_off[j] = (R * H + (ls ^ swz(R)) * 8) * 2;
        }
        auto nx = [&](int j) { return (kX && j + kXAhead >= 0 && j + kXAhead < nst) ? 4 : 0; };
        auto nw = [&](int j) { return (kW && j + kWAhead >= 0 && j + kWAhead < nst) ? 8 : 0; };
        auto issue = [&](int j) {
            if (nx(j)) {
                const int k0 = kb + (j + kXAhead) * kBK;
                unsigned char* slot = xring + ((j + kXAhead) % kXSlots) * kXStage;
#pragma unroll
                for (int q = 0; q < 4; ++q) dma16(xr, a_off[q] + k0 * 2, slot + (pi * 4 + q) * 1024);
            }
            if (nw(j)) {
                const int k0 = kWHot ? 0 : kb + (j + kWAhead) * kBK;
                unsigned char* slot = wring + ((j + kWAhead) % kWSlots) * kWStage;
#pragma unroll
                for (int q = 0; q < 8; ++q) dma16(wr, b_off[q] + k0 * 2, slot + (pi * 8 + q) * 1024);
            }
        };
        for (int j = -kXAhead; j < 0; ++j) issue(j);
        for (int ks = 0; ks < nst; ++ks) {
            // stage ks is complete once at most the loads issued after the
            // later of X[ks] (issue(ks - 3)) and W[ks] (issue(ks - 2)) remain
            int after = 0;
            const int first = kW ? ks - kWAhead + 1 : ks - kXAhead + 1;
            for (int j = first; j <= ks - 1; ++j) after += nx(j) + nw(j);
            wait_vm_rt(after);
            raw_barrier();
            issue(ks);
        }
        wait_vm<0>();
    } else {
        const int wm = wave >> 1, wn = wave & 1, fr = lane & 15, g = lane >> 4;
        for (int ks = 0; ks < nst; ++ks) {
            raw_barrier();
            if constexpr (kMfma) {
                const unsigned char* xs = xring + (ks % kXSlots) * kXStage;
                const unsigned char* ws = wring + (ks % kWSlots) * kWStage;
                bf16x8 af[2][4], bf[2][8];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int c = kk * 4 + g;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int R = wm * 64 + i * 16 + fr;
                        af[kk][i] = *reinterpret_cast<const bf16x8*>(xs + R * 128 + ((c ^ swz(R)) << 4));
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int R = wn * 128 + j * 16 + fr;
                        bf[kk][j] = *reinterpret_cast<const bf16x8*>(ws + R * 128 + ((c ^ swz(R)) << 4));
                    }
                }
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kk][i], bf[kk][j], acc[i][j], 0, 0, 0);
            }
        }
    }
    __syncthreads();
    if (tid < 64) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) t += acc[i][j][0];
        for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
        if (tid == 0) out[blockIdx.x] = t;
    }
}

}  // namespace

extern "C" {

// x: bf16 [M, H]; w: bf16 [256, H]; out: (M / 128) * 4 floats.
// M a multiple of 1024 (whole groups of 8 tiles), H a multiple of 256.
int pf_stream_probe(const void* x, const void* w, int M, int H, int mode, float* out, hipStream_t stream)
{
    if (!x || !w || !out || M < 1024 || M % 1024 != 0 || H < 256 || H % 256 != 0 || mode < 0 || mode > 4 ||
        (int64_t)kBM * H * 2 > 0x7fffffff || (int64_t)256 * H * 2 > 0x7fffffff)
        return -1;
    const dim3 grid((unsigned)(M / kBM * kSplits)), block(kThreads);
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const uint16_t* wp = static_cast<const uint16_t*>(w);
    switch (mode) {
    case 0: hipLaunchKernelGGL(pf_stream_kernel<0>, grid, block, 0, stream, xp, wp, H, out); break;
    case 1: hipLaunchKernelGGL(pf_stream_kernel<1>, grid, block, 0, stream, xp, wp, H, out); break;
    case 2: hipLaunchKernelGGL(pf_stream_kernel<2>, grid, block, 0, stream, xp, wp, H, out); break;
    case 3: hipLaunchKernelGGL(pf_stream_kernel<3>, grid, block, 0, stream, xp, wp, H, out); break;
    default: hipLaunchKernelGGL(pf_stream_kernel<4>, grid, block, 0, stream, xp, wp, H, out); break;
    }
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
