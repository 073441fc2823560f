// Floor probes for the single-token decode router: what one launch on the
// router's grid costs before any routing, step by step.  Measurement only:
// built into a library of its own (libfloorprobes.so) that the benchmark
// loads; the router never calls these.
//
// Each probe runs on G workgroups of 256 threads (the decode router's grid
// at E = 256: one workgroup per expert) and adds one ingredient of the
// router's launch to the one before:
//   floor_empty     the launch alone (any grid and workgroup size);
//   floor_read      each workgroup reads its slice of a gate-sized matrix
//                   (one HBM round trip: every 16-byte load issued before the
//                   first use) and reduces it to one value;
//   floor_ticket    the read, plus the two-level arrival ticket on a control
//                   wave (groups of 16 workgroups, then the groups); the last
//                   arrival writes one word;
//   floor_handoff   the ticket, plus the hand-off: every workgroup publishes
//                   its value as a tagged 8-byte slot with a device-coherent
//                   store, and the last arrival polls all G slots (lane L:
//                   slots 4L..4L+3) until every tag is this launch's, then
//                   writes their sum;
//   floor_handoff_fixed  the same publish and poll with no ticket: workgroup
//                   0 is the finisher whatever the arrival order.
// floor_latency: one wave times dependent round trips with the 100 MHz
// realtime clock: a device-scope atomic, a device-coherent load of a line
// another XCD wrote, and a plain load of a line not yet in any cache.
// floor_stream_read: the practical HBM read ceiling the roofline fractions
// sit under: every 16-byte unit of a buffer far larger than the Infinity
// Cache read once (each workgroup a contiguous chunk, four loads in flight
// per thread), one value written per workgroup; floor_stream_read_nt: the
// same with non-temporal loads (streaming replacement in the caches).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kMaxLoads = 8;  // 16-byte loads per thread per workgroup slice

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kCoherent = 16;  // buffer cache-policy bit: device scope

__device__ __forceinline__ float lane_sum(u32x4 v)
{
    // any fixed function of the bytes read; keeps the loads alive
    return __uint_as_float(v[0] & 0x3fffffffu) + __uint_as_float(v[1] & 0x3fffffffu) +
           __uint_as_float(v[2] & 0x3fffffffu) + __uint_as_float(v[3] & 0x3fffffffu);
}

__device__ __forceinline__ float wave_sum(float v)
{
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// The workgroup's slice: n16 16-byte units starting at blockIdx.x * n16,
// thread t taking units t, t + 256, ...; n16 <= kThreads * kMaxLoads (host-checked).
__device__ float read_slice(const u32x4* w, int n16)
{
    __shared__ float part[kThreads / 64];
    const u32x4* base = w + (int64_t)blockIdx.x * n16;
    u32x4 v[kMaxLoads];
#pragma unroll
    for (int i = 0; i < kMaxLoads; ++i) {
        const int u = (int)threadIdx.x + i * kThreads;
        v[i] = u < n16 ? base[u] : u32x4{0u, 0u, 0u, 0u};
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxLoads; ++i) s += lane_sum(v[i]);
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    return ((part[0] + part[1]) + part[2]) + part[3];
}

// Two-level ticket on ctr (words 16 apart: groups of 16 workgroups, then the
// group counter at index 16 * 16).  Returns true for the last arrival.  The
// counters return to zero.
__device__ bool last_arrival(uint32_t* ctr)
{
    const int G = (int)gridDim.x;
    const int g = (int)blockIdx.x / 16;
    const int ng = min(16, G - 16 * g);
    const int B = (G + 15) / 16;
    uint32_t* l1 = ctr + 16 * g;
    uint32_t* l2 = ctr + 16 * 16;
    if (__hip_atomic_fetch_add(l1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != (uint32_t)ng - 1u)
        return false;
    __hip_atomic_store(l1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__hip_atomic_fetch_add(l2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != (uint32_t)B - 1u)
        return false;
    __hip_atomic_store(l2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

__global__ __launch_bounds__(1024) void floor_empty_kernel() {}

__global__ __launch_bounds__(kThreads) void floor_read_kernel(const u32x4* w, int n16, float* out)
{
    const float s = read_slice(w, n16);
    if (threadIdx.x == 0) out[blockIdx.x] = s;
}

// mode 0: ticket only; mode 1: ticket + tagged publish + poll; mode 2: the
// tagged publish and poll with no ticket, workgroup 0 the fixed finisher;
// mode 3: publish first, wait for the store, then the ticket: the last
// arrival reads every slot once (all were published before their tickets).
// ctr: 16 * 17 words, zero between launches; slots: G 8-byte slots;
// epoch: one word, advanced by the last arrival (tags are epoch + 1, never 0).
__global__ __launch_bounds__(kThreads + 64) void floor_ticket_kernel(const u32x4* w, int n16, float* out,
                                                                      uint32_t* ctr, u32x2* slots,
                                                                      uint32_t* epoch, int mode)
{
    __shared__ int s_last;
    __shared__ uint32_t s_tag;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float s = 0.f;
    if (wave == kThreads / 64) {  // control wave
        if (lane == 0) {
            const uint32_t tag = __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
            s_tag = tag;  // read before the ticket: the last arrival advances it
            if (mode != 3) s_last = mode == 2 ? (blockIdx.x == 0 ? 1 : 0) : (last_arrival(ctr) ? 1 : 0);
        }
    }
    // the read (the control wave takes part in the barrier only)
    {
        __shared__ float part[kThreads / 64];
        const u32x4* base = w + (int64_t)blockIdx.x * n16;
        if (wave < kThreads / 64) {
            u32x4 v[kMaxLoads];
#pragma unroll
            for (int i = 0; i < kMaxLoads; ++i) {
                const int u = (int)threadIdx.x + i * kThreads;
                v[i] = u < n16 ? base[u] : u32x4{0u, 0u, 0u, 0u};
            }
            float t = 0.f;
#pragma unroll
            for (int i = 0; i < kMaxLoads; ++i) t += lane_sum(v[i]);
            t = wave_sum(t);
            if (lane == 0) part[wave] = t;
        }
        __syncthreads();
        s = ((part[0] + part[1]) + part[2]) + part[3];
    }
    const int G = (int)gridDim.x;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(slots, 0, G * 8, 0x00020000);
    if (mode >= 1 && threadIdx.x == 0) {
        const u32x2 v = {__float_as_uint(s), s_tag};
        __builtin_amdgcn_raw_buffer_store_b64(v, rs, (int)blockIdx.x * 8, 0, kCoherent);
        if (mode == 3) {
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the write-through store has completed
            s_last = last_arrival(ctr) ? 1 : 0;
        }
    }
    if (mode == 3) __syncthreads();  // s_last
    if (!s_last) return;
    if (mode == 0) {
        if (threadIdx.x == 0) out[0] = s;
        if (threadIdx.x == 0) __hip_atomic_store(epoch, s_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    if (wave != 0) return;
    // poll: lane L owns slots 4L..4L+3 (two 16-byte loads; out-of-range loads read 0)
    const uint32_t tag = s_tag;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    float sum = 0.f;
    for (;;) {
        asm volatile("" ::: "memory");
        const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 32, 0, kCoherent);
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 32 + 16, 0, kCoherent);
        const bool ok = (4 * lane + 0 >= G || a[1] == tag) && (4 * lane + 1 >= G || a[3] == tag) &&
                        (4 * lane + 2 >= G || b[1] == tag) && (4 * lane + 3 >= G || b[3] == tag);
        if (__builtin_amdgcn_ballot_w64(!ok) == 0) {
            sum = (4 * lane + 0 < G ? __uint_as_float(a[0]) : 0.f) + (4 * lane + 1 < G ? __uint_as_float(a[2]) : 0.f) +
                  (4 * lane + 2 < G ? __uint_as_float(b[0]) : 0.f) + (4 * lane + 3 < G ? __uint_as_float(b[2]) : 0.f);
            break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > 10000000u) {  // 100 ms guard
            sum = __builtin_nanf("");
            break;
        }
    }
    sum = wave_sum(sum);
    if (lane == 0) {
        out[0] = sum;
        __hip_atomic_store(epoch, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// One wave, reps dependent round trips of each kind; out[0..2] = mean ticks
// (100 MHz) per atomic, per coherent load, per cold plain load.
// scratch: >= 4 KiB of device memory; cold: >= reps * 4 KiB of memory not
// touched since the last launch over it (the host rotates a large pool).
__global__ __launch_bounds__(64) void floor_latency_kernel(uint32_t* scratch, const uint32_t* cold, int reps,
                                                           float* out)
{
    if (threadIdx.x != 0) return;
    uint32_t acc = 0;
    uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < reps; ++i)
        acc += __hip_atomic_fetch_add(scratch + (acc & 1u), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t t1 = __builtin_amdgcn_s_memrealtime();
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(scratch, 0, 4096, 0x00020000);
    for (int i = 0; i < reps; ++i) {
        asm volatile("" ::: "memory");
        acc += __builtin_amdgcn_raw_buffer_load_b32(rs, 64 + (int)(acc & 4u), 0, kCoherent);
    }
    uint64_t t2 = __builtin_amdgcn_s_memrealtime();
    for (int i = 0; i < reps; ++i) {
        asm volatile("" ::: "memory");
        acc += cold[(int64_t)i * 1024 + (acc & 1u)];
    }
    uint64_t t3 = __builtin_amdgcn_s_memrealtime();
    out[0] = (float)(t1 - t0) / reps;
    out[1] = (float)(t2 - t1) / reps;
    out[2] = (float)(t3 - t2) / reps;
    out[3] = (float)acc;  // keeps the chains alive
}

// Every unit i < n16 read once: workgroup b reads the contiguous units
// [b*per, (b+1)*per) (per = n16 / grid rounded up), 1024 units (16 KiB) per
// round with four 16-byte loads in flight per thread.
template <bool kNT>
__device__ __forceinline__ u32x4 stream_load(const u32x4* p)
{
    if constexpr (kNT)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <bool kNT>
__global__ __launch_bounds__(kThreads) void floor_stream_read_kernel(const u32x4* p, int64_t n16, float* out)
{
    __shared__ float part[kThreads / 64];
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const int64_t lo = (int64_t)blockIdx.x * per;
    const int64_t hi = lo + per < n16 ? lo + per : n16;
    int64_t i = lo + threadIdx.x;
    float s = 0.f;
    for (; i + 3 * kThreads < hi; i += 4 * kThreads) {
        const u32x4 a = stream_load<kNT>(p + i), b = stream_load<kNT>(p + i + kThreads);
        const u32x4 c = stream_load<kNT>(p + i + 2 * kThreads), d = stream_load<kNT>(p + i + 3 * kThreads);
        s += (lane_sum(a) + lane_sum(b)) + (lane_sum(c) + lane_sum(d));
    }
    for (; i < hi; i += kThreads) s += lane_sum(stream_load<kNT>(p + i));
    s = wave_sum(s);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = ((part[0] + part[1]) + part[2]) + part[3];
}

}  // namespace

extern "C" {

// threads: 64..1024, a multiple of 64 (the launch's workgroup size)
int floor_empty(int grid, int threads, hipStream_t stream)
{
    if (grid < 1 || threads < 64 || threads > 1024 || threads % 64 != 0) return -1;
    hipLaunchKernelGGL(floor_empty_kernel, dim3(grid), dim3(threads), 0, stream);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// w: grid * n16 16-byte units; out: grid floats.
int floor_read(const void* w, int n16, int grid, float* out, hipStream_t stream)
{
    if (grid < 1 || n16 < 1 || n16 > kThreads * kMaxLoads || !w || !out) return -1;
    hipLaunchKernelGGL(floor_read_kernel, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(w), n16, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// ctr: 16 * 17 zeroed words; slots: grid * 8 bytes, zeroed before the first
// launch; epoch: one word, zeroed before the first launch.  grid <= 256.
int floor_ticket(const void* w, int n16, int grid, float* out, uint32_t* ctr, void* slots, uint32_t* epoch,
                 int mode, hipStream_t stream)
{
    if (grid < 1 || grid > 256 || n16 < 1 || n16 > kThreads * kMaxLoads || !w || !out || !ctr || !slots ||
        !epoch || mode < 0 || mode > 3)
        return -1;
    hipLaunchKernelGGL(floor_ticket_kernel, dim3(grid), dim3(kThreads + 64), 0, stream,
                       static_cast<const u32x4*>(w), n16, out, ctr, static_cast<u32x2*>(slots), epoch, mode);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// scratch: >= 4 KiB; cold: >= reps * 4 KiB readable; out: 4 floats.
int floor_latency(uint32_t* scratch, const uint32_t* cold, int reps, float* out, hipStream_t stream)
{
    if (reps < 1 || !scratch || !cold || !out) return -1;
    hipLaunchKernelGGL(floor_latency_kernel, dim3(1), dim3(64), 0, stream, scratch, cold, reps, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// p: bytes (a multiple of 16) readable; out: grid floats.
int floor_stream_read(const void* p, int64_t bytes, int grid, float* out, hipStream_t stream)
{
    if (grid < 1 || bytes < 16 || bytes % 16 != 0 || !p || !out) return -1;
    hipLaunchKernelGGL(floor_stream_read_kernel<false>, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(p), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

int floor_stream_read_nt(const void* p, int64_t bytes, int grid, float* out, hipStream_t stream)
{
    if (grid < 1 || bytes < 16 || bytes % 16 != 0 || !p || !out) return -1;
    hipLaunchKernelGGL(floor_stream_read_kernel<true>, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(p), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
