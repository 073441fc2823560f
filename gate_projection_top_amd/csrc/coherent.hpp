// Device-coherent 16-byte stores and loads for handing partial results from
// one workgroup to another.  gfx950's L2 is private to each XCD, so data that
// a workgroup on another XCD will read must not stay in a non-coherent L2
// line: these accesses carry the device-scope cache-policy bit, so the store
// writes through to the coherent level and the load reads from it.  No
// cache-wide writeback or invalidate is then needed around the hand-off.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kCoherent = 16;     // buffer cache-policy bit: device scope
constexpr int kNonTemporal = 2;   // buffer cache-policy bit: streaming replacement

// Raw buffer over a workspace of at most 2 GiB (offsets are 32-bit bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(float* base)
{
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ void publish4(__amdgpu_buffer_rsrc_t r, int byte_off, f32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, byte_off, 0, kCoherent);
}

// A published value is read back once, so the load is also non-temporal
// (the prefill's exchange at 8192 tokens: ~0.7 us shorter with cold
// activations, unchanged with cache-hot ones; a non-temporal publish measured
// slower).
__device__ __forceinline__ f32x4 fetch4(__amdgpu_buffer_rsrc_t r, int byte_off)
{
    return __builtin_bit_cast(f32x4,
                              __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kCoherent | kNonTemporal));
}

}  // namespace gpt
