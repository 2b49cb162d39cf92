// Shared device helpers for the gfx950 kernels of libspecverify.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define SPEC_WAVE 64

namespace spec {

// ---- element loads -------------------------------------------------------

typedef unsigned int v4u32 __attribute__((ext_vector_type(4)));

// 16-byte load marked nontemporal (streamed once; keeps caches for data that is reused).
__device__ __forceinline__ uint4 load_nt(const uint4* p) {
  const v4u32 v = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// bf16 -> fp32 is exact: a bf16 value is the high half of an fp32 word.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* row, int64_t v) {
  if constexpr (BF16) {
    uint32_t h = reinterpret_cast<const uint16_t*>(row)[v];
    return __uint_as_float(h << 16);
  } else {
    return reinterpret_cast<const float*>(row)[v];
  }
}

// ---- wave reductions (wave64) -------------------------------------------

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, SPEC_WAVE));
  return x;
}

// Workgroup barrier for LDS data: the LDS writes issued before it are complete and seen by every
// wave after it, while global loads in flight stay in flight (__syncthreads waits for those too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, SPEC_WAVE);
  return x;
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, SPEC_WAVE);
  return x;
}

__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, SPEC_WAVE));
  return x;
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, SPEC_WAVE));
  return x;
}

__device__ __forceinline__ int wave_or_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x |= __shfl_xor(x, o, SPEC_WAVE);
  return x;
}

// Inclusive prefix sum of a double across the wave (lane order).
__device__ __forceinline__ double wave_inclusive_sum(double x, int lane) {
#pragma unroll
  for (int o = 1; o < SPEC_WAVE; o <<= 1) {
    double y = __shfl_up(x, o, SPEC_WAVE);
    if (lane >= o) x += y;
  }
  return x;
}

__device__ __forceinline__ long long wave_inclusive_sum_i64(long long x, int lane) {
#pragma unroll
  for (int o = 1; o < SPEC_WAVE; o <<= 1) {
    long long y = __shfl_up(x, o, SPEC_WAVE);
    if (lane >= o) x += y;
  }
  return x;
}

}  // namespace spec
