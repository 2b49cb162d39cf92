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

// ---- wave reductions and scans (wave64) -----------------------------------
//
// Lanes exchange values through DPP (the vector ALU's cross-lane operand modes of gfx9: quad
// permutes, row mirrors, row shifts and row broadcasts within and across rows of 16 lanes) and
// v_readlane, not through the LDS crossbar (ds_bpermute), which shares the LDS with table reads.

namespace dpp {
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowMirror = 0x140;      // lane i of a row takes lane 15 - i
constexpr int kRowHalfMirror = 0x141;  // lane i of a half row takes lane 7 - i
constexpr int kRowShr = 0x110;         // + n: lane i takes lane i - n of its row
constexpr int kRowBcast15 = 0x142;     // lane 15 of each row, to the next row
constexpr int kRowBcast31 = 0x143;     // lane 31, to rows 2 and 3
}  // namespace dpp

template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp32(uint32_t x, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROWS, 0xF, false);
}

// x of the lane CTRL selects, for a 4- or 8-byte T; a lane whose source lies outside its row, or
// which lies outside the rows ROWS selects, keeps `old`.
template <int CTRL, int ROWS = 0xF, class T>
__device__ __forceinline__ T dpp_move(T x, T old) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "4- or 8-byte values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, dpp32<CTRL, ROWS>(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, old)));
  } else {
    const uint2 v = __builtin_bit_cast(uint2, x), o = __builtin_bit_cast(uint2, old);
    uint2 r;
    r.x = dpp32<CTRL, ROWS>(v.x, o.x);
    r.y = dpp32<CTRL, ROWS>(v.y, o.y);
    return __builtin_bit_cast(T, r);
  }
}

template <class T>
__device__ __forceinline__ T read_lane(T x, int l) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
  } else {
    const int2 v = __builtin_bit_cast(int2, x);
    int2 r;
    r.x = __builtin_amdgcn_readlane(v.x, l);
    r.y = __builtin_amdgcn_readlane(v.y, l);
    return __builtin_bit_cast(T, r);
  }
}

// Reduction over the wave (all lanes active); every lane gets the same result.  Within a row the
// lanes are paired by quad permutes and mirrors, both lanes of a pair combining the same two values;
// the rows' values (lanes 0, 16, 32, 48) are then combined as (r0 op r1) op (r2 op r3).
template <class T, class Op>
__device__ __forceinline__ T wave_reduce(T x, Op op) {
  x = op(x, dpp_move<dpp::kQuadXor1>(x, x));
  x = op(x, dpp_move<dpp::kQuadXor2>(x, x));
  x = op(x, dpp_move<dpp::kRowHalfMirror>(x, x));
  x = op(x, dpp_move<dpp::kRowMirror>(x, x));
  return op(op(read_lane(x, 0), read_lane(x, 16)), op(read_lane(x, 32), read_lane(x, 48)));
}

// Inclusive prefix sum in lane order (all lanes active): shifts by 1, 2, 4, 8 within each row, then
// the row totals carried by the row broadcasts.
template <class T>
__device__ __forceinline__ T wave_inclusive_scan(T x) {
  const T z = T(0);
  x += dpp_move<dpp::kRowShr + 1>(x, z);
  x += dpp_move<dpp::kRowShr + 2>(x, z);
  x += dpp_move<dpp::kRowShr + 4>(x, z);
  x += dpp_move<dpp::kRowShr + 8>(x, z);
  x += dpp_move<dpp::kRowBcast15, 0xA>(x, z);
  x += dpp_move<dpp::kRowBcast31, 0xC>(x, z);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
  return wave_reduce(x, [](float p, float q) { return fmaxf(p, q); });
}

// Workgroup barrier for LDS data: the LDS writes issued before it are complete and seen by every
// wave after it, while global loads in flight stay in flight (__syncthreads waits for those too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ double wave_sum(double x) {
  return wave_reduce(x, [](double p, double q) { return p + q; });
}

__device__ __forceinline__ int wave_sum_i(int x) {
  return wave_reduce(x, [](int p, int q) { return p + q; });
}

__device__ __forceinline__ int wave_max_i(int x) {
  return wave_reduce(x, [](int p, int q) { return max(p, q); });
}

__device__ __forceinline__ int wave_min_i(int x) {
  return wave_reduce(x, [](int p, int q) { return min(p, q); });
}

__device__ __forceinline__ int wave_or_i(int x) {
  return wave_reduce(x, [](int p, int q) { return p | q; });
}

// Inclusive prefix sum of a double across the wave (lane order).
__device__ __forceinline__ double wave_inclusive_sum(double x, int) { return wave_inclusive_scan(x); }

__device__ __forceinline__ long long wave_inclusive_sum_i64(long long x, int) { return wave_inclusive_scan(x); }

}  // namespace spec
