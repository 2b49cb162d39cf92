// Philox4x64-10 (J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11), device side.
//
// A block maps a 4 x 64-bit counter and a 2 x 64-bit key to 4 x 64-bit words
// through 10 rounds.  A round multiplies counter words 0 and 2 by two fixed
// odd 64-bit multipliers, keeps both halves of each 128-bit product, and
// forms the next counter from (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2),
// hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); the key is advanced by two Weyl
// increments (the golden ratio and sqrt(3) - 1 in 64-bit fixed point) before
// every round but the first.
//
// Draw layout used by the verifier: key (seed, 0), counter (k + 1, i, 0, 0)
// for request i and draft position k; word 0 -> acceptance uniform, word 1
// -> emitted-token uniform, each (w >> 11) * 2^-53.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spec {

struct Philox4x64 {
  uint64_t w0, w1, w2, w3;
};

__device__ __forceinline__ Philox4x64 philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                                    uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull;
  constexpr uint64_t kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull;
  constexpr uint64_t kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += kW0;
      k1 += kW1;
    }
    const uint64_t lo0 = kM0 * c0, hi0 = __umul64hi(kM0, c0);
    const uint64_t lo1 = kM1 * c2, hi1 = __umul64hi(kM1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0;
    const uint64_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return Philox4x64{c0, c1, c2, c3};
}

__device__ __forceinline__ double uniform53(uint64_t w) {
  return (double)(w >> 11) * 0x1p-53;
}

// (u_accept, u_emit) for request i, draft position k, seed s.
__device__ __forceinline__ void verify_uniforms(uint64_t seed, uint64_t i, uint64_t k,
                                                double* u_acc, double* u_emit) {
  Philox4x64 b = philox4x64_10(k + 1, i, 0, 0, seed, 0);
  *u_acc = uniform53(b.w0);
  *u_emit = uniform53(b.w1);
}

}  // namespace spec
