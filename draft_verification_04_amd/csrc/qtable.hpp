// The Q table of the sampling kernels: Q(z) = exp(z/T - R) in fp64 for bf16 logits z, evaluated
// once per bf16 value into LDS and looked up per token, with the exact direct evaluation for the
// values outside the table.  Any offset R gives the same probabilities (p = Q / sum Q over the
// row); the callers choose one that keeps the row's largest entries near 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spec {

constexpr int kQefLo = 107, kQefHi = 133;               // bf16 exponent fields tabulated
constexpr int kQper = (kQefHi - kQefLo + 1) * 128;      // 3456 values per sign
constexpr int kQsize = 2 * kQper;                       // 6912 entries, 55296 bytes
constexpr uint32_t kFill2 = 0x3f803f80u;                // two bf16 ones: tabulated filler bits

// exp(x) in fp64 by Tang's table-driven method (ACM TOMS 15(2), 1989), for
// x in [-1000, 709]: x = k ln2/64 + r with |r| <= ln2/128 (two-part ln2/64),
// e^x = 2^(k div 64) * 2^((k mod 64)/64) * e^r, e^r by its degree-5 Taylor
// polynomial (truncation < 4e-17); T64[j] = 2^(j/64).  Underflows to 0.
__device__ __forceinline__ double exp_tang(double x, const double* T64) {
  const double k = rint(x * 92.332482616893657);
  double r = fma(-k, 0.010830424696249145, x);
  r = fma(-k, 3.623510646634843e-19, r);
  double p = fma(r, 1.0 / 120.0, 1.0 / 24.0);
  p = fma(r, p, 1.0 / 6.0);
  p = fma(r, p, 0.5);
  p = fma(r, p, 1.0);
  p = fma(r, p, 1.0);
  const int ki = (int)k;
  return ldexp(T64[ki & 63] * p, ki >> 6);
}

// Q(z) = exp(z/T - R), z/T taken as the fp64 product z * (1/T); -inf -> 0.
__device__ __forceinline__ double q_direct(float z, double invT, double R, const double* T64) {
  return exp_tang(fmax(fma((double)z, invT, -R), -1000.0), T64);
}

__device__ __forceinline__ void init_t64(double* T64) {
  if (threadIdx.x < 64) T64[threadIdx.x] = exp2((double)threadIdx.x * (1.0 / 64.0));
}

// The table of Q over the tabulated bf16 values.  Entry 2 (m - m0) + s holds the value with sign
// s and magnitude bits m (m0 the first tabulated magnitude): the index is the bf16 bit pattern
// rotated left by one, less 2 m0, which two 16-bit integer instructions give for a pair of values.
__device__ inline void build_qtab_part(double* Qt, double invT, double R, const double* T64, int t0, int nthr) {
  for (int idx = t0; idx < kQsize; idx += nthr) {
    const uint32_t bits = ((uint32_t)(idx & 1) << 15) | ((uint32_t)(kQefLo << 7) + ((uint32_t)idx >> 1));
    Qt[idx] = q_direct(__uint_as_float(bits << 16), invT, R, T64);
  }
}

__device__ __forceinline__ void build_qtab(double* Qt, double invT, double R, const double* T64) {
  build_qtab_part(Qt, invT, R, T64, (int)threadIdx.x, (int)blockDim.x);
}

// Table slot of one bf16 value (see build_qtab); kQsize or more when it is not tabulated.
__device__ __forceinline__ uint32_t q_slot1(uint32_t b) {
  return (((b << 1) | (b >> 15)) - (uint32_t)(2 * (kQefLo << 7))) & 0xffffu;
}

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// Table slots of the two bf16 values of a word, one per 16-bit half; a slot is below kQsize
// exactly when its value is tabulated (otherwise it wrapped past it).
__device__ __forceinline__ us2 q_slots(uint32_t w) {
  const us2 v = __builtin_bit_cast(us2, w);
  return ((v << (unsigned short)1) | (v >> (unsigned short)15)) - (us2)(unsigned short)(2 * (kQefLo << 7));
}

__device__ __forceinline__ uint32_t slot_of(const us2 (&k)[4], int j) {
  return (j & 1) ? (uint32_t)k[j >> 1].y : (uint32_t)k[j >> 1].x;
}

__device__ __forceinline__ uint32_t half16(const uint32_t (&w)[4], int j) {
  return (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu);
}

}  // namespace spec
