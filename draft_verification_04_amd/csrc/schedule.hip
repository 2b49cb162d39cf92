// Confidence-scheduled verify lengths on gfx950 (one workgroup).
//
// Follows the DSpark paper, §3.2.2 (survival a_{r,j} = product of c_{r,1..j};
// marginal gain of extending request r to j is a_{r,j}; admit candidates in
// descending survival; objective Theta = tau * SPS(batch tokens) read from a
// profiled cost table) and Algorithm 1 of the paper's Chinese translation
// (stop at the first admission that does not raise Theta); the global mode is
// the search without the break of §5.2.
//
// Exactness: survivals are float32 products taken left to right; tau is an
// int64 in fixed point with 50 fractional bits (each survival floored to a
// multiple of 2^-50), so the parallel prefix sum is exact and independent of
// its association; Theta(m) = fp64(tau(m)) * 2^-50 * sps[B + m].
//
// Steps: survivals and 64-bit sort keys (inverted survival bits | candidate
// index, so ascending key = survival descending, then request, then
// position) -> bitonic sort in LDS -> exclusive int64 scan -> Theta(m) ->
// first non-rise (early stop) or first maximum (global) -> per-request counts.
#include "common.hpp"
#include "spec_verify.h"

#include <math.h>

namespace spec {

constexpr int kSchedThreads = 1024;
constexpr int kSchedMaxKeys = SPEC_MAX_SCHED_CANDIDATES;  // power of two
constexpr long long kOne = 1ll << 50;

struct SchedArgs {
  int B, G, budget, mode;
  const float* conf;
  const double* sps;
  int32_t* lengths;
  double* theta;
  int32_t* status;
};

struct SchedShared {
  unsigned long long keys[kSchedMaxKeys];
  long long wsum[kSchedThreads / SPEC_WAVE];
  double wth[kSchedThreads / SPEC_WAVE];
  int wm[kSchedThreads / SPEC_WAVE];
  int ncand;
  int mstar;
  double theta_star;
};

__device__ __forceinline__ long long fixed_q(float a) {
  // floor(a * 2^50): a is a float32 in [0, 1]; the product is exact in fp64
  return (long long)floor((double)a * 0x1p50);
}

__device__ __forceinline__ double theta_of(long long tau, double sps) {
  return ((double)tau * 0x1p-50) * sps;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(SchedArgs a) {
  __shared__ SchedShared sh;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int NW = kSchedThreads / SPEC_WAVE;
  const int B = a.B, G = a.G;
  const int N = B * G;
  int NP = 1;
  while (NP < N) NP <<= 1;
  if (tid == 0) sh.ncand = 0;
  for (int p = N + tid; p < NP; p += kSchedThreads) sh.keys[p] = ~0ull;
  __syncthreads();

  // survival products and keys, one request per thread
  for (int r = tid; r < B; r += kSchedThreads) {
    const float* c = a.conf + (size_t)r * G;
    int bad = 0;
    for (int j = 0; j < G; ++j) bad |= !(c[j] >= 0.f && c[j] <= 1.f);
    if (a.status) a.status[r] = bad ? SPEC_REQ_BAD_CONFIDENCE : 0;
    float s = 1.f;
    int n = 0;
    for (int j = 0; j < G; ++j) {
      s = (j == 0) ? c[0] : __fmul_rn(s, c[j]);
      unsigned long long key = ~0ull;
      if (!bad && s > 0.f) {
        key = ((unsigned long long)(~__float_as_uint(s)) << 32) | (unsigned)(r * G + j);
        ++n;
      }
      sh.keys[r * G + j] = key;
    }
    if (n) atomicAdd(&sh.ncand, n);
  }
  __syncthreads();

  // bitonic sort, ascending
  for (int size = 2; size <= NP; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < (NP >> 1); t += kSchedThreads) {
        const int pos = 2 * t - (t & (stride - 1));
        const int par = pos + stride;
        const unsigned long long x = sh.keys[pos], y = sh.keys[par];
        const bool up = (pos & size) == 0;
        if ((x > y) == up) {
          sh.keys[pos] = y;
          sh.keys[par] = x;
        }
      }
      __syncthreads();
    }
  }

  const int E = sh.ncand;
  int m_max = a.budget - B;
  if (m_max > E) m_max = E;
  if (m_max < 0) m_max = 0;

  // exclusive scan of q over sorted positions 0 .. m_max-1 (chunk per thread)
  const int cpt = (NP + kSchedThreads - 1) / kSchedThreads;
  const int p0 = tid * cpt;
  long long local = 0;
  for (int p = p0; p < p0 + cpt; ++p)
    if (p < m_max) local += fixed_q(__uint_as_float(~(unsigned)(sh.keys[p] >> 32)));
  long long incl = wave_inclusive_sum_i64(local, lane);
  if (lane == 63) sh.wsum[wave] = incl;
  __syncthreads();
  long long before = 0;
  for (int w = 0; w < wave; ++w) before += sh.wsum[w];
  long long tau = (long long)B * kOne + before + (incl - local);  // tau at m = p0

  // Theta along the path; admission m uses sorted position m-1
  const double th0 = theta_of((long long)B * kOne, a.sps[B]);
  int brk = 0x7fffffff;           // first m >= 1 with Theta(m) <= Theta(m-1)
  double best = -INFINITY;        // global: max Theta over this thread's m
  int best_m = 0x7fffffff;
  for (int p = p0; p < p0 + cpt; ++p) {
    const int m = p + 1;
    if (m > m_max) break;
    const long long prev = tau;
    tau += fixed_q(__uint_as_float(~(unsigned)(sh.keys[p] >> 32)));
    const double tm = theta_of(tau, a.sps[B + m]);
    const double tp = theta_of(prev, a.sps[B + m - 1]);
    if (!(tm > tp) && m < brk) brk = m;
    if (tm > best) {
      best = tm;
      best_m = m;
    }
  }
  // block reductions
  int wb = wave_min_i(brk);
  double wbest = best;
  int wbm = best_m;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double ob = __shfl_xor(wbest, o, SPEC_WAVE);
    const int om = __shfl_xor(wbm, o, SPEC_WAVE);
    if (ob > wbest || (ob == wbest && om < wbm)) {
      wbest = ob;
      wbm = om;
    }
  }
  __syncthreads();
  if (lane == 0) {
    sh.wm[wave] = wb;
    sh.wth[wave] = wbest;
    sh.wsum[wave] = wbm;
  }
  __syncthreads();
  if (tid == 0) {
    int mstar;
    double th;
    if (a.mode == SPEC_SCHED_EARLY_STOP) {
      int b = 0x7fffffff;
      for (int w = 0; w < NW; ++w) b = min(b, sh.wm[w]);
      mstar = (b == 0x7fffffff) ? m_max : b - 1;
    } else {
      double bt = th0;
      int bm = 0;
      for (int w = 0; w < NW; ++w) {
        const double t = sh.wth[w];
        const int m = (int)sh.wsum[w];
        if (t > bt || (t == bt && m < bm)) {
          bt = t;
          bm = m;
        }
      }
      mstar = bm;
    }
    // Theta at m*: recompute tau exactly
    long long t = (long long)B * kOne;
    for (int p = 0; p < mstar; ++p) t += fixed_q(__uint_as_float(~(unsigned)(sh.keys[p] >> 32)));
    th = theta_of(t, a.sps[B + mstar]);
    sh.mstar = mstar;
    sh.theta_star = th;
    if (a.theta) a.theta[0] = th;
  }
  for (int r = tid; r < B; r += kSchedThreads) a.lengths[r] = 0;
  __syncthreads();
  const int mstar = sh.mstar;
  for (int p = tid; p < mstar; p += kSchedThreads) {
    const unsigned idx = (unsigned)(sh.keys[p] & 0xffffffffu);
    const int r = (int)(idx / (unsigned)G), j = (int)(idx % (unsigned)G);
    atomicMax(&a.lengths[r], j + 1);
  }
}

}  // namespace spec

using namespace spec;

extern "C" size_t spec_schedule_workspace_size(int32_t B, int32_t gamma) {
  (void)B;
  (void)gamma;
  return 0;
}

extern "C" int32_t spec_schedule_lengths(int32_t B, int32_t gamma, const float* conf, const double* sps,
                                         int32_t sps_len, int32_t budget_tokens, int32_t mode,
                                         int32_t* lengths_out, double* theta_out, int32_t* status,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (B < 1 || gamma < 1 || gamma > SPEC_MAX_GAMMA) return SPEC_ERR_INVALID_ARG;
  if ((long long)B * gamma > SPEC_MAX_SCHED_CANDIDATES) return SPEC_ERR_UNSUPPORTED;
  if (mode != SPEC_SCHED_EARLY_STOP && mode != SPEC_SCHED_GLOBAL) return SPEC_ERR_INVALID_ARG;
  if (!conf || !sps || !lengths_out) return SPEC_ERR_INVALID_ARG;
  long long m_cap = (long long)budget_tokens - B;
  if (m_cap < 0) m_cap = 0;
  if (m_cap > (long long)B * gamma) m_cap = (long long)B * gamma;
  if ((long long)sps_len <= (long long)B + m_cap) return SPEC_ERR_INVALID_ARG;
  SchedArgs a{B, gamma, budget_tokens, mode, conf, sps, lengths_out, theta_out, status};
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, reinterpret_cast<hipStream_t>(stream), a);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}
