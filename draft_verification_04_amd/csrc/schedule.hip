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
// position) -> bitonic sort held in registers (lane shuffles, LDS only for the
// longest strides) -> exclusive int64 scan -> Theta(m) -> first non-rise
// (early stop) or first maximum (global) -> per-request counts.
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
};

__device__ __forceinline__ long long fixed_q(float a) {
  // floor(a * 2^50): a is a float32 in [0, 1]; the product is exact in fp64
  return (long long)floor((double)a * 0x1p50);
}

__device__ __forceinline__ double theta_of(long long tau, double sps) {
  return ((double)tau * 0x1p-50) * sps;
}

// Bitonic sort of NP = K * kSchedThreads keys, ascending; thread t holds positions t*K .. t*K+K-1.
// Strides below K compare in registers, strides below 64*K across lanes of a wave, longer ones
// through LDS.
template <int K>
__device__ __forceinline__ void bitonic_regs(unsigned long long (&key)[K], unsigned long long* lds, int tid,
                                             int lane) {
  constexpr int NP = K * kSchedThreads;
  for (int size = 2; size <= NP; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < K) {
#pragma unroll
        for (int e = 0; e < K; ++e) {
          const int pe = e ^ stride;
          if (pe > e) {
            const int pos = tid * K + e;
            const bool up = (pos & size) == 0;
            const unsigned long long x = key[e], y = key[pe];
            if ((x > y) == up) {
              key[e] = y;
              key[pe] = x;
            }
          }
        }
      } else if (stride < 64 * K) {
        const int lx = stride / K;
        const bool lower = (lane & lx) == 0;
#pragma unroll
        for (int e = 0; e < K; ++e) {
          const int pos = tid * K + e;
          const bool up = (pos & size) == 0;
          const unsigned long long y = __shfl_xor(key[e], lx, SPEC_WAVE);
          const unsigned long long x = key[e];
          // the lower position keeps the smaller key when ascending
          key[e] = (lower == up) ? (x < y ? x : y) : (x < y ? y : x);
        }
      } else {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < K; ++e) lds[tid * K + e] = key[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < K; ++e) {
          const int pos = tid * K + e;
          const bool up = (pos & size) == 0;
          const bool lower = (pos & stride) == 0;
          const unsigned long long y = lds[pos ^ stride];
          const unsigned long long x = key[e];
          key[e] = (lower == up) ? (x < y ? x : y) : (x < y ? y : x);
        }
      }
    }
  }
}

template <int K>
__device__ void schedule_body(const SchedArgs& a, SchedShared& sh) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int NW = kSchedThreads / SPEC_WAVE;
  const int B = a.B, G = a.G;
  const int N = B * G;
  constexpr int NP = K * kSchedThreads;
  if (tid == 0) sh.ncand = 0;
  // confidences staged in the key slots (coalesced loads); each request's thread then reads
  // its slots and overwrites them with the keys
  for (int p = tid; p < NP; p += kSchedThreads)
    sh.keys[p] = (p < N) ? (unsigned long long)__float_as_uint(a.conf[p]) : ~0ull;
  __syncthreads();

  // survival products and keys, one request per thread
  for (int r = tid; r < B; r += kSchedThreads) {
    unsigned long long* c = sh.keys + (size_t)r * G;   // confidence bits, read before overwritten
    int bad = 0;
    for (int j = 0; j < G; ++j) {
      const float cj = __uint_as_float((unsigned)c[j]);
      bad |= !(cj >= 0.f && cj <= 1.f);
    }
    if (a.status) a.status[r] = bad ? SPEC_REQ_BAD_CONFIDENCE : 0;
    float s = 1.f;
    int n = 0;
    for (int j = 0; j < G; ++j) {
      const float cj = __uint_as_float((unsigned)c[j]);
      s = (j == 0) ? cj : __fmul_rn(s, cj);
      unsigned long long key = ~0ull;
      if (!bad && s > 0.f) {
        key = ((unsigned long long)(~__float_as_uint(s)) << 32) | (unsigned)(r * G + j);
        ++n;
      }
      c[j] = key;
    }
    if (n) atomicAdd(&sh.ncand, n);
  }
  __syncthreads();
  unsigned long long key[K];
#pragma unroll
  for (int e = 0; e < K; ++e) key[e] = sh.keys[tid * K + e];
  bitonic_regs<K>(key, sh.keys, tid, lane);

  const int E = sh.ncand;
  int m_max = a.budget - B;
  if (m_max > E) m_max = E;
  if (m_max < 0) m_max = 0;

  // exclusive scan of q over sorted positions 0 .. m_max-1 (K per thread)
  const int p0 = tid * K;
  long long q[K];
  long long local = 0;
#pragma unroll
  for (int e = 0; e < K; ++e) {
    q[e] = (p0 + e < m_max) ? fixed_q(__uint_as_float(~(unsigned)(key[e] >> 32))) : 0;
    local += q[e];
  }
  long long incl = wave_inclusive_sum_i64(local, lane);
  __syncthreads();
  if (lane == 63) sh.wsum[wave] = incl;
  __syncthreads();
  long long before = 0;
  for (int w = 0; w < wave; ++w) before += sh.wsum[w];
  long long tau = (long long)B * kOne + before + (incl - local);  // tau at m = p0
  const long long tau_p0 = tau;

  // Theta along the path; admission m uses sorted position m-1
  const double th0 = theta_of((long long)B * kOne, a.sps[B]);
  int brk = 0x7fffffff;           // first m >= 1 with Theta(m) <= Theta(m-1)
  double best = -INFINITY;        // global: max Theta over this thread's m
  int best_m = 0x7fffffff;
#pragma unroll
  for (int e = 0; e < K; ++e) {
    const int m = p0 + e + 1;
    if (m <= m_max) {
      const long long prev = tau;
      tau += q[e];
      const double tm = theta_of(tau, a.sps[B + m]);
      const double tp = theta_of(prev, a.sps[B + m - 1]);
      if (!(tm > tp) && m < brk) brk = m;
      if (tm > best) {
        best = tm;
        best_m = m;
      }
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
    sh.mstar = mstar;
    if (mstar == 0 && a.theta) a.theta[0] = th0;
  }
  for (int r = tid; r < B; r += kSchedThreads) a.lengths[r] = 0;
  __syncthreads();
  const int mstar = sh.mstar;
  // Theta at m*: the thread holding sorted position m*-1 recomputes tau from its chunk
  if (mstar > 0 && mstar - 1 >= p0 && mstar - 1 < p0 + K && a.theta) {
    long long t = tau_p0;
#pragma unroll
    for (int e = 0; e < K; ++e)
      if (p0 + e < mstar) t += q[e];
    a.theta[0] = theta_of(t, a.sps[B + mstar]);
  }
  // per-request counts: admitted positions form a prefix of each request's candidates
#pragma unroll
  for (int e = 0; e < K; ++e) {
    if (p0 + e < mstar) {
      const unsigned idx = (unsigned)(key[e] & 0xffffffffu);
      const int r = (int)(idx / (unsigned)G), j = (int)(idx % (unsigned)G);
      atomicMax(&a.lengths[r], j + 1);
    }
  }
}

template <int K>
__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(SchedArgs a) {
  __shared__ SchedShared sh;
  schedule_body<K>(a, sh);
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
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const long long n = (long long)B * gamma;
  if (n <= 1 * kSchedThreads) hipLaunchKernelGGL(schedule_kernel<1>, dim3(1), dim3(kSchedThreads), 0, s, a);
  else if (n <= 2 * kSchedThreads) hipLaunchKernelGGL(schedule_kernel<2>, dim3(1), dim3(kSchedThreads), 0, s, a);
  else if (n <= 4 * kSchedThreads) hipLaunchKernelGGL(schedule_kernel<4>, dim3(1), dim3(kSchedThreads), 0, s, a);
  else if (n <= 8 * kSchedThreads) hipLaunchKernelGGL(schedule_kernel<8>, dim3(1), dim3(kSchedThreads), 0, s, a);
  else hipLaunchKernelGGL(schedule_kernel<16>, dim3(1), dim3(kSchedThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}
