// Sequential Temperature Scaling of the confidence head on gfx950.
//
// DSpark paper, §3.2.1 (post-hoc calibration): per-position temperatures tau_k, fitted left to
// right; position k takes the grid value that minimises the Expected Calibration Error of the
// survival product a_k = c_1(tau_1) ... c_k(tau_k), c_i(tau) = sigmoid(t_i / tau), with the
// temperatures of positions < k fixed.  ECE over equal-width bins: (1/N) sum_b |sum_{n in b}
// (a_n - y_n)|, y_n = 1 when the prefix through k survived.
//
// Per position:
//   sts_bins_kernel   -- one workgroup per chunk of instances, one thread per grid temperature:
//                        the chunk's t_k, a_{k-1} and labels are staged in LDS (every thread reads
//                        the same instance at once: broadcast), each thread accumulates its own
//                        bins in a private LDS column, in instance order, and writes them out.
//                        Deterministic: no atomics, every sum has a fixed order.
//   sts_ece_kernel    -- one workgroup per grid temperature: the chunk partials of each bin summed
//                        in a fixed tree order, the ECE.
//   sts_select_kernel -- the first grid value with the smallest ECE (NaN never wins).
//   sts_update_kernel -- a_k = a_{k-1} * sigmoid(t_k / tau_k) for every instance.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.hpp"
#include "spec_verify.h"

namespace spec {
namespace {

constexpr int kStsThreads = 256;   // grid temperatures per workgroup of sts_bins_kernel
constexpr int kStsChunk = 512;     // instances per workgroup of sts_bins_kernel (4 per CU at 15 bins)
constexpr int kStsMaxBins = 32;
constexpr int kStsMaxTaus = 4096;

struct StsArgs {
  int N, G, k, ntau, bins, nchunk;
  const float* logits;     // [N, G]
  const uint8_t* labels;   // [N, G]
  const double* taus;      // [ntau]
  double* tau_out;         // [G]
  int32_t* index_out;      // [G] or null
  double* ece_out;         // [G, ntau] or null
  double* a_prev;          // [N] workspace
  double* part;            // [ntau, bins, nchunk] workspace
  double* ece;             // [ntau] workspace
};

__device__ __forceinline__ double sigmoid64(double x) { return 1.0 / (1.0 + exp(-x)); }

__global__ __launch_bounds__(256) void sts_init_kernel(double* a, int N) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n < N) a[n] = 1.0;
}

__global__ __launch_bounds__(kStsThreads) void sts_bins_kernel(StsArgs a) {
  __shared__ float sl[kStsChunk];
  __shared__ double sa[kStsChunk];
  __shared__ float sy[kStsChunk];
  extern __shared__ double sb[];  // [bins][kStsThreads]: thread-private columns
  const int tid = threadIdx.x;
  const int c = blockIdx.x;                     // chunk
  const int g = blockIdx.y * kStsThreads + tid;  // grid temperature
  const int n0 = c * kStsChunk;
  const int cn = min(kStsChunk, a.N - n0);
  for (int i = tid; i < cn; i += kStsThreads) {
    const size_t n = (size_t)(n0 + i);
    sl[i] = a.logits[n * a.G + a.k];
    sa[i] = a.a_prev[n];
    sy[i] = a.labels[n * a.G + a.k] ? 1.f : 0.f;
  }
  const int M = a.bins;
  for (int b = 0; b < M; ++b) sb[b * kStsThreads + tid] = 0.0;
  __syncthreads();
  if (g < a.ntau) {
    const double tau = a.taus[g];
    const double fM = (double)M;
    for (int i = 0; i < cn; ++i) {
      const double v = sa[i] * sigmoid64((double)sl[i] / tau);
      int b = 0;
      if (v == v) b = (int)fmin(floor(v * fM), fM - 1.0);  // NaN adds to bin 0 (and stays NaN)
      b = max(b, 0);
      sb[b * kStsThreads + tid] += v - (double)sy[i];
    }
    double* out = a.part + (size_t)g * M * a.nchunk + c;
    for (int b = 0; b < M; ++b) out[(size_t)b * a.nchunk] = sb[b * kStsThreads + tid];
  }
}

// One workgroup per grid temperature: per bin, the chunk partials summed in a fixed order (each
// thread its strided share, then the wave by a DPP reduction, then the four waves in order).
__global__ __launch_bounds__(256) void sts_ece_kernel(StsArgs a) {
  __shared__ double wpart[kStsMaxBins][4];
  const int g = blockIdx.x, tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int M = a.bins;
  for (int b = 0; b < M; ++b) {
    const double* p = a.part + ((size_t)g * M + b) * a.nchunk;
    double s = 0.0;
    for (int c = tid; c < a.nchunk; c += 256) s += p[c];
    s = wave_sum(s);
    if (lane == 0) wpart[b][wave] = s;
  }
  __syncthreads();
  if (tid == 0) {
    double e = 0.0;
    for (int b = 0; b < M; ++b) e += fabs((wpart[b][0] + wpart[b][1]) + (wpart[b][2] + wpart[b][3]));
    e /= (double)a.N;
    a.ece[g] = e;
    if (a.ece_out) a.ece_out[(size_t)a.k * a.ntau + g] = e;
  }
}

// The first grid value with the smallest ECE; NaN values never win (all NaN: tau = NaN).
__global__ __launch_bounds__(256) void sts_select_kernel(StsArgs a) {
  __shared__ double bv[256];
  __shared__ int bi[256];
  const int tid = threadIdx.x;
  double best = __builtin_nan("");
  int bidx = 0x7fffffff;
  for (int g = tid; g < a.ntau; g += 256) {
    const double e = a.ece[g];
    if (e == e && (!(best == best) || e < best)) {  // ascending g: the first minimum is kept
      best = e;
      bidx = g;
    }
  }
  bv[tid] = best;
  bi[tid] = bidx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) {
      const double e = bv[tid + o];
      const int i = bi[tid + o];
      const double m = bv[tid];
      if (e == e && (!(m == m) || e < m || (e == m && i < bi[tid]))) {
        bv[tid] = e;
        bi[tid] = i;
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    const bool found = bv[0] == bv[0];
    a.tau_out[a.k] = found ? a.taus[bi[0]] : __builtin_nan("");
    if (a.index_out) a.index_out[a.k] = found ? bi[0] : -1;
  }
}

__global__ __launch_bounds__(256) void sts_update_kernel(StsArgs a) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  if (n >= a.N) return;
  const double tau = a.tau_out[a.k];
  a.a_prev[n] = a.a_prev[n] * sigmoid64((double)a.logits[(size_t)n * a.G + a.k] / tau);
}

__global__ __launch_bounds__(256) void sts_apply_kernel(const float* t, const double* tau, float* out, int B, int G) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)B * G) return;
  out[i] = (float)sigmoid64((double)t[i] / tau[i % G]);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int num_chunks(int N) { return (N + kStsChunk - 1) / kStsChunk; }

size_t sts_ws_bytes(int N, int ntau, int bins) {
  return align256((size_t)N * sizeof(double)) + align256((size_t)ntau * bins * num_chunks(N) * sizeof(double)) +
         align256((size_t)ntau * sizeof(double));
}

bool sts_shape_ok(int N, int G, int ntau, int bins) {
  return N >= 1 && N <= (1 << 26) && G >= 1 && G <= SPEC_MAX_GAMMA && ntau >= 1 && ntau <= kStsMaxTaus &&
         bins >= 1 && bins <= kStsMaxBins;
}

}  // namespace
}  // namespace spec

using namespace spec;

extern "C" size_t spec_sts_workspace_size(int32_t N, int32_t ntau, int32_t bins) {
  if (!sts_shape_ok(N, 1, ntau, bins)) return 0;
  return sts_ws_bytes(N, ntau, bins);
}

extern "C" int32_t spec_sts_fit(int32_t N, int32_t gamma, const float* conf_logits, const uint8_t* labels,
                                int32_t ntau, const double* taus, int32_t bins, double* tau_out, int32_t* index_out,
                                double* ece_out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!sts_shape_ok(N, gamma, ntau, bins)) return SPEC_ERR_INVALID_ARG;
  if (!conf_logits || !labels || !taus || !tau_out) return SPEC_ERR_INVALID_ARG;
  const size_t need = sts_ws_bytes(N, ntau, bins);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return SPEC_ERR_WORKSPACE;
  StsArgs a{};
  a.N = N; a.G = gamma; a.ntau = ntau; a.bins = bins; a.nchunk = num_chunks(N);
  a.logits = conf_logits; a.labels = labels; a.taus = taus;
  a.tau_out = tau_out; a.index_out = index_out; a.ece_out = ece_out;
  char* ws = reinterpret_cast<char*>(workspace);
  a.a_prev = reinterpret_cast<double*>(ws);
  ws += align256((size_t)N * sizeof(double));
  a.part = reinterpret_cast<double*>(ws);
  ws += align256((size_t)ntau * bins * a.nchunk * sizeof(double));
  a.ece = reinterpret_cast<double*>(ws);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned ng = (unsigned)((N + 255) / 256);
  hipLaunchKernelGGL(sts_init_kernel, dim3(ng), dim3(256), 0, s, a.a_prev, N);
  const dim3 bgrid((unsigned)a.nchunk, (unsigned)((ntau + kStsThreads - 1) / kStsThreads));
  for (int k = 0; k < gamma; ++k) {
    a.k = k;
    hipLaunchKernelGGL(sts_bins_kernel, bgrid, dim3(kStsThreads), (size_t)bins * kStsThreads * sizeof(double), s, a);
    hipLaunchKernelGGL(sts_ece_kernel, dim3((unsigned)ntau), dim3(256), 0, s, a);
    hipLaunchKernelGGL(sts_select_kernel, dim3(1), dim3(256), 0, s, a);
    hipLaunchKernelGGL(sts_update_kernel, dim3(ng), dim3(256), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

extern "C" int32_t spec_sts_apply(int32_t B, int32_t gamma, const float* conf_logits, const double* tau,
                                  float* conf_out, void* stream) {
  if (B < 1 || gamma < 1 || gamma > SPEC_MAX_GAMMA || (size_t)B * gamma > ((size_t)1 << 30))
    return SPEC_ERR_INVALID_ARG;
  if (!conf_logits || !tau || !conf_out) return SPEC_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned grid = (unsigned)(((size_t)B * gamma + 255) / 256);
  hipLaunchKernelGGL(sts_apply_kernel, dim3(grid), dim3(256), 0, s, conf_logits, tau, conf_out, B, gamma);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}
