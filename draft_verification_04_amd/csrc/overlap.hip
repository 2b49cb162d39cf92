// Overlap mass per draft position on gfx950: c*_{i,k} = sum_v min(p_t,k(v), p_d,k(v)).
//
// DSpark paper, §3.2.1, Eq. 8: the probability that draft position k is accepted once it is
// reached is the overlap of the target and draft distributions there (also
// 1 - (1/2) ||p_t - p_d||_1); it is the label of the confidence head and the per-position
// factor of the expected accepted length.  The distributions are those of verification:
// softmax of z / T over the kept set (top-k with ties kept).
//
// Steps: the verification work list restricted to draft positions k < L_i, the streaming
// statistics and the combining step (row lse2 and top-k thresholds, no acceptance test), then
// overlap_pass_kernel streams target row k and draft row k together a second time, segment by
// segment, adding min(p_t, p_d) per token (p = 2^(z c - lse2) in fp32 with the split constants
// of the streaming kernel, sums in fp64), and overlap_finish_kernel adds the segments and writes
// the outputs and status words.
#include "common.hpp"
#include "verify_impl.hpp"
#include "spec_verify.h"

#include <math.h>

namespace spec {

constexpr int kOverlapThreads = 512;

// p = 2^(z c - l2) for a kept token (z >= th), else 0: c = c_hi + c_lo and l2 = l2_hi + l2_lo
// split into float pairs, so that the exponent carries one rounding at its own scale.
__device__ __forceinline__ float row_prob(float z, float c_hi, float c_lo, float l2_hi, float l2_lo, float th) {
  const float e = fmaf(z, c_lo, fmaf(z, c_hi, -l2_hi) - l2_lo);
  return (z >= th) ? __builtin_amdgcn_exp2f(e) : 0.f;
}

struct OverlapShared {
  double wsum[kOverlapThreads / SPEC_WAVE];
};

template <bool BF16>
__global__ __launch_bounds__(kOverlapThreads) void overlap_pass_kernel(VerifyArgs a, double* part) {
  __shared__ OverlapShared sh;
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  const int nseg = a.nseg;
  const int g = (int)blockIdx.x / nseg, seg = (int)blockIdx.x - g * nseg;
  if (g >= *a.nitems) return;
  const int item = a.items[g];
  const int i = item >> 7, k = item & 127;
  const int G = a.G, V = a.V;
  const float T = a.temperature[i];
  if (!(T > 0.f && T < INFINITY)) return;
  if (a.top_k && a.top_k[i] < 0) return;
  const RowStat rt = a.rows_t[(size_t)i * (G + 1) + k];
  const RowStat rd = a.rows_d[(size_t)i * G + k];
  if (!(rt.lse2 == rt.lse2) || !(rd.lse2 == rd.lse2)) return;   // reported as bad data
  const double c64 = kLog2e / (double)T;
  const float c_hi = __double2float_rz(c64);
  const float c_lo = (float)(c64 - (double)c_hi);
  const float lt_hi = (float)rt.lse2, lt_lo = (float)(rt.lse2 - (double)lt_hi);
  const float ld_hi = (float)rd.lse2, ld_lo = (float)(rd.lse2 - (double)ld_hi);
  const char* trow = target_row<ES>(a, i, k);
  const char* drow = draft_row<ES>(a, i, k);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  double acc = 0.0;
  const bool vec = ((reinterpret_cast<uintptr_t>(trow) | reinterpret_cast<uintptr_t>(drow)) & 15u) == 0;
  const int nvec = vec ? V / EPV : 0;   // whole 16-byte vectors of both rows, then a scalar tail
  const int vb = (int)((long long)nvec * seg / nseg), ve = (int)((long long)nvec * (seg + 1) / nseg);
  const uint4* tv = reinterpret_cast<const uint4*>(trow);
  const uint4* dv = reinterpret_cast<const uint4*>(drow);
  for (int v = vb + tid; v < ve; v += kOverlapThreads) {
    const uint4 xt = load_nt(tv + v), xd = load_nt(dv + v);
    const uint32_t wt[4] = {xt.x, xt.y, xt.z, xt.w}, wd[4] = {xd.x, xd.y, xd.z, xd.w};
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (BF16) {
        s += fminf(row_prob(bf16_lo(wt[q]), c_hi, c_lo, lt_hi, lt_lo, rt.theta),
                   row_prob(bf16_lo(wd[q]), c_hi, c_lo, ld_hi, ld_lo, rd.theta));
        s += fminf(row_prob(bf16_hi(wt[q]), c_hi, c_lo, lt_hi, lt_lo, rt.theta),
                   row_prob(bf16_hi(wd[q]), c_hi, c_lo, ld_hi, ld_lo, rd.theta));
      } else {
        s += fminf(row_prob(__uint_as_float(wt[q]), c_hi, c_lo, lt_hi, lt_lo, rt.theta),
                   row_prob(__uint_as_float(wd[q]), c_hi, c_lo, ld_hi, ld_lo, rd.theta));
      }
    }
    acc += (double)s;
  }
  if (seg == nseg - 1) {
    // the scalar tail (or the whole row when the rows are not both 16-byte aligned)
    for (int v = nvec * EPV + tid; v < V; v += kOverlapThreads) {
      const float zt = load_elem<BF16>(trow, v), zd = load_elem<BF16>(drow, v);
      acc += (double)fminf(row_prob(zt, c_hi, c_lo, lt_hi, lt_lo, rt.theta),
                           row_prob(zd, c_hi, c_lo, ld_hi, ld_lo, rd.theta));
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) sh.wsum[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int w = 0; w < kOverlapThreads / SPEC_WAVE; ++w) t += sh.wsum[w];
    part[((size_t)i * G + k) * nseg + seg] = t;
  }
}

// One thread per (request, draft position): status and c* = the sum of the segment parts.
__global__ __launch_bounds__(256) void overlap_finish_kernel(VerifyArgs a, const double* part, double* out) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int G = a.G;
  if (t >= (long long)a.B * G) return;
  const int i = (int)(t / G), k = (int)(t - (long long)i * G);
  const int L = a.lengths ? a.lengths[i] : G;
  const float T = a.temperature[i];
  const int K = a.top_k ? a.top_k[i] : 0;
  int st = 0;
  if (L < 0 || L > G) {
    st = SPEC_REQ_BAD_LENGTH;
  } else {
    if (!(T >= 0.f && T < INFINITY)) st |= SPEC_REQ_BAD_TEMPERATURE;
    if (K < 0) st |= SPEC_REQ_BAD_TOPK;
    if (st == 0 && T > 0.f) st |= a.req_status[i];
  }
  if (k == 0 && a.status) a.status[i] = st;
  double c = NAN;
  if (st == 0 && T > 0.f && k < L) {
    c = 0.0;
    for (int s = 0; s < a.nseg; ++s) c += part[((size_t)i * G + k) * a.nseg + s];
  }
  out[t] = c;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline size_t part_bytes(int B, int G) { return align256(sizeof(double) * (size_t)B * G * 16); }

}  // namespace spec

using namespace spec;

extern "C" size_t spec_overlap_workspace_size(int32_t B, int32_t gamma, int32_t V) {
  if (B < 1 || gamma < 1 || gamma > SPEC_MAX_GAMMA || V < 1 || V > SPEC_MAX_V) return 0;
  return workspace_bytes(B, gamma, V, false, true) + part_bytes(B, gamma);
}

extern "C" int32_t spec_overlap_mass(int32_t B, int32_t gamma, int32_t V, int32_t dtype, const void* target_logits,
                                     const void* draft_logits, const int32_t* lengths, const float* temperature,
                                     const int32_t* top_k, double* overlap_out, int32_t* status, void* workspace,
                                     size_t workspace_bytes_, void* stream) {
  if (!shape_ok(B, gamma, V, dtype)) return SPEC_ERR_INVALID_ARG;
  if (!target_logits || !draft_logits || !temperature || !overlap_out) return SPEC_ERR_INVALID_ARG;
  if (!aligned16(target_logits) || !aligned16(draft_logits)) return SPEC_ERR_INVALID_ARG;
  VerifyArgs a{};
  a.B = B; a.G = gamma; a.V = V; a.greedy_only = 0; a.overlap_only = 1;
  a.target = target_logits; a.draft = draft_logits; a.tokens = nullptr; a.lengths = lengths;
  a.temperature = temperature; a.top_k = top_k; a.seed = nullptr; a.status = status;
  char* extra = nullptr;
  const int32_t rc = bind_workspace(a, dtype, workspace, workspace_bytes_, part_bytes(B, gamma), &extra);
  if (rc != SPEC_OK) return rc;
  double* part = reinterpret_cast<double*>(extra);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  launch_statistics(a, dtype, s, nullptr, nullptr);
  launch_combine(a, s);
  const unsigned grid = (unsigned)((size_t)B * gamma * a.nseg);
  if (dtype == SPEC_BF16)
    hipLaunchKernelGGL(overlap_pass_kernel<true>, dim3(grid), dim3(kOverlapThreads), 0, s, a, part);
  else
    hipLaunchKernelGGL(overlap_pass_kernel<false>, dim3(grid), dim3(kOverlapThreads), 0, s, a, part);
  const unsigned fgrid = (unsigned)(((size_t)B * gamma + 255) / 256);
  hipLaunchKernelGGL(overlap_finish_kernel, dim3(fgrid), dim3(256), 0, s, a, part, overlap_out);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}
