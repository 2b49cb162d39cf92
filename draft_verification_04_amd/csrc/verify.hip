// Lossless draft verification on gfx950: work list, row-streaming statistics
// with the acceptance test.  The emitted token is computed in emit.hip.
//
// What is computed follows the DSpark paper, §2.1 (accept x_k with
// probability min(1, p_t(x_k) / p_d(x_k)), left to right, the first
// rejection ends the block) and §1 (one extra token from the target after the
// accepted prefix); a request verified at length 0 draws a fresh target token
// (the paper's appendix counterexample).  The correction after a rejection
// is drawn from the normalised max(0, p_t - p_d).
//
// Kernels
//   worklist_kernel  one workgroup: (request, position) items in
//                    position-major order for every position k <= L_i.
//   stream_kernel    one workgroup per item: streams target row k (and draft
//                    row k when k < L_i) once from HBM with 16-byte loads,
//                    computes log2-sum-exp of z * log2(e) / T (or the argmax
//                    for the greedy rule, or the top-k threshold first), then
//                    the acceptance test of x_k with its Philox uniform.
//   (emit.hip)       the emitted token of every request and all outputs.
#include "common.hpp"
#include "philox.hpp"
#include "verify_impl.hpp"

#include <hip/hip_ext.h>
#include "spec_verify.h"

#include <algorithm>
#include <mutex>

#include <float.h>
#include <math.h>

namespace spec {

// ---------------------------------------------------------------------------
// worklist
// ---------------------------------------------------------------------------

// Last position k of request i that gets a work item: L_i (verification: the rows k <= L_i), or
// L_i - 1 when only the draft positions' statistics are wanted; -1 for none or a bad length.
__device__ __forceinline__ int last_item(const VerifyArgs& a, int i) {
  const int L = a.lengths ? a.lengths[i] : a.G;
  if (L < 0 || L > a.G) return -1;
  if (a.req_status[i] & (SPEC_REQ_OVER_BUDGET | SPEC_REQ_BAD_ROWS)) return -1;
  return a.overlap_only ? L - 1 : L;
}

__global__ __launch_bounds__(kWorklistThreads) void worklist_kernel(VerifyArgs a) {
  __shared__ int hist[SPEC_MAX_GAMMA + 2];
  __shared__ int off[SPEC_MAX_GAMMA + 2];
  __shared__ int carry[SPEC_MAX_GAMMA + 1];
  __shared__ int cnt[kWorklistThreads / SPEC_WAVE][SPEC_MAX_GAMMA + 1];
  __shared__ long long woff_t[kWorklistThreads / SPEC_WAVE], woff_d[kWorklistThreads / SPEC_WAVE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = a.G, B = a.B;
  for (int t = tid; t < G + 2; t += blockDim.x) hist[t] = 0;
  for (int t = tid; t < G + 1; t += blockDim.x) carry[t] = 0;
  if (a.max_items > 0) {
    // token cap: requests are admitted in index order while sum (L_i + 1) stays within it; the
    // rest are marked and get no work items
    long long carry_n = 0;
    for (int b0 = 0; b0 < B; b0 += blockDim.x) {
      const int i = b0 + tid;
      const int L = (i < B) ? (a.lengths ? a.lengths[i] : G) : -1;
      const long long n = (L >= 0 && L <= G) ? L + 1 : 0;
      const long long in = wave_inclusive_sum_i64(n, lane);
      __syncthreads();
      if (lane == 63) woff_t[wave] = in;
      __syncthreads();
      long long bt = carry_n, tt = 0;
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
        if (w < wave) bt += woff_t[w];
        tt += woff_t[w];
      }
      if (i < B) a.req_status[i] = (n > 0 && bt + in > (long long)a.max_items) ? SPEC_REQ_OVER_BUDGET : 0;
      carry_n += tt;
    }
  } else {
    for (int i = tid; i < B; i += blockDim.x) a.req_status[i] = 0;
  }
  __syncthreads();
  if (a.flat) {
    // first target / draft row of every request in the flattened layout (a bad length counts
    // as no rows): exclusive prefix sums of L_i + 1 and L_i, block by block.  Thread tid
    // handles requests b0 + tid, as when the status words were set above.
    long long carry_t = 0, carry_d = 0;
    for (int b0 = 0; b0 < B; b0 += blockDim.x) {
      const int i = b0 + tid;
      const int L = (i < B) ? (a.lengths ? a.lengths[i] : G) : -1;
      const long long nt = (L >= 0 && L <= G) ? L + 1 : 0, nd = (L >= 0 && L <= G) ? L : 0;
      const long long it = wave_inclusive_sum_i64(nt, lane), id = wave_inclusive_sum_i64(nd, lane);
      __syncthreads();
      if (lane == 63) {
        woff_t[wave] = it;
        woff_d[wave] = id;
      }
      __syncthreads();
      long long bt = carry_t, bd = carry_d, tt = 0, td = 0;
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
        if (w < wave) {
          bt += woff_t[w];
          bd += woff_d[w];
        }
        tt += woff_t[w];
        td += woff_d[w];
      }
      if (i < B) {
        const long long t0 = bt + it - nt, d0 = bd + id - nd;
        a.t_off[i] = t0;
        a.d_off[i] = d0;
        // rows the caller did not pass: the request is marked and gets no work items
        if (t0 + nt > a.flat_trows || d0 + nd > a.flat_drows) a.req_status[i] |= SPEC_REQ_BAD_ROWS;
      }
      carry_t += tt;
      carry_d += td;
    }
  }
  __syncthreads();   // the marks are read below (global memory, this workgroup)
  for (int i = tid; i < B; i += blockDim.x) {
    a.ereq[i].amb_n = 0;
    const int L = last_item(a, i);
    if (L >= 0) atomicAdd(&hist[L], 1);
  }
  __syncthreads();
  if (tid == 0) {
    // c_k = #{i : L_i >= k}; items of position k start at off[k]
    int suffix = 0;
    for (int l = G; l >= 0; --l) {
      suffix += hist[l];
      hist[l] = suffix;
    }
    off[0] = 0;
    for (int k = 0; k <= G; ++k) off[k + 1] = off[k] + hist[k];
    *a.nitems = off[G + 1];
  }
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < B; base += blockDim.x) {
    const int i = base + tid;
    int L = -1;
    if (i < B) L = last_item(a, i);
    for (int k = 0; k <= G; ++k) {
      const unsigned long long m = __ballot(L >= k);
      if (lane == 0) cnt[wave][k] = __popcll(m);
    }
    __syncthreads();
    if (tid <= G) {
      int run = carry[tid];
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
        const int c = cnt[w][tid];
        cnt[w][tid] = run;
        run += c;
      }
      carry[tid] = run;
    }
    __syncthreads();
    // eight positions at a time: their draft tokens are loaded together, then the items written
    const bool want_x = a.tokens && !a.overlap_only;
    for (int k0 = 0; k0 <= G; k0 += 8) {
      int xs[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u;
        xs[u] = (want_x && k < L) ? a.tokens[(size_t)i * G + k] : -1;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k0 + u;
        if (k > G) break;
        const unsigned long long m = __ballot(L >= k);
        if (L >= k) {
          const int idx = off[k] + cnt[wave][k] + __popcll(m & below);
          a.items[idx] = (i << 7) | k;
          a.items_x[idx] = xs[u];
        }
      }
    }
    __syncthreads();
  }
}

// The same work list when every request has a thread of one workgroup (B <= kWorklistThreads,
// padded layout): the length, the cap mark and the first draft tokens stay in registers, and the
// per-position counts come from ballots, so the only global round trips are the lengths' and the
// tokens'.  Items are ordered as by worklist_kernel.
__global__ __launch_bounds__(kWorklistThreads) void worklist_small_kernel(VerifyArgs a) {
  __shared__ WorklistShared sh;
  const int tid = threadIdx.x;
  const int L = (tid < a.B) ? (a.lengths ? a.lengths[tid] : a.G) : -1;
  int xp[kWlPre];
  worklist_prefetch(a, xp);
  worklist_from_lengths(sh, a, L, xp);
}

// ---------------------------------------------------------------------------
// streaming statistics
// ---------------------------------------------------------------------------

// Row geometry: elements before the first 16-byte boundary (head), whole
// 16-byte vectors, and the elements after the last one (tail).
struct RowGeom {
  int head, nvec, tail;
};

template <bool BF16>
__device__ __forceinline__ RowGeom row_geom(const char* row, int V) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int h = (int)(((16u - (unsigned)(addr & 15u)) & 15u) / ES);
  if (h > V) h = V;
  const int nv = (V - h) / EPV;
  return RowGeom{h, nv, V - h - nv * EPV};
}

template <bool BF16>
__device__ __forceinline__ void unpack(const uint4& d, float (&z)[BF16 ? 8 : 4]) {
  if constexpr (BF16) {
    z[0] = bf16_lo(d.x); z[1] = bf16_hi(d.x);
    z[2] = bf16_lo(d.y); z[3] = bf16_hi(d.y);
    z[4] = bf16_lo(d.z); z[5] = bf16_hi(d.z);
    z[6] = bf16_lo(d.w); z[7] = bf16_hi(d.w);
  } else {
    z[0] = __uint_as_float(d.x); z[1] = __uint_as_float(d.y);
    z[2] = __uint_as_float(d.z); z[3] = __uint_as_float(d.w);
  }
}

// Per-thread running sum S of 2^(z*c - M) with an integer-valued reference M
// that only moves up.  z*c is formed as fma(z, c_lo, fma(z, c_hi, -M)), with
// c_hi + c_lo = log2(e)/T to ~2^-48 relative and c_lo > 0 (so -inf logits give
// -inf exponents).  M is raised only when a group's sum exceeds 2^32; then S
// is rescaled by an exact power of two.  A NaN or +inf logit sets `bad`.
template <int N>
__device__ __forceinline__ void accum(const float (&z)[N], float c_hi, float c_lo, float& M, float& S,
                                      int& bad) {
  float e[N];
#pragma unroll
  for (int j = 0; j < N; ++j) e[j] = __builtin_amdgcn_exp2f(fmaf(z[j], c_lo, fmaf(z[j], c_hi, -M)));
  float s = 0.f;
#pragma unroll
  for (int w = 1; w < N; w <<= 1)
#pragma unroll
    for (int j = 0; j + w < N; j += 2 * w) e[j] += e[j + w];
  s = e[0];
  if (!(s <= 0x1p32f)) {
    float vmax = z[0];
#pragma unroll
    for (int j = 1; j < N; ++j) vmax = fmaxf(vmax, z[j]);
    if (!(vmax < INFINITY)) {
      bad = 1;
      s = 0.f;
    } else {
      const float mc = ceilf(vmax * c_hi);
      if (mc > M) {
        const float d = M - mc;
        S = (d < -126.f) ? 0.f : ldexpf(S, (int)d);
        M = mc;
      }
#pragma unroll
      for (int j = 0; j < N; ++j) e[j] = __builtin_amdgcn_exp2f(fmaf(z[j], c_lo, fmaf(z[j], c_hi, -M)));
#pragma unroll
      for (int w = 1; w < N; w <<= 1)
#pragma unroll
        for (int j = 0; j + w < N; j += 2 * w) e[j] += e[j + w];
      s = e[0];
      if (!(s <= 0x1p32f)) {
        bad = 1;
        s = 0.f;
      }
    }
  }
  S += s;
}

// The largest of a vector's values by the IEEE 754-2019 maximum (v_maximum3_f32), which returns
// NaN when any operand is NaN: the result is NaN or +inf exactly when a value is, so one compare
// screens the vector for bad values.  Unlike fmaxf it needs no canonicalising of its operands.
template <int N>
__device__ __forceinline__ float vec_maximum(const float (&z)[N]) {
  float m = z[0];
#pragma unroll
  for (int j = 1; j < N; ++j) m = __builtin_elementwise_maximum(m, z[j]);
  return m;
}

// Vectors [vb, ve) of a row's 16-byte body, plus its scalar head and tail when `ends`.
template <bool BF16>
__device__ void stream_sum(const char* row, int V, int vb, int ve, bool ends, float c_hi, float c_lo, int lt,
                           int nthr, float& M, float& S, int& bad) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int U = 4;
  const RowGeom g = row_geom<BF16>(row, V);
  const uint4* vp = reinterpret_cast<const uint4*>(row + (size_t)g.head * ES);
  int v = vb + lt;
  for (; v + (U - 1) * nthr < ve; v += U * nthr) {
    uint4 d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = load_nt(vp + v + u * nthr);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float z[EPV];
      unpack<BF16>(d[u], z);
      accum<EPV>(z, c_hi, c_lo, M, S, bad);
    }
  }
  if (v < ve) {  // the last (fewer than U) vectors: loads issued together, clamped in bounds
    uint4 d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = load_nt(vp + min(v + u * nthr, ve - 1));
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v + u * nthr < ve) {
        float z[EPV];
        unpack<BF16>(d[u], z);
        accum<EPV>(z, c_hi, c_lo, M, S, bad);
      }
  }
  if (ends) {
    float z[2] = {-INFINITY, -INFINITY};
    if (lt < g.head) z[0] = load_elem<BF16>(row, lt);
    if (lt < g.tail) z[1] = load_elem<BF16>(row, g.head + g.nvec * EPV + lt);
    accum<2>(z, c_hi, c_lo, M, S, bad);
  }
}

// Greedy statistic: first-occurrence argmax; `bad` on NaN or +inf.
template <bool BF16>
__device__ void stream_argmax(const char* row, int V, int vb, int ve, bool ends, int lt, int nthr, float& best,
                              int& bidx, int& bad) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int U = 4;
  const RowGeom g = row_geom<BF16>(row, V);
  const uint4* vp = reinterpret_cast<const uint4*>(row + (size_t)g.head * ES);
  auto take = [&](const float (&z)[EPV], int vbase) {
    // the NaN-propagating maximum: NaN or +inf exactly when the vector holds one (a bad row,
    // whose argmax is never used)
    const float vmax = vec_maximum<EPV>(z);
    bad |= !(vmax <= FLT_MAX);
    if (vmax > best) {  // vectors of one thread arrive in increasing token order
      int j = 0;
      while (j < EPV - 1 && !(z[j] == vmax)) ++j;
      best = vmax;
      bidx = vbase + j;
    }
  };
  int v = vb + lt;
  for (; v + (U - 1) * nthr < ve; v += U * nthr) {
    uint4 d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = load_nt(vp + v + u * nthr);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float z[EPV];
      unpack<BF16>(d[u], z);
      take(z, g.head + (v + u * nthr) * EPV);
    }
  }
  if (v < ve) {  // the last (fewer than U) vectors: loads issued together, clamped in bounds
    uint4 d[U];
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = load_nt(vp + min(v + u * nthr, ve - 1));
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (v + u * nthr < ve) {
        float z[EPV];
        unpack<BF16>(d[u], z);
        take(z, g.head + (v + u * nthr) * EPV);
      }
  }
  if (!ends) return;
  // head and tail elements: compare with the index tie-break
  if (lt < g.head) {
    const float z = load_elem<BF16>(row, lt);
    bad |= !(z <= FLT_MAX);
    if (z > best || (z == best && lt < bidx)) { best = z; bidx = lt; }
  }
  if (lt < g.tail) {
    const int idx = g.head + g.nvec * EPV + lt;
    const float z = load_elem<BF16>(row, idx);
    bad |= !(z <= FLT_MAX);
    if (z > best || (z == best && idx < bidx)) { best = z; bidx = idx; }
  }
}

// Order-preserving 32-bit key of a float (larger float -> larger key).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

struct StreamShared {
  float M[8];
  double S[8];
  int bad[8];
  float best[8];
  int bidx[8];
  double lse2[2];
  float theta[2];
  // top-k
  float tau_w[8];
  float lane_max[8][64];
  int cand_n[2];
  int cnt[2][8];
  long long sum_q[8];   // per-wave fixed-point sums of the kept candidates
  // segmented top-k rows
  int wcnt[8];          // candidates per LDS region (a wave's; in the merge, a segment's entries)
  int over[2];          // merge: a segment of the row could not be listed
  int lists[2];         // merge: the row's kept entries are few enough for the emit to draw from
  int last;             // this workgroup finished its item's last segment
  union {
    float cand[2][kTopkCap];
    char tkr[8][kTopkRegionBytes];   // segmented top-k: wave w's region (see topk_segment)
  };
};

// Wave w's region of a segmented top-k row: while streaming, the raw vectors holding a candidate and
// their vector indices; afterwards the candidates, values from tk_cand_z and token ids from tk_cand_id.
__device__ __forceinline__ uint4* tk_hits(StreamShared& sh, int w) { return reinterpret_cast<uint4*>(sh.tkr[w]); }
__device__ __forceinline__ int32_t* tk_hit_idx(StreamShared& sh, int w) {
  return reinterpret_cast<int32_t*>(sh.tkr[w] + kTopkWaveHits * 16);
}
__device__ __forceinline__ float* tk_cand_z(StreamShared& sh, int w) { return reinterpret_cast<float*>(sh.tkr[w]); }
__device__ __forceinline__ int32_t* tk_cand_id(StreamShared& sh, int w) {
  return reinterpret_cast<int32_t*>(sh.tkr[w] + kTopkWaveCand * 4);
}

// Wave-wide: the largest key t such that at least `need` lanes hold a key >= t (bitwise from the top).
// bf16 keys have a zero low half (positive values) or 0xffff (negative ones): the search stops at bit
// 16, and the low half of a negative result is filled in.
template <bool BF16>
__device__ __forceinline__ uint32_t wave_kth_key(uint32_t key, int need) {
  uint32_t t = 0;
  for (int bit = 31; bit >= (BF16 ? 16 : 0); --bit) {
    const uint32_t trial = t | (1u << bit);
    if ((int)__popcll(__ballot(key >= trial)) >= need) t = trial;
  }
  if (BF16 && t < 0x80000000u) t |= 0xffffu;
  return t;
}

// One wave: the K-th largest key (ties counted) among the values in LDS regions w0 .. w0 + nw - 1 of
// z (region w holds cnt[w] of them from w * stride; nw <= 8).  Key 0 marks an empty slot (no value
// has it: it would be a NaN).  0 when there are fewer than K values.  Up to 512 values are searched
// in registers (eight per lane, over the regions one after another) when REGS, more (or all) from LDS.
template <bool BF16, bool REGS = true>
__device__ __forceinline__ uint32_t kth_region_key(const float* z, int stride, const int* cnt, int w0, int nw,
                                                   int K, int lane) {
  int off[9];   // region w's values are entries off[w] .. off[w + 1] - 1 of the concatenation
  off[0] = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) off[w + 1] = off[w] + ((w < nw) ? cnt[w0 + w] : 0);
  const int n = off[8];
  const int lo = BF16 ? 16 : 0;
  uint32_t t = 0;
  if (REGS && n <= 8 * SPEC_WAVE) {
    uint32_t kr[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = lane + j * SPEC_WAVE;
      int r = 0;
#pragma unroll
      for (int w = 1; w < 8; ++w) r += q >= off[w];
      int base = 0;
#pragma unroll
      for (int w = 1; w < 8; ++w)
        if (r == w) base = off[w];
      kr[j] = (q < n) ? fkey(z[(w0 + r) * stride + (q - base)]) : 0u;
    }
    for (int bit = 31; bit >= lo; --bit) {
      const uint32_t trial = t | (1u << bit);
      int c = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) c += (int)__popcll(__ballot(kr[j] >= trial));
      if (c >= K) t = trial;
    }
  } else {
    for (int bit = 31; bit >= lo; --bit) {
      const uint32_t trial = t | (1u << bit);
      int c = 0;
      for (int w = 0; w < nw; ++w) {
        const int nr = cnt[w0 + w];
        const float* zr = z + (w0 + w) * stride;
        for (int q0 = 0; q0 < nr; q0 += SPEC_WAVE)
          c += (int)__popcll(__ballot(q0 + lane < nr && fkey(zr[q0 + lane]) >= trial));
      }
      if (c >= K) t = trial;
    }
  }
  if (BF16 && t != 0u && t < 0x80000000u) t |= 0xffffu;
  return t;
}

// Combine the per-thread (M, S) of one row's waves; result in sh.lse2[which].
__device__ __forceinline__ void row_combine_sum(StreamShared& sh, float M, float S, int bad, int wave, int lane,
                                                int first_wave, int nwaves, int lt, int which) {
  const float Mw = wave_max(M);
  double Sd = (S > 0.f) ? ldexp((double)S, (int)fmaxf(M - Mw, -2000.f)) : 0.0;
  Sd = wave_sum(Sd);
  const int bw = wave_or_i(bad);
  if (lane == 0) {
    sh.M[wave] = Mw;
    sh.S[wave] = Sd;
    sh.bad[wave] = bw;
  }
  __syncthreads();
  if (lt == 0) {
    float Mr = -INFINITY;
    int b = 0;
    for (int w = first_wave; w < first_wave + nwaves; ++w) {
      Mr = fmaxf(Mr, sh.M[w]);
      b |= sh.bad[w];
    }
    double Sr = 0.0;
    for (int w = first_wave; w < first_wave + nwaves; ++w)
      if (sh.S[w] > 0.0) Sr += ldexp(sh.S[w], (int)fmaxf(sh.M[w] - Mr, -2000.f));
    // no finite kept logit, or a NaN / +inf: invalid row
    sh.lse2[which] = (b || !(Sr > 0.0)) ? NAN : (double)Mr + log2(Sr);
  }
}

// Exact K-th largest raw logit of a row (ties counted) and the log2-sum-exp
// over {z >= theta}.  Candidates z >= tau are collected in LDS, where tau is a
// lower bound of the K-th largest value: every wave of the row contributes
// ceil(K / waves) of its lane maxima over the first vectors, so at least K
// logits are >= tau.  If more than kTopkCap candidates arrive, the threshold
// is found by counting passes over the row instead.
template <bool BF16>
__device__ __forceinline__ void topk_stats(StreamShared& sh, const char* row, int V, int K, float c_hi, float c_lo, int lt,
                           int nthr, int wave, int lane, int first_wave, int nwaves, int which) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  const RowGeom g = row_geom<BF16>(row, V);
  const uint4* vp = reinterpret_cast<const uint4*>(row + (size_t)g.head * ES);
  if (lt == 0) sh.cand_n[which] = 0;
  // phase A: first vectors in registers, lane maxima
  uint4 pre[kTopkPre];
  float tmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < kTopkPre; ++u) {
    const int v = lt + u * nthr;
    if (v < g.nvec) {
      pre[u] = vp[v];
      float z[EPV];
      unpack<BF16>(pre[u], z);
#pragma unroll
      for (int j = 0; j < EPV; ++j) tmax = fmaxf(tmax, z[j]);
    }
  }
  sh.lane_max[wave][lane] = tmax;
  __syncthreads();
  {
    const int Kw = (K + nwaves - 1) / nwaves;
    if (Kw <= 64) {
      int rank = 0;
      for (int s = 0; s < 64; ++s) {
        const float o = sh.lane_max[wave][s];
        rank += (o > tmax) || (o == tmax && s < lane);
      }
      if (rank == Kw - 1) sh.tau_w[wave] = tmax;
    } else if (lane == 0) {
      sh.tau_w[wave] = -INFINITY;
    }
  }
  __syncthreads();
  float tau = INFINITY;
  for (int w = first_wave; w < first_wave + nwaves; ++w) tau = fminf(tau, sh.tau_w[w]);
  if (!(tau > -INFINITY)) tau = -INFINITY;  // also catches NaN
  // phase B: filter everything into the candidate buffer
  int bad = 0;
  float vmax_all = -INFINITY;
  float* cand = sh.cand[which];
  int* cn = &sh.cand_n[which];
  auto push = [&](const float* z, int n) {
    float vmax = z[0];
    for (int j = 1; j < n; ++j) vmax = fmaxf(vmax, z[j]);
    for (int j = 0; j < n; ++j) bad |= (z[j] != z[j]) || (z[j] == INFINITY);
    vmax_all = fmaxf(vmax_all, vmax);
    if (vmax >= tau) {
      for (int j = 0; j < n; ++j)
        if (z[j] >= tau) {
          const int slot = atomicAdd(cn, 1);
          if (slot < kTopkCap) cand[slot] = z[j];
        }
    }
  };
#pragma unroll
  for (int u = 0; u < kTopkPre; ++u) {
    const int v = lt + u * nthr;
    if (v < g.nvec) {
      float z[EPV];
      unpack<BF16>(pre[u], z);
      push(z, EPV);
    }
  }
  {
    constexpr int U = 4;  // the rest of the row, U vectors per thread in flight
    for (int v0 = lt + kTopkPre * nthr; v0 < g.nvec; v0 += U * nthr) {
      uint4 d[U];
#pragma unroll
      for (int u = 0; u < U; ++u) d[u] = load_nt(vp + min(v0 + u * nthr, g.nvec - 1));
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (v0 + u * nthr < g.nvec) {
          float z[EPV];
          unpack<BF16>(d[u], z);
          push(z, EPV);
        }
    }
  }
  {
    float z[2];
    int n = 0;
    if (lt < g.head) z[n++] = load_elem<BF16>(row, lt);
    if (lt < g.tail) z[n++] = load_elem<BF16>(row, g.head + g.nvec * EPV + lt);
    if (n) push(z, n);
  }
  // row max and bad flag
  {
    const float wm = wave_max(vmax_all);
    const int wb = wave_or_i(bad);
    if (lane == 0) {
      sh.M[wave] = wm;
      sh.bad[wave] = wb;
    }
  }
  __syncthreads();
  float rmax = -INFINITY;
  int rbad = 0;
  for (int w = first_wave; w < first_wave + nwaves; ++w) {
    rmax = fmaxf(rmax, sh.M[w]);
    rbad |= sh.bad[w];
  }
  const int ncand = sh.cand_n[which];
  const bool overflow = ncand > kTopkCap;
  // threshold: the largest key t with #{key >= t} >= K (bitwise from the top)
  uint32_t t = 0;
  const int low_bit = BF16 ? 16 : 0;
  for (int bit = 31; bit >= low_bit; --bit) {
    const uint32_t trial = t | (1u << bit);
    int c = 0;
    if (!overflow) {
      for (int s = lt; s < ncand; s += nthr) c += fkey(cand[s]) >= trial;
    } else {
      for (int v = lt; v < g.nvec; v += nthr) {
        float z[EPV];
        unpack<BF16>(vp[v], z);
#pragma unroll
        for (int j = 0; j < EPV; ++j) c += (z[j] == z[j]) && fkey(z[j]) >= trial;
      }
      if (lt < g.head) { const float z = load_elem<BF16>(row, lt); c += (z == z) && fkey(z) >= trial; }
      if (lt < g.tail) {
        const float z = load_elem<BF16>(row, g.head + g.nvec * EPV + lt);
        c += (z == z) && fkey(z) >= trial;
      }
    }
    c = (int)wave_sum((double)c);
    const int par = bit & 1;
    if (lane == 0) sh.cnt[par][wave] = c;
    __syncthreads();
    int tot = 0;
    for (int w = first_wave; w < first_wave + nwaves; ++w) tot += sh.cnt[par][w];
    if (tot >= K) t = trial;
  }
  if (BF16 && t < 0x80000000u) t |= 0xffffu;  // negative bf16 keys end in 0xffff
  const float theta = key_to_float(t);
  // log2-sum-exp over the kept set, referenced at M = ceil(max * c_hi)
  const float M = ceilf(rmax * c_hi);
  float S = 0.f;
  int b2 = 0;
  if (!overflow) {
    // The candidates sit in LDS in arrival order, which varies from run to run: their terms
    // (each at most about 1, at most kTopkCap of them) are added as fixed-point integers in units
    // of 2^-48, exact in any order, and the row's total is rounded once.
    long long q = 0;
    for (int s = lt; s < ncand; s += nthr) {
      const float z = cand[s];
      if (z >= theta) q += (long long)rint((double)__builtin_amdgcn_exp2f(fmaf(z, c_lo, fmaf(z, c_hi, -M))) * 0x1p48);
    }
    q = read_lane(wave_inclusive_sum_i64(q, lane), 63);
    if (lane == 0) sh.sum_q[wave] = q;
    __syncthreads();
    if (lt == 0) {
      long long tot = 0;
      for (int w = first_wave; w < first_wave + nwaves; ++w) tot += sh.sum_q[w];
      const double Sr = (double)tot * 0x1p-48;
      // no finite kept logit, or a NaN / +inf: invalid row
      sh.lse2[which] = (rbad || !(rmax < INFINITY) || !(Sr > 0.0)) ? NAN : (double)M + log2(Sr);
      sh.theta[which] = theta;
    }
    return;
  } else {
    float Mt = M;
    for (int v = lt; v < g.nvec; v += nthr) {
      float z[EPV];
      unpack<BF16>(vp[v], z);
#pragma unroll
      for (int j = 0; j < EPV; ++j) z[j] = (z[j] >= theta) ? z[j] : -INFINITY;
      accum<EPV>(z, c_hi, c_lo, Mt, S, b2);
    }
    float z[2] = {-INFINITY, -INFINITY};
    if (lt < g.head) { z[0] = load_elem<BF16>(row, lt); z[0] = z[0] >= theta ? z[0] : -INFINITY; }
    if (lt < g.tail) {
      z[1] = load_elem<BF16>(row, g.head + g.nvec * EPV + lt);
      z[1] = z[1] >= theta ? z[1] : -INFINITY;
    }
    accum<2>(z, c_hi, c_lo, Mt, S, b2);
    // Mt == M unless the reference moved; fold back to M
    if (Mt != M) S = ldexpf(S, (int)fmaxf(Mt - M, -2000.f));
  }
  row_combine_sum(sh, M, S, rbad | b2 | !(rmax < INFINITY), wave, lane, first_wave, nwaves, lt, which);
  if (lt == 0) sh.theta[which] = theta;
}

// Acceptance test of item (i, k) from finished row statistics; one thread.
// lists_t, lists_d: 1 when the target / draft row's kept tokens are listed with their logits, few
// enough for the emit to draw from (RowStat's third field, which the emit reads for top-k rows).
template <bool BF16>
__device__ __forceinline__ void accept_item(const VerifyArgs& a, int i, int k, bool two, double c64, double l2t, float tht,
                            double l2d, float thd, const char* trow, const char* drow, int lists_t = 0,
                            int lists_d = 0) {
  const int G = a.G, V = a.V;
  a.rows_t[(size_t)i * (G + 1) + k] = RowStat{l2t, tht, lists_t};
  bool bad = !(l2t == l2t);
  if (two) {
    a.rows_d[(size_t)i * G + k] = RowStat{l2d, thd, lists_d};
    bad |= !(l2d == l2d);
    const int x = (a.tokens && !a.overlap_only) ? a.tokens[(size_t)i * G + k] : -1;
    if (!bad && x >= 0 && x < V) {
      const double r = acceptance_ratio(load_elem<BF16>(trow, x), load_elem<BF16>(drow, x), c64, l2t, tht, l2d,
                                        thd);
      double ua, ue;
      verify_uniforms(a.seed[i], (uint64_t)i, (uint64_t)k, &ua, &ue);
      a.acc[(size_t)i * G + k] = AccRec{r, ua < r ? 1 : 0, 1};
    }
  }
  if (bad) atomicOr(&a.req_status[i], SPEC_REQ_NONFINITE);
}

// One segment of a top-k row with K <= kTopkSegMaxK: vectors [vb, ve) of the row's 16-byte body, plus
// the scalar head and tail when `ends`.  Lists the segment's values at or above its K-th largest value
// theta_s (ties counted) with their token ids into vals / ids, and records theta_s, the segment's
// largest value and whether it holds a NaN or +inf in *rec.  The row's K-th largest is at least
// theta_s, so the list holds every kept token of the segment.
// Candidates are the values >= tau, tau the smallest over the row's waves of each wave's
// ceil(K / waves)-th largest lane maximum over the lanes' first vectors: every wave has that many
// values >= its own bound, so at least K values are >= tau and theta_s >= tau.  While streaming, a
// lane whose vector holds a candidate only copies the raw vector and its index to its wave's LDS
// region (slot by ballot); after the segment each wave expands its vectors into (value, token id)
// candidates in place, and the row's first wave finds theta_s among them.  A region overflowing, or
// more than kTopkSegCap values at the cut, sets rec->n = kTopkSegCap + 1: the merge then counts over
// the row.  Called by the nthr threads of one row (both rows of the workgroup call it: it contains
// workgroup barriers); the streaming loop's trip count is the same in every lane of a wave (its
// ballots need the whole wave).
template <bool BF16>
__device__ __forceinline__ void topk_segment(StreamShared& sh, const char* row, int V, int vb, int ve, bool ends,
                                             int K, int lt, int nthr, int wave, int lane, int first_wave,
                                             int nwaves, TopkSeg* rec, float* vals, int32_t* ids) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  constexpr int U = 4;                               // vectors per thread in flight
  constexpr int RF = kTopkRegionBytes / 4;           // region stride in floats
  constexpr int HJ = kTopkWaveHits / SPEC_WAVE;      // stored vectors per lane when expanding
  static_assert(HJ * SPEC_WAVE == kTopkWaveHits, "whole waves of stored vectors");
  const RowGeom g = row_geom<BF16>(row, V);
  const uint4* vp = reinterpret_cast<const uint4*>(row + (size_t)g.head * ES);
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int vlast = max(ve - 1, 0);
  const int base0 = vb + (lt - lane);   // the wave's first vector
  // the scalar head and tail (segment 0), loaded early
  const bool hv = ends && lt < g.head, tv = ends && lt < g.tail;
  const int ttok = g.head + g.nvec * EPV + lt;
  const float zh = hv ? load_elem<BF16>(row, lt) : NAN;
  const float zt = tv ? load_elem<BF16>(row, ttok) : NAN;
  uint4 d[U];
#pragma unroll
  for (int u = 0; u < U; ++u) d[u] = load_nt(vp + min(base0 + lane + u * nthr, vlast));
  float tmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (base0 + lane + u * nthr < ve) {
      float z[EPV];
      unpack<BF16>(d[u], z);
#pragma unroll
      for (int j = 0; j < EPV; ++j) tmax = fmaxf(tmax, z[j]);
    }
  {
    const float tw = key_to_float(wave_kth_key<BF16>(fkey(tmax), (K + nwaves - 1) / nwaves));
    if (lane == 0) sh.tau_w[wave] = tw;
  }
  __syncthreads();
  float tau = INFINITY;
  for (int w = first_wave; w < first_wave + nwaves; ++w) tau = fminf(tau, sh.tau_w[w]);
  uint4* hvec = tk_hits(sh, wave);
  int32_t* hidx = tk_hit_idx(sh, wave);
  int nh = 0;   // the wave's stored vectors (the same in every lane)
  int bad = 0;
  float vmax = -INFINITY;
  auto scan_vec = [&](const uint4& dv, int v) {
    const bool valid = v < ve;
    float z[EPV];
    unpack<BF16>(dv, z);
    // NaN or +inf exactly when the vector holds one; then the row is bad and its list, maximum
    // and hits are never used
    const float m = vec_maximum<EPV>(z);
    if (valid) {
      bad |= !(m < INFINITY);
      vmax = __builtin_elementwise_maximum(vmax, m);
    }
    const bool hit = valid && m >= tau;
    const unsigned long long mh = __ballot(hit);
    if (mh) {
      const int slot = nh + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(mh >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((unsigned)mh, 0u));
      if (hit && slot < kTopkWaveHits) {
        hvec[slot] = dv;
        hidx[slot] = v;
      }
      nh += (int)__popcll(mh);
    }
  };
#pragma unroll
  for (int u = 0; u < U; ++u) scan_vec(d[u], base0 + lane + u * nthr);
  for (int b = base0 + U * nthr; b < ve; b += U * nthr) {
#pragma unroll
    for (int u = 0; u < U; ++u) d[u] = load_nt(vp + min(b + lane + u * nthr, vlast));
#pragma unroll
    for (int u = 0; u < U; ++u) scan_vec(d[u], b + lane + u * nthr);
  }
  if (hv) {
    bad |= !(zh < INFINITY);
    vmax = fmaxf(vmax, zh);
  }
  if (tv) {
    bad |= !(zt < INFINITY);
    vmax = fmaxf(vmax, zt);
  }
  {
    const float wm = wave_max(vmax);
    const int wb = wave_or_i(bad);
    if (lane == 0) {
      sh.M[wave] = wm;
      sh.bad[wave] = wb;
    }
  }
  // expand the stored vectors into candidates, in place: read them all, then write
  const int nhv = min(nh, kTopkWaveHits);
  uint4 hx[HJ];
  int hi[HJ];
#pragma unroll
  for (int j = 0; j < HJ; ++j) {
    const int q = lane + j * SPEC_WAVE;
    hi[j] = (q < nhv) ? hidx[q] : -1;
    if (q < nhv) hx[j] = hvec[q];
  }
  int c = (zh >= tau) + (zt >= tau);
#pragma unroll
  for (int j = 0; j < HJ; ++j)
    if (hi[j] >= 0) {
      float z[EPV];
      unpack<BF16>(hx[j], z);
#pragma unroll
      for (int e = 0; e < EPV; ++e) c += z[e] >= tau;
    }
  // each lane's first slot: the lower lanes' counts, bit plane by bit plane (c < 32)
  int pre = 0, tot = 0;
#pragma unroll
  for (int bb = 0; bb < 5; ++bb) {
    const unsigned long long mb = __ballot((c >> bb) & 1);
    pre += (int)__popcll(mb & below) << bb;
    tot += (int)__popcll(mb) << bb;
  }
  // the region is the wave's own: its reads are done before it is rewritten
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  {
    float* cz = tk_cand_z(sh, wave);
    int32_t* cv = tk_cand_id(sh, wave);
    int slot = pre;
    auto put = [&](float z, int tok) {
      if (z >= tau) {
        if (slot < kTopkWaveCand) {
          cz[slot] = z;
          cv[slot] = tok;
        }
        ++slot;
      }
    };
#pragma unroll
    for (int j = 0; j < HJ; ++j)
      if (hi[j] >= 0) {
        float z[EPV];
        unpack<BF16>(hx[j], z);
#pragma unroll
        for (int e = 0; e < EPV; ++e) put(z[e], g.head + hi[j] * EPV + e);
      }
    put(zh, lt);
    put(zt, ttok);
    if (lane == 0) sh.wcnt[wave] = (nh > kTopkWaveHits || tot > kTopkWaveCand) ? kTopkWaveCand + 1 : tot;
  }
  __syncthreads();
  if (wave != first_wave) return;
  // the row's first wave: theta_s and the list
  float rmax = -INFINITY;
  int rbad = 0, total = 0, full = 0;
  for (int w = first_wave; w < first_wave + nwaves; ++w) {
    rmax = fmaxf(rmax, sh.M[w]);
    rbad |= sh.bad[w];
    total += sh.wcnt[w];
    full |= sh.wcnt[w] > kTopkWaveCand;
  }
  TopkSeg r{kTopkSegCap + 1, -INFINITY, rmax, rbad};
  // fewer than K candidates happens only when every value was one (no bound): all are listed
  const bool all = total < K && tau == -INFINITY;
  if (!full && total <= 8 * SPEC_WAVE && (total >= K || all)) {
    // the row's candidates in registers, eight per lane over the waves' regions one after another:
    // theta_s by a bitwise search on their keys, then the list straight from the registers
    int off[9];
    off[0] = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) off[w + 1] = off[w] + ((w < nwaves) ? sh.wcnt[first_wave + w] : 0);
    uint32_t kr[8];
    int32_t ir[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = lane + j * SPEC_WAVE;
      int rg = 0, base = 0;
#pragma unroll
      for (int w = 1; w < 8; ++w)
        if (q >= off[w]) {
          rg = w;
          base = off[w];
        }
      const bool on = q < total;
      kr[j] = on ? fkey(tk_cand_z(sh, first_wave + rg)[q - base]) : 0u;
      ir[j] = on ? tk_cand_id(sh, first_wave + rg)[q - base] : 0;
    }
    uint32_t t = 0;
    if (!all)
      for (int bit = 31; bit >= (BF16 ? 16 : 0); --bit) {
        const uint32_t trial = t | (1u << bit);
        int c = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) c += (int)__popcll(__ballot(kr[j] >= trial));
        if (c >= K) t = trial;
      }
    if (BF16 && t != 0u && t < 0x80000000u) t |= 0xffffu;
    const float th = all ? -INFINITY : key_to_float(t);
    int m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bool keep = kr[j] != 0u && kr[j] >= t;
      const unsigned long long mk = __ballot(keep);
      const int slot = m + (int)__popcll(mk & below);
      if (keep && slot < kTopkSegCap) {
        vals[slot] = key_to_float(kr[j]);
        ids[slot] = ir[j];
      }
      m += (int)__popcll(mk);
    }
    if (m <= kTopkSegCap) r = TopkSeg{m, th, rmax, rbad};
  } else if (!full && (total >= K || all)) {
    const float* z0 = tk_cand_z(sh, 0);
    const uint32_t t = all ? 0u : kth_region_key<BF16, false>(z0, RF, sh.wcnt, first_wave, nwaves, K, lane);
    const float th = all ? -INFINITY : key_to_float(t);
    int m = 0;
    for (int w = first_wave; w < first_wave + nwaves; ++w) {
      const int nw = sh.wcnt[w];
      const float* zr = tk_cand_z(sh, w);
      const int32_t* vr = tk_cand_id(sh, w);
      for (int q0 = 0; q0 < nw; q0 += SPEC_WAVE) {
        const int q = q0 + lane;
        const float z = (q < nw) ? zr[q] : NAN;
        const bool keep = q < nw && fkey(z) >= t;
        const unsigned long long mk = __ballot(keep);
        const int slot = m + (int)__popcll(mk & below);
        if (keep && slot < kTopkSegCap) {
          vals[slot] = z;
          ids[slot] = vr[q];
        }
        m += (int)__popcll(mk);
      }
    }
    if (m <= kTopkSegCap) r = TopkSeg{m, th, rmax, rbad};
  }
  if (lane == 0) *rec = r;
}

struct MergeShared {
  float z[2][kTopkSegs * kTopkSegCap];   // per row: its listed values, segment s's from s * kTopkSegCap
  int cnt[2][kTopkSegs];
  double lse2[2];
  float theta[2];
  int lists[2];
};

// One wave: row statistics of a segmented top-k row from its segment records (row `which` of item
// (i, k)): the row's K-th largest raw logit theta and the log2-sum-exp over the values >= theta (terms
// as 2^-48 fixed-point integers referenced at M = ceil(max * c_hi), exact in any order: the value
// topk_stats gives), into sh.lse2 / sh.theta / sh.lists[w] (lists: every segment was listed and the
// row keeps at most kTopkEmitKept entries, so the emit may draw from the lists).  theta is the K-th
// largest over the union of the segments' lists when every segment was listed (the union holds every
// value >= theta); otherwise the wave finds it by counting passes over the row itself.
template <bool BF16>
__device__ __forceinline__ void merge_row(MergeShared& sh, const VerifyArgs& a, int i, int k, int which,
                                          const char* row, int K, float c_hi, float c_lo, int w, int lane) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int EPV = 16 / ES;
  static_assert(kTopkSegCap <= 2 * SPEC_WAVE, "two list entries per lane");
  const int nsk = a.nseg_topk;
  const size_t slot = topk_slot(a.G, i, k, which);
  const TopkSeg r = (lane < nsk) ? a.tk_seg[slot + lane] : TopkSeg{0, -INFINITY, -INFINITY, 0};
  const bool over = __ballot(r.n > kTopkSegCap) != 0ull;
  const float rmax = wave_max(r.vmax);
  const int rbad = wave_or_i(r.bad);
  const float M = ceilf(rmax * c_hi);
  float* zs = sh.z[w];
  uint32_t t = 0;
  long long q64 = 0;
  int kept = 0;
  if (!over) {
    // the segments' values into LDS region s (loads of every segment issued together)
    float zl[kTopkSegs][2];
#pragma unroll
    for (int s = 0; s < kTopkSegs; ++s) {
      const int ns = (s < nsk) ? read_lane(r.n, s) : 0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = lane + h * SPEC_WAVE;
        zl[s][h] = (q < ns) ? a.tk_val[(slot + s) * kTopkSegCap + q] : -INFINITY;
      }
    }
#pragma unroll
    for (int s = 0; s < kTopkSegs; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = lane + h * SPEC_WAVE;
        if (q < kTopkSegCap) zs[s * kTopkSegCap + q] = zl[s][h];
      }
    if (lane < kTopkSegs) sh.cnt[w][lane] = (lane < nsk) ? r.n : 0;
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    t = kth_region_key<BF16>(zs, kTopkSegCap, sh.cnt[w], 0, nsk, K, lane);
    for (int s = 0; s < nsk; ++s) {
      const int ns = sh.cnt[w][s];
      for (int q0 = 0; q0 < ns; q0 += SPEC_WAVE) {
        const int q = q0 + lane;
        const float z = (q < ns) ? zs[s * kTopkSegCap + q] : -INFINITY;
        const bool keep = q < ns && fkey(z) >= t;
        kept += (int)__popcll(__ballot(keep));
        if (keep)
          q64 += (long long)rint((double)__builtin_amdgcn_exp2f(fmaf(z, c_lo, fmaf(z, c_hi, -M))) * 0x1p48);
      }
    }
  } else {
    // counting passes over the row: t = the largest key with at least K values' keys >= t
    const RowGeom g = row_geom<BF16>(row, a.V);
    const uint4* vp = reinterpret_cast<const uint4*>(row + (size_t)g.head * ES);
    auto count_ge = [&](uint32_t trial) {
      int c = 0;
      for (int v = lane; v < g.nvec; v += SPEC_WAVE) {
        float z[EPV];
        unpack<BF16>(vp[v], z);
#pragma unroll
        for (int j = 0; j < EPV; ++j) c += (z[j] == z[j]) && fkey(z[j]) >= trial;
      }
      for (int e = lane; e < g.head + g.tail; e += SPEC_WAVE) {
        const float z = load_elem<BF16>(row, e < g.head ? e : g.nvec * EPV + e);
        c += (z == z) && fkey(z) >= trial;
      }
      return wave_sum_i(c);
    };
    for (int bit = 31; bit >= (BF16 ? 16 : 0); --bit) {
      const uint32_t trial = t | (1u << bit);
      if (count_ge(trial) >= K) t = trial;
    }
    if (BF16 && t != 0u && t < 0x80000000u) t |= 0xffffu;
    for (int v = lane; v < g.nvec; v += SPEC_WAVE) {
      float z[EPV];
      unpack<BF16>(vp[v], z);
#pragma unroll
      for (int j = 0; j < EPV; ++j)
        if (z[j] == z[j] && fkey(z[j]) >= t)
          q64 += (long long)rint((double)__builtin_amdgcn_exp2f(fmaf(z[j], c_lo, fmaf(z[j], c_hi, -M))) * 0x1p48);
    }
    for (int e = lane; e < g.head + g.tail; e += SPEC_WAVE) {
      const float z = load_elem<BF16>(row, e < g.head ? e : g.nvec * EPV + e);
      if (z == z && fkey(z) >= t)
        q64 += (long long)rint((double)__builtin_amdgcn_exp2f(fmaf(z, c_lo, fmaf(z, c_hi, -M))) * 0x1p48);
    }
  }
  q64 = read_lane(wave_inclusive_sum_i64(q64, lane), 63);
  if (lane == 0) {
    const double Sr = (double)q64 * 0x1p-48;
    sh.lse2[w] = (rbad || !(rmax < INFINITY) || !(Sr > 0.0)) ? NAN : (double)M + log2(Sr);
    sh.theta[w] = (t == 0u) ? -INFINITY : key_to_float(t);   // t = 0: fewer than K values, all kept
    sh.lists[w] = !over && kept <= kTopkEmitKept;
  }
}

// Reduce the per-thread (M, S, bad) of one row's waves into a segment Partial (written by lt == 0).
__device__ __forceinline__ void row_partial_sum(StreamShared& sh, float M, float S, int bad, int wave, int lane,
                                                int first_wave, int nwaves, int lt, float zx, Partial* out) {
  const float Mw = wave_max(M);
  double Sd = (S > 0.f) ? ldexp((double)S, (int)fmaxf(M - Mw, -2000.f)) : 0.0;
  Sd = wave_sum(Sd);
  const int bw = wave_or_i(bad);
  if (lane == 0) {
    sh.M[wave] = Mw;
    sh.S[wave] = Sd;
    sh.bad[wave] = bw;
  }
  __syncthreads();
  if (lt == 0) {
    float Mr = -INFINITY;
    int b = 0;
    for (int w = first_wave; w < first_wave + nwaves; ++w) {
      Mr = fmaxf(Mr, sh.M[w]);
      b |= sh.bad[w];
    }
    double Sr = 0.0;
    for (int w = first_wave; w < first_wave + nwaves; ++w)
      if (sh.S[w] > 0.0) Sr += ldexp(sh.S[w], (int)fmaxf(sh.M[w] - Mr, -2000.f));
    *out = Partial{Sr, Mr, 0, b, zx};
  }
}

// Work item g of a call whose work list is request-major (a.derive_items): items[r] holds request
// r's first item (the items of request r are its positions k_base, k_base + 1, ... one after
// another; a request with no items has the next one's first item) and *nitems the total.  Each wave finds g's request
// by itself: the number of requests whose first item is <= g, counted with ballots over the B <=
// 2 * kStreamThreads first-item words (one load each, all issued together; no barrier).  Returns
// false when g lies past the last item.
__device__ __forceinline__ bool derive_item(const VerifyArgs& a, int g, int& i_out, int& k_out) {
  constexpr int NQ = 2 * kStreamThreads / SPEC_WAVE;   // chunks of 64 requests
  const int lane = threadIdx.x & 63;
  const int B = a.B;
  if (g >= *a.nitems) return false;
  int o[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int r = q * SPEC_WAVE + lane;
    o[q] = (q * SPEC_WAVE < B) ? a.items[min(r, B - 1)] : 0x7fffffff;
    if (r >= B) o[q] = 0x7fffffff;
  }
  int n = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q) n += (int)__popcll(__ballot(o[q] <= g));
  const int i = n - 1;                 // a request with no items shares its first item with the next
  int first = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q)
    if (q == (i >> 6)) first = __builtin_amdgcn_readlane(o[q], i & 63);
  i_out = i;
  k_out = a.k_base + g - first;
  return true;
}

// Work item g of the second streaming pass of a left-to-right call: the positions k_base .. npos_r - 1
// of every request r whose walk went past the first pass, request after request.  Each wave forms
// the list itself from the B <= 2 * kStreamThreads npos words (one load each, all issued
// together): per 64 requests a prefix sum of their item counts, and a ballot for the request whose
// items hold g.  Returns false when g lies past the last item (*nwalk, summed by the walk).
__device__ __forceinline__ bool derive_item_walk(const VerifyArgs& a, int g, int& i_out, int& k_out) {
  constexpr int NQ = 2 * kStreamThreads / SPEC_WAVE;   // chunks of 64 requests
  const int lane = threadIdx.x & 63;
  const int B = a.B, cap = a.k_base;
  if (g >= *a.nwalk) return false;
  int c[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int r = q * SPEC_WAVE + lane;
    c[q] = (q * SPEC_WAVE < B) ? max(a.npos[min(r, B - 1)] - cap, 0) : 0;
    if (r >= B) c[q] = 0;
  }
  int base = 0, i = -1, first = 0;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (q * SPEC_WAVE >= B) break;
    const int incl = wave_inclusive_scan(c[q]);
    const int excl = base + incl - c[q];
    const unsigned long long m = __ballot(excl <= g && g < excl + c[q]);
    if (m) {
      const int l = (int)__ffsll((long long)m) - 1;
      i = q * SPEC_WAVE + l;
      first = __builtin_amdgcn_readlane(excl, l);
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  if (i < 0) return false;
  i_out = i;
  k_out = cap + g - first;
  return true;
}

// log2-sum-exp of a row from its segment partials (fixed segment order); NaN when invalid.

// One workgroup per (work item, segment).  Target row k and, when k < L, draft row k of
// the item are streamed together by the two halves of the workgroup; a lone target row uses
// all eight waves.  combine_kernel then finishes each item from its segment partials.
// Top-k items with top_k <= kTopkSegMaxK list their segments' largest values (at most kTopkSegs
// segments) for topk_merge_kernel; with a larger top_k, segment 0 streams the whole rows and
// finishes the item.  The grid holds the largest work list the call allows (every position of
// every request, or the caller's token cap); workgroups past the actual list exit at once.
// TOPK: the call passes top_k (a separate instance, so that the register budget of calls without
// top-k rows is not set by the top-k code).
template <bool BF16, bool TOPK>
__global__ __launch_bounds__(kStreamThreads) __attribute__((amdgpu_waves_per_eu(8)))
void stream_kernel(VerifyArgs a) {
  __shared__ StreamShared sh;
  const int nseg = a.nseg;
  const int g = blockIdx.x / nseg, seg = blockIdx.x - g * nseg;
  int i, k;
  if (a.derive_items) {
    if (a.k_base > 0) {
      if (!derive_item_walk(a, g, i, k)) return;
    } else if (!derive_item(a, g, i, k)) {
      return;
    }
  } else {
    if (g >= *a.nitems) return;
    const int item = a.items[g];
    i = item >> 7;
    k = item & 127;
  }
  const int G = a.G, V = a.V;
  constexpr int ES = BF16 ? 2 : 4;
  const float T = a.greedy_only ? 0.f : a.temperature[i];
  if (!(T >= 0.f && T < INFINITY)) return;          // reported by emit_final_kernel
  int K = (TOPK && a.top_k && !a.greedy_only) ? a.top_k[i] : 0;
  if (K < 0) return;
  if (K >= V || T == 0.f) K = 0;   // the greedy rule reads raw rows: no kept set
  const int L = a.lengths ? a.lengths[i] : G;
  const bool greedy = (T == 0.f);
  if (greedy && a.overlap_only) return;   // no draft distribution to overlap with
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool two = !greedy && k < L;
  const int nthr = two ? kStreamThreads / 2 : kStreamThreads;
  const int which = two ? (tid >= nthr) : 0;
  const int lt = tid - which * nthr;
  const int nwaves = nthr >> 6, first_wave = which * nwaves;
  const char* trow = target_row<ES>(a, i, k);
  const char* drow = two ? draft_row<ES>(a, i, k) : nullptr;
  const char* row = which ? drow : trow;
  const double c64 = greedy ? 0.0 : kLog2e / (double)T;
  const float c_hi = __double2float_rz(c64);
  const float c_lo = fmaxf((float)(c64 - (double)c_hi), 1e-30f);

  if (TOPK && K > 0) {
    const int nsk = a.nseg_topk;
    if (nsk > 1 && K <= kTopkSegMaxK) {
      // one of the row's nsk segments, listed; topk_merge_kernel finishes the item
      if (seg >= nsk) return;
      const RowGeom geo = row_geom<BF16>(row, V);
      const int vb = (int)((long long)geo.nvec * seg / nsk);
      const int ve = (int)((long long)geo.nvec * (seg + 1) / nsk);
      const size_t slot = topk_slot(G, i, k, which) + seg;
      topk_segment<BF16>(sh, row, V, vb, ve, seg == 0, K, lt, nthr, wave, lane, first_wave, nwaves,
                         a.tk_seg + slot, a.tk_val + slot * kTopkSegCap, a.tk_ids + slot * kTopkSegCap);
      return;
    }
    if (seg != 0) return;
    topk_stats<BF16>(sh, row, V, K, c_hi, c_lo, lt, nthr, wave, lane, first_wave, nwaves, which);
    __syncthreads();
    if (tid == 0) accept_item<BF16>(a, i, k, two, c64, sh.lse2[0], sh.theta[0], two ? sh.lse2[1] : 0.0,
                                    two ? sh.theta[1] : -INFINITY, trow, drow);
    return;
  }

  // this segment's share of the row's 16-byte body; segment 0 also takes the scalar ends
  const RowGeom geo = row_geom<BF16>(row, V);
  const int vb = (int)((long long)geo.nvec * seg / nseg);
  const int ve = (int)((long long)geo.nvec * (seg + 1) / nseg);
  const bool ends = (seg == 0);
  Partial* pt = a.part_t + ((size_t)i * (G + 1) + k) * nseg;
  Partial* pd = a.part_d + ((size_t)i * (G + 1) + k) * nseg;

  if (greedy) {
    float best = -INFINITY;
    int bidx = 0x7fffffff, bad = 0;
    stream_argmax<BF16>(row, V, vb, ve, ends, lt, nthr, best, bidx, bad);
    // wave: max value, then lowest index among equal values
    const float wb = wave_max(best);
    int cand = (best == wb) ? bidx : 0x7fffffff;
    cand = wave_min_i(cand);
    bad = wave_or_i(bad);
    if (lane == 0) {
      sh.best[wave] = wb;
      sh.bidx[wave] = cand;
      sh.bad[wave] = bad;
    }
    __syncthreads();
    if (tid == 0) {
      float rb = -INFINITY;
      int ri = 0x7fffffff, rbad = 0;
      for (int w = 0; w < nwaves; ++w) rb = fmaxf(rb, sh.best[w]);
      for (int w = 0; w < nwaves; ++w) {
        rbad |= sh.bad[w];
        if (sh.best[w] == rb) ri = min(ri, sh.bidx[w]);
      }
      pt[seg] = Partial{(double)rb, 0.f, ri, rbad, NAN};
    }
  } else {
    // the writer of segment 0 also fetches the row's logit at the draft token, which the
    // acceptance test needs (its load overlaps the streaming)
    float zx = NAN;
    if (seg == 0 && two && lt == 0) {
      const int x = a.derive_items ? a.tokens[(size_t)i * G + k] : a.items_x[g];
      if (x >= 0 && x < V) zx = load_elem<BF16>(row, x);
    }
    float M = -0x1p30f, S = 0.f;
    int bad = 0;
    stream_sum<BF16>(row, V, vb, ve, ends, c_hi, c_lo, lt, nthr, M, S, bad);
    row_partial_sum(sh, M, S, bad, wave, lane, first_wave, nwaves, lt, zx, which ? &pd[seg] : &pt[seg]);
  }
}

// The segmented top-k items (0 < K <= kTopkSegMaxK, rows in more than one segment), one 128-thread
// workgroup each: wave 0 merges the target row's segments, wave 1 the draft row's (k < L), then the
// acceptance test.  Other items exit at once.
template <bool BF16>
__global__ __launch_bounds__(2 * SPEC_WAVE) void topk_merge_kernel(VerifyArgs a) {
  __shared__ MergeShared sh;
  int i, k;
  if (a.derive_items) {
    if (!derive_item(a, (int)blockIdx.x, i, k)) return;
  } else {
    if ((int)blockIdx.x >= *a.nitems) return;
    const int item = a.items[blockIdx.x];
    i = item >> 7;
    k = item & 127;
  }
  const int G = a.G, V = a.V;
  constexpr int ES = BF16 ? 2 : 4;
  const float T = a.temperature[i];
  if (!(T > 0.f && T < INFINITY)) return;
  const int K = a.top_k[i];
  if (!(K > 0 && K < V && K <= kTopkSegMaxK)) return;
  const int L = a.lengths ? a.lengths[i] : G;
  const bool two = k < L;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const char* trow = target_row<ES>(a, i, k);
  const char* drow = two ? draft_row<ES>(a, i, k) : nullptr;
  const double c64 = kLog2e / (double)T;
  const float c_hi = __double2float_rz(c64);
  const float c_lo = fmaxf((float)(c64 - (double)c_hi), 1e-30f);
  if (wave == 0 || two) merge_row<BF16>(sh, a, i, k, wave, wave ? drow : trow, K, c_hi, c_lo, wave, lane);
  __syncthreads();
  if (threadIdx.x == 0)
    accept_item<BF16>(a, i, k, two, c64, sh.lse2[0], sh.theta[0], two ? sh.lse2[1] : 0.0,
                      two ? sh.theta[1] : -INFINITY, trow, drow, sh.lists[0], two ? sh.lists[1] : 0);
}

// Finish every segmented work item: combine its segment partials and run the acceptance
// test (one thread per item).  Top-k items were finished by the streaming or merging kernel.
__global__ __launch_bounds__(256) void combine_kernel(VerifyArgs a) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= *a.nitems) return;
  const int item = a.items[g];
  const int i = item >> 7, k = item & 127;
  const int G = a.G, V = a.V, nseg = a.nseg;
  const float T = a.greedy_only ? 0.f : a.temperature[i];
  if (!(T >= 0.f && T < INFINITY)) return;
  const int K = (a.top_k && !a.greedy_only && T > 0.f) ? a.top_k[i] : 0;   // greedy: no kept set
  if (K < 0 || (K > 0 && K < V)) return;
  const int L = a.lengths ? a.lengths[i] : G;
  const Partial* pt = a.part_t + ((size_t)i * (G + 1) + k) * nseg;
  const Partial* pd = a.part_d + ((size_t)i * (G + 1) + k) * nseg;
  if (T == 0.f && a.overlap_only) return;   // not streamed: no draft distribution to overlap with
  if (T == 0.f) {
    int am = combine_argmax(pt, nseg);
    if (am < 0) {
      atomicOr(&a.req_status[i], SPEC_REQ_NONFINITE);
      am = 0;
    }
    a.rows_t[(size_t)i * (G + 1) + k] = RowStat{0.0, -INFINITY, am};
    if (k < L) {
      const int m = (a.items_x[g] == am);
      a.acc[(size_t)i * G + k] = AccRec{m ? 1.0 : 0.0, m, 1};
    }
    return;
  }
  const double c64 = kLog2e / (double)T;
  const double l2t = combine_sum(pt, nseg);
  a.rows_t[(size_t)i * (G + 1) + k] = RowStat{l2t, -INFINITY, 0};
  bool bad = !(l2t == l2t);
  if (k < L) {
    const double l2d = combine_sum(pd, nseg);
    a.rows_d[(size_t)i * G + k] = RowStat{l2d, -INFINITY, 0};
    bad |= !(l2d == l2d);
    const int x = a.items_x[g];
    if (!bad && x >= 0 && x < V) {
      const double r = acceptance_ratio(pt[0].zx, pd[0].zx, c64, l2t, -INFINITY, l2d, -INFINITY);
      double ua, ue;
      verify_uniforms(a.seed[i], (uint64_t)i, (uint64_t)k, &ua, &ue);
      a.acc[(size_t)i * G + k] = AccRec{r, ua < r ? 1 : 0, 1};
    }
  }
  if (bad) atomicOr(&a.req_status[i], SPEC_REQ_NONFINITE);
}

__global__ void philox_kernel(int n, const uint64_t* seed, const int32_t* req, const int32_t* pos, double* ua,
                              double* ue) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n) return;
  double a, b;
  verify_uniforms(seed[t], (uint64_t)(uint32_t)req[t], (uint64_t)(uint32_t)pos[t], &a, &b);
  ua[t] = a;
  ue[t] = b;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t rows_t, rows_d, acc, items, items_x, nitems, req_status, ereq, ranges, amb, part_t, part_d, t_off, d_off,
      tk_seg, tk_val, tk_ids, npos, nwalk, total;
};

// Segments per row in the streaming kernel: about 48 KB of logits each, 1 .. 16.
static int stream_segments(int V, int es) {
  const long long n = (long long)V * es / 49152;
  return (int)(n < 1 ? 1 : (n > kMaxStreamSegs ? kMaxStreamSegs : n));
}

// V = 1 for calls with no emit ranges; topk = false for calls that never stream top-k rows (greedy).
static WsLayout ws_layout(int B, int G, int V, int nseg, bool topk) {
  WsLayout l;
  size_t o = 0;
  l.rows_t = o; o = align256(o + sizeof(RowStat) * (size_t)B * (G + 1));
  l.rows_d = o; o = align256(o + sizeof(RowStat) * (size_t)B * G);
  l.acc = o; o = align256(o + sizeof(AccRec) * (size_t)B * G);
  l.items = o; o = align256(o + sizeof(int32_t) * (size_t)B * (G + 1));
  l.items_x = o; o = align256(o + sizeof(int32_t) * (size_t)B * (G + 1));
  l.nitems = o; o = align256(o + sizeof(int32_t));
  l.req_status = o; o = align256(o + sizeof(int32_t) * (size_t)B);
  l.ereq = o; o = align256(o + sizeof(EmitReq) * (size_t)B);
  l.ranges = o; o = align256(o + sizeof(EmitRange) * (size_t)B * num_ranges(V));
  l.amb = o; o = align256(o + sizeof(int32_t) * (size_t)B * kAmbCap);
  l.part_t = o; o = align256(o + sizeof(Partial) * (size_t)B * (G + 1) * nseg);
  l.part_d = o; o = align256(o + sizeof(Partial) * (size_t)B * (G + 1) * nseg);
  l.t_off = o; o = align256(o + sizeof(int64_t) * (size_t)B);
  l.d_off = o; o = align256(o + sizeof(int64_t) * (size_t)B);
  const size_t tk = topk ? topk_slot(G, B, 0, 0) : 0;   // records: every (item, row, segment)
  l.tk_seg = o; o = align256(o + sizeof(TopkSeg) * tk);
  l.tk_val = o; o = align256(o + sizeof(float) * tk * kTopkSegCap);
  l.tk_ids = o; o = align256(o + sizeof(int32_t) * tk * kTopkSegCap);
  l.npos = o; o = align256(o + sizeof(int32_t) * (size_t)B);
  l.nwalk = o; o = align256(o + sizeof(int32_t));
  l.total = o;
  return l;
}

bool shape_ok(int B, int G, int V, int dtype) {
  if (B < 1 || B > (1 << 24)) return false;
  if (G < 1 || G > SPEC_MAX_GAMMA) return false;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return false;
  const int vmax = dtype == SPEC_BF16 ? SPEC_MAX_V : SPEC_MAX_V / 2;
  if (V < 1 || V > vmax) return false;
  return true;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A launch's work-item count (workgroups x threads) must fit the 32-bit grid size of the dispatch
// packet.
static bool grid_fits(uint64_t groups, uint64_t threads) { return groups * threads <= 0xffffffffull; }

int32_t bind_workspace(VerifyArgs& a, int dtype, void* ws, size_t ws_bytes, size_t extra_bytes, char** extra) {
  a.nseg = stream_segments(a.V, dtype == SPEC_BF16 ? 2 : 4);
  // the largest grids of the call: the streaming kernel's (work items x segments), the fused
  // emit's (a 1024-thread workgroup per request) and the combine's (a thread per item)
  uint64_t items = (uint64_t)a.B * (uint64_t)(a.G + 1);
  if (a.max_items > 0 && (uint64_t)a.max_items < items) items = (uint64_t)a.max_items;
  if (!grid_fits(items * (uint64_t)a.nseg, kStreamThreads) || !grid_fits((uint64_t)a.B, kFusedThreads) ||
      !grid_fits((uint64_t)a.B * (uint64_t)(a.G + 1), 1))
    return SPEC_ERR_UNSUPPORTED;
  // greedy and overlap calls have no emit ranges
  const WsLayout l = ws_layout(a.B, a.G, (a.greedy_only || a.overlap_only) ? 1 : a.V, a.nseg, !a.greedy_only);
  if (!ws || ws_bytes < l.total + extra_bytes) return SPEC_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return SPEC_ERR_WORKSPACE;
  char* w = reinterpret_cast<char*>(ws);
  a.rows_t = reinterpret_cast<RowStat*>(w + l.rows_t);
  a.rows_d = reinterpret_cast<RowStat*>(w + l.rows_d);
  a.acc = reinterpret_cast<AccRec*>(w + l.acc);
  a.items = reinterpret_cast<int32_t*>(w + l.items);
  a.items_x = reinterpret_cast<int32_t*>(w + l.items_x);
  a.nitems = reinterpret_cast<int32_t*>(w + l.nitems);
  a.req_status = reinterpret_cast<int32_t*>(w + l.req_status);
  a.ereq = reinterpret_cast<EmitReq*>(w + l.ereq);
  a.ranges = reinterpret_cast<EmitRange*>(w + l.ranges);
  a.amb = reinterpret_cast<int32_t*>(w + l.amb);
  a.part_t = reinterpret_cast<Partial*>(w + l.part_t);
  a.part_d = reinterpret_cast<Partial*>(w + l.part_d);
  a.t_off = reinterpret_cast<int64_t*>(w + l.t_off);
  a.d_off = reinterpret_cast<int64_t*>(w + l.d_off);
  a.tk_seg = reinterpret_cast<TopkSeg*>(w + l.tk_seg);
  a.tk_val = reinterpret_cast<float*>(w + l.tk_val);
  a.tk_ids = reinterpret_cast<int32_t*>(w + l.tk_ids);
  a.npos = reinterpret_cast<int32_t*>(w + l.npos);
  a.nwalk = reinterpret_cast<int32_t*>(w + l.nwalk);
  a.nseg_topk = std::min(a.nseg, kTopkSegs);
  if (extra) *extra = w + l.total;
  return SPEC_OK;
}

size_t workspace_bytes(int B, int G, int V, bool emit, bool topk) {
  return ws_layout(B, G, emit ? V : 1, kMaxStreamSegs, topk).total;   // the largest segment count, fp32 or bf16
}

void launch_statistics(const VerifyArgs& a, int dtype, hipStream_t s, void* ev0, void* ev1, size_t item_bound) {
  if (a.wl_ready) {
  } else if (!a.flat && a.B <= kWorklistThreads)
    hipLaunchKernelGGL(worklist_small_kernel, dim3(1), dim3(kWorklistThreads), 0, s, a);
  else
    hipLaunchKernelGGL(worklist_kernel, dim3(1), dim3(kWorklistThreads), 0, s, a);
  size_t items = (size_t)a.B * (a.G + 1);
  if (a.max_items > 0 && (size_t)a.max_items < items) items = (size_t)a.max_items;
  if (item_bound > 0 && item_bound < items) items = item_bound;
  const dim3 grid((unsigned)(items * a.nseg)), block(kStreamThreads);
  // The events take the dispatch's own start and end times (no marker packets around it, which
  // would stall the stream before and after the kernel); a failure shows on the caller's event query.
  const hipEvent_t e0 = reinterpret_cast<hipEvent_t>(ev0), e1 = reinterpret_cast<hipEvent_t>(ev1);
  const bool topk = a.top_k && !a.greedy_only;
  if (dtype == SPEC_BF16) {
    if (topk) hipExtLaunchKernelGGL((stream_kernel<true, true>), grid, block, 0, s, e0, e1, 0, a);
    else hipExtLaunchKernelGGL((stream_kernel<true, false>), grid, block, 0, s, e0, e1, 0, a);
  } else {
    if (topk) hipExtLaunchKernelGGL((stream_kernel<false, true>), grid, block, 0, s, e0, e1, 0, a);
    else hipExtLaunchKernelGGL((stream_kernel<false, false>), grid, block, 0, s, e0, e1, 0, a);
  }
  // segmented top-k rows are merged before anything reads their statistics
  if (topk && a.nseg_topk > 1) {
    const dim3 mgrid((unsigned)items), mblock(2 * SPEC_WAVE);
    if (dtype == SPEC_BF16)
      hipLaunchKernelGGL(topk_merge_kernel<true>, mgrid, mblock, 0, s, a);
    else
      hipLaunchKernelGGL(topk_merge_kernel<false>, mgrid, mblock, 0, s, a);
  }
}

void launch_combine(const VerifyArgs& a, hipStream_t s) {
  const unsigned cgrid = (unsigned)(((size_t)a.B * (a.G + 1) + 255) / 256);
  hipLaunchKernelGGL(combine_kernel, dim3(cgrid), dim3(256), 0, s, a);
}

int32_t launch_verify_bound(VerifyArgs a, int dtype, hipStream_t s, void* ev0, void* ev1) {
  launch_statistics(a, dtype, s, ev0, ev1);
  a.r0 = 0;
  a.r1 = a.B;
  // one workgroup per request doing acceptance and the whole emit when that covers the chip;
  // else a combining kernel, about 512 emit-pass workgroups so that small batches still cover
  // the chip, and a separate finishing kernel
  const bool fused = !a.greedy_only && a.B >= kFuseMinRequests;
  a.emit_segs = fused ? 1 : std::max(2, std::min(kMaxEmitSegs, (512 + a.B - 1) / a.B));
  if (!fused) launch_combine(a, s);
  launch_emit(a, dtype == SPEC_BF16, s);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

// A left-to-right call (fused emit; the scheduler's last kernel writes the first pass's request-major
// work list, positions 0 .. phase_cap - 1 of every request): the first streaming pass, the walk over
// its positions (ltr_walk_kernel: npos), the second pass over positions phase_cap .. npos - 1 (each
// of its workgroups forms that list from npos), then the fused emit.  The second pass's grid holds
// the largest list the budget allows; workgroups past the actual list exit at once.  ev0 takes the
// start of the first pass's dispatch, ev1 the end of the second's.
int32_t launch_verify_ltr(VerifyArgs a, int dtype, hipStream_t s, void* ev0, void* ev1) {
  a.k_base = 0;
  launch_statistics(a, dtype, s, ev0, nullptr, (size_t)a.B * (size_t)a.phase_cap);
  launch_ltr_walk(a, s);
  VerifyArgs b = a;   // the second pass: its workgroups list the items from npos themselves
  b.k_base = a.phase_cap;
  b.wl_ready = 1;
  launch_statistics(b, dtype, s, nullptr, ev1, (size_t)a.B * (size_t)(a.G + 1 - a.phase_cap));
  a.r0 = 0;
  a.r1 = a.B;
  a.emit_segs = 1;
  launch_emit(a, dtype == SPEC_BF16, s);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

static int32_t launch_verify(VerifyArgs a, int dtype, void* ws, size_t ws_bytes, hipStream_t s, void* ev0,
                             void* ev1) {
  const int32_t rc = bind_workspace(a, dtype, ws, ws_bytes, 0, nullptr);
  if (rc != SPEC_OK) return rc;
  return launch_verify_bound(a, dtype, s, ev0, ev1);
}

}  // namespace spec

using namespace spec;

extern "C" int32_t spec_left_to_right_first_pass(int32_t gamma, int32_t V, int32_t dtype) {
  if (!shape_ok(1, gamma, V, dtype)) return 0;
  return ltr_first_pass(gamma, stream_segments(V, dtype == SPEC_BF16 ? 2 : 4));
}

extern "C" size_t spec_verify_workspace_size(int32_t B, int32_t gamma, int32_t V) {
  if (B < 1 || gamma < 1 || gamma > SPEC_MAX_GAMMA || V < 1 || V > SPEC_MAX_V) return 0;
  return workspace_bytes(B, gamma, V, true, true);
}

extern "C" size_t spec_verify_greedy_workspace_size(int32_t B, int32_t gamma) {
  if (B < 1 || gamma < 1 || gamma > SPEC_MAX_GAMMA) return 0;
  return workspace_bytes(B, gamma, 1, false, false);
}

static int32_t verify_entry(int32_t B, int32_t gamma, int32_t V, int32_t dtype, const void* target_logits,
                            const void* draft_logits, const int32_t* draft_tokens, const int32_t* lengths,
                            const float* temperature, const int32_t* top_k, const uint64_t* seed,
                            int32_t* num_accepted, int32_t* out_tokens, float* accept_prob, int32_t* status,
                            void* workspace, size_t workspace_bytes, void* stream, int32_t max_tokens,
                            void* event_before, void* event_after) {
  if (!shape_ok(B, gamma, V, dtype) || max_tokens < 0) return SPEC_ERR_INVALID_ARG;
  if (!target_logits || !draft_logits || !draft_tokens || !temperature || !seed || !num_accepted || !out_tokens)
    return SPEC_ERR_INVALID_ARG;
  if (!aligned16(target_logits) || !aligned16(draft_logits)) return SPEC_ERR_INVALID_ARG;
  VerifyArgs a{};
  a.B = B; a.G = gamma; a.V = V; a.greedy_only = 0;
  a.target = target_logits; a.draft = draft_logits; a.tokens = draft_tokens; a.lengths = lengths;
  a.temperature = temperature; a.top_k = top_k; a.seed = seed;
  a.num_accepted = num_accepted; a.out_tokens = out_tokens; a.accept_prob = accept_prob; a.status = status;
  a.max_items = max_tokens;
  return launch_verify(a, dtype, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream), event_before,
                       event_after);
}

extern "C" int32_t spec_verify_profiled(int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                                        const void* target_logits, const void* draft_logits,
                                        const int32_t* draft_tokens, const int32_t* lengths,
                                        const float* temperature, const int32_t* top_k, const uint64_t* seed,
                                        int32_t* num_accepted, int32_t* out_tokens, float* accept_prob,
                                        int32_t* status, void* workspace, size_t workspace_bytes, void* stream,
                                        void* event_before, void* event_after) {
  return verify_entry(B, gamma, V, dtype, target_logits, draft_logits, draft_tokens, lengths, temperature, top_k,
                      seed, num_accepted, out_tokens, accept_prob, status, workspace, workspace_bytes, stream, 0,
                      event_before, event_after);
}

extern "C" int32_t spec_verify_bounded(int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                                       const void* target_logits, const void* draft_logits,
                                       const int32_t* draft_tokens, const int32_t* lengths,
                                       const float* temperature, const int32_t* top_k, const uint64_t* seed,
                                       int32_t* num_accepted, int32_t* out_tokens, float* accept_prob,
                                       int32_t* status, void* workspace, size_t workspace_bytes, void* stream,
                                       int32_t max_tokens, void* event_before, void* event_after) {
  if (max_tokens < 1) return SPEC_ERR_INVALID_ARG;
  return verify_entry(B, gamma, V, dtype, target_logits, draft_logits, draft_tokens, lengths, temperature, top_k,
                      seed, num_accepted, out_tokens, accept_prob, status, workspace, workspace_bytes, stream,
                      max_tokens, event_before, event_after);
}

extern "C" int32_t spec_verify(int32_t B, int32_t gamma, int32_t V, int32_t dtype, const void* target_logits,
                               const void* draft_logits, const int32_t* draft_tokens, const int32_t* lengths,
                               const float* temperature, const int32_t* top_k, const uint64_t* seed,
                               int32_t* num_accepted, int32_t* out_tokens, float* accept_prob, int32_t* status,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return spec_verify_profiled(B, gamma, V, dtype, target_logits, draft_logits, draft_tokens, lengths, temperature,
                              top_k, seed, num_accepted, out_tokens, accept_prob, status, workspace,
                              workspace_bytes, stream, nullptr, nullptr);
}

// ---------------------------------------------------------------------------
// spec_verify_static: spec_verify with its workspace in a file-scope device array
// ---------------------------------------------------------------------------

namespace {

// The workspace of spec_verify_static.  Each GPU the library runs on holds its own copy, at its own
// address, until the process ends.  Host code never uses this name as an address (on the host it
// is a stand-in symbol): it asks the runtime for the device address once per device.
static __device__ __align__(256) unsigned char scratch[SPEC_STATIC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The device address of `scratch` on the calling thread's current device, looked up on the first
// call made with that device current and kept.
int32_t static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SPEC_ERR_HIP;
  if (dev < 0 || dev >= kMaxScratchDevices) return SPEC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SPEC_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_OK;
}

}  // namespace

extern "C" int32_t spec_verify_static(int32_t B, int32_t gamma, int32_t V, int32_t dtype, const void* target_logits,
                                      const void* draft_logits, const int32_t* draft_tokens, const int32_t* lengths,
                                      const float* temperature, const int32_t* top_k, const uint64_t* seed,
                                      int32_t* num_accepted, int32_t* out_tokens, float* accept_prob,
                                      int32_t* status, void* stream) {
  if (!shape_ok(B, gamma, V, dtype)) return SPEC_ERR_INVALID_ARG;
  if (!target_logits || !draft_logits || !draft_tokens || !temperature || !seed || !num_accepted || !out_tokens)
    return SPEC_ERR_INVALID_ARG;
  if (!aligned16(target_logits) || !aligned16(draft_logits)) return SPEC_ERR_INVALID_ARG;
  // a shape whose workspace does not fit the array is refused before any HIP call
  if (workspace_bytes(B, gamma, V, true, true) > (size_t)SPEC_STATIC_SCRATCH_BYTES) return SPEC_ERR_WORKSPACE;
  void* ws = nullptr;
  const int32_t rc = static_scratch(&ws);
  if (rc != SPEC_OK) return rc;
  // every workspace word the kernels read is written earlier in the same call (the work list
  // sets the item count, the status words and the emit counters), so nothing is cleared here
  return verify_entry(B, gamma, V, dtype, target_logits, draft_logits, draft_tokens, lengths, temperature, top_k,
                      seed, num_accepted, out_tokens, accept_prob, status, ws, (size_t)SPEC_STATIC_SCRATCH_BYTES,
                      stream, 0, nullptr, nullptr);
}

extern "C" int32_t spec_verify_flat(int32_t B, int32_t gamma, int32_t V, int32_t dtype, const void* target_rows,
                                    int64_t target_row_count, const void* draft_rows, int64_t draft_row_count,
                                    const int32_t* draft_tokens, const int32_t* lengths,
                                    const float* temperature, const int32_t* top_k, const uint64_t* seed,
                                    int32_t* num_accepted, int32_t* out_tokens, float* accept_prob,
                                    int32_t* status, void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape_ok(B, gamma, V, dtype)) return SPEC_ERR_INVALID_ARG;
  if (!target_rows || !draft_rows || !draft_tokens || !lengths || !temperature || !seed || !num_accepted ||
      !out_tokens)
    return SPEC_ERR_INVALID_ARG;
  if (!aligned16(target_rows) || !aligned16(draft_rows)) return SPEC_ERR_INVALID_ARG;
  if (target_row_count < 0 || draft_row_count < 0) return SPEC_ERR_INVALID_ARG;
  VerifyArgs a{};
  a.B = B; a.G = gamma; a.V = V; a.greedy_only = 0; a.flat = 1;
  a.flat_trows = target_row_count; a.flat_drows = draft_row_count;
  a.target = target_rows; a.draft = draft_rows; a.tokens = draft_tokens; a.lengths = lengths;
  a.temperature = temperature; a.top_k = top_k; a.seed = seed;
  a.num_accepted = num_accepted; a.out_tokens = out_tokens; a.accept_prob = accept_prob; a.status = status;
  return launch_verify(a, dtype, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream), nullptr,
                       nullptr);
}

extern "C" int32_t spec_verify_greedy(int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                                      const void* target_logits, const int32_t* draft_tokens,
                                      const int32_t* lengths, int32_t* num_accepted, int32_t* out_tokens,
                                      int32_t* status, void* workspace, size_t workspace_bytes, void* stream) {
  if (!shape_ok(B, gamma, V, dtype)) return SPEC_ERR_INVALID_ARG;
  if (!target_logits || !draft_tokens || !num_accepted || !out_tokens) return SPEC_ERR_INVALID_ARG;
  if (!aligned16(target_logits)) return SPEC_ERR_INVALID_ARG;
  VerifyArgs a{};
  a.B = B; a.G = gamma; a.V = V; a.greedy_only = 1;
  a.target = target_logits; a.tokens = draft_tokens; a.lengths = lengths;
  a.num_accepted = num_accepted; a.out_tokens = out_tokens; a.status = status;
  return launch_verify(a, dtype, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream), nullptr,
                       nullptr);
}

extern "C" int32_t spec_philox_uniforms(int32_t n, const uint64_t* seed, const int32_t* request,
                                        const int32_t* position, double* u_accept, double* u_emit, void* stream) {
  if (n < 0) return SPEC_ERR_INVALID_ARG;
  if (n == 0) return SPEC_OK;
  if (!seed || !request || !position || !u_accept || !u_emit) return SPEC_ERR_INVALID_ARG;
  const int threads = 256;
  hipLaunchKernelGGL(philox_kernel, dim3((n + threads - 1) / threads), dim3(threads), 0,
                     reinterpret_cast<hipStream_t>(stream), n, seed, request, position, u_accept, u_emit);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}
