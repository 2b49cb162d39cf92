// Markov-head sequential draft sampler and confidence head on gfx950.
//
// DSpark paper, §3.1 (sequential stage): the block is drafted left to right; position k draws x_k
// from softmax(U_k + B(x_{k-1}, .)) (Eq. 4), where the Markov head's transition bias is row
// x_{k-1} of a low-rank product, B(x_{k-1}, .) = W1[x_{k-1}] W2 (Eq. 5, r = 256 by default).
// §3.2.1 (Eq. 7): the confidence of position k is sigmoid(w . [h_k ; W1[x_{k-1}]]).
//
// One draft step k is two kernels:
//   markov_logits_kernel -- for every request at once, the bias is a dense product
//       [B x r] (gathered embedding rows) x [r x V] (projection): MFMA 32x32x16 bf16 tiles with
//       fp32 accumulation.  Each wave keeps the projection rows of its 32 tokens in registers and
//       walks the requests 32 at a time; the epilogue adds U_k, rounds to the storage type, writes
//       the draft logits and folds the stored values into per-(request, 128-token tile)
//       statistics: the largest value and its first token, and, for sampling rows, an fp64 sum of
//       2^(z log2(e)/T - m) against an integer reference m (so tiles combine by exact power-of-two
//       scaling).
//   markov_sample_kernel -- one wave per request combines its tiles, draws u from the request's
//       counter-based stream, finds the tile where the running sum (ascending token order)
//       passes u * total, re-reads that tile's 128 stored logits and picks the token.  T = 0
//       takes the first-occurrence argmax.
// After the last step markov_finish_kernel writes the confidences (fp64 dot products) and the
// per-request status.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.hpp"
#include "philox.hpp"
#include "spec_verify.h"

namespace spec {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));

constexpr int kDraftThreads = 256;   // markov_logits_kernel: 4 waves
constexpr int kTileTokens = 128;     // tokens per workgroup (32 per wave)
constexpr int kReqBlock = 32;        // requests per MFMA block
constexpr int kMaxSteps = 16;        // rank / 16 at most (r <= 256)
constexpr int kSampleThreads = 256;  // markov_sample_kernel / markov_finish_kernel: a wave per item

constexpr double kLog2eD = 1.44269504088896340736;

// Statistics of the stored logits of one request over a set of tokens.
struct Stat {
  double s;     // sum of 2^(z c - m) (sampling rows), else 0
  double m;     // integer reference of s (-inf while s == 0)
  float zmax;   // largest stored value (-inf when none)
  int32_t idx;  // first token holding zmax
  int32_t bad;  // NaN or +inf seen
};

struct alignas(16) DPart {
  double s, m;
  float zmax;
  int32_t idx, bad, pad;
};

struct DraftArgs {
  int B, G, V, r, d, k, nwg;
  const void* base;          // U [B, G, V]
  const uint16_t* W1;        // [V, r] bf16
  const uint16_t* W2t;       // [V, r] bf16, row v = column v of W2
  const int32_t* anchor;     // [B]
  const float* temperature;  // [B]
  const uint64_t* seed;      // [B] or null (all 0)
  const void* hidden;        // [B, G, d] or null
  const float* conf_w;       // [d + r] or null
  int32_t* tokens;           // [B, G]
  void* logits;              // [B, G, V]
  float* conf;               // [B, G] or null
  int32_t* status;           // [B]
  DPart* part;               // [B, nwg] workspace
  int32_t* req_status;       // [B] workspace
};

__device__ __forceinline__ Stat stat_empty() {
  Stat s;
  s.s = 0.0;
  s.m = -__builtin_inf();
  s.zmax = -__builtin_inff();
  s.idx = 0x7fffffff;
  s.bad = 0;
  return s;
}

// a <- a (+) b.  Sums are brought to the larger reference by exact power-of-two scaling; the
// maximum keeps the lower token on equal values.
__device__ __forceinline__ void stat_merge(Stat& a, const Stat& b) {
  if (b.s > 0.0) {
    if (a.s > 0.0) {
      const double M = fmax(a.m, b.m);
      a.s = ldexp(a.s, (int)fmax(a.m - M, -2000.0)) + ldexp(b.s, (int)fmax(b.m - M, -2000.0));
      a.m = M;
    } else {
      a.s = b.s;
      a.m = b.m;
    }
  }
  if (b.zmax > a.zmax || (b.zmax == a.zmax && b.idx < a.idx)) {
    a.zmax = b.zmax;
    a.idx = b.idx;
  }
  a.bad |= b.bad;
}

__device__ __forceinline__ Stat stat_shfl_xor(const Stat& a, int o) {
  Stat b;
  b.s = __shfl_xor(a.s, o, SPEC_WAVE);
  b.m = __shfl_xor(a.m, o, SPEC_WAVE);
  b.zmax = __shfl_xor(a.zmax, o, SPEC_WAVE);
  b.idx = __shfl_xor(a.idx, o, SPEC_WAVE);
  b.bad = __shfl_xor(a.bad, o, SPEC_WAVE);
  return b;
}

__device__ __forceinline__ Stat from_part(const DPart& p) {
  Stat s;
  s.s = p.s;
  s.m = p.m;
  s.zmax = p.zmax;
  s.idx = p.idx;
  s.bad = p.bad;
  return s;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const v4u32*>(p));
}

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int ES>
__device__ __forceinline__ float load_logit(const void* base, size_t i) {
  if constexpr (ES == 2) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[i] << 16);
  else return reinterpret_cast<const float*>(base)[i];
}

// Step k: draft logits z_k = U_k + W1[x_{k-1}] W2 for every request, and per-tile statistics.
template <int ES>
__global__ __launch_bounds__(kDraftThreads) void markov_logits_kernel(DraftArgs a) {
  __shared__ Stat sp[2][kDraftThreads / 64][kReqBlock];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int tl = lane & 31, h = lane >> 5;
  const int V = a.V, r = a.r, G = a.G, k = a.k;
  const int nk = r >> 4;
  const int n0 = blockIdx.x * kTileTokens + wv * 32;

  // Projection operand (MFMA A: row = token, 8 consecutive k per lane half): token n0 + tl.
  const uint16_t* w2 = a.W2t + (size_t)min(n0 + tl, V - 1) * r + 8 * h;
  bf16x8 wop[kMaxSteps];
#pragma unroll
  for (int kk = 0; kk < kMaxSteps; ++kk)
    if (kk < nk) wop[kk] = load_bf16x8(w2 + kk * 16);

  const bool vec = (V & 3) == 0;
  const int nrb = (a.B + kReqBlock - 1) / kReqBlock;
  for (int rb = 0; rb < nrb; ++rb) {
    const int j = rb * kReqBlock + tl;
    const bool valid = j < a.B;
    int prev = 0;
    float T = 0.f;
    if (valid) {
      prev = (k == 0) ? a.anchor[j] : a.tokens[(size_t)j * G + k - 1];
      T = a.temperature[j];
    }
    if (prev < 0 || prev >= V) prev = 0;  // a bad request: its rows are not defined

    // Embedding operand (MFMA B: column = request, 8 consecutive k per lane half).
    const uint16_t* w1 = a.W1 + (size_t)prev * r + 8 * h;
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < kMaxSteps; ++kk)
      if (kk < nk) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wop[kk], load_bf16x8(w1 + kk * 16), acc, 0, 0, 0);

    // Epilogue: lane holds D[token n0 + 8g + 4h + p][request j] in acc[4g + p].
    const size_t row = ((size_t)(valid ? j : 0) * G + k) * V;
    Stat st = stat_empty();
    float zq[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int t0 = n0 + 8 * g + 4 * h;
      float u[4];
      if (valid && vec && t0 + 3 < V) {
        if constexpr (ES == 2) {
          const v2u32 w = __builtin_nontemporal_load(reinterpret_cast<const v2u32*>(
              reinterpret_cast<const uint16_t*>(a.base) + row + t0));
          u[0] = bf16_lo(w.x); u[1] = bf16_hi(w.x); u[2] = bf16_lo(w.y); u[3] = bf16_hi(w.y);
        } else {
          const v4u32 w = __builtin_nontemporal_load(reinterpret_cast<const v4u32*>(
              reinterpret_cast<const float*>(a.base) + row + t0));
          u[0] = __uint_as_float(w.x); u[1] = __uint_as_float(w.y);
          u[2] = __uint_as_float(w.z); u[3] = __uint_as_float(w.w);
        }
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) u[p] = (valid && t0 + p < V) ? load_logit<ES>(a.base, row + t0 + p) : 0.f;
      }
      float zs[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float z = u[p] + acc[4 * g + p];
        if constexpr (ES == 2) zs[p] = __uint_as_float(f32_to_bf16_rne(z) << 16);
        else zs[p] = z;
      }
      if (valid && vec && t0 + 3 < V) {
        if constexpr (ES == 2) {
          uint2 w;
          w.x = (__float_as_uint(zs[0]) >> 16) | (__float_as_uint(zs[1]) & 0xffff0000u);
          w.y = (__float_as_uint(zs[2]) >> 16) | (__float_as_uint(zs[3]) & 0xffff0000u);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.logits) + row + t0) = w;
        } else {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.logits) + row + t0) =
              make_float4(zs[0], zs[1], zs[2], zs[3]);
        }
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p)
          if (valid && t0 + p < V) {
            if constexpr (ES == 2)
              reinterpret_cast<uint16_t*>(a.logits)[row + t0 + p] = (uint16_t)(__float_as_uint(zs[p]) >> 16);
            else
              reinterpret_cast<float*>(a.logits)[row + t0 + p] = zs[p];
          }
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const bool in = valid && t0 + p < V;
        const float z = in ? zs[p] : -__builtin_inff();
        zq[4 * g + p] = z;
        if (in && (z != z || z == __builtin_inff())) st.bad = 1;
        if (z > st.zmax) {  // tokens visited in ascending order: the first maximum is kept
          st.zmax = z;
          st.idx = t0 + p;
        }
      }
    }
    if (valid && T > 0.f && T < __builtin_inff() && st.zmax > -__builtin_inff() && !st.bad) {
      const double c = kLog2eD / (double)T;
      const double m = ceil((double)st.zmax * c);
      double s = 0.0;
#pragma unroll
      for (int i = 0; i < 16; ++i) s += exp2((double)zq[i] * c - m);
      st.s = s;
      st.m = m;
    }
    // the two lane halves hold the same request
    stat_merge(st, stat_shfl_xor(st, 32));
    const int buf = rb & 1;
    if (h == 0) sp[buf][wv][tl] = st;
    __syncthreads();
    if (wv == 0 && h == 0 && valid) {
      Stat t = sp[buf][0][tl];
#pragma unroll
      for (int w = 1; w < kDraftThreads / 64; ++w) stat_merge(t, sp[buf][w][tl]);
      DPart p;
      p.s = t.s;
      p.m = t.m;
      p.zmax = t.zmax;
      p.idx = t.idx;
      p.bad = t.bad;
      p.pad = 0;
      a.part[(size_t)j * a.nwg + blockIdx.x] = p;
    }
  }
}

// Step k: draw x_k for every request (one wave each).
template <int ES>
__global__ __launch_bounds__(kSampleThreads) void markov_sample_kernel(DraftArgs a) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * (kSampleThreads / 64) + (threadIdx.x >> 6);
  if (j >= a.B) return;
  const int k = a.k, V = a.V, nwg = a.nwg;
  int st = (k == 0) ? 0 : a.req_status[j];
  const float T = a.temperature[j];
  if (k == 0) {
    if (!(T >= 0.f && T < __builtin_inff())) st |= SPEC_REQ_BAD_TEMPERATURE;
    const int x0 = a.anchor[j];
    if (x0 < 0 || x0 >= V) st |= SPEC_REQ_BAD_TOKEN;
  }
  const DPart* P = a.part + (size_t)j * nwg;
  const int per = (nwg + 63) / 64;
  const int w0 = min(nwg, lane * per), w1 = min(nwg, w0 + per);
  Stat acc = stat_empty();
  for (int w = w0; w < w1; ++w) stat_merge(acc, from_part(P[w]));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) stat_merge(acc, stat_shfl_xor(acc, o));

  int x = -1;
  if (st == 0) {
    if (acc.bad || !(acc.zmax > -__builtin_inff())) {
      st |= SPEC_REQ_NONFINITE;
    } else if (T == 0.f) {
      x = acc.idx;
    } else {
      const double M = acc.m;
      const double c = kLog2eD / (double)T;
      // this lane's tiles, scaled to the common reference, in token order
      double ls = 0.0;
      int mylast = -1;
      for (int w = w0; w < w1; ++w) {
        if (!(P[w].s > 0.0)) continue;
        const double e = ldexp(P[w].s, (int)fmax(P[w].m - M, -2000.0));
        ls += e;
        if (e > 0.0) mylast = w;
      }
      const double incl = wave_inclusive_sum(ls, lane);
      const double S = __shfl(incl, 63, SPEC_WAVE);
      const uint64_t seed = a.seed ? a.seed[j] : 0ull;
      const Philox4x64 blk = philox4x64_10((uint64_t)k + 1, (uint64_t)j, 1, 0, seed, 0);
      const double target = uniform53(blk.w0) * S;
      // the first lane whose running sum passes the target walks its tiles
      const unsigned long long hit = __ballot(incl > target);
      int wsel = -1;
      double before = -__builtin_inf();  // -inf: no crossing, take the tile's last weighted token
      if (hit) {
        const int L = __ffsll((long long)hit) - 1;
        if (lane == L) {
          double cum = incl - ls;
          for (int w = w0; w < w1; ++w) {
            if (!(P[w].s > 0.0)) continue;
            const double e = ldexp(P[w].s, (int)fmax(P[w].m - M, -2000.0));
            if (!(e > 0.0)) continue;
            if (cum + e > target) {
              wsel = w;
              before = cum;
              break;
            }
            cum += e;
          }
          if (wsel < 0) wsel = mylast;  // rounding: the last weighted tile, its last token
        }
        wsel = __shfl(wsel, L, SPEC_WAVE);
        before = __shfl(before, L, SPEC_WAVE);
      } else {  // u * S rounded up to S: the last weighted tile, its last token
        wsel = wave_max_i(mylast);
      }
      if (wsel < 0) wsel = acc.idx / kTileTokens;  // cannot happen when S > 0
      // the chosen tile's tokens, two per lane, in ascending order
      const size_t row = ((size_t)j * a.G + k) * V;
      const int t0 = wsel * kTileTokens + 2 * lane;
      double e0 = 0.0, e1 = 0.0;
      if (t0 < V) e0 = exp2((double)load_logit<ES>(a.logits, row + t0) * c - M);
      if (t0 + 1 < V) e1 = exp2((double)load_logit<ES>(a.logits, row + t0 + 1) * c - M);
      const double pair = e0 + e1;
      const double incl2 = wave_inclusive_sum(pair, lane);
      double excl2 = __shfl_up(incl2, 1, SPEC_WAVE);
      if (lane == 0) excl2 = 0.0;
      const double c0 = before + (excl2 + e0);
      const double c1 = before + ((excl2 + e0) + e1);
      const bool p0 = e0 > 0.0 && c0 > target;
      const bool p1 = e1 > 0.0 && c1 > target;
      const unsigned long long hb = __ballot(p0 || p1);
      if (hb) {
        const int Lb = __ffsll((long long)hb) - 1;
        const int pick = __shfl(p0 ? t0 : t0 + 1, Lb, SPEC_WAVE);
        x = pick;
      } else {  // past the end of the tile: its last weighted token
        const unsigned long long nz = __ballot(e0 > 0.0 || e1 > 0.0);
        if (nz) {
          const int Ln = 63 - __clzll((long long)nz);
          x = __shfl(e1 > 0.0 ? t0 + 1 : t0, Ln, SPEC_WAVE);
        } else {
          x = acc.idx;
        }
      }
    }
  }
  if (lane == 0) {
    a.tokens[(size_t)j * a.G + k] = (st == 0) ? x : -1;
    a.req_status[j] = st;
  }
}

// After the last step: status, the tokens of bad requests, and the confidences (Eq. 7).
template <int ES>
__global__ __launch_bounds__(kSampleThreads) void markov_finish_kernel(DraftArgs a) {
  const int lane = threadIdx.x & 63;
  const size_t wid = (size_t)blockIdx.x * (kSampleThreads / 64) + (threadIdx.x >> 6);
  if (wid >= (size_t)a.B * a.G) return;
  const int j = (int)(wid / a.G), k = (int)(wid % a.G);
  const int st = a.req_status[j];
  if (k == 0 && lane == 0) a.status[j] = st;
  if (st != 0) {
    if (lane == 0) {
      a.tokens[wid] = -1;
      if (a.conf) a.conf[wid] = __builtin_nanf("");
    }
    return;
  }
  if (!a.conf) return;
  const int prev = (k == 0) ? a.anchor[j] : a.tokens[wid - 1];
  double t = 0.0;
  for (int i = lane; i < a.d; i += 64)
    t += (double)a.conf_w[i] * (double)load_logit<ES>(a.hidden, wid * (size_t)a.d + i);
  const uint16_t* e = a.W1 + (size_t)prev * a.r;
  for (int i = lane; i < a.r; i += 64)
    t += (double)a.conf_w[a.d + i] * (double)__uint_as_float((uint32_t)e[i] << 16);
  t = wave_sum(t);
  if (lane == 0) a.conf[wid] = (float)(1.0 / (1.0 + exp(-t)));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int num_tiles(int V) { return (V + kTileTokens - 1) / kTileTokens; }

size_t draft_ws_bytes(int B, int V) {
  return align256((size_t)B * num_tiles(V) * sizeof(DPart)) + align256((size_t)B * sizeof(int32_t));
}

bool draft_shape_ok(int B, int G, int V, int r, int d, int dtype) {
  if (dtype != SPEC_BF16 && dtype != SPEC_F32) return false;
  if (B < 1 || G < 1 || G > SPEC_MAX_GAMMA || V < 1 || V > SPEC_MAX_V) return false;
  if (dtype == SPEC_F32 && V > SPEC_MAX_V / 2) return false;
  if (r < 16 || r > 16 * kMaxSteps || (r & 15) != 0 || d < 0 || d > (1 << 20)) return false;
  if ((size_t)B * G > (size_t)1 << 24) return false;
  return true;
}

bool is_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace
}  // namespace spec

using namespace spec;

extern "C" size_t spec_draft_workspace_size(int32_t B, int32_t gamma, int32_t V) {
  if (B < 1 || gamma < 1 || gamma > SPEC_MAX_GAMMA || V < 1 || V > SPEC_MAX_V) return 0;
  return draft_ws_bytes(B, V);
}

extern "C" int32_t spec_draft_markov(int32_t B, int32_t gamma, int32_t V, int32_t r, int32_t dtype,
                                     const void* base_logits, const void* W1, const void* W2t,
                                     const int32_t* anchor, const float* temperature, const uint64_t* seed,
                                     int32_t d, const void* hidden, const float* conf_w, int32_t* tokens,
                                     void* draft_logits, float* conf, int32_t* status, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (!draft_shape_ok(B, gamma, V, r, d, dtype)) return SPEC_ERR_INVALID_ARG;
  if (!base_logits || !W1 || !W2t || !anchor || !temperature || !tokens || !draft_logits || !status)
    return SPEC_ERR_INVALID_ARG;
  if (!is_aligned16(base_logits) || !is_aligned16(draft_logits) || !is_aligned16(W1) || !is_aligned16(W2t))
    return SPEC_ERR_INVALID_ARG;
  if (conf && (!conf_w || (d > 0 && !hidden))) return SPEC_ERR_INVALID_ARG;
  const size_t need = draft_ws_bytes(B, V);
  if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255))
    return SPEC_ERR_WORKSPACE;
  DraftArgs a{};
  a.B = B; a.G = gamma; a.V = V; a.r = r; a.d = conf ? d : 0; a.nwg = num_tiles(V);
  a.base = base_logits;
  a.W1 = reinterpret_cast<const uint16_t*>(W1);
  a.W2t = reinterpret_cast<const uint16_t*>(W2t);
  a.anchor = anchor; a.temperature = temperature; a.seed = seed;
  a.hidden = hidden; a.conf_w = conf_w;
  a.tokens = tokens; a.logits = draft_logits; a.conf = conf; a.status = status;
  char* ws = reinterpret_cast<char*>(workspace);
  a.part = reinterpret_cast<DPart*>(ws);
  a.req_status = reinterpret_cast<int32_t*>(ws + align256((size_t)B * a.nwg * sizeof(DPart)));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned sgrid = (unsigned)((B + 3) / 4);
  for (int k = 0; k < gamma; ++k) {
    a.k = k;
    if (dtype == SPEC_BF16) {
      hipLaunchKernelGGL(markov_logits_kernel<2>, dim3(a.nwg), dim3(kDraftThreads), 0, s, a);
      hipLaunchKernelGGL(markov_sample_kernel<2>, dim3(sgrid), dim3(kSampleThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL(markov_logits_kernel<4>, dim3(a.nwg), dim3(kDraftThreads), 0, s, a);
      hipLaunchKernelGGL(markov_sample_kernel<4>, dim3(sgrid), dim3(kSampleThreads), 0, s, a);
    }
  }
  const unsigned fgrid = (unsigned)(((size_t)B * gamma + 3) / 4);
  if (dtype == SPEC_BF16)
    hipLaunchKernelGGL(markov_finish_kernel<2>, dim3(fgrid), dim3(kSampleThreads), 0, s, a);
  else
    hipLaunchKernelGGL(markov_finish_kernel<4>, dim3(fgrid), dim3(kSampleThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}
