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

#include <type_traits>

#include "common.hpp"
#include "philox.hpp"
#include "spec_verify.h"

namespace spec {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
  int32_t bad;  // NaN or +inf seen
};

struct alignas(16) DPart {
  double s, m;
  float zmax;
  int32_t bad, pad0, pad1;
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
  const double* conf_tau;    // [G] per-position temperatures of the confidences, or null (1)
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
  s.bad = 0;
  return s;
}

// a <- a (+) b.  Sums are brought to the larger reference by exact power-of-two scaling.
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
  a.zmax = fmaxf(a.zmax, b.zmax);
  a.bad |= b.bad;
}

__device__ __forceinline__ Stat stat_shfl_xor(const Stat& a, int o) {
  Stat b;
  b.s = __shfl_xor(a.s, o, SPEC_WAVE);
  b.m = __shfl_xor(a.m, o, SPEC_WAVE);
  b.zmax = __shfl_xor(a.zmax, o, SPEC_WAVE);
  b.bad = __shfl_xor(a.bad, o, SPEC_WAVE);
  return b;
}

__device__ __forceinline__ Stat from_part(const DPart& p) {
  Stat s;
  s.s = p.s;
  s.m = p.m;
  s.zmax = p.zmax;
  s.bad = p.bad;
  return s;
}

// 2^t for t <= 0 in fp64, table-driven (P. T. P. Tang, "Table-driven implementation of the
// exponential function in IEEE floating-point arithmetic", ACM TOMS 15(2), 1989): t = n + j/64 + r
// with |r| <= 1/128, 2^t = 2^n * 2^(j/64) * 2^r; the 64 values 2^(j/64) come from `tab`, 2^r from
// its Taylor series to degree 5 (truncation below 4e-17 relative).  t below -1100 (or -inf) gives 0.
__device__ __forceinline__ double exp2_tab(double t, const double* tab) {
  t = fmax(t, -1100.0);
  const double N = rint(t * 64.0);
  const double r = fma(N, -0.015625, t);  // exact
  const int Ni = (int)N;
  double p = 0x1.5d87fe78a6731p-10;       // (ln 2)^k / k!, k = 5 .. 0
  p = fma(p, r, 0x1.3b2ab6fba4e77p-7);
  p = fma(p, r, 0x1.c6b08d704a0c0p-5);
  p = fma(p, r, 0x1.ebfbdff82c58fp-3);
  p = fma(p, r, 0x1.62e42fefa39efp-1);
  p = fma(p, r, 1.0);
  return ldexp(tab[Ni & 63] * p, Ni >> 6);
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
//
// A workgroup owns 128 tokens (32 per wave) and walks the requests 32 at a time.  Per request
// block: the MFMA chain multiplies the wave's projection rows (registers) by the block's embedding
// rows (LDS); the epilogue reads U_k from an LDS tile, writes the rounded z_k back in place and
// folds the values into statistics; after the block's barrier the workgroup stores the z_k tile
// with whole-line 16-byte stores.  The embedding rows and the U_k tile of the next block are
// loaded (whole lines, 16 bytes per thread) while the current block computes.  Tiles that are not
// whole (the last one, or rows not 16-byte aligned) take per-element global accesses instead.
// Operand steps beyond r/16 are zero on both sides (exact zeros).
template <int ES>
__global__ __launch_bounds__(kDraftThreads) void markov_logits_kernel(DraftArgs a) {
  constexpr int RS = kMaxSteps * 16 + 8;            // LDS row stride of the embedding rows (bf16)
  constexpr int USB = kTileTokens * ES + 16;        // LDS row stride of the U/z tile (bytes)
  constexpr int UCPR = kTileTokens * ES / 16;       // 16-byte chunks per tile row
  constexpr int UPT = kReqBlock * UCPR / kDraftThreads;  // chunks per thread (2 bf16, 4 fp32)
  __shared__ Stat sp[2][kDraftThreads / 64][kReqBlock];
  __shared__ double tab[64];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kReqBlock * RS];
  __shared__ __attribute__((aligned(16))) unsigned char sU[3][kReqBlock * USB];
  __shared__ int sPrev[2][kReqBlock];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tl = lane & 31, h = lane >> 5;
  const int V = a.V, r = a.r, G = a.G, k = a.k, B = a.B;
  const int nk = r >> 4;
  const int tile0 = blockIdx.x * kTileTokens;
  const int n0 = tile0 + wv * 32;
  const bf16x8 zero8 = {};
  if (tid < 64) tab[tid] = exp2((double)tid * 0.015625);

  // Projection operand (MFMA A: row = token, 8 consecutive k per lane half): token n0 + tl.
  const uint16_t* w2 = a.W2t + (size_t)min(n0 + tl, V - 1) * r + 8 * h;
  bf16x8 wop[kMaxSteps];
#pragma unroll
  for (int kk = 0; kk < kMaxSteps; ++kk) {
    const bf16x8 v = load_bf16x8(w2 + min(kk, nk - 1) * 16);
    wop[kk] = kk < nk ? v : zero8;
  }

  // x_{k-1} of request j (index clamped; a bad value selects row 0: a bad request's rows are
  // not defined)
  const int* prevp = (k == 0) ? a.anchor : a.tokens + (k - 1);
  const int pstride = (k == 0) ? 1 : G;
  auto prev_raw = [&](int j) -> int { return prevp[(size_t)min(j, B - 1) * pstride]; };
  auto prev_ok = [&](int p) -> int { return (p < 0 || p >= V) ? 0 : p; };
  auto prev_of = [&](int j) -> int { return prev_ok(prev_raw(j)); };
  // Embedding rows W1[x_{k-1}] of a request block: 32 rows of r bf16, 16-byte chunks.
  const int cpr = r >> 3;
  const int nchunk = kReqBlock * cpr;  // <= 1024: at most 4 per thread
  v4u32 gw[4];
  auto load_rows = [&](int pb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * kDraftThreads;
      if (c < nchunk) {
        const int row = c / cpr, col = c - row * cpr;
        gw[i] = *reinterpret_cast<const v4u32*>(a.W1 + (size_t)sPrev[pb][row] * r + col * 8);
      }
    }
  };
  auto store_rows = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * kDraftThreads;
      if (c < nchunk) {
        const int row = c / cpr, col = c - row * cpr;
        *reinterpret_cast<v4u32*>(&sB[buf][row * RS + col * 8]) = gw[i];
      }
    }
  };
  // U_k tile of a request block (whole tiles only): row = request, 16-byte chunks.
  const bool fast_tile = (((size_t)V * ES) % 16 == 0) && (tile0 + kTileTokens <= V);
  const size_t rowstep = (size_t)G * V;  // elements between consecutive requests' rows
  const char* ubase = reinterpret_cast<const char*>(a.base) + ((size_t)k * V + tile0) * ES;
  char* zbase = reinterpret_cast<char*>(a.logits) + ((size_t)k * V + tile0) * ES;
  v4u32 gu[UPT];
  auto load_tile = [&](int rb) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int c = tid + i * kDraftThreads;
      const int row = c / UCPR, col = c - row * UCPR;
      const int j = rb * kReqBlock + row;
      if (j < B)
        gu[i] = __builtin_nontemporal_load(
            reinterpret_cast<const v4u32*>(ubase + (size_t)j * rowstep * ES + col * 16));
    }
  };
  auto store_tile_lds = [&](int ub) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int c = tid + i * kDraftThreads;
      const int row = c / UCPR, col = c - row * UCPR;
      *reinterpret_cast<v4u32*>(&sU[ub][row * USB + col * 16]) = gu[i];
    }
  };
  auto store_tile_global = [&](int rb, int ub) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int c = tid + i * kDraftThreads;
      const int row = c / UCPR, col = c - row * UCPR;
      const int j = rb * kReqBlock + row;
      if (j < B)
        *reinterpret_cast<v4u32*>(zbase + (size_t)j * rowstep * ES + col * 16) =
            *reinterpret_cast<const v4u32*>(&sU[ub][row * USB + col * 16]);
    }
  };

  const int nrb = (B + kReqBlock - 1) / kReqBlock;
  if (tid < kReqBlock) {
    sPrev[0][tid] = prev_of(tid);
    sPrev[1][tid] = prev_of(tid + kReqBlock);
  }
  if (fast_tile) load_tile(0);
  __syncthreads();  // tab, sPrev
  load_rows(0);
  store_rows(0);
  if (fast_tile) store_tile_lds(0);
  __syncthreads();

  for (int rb = 0; rb < nrb; ++rb) {
    const int j = rb * kReqBlock + tl;
    const bool valid = j < B;
    const int buf = rb & 1, ub = rb % 3;
    const float T = a.temperature[min(j, B - 1)];
    const bool more = rb + 1 < nrb;
    if (more) {
      load_rows(buf ^ 1);                 // rows of block rb + 1 (their ids were stored a block ago)
      if (fast_tile) load_tile(rb + 1);
    }
    int pn2 = 0;  // wave 1 fetches the ids of block rb + 2; clamped when stored
    const bool idw = tid >= 64 && tid < 64 + kReqBlock;
    if (idw) pn2 = prev_raw((rb + 2) * kReqBlock + tid - 64);
    // this lane's U_k values of the current block (stored in LDS before the last barrier)
    unsigned char* urow = &sU[ub][tl * USB + (wv * 32 + 4 * h) * ES];
    typedef typename std::conditional<ES == 2, uint2, float4>::type UVec;
    UVec uv[4];
    if (fast_tile) {
#pragma unroll
      for (int g = 0; g < 4; ++g) uv[g] = *reinterpret_cast<const UVec*>(urow + 8 * g * ES);
    }

    // Embedding operand (MFMA B: column = request, 8 consecutive k per lane half) from LDS.
    const uint16_t* rowp = &sB[buf][tl * RS + 8 * h];
    bf16x8 bop[kMaxSteps];  // every step's operand is read before the chain: the reads overlap
#pragma unroll
    for (int kk = 0; kk < kMaxSteps; ++kk)
      bop[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const v4u32*>(rowp + min(kk, nk - 1) * 16));
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < kMaxSteps; ++kk)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wop[kk], kk < nk ? bop[kk] : zero8, acc, 0, 0, 0);

    // Epilogue: lane holds D[token n0 + 8g + 4h + p][request j] in acc[4g + p].
    const size_t row = ((size_t)(valid ? j : 0) * G + k) * V;
    float zq[16];
    int bad = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int t0 = n0 + 8 * g + 4 * h;
      float zs[4];
      if (fast_tile) {
        unsigned char* q = urow + 8 * g * ES;
        if constexpr (ES == 2) {
          const uint2 w = uv[g];
          zs[0] = bf16_lo(w.x) + acc[4 * g];
          zs[1] = bf16_hi(w.x) + acc[4 * g + 1];
          zs[2] = bf16_lo(w.y) + acc[4 * g + 2];
          zs[3] = bf16_hi(w.y) + acc[4 * g + 3];
          uint2 o;
          const f32x2 v0 = {zs[0], zs[1]}, v1 = {zs[2], zs[3]};
          o.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(v0, bf16x2));
          o.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(v1, bf16x2));
          *reinterpret_cast<uint2*>(q) = o;
          zs[0] = bf16_lo(o.x); zs[1] = bf16_hi(o.x); zs[2] = bf16_lo(o.y); zs[3] = bf16_hi(o.y);
        } else {
          const float4 w = uv[g];
          zs[0] = w.x + acc[4 * g];
          zs[1] = w.y + acc[4 * g + 1];
          zs[2] = w.z + acc[4 * g + 2];
          zs[3] = w.w + acc[4 * g + 3];
          *reinterpret_cast<float4*>(q) = make_float4(zs[0], zs[1], zs[2], zs[3]);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          zq[4 * g + p] = valid ? zs[p] : -__builtin_inff();
          bad |= valid && __builtin_amdgcn_classf(zs[p], 0x203);  // NaN or +inf
        }
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const bool in = valid && t0 + p < V;
          float z = (in ? load_logit<ES>(a.base, row + t0 + p) : 0.f) + acc[4 * g + p];
          if constexpr (ES == 2) {
            const f32x2 v = {z, 0.f};
            const uint32_t o = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
            z = bf16_lo(o);
            if (in) reinterpret_cast<uint16_t*>(a.logits)[row + t0 + p] = (uint16_t)o;
          } else {
            if (in) reinterpret_cast<float*>(a.logits)[row + t0 + p] = z;
          }
          zq[4 * g + p] = in ? z : -__builtin_inff();
          bad |= in && __builtin_amdgcn_classf(z, 0x203);
        }
      }
    }
    Stat st = stat_empty();
    st.bad = bad;
    float zm = zq[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) zm = fmaxf(zm, zq[i]);
    st.zmax = zm;
    if (valid && T > 0.f && T < __builtin_inff() && zm > -__builtin_inff() && !bad) {
      const double c = kLog2eD / (double)T;
      const double m = ceil((double)zm * c);
      double s = 0.0;
#pragma unroll
      for (int i = 0; i < 16; ++i) s += exp2_tab(fma((double)zq[i], c, -m), tab);
      st.s = s;
      st.m = m;
    }
    // the two lane halves hold the same request
    stat_merge(st, stat_shfl_xor(st, 32));
    if (h == 0) sp[buf][wv][tl] = st;
    if (more) {
      store_rows(buf ^ 1);                            // read after the barrier below
      if (fast_tile) store_tile_lds((rb + 1) % 3);
    }
    if (idw) sPrev[buf][tid - 64] = prev_ok(pn2);    // ids of block rb + 2
    __syncthreads();
    if (fast_tile) store_tile_global(rb, ub);
    if (wv == 3 && h == 0 && valid) {
      Stat t = sp[buf][0][tl];
#pragma unroll
      for (int w = 1; w < kDraftThreads / 64; ++w) stat_merge(t, sp[buf][w][tl]);
      DPart p;
      p.s = t.s;
      p.m = t.m;
      p.zmax = t.zmax;
      p.bad = t.bad;
      p.pad0 = p.pad1 = 0;
      a.part[(size_t)j * a.nwg + blockIdx.x] = p;
    }
  }
}

// Step k: draw x_k for every request (one workgroup each).  Every thread takes a contiguous run of
// tiles; the workgroup finds the common reference, the total and the tile where the running sum
// (tile order = token order) passes u * total; wave 0 then walks that tile's 128 tokens.
template <int ES>
__global__ __launch_bounds__(kSampleThreads) void markov_sample_kernel(DraftArgs a) {
  constexpr int NW = kSampleThreads / 64;
  __shared__ Stat red[NW];
  __shared__ double wtot[NW];
  __shared__ int hitw[NW], lastw[NW];
  __shared__ int sel_w, first_max;
  __shared__ double sel_before;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int j = blockIdx.x;
  const int k = a.k, V = a.V, nwg = a.nwg;
  int st = (k == 0) ? 0 : a.req_status[j];
  const float T = a.temperature[j];
  if (k == 0) {
    if (!(T >= 0.f && T < __builtin_inff())) st |= SPEC_REQ_BAD_TEMPERATURE;
    const int x0 = a.anchor[j];
    if (x0 < 0 || x0 >= V) st |= SPEC_REQ_BAD_TOKEN;
  }
  const DPart* P = a.part + (size_t)j * nwg;
  const int per = (nwg + kSampleThreads - 1) / kSampleThreads;
  const int w0 = min(nwg, tid * per), w1 = min(nwg, w0 + per);
  Stat acc = stat_empty();
  for (int w = w0; w < w1; ++w) stat_merge(acc, from_part(P[w]));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) stat_merge(acc, stat_shfl_xor(acc, o));
  if (lane == 0) red[wv] = acc;
  __syncthreads();
  acc = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) stat_merge(acc, red[w]);

  if (st == 0 && (acc.bad || !(acc.zmax > -__builtin_inff()))) st |= SPEC_REQ_NONFINITE;
  // the first tile holding the row's maximum (greedy rows; a fallback of the draw)
  int myw = 0x7fffffff;
  if (st == 0)
    for (int w = w0; w < w1; ++w)
      if (P[w].zmax == acc.zmax) {
        myw = w;
        break;
      }
  myw = wave_min_i(myw);
  if (lane == 0) hitw[wv] = myw;
  __syncthreads();
  int wmax = hitw[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) wmax = min(wmax, hitw[w]);
  __syncthreads();
  const size_t row = ((size_t)j * a.G + k) * V;
  // wave 0: the first token of tile w holding the maximum
  auto first_max_token = [&](int w) -> int {
    const int t0 = w * kTileTokens + 2 * lane;
    const bool q0 = t0 < V && load_logit<ES>(a.logits, row + t0) == acc.zmax;
    const bool q1 = t0 + 1 < V && load_logit<ES>(a.logits, row + t0 + 1) == acc.zmax;
    const unsigned long long hb = __ballot(q0 || q1);
    const int L = hb ? __ffsll((long long)hb) - 1 : 0;
    return __shfl(q0 ? t0 : t0 + 1, L, SPEC_WAVE);
  };

  int x = -1;
  if (st == 0 && T == 0.f && wv == 0) x = first_max_token(wmax);
  if (st == 0 && T != 0.f) {  // uniform over the workgroup
    const double M = acc.m;
    const double c = kLog2eD / (double)T;
    double ls = 0.0;
    int mylast = -1;
    for (int w = w0; w < w1; ++w) {
      if (!(P[w].s > 0.0)) continue;
      const double e = ldexp(P[w].s, (int)fmax(P[w].m - M, -2000.0));
      ls += e;
      if (e > 0.0) mylast = w;
    }
    const double iw = wave_inclusive_sum(ls, lane);
    if (lane == 63) wtot[wv] = iw;
    __syncthreads();
    double base = 0.0, S = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wv) base += wtot[w];
      S += wtot[w];
    }
    const double incl = base + iw;
    const uint64_t seed = a.seed ? a.seed[j] : 0ull;
    const Philox4x64 blk = philox4x64_10((uint64_t)k + 1, (uint64_t)j, 1, 0, seed, 0);
    const double target = uniform53(blk.w0) * S;
    const unsigned long long hit = __ballot(incl > target);
    const int wl = wave_max_i(mylast);
    if (lane == 0) {
      hitw[wv] = hit ? wv * 64 + (__ffsll((long long)hit) - 1) : 0x7fffffff;
      lastw[wv] = wl;
    }
    __syncthreads();
    int first = 0x7fffffff, lastt = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      first = min(first, hitw[w]);
      lastt = max(lastt, lastw[w]);
    }
    if (tid == 0) {
      sel_w = lastt;                 // u * S rounded up to S: the last weighted tile,
      sel_before = -__builtin_inf(); // and in it the last weighted token
    }
    __syncthreads();
    if (tid == first) {  // the first thread whose running sum passes the target walks its tiles
      double cum = incl - ls;
      int ws = -1;
      double before = 0.0;
      for (int w = w0; w < w1; ++w) {
        if (!(P[w].s > 0.0)) continue;
        const double e = ldexp(P[w].s, (int)fmax(P[w].m - M, -2000.0));
        if (!(e > 0.0)) continue;
        if (cum + e > target) {
          ws = w;
          before = cum;
          break;
        }
        cum += e;
      }
      if (ws >= 0) {
        sel_w = ws;
        sel_before = before;
      } else if (mylast >= 0) {  // rounding: this run's last weighted tile, its last token
        sel_w = mylast;
      }
    }
    __syncthreads();
    int wsel = sel_w;
    const double before = sel_before;
    if (wsel < 0) wsel = wmax;  // cannot happen when S > 0
    if (wv == 0) {
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
        x = __shfl(p0 ? t0 : t0 + 1, Lb, SPEC_WAVE);
      } else {  // past the end of the tile: its last weighted token
        const unsigned long long nz = __ballot(e0 > 0.0 || e1 > 0.0);
        if (nz) {
          const int Ln = 63 - __clzll((long long)nz);
          x = __shfl(e1 > 0.0 ? t0 + 1 : t0, Ln, SPEC_WAVE);
        } else {  // cannot happen: the tile's largest token has weight
          x = first_max_token(wmax);
        }
      }
    }
  }
  if (tid == 0) {
    a.tokens[(size_t)j * a.G + k] = (st == 0) ? x : -1;
    a.req_status[j] = st;
  }
}

// After the last step: status, the tokens of bad requests, and the confidences (Eq. 7), one
// wave per (request, position), fp64 dot products.
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
  const int d = a.d;
  double t = 0.0;
  constexpr int VE = 16 / ES;  // elements per 16-byte vector
  const char* hrow = reinterpret_cast<const char*>(a.hidden) + wid * (size_t)d * ES;
  if ((d % VE) == 0 && ((reinterpret_cast<uintptr_t>(hrow) & 15) == 0)) {
    for (int v = lane; v < d / VE; v += 64) {
      const v4u32 q = *reinterpret_cast<const v4u32*>(hrow + (size_t)v * 16);
      const float* wp = a.conf_w + v * VE;
      if constexpr (ES == 2) {
        const uint32_t qs[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          t += (double)wp[2 * i] * (double)bf16_lo(qs[i]);
          t += (double)wp[2 * i + 1] * (double)bf16_hi(qs[i]);
        }
      } else {
        t += (double)wp[0] * (double)__uint_as_float(q.x);
        t += (double)wp[1] * (double)__uint_as_float(q.y);
        t += (double)wp[2] * (double)__uint_as_float(q.z);
        t += (double)wp[3] * (double)__uint_as_float(q.w);
      }
    }
  } else {
    for (int i = lane; i < d; i += 64) t += (double)a.conf_w[i] * (double)load_logit<ES>(a.hidden, wid * (size_t)d + i);
  }
  const uint16_t* e = a.W1 + (size_t)prev * a.r;  // rows are 16-byte aligned (r % 16 == 0)
  for (int v = lane; v < a.r / 8; v += 64) {
    const v4u32 q = *reinterpret_cast<const v4u32*>(e + v * 8);
    const float* wp = a.conf_w + d + v * 8;
    const uint32_t qs[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t += (double)wp[2 * i] * (double)bf16_lo(qs[i]);
      t += (double)wp[2 * i + 1] * (double)bf16_hi(qs[i]);
    }
  }
  t = wave_sum(t);
  if (a.conf_tau) t /= a.conf_tau[k];
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
                                     int32_t d, const void* hidden, const float* conf_w, const double* conf_tau,
                                     int32_t* tokens,
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
  a.hidden = hidden; a.conf_w = conf_w; a.conf_tau = conf_tau;
  a.tokens = tokens; a.logits = draft_logits; a.conf = conf; a.status = status;
  char* ws = reinterpret_cast<char*>(workspace);
  a.part = reinterpret_cast<DPart*>(ws);
  a.req_status = reinterpret_cast<int32_t*>(ws + align256((size_t)B * a.nwg * sizeof(DPart)));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned sgrid = (unsigned)B;
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
