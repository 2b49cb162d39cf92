// Markov-head sequential draft sampler and confidence head on gfx950.
//
// DSpark paper, §3.1 (sequential stage): the block is drafted left to right; position k draws x_k
// from softmax(U_k + B(x_{k-1}, .)) (Eq. 4), where the Markov head's transition bias is row
// x_{k-1} of a low-rank product, B(x_{k-1}, .) = W1[x_{k-1}] W2 (Eq. 5, r = 256 by default).
// §3.2.1 (Eq. 7): the confidence of position k is sigmoid(w . [h_k ; W1[x_{k-1}]]).
//
// One draft step k is two kernels:
//   markov_logits_kernel -- for every request at once, the bias is a dense product
//       [B x r] (gathered embedding rows) x [r x V] (projection): MFMA 16x16x32 bf16 tiles with
//       fp32 accumulation.  Each wave keeps the projection rows of its 32 tokens in registers and
//       walks the requests 32 at a time; the epilogue adds U_k, rounds to the storage type, writes
//       the draft logits and records per (request, 128-token tile) the largest stored value and
//       whether a NaN or +inf was stored.
//   markov_sample_kernel -- one 1024-thread workgroup per request.  T > 0: the weight of token v
//       is Q(z_v) = exp(z_v/T - zmax/T) in fp64, looked up for bf16 rows in an LDS table over the
//       bf16 values (evaluated once per value, the rest directly); one pass over the stored row
//       sums Q per range of 2048 tokens, u * total (u from the request's counter-based stream)
//       picks the range, and that range is walked again token by token in ascending order.  T = 0
//       takes the first-occurrence argmax from the tile records and one tile.
// After the last step markov_finish_kernel writes the confidences (fp64 dot products) and the
// per-request status.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "common.hpp"
#include "philox.hpp"
#include "qtable.hpp"
#include "spec_verify.h"

namespace spec {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int v2u32 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kDraftThreads = 256;   // markov_logits_kernel: 4 waves
constexpr int kTileTokens = 128;     // tokens per workgroup (32 per wave)
constexpr int kWaveTokens = kTileTokens / (kDraftThreads / 64);
constexpr int kReqBlock = 32;        // requests per block (two MFMA columns of 16)
constexpr int kMaxSteps = 16;        // rank / 16 at most (r <= 256)
constexpr int kSampleThreads = 256;  // markov_finish_kernel: a wave per item
constexpr int kDrawThreads = 1024;   // markov_sample_kernel: one workgroup per request
constexpr int kDrawWaves = kDrawThreads / 64;
constexpr int kDrawRange = 2048;     // tokens per range of the sampling pass (a wave step: 64 x 8)
constexpr int kDrawMaxRanges = (SPEC_MAX_V + kDrawRange - 1) / kDrawRange;

constexpr double kLog2eD = 1.44269504088896340736;

// The stored logits of one request over one 128-token tile: the largest value (-inf when none)
// and whether a NaN or +inf was stored.
struct DPart {
  float zmax;
  int32_t bad;
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
  DPart* part;               // [B rounded up to kReqBlock, nwg] workspace
  int32_t* req_status;       // [B] workspace
};

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
// block: each wave multiplies its projection rows (registers: two MFMA tiles of 16 tokens x r,
// 64 VGPRs at r = 256) by the block's embedding rows (LDS, two columns of 16 requests), each
// embedding operand read from LDS once for both token tiles (LDS reads of the operand bound this
// kernel: 32 tokens per wave halve them against 16); the epilogue reads U_k from an LDS tile,
// writes the rounded z_k back in place and folds the values into statistics; after the block's
// barrier the workgroup stores the z_k tile with whole-line 16-byte stores.  The embedding rows and
// the U_k tile of the next block are loaded (whole lines, 16 bytes per thread) while the current
// block computes.  Tiles that are not whole (the last one, or rows not 16-byte aligned) take
// per-element global accesses instead.  Operand k beyond r is zero on both sides (exact zeros).
// About 51 KB of LDS (bf16) and at most 168 VGPRs let three 4-wave workgroups share a CU.
template <int ES>
__global__ __launch_bounds__(kDraftThreads) __attribute__((amdgpu_waves_per_eu(3)))
void markov_logits_kernel(DraftArgs a) {
  constexpr int RS = kMaxSteps * 16 + 8;            // LDS row stride of the embedding rows (bf16)
  constexpr int USB = kTileTokens * ES + 16;        // LDS row stride of the U/z tile (bytes)
  constexpr int UCPR = kTileTokens * ES / 16;       // 16-byte chunks per tile row
  constexpr int UPT = kReqBlock * UCPR / kDraftThreads;  // chunks per thread (2 bf16, 4 fp32)
  constexpr int NW = kDraftThreads / 64;
  constexpr int NK = kMaxSteps / 2;                 // 16x16x32 steps at the largest rank
  constexpr int RPT = kReqBlock * (kMaxSteps * 16 / 8) / kDraftThreads;   // embedding chunks per thread
  static_assert(kWaveTokens == 32, "two 16-token MFMA tiles per wave");
  __shared__ DPart sp[2][NW][kReqBlock];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kReqBlock * RS];
  __shared__ __attribute__((aligned(16))) unsigned char sU[2][kReqBlock * USB];
  __shared__ int sPrev[4][kReqBlock];   // ids x_{k-1} of block b in sPrev[b % 4]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tn = lane & 15, q = lane >> 4;   // MFMA row (token) / column (request), and k or row group
  const int V = a.V, r = a.r, G = a.G, k = a.k, B = a.B;
  const int tile0 = blockIdx.x * kTileTokens;
  const int n0 = tile0 + wv * kWaveTokens;
  const bf16x8 zero8 = {};

  // Projection operands (MFMA A of token tile t: row = token n0 + 16 t + tn, k = 32 s + 8 q .. + 7).
  bf16x8 wop[2][NK];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint16_t* w2 = a.W2t + (size_t)min(n0 + 16 * t + tn, V - 1) * r;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const int kc = 32 * s + 8 * q;
      const bf16x8 v = load_bf16x8(w2 + min(kc, r - 8));
      wop[t][s] = kc < r ? v : zero8;
    }
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
  const int nchunk = kReqBlock * cpr;  // <= kReqBlock * 32: at most RPT per thread
  v4u32 gw[RPT];
  auto load_rows = [&](int pb) {   // unconditional: chunks past the rows reload the last one
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int c = min(tid + i * kDraftThreads, nchunk - 1);
      const int row = c / cpr, col = c - row * cpr;
      gw[i] = *reinterpret_cast<const v4u32*>(a.W1 + (size_t)sPrev[pb][row] * r + col * 8);
    }
  };
  auto store_rows = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
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
  auto load_tile = [&](int rb) {   // unconditional: rows past B reload the last request's
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int c = tid + i * kDraftThreads;
      const int row = c / UCPR, col = c - row * UCPR;
      const int j = min(rb * kReqBlock + row, B - 1);
      gu[i] = __builtin_nontemporal_load(
          reinterpret_cast<const v4u32*>(ubase + (size_t)j * rowstep * ES + col * 16));
    }
  };
  // the same thread mapping for the tile's LDS writes and the global stores' LDS reads, so that a
  // slot rewritten a block after its global store is ordered by program order
  auto store_tile_lds = [&](int ub) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int c = tid + i * kDraftThreads;
      const int row = c / UCPR, col = c - row * UCPR;
      *reinterpret_cast<v4u32*>(&sU[ub][row * USB + col * 16]) = gu[i];
    }
  };
  // Rows past B in the last block hold exactly request B-1's values (its id, its U_k row), so
  // they are stored to row B-1 again, which keeps the stores unconditional.
  auto store_tile_global = [&](int rb, int ub) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int c = tid + i * kDraftThreads;
      const int row = c / UCPR, col = c - row * UCPR;
      const int j = min(rb * kReqBlock + row, B - 1);
      *reinterpret_cast<v4u32*>(zbase + (size_t)j * rowstep * ES + col * 16) =
          *reinterpret_cast<const v4u32*>(&sU[ub][row * USB + col * 16]);
    }
  };

  // The loads of block b + 2 are issued while block b computes and land in LDS at the end of
  // block b + 1, a whole block later, so no block waits for its own loads; the ids of block b + 4
  // are fetched by wave 1 during block b and stored during block b + 1.  Tile slot b % 2 is
  // rewritten at the end of block b + 1, after its global store (issued after the barrier ending
  // block b) by the same threads.
  const int nrb = (B + kReqBlock - 1) / kReqBlock;
  const bool idw = tid >= 64 && tid < 64 + kReqBlock;
  if (tid < kReqBlock) {
#pragma unroll
    for (int b = 0; b < 3; ++b) sPrev[b][tid] = prev_of(b * kReqBlock + tid);
  }
  // every thread fetches the ids (only wave 1 stores them): no load under a condition in the loop
  int pn = prev_raw(3 * kReqBlock + (tid & (kReqBlock - 1)));   // ids of block 3
  // whole tiles (FAST) and the rest take separate copies of the walk, so no branch on the tile
  // kind sits inside it
  auto walk = [&](auto fast_c) {
  constexpr bool FAST = decltype(fast_c)::value;
  if constexpr (FAST) load_tile(0);
  __syncthreads();  // sPrev
  load_rows(0);
  store_rows(0);
  if constexpr (FAST) store_tile_lds(0);
  load_rows(1);     // block 1, in flight
  if constexpr (FAST) load_tile(1);
  __syncthreads();

  for (int rb = 0; rb < nrb; ++rb) {
    const int buf = rb & 1, ub = rb & 1;
    const bool more = rb + 1 < nrb;
    if (idw) sPrev[(rb + 3) & 3][tid - 64] = prev_ok(pn);    // ids of block rb + 3 (fetched a block ago)
    pn = prev_raw((rb + 4) * kReqBlock + (tid & (kReqBlock - 1)));   // ids of block rb + 4
    // this lane's U_k values of the current block (stored in LDS before the last barrier):
    // requests 16 c + tn of the block (c = 0, 1), tokens n0 + 16 t + 4 q .. + 3
    auto urow = [&](int t, int c) -> unsigned char* {
      return &sU[ub][(16 * c + tn) * USB + (wv * kWaveTokens + 16 * t + 4 * q) * ES];
    };

    // Embedding operand (MFMA B: column = request 16 c + tn, k = 32 s + 8 q .. + 7) from LDS,
    // each one used for both token tiles.
    f32x4 acc[2][2] = {};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint16_t* rowp = &sB[buf][(16 * c + tn) * RS + 8 * q];
      bf16x8 bop[NK];
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const v4u32*>(rowp + 32 * s));
        bop[s] = 32 * s + 8 * q < r ? v : zero8;
      }
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        acc[0][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop[0][s], bop[s], acc[0][c], 0, 0, 0);
        acc[1][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop[1][s], bop[s], acc[1][c], 0, 0, 0);
      }
    }

    // Epilogue: lane holds D[token n0 + 16 t + 4 q + p][request 16 c + tn] in acc[t][c][p].
    float zm[2];
    int bad[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int j = rb * kReqBlock + 16 * c + tn;
      const bool valid = j < B;
      const size_t row = ((size_t)(valid ? j : 0) * G + k) * V;
      float m = -__builtin_inff();
      int bd = 0;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int t0 = n0 + 16 * t + 4 * q;
        float zq[4];
        if constexpr (FAST) {
          float zs[4];
          if constexpr (ES == 2) {
            const uint2 w = *reinterpret_cast<const uint2*>(urow(t, c));
            zs[0] = bf16_lo(w.x) + acc[t][c][0];
            zs[1] = bf16_hi(w.x) + acc[t][c][1];
            zs[2] = bf16_lo(w.y) + acc[t][c][2];
            zs[3] = bf16_hi(w.y) + acc[t][c][3];
            uint2 o;
            const f32x2 v0 = {zs[0], zs[1]}, v1 = {zs[2], zs[3]};
            o.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(v0, bf16x2));
            o.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(v1, bf16x2));
            *reinterpret_cast<uint2*>(urow(t, c)) = o;
            zs[0] = bf16_lo(o.x); zs[1] = bf16_hi(o.x); zs[2] = bf16_lo(o.y); zs[3] = bf16_hi(o.y);
          } else {
            const float4 w = *reinterpret_cast<const float4*>(urow(t, c));
            zs[0] = w.x + acc[t][c][0];
            zs[1] = w.y + acc[t][c][1];
            zs[2] = w.z + acc[t][c][2];
            zs[3] = w.w + acc[t][c][3];
            *reinterpret_cast<float4*>(urow(t, c)) = make_float4(zs[0], zs[1], zs[2], zs[3]);
          }
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            zq[p] = valid ? zs[p] : -__builtin_inff();
            bd |= valid && __builtin_amdgcn_classf(zs[p], 0x203);  // NaN or +inf
          }
        } else {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const bool in = valid && t0 + p < V;
            float z = (in ? load_logit<ES>(a.base, row + t0 + p) : 0.f) + acc[t][c][p];
            if constexpr (ES == 2) {
              const f32x2 v = {z, 0.f};
              const uint32_t o = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
              z = bf16_lo(o);
              if (in) reinterpret_cast<uint16_t*>(a.logits)[row + t0 + p] = (uint16_t)o;
            } else {
              if (in) reinterpret_cast<float*>(a.logits)[row + t0 + p] = z;
            }
            zq[p] = in ? z : -__builtin_inff();
            bd |= in && __builtin_amdgcn_classf(z, 0x203);
          }
        }
        m = fmaxf(m, fmaxf(fmaxf(zq[0], zq[1]), fmaxf(zq[2], zq[3])));
      }
      // the four lane groups hold the same request
      m = fmaxf(m, __shfl_xor(m, 16, SPEC_WAVE));
      m = fmaxf(m, __shfl_xor(m, 32, SPEC_WAVE));
      bd |= __shfl_xor(bd, 16, SPEC_WAVE);
      bd |= __shfl_xor(bd, 32, SPEC_WAVE);
      zm[c] = m;
      bad[c] = bd;
    }
    if (q == 0) {
      sp[buf][wv][tn] = DPart{zm[0], bad[0]};
      sp[buf][wv][16 + tn] = DPart{zm[1], bad[1]};
    }
    if (more) {
      store_rows(buf ^ 1);                            // block rb + 1, read after the barrier below
      if constexpr (FAST) store_tile_lds((rb + 1) & 1);
    }
    load_rows((rb + 2) & 3);                          // block rb + 2 (past the end: valid ids, unused)
    if constexpr (FAST) load_tile(rb + 2);
    __syncthreads();
    if constexpr (FAST) store_tile_global(rb, ub);
    // the block's tile records (rows padded to whole blocks: a row past B is never read)
    if (wv == NW - 1 && lane < kReqBlock) {
      DPart t = sp[buf][0][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        t.zmax = fmaxf(t.zmax, sp[buf][w][lane].zmax);
        t.bad |= sp[buf][w][lane].bad;
      }
      a.part[(size_t)(rb * kReqBlock + lane) * a.nwg + blockIdx.x] = t;
    }
  }
  };
  if (fast_tile) walk(std::true_type{});
  else walk(std::false_type{});
}

// Step k: draw x_k for every request (one workgroup each).
struct DrawShared {
  double T64[64];
  double Qt[kQsize];
  double rsum[kDrawMaxRanges];  // Q summed per range of the row
  double wsum[kDrawWaves];
  float wz[kDrawWaves];
  int wb[kDrawWaves], cross[kDrawWaves], lastl[kDrawWaves];
  int sel, past, token;
  double target, before;
};

// Exact weight Q(z_v) of token v of a stored row (table when given and the value is tabulated).
template <int ES>
__device__ __forceinline__ double draw_weight(const char* row, int v, double invT, double R, const double* T64,
                                              const double* Qt) {
  if constexpr (ES == 2) {
    const uint32_t b = reinterpret_cast<const uint16_t*>(row)[v];
    if (Qt) {
      const uint32_t q = q_slot1(b);
      if (q < (uint32_t)kQsize) return Qt[q];
    }
    return q_direct(__uint_as_float(b << 16), invT, R, T64);
  } else {
    return q_direct(reinterpret_cast<const float*>(row)[v], invT, R, T64);
  }
}

// Sum of Q over the 8 bf16 tokens of one lane's 16-byte vector (lanes past the row's end hold
// tabulated filler and add nothing when MASK).
template <bool MASK>
__device__ __forceinline__ double draw_step(const uint4& d, double invT, double R, const double* T64,
                                            const double* Qt, bool live) {
  uint32_t w[4] = {d.x, d.y, d.z, d.w};
  if (MASK && !live) {
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = kFill2;
  }
  us2 kt[4];
  us2 kmax = (us2)(unsigned short)0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    kt[q] = q_slots(w[q]);
    kmax = __builtin_elementwise_max(kmax, kt[q]);
  }
  double s = 0.0;
  if (max((uint32_t)kmax.x, (uint32_t)kmax.y) < (uint32_t)kQsize) {
#pragma unroll
    for (int j = 0; j < 8; ++j) s += Qt[slot_of(kt, j)];
    if (MASK && !live) s = 0.0;
  } else {
#pragma unroll 1
    for (int j = 0; j < 8; ++j) s += q_direct(__uint_as_float(half16(w, j) << 16), invT, R, T64);
  }
  return s;
}

template <int ES>
__global__ __launch_bounds__(kDrawThreads) void markov_sample_kernel(DraftArgs a) {
  __shared__ DrawShared sh;
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
  init_t64(sh.T64);
  // the tile records: two per thread cover V <= 262144 (clamped indices, masked below)
  const DPart* P = a.part + (size_t)j * nwg;
  const DPart p0 = P[min(tid, nwg - 1)], p1 = P[min(tid + kDrawThreads, nwg - 1)];
  const char* row = reinterpret_cast<const char*>(a.logits) + ((size_t)j * a.G + k) * (size_t)V * ES;
  const int NR = (V + kDrawRange - 1) / kDrawRange;
  const bool vec = ES == 2 && (reinterpret_cast<uintptr_t>(row) & 15u) == 0 && (V & 7) == 0 && V >= 8;
  // a lane past the row's end loads a clamped address and is masked in its step
  auto load = [&](int rr, int sub) -> uint4 {
    const int v0 = min(rr * kDrawRange + sub * 512 + lane * 8, V - 8);
    return *reinterpret_cast<const uint4*>(row + (size_t)v0 * 2);
  };
  // A sampled row (T > 0) is read from the start: the first two ranges of each wave are in flight
  // while the tile records are reduced and the table is built (a request found bad meanwhile leaves
  // them unused).
  uint4 buf[8];
  if (vec && T > 0.f) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int sub = 0; sub < 4; ++sub) buf[4 * h + sub] = load(wv + h * kDrawWaves, sub);
  }
  // the row's largest stored value and bad flag
  float zm = (tid < nwg) ? p0.zmax : -__builtin_inff();
  int bad = (tid < nwg) ? p0.bad : 0;
  if (tid + kDrawThreads < nwg) {
    zm = fmaxf(zm, p1.zmax);
    bad |= p1.bad;
  }
  for (int w = tid + 2 * kDrawThreads; w < nwg; w += kDrawThreads) {
    const DPart p = P[w];
    zm = fmaxf(zm, p.zmax);
    bad |= p.bad;
  }
  zm = wave_max(zm);
  bad = wave_or_i(bad);
  if (lane == 0) {
    sh.wz[wv] = zm;
    sh.wb[wv] = bad;
  }
  __syncthreads();
  zm = sh.wz[0];
  bad = sh.wb[0];
#pragma unroll
  for (int w = 1; w < kDrawWaves; ++w) {
    zm = fmaxf(zm, sh.wz[w]);
    bad |= sh.wb[w];
  }
  if (st == 0 && (bad || !(zm > -__builtin_inff()))) st |= SPEC_REQ_NONFINITE;
  int x = -1;
  if (st == 0 && T == 0.f) {
    // the first tile holding the maximum, then its first token holding it
    int myw = 0x7fffffff;
    for (int w = tid; w < nwg; w += kDrawThreads)
      if (P[w].zmax == zm) {
        myw = w;
        break;
      }
    myw = wave_min_i(myw);
    if (lane == 0) sh.cross[wv] = myw;
    __syncthreads();
    if (wv == 0) {
      int w0 = sh.cross[0];
#pragma unroll
      for (int w = 1; w < kDrawWaves; ++w) w0 = min(w0, sh.cross[w]);
      const int t0 = w0 * kTileTokens + 2 * lane;
      const bool q0 = t0 < V && load_logit<ES>(row, t0) == zm;
      const bool q1 = t0 + 1 < V && load_logit<ES>(row, t0 + 1) == zm;
      const unsigned long long hb = __ballot(q0 || q1);
      const int Lb = hb ? __ffsll((long long)hb) - 1 : 0;
      x = read_lane(q0 ? t0 : t0 + 1, Lb);
    }
  } else if (st == 0) {  // uniform over the workgroup
    const double invT = 1.0 / (double)T;
    const double R = (double)zm * invT;      // the largest weight is exp(0) = 1
    const double* Qt = (ES == 2) ? sh.Qt : nullptr;
    if (ES == 2) build_qtab(sh.Qt, invT, R, sh.T64);
    lds_barrier();   // the table; the row loads stay in flight
    if (vec) {
      // the wave's ranges wv + q NS, q = 0 .. nq - 1, two in flight (8 vectors per lane): slots
      // 0..3 hold the even q, 4..7 the odd q.  The main loop runs while both refills exist and
      // refills unconditionally (a load under a condition would leave the compiler unsure of the
      // order of the loads in flight, and it would then wait for all of them before every step);
      // the last two or three ranges follow.  Only a wave's last range can be the row's partial one.
      const int NS = kDrawWaves;
      const int nq = (wv < NR) ? (NR - wv + NS - 1) / NS : 0;
      auto range = [&](int rr, int h, bool refill, int rnext) {
        double s = 0.0;
        const bool tail = (rr + 1) * kDrawRange > V;
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
          const int v0 = rr * kDrawRange + sub * 512 + lane * 8;
          if (!tail) s += draw_step<false>(buf[4 * h + sub], invT, R, sh.T64, Qt, true);
          else if (rr * kDrawRange + sub * 512 < V)
            s += draw_step<true>(buf[4 * h + sub], invT, R, sh.T64, Qt, v0 < V);
          if (refill) buf[4 * h + sub] = load(rnext, sub);
        }
        s = wave_sum(s);
        if (lane == 0) sh.rsum[rr] = s;
      };
      int q = 0;
      for (; q + 3 < nq; q += 2) {
        range(wv + q * NS, 0, true, wv + (q + 2) * NS);
        range(wv + (q + 1) * NS, 1, true, wv + (q + 3) * NS);
      }
      if (q < nq) range(wv + q * NS, 0, q + 2 < nq, wv + (q + 2) * NS);
      if (q + 1 < nq) range(wv + (q + 1) * NS, 1, false, 0);
      if (q + 2 < nq) range(wv + (q + 2) * NS, 0, false, 0);
    } else {
      for (int rr = wv; rr < NR; rr += kDrawWaves) {
        double s = 0.0;
        const int e = min(V, (rr + 1) * kDrawRange);
        for (int v = rr * kDrawRange + lane; v < e; v += 64) s += draw_weight<ES>(row, v, invT, R, sh.T64, Qt);
        s = wave_sum(s);
        if (lane == 0) sh.rsum[rr] = s;
      }
    }
    __syncthreads();
    // wave 0: prefix over the ranges (four per lane), the total, u * total and the first range
    // whose prefix passes it
    static_assert(kDrawMaxRanges <= 4 * SPEC_WAVE, "four ranges per lane");
    if (wv == 0) {
      double v4[4], pre[4], t = 0.0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = lane * 4 + u;
        v4[u] = (r < NR) ? sh.rsum[r] : 0.0;
        t += v4[u];
      }
      const double incl = wave_inclusive_sum(t, lane);
      double run = incl - t;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        run += v4[u];
        pre[u] = run;
      }
      const double W = read_lane(incl, 63);
      const uint64_t seed = a.seed ? a.seed[j] : 0ull;
      const Philox4x64 blk = philox4x64_10((uint64_t)k + 1, (uint64_t)j, 1, 0, seed, 0);
      const double target = uniform53(blk.w0) * W;
      int f = 4;
#pragma unroll
      for (int u = 3; u >= 0; --u)
        if (lane * 4 + u < NR && pre[u] > target) f = u;
      const unsigned long long m = __ballot(f < 4);
      int sel = NR;
      double before = 0.0;
      if (m) {
        const int fl = (int)__ffsll((long long)m) - 1;
        sel = fl * 4 + read_lane(f, fl);
        if (sel > 0) {
          const int ub = (sel - 1) & 3;
          const double mine = ub == 0 ? pre[0] : ub == 1 ? pre[1] : ub == 2 ? pre[2] : pre[3];
          before = read_lane(mine, (sel - 1) >> 2);
        }
      }
      if (lane == 0) {
        sh.target = target;
        sh.sel = sel;
        sh.past = (sel >= NR);
        sh.before = before;
        sh.token = -1;
      }
    }
    __syncthreads();
    const double target = sh.target;
    if (sh.past) {
      // u * total at or past the total (rounding): the last token with weight
      for (int r = NR - 1; r >= 0; --r) {
        int best = -1;
        for (int v = r * kDrawRange + tid; v < min(V, (r + 1) * kDrawRange); v += kDrawThreads)
          if (draw_weight<ES>(row, v, invT, R, sh.T64, Qt) > 0.0) best = v;
        best = wave_max_i(best);
        if (lane == 0) sh.lastl[wv] = best;
        __syncthreads();
        if (tid == 0) {
          int b = -1;
#pragma unroll
          for (int w = 0; w < kDrawWaves; ++w) b = max(b, sh.lastl[w]);
          if (b >= 0) sh.token = b;
        }
        __syncthreads();
        if (sh.token >= 0) break;
      }
    } else {
      // the selected range, two tokens per thread in ascending order
      constexpr int TPT = kDrawRange / kDrawThreads;
      const int base = sh.sel * kDrawRange + tid * TPT;
      double wt[TPT];
      double xs = 0.0;
#pragma unroll
      for (int q = 0; q < TPT; ++q) {
        const int v = base + q;
        wt[q] = (v < V) ? draw_weight<ES>(row, v, invT, R, sh.T64, Qt) : 0.0;
        xs += wt[q];
      }
      const double incl = wave_inclusive_sum(xs, lane);
      if (lane == 63) sh.wsum[wv] = incl;
      __syncthreads();
      double wb = 0.0;
#pragma unroll
      for (int q = 0; q < kDrawWaves; ++q) wb += (q < wv) ? sh.wsum[q] : 0.0;   // reads issued together
      const double Pb = sh.before + wb;
      const double excl = incl - xs;
      const unsigned long long m = __ballot(Pb + incl > target);
      const unsigned long long pos = __ballot(xs > 0.0);
      if (lane == 0) {
        sh.cross[wv] = m ? (int)(__ffsll((long long)m) - 1) : 64;
        sh.lastl[wv] = pos ? 63 - __clzll((long long)pos) : -1;
      }
      __syncthreads();
      // the first wave with a crossing, else the last wave with weight (all records read at once)
      int cw = -1, cl = -1, lw = -1, ll = -1;
#pragma unroll
      for (int q = kDrawWaves - 1; q >= 0; --q) {
        const int c = sh.cross[q], l = sh.lastl[q];
        if (c < 64) {
          cw = q;
          cl = c;
        }
        if (lw < 0 && l >= 0) {
          lw = q;
          ll = l;
        }
      }
      if (cw < 0) {  // rounding left no crossing: the last thread with weight
        cw = lw;
        cl = ll;
      }
      if (wv == cw && lane == cl) {
        double acc = Pb + excl;
        int tok = -1, lastpos = -1;
#pragma unroll
        for (int q = 0; q < TPT; ++q) {
          if (wt[q] > 0.0) lastpos = base + q;
          acc += wt[q];
          if (tok < 0 && acc > target && wt[q] > 0.0) tok = base + q;
        }
        sh.token = (tok >= 0) ? tok : lastpos;
      }
    }
    __syncthreads();
    x = sh.token;
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

// Tile records [B rounded up to whole request blocks, tiles], then the request status.
size_t draft_part_rows(int B) { return ((size_t)B + kReqBlock - 1) / kReqBlock * kReqBlock; }
size_t draft_ws_bytes(int B, int V) {
  return align256(draft_part_rows(B) * num_tiles(V) * sizeof(DPart)) + align256((size_t)B * sizeof(int32_t));
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
  a.req_status = reinterpret_cast<int32_t*>(ws + align256(draft_part_rows(B) * a.nwg * sizeof(DPart)));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned sgrid = (unsigned)B;
  for (int k = 0; k < gamma; ++k) {
    a.k = k;
    if (dtype == SPEC_BF16) {
      hipLaunchKernelGGL(markov_logits_kernel<2>, dim3(a.nwg), dim3(kDraftThreads), 0, s, a);
      hipLaunchKernelGGL(markov_sample_kernel<2>, dim3(sgrid), dim3(kDrawThreads), 0, s, a);
    } else {
      hipLaunchKernelGGL(markov_logits_kernel<4>, dim3(a.nwg), dim3(kDraftThreads), 0, s, a);
      hipLaunchKernelGGL(markov_sample_kernel<4>, dim3(sgrid), dim3(kDrawThreads), 0, s, a);
    }
  }
  const unsigned fgrid = (unsigned)(((size_t)B * gamma + 3) / 4);
  if (dtype == SPEC_BF16)
    hipLaunchKernelGGL(markov_finish_kernel<2>, dim3(fgrid), dim3(kSampleThreads), 0, s, a);
  else
    hipLaunchKernelGGL(markov_finish_kernel<4>, dim3(fgrid), dim3(kSampleThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}
