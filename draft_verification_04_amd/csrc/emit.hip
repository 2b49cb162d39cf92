// The emitted token of every request, on gfx950.
//
// After the first rejection n < L the target appends a token drawn from the
// normalised residual max(0, p_t - p_d) of row n; when all L drafts passed it
// appends a token from target row L (DSpark paper §1; with L = 0 this is the
// fresh target token of the paper's appendix counterexample).  The draw is an
// inverse CDF in ascending token order at the emit uniform: the smallest v
// with C(v) > u * W.
//
// Every quantity here is fp64: tokens sit ~1/V apart on the CDF, so the
// cumulative sums must be right to ~1e-12 relative for the draw to agree with
// an exact computation except on a vanishing set of uniforms.
//
// One function gives every token's weight:  Q(z) = exp(z/T - R_t), R_t the
// streaming kernel's log-normaliser of target row n (accurate to ~1e-8).
// For both rows p = Q(z) / sum Q(z) over the row (the draft row's own offset
// cancels), so with S_t = sum Q(z_t), S_d = sum Q(z_d) the residual weight of
// token v is  w_v = max(0, Q(z_t,v)/S_t - Q(z_d,v)/S_d).
//
// emit_pass_kernel   (request, segment) workgroups read the emit row(s) once.
//   bf16 rows: Q of every bf16 value with |z| in [2^-20, 128) is tabulated in
//   LDS (6912 fp64 entries, each computed by the same formula as the direct
//   path, so both give identical bits).  The sign of p_t - p_d is decided
//   with the approximate normalisers (S_t ~ 1, S_d ~ exp(R_d - R_t)) whenever
//   the ratio clears a 1e-5 margin, far above their error; the few tokens
//   inside the margin are recorded and weighed exactly later.  Per range of
//   2048 tokens a wave leaves A = sum Q(z_t) and D = sum Q(z_d) over tokens
//   with p_t > p_d, and Tall = sum Q(z_t) over all tokens.
// emit_final_kernel  one workgroup per request: S_t, S_d, range weights
//   A/S_t - D/S_d (+ recorded tokens), prefix scan, and the range holding
//   u * W recomputed token by token.  It also writes every output.
#include "common.hpp"
#include "philox.hpp"
#include "verify_impl.hpp"

#include <float.h>
#include <math.h>

namespace spec {

constexpr double kAmbTol = 1e-5;
constexpr int kQefLo = 107, kQefHi = 133;               // bf16 exponent fields tabulated
constexpr int kQper = (kQefHi - kQefLo + 1) * 128;      // 3456 values per sign
constexpr int kQsize = 2 * kQper;                       // 6912 entries, 55296 bytes
constexpr int kSub = 512;                               // tokens per wave step (64 lanes x 8)
constexpr int kSubPerRange = kRangeElems / kSub;        // 4

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

// Q of a bf16 bit pattern, from the table when tabulated.
__device__ __forceinline__ double q_bf16(uint32_t b, double invT, double R, const double* T64, const double* Qt) {
  const uint32_t t = (b & 0x7fffu) - (uint32_t)(kQefLo << 7);
  if (t < (uint32_t)kQper) return Qt[t + ((b & 0x8000u) ? kQper : 0)];
  return q_direct(__uint_as_float(b << 16), invT, R, T64);
}

__device__ __forceinline__ void init_t64(double* T64) {
  if (threadIdx.x < 64) T64[threadIdx.x] = exp2((double)threadIdx.x * (1.0 / 64.0));
}

__device__ void build_qtab(double* Qt, double invT, double R, const double* T64) {
  for (int idx = threadIdx.x; idx < kQsize; idx += blockDim.x) {
    const uint32_t s = idx >= kQper;
    const uint32_t t = idx - s * kQper;
    const uint32_t bits = (s << 15) | ((uint32_t)(kQefLo << 7) + t);
    Qt[idx] = q_direct(__uint_as_float(bits << 16), invT, R, T64);
  }
}

struct EmitRows {
  const char* t;
  const char* d;  // nullptr: single target row (appended / fresh token)
  double invT, R;
  float tht, thd;
  double cd;      // exp(R_t - R_d): p_d ~ cd * Q(z_d) with the approximate normalisers
};

template <bool BF16>
__device__ __forceinline__ EmitRows emit_rows(const VerifyArgs& a, int i, int n) {
  constexpr int ES = BF16 ? 2 : 4;
  const int G = a.G, V = a.V;
  const int L = a.lengths ? a.lengths[i] : G;
  EmitRows e;
  const RowStat rt = a.rows_t[(size_t)i * (G + 1) + n];
  e.t = target_row<ES>(a, i, n);
  e.R = rt.lse2 * kLn2;
  e.tht = rt.theta;
  e.invT = 1.0 / (double)a.temperature[i];
  e.d = nullptr;
  e.thd = -INFINITY;
  e.cd = 1.0;
  if (n < L) {
    const RowStat rd = a.rows_d[(size_t)i * G + n];
    e.d = draft_row<ES>(a, i, n);
    e.thd = rd.theta;
    e.cd = exp(e.R - rd.lse2 * kLn2);
  }
  return e;
}

// Q of token v of a row (any dtype, any alignment), kept-set aware.
template <bool BF16>
__device__ __forceinline__ double q_at(const char* row, int v, float th, double invT, double R, const double* T64) {
  const float z = load_elem<BF16>(row, v);
  return (z >= th) ? q_direct(z, invT, R, T64) : 0.0;
}

// Per-lane accumulators for one range.
struct Acc {
  double sd;       // running total of E_d over everything this lane saw
  double A, D, T;  // this range
};

// Accumulate one token pair; returns whether its residual sign is uncertain (p_t and p_d
// within the margin of each other with the approximate normalisers): such tokens are
// recorded by the caller and weighed exactly later.  No branches, so the table reads of a
// whole step can be in flight together.
__device__ __forceinline__ bool classify(Acc& c, double qt, double qd, double cdh, double cdl) {
  c.sd += qd;
  c.T += qt;
  const bool pos = qt > cdh * qd;
  // fma(1, q, s) = s + q and fma(0, q, s) = s, rounded as the plain sums (q is finite here, or
  // the normaliser check sends the request to the exact path): one select instead of four
  const double one = pos ? 1.0 : 0.0;
  c.A = fma(one, qt, c.A);
  c.D = fma(one, qd, c.D);
  return !pos && qt > 0.0 && qt >= cdl * qd;
}

// Record token v as uncertain (rare).
__device__ __forceinline__ void record_uncertain(const VerifyArgs& a, int i, int v) {
  const int slot = atomicAdd(&a.ereq[i].amb_n, 1);
  if (slot < kAmbCap) a.amb[(size_t)i * kAmbCap + slot] = v;
}

constexpr int kMaxWaves = 1024 / SPEC_WAVE;  // largest emit workgroup, in waves

struct PassShared {
  double T64[64];
  double Qt[kQsize];
  double red[2][kMaxWaves];
  int st, n;
};

// Table slot of a bf16 bit pattern, or -1 when it is not tabulated.
__device__ __forceinline__ int q_slot(uint32_t b) {
  const uint32_t t = (b & 0x7fffu) - (uint32_t)(kQefLo << 7);
  return (t < (uint32_t)kQper) ? (int)(t + ((b & 0x8000u) ? kQper : 0)) : -1;
}

__device__ __forceinline__ uint32_t half16(const uint32_t (&w)[4], int j) {
  return (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu);
}

// One step (64 lanes x 8 tokens) of a bf16 row pair from registers.  A lane whose 16 tokens
// are all tabulated reads Q from the table; otherwise (rare: |z| < 2^-20, |z| >= 128,
// infinities) it evaluates the same formula directly for the whole step.
template <bool RESID>
__device__ __forceinline__ void step_bf16(Acc& c, const uint4& dt, const uint4& dd, const EmitRows& e,
                                          double cdh, double cdl, int v0, const VerifyArgs& a, int i,
                                          const double* T64, const double* Qt) {
  constexpr bool resid = RESID;
  const uint32_t wt[4] = {dt.x, dt.y, dt.z, dt.w};
  const uint32_t wd[4] = {dd.x, dd.y, dd.z, dd.w};
  bool miss = false;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    miss |= q_slot(half16(wt, j)) < 0;
    if (resid) miss |= q_slot(half16(wd, j)) < 0;
  }
  unsigned amb = 0;
  if (!miss) {
    // two halves of four tokens: eight table reads in flight, registers kept in check
#pragma unroll
    for (int h = 0; h < 8; h += 4) {
      double qt[4], qd[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qt[j] = Qt[q_slot(half16(wt, h + j))];
        qd[j] = resid ? Qt[q_slot(half16(wd, h + j))] : 0.0;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (resid) amb |= (unsigned)classify(c, qt[j], qd[j], cdh, cdl) << (h + j);
        else c.T += qt[j];
      }
    }
  } else {
#pragma unroll 1
    for (int j = 0; j < 8; ++j) {
      const double qt = q_direct(__uint_as_float(half16(wt, j) << 16), e.invT, e.R, T64);
      if (resid) {
        const double qd = q_direct(__uint_as_float(half16(wd, j) << 16), e.invT, e.R, T64);
        amb |= (unsigned)classify(c, qt, qd, cdh, cdl) << j;
      } else {
        c.T += qt;
      }
    }
  }
  if (amb) {
#pragma unroll 1
    for (int j = 0; j < 8; ++j)
      if ((amb >> j) & 1u) record_uncertain(a, i, v0 + j);
  }
}

// The ranges of request i that segment `seg` owns, each written as an EmitRange to out[r]
// (global memory, or LDS when the same workgroup finishes the request); each wave's sum of
// E_d goes to sh.red[1][wave].
template <bool BF16, bool TOPK>
__device__ void pass_ranges(PassShared& sh, const VerifyArgs& a, int i, int seg, const EmitRows& e,
                            EmitRange* out) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int NWPB = (int)(blockDim.x >> 6);
  const int NWT = a.emit_segs * NWPB;
  const int V = a.V, NR = num_ranges(V);
  const bool resid = (e.d != nullptr);
  const double cdh = e.cd * (1.0 + kAmbTol), cdl = e.cd * (1.0 - kAmbTol);
  const bool aligned = ((reinterpret_cast<uintptr_t>(e.t) | reinterpret_cast<uintptr_t>(e.d)) & 15u) == 0;
  // ranges a wave can read whole with 16-byte loads
  const int NRfull = (BF16 && !TOPK && aligned) ? V / kRangeElems : 0;
  Acc c{0.0, 0.0, 0.0, 0.0};
  int r = seg * NWPB + wave;
  if (BF16 && !TOPK) {
    // the 4 steps of a range are in flight at once; each register slot is refilled with
    // the same step of the wave's next range as soon as it has been consumed
    uint4 bt[kSubPerRange], bd[kSubPerRange];
    auto load = [&](int rr, int sub, uint4& t, uint4& d) {
      const size_t off = ((size_t)rr * kRangeElems + sub * kSub + lane * 8) * 2;
      t = *reinterpret_cast<const uint4*>(e.t + off);
      d = resid ? *reinterpret_cast<const uint4*>(e.d + off) : make_uint4(0, 0, 0, 0);
    };
    if (r < NRfull) {
#pragma unroll
      for (int sub = 0; sub < kSubPerRange; ++sub) load(r, sub, bt[sub], bd[sub]);
    }
    while (r < NRfull) {
      const int rn = r + NWT;
      c.A = c.D = c.T = 0.0;
#pragma unroll
      for (int sub = 0; sub < kSubPerRange; ++sub) {
        const int v0 = r * kRangeElems + sub * kSub + lane * 8;
        if (resid) step_bf16<true>(c, bt[sub], bd[sub], e, cdh, cdl, v0, a, i, sh.T64, sh.Qt);
        else step_bf16<false>(c, bt[sub], bd[sub], e, cdh, cdl, v0, a, i, sh.T64, sh.Qt);
        if (rn < NRfull) load(rn, sub, bt[sub], bd[sub]);
      }
      const double A = wave_sum(c.A), D = wave_sum(c.D), T = wave_sum(c.T);
      if (lane == 0) out[r] = EmitRange{A, D, T};
      r = rn;
    }
  }
  // ranges with a ragged end, unaligned rows, fp32 rows and top-k rows: token by token
  for (; r < NR; r += NWT) {
    c.A = c.D = c.T = 0.0;
    for (int sub = 0; sub < kSubPerRange; ++sub) {
      const int base = r * kRangeElems + sub * kSub + lane * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int v = base + j;
        if (v < V) {
          const float zt = load_elem<BF16>(e.t, v);
          const float zd = resid ? load_elem<BF16>(e.d, v) : -INFINITY;
          if (!TOPK || zt >= e.tht || (resid && zd >= e.thd)) {
            const double qt = (zt >= e.tht) ? q_direct(zt, e.invT, e.R, sh.T64) : 0.0;
            if (resid) {
              const double qd = (zd >= e.thd) ? q_direct(zd, e.invT, e.R, sh.T64) : 0.0;
              if (classify(c, qt, qd, cdh, cdl)) record_uncertain(a, i, v);
            } else {
              c.T += qt;
            }
          }
        }
      }
    }
    const double A = wave_sum(c.A), D = wave_sum(c.D), T = wave_sum(c.T);
    if (lane == 0) out[r] = EmitRange{A, D, T};
  }
  const double sd = wave_sum(c.sd);
  if (lane == 0) {
    sh.red[1][wave] = sd;
  }
}

// Decision of request i by wave 0 into sh.st / sh.n (the whole block waits for it).
__device__ __forceinline__ void decide_into(PassShared& sh, const VerifyArgs& a, int i) {
  if (threadIdx.x < SPEC_WAVE) {
    int st, n;
    request_decision(a, i, &st, &n);
    if (threadIdx.x == 0) {
      sh.st = st;
      sh.n = n;
    }
  }
  __syncthreads();
}

// The emit pass over segment `seg` of request i (after its decision, sampling only).
template <bool BF16>
__device__ void run_pass(PassShared& sh, const VerifyArgs& a, int i, int seg, int n, EmitRange* out) {
  const EmitRows e = emit_rows<BF16>(a, i, n);
  const int K = a.top_k ? a.top_k[i] : 0;
  const bool topk = K > 0 && K < a.V;
  if (BF16 && !topk) {
    build_qtab(sh.Qt, e.invT, e.R, sh.T64);
    __syncthreads();
    pass_ranges<BF16, false>(sh, a, i, seg, e, out);
  } else if (topk) {
    pass_ranges<BF16, true>(sh, a, i, seg, e, out);
  } else {
    pass_ranges<BF16, false>(sh, a, i, seg, e, out);
  }
  __syncthreads();
}

template <bool BF16>
__global__ __launch_bounds__(kPassThreads) void emit_pass_kernel(VerifyArgs a) {
  __shared__ PassShared sh;
  const int i = a.r0 + (int)blockIdx.x / a.emit_segs, seg = (int)blockIdx.x % a.emit_segs;
  init_t64(sh.T64);
  decide_into(sh, a, i);
  const int st = sh.st, n = sh.n;
  if (st || a.temperature[i] == 0.f) return;
  run_pass<BF16>(sh, a, i, seg, n, a.ranges + (size_t)i * num_ranges(a.V));
  if (threadIdx.x == 0) {
    double y = 0.0;
    for (int w = 0; w < kPassThreads / SPEC_WAVE; ++w) y += sh.red[1][w];
    a.ereq[i].sd_part[seg] = y;
  }
}

constexpr int kMaxRanges = (SPEC_MAX_V + kRangeElems - 1) / kRangeElems;

struct FinalShared {
  double T64[64];
  double R[kMaxRanges];     // range weights, then inclusive prefix sums
  double corr[kMaxRanges];  // weights of the recorded uncertain-sign tokens
  EmitRange rg[kMaxRanges]; // the emit pass's range sums, fetched early
  int na;                   // uncertain-sign tokens recorded
  double wsum[kMaxWaves];
  double amb_w[kAmbCap];
  int amb_v[kAmbCap];
  int amb_sorted[kAmbCap];
  int st, n, slow, use_t, sel, past, token;
  double St, Sd, target, before;
};

// Exact weight of token v: residual (resid) or Q(z_t) (target row, any scale).
template <bool BF16>
__device__ __forceinline__ double weight(const EmitRows& e, int v, bool resid, double St, double Sd,
                                         const double* T64) {
  const double qt = q_at<BF16>(e.t, v, e.tht, e.invT, e.R, T64);
  if (!resid) return qt;
  const double qd = q_at<BF16>(e.d, v, e.thd, e.invT, e.R, T64);
  return fmax(0.0, qt / St - qd / Sd);
}

// Everything after request i's decision (st, n): status and outputs, then, for a sampling
// request, the emitted token from the emit pass's range sums (sh.rg, sh.St, sh.Sd, sh.na
// filled).  Works for any block of 256 .. 1024 threads (a multiple of 256); the token octets
// of the crossing range belong to the first 256 threads, the others only join loops and
// barriers.
template <bool BF16>
__device__ void finish_request(FinalShared& sh, const VerifyArgs& a, int i, int st, int n) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int NW = (int)(blockDim.x >> 6);
  const int G = a.G, V = a.V;
  const int NR = num_ranges(V);
  const int L = a.lengths ? a.lengths[i] : G;
  if (a.status && tid == 0) a.status[i] = st;
  if (st) {
    if (tid == 0) a.num_accepted[i] = 0;
    for (int k = tid; k <= G; k += blockDim.x) a.out_tokens[(size_t)i * (G + 1) + k] = -1;
    if (a.accept_prob)
      for (int k = tid; k < G; k += blockDim.x) a.accept_prob[(size_t)i * G + k] = NAN;
    return;
  }
  if (tid == 0) a.num_accepted[i] = n;
  if (a.accept_prob)
    for (int k = tid; k < G; k += blockDim.x)
      a.accept_prob[(size_t)i * G + k] = (k < L) ? (float)a.acc[(size_t)i * G + k].r : NAN;
  for (int k = tid; k <= G; k += blockDim.x) {
    if (k < n) a.out_tokens[(size_t)i * (G + 1) + k] = a.tokens[(size_t)i * G + k];
    else if (k > n) a.out_tokens[(size_t)i * (G + 1) + k] = -1;
  }
  const bool greedy = a.greedy_only || a.temperature[i] == 0.f;
  if (greedy) {
    if (tid == 0) a.out_tokens[(size_t)i * (G + 1) + n] = a.rows_t[(size_t)i * (G + 1) + n].argmax;
    return;
  }

  const EmitRows e = emit_rows<BF16>(a, i, n);
  const bool resid = (e.d != nullptr);
  double ua, ue;
  verify_uniforms(a.seed[i], (uint64_t)i, (uint64_t)n, &ua, &ue);
  const double St = sh.St, Sd = sh.Sd;
  // the sign classification assumed cd * S_d / S_t = 1 to within half its margin
  const double rho = resid ? e.cd * Sd / St : 1.0;
  const bool slow = resid && (!(fabs(rho - 1.0) <= 0.5 * kAmbTol) || sh.na > kAmbCap);
  if (tid == 0) sh.use_t = !resid;

  // range weights
  if (resid && !slow) {
    const int na = sh.na;
    for (int q = tid; q < na; q += blockDim.x) sh.amb_v[q] = a.amb[(size_t)i * kAmbCap + q];
    for (int r = tid; r < NR; r += blockDim.x) sh.corr[r] = 0.0;
    __syncthreads();
    for (int q = tid; q < na; q += blockDim.x) {
      const int v = sh.amb_v[q];
      int rank = 0;
      for (int p = 0; p < na; ++p) rank += sh.amb_v[p] < v;
      sh.amb_sorted[rank] = v;
      sh.amb_w[rank] = weight<BF16>(e, v, true, St, Sd, sh.T64);
    }
    __syncthreads();
    if (tid == 0)
      for (int q = 0; q < na; ++q) sh.corr[sh.amb_sorted[q] / kRangeElems] += sh.amb_w[q];
    __syncthreads();
    for (int r = tid; r < NR; r += blockDim.x) sh.R[r] = (sh.rg[r].a / St - sh.rg[r].d / Sd) + sh.corr[r];
  } else if (resid && slow) {
    // exact weight of every token (rare: nearly identical target and draft rows)
    for (int r = 0; r < NR; ++r) {
      double s = 0.0;
      for (int v = r * kRangeElems + tid; v < min(V, (r + 1) * kRangeElems); v += blockDim.x)
        s += weight<BF16>(e, v, true, St, Sd, sh.T64);
      s = wave_sum(s);
      if (lane == 0) sh.wsum[wave] = s;
      __syncthreads();
      if (tid == 0) {
        double t = 0.0;
        for (int w = 0; w < NW; ++w) t += sh.wsum[w];
        sh.R[r] = t;
      }
      __syncthreads();
    }
  } else {
    for (int r = tid; r < NR; r += blockDim.x) sh.R[r] = sh.rg[r].t;
  }
  __syncthreads();

  for (int attempt = 0; attempt < 2; ++attempt) {
    // inclusive prefix over the ranges (wave 0, four per lane), then the first range whose
    // prefix passes u * W
    static_assert(kMaxRanges <= 4 * SPEC_WAVE, "four ranges per lane");
    if (wave == 0) {
      double v[4], t = 0.0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = lane * 4 + u;
        v[u] = (r < NR) ? sh.R[r] : 0.0;
        t += v[u];
      }
      const double incl = wave_inclusive_sum(t, lane);
      double run = incl - t;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = lane * 4 + u;
        run += v[u];
        if (r < NR) sh.R[r] = run;
      }
      const double W = __shfl(incl, 63, SPEC_WAVE);
      if (lane == 0) {
        if (resid && !sh.use_t && !(W > 0.0)) {
          sh.use_t = 2;  // no residual mass (rounding): fall back to p_t of the same row
        } else {
          sh.use_t = sh.use_t ? 1 : 0;
          sh.target = ue * W;
          sh.sel = NR;
        }
      }
    }
    __syncthreads();
    if (sh.use_t == 2) {
      for (int r = tid; r < NR; r += blockDim.x) sh.R[r] = sh.rg[r].t;
      if (tid == 0) sh.use_t = 1;
      __syncthreads();
      continue;
    }
    const double target = sh.target;
    for (int r = tid; r < NR; r += blockDim.x)
      if (sh.R[r] > target && (r == 0 || !(sh.R[r - 1] > target))) sh.sel = r;
    __syncthreads();
    if (tid == 0) {
      const int lo = sh.sel;
      sh.past = (lo >= NR);
      sh.before = (lo > 0 && lo < NR) ? sh.R[lo - 1] : 0.0;
    }
    __syncthreads();
    break;
  }
  const bool wres = resid && sh.use_t == 0;

  if (sh.past) {
    // target at or beyond the total (rounding): the last token with positive weight
    if (tid == 0) sh.token = -1;
    __syncthreads();
    for (int r = NR - 1; r >= 0; --r) {
      int best = -1;
      for (int v = r * kRangeElems + tid; v < min(V, (r + 1) * kRangeElems); v += blockDim.x)
        if (weight<BF16>(e, v, wres, St, Sd, sh.T64) > 0.0) best = v;
      best = wave_max_i(best);
      if (lane == 0) sh.wsum[wave] = (double)best;
      __syncthreads();
      if (tid == 0) {
        int b = -1;
        for (int w = 0; w < NW; ++w) b = max(b, (int)sh.wsum[w]);
        if (b >= 0) sh.token = b;
      }
      __syncthreads();
      if (sh.token >= 0) break;
    }
  } else {
    // the selected range, token by token: thread t holds tokens base + 8t .. base + 8t + 7
  static_assert(kEmitThreads * 8 == kRangeElems, "one token octet per thread");
    const bool mine = tid < kEmitThreads;
    const int base = sh.sel * kRangeElems + tid * 8;
    double w[8];
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int v = base + j;
      w[j] = (mine && v < V) ? weight<BF16>(e, v, wres, St, Sd, sh.T64) : 0.0;
      s += w[j];
    }
    const double incl = wave_inclusive_sum(s, lane);
    if (lane == 63) sh.wsum[wave] = incl;
    __syncthreads();
    double wb = 0.0;
    for (int q = 0; q < wave; ++q) wb += sh.wsum[q];
    const double P = sh.before + wb, target = sh.target;
    const double excl = incl - s;
    const bool cross = (P + incl > target);
    // first thread whose running total passes the target
    const unsigned long long m = __ballot(cross);
    if (lane == 0) sh.amb_v[wave] = m ? (int)(__ffsll((long long)m) - 1) : 64;
    const unsigned long long pos = __ballot(s > 0.0);
    if (lane == 0) sh.amb_v[NW + wave] = pos ? 63 - __clzll((long long)pos) : -1;
    __syncthreads();
    int cw = -1, cl = -1;
    constexpr int NWO = kEmitThreads / SPEC_WAVE;  // waves holding the range's octets
    for (int q = 0; q < NWO && cw < 0; ++q)
      if (sh.amb_v[q] < 64) {
        cw = q;
        cl = sh.amb_v[q];
      }
    if (cw < 0) {  // rounding left no crossing: the last thread with weight
      for (int q = NWO - 1; q >= 0 && cw < 0; --q)
        if (sh.amb_v[NW + q] >= 0) {
          cw = q;
          cl = sh.amb_v[NW + q];
        }
    }
    if (wave == cw && lane == cl) {
      double acc = P + excl;
      int tok = -1, lastpos = -1;
      for (int j = 0; j < 8; ++j) {
        if (w[j] > 0.0) lastpos = base + j;
        acc += w[j];
        if (tok < 0 && acc > target && w[j] > 0.0) tok = base + j;
      }
      sh.token = (tok >= 0) ? tok : lastpos;
    }
  }
  __syncthreads();
  if (tid == 0) a.out_tokens[(size_t)i * (G + 1) + n] = sh.token;
}

template <bool BF16>
__global__ __launch_bounds__(kEmitThreads) void emit_final_kernel(VerifyArgs a) {
  __shared__ FinalShared sh;
  const int i = a.r0 + (int)blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = a.G, V = a.V;
  init_t64(sh.T64);
  const int NR = num_ranges(V);
  const EmitReq* er = &a.ereq[i];
  if (tid < SPEC_WAVE) {
    int st, n;
    request_decision(a, i, &st, &n);
    if (tid == 0) {
      sh.st = st;
      sh.n = n;
    }
  } else if (!a.greedy_only) {
    // meanwhile the other waves fetch what the emit pass left for this request
    const int t = tid - SPEC_WAVE;
    for (int r = t; r < NR; r += kEmitThreads - SPEC_WAVE) sh.rg[r] = a.ranges[(size_t)i * NR + r];
    if (t == 0) {
      double y = 0.0;
      for (int q = 0; q < a.emit_segs; ++q) y += er->sd_part[q];
      sh.Sd = y;
      sh.na = er->amb_n;
    }
  }
  __syncthreads();
  if (tid < SPEC_WAVE && !a.greedy_only) {
    // S_t = the sum of the range totals of E_t (wave 0, four ranges per lane)
    double x = 0.0;
    for (int r = tid; r < NR; r += SPEC_WAVE) x += sh.rg[r].t;
    x = wave_sum(x);
    if (tid == 0) sh.St = x;
  }
  __syncthreads();
  finish_request<BF16>(sh, a, i, sh.st, sh.n);
}

// The acceptance test of every position of request i and its first rejection, taken by wave 0
// (lane per position) straight from the streaming kernel's segment partials: row statistics,
// r = min(1, p_t(x)/p_d(x)) with the logits at x the partials carry, the Philox uniform; top-k
// positions were finished by the streaming kernel.  Writes the row and acceptance records
// (read by the emit pass and finish_request) and sh.st / sh.n.
__device__ void decide_full(PassShared& sh, const VerifyArgs& a, int i) {
  const int lane = threadIdx.x;
  const int G = a.G, V = a.V, nseg = a.nseg;
  const int L = a.lengths ? a.lengths[i] : G;
  int st = 0;
  if (L < 0 || L > G) {
    if (lane == 0) {
      sh.st = SPEC_REQ_BAD_LENGTH;
      sh.n = 0;
    }
    return;
  }
  const float T = a.temperature[i];
  const int K0 = a.top_k ? a.top_k[i] : 0;
  if (!(T >= 0.f && T < INFINITY)) st |= SPEC_REQ_BAD_TEMPERATURE;
  if (K0 < 0) st |= SPEC_REQ_BAD_TOPK;
  const int x = (lane < L) ? a.tokens[(size_t)i * G + lane] : 0;
  if (__ballot(lane < L && (x < 0 || x >= V))) st |= SPEC_REQ_BAD_TOKEN;
  if (st == 0) st |= a.req_status[i];
  if (st) {
    if (lane == 0) {
      sh.st = st;
      sh.n = 0;
    }
    return;
  }
  const bool greedy = (T == 0.f);
  const bool topk = !greedy && K0 > 0 && K0 < V;
  const double c64 = greedy ? 0.0 : kLog2e / (double)T;
  int accept = 1, bad = 0;
  for (int k = lane; k <= L; k += SPEC_WAVE) {
    const size_t rt_i = (size_t)i * (G + 1) + k, rd_i = (size_t)i * G + k;
    const Partial* pt = a.part_t + rt_i * nseg;
    const Partial* pd = a.part_d + rt_i * nseg;
    int acc_k = 1;
    if (topk) {
      bad |= !(a.rows_t[rt_i].lse2 == a.rows_t[rt_i].lse2);
      if (k < L) acc_k = a.acc[rd_i].accept;
    } else if (greedy) {
      const int am = combine_argmax(pt, nseg);
      bad |= am < 0;
      a.rows_t[rt_i] = RowStat{0.0, -INFINITY, am < 0 ? 0 : am};
      if (k < L) {
        acc_k = (x == am);
        a.acc[rd_i] = AccRec{acc_k ? 1.0 : 0.0, acc_k, 1};
      }
    } else {
      const double l2t = combine_sum(pt, nseg);
      bad |= !(l2t == l2t);
      a.rows_t[rt_i] = RowStat{l2t, -INFINITY, 0};
      if (k < L) {
        const double l2d = combine_sum(pd, nseg);
        bad |= !(l2d == l2d);
        a.rows_d[rd_i] = RowStat{l2d, -INFINITY, 0};
        const double r = acceptance_ratio(pt[0].zx, pd[0].zx, c64, l2t, -INFINITY, l2d, -INFINITY);
        double ua, ue;
        verify_uniforms(a.seed[i], (uint64_t)i, (uint64_t)k, &ua, &ue);
        acc_k = ua < r;
        a.acc[rd_i] = AccRec{r, acc_k, 1};
      }
    }
    if (k < L) accept = acc_k;   // k < L <= 64: the lane's first round
  }
  if (__ballot(bad)) {
    if (lane == 0) {
      sh.st = SPEC_REQ_NONFINITE;
      sh.n = 0;
    }
    return;
  }
  const unsigned long long rej = __ballot(lane < L && !accept);
  if (lane == 0) {
    sh.st = 0;
    sh.n = rej ? (int)__ffsll((long long)rej) - 1 : L;
  }
}

// One 1024-thread workgroup per request does all of the request's work after the streaming:
// the acceptance decision from the segment partials, the emit pass over the whole emit row pair
// (16 waves), then finish_request from the range sums it keeps in LDS.  Used when there are
// at least as many requests as compute units.
template <bool BF16>
__global__ __launch_bounds__(kFusedThreads) void emit_fused_kernel(VerifyArgs a) {
  __shared__ PassShared ps;
  __shared__ FinalShared fs;
  const int i = a.r0 + (int)blockIdx.x;
  const int tid = threadIdx.x;
  const int NR = num_ranges(a.V);
  init_t64(ps.T64);
  init_t64(fs.T64);
  if (tid < SPEC_WAVE) decide_full(ps, a, i);
  __syncthreads();
  const int st = ps.st, n = ps.n;
  if (!st && !a.greedy_only && a.temperature[i] != 0.f) {
    run_pass<BF16>(ps, a, i, 0, n, fs.rg);
    if (tid < SPEC_WAVE) {
      double x = 0.0;
      for (int r = tid; r < NR; r += SPEC_WAVE) x += fs.rg[r].t;
      x = wave_sum(x);
      if (tid == 0) {
        double y = 0.0;
        for (int w = 0; w < kFusedThreads / SPEC_WAVE; ++w) y += ps.red[1][w];
        fs.St = x;
        fs.Sd = y;
        fs.na = atomicAdd(&a.ereq[i].amb_n, 0);   // read at L2, where the pass counted
      }
    }
    __syncthreads();
  }
  finish_request<BF16>(fs, a, i, st, n);
}

void launch_emit(const VerifyArgs& a, int bf16, hipStream_t s) {
  const unsigned nreq = (unsigned)(a.r1 - a.r0);
  if (nreq == 0) return;
  if (!a.greedy_only && a.emit_segs == 1) {
    if (bf16)
      hipLaunchKernelGGL(emit_fused_kernel<true>, dim3(nreq), dim3(kFusedThreads), 0, s, a);
    else
      hipLaunchKernelGGL(emit_fused_kernel<false>, dim3(nreq), dim3(kFusedThreads), 0, s, a);
    return;
  }
  if (!a.greedy_only) {
    const dim3 grid(nreq * (unsigned)a.emit_segs);
    if (bf16)
      hipLaunchKernelGGL(emit_pass_kernel<true>, grid, dim3(kPassThreads), 0, s, a);
    else
      hipLaunchKernelGGL(emit_pass_kernel<false>, grid, dim3(kPassThreads), 0, s, a);
  }
  if (bf16)
    hipLaunchKernelGGL(emit_final_kernel<true>, dim3(nreq), dim3(kEmitThreads), 0, s, a);
  else
    hipLaunchKernelGGL(emit_final_kernel<false>, dim3(nreq), dim3(kEmitThreads), 0, s, a);
}

}  // namespace spec
