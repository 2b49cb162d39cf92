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
// emit_fused_kernel  one 1024-thread workgroup per request (batches that
//   give every CU a request): the acceptance decision from the streaming
//   kernel's segment partials, the pass and the finish above, in one kernel.
// ltr_walk_kernel  between the two streaming passes of a left-to-right call:
//   each request's walk over the first pass's positions (DSpark paper §2.1:
//   the first rejection discards every later draft), so that the second
//   pass streams only the positions the walk can still reach.
#include "common.hpp"
#include "philox.hpp"
#include "verify_impl.hpp"
#include "qtable.hpp"

#include <float.h>
#include <math.h>

namespace spec {

// Relative margin of the residual-sign classification with the streaming normalisers.  Their ratio
// rho = cd * S_d / S_t is checked to lie within half of it (measured |rho - 1| <= 2.3e-7 on the
// verification workloads); a wider margin records more tokens for the exact second look.
constexpr double kAmbTol = 2e-6;
constexpr int kSub = 512;                               // tokens per wave step (64 lanes x 8)
constexpr int kSubPerRange = kRangeElems / kSub;        // 4

struct EmitRows {
  int V;
  const char* t;
  const char* d;  // nullptr: single target row (appended / fresh token)
  double invT, R;
  float tht, thd;
  double cd;      // exp(R_t - R_d): p_d ~ cd * Q(z_d) with the approximate normalisers
  int* amb_n;     // uncertain-sign tokens: count and list (global memory, or LDS in the fused kernel)
  int* amb_v;
  const double* Qt;  // the Q table when it holds this row's values (bf16 rows without top-k), else null
};

// The emit row(s) of request i at position n from the row records of target row n and, when
// n < L, draft row n.
template <bool BF16>
__device__ __forceinline__ EmitRows emit_rows_from(const VerifyArgs& a, int i, int n, int L, float T,
                                                   const RowStat& rt, const RowStat& rd) {
  constexpr int ES = BF16 ? 2 : 4;
  EmitRows e;
  e.V = a.V;
  e.t = target_row<ES>(a, i, n);
  e.R = rt.lse2 * kLn2;
  e.tht = rt.theta;
  e.invT = 1.0 / (double)T;
  e.d = nullptr;
  e.thd = -INFINITY;
  e.cd = 1.0;
  if (n < L) {
    e.d = draft_row<ES>(a, i, n);
    e.thd = rd.theta;
    e.cd = exp(e.R - rd.lse2 * kLn2);
  }
  e.amb_n = &a.ereq[i].amb_n;
  e.amb_v = a.amb + (size_t)i * kAmbCap;
  e.Qt = nullptr;
  return e;
}

template <bool BF16>
__device__ __forceinline__ EmitRows emit_rows(const VerifyArgs& a, int i, int n) {
  const int G = a.G;
  const int L = a.lengths ? a.lengths[i] : G;
  const RowStat rt = a.rows_t[(size_t)i * (G + 1) + n];
  const RowStat rd = (n < L) ? a.rows_d[(size_t)i * G + n] : RowStat{0.0, -INFINITY, 0};
  return emit_rows_from<BF16>(a, i, n, L, a.temperature[i], rt, rd);
}

// Q of token v of a row (any dtype, any alignment), kept-set aware; from the table Qt when given
// and the value is tabulated (the same bits as the direct evaluation).
template <bool BF16>
__device__ __forceinline__ double q_at(const char* row, int v, float th, double invT, double R, const double* T64,
                                       const double* Qt) {
  if constexpr (BF16) {
    const uint32_t b = reinterpret_cast<const uint16_t*>(row)[v];
    const float z = __uint_as_float(b << 16);
    if (!(z >= th)) return 0.0;
    if (Qt) {
      const uint32_t k = q_slot1(b);
      if (k < (uint32_t)kQsize) return Qt[k];
    }
    return q_direct(z, invT, R, T64);
  } else {
    const float z = load_elem<false>(row, v);
    return (z >= th) ? q_direct(z, invT, R, T64) : 0.0;
  }
}

// Per-lane accumulators for one range.
struct Acc {
  double sd;       // running total of E_d over everything this lane saw
  double A, D, T;  // this range
};

// Whether the residual sign of a token pair is uncertain: not clearly positive, yet p_t is above
// p_d less the margin, with the approximate normalisers.  A pair with p_t = p_d = 0 is not (its
// residual is 0), nor one exactly at the lower margin, whose residual is negative since the
// normalisers are checked to be within half the margin.  Such tokens are weighed exactly later.
__device__ __forceinline__ bool uncertain(double qt, double qd, double cdh, double cdl) {
  return !(qt > cdh * qd) && qt > cdl * qd;
}

// Accumulate one token pair; returns uncertain(qt, qd, ...).  No branches, so the table reads
// of a whole step can be in flight together.
__device__ __forceinline__ bool classify(Acc& c, double qt, double qd, double cdh, double cdl) {
  c.sd += qd;
  c.T += qt;
  const bool pos = qt > cdh * qd;
  // fma(1, q, s) = s + q and fma(0, q, s) = s, rounded as the plain sums (q is finite here, or
  // the normaliser check sends the request to the exact path): one select instead of four
  const double one = pos ? 1.0 : 0.0;
  c.A = fma(one, qt, c.A);
  c.D = fma(one, qd, c.D);
  return !pos && qt > cdl * qd;
}

// Record token v as uncertain (rare).
__device__ __forceinline__ void record_uncertain(const EmitRows& e, int v) {
  const int slot = atomicAdd(e.amb_n, 1);
  if (slot < kAmbCap) e.amb_v[slot] = v;
}

constexpr int kMaxWaves = 1024 / SPEC_WAVE;  // largest emit workgroup, in waves

struct PassShared {
  double T64[64];
  double Qt[kQsize];
  double red[2][kMaxWaves];
  int st, n;
};

// The fused kernel's decision: the request's segment partials (target rows, then draft rows), per
// draft position the row records, acceptance uniforms and ratios and draft tokens, the offset of
// the table built meanwhile, and the list of uncertain-sign tokens of the pass.
struct DecideShared {
  Partial stage[2 * (SPEC_MAX_GAMMA + 1) * kMaxStreamSegs];
  RowStat rt[SPEC_MAX_GAMMA + 1], rd[SPEC_MAX_GAMMA];
  double accr[SPEC_MAX_GAMMA];
  double ua[SPEC_MAX_GAMMA];
  int tacc[SPEC_MAX_GAMMA];
  int x[SPEC_MAX_GAMMA];
  int st, n, L, greedy, bad_t, bad_d;
  unsigned long long badm_t, badm_d;   // positions 0 .. 63 whose target / draft row is bad
  double R0;
  int table_ok;
  int amb_cnt;
  int amb_list[kAmbCap];
};

// One step (64 lanes x 8 tokens) of a bf16 row pair from registers.  A lane whose 16 tokens
// are all tabulated reads Q from the table; otherwise (rare: |z| < 2^-20, |z| >= 128,
// infinities) it evaluates the same formula directly for the whole step.  MASK: the step of a
// row's last, partial range, where a lane past the row's end (live = false) holds tabulated
// filler bits and adds nothing.  Uncertain tokens are rare: the table path only notes that the
// lane saw one and then finds and records it in a second look at its 8 tokens.
template <bool RESID, bool MASK = false>
__device__ __forceinline__ void step_bf16(Acc& c, const uint4& dt, const uint4& dd, const EmitRows& e,
                                          double cdh, double cdl, int v0, const double* T64, const double* Qt,
                                          bool live = true) {
  constexpr bool resid = RESID;
  uint32_t wt[4] = {dt.x, dt.y, dt.z, dt.w};
  uint32_t wd[4] = {dd.x, dd.y, dd.z, dd.w};
  if (MASK && !live) {
#pragma unroll
    for (int q = 0; q < 4; ++q) wt[q] = wd[q] = kFill2;
  }
  us2 kt[4], kd[4];
  us2 kmax = (us2)(unsigned short)0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    kt[q] = q_slots(wt[q]);
    kmax = __builtin_elementwise_max(kmax, kt[q]);
    if (resid) {
      kd[q] = q_slots(wd[q]);
      kmax = __builtin_elementwise_max(kmax, kd[q]);
    }
  }
  const bool miss = max((uint32_t)kmax.x, (uint32_t)kmax.y) >= (uint32_t)kQsize;
  if (!miss) {
    bool any = false;
    // two halves of four tokens: eight table reads in flight, registers kept in check
#pragma unroll
    for (int h = 0; h < 8; h += 4) {
      double qt[4], qd[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qt[j] = Qt[slot_of(kt, h + j)];
        qd[j] = resid ? Qt[slot_of(kd, h + j)] : 0.0;
        if (MASK && !live) qt[j] = qd[j] = 0.0;   // filler bits: tabulated, and worth nothing
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (resid) any |= classify(c, qt[j], qd[j], cdh, cdl);
        else c.T += qt[j];
      }
    }
    if (resid && any) {
      // the slots again from the loaded words (kept, unlike the slots, until the next refill)
#pragma unroll 1
      for (int j = 0; j < 8; ++j) {
        const us2 st = q_slots(wt[j >> 1]), sd = q_slots(wd[j >> 1]);
        const uint32_t it = (j & 1) ? st.y : st.x, id = (j & 1) ? sd.y : sd.x;
        if (uncertain(Qt[it], Qt[id], cdh, cdl)) record_uncertain(e, v0 + j);
      }
    }
  } else {
#pragma unroll 1
    for (int j = 0; j < 8; ++j) {
      const double qt = q_direct(__uint_as_float(half16(wt, j) << 16), e.invT, e.R, T64);
      if (resid) {
        const double qd = q_direct(__uint_as_float(half16(wd, j) << 16), e.invT, e.R, T64);
        if (classify(c, qt, qd, cdh, cdl)) record_uncertain(e, v0 + j);
      } else {
        c.T += qt;
      }
    }
  }
}

// The 16-byte vector path of a bf16 row pair (rows 16-byte aligned, V a multiple of 8): the wave's
// ranges r, r + NWT, ... below NRv, the four steps of a range in flight at once.  Each register
// slot is refilled with the same step of the wave's next range as soon as it has been consumed,
// unconditionally inside the loop (the loop runs over ranges that have a successor; the wave's last
// range is taken after it): loads under a condition would leave the compiler unsure of the order
// of the loads in flight, and it would then wait for all of them before every step.  The row's
// last, partial range (lanes past the end load a clamped address and are masked) is only ever a
// wave's last.  The Q table is built (unless table_ready) while the first loads are in flight;
// r is advanced past the ranges done.
template <bool RESID>
__device__ __forceinline__ void vec_ranges(PassShared& sh, const EmitRows& e, Acc& c, double cdh, double cdl,
                                           EmitRange* out, int& r, int NRv, int NRfull, int NWT,
                                           bool table_ready) {
  const int lane = threadIdx.x & 63;
  uint4 bt[kSubPerRange], bd[kSubPerRange];
  const int Vt = e.V;
  auto load = [&](int rr, int sub, uint4& t, uint4& d) {
    const int v0 = min(rr * kRangeElems + sub * kSub + lane * 8, Vt - 8);
    const size_t off = (size_t)v0 * 2;
    t = *reinterpret_cast<const uint4*>(e.t + off);
    if constexpr (RESID) d = *reinterpret_cast<const uint4*>(e.d + off);
    else d = make_uint4(0, 0, 0, 0);
  };
  const bool any = r < NRv;
  const int r0 = any ? r : 0;   // a wave without a range loads range 0 and leaves it unused
  if (NRv > 0) {
#pragma unroll
    for (int sub = 0; sub < kSubPerRange; ++sub) load(r0, sub, bt[sub], bd[sub]);
  }
  if (!table_ready) build_qtab(sh.Qt, e.invT, e.R, sh.T64);
  lds_barrier();   // the table; the loads stay in flight
  auto finish = [&](int rr) {
    const double A = wave_sum(c.A), D = wave_sum(c.D), T = wave_sum(c.T);
    if (lane == 0) out[rr] = EmitRange{A, D, T};
  };
  for (; r + NWT < NRv; r += NWT) {   // a full range with a successor
    const int rn = r + NWT;
    c.A = c.D = c.T = 0.0;
#pragma unroll
    for (int sub = 0; sub < kSubPerRange; ++sub) {
      const int v0 = r * kRangeElems + sub * kSub + lane * 8;
      step_bf16<RESID>(c, bt[sub], bd[sub], e, cdh, cdl, v0, sh.T64, sh.Qt);
      load(rn, sub, bt[sub], bd[sub]);
    }
    finish(r);
  }
  if (r < NRv) {   // the wave's last range
    c.A = c.D = c.T = 0.0;
    if (r < NRfull) {
#pragma unroll
      for (int sub = 0; sub < kSubPerRange; ++sub) {
        const int v0 = r * kRangeElems + sub * kSub + lane * 8;
        step_bf16<RESID>(c, bt[sub], bd[sub], e, cdh, cdl, v0, sh.T64, sh.Qt);
      }
    } else {
#pragma unroll
      for (int sub = 0; sub < kSubPerRange; ++sub) {
        const int vs = r * kRangeElems + sub * kSub, v0 = vs + lane * 8;
        if (vs >= Vt) break;
        step_bf16<RESID, true>(c, bt[sub], bd[sub], e, cdh, cdl, v0, sh.T64, sh.Qt, v0 < Vt);
      }
    }
    finish(r);
    r += NWT;
  }
}

// The ranges of request i that segment `seg` owns, each written as an EmitRange to out[r]
// (global memory, or LDS when the same workgroup finishes the request); each wave's sum of
// E_d goes to sh.red[1][wave].  bf16 rows without top-k build the Q table in sh.Qt here unless
// table_ready (the whole workgroup calls this function).
template <bool BF16, bool TOPK>
__device__ __forceinline__ void pass_ranges(PassShared& sh, const VerifyArgs& a, int i, int seg, const EmitRows& e,
                            EmitRange* out, bool table_ready) {
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
    const int NRv = (aligned && (V & 7) == 0 && V >= 8) ? NR : NRfull;
    if (resid) vec_ranges<true>(sh, e, c, cdh, cdl, out, r, NRv, NRfull, NWT, table_ready);
    else vec_ranges<false>(sh, e, c, cdh, cdl, out, r, NRv, NRfull, NWT, table_ready);
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
              if (classify(c, qt, qd, cdh, cdl)) record_uncertain(e, v);
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
__device__ __forceinline__ void run_pass(PassShared& sh, const VerifyArgs& a, int i, int seg, const EmitRows& e, EmitRange* out,
                         int K, bool table_ready = false) {
  if (K > 0 && K < a.V) pass_ranges<BF16, true>(sh, a, i, seg, e, out, false);
  else pass_ranges<BF16, false>(sh, a, i, seg, e, out, table_ready);
  __syncthreads();
}

// ---- top-k requests whose kept tokens are all in their segment lists ----

struct TopkEmitShared {
  int32_t id[2][kTopkEmitKept];   // the kept entries of target row n and draft row n: token ids
  float z[2][kTopkEmitKept];      //   and raw logits
  double w[kTopkEmitKept];        // the target's kept tokens' weights in ascending token order
  int32_t sorted[kTopkEmitKept];  //   and their ids
  int nk[2];
  double sd;                      // S_d
  int token;
};

// Whether request i's emit at position n can draw from the segment lists: a sampling request with
// 0 < K < V whose target row n (and draft row n after a rejection) had its kept tokens listed with
// their logits, at most kTopkEmitKept of them (RowStat's third field; set only by the merge of
// segmented top-k rows).
__device__ __forceinline__ bool topk_lists_complete(const VerifyArgs& a, int i, int n, int L, float T, int K,
                                                    const RowStat& rt, const RowStat& rd) {
  return T > 0.f && K > 0 && K < a.V && rt.argmax == 1 && (n >= L || rd.argmax == 1);
}

// The emitted token of top-k request i at position n from the segment lists: the kept entries (listed
// values at or above the row's threshold) of target row n and, after a rejection, draft row n;
// Q = exp(z / T - R) in fp64 (R the target row's log-normaliser); S_t, S_d the kept Q sums; weights
// w = max(0, Q_t / S_t - Q_d / S_d) after a rejection (Q_d = 0 outside the draft's kept set),
// w = Q_t for the appended token; the token is the first in ascending token order whose running sum
// of w passes u * W (u the emit uniform of position n), or the last with w > 0 when rounding leaves
// no crossing.  With W <= 0 after a rejection, w = Q_t (as the row-based path).  These are the weights
// the row-based path gives every token (zero outside the target's kept set), so the draw is the same.
// Wave 0 gathers the target's entries, wave 1 the draft's (and S_d); wave 0 then ranks the target's
// by token id, joins the draft's logits and walks the weights.  Called by a whole workgroup of at
// least two waves; every thread gets the token.
template <bool BF16>
__device__ __forceinline__ int emit_topk_lists(TopkEmitShared& sh, const VerifyArgs& a, int i, int n, int L,
                                               float T, const RowStat& rt, const RowStat& rd, const double* T64) {
  constexpr int J = kTopkEmitKept / SPEC_WAVE;
  static_assert(kTopkSegCap <= 2 * SPEC_WAVE, "two list entries per lane");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const bool resid = n < L;
  const double invT = 1.0 / (double)T, R = rt.lse2 * kLn2;
  if (wave < (resid ? 2 : 1)) {
    // row `wave`'s kept entries, compacted in list order
    const size_t slot = topk_slot(a.G, i, n, wave);
    const float th = wave ? rd.theta : rt.theta;
    const int nsk = a.nseg_topk;
    const int ns = (lane < nsk) ? a.tk_seg[slot + lane].n : 0;
    float zl[kTopkSegs][2];
    int il[kTopkSegs][2];
#pragma unroll
    for (int s = 0; s < kTopkSegs; ++s) {
      const int nss = read_lane(ns, s);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = lane + h * SPEC_WAVE;
        const bool on = s < nsk && q < nss;
        zl[s][h] = on ? a.tk_val[(slot + s) * kTopkSegCap + q] : -INFINITY;
        il[s][h] = on ? a.tk_ids[(slot + s) * kTopkSegCap + q] : -1;
      }
    }
    int m = 0;
    double sd = 0.0;
#pragma unroll
    for (int s = 0; s < kTopkSegs; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bool keep = il[s][h] >= 0 && zl[s][h] >= th;
        const unsigned long long mk = __ballot(keep);
        const int q = m + (int)__popcll(mk & below);
        if (keep && q < kTopkEmitKept) {
          sh.id[wave][q] = il[s][h];
          sh.z[wave][q] = zl[s][h];
        }
        if (keep && wave == 1) sd += q_direct(zl[s][h], invT, R, T64);
        m += (int)__popcll(mk);
      }
    if (wave == 1) sd = wave_sum(sd);   // a fixed lane per entry: the same sum run after run
    if (lane == 0) {
      sh.nk[wave] = m;
      if (wave == 1) sh.sd = sd;
    }
  }
  __syncthreads();
  if (wave == 0) {
    const int nkt = sh.nk[0], nkd = resid ? sh.nk[1] : 0;
    // entry lane + 64 j of each row in registers
    int it[J], id[J];
    float zt[J], zd[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = lane + j * SPEC_WAVE;
      it[j] = (q < nkt) ? sh.id[0][q] : 0x7fffffff;
      zt[j] = (q < nkt) ? sh.z[0][q] : -INFINITY;
      id[j] = (q < nkd) ? sh.id[1][q] : -1;
      zd[j] = (q < nkd) ? sh.z[1][q] : -INFINITY;
    }
    // rank of each target entry among the target's (ids are distinct) and its draft logit, if the
    // draft kept the token (else -inf: Q_d = 0)
    int rank[J];
    float zj[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      rank[j] = 0;
      zj[j] = -INFINITY;
    }
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      if (jj * SPEC_WAVE >= max(nkt, nkd)) break;
      for (int src = 0; src < SPEC_WAVE; ++src) {
        const int ot = read_lane(it[jj], src), od = read_lane(id[jj], src);
        const float oz = read_lane(zd[jj], src);
#pragma unroll
        for (int j = 0; j < J; ++j) {
          rank[j] += ot < it[j];
          if (od == it[j]) zj[j] = oz;
        }
      }
    }
    double qt[J], st = 0.0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      qt[j] = (lane + j * SPEC_WAVE < nkt) ? q_direct(zt[j], invT, R, T64) : 0.0;
      st += qt[j];
    }
    st = wave_sum(st);
    const double iSt = 1.0 / st, iSd = resid ? 1.0 / sh.sd : 0.0;
    double tot = 0.0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const double qd = (resid && zj[j] > -INFINITY) ? q_direct(zj[j], invT, R, T64) : 0.0;
      const double w = resid ? fmax(0.0, qt[j] * iSt - qd * iSd) : qt[j];
      tot += w;
      if (lane + j * SPEC_WAVE < nkt) {
        sh.w[rank[j]] = w;
        sh.sorted[rank[j]] = it[j];
      }
    }
    // no residual mass (rounding): p_t of the same row
    const bool plain = resid && !(wave_sum(tot) > 0.0);
    if (plain) {
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (lane + j * SPEC_WAVE < nkt) sh.w[rank[j]] = qt[j];
    }
  }
  __syncthreads();
  if (wave == 0) {
    // lane l walks ranks l * JJ .. l * JJ + JJ - 1
    const int nkt = sh.nk[0];
    const int JJ = (nkt + SPEC_WAVE - 1) / SPEC_WAVE;
    double w[J], tot = 0.0;
    int vid[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int r = lane * JJ + j;
      const bool on = j < JJ && r < nkt;
      w[j] = on ? sh.w[r] : 0.0;
      vid[j] = on ? sh.sorted[r] : -1;
      tot += w[j];
    }
    const double W = wave_sum(tot);
    double ua, ue;
    verify_uniforms(a.seed[i], (uint64_t)i, (uint64_t)n, &ua, &ue);
    const double target = ue * W;
    double run = wave_inclusive_sum(tot, lane) - tot;
    int cross = -1, lastpos = -1;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (w[j] > 0.0) lastpos = vid[j];
      run += w[j];
      if (cross < 0 && w[j] > 0.0 && run > target) cross = vid[j];
    }
    const unsigned long long mc = __ballot(cross >= 0), mp = __ballot(lastpos >= 0);
    int tok;
    if (mc) tok = read_lane(cross, (int)__ffsll((long long)mc) - 1);
    else tok = mp ? read_lane(lastpos, 63 - __clzll((long long)mp)) : -1;
    if (lane == 0) sh.token = tok;
  }
  __syncthreads();
  return sh.token;
}

template <bool BF16>
__global__ __launch_bounds__(kPassThreads, 4) void emit_pass_kernel(VerifyArgs a) {
  __shared__ PassShared sh;
  const int i = a.r0 + (int)blockIdx.x / a.emit_segs, seg = (int)blockIdx.x % a.emit_segs;
  init_t64(sh.T64);
  decide_into(sh, a, i);
  const int st = sh.st, n = sh.n;
  if (st || a.temperature[i] == 0.f) return;
  {
    const int L = a.lengths ? a.lengths[i] : a.G;
    const int K = a.top_k ? a.top_k[i] : 0;
    const RowStat rt = a.rows_t[(size_t)i * (a.G + 1) + n];
    const RowStat rd = (n < L) ? a.rows_d[(size_t)i * a.G + n] : RowStat{0.0, -INFINITY, 0};
    if (topk_lists_complete(a, i, n, L, a.temperature[i], K, rt, rd)) return;   // drawn from the lists
  }
  run_pass<BF16>(sh, a, i, seg, emit_rows<BF16>(a, i, n), a.ranges + (size_t)i * num_ranges(a.V),
                 a.top_k ? a.top_k[i] : 0);
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
  int cross_lane[kMaxWaves], last_lane[kMaxWaves];
  double amb_w[kAmbCap];
  int amb_v[kAmbCap];
  int amb_sorted[kAmbCap];
  int st, n, slow, use_t, sel, past, token;
  double St, Sd, target, before;
};

// Exact weight of token v: residual (resid) or Q(z_t) (target row, any scale).  iSt and iSd are
// the reciprocals of the row sums S_t and S_d: p = Q * (1/S) to one rounding more than Q / S,
// far below the precision the draw needs (range weights and the token walk use the same form).
template <bool BF16>
__device__ __forceinline__ double weight(const EmitRows& e, int v, bool resid, double iSt, double iSd,
                                         const double* T64) {
  const double qt = q_at<BF16>(e.t, v, e.tht, e.invT, e.R, T64, e.Qt);
  if (!resid) return qt;
  const double qd = q_at<BF16>(e.d, v, e.thd, e.invT, e.R, T64, e.Qt);
  return fmax(0.0, qt * iSt - qd * iSd);
}

template <bool BF16, int NT>
__device__ __forceinline__ void sample_emit(FinalShared& sh, const VerifyArgs& a, int i, int n, const EmitRows& e);

// Everything after request i's decision (st, n): status and outputs, then, for a sampling
// request, the emitted token (sample_emit).
template <bool BF16>
__device__ __forceinline__ void finish_request(FinalShared& sh, TopkEmitShared& tes, const VerifyArgs& a, int i, int st, int n) {
  const int tid = threadIdx.x;
  const int G = a.G;
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
  {
    const int K = a.top_k ? a.top_k[i] : 0;
    const RowStat rt = a.rows_t[(size_t)i * (G + 1) + n];
    const RowStat rd = (n < L) ? a.rows_d[(size_t)i * G + n] : RowStat{0.0, -INFINITY, 0};
    if (topk_lists_complete(a, i, n, L, a.temperature[i], K, rt, rd)) {
      const int tok = emit_topk_lists<BF16>(tes, a, i, n, L, a.temperature[i], rt, rd, sh.T64);
      if (tid == 0) a.out_tokens[(size_t)i * (G + 1) + n] = tok;
      return;
    }
  }
  sample_emit<BF16, kEmitThreads>(sh, a, i, n, emit_rows<BF16>(a, i, n));
}

// The emitted token of sampling request i at position n (rows e), from the emit pass's range sums
// (sh.rg, sh.St, sh.Sd, sh.na filled; the uncertain-sign tokens listed at e.amb_v), written to
// out_tokens.  Called by a block of NT threads; each holds kRangeElems / NT consecutive tokens
// of the range where the draw lands.
template <bool BF16, int NT>
__device__ __forceinline__ void sample_emit(FinalShared& sh, const VerifyArgs& a, int i, int n, const EmitRows& e) {
  constexpr int TPT = kRangeElems / NT;
  constexpr int NW = NT / SPEC_WAVE;
  static_assert(TPT * NT == kRangeElems && NW * SPEC_WAVE == NT && NW <= kMaxWaves, "block shape");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = a.G, V = a.V;
  const int NR = num_ranges(V);
  const bool resid = (e.d != nullptr);
  double ua, ue;
  verify_uniforms(a.seed[i], (uint64_t)i, (uint64_t)n, &ua, &ue);
  const double St = sh.St, Sd = sh.Sd;
  const double iSt = 1.0 / St, iSd = 1.0 / Sd;
  // the sign classification assumed cd * S_d / S_t = 1 to within half its margin
  const double rho = resid ? e.cd * Sd / St : 1.0;
  const bool slow = resid && (!(fabs(rho - 1.0) <= 0.5 * kAmbTol) || sh.na > kAmbCap);

  // range weights
  if (resid && !slow) {
    const int na = sh.na;
    for (int q = tid; q < na; q += NT) sh.amb_v[q] = e.amb_v[q];
    for (int r = tid; r < NR; r += NT) sh.corr[r] = 0.0;
    __syncthreads();
    for (int q = tid; q < na; q += NT) {
      // rank by token id (the tokens are distinct): eight comparisons per step, reads in flight
      const int v = sh.amb_v[q];
      int rank = 0;
      for (int p = 0; p < na; p += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) rank += (p + u < na) && sh.amb_v[min(p + u, na - 1)] < v;
      }
      sh.amb_sorted[rank] = v;
      sh.amb_w[rank] = weight<BF16>(e, v, true, iSt, iSd, sh.T64);
    }
    __syncthreads();
    // each range's corrections summed in token order by the first of its tokens
    for (int q = tid; q < na; q += NT) {
      const int r = sh.amb_sorted[q] / kRangeElems;
      if (q == 0 || sh.amb_sorted[q - 1] / kRangeElems != r) {
        double x = 0.0;
        for (int p = q; p < na && sh.amb_sorted[p] / kRangeElems == r; ++p) x += sh.amb_w[p];
        sh.corr[r] = x;
      }
    }
    __syncthreads();
    for (int r = tid; r < NR; r += NT) sh.R[r] = (sh.rg[r].a * iSt - sh.rg[r].d * iSd) + sh.corr[r];
  } else if (resid && slow) {
    // exact weight of every token (rare: nearly identical target and draft rows)
    for (int r = 0; r < NR; ++r) {
      double x = 0.0;
      for (int v = r * kRangeElems + tid; v < min(V, (r + 1) * kRangeElems); v += NT)
        x += weight<BF16>(e, v, true, iSt, iSd, sh.T64);
      x = wave_sum(x);
      if (lane == 0) sh.wsum[wave] = x;
      __syncthreads();
      if (tid == 0) {
        double t = 0.0;
        for (int w = 0; w < NW; ++w) t += sh.wsum[w];
        sh.R[r] = t;
      }
      __syncthreads();
    }
  } else {
    for (int r = tid; r < NR; r += NT) sh.R[r] = sh.rg[r].t;
  }
  __syncthreads();

  // wave 0: inclusive prefix over the ranges (four per lane), the total W, the target u * W and
  // the first range whose prefix passes it; the whole block then waits once
  static_assert(kMaxRanges <= 4 * SPEC_WAVE, "four ranges per lane");
  if (wave == 0) {
    int use_t = !resid;
    for (int attempt = 0; attempt < 2; ++attempt) {
      double v[4], pre[4], t = 0.0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = lane * 4 + u;
        v[u] = (r < NR) ? (attempt ? sh.rg[r].t : sh.R[r]) : 0.0;
        t += v[u];
      }
      const double incl = wave_inclusive_sum(t, lane);
      double run = incl - t;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        run += v[u];
        pre[u] = run;
      }
      const double W = read_lane(incl, 63);
      if (attempt == 0 && !use_t && !(W > 0.0)) {
        use_t = 1;   // no residual mass (rounding): fall back to p_t of the same row
        continue;
      }
      const double target = ue * W;
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
        sh.use_t = use_t;
        sh.target = target;
        sh.sel = sel;
        sh.past = (sel >= NR);
        sh.before = before;
      }
      break;
    }
  }
  __syncthreads();
  const bool wres = resid && sh.use_t == 0;

  if (sh.past) {
    // target at or beyond the total (rounding): the last token with positive weight
    if (tid == 0) sh.token = -1;
    __syncthreads();
    for (int r = NR - 1; r >= 0; --r) {
      int best = -1;
      for (int v = r * kRangeElems + tid; v < min(V, (r + 1) * kRangeElems); v += NT)
        if (weight<BF16>(e, v, wres, iSt, iSd, sh.T64) > 0.0) best = v;
      best = wave_max_i(best);
      if (lane == 0) sh.last_lane[wave] = best;
      __syncthreads();
      if (tid == 0) {
        int b = -1;
        for (int w = 0; w < NW; ++w) b = max(b, sh.last_lane[w]);
        if (b >= 0) sh.token = b;
      }
      __syncthreads();
      if (sh.token >= 0) break;
    }
  } else {
    // the selected range, token by token: thread t holds tokens base + TPT t .. + TPT - 1
    const int base = sh.sel * kRangeElems + tid * TPT;
    double w[TPT];
    double x = 0.0;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int v = base + j;
      w[j] = (v < V) ? weight<BF16>(e, v, wres, iSt, iSd, sh.T64) : 0.0;
      x += w[j];
    }
    const double incl = wave_inclusive_sum(x, lane);
    if (lane == 63) sh.wsum[wave] = incl;
    __syncthreads();
    double wb = 0.0;   // the earlier waves' totals, in wave order (reads issued together)
#pragma unroll
    for (int q = 0; q < NW; ++q) wb += (q < wave) ? sh.wsum[q] : 0.0;
    const double P = sh.before + wb, target = sh.target;
    const double excl = incl - x;
    // first thread whose running total passes the target; the last thread with weight
    const unsigned long long m = __ballot(P + incl > target);
    const unsigned long long pos = __ballot(x > 0.0);
    if (lane == 0) {
      sh.cross_lane[wave] = m ? (int)(__ffsll((long long)m) - 1) : 64;
      sh.last_lane[wave] = pos ? 63 - __clzll((long long)pos) : -1;
    }
    __syncthreads();
    // the first wave with a crossing, else the last wave with weight (all records read at once)
    int cw = -1, cl = -1, lw = -1, ll = -1;
#pragma unroll
    for (int q = NW - 1; q >= 0; --q) {
      const int c = sh.cross_lane[q], l = sh.last_lane[q];
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
    if (wave == cw && lane == cl) {
      double acc = P + excl;
      int tok = -1, lastpos = -1;
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
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
  __shared__ TopkEmitShared tes;
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
  finish_request<BF16>(sh, tes, a, i, sh.st, sh.n);
}

// What the fused decision of request i reads besides the segment partials: loaded by wave 0 before
// the partials are staged, so that every load of the decision is in flight at once.
struct DecideIn {
  uint64_t seed;
  int L, K0, rs, x;
  int P;   // positions whose rows were streamed (left-to-right calls; else every position)
  float T;
};

__device__ __forceinline__ DecideIn decide_loads(const VerifyArgs& a, int i) {
  const int lane = threadIdx.x & 63;
  DecideIn d;
  d.seed = a.seed[i];
  d.L = a.lengths ? a.lengths[i] : a.G;
  d.T = a.temperature[i];
  d.K0 = a.top_k ? a.top_k[i] : 0;
  d.rs = a.req_status[i];
  d.x = (lane < a.G) ? a.tokens[(size_t)i * a.G + lane] : 0;
  d.P = a.ltr ? a.npos[i] : a.G + 1;
  return d;
}

// The segment partials of every row of request i (target rows, then draft rows; those of rows
// past L are read but not used) copied to sh.stage by the whole workgroup.
__device__ __forceinline__ void stage_partials(DecideShared& sh, const VerifyArgs& a, int i) {
  const int per = (a.G + 1) * a.nseg;
  const Partial* gt = a.part_t + (size_t)i * per;
  const Partial* gd = a.part_d + (size_t)i * per;
  for (int q = threadIdx.x; q < 2 * per; q += blockDim.x) sh.stage[q] = (q < per) ? gt[q] : gd[q - per];
}

// Status of request i from its arguments (every lane of a wave gets it; 0 when well formed).
__device__ __forceinline__ int decide_status(const VerifyArgs& a, const DecideIn& in) {
  const int lane = threadIdx.x & 63;
  const int L = in.L;
  if (L < 0 || L > a.G) return SPEC_REQ_BAD_LENGTH;
  int st = 0;
  if (!(in.T >= 0.f && in.T < INFINITY)) st |= SPEC_REQ_BAD_TEMPERATURE;
  if (in.K0 < 0) st |= SPEC_REQ_BAD_TOPK;
  if (__ballot(lane < L && (in.x < 0 || in.x >= a.V))) st |= SPEC_REQ_BAD_TOKEN;
  if (st == 0) st |= in.rs;
  return st;
}

// First half of the fused decision of request i, three waves at once (lane per position), from
// the staged segment partials:
//   wave 0: target row statistics of positions k <= L (log2-sum-exp, or the argmax for the
//           greedy rule; top-k rows were finished by the streaming or merging kernel),
//   wave 1: draft row statistics of positions k < L (top-k: the streaming kernel's test),
//   wave 2: the acceptance uniforms of positions k < L (sampling rows without top-k).
__device__ __forceinline__ void decide_stats(DecideShared& sh, const VerifyArgs& a, int i, const DecideIn& in) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int G = a.G, V = a.V, nseg = a.nseg;
  const int L = in.L;
  if (decide_status(a, in)) return;
  const float T = in.T;
  const bool greedy = (T == 0.f);
  const bool topk = !greedy && in.K0 > 0 && in.K0 < V;
  if (wave == 0) {
    int bad = 0, bad0 = 0;
    for (int k = lane; k <= L && k < in.P; k += SPEC_WAVE) {
      const Partial* pt = sh.stage + k * nseg;
      if (topk) {
        const RowStat rt = a.rows_t[(size_t)i * (G + 1) + k];
        bad |= !(rt.lse2 == rt.lse2);
        sh.rt[k] = rt;
      } else if (greedy) {
        const int am = combine_argmax(pt, nseg);
        bad |= am < 0;
        sh.rt[k] = RowStat{0.0, -INFINITY, am < 0 ? 0 : am};
      } else {
        const double l2t = combine_sum(pt, nseg);
        bad |= !(l2t == l2t);
        sh.rt[k] = RowStat{l2t, -INFINITY, 0};
      }
      if (k == lane) bad0 = bad;
    }
    const unsigned long long m = __ballot(bad);
    const unsigned long long m0 = __ballot(bad0);
    if (lane == 0) {
      sh.bad_t = m != 0ull;
      sh.badm_t = m0;
    }
  } else if (wave == 1) {
    int bad = 0, bad0 = 0;
    const Partial* stage_d = sh.stage + (G + 1) * nseg;
    for (int k = lane; k < L && k < in.P; k += SPEC_WAVE) {
      if (topk) {
        const AccRec ar = a.acc[(size_t)i * G + k];
        sh.tacc[k] = ar.accept;
        sh.accr[k] = ar.r;
        sh.rd[k] = a.rows_d[(size_t)i * G + k];
      } else if (!greedy) {
        const double l2d = combine_sum(stage_d + k * nseg, nseg);
        bad |= !(l2d == l2d);
        sh.rd[k] = RowStat{l2d, -INFINITY, 0};
      }
      if (k == lane) bad0 = bad;
    }
    const unsigned long long m = __ballot(bad);
    const unsigned long long m0 = __ballot(bad0);
    if (lane == 0) {
      sh.bad_d = m != 0ull;
      sh.badm_d = m0;
    }
  } else if (!greedy && !topk) {
    for (int k = lane; k < L; k += SPEC_WAVE) {
      double ua, ue;
      verify_uniforms(in.seed, (uint64_t)i, (uint64_t)k, &ua, &ue);
      sh.ua[k] = ua;
    }
  }
}

// Second half (wave 0, after a barrier): r = min(1, p_t(x)/p_d(x)) with the logits at x the
// partials carry, the test, the first rejection.  Leaves in sh: st, n, L, greedy, and per position
// the acceptance ratio and the draft token.
__device__ __forceinline__ void decide_final(DecideShared& sh, const VerifyArgs& a, int i, const DecideIn& in) {
  const int lane = threadIdx.x;
  const int G = a.G, V = a.V, nseg = a.nseg;
  const int L = in.L;
  const float T = in.T;
  if (lane == 0) {
    sh.L = L;
    sh.greedy = (T == 0.f);
  }
  const int st = decide_status(a, in);
  if (st) {
    if (lane == 0) {
      sh.st = st;
      sh.n = 0;
    }
    return;
  }
  if (!a.ltr && (sh.bad_t | sh.bad_d)) {
    if (lane == 0) {
      sh.st = SPEC_REQ_NONFINITE;
      sh.n = 0;
    }
    return;
  }
  if (lane < G) sh.x[lane] = in.x;
  const bool greedy = (T == 0.f);
  const bool topk = !greedy && in.K0 > 0 && in.K0 < V;
  const double c64 = greedy ? 0.0 : kLog2e / (double)T;
  const Partial* stage_d = sh.stage + (G + 1) * nseg;
  int accept = 1;
  if (lane < L && lane < in.P) {   // L <= 64: one position per lane
    const int k = lane;
    int acc_k;
    double r;
    if (topk) {
      acc_k = sh.tacc[k];
      r = sh.accr[k];
    } else if (greedy) {
      acc_k = (in.x == sh.rt[k].argmax);
      r = acc_k ? 1.0 : 0.0;
    } else {
      r = acceptance_ratio(sh.stage[k * nseg].zx, stage_d[k * nseg].zx, c64, sh.rt[k].lse2, -INFINITY,
                           sh.rd[k].lse2, -INFINITY);
      acc_k = sh.ua[k] < r;
    }
    accept = acc_k;
    sh.accr[k] = r;
  }
  if (a.ltr) {
    // the walk: the first position that is bad or rejected ends it (gamma < 64: one ballot)
    const unsigned long long badm = sh.badm_t | sh.badm_d;
    const unsigned long long rej = __ballot(lane < L && lane < in.P && !accept) & ~badm;
    const int j = rej ? (int)__ffsll((long long)rej) - 1 : SPEC_WAVE;
    const int b = badm ? (int)__ffsll((long long)badm) - 1 : SPEC_WAVE;
    if (lane == 0) {
      if (j < b) {
        sh.st = 0;
        sh.n = j;
      } else if (b < SPEC_WAVE || in.P <= L) {
        // a bad row the walk reaches (or, never with the first pass's split, a walk that passed
        // every streamed position without reaching row L)
        sh.st = SPEC_REQ_NONFINITE;
        sh.n = 0;
      } else {
        sh.st = 0;
        sh.n = L;
      }
    }
    return;
  }
  const unsigned long long rej = __ballot(lane < L && !accept);
  if (lane == 0) {
    sh.st = 0;
    sh.n = rej ? (int)__ffsll((long long)rej) - 1 : L;
  }
}

// The Q table of a sampling request without top-k, built by the waves the decision leaves idle
// (waves 3 .. 15 of the fused workgroup) before the emit row is known.  Any offset R gives the
// same probabilities (p = Q / sum Q over the row); this one is an upper bound of z/T over every
// row the emit may read: a segment's reference m satisfies z log2(e)/T <= m + 32 for each of its
// values (the streaming kernel raises m whenever a term would pass 2^32), so with
// R0 = ln2 (max m + 40) every entry is below 2^-7.  The reference is also at most one above the
// segment's largest value, so the emit row's own largest entries stay normal unless its lse lies
// far below R0; the fused kernel then rebuilds the table with that lse.
template <bool BF16>
__device__ __forceinline__ void early_table(PassShared& ps, DecideShared& sh, const VerifyArgs& a, int i, const DecideIn& in) {
  const int t = (int)threadIdx.x - 3 * SPEC_WAVE, lane = threadIdx.x & 63;
  const int nthr = (int)blockDim.x - 3 * SPEC_WAVE;
  const int L = in.L, nseg = a.nseg;
  const bool sampling = !decide_status(a, in) && in.T > 0.f && !(in.K0 > 0 && in.K0 < a.V);
  if (!BF16 || !sampling) {
    if (t == 0) sh.table_ok = 0;
    return;
  }
  float mmax = -INFINITY;
  for (int q = lane; q < min(L + 1, in.P) * nseg; q += SPEC_WAVE) {
    const Partial& p = sh.stage[q];
    if (p.v > 0.0) mmax = fmaxf(mmax, p.m);
  }
  mmax = wave_max(mmax);
  const bool ok = mmax > -INFINITY && mmax < INFINITY;
  const double R0 = ((double)mmax + 40.0) * kLn2;
  if (ok) build_qtab_part(ps.Qt, 1.0 / (double)in.T, R0, ps.T64, t, nthr);
  if (t == 0) {
    sh.table_ok = ok;
    sh.R0 = R0;
  }
}

// Status, num_accepted, accept_prob and the output tokens of request i from the fused decision
// in sh (threads 0 .. G); the emitted token of a sampling request is left to sample_emit.
__device__ __forceinline__ void decided_outputs(const DecideShared& sh, const VerifyArgs& a, int i) {
  const int tid = threadIdx.x, G = a.G;
  const int st = sh.st, n = sh.n, L = sh.L;
  if (tid == 0) {
    if (a.status) a.status[i] = st;
    a.num_accepted[i] = st ? 0 : n;
  }
  if (a.accept_prob && tid < G)
    a.accept_prob[(size_t)i * G + tid] = (!st && tid < L && (!a.ltr || tid <= n)) ? (float)sh.accr[tid] : NAN;
  if (tid <= G) {
    int v = -1;
    if (!st && tid < n) v = sh.x[tid];
    else if (!st && tid == n && sh.greedy) v = sh.rt[n].argmax;
    if (st || tid != n || sh.greedy) a.out_tokens[(size_t)i * (G + 1) + tid] = v;
  }
}

// One 1024-thread workgroup per request does all of the request's work after the streaming:
// the acceptance decision from the segment partials, the emit pass over the whole emit row pair
// (16 waves), then sample_emit from the range sums it keeps in LDS.  Used when there are at
// least as many requests as compute units.
template <bool BF16>
__global__ __launch_bounds__(kFusedThreads) void emit_fused_kernel(VerifyArgs a) {
  __shared__ PassShared ps;
  __shared__ DecideShared ds;
  __shared__ FinalShared fs;
  const int i = a.r0 + (int)blockIdx.x;
  const int tid = threadIdx.x;
  const int NR = num_ranges(a.V);
  init_t64(ps.T64);
  init_t64(fs.T64);
  if (tid == 0) ds.amb_cnt = 0;
  const DecideIn din = decide_loads(a, i);
  stage_partials(ds, a, i);
  __syncthreads();
  if (tid < 3 * SPEC_WAVE) decide_stats(ds, a, i, din);
  else early_table<BF16>(ps, ds, a, i, din);
  __syncthreads();
  if (tid < SPEC_WAVE) decide_final(ds, a, i, din);
  __syncthreads();
  const int st = ds.st, n = ds.n;
  if (st || ds.greedy) {
    decided_outputs(ds, a, i);
    return;
  }
  {
    const RowStat rd = ds.rd[n < ds.L ? n : 0];
    if (topk_lists_complete(a, i, n, ds.L, din.T, din.K0, ds.rt[n], rd)) {
      // a top-k request with its kept tokens listed: no pass over the rows (the Q table is unused
      // by top-k requests, so its storage holds the lists)
      static_assert(sizeof(TopkEmitShared) <= sizeof(ps.Qt), "the lists fit the table's storage");
      decided_outputs(ds, a, i);
      const int tok = emit_topk_lists<BF16>(*reinterpret_cast<TopkEmitShared*>(ps.Qt), a, i, n, ds.L, din.T,
                                            ds.rt[n], rd, ps.T64);
      if (threadIdx.x == 0) a.out_tokens[(size_t)i * (a.G + 1) + n] = tok;
      return;
    }
  }
  EmitRows e = emit_rows_from<BF16>(a, i, n, ds.L, din.T, ds.rt[n], ds.rd[n < ds.L ? n : 0]);
  e.amb_n = &ds.amb_cnt;
  e.amb_v = ds.amb_list;
  const bool table = BF16 && !(din.K0 > 0 && din.K0 < a.V);
  e.Qt = table ? ps.Qt : nullptr;
  // the early table serves unless the emit row's lse lies far below its offset (then the pass
  // builds another with the row's own)
  const bool ready = table && ds.table_ok && ds.R0 - e.R <= 600.0;
  if (ready) e.R = ds.R0;
  run_pass<BF16>(ps, a, i, 0, e, fs.rg, din.K0, ready);
  // the outputs known since the decision, written once the pass's loads are under way (a later
  // wait for a load would otherwise wait for these stores too)
  decided_outputs(ds, a, i);
  if (tid < SPEC_WAVE) {
    double x = 0.0;
    for (int r = tid; r < NR; r += SPEC_WAVE) x += fs.rg[r].t;
    x = wave_sum(x);
    if (tid == 0) {
      double y = 0.0;
      for (int w = 0; w < kFusedThreads / SPEC_WAVE; ++w) y += ps.red[1][w];
      fs.St = x;
      fs.Sd = y;
      fs.na = ds.amb_cnt;
    }
  }
  __syncthreads();
  sample_emit<BF16, kFusedThreads>(fs, a, i, n, e);
}

// Between the two streaming passes of a left-to-right call: request r walks the positions
// k < min(L, phase_cap) that the first pass streamed, with the acceptance test the fused emit makes
// (the same partials, combined in the same order, the same arithmetic), and npos[r] records the
// positions whose rows are streamed in all: L + 1 when the walk passed every one of them with
// valid rows and L >= phase_cap (the second pass then streams positions phase_cap .. L), else
// min(L + 1, phase_cap).  A request with bad arguments gets 0 (the fused emit reports it).  The
// second pass's item count, L + 1 - phase_cap per request that goes on, is summed into *nwalk.
// One wave per request: with b = 3 segment bits (rows of at most 8 segments) or 4 (at most 16), lane
// l loads segment l mod 2^b of row (l >> b) & 1 (target, draft) of position l >> (b + 1), so every
// load of the walk is in flight at once (phase_cap <= 2^(5 - b) positions); the first lane of each
// row combines its segments in segment order, and the first lane of each position makes its test.
constexpr int kWalkThreads = 256;
static_assert(kMaxStreamSegs <= 16, "a row's partials fit 16 lanes");

__host__ __device__ inline int walk_seg_bits(int nseg) { return nseg > 8 ? 4 : 3; }
__host__ __device__ inline int walk_max_cap(int nseg) { return SPEC_WAVE >> (walk_seg_bits(nseg) + 1); }

__global__ __launch_bounds__(kWalkThreads) void ltr_walk_kernel(VerifyArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = (int)blockIdx.x * (kWalkThreads / SPEC_WAVE) + ((int)threadIdx.x >> 6);
  if (r >= a.B) return;   // whole waves
  const int G = a.G, V = a.V, nseg = a.nseg, cap = a.phase_cap;
  const int sb = walk_seg_bits(nseg), grp = 1 << sb;
  const int k = lane >> (sb + 1), row = (lane >> sb) & 1, sg = lane & (grp - 1);
  const int L = a.lengths[r];
  const float T = a.temperature[r];
  const int rs = a.req_status[r];
  const uint64_t seed = a.seed[r];
  const int kc = min(k, G);   // positions past gamma load position gamma's partials (unused)
  const int x = a.tokens[(size_t)r * G + min(k, G - 1)];
  const Partial* ps = (row ? a.part_d : a.part_t) + ((size_t)r * (G + 1) + kc) * nseg + min(sg, nseg - 1);
  const double v = ps->v;
  const float m = ps->m;
  const int idx = ps->idx, bad = ps->bad;
  const float zx = ps->zx;
  // the row's first lane: combine_sum's and combine_argmax's steps over segments 0 .. nseg-1
  const int base = lane & ~(grp - 1);
  float Mr = -INFINITY, rb = -INFINITY;
  int bd = 0, ri = 0x7fffffff;
  for (int t = 0; t < nseg; ++t) {
    const double vt = __shfl(v, base + t, SPEC_WAVE);
    const float mt = __shfl(m, base + t, SPEC_WAVE);
    const int it = __shfl(idx, base + t, SPEC_WAVE);
    bd |= __shfl(bad, base + t, SPEC_WAVE);
    if (vt > 0.0) Mr = fmaxf(Mr, mt);
    const float xt = (float)vt;
    if (xt > rb) {
      rb = xt;
      ri = it;
    } else if (xt == rb) {
      ri = min(ri, it);
    }
  }
  double Sr = 0.0;
  for (int t = 0; t < nseg; ++t) {
    const double vt = __shfl(v, base + t, SPEC_WAVE);
    const float mt = __shfl(m, base + t, SPEC_WAVE);
    if (vt > 0.0) Sr += ldexp(vt, (int)fmaxf(mt - Mr, -2000.f));
  }
  const double l2 = (bd || !(Sr > 0.0)) ? __builtin_nan("") : (double)Mr + log2(Sr);
  const int am = (bd || !(rb > -INFINITY)) ? -1 : ri;
  // position k's test by its first lane, with its draft row's values from the lane grp above
  const double l2d = __shfl(l2, lane + grp, SPEC_WAVE);
  const float zxd = __shfl(zx, lane + grp, SPEC_WAVE);
  const bool valid = L >= 0 && L <= G && rs == 0 && T >= 0.f && T < INFINITY;
  int ok = 0;
  if ((lane & (2 * grp - 1)) == 0 && k < cap && k < L && valid && x >= 0 && x < V) {
    if (T == 0.f) {
      ok = am == x;   // -1 (a bad row) never matches
    } else if (l2 == l2 && l2d == l2d) {
      const double rr = acceptance_ratio(zx, zxd, kLog2e / (double)T, l2, -INFINITY, l2d, -INFINITY);
      double ua, ue;
      verify_uniforms(seed, (uint64_t)r, (uint64_t)k, &ua, &ue);
      ok = ua < rr;
    }
  }
  const unsigned long long okm = __ballot(ok);
  if (lane == 0) {
    bool more = valid && L >= cap;
    for (int q = 0; q < cap; ++q) more = more && ((okm >> (q << (sb + 1))) & 1ull);
    a.npos[r] = valid ? (more ? L + 1 : min(L + 1, cap)) : 0;
    if (more) atomicAdd(a.nwalk, L + 1 - cap);   // the second pass's items (cleared by the list)
  }
}

int ltr_first_pass(int gamma, int nseg) { return std::min(std::min(kLtrFirstPass, gamma), walk_max_cap(nseg)); }

void launch_ltr_walk(const VerifyArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)((a.B + kWalkThreads / SPEC_WAVE - 1) / (kWalkThreads / SPEC_WAVE));
  hipLaunchKernelGGL(ltr_walk_kernel, dim3(grid), dim3(kWalkThreads), 0, s, a);
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
