// Internal layout shared by the verification kernels and their host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"

namespace spec {

// Per logit row, written by the streaming kernel.
struct RowStat {
  double lse2;    // log2 sum_v 2^(z_v * log2(e) / T) over the kept set (sampling rows)
  float theta;    // kept-set threshold on raw logits (-inf when no top-k)
  int32_t argmax; // first-occurrence argmax (greedy rows)
};

// Per (request, draft position) acceptance record.
struct AccRec {
  double r;        // min(1, p_t(x)/p_d(x)) (greedy: 1 match / 0 mismatch)
  int32_t accept;  // 1 accepted, 0 rejected
  int32_t valid;   // 1 when computed
};

// Statistics of one segment of a row (the streaming kernel splits every row into nseg segments).
struct Partial {
  double v;     // sampling: sum of 2^(z*c - m) over the segment; greedy: the segment's maximum
  float m;      // sampling: the segment's integer reference
  int32_t idx;  // greedy: first index of the maximum
  int32_t bad;  // NaN or +inf seen
  float zx;     // segment 0 of a row with a draft token x: the row's raw logit at x (else NaN)
};

// Emitted-token work: one range = kRangeElems consecutive tokens of the emit row.
constexpr int kRangeElems = 2048; // tokens per emit range (one wave, 4 steps of 64 x 8)
constexpr int kMaxEmitSegs = 16;  // workgroups per request in the emit pass, at most
constexpr int kAmbCap = 256;      // tokens of uncertain residual sign recorded per request

struct EmitRange {
  double a;  // sum of E_t over tokens with p_t > p_d
  double d;  // sum of E_d over the same tokens
  double t;  // sum of E_t over every token
};

struct EmitReq {
  double sd_part[kMaxEmitSegs];  // per-segment sums of E_d = exp(z_d/T - R) (E_t sums are the ranges')
  int32_t amb_n;              // number of uncertain-sign tokens seen
  int32_t pad;
};

// Top-k rows (sampling requests with 0 < top_k <= kTopkSegMaxK) are streamed in up to kTopkSegs
// segments.  Each segment lists its values at or above its own K-th largest value, with their token
// ids: a superset of the row's kept tokens inside it, since a segment's K-th largest is at most the
// row's.  The last of an item's segment workgroups to finish merges the lists into the row's exact
// threshold and normaliser, and the emit draws from the lists instead of reading the rows again.
constexpr int kTopkSegs = 4;        // segments of a top-k row, at most
constexpr int kTopkSegMaxK = 64;    // larger top_k: the row is streamed whole by one workgroup
constexpr int kTopkSegCap = 96;     // (value, id) entries kept per (row, segment)
// A wave's LDS region while streaming a segment: the raw 16-byte vectors holding a candidate (and
// their vector indices), then, expanded in place, the candidates (value, token id).
constexpr int kTopkWaveHits = 192;                       // candidate vectors a wave may keep
constexpr int kTopkRegionBytes = kTopkWaveHits * 20;     // 16-byte vector + 4-byte index each
constexpr int kTopkWaveCand = kTopkRegionBytes / 8;      // candidates a region holds (480)
constexpr int kTopkSegCand = 8 * kTopkWaveCand;          // the workgroup's candidate buffer (8 waves)
constexpr int kTopkEmitKept = 2 * SPEC_WAVE;      // kept entries per row the emit draws from, at most

struct TopkSeg {
  int32_t n;      // entries stored; kTopkSegCap + 1 when the segment could not be listed (too many
                  // values at its cut, or too many candidates)
  float theta;    // the segment's K-th largest raw logit (ties counted)
  float vmax;     // the segment's largest raw logit
  int32_t bad;    // NaN or +inf seen in the segment
};

struct VerifyArgs {
  int B, G, V;
  int greedy_only;
  int overlap_only;    // statistics of the draft positions' row pairs only (no bonus rows, no test)
  int flat;            // rows stored flattened: only request i's verified rows, request after request
  const void* target;
  const void* draft;
  const int32_t* tokens;
  const int32_t* lengths;
  const float* temperature;
  const int32_t* top_k;
  const uint64_t* seed;
  int32_t* num_accepted;
  int32_t* out_tokens;
  float* accept_prob;
  int32_t* status;
  // workspace
  RowStat* rows_t;     // [B, G+1]
  RowStat* rows_d;     // [B, G]
  AccRec* acc;         // [B, G]
  int32_t* items;      // [B * (G+1)] work items, (request << 7) | position
  int32_t* items_x;    // [B * (G+1)] the item's draft token x_k (-1 for a bonus row)
  int32_t* nitems;     // [1]
  int32_t* req_status; // [B] SPEC_REQ_* bits raised while streaming
  int nseg;            // segments per row in the streaming kernel
  Partial* part_t;     // [B, G+1, nseg] by (request, position, segment)
  Partial* part_d;     // [B, G+1, nseg]
  EmitReq* ereq;       // [B]
  EmitRange* ranges;   // [B, ceil(V / kRangeElems)]
  int32_t* amb;        // [B, kAmbCap]
  int64_t* t_off;      // [B] flattened layout: first target row of request i (else unused)
  int64_t* d_off;      // [B] flattened layout: first draft row of request i
  int64_t flat_trows;  // flattened layout: target rows and draft rows the caller passed
  int64_t flat_drows;
  int r0, r1;          // the emit kernels handle requests [r0, r1)
  int emit_segs;       // emit-pass workgroups per request (1 = one fused workgroup, else 2 .. kMaxEmitSegs)
  int max_items;       // caller's bound on the number of work items (0: none); sizes the streaming grid
  int wl_ready;        // the work list was written by the scheduler's last kernel (no work-list kernel)
  int derive_items;    // request-major work list: items[r] = request r's first item, *nitems the total
                       // (B <= 2 * kStreamThreads); each streaming workgroup finds its own request
  int nseg_topk;       // segments of a top-k row (1: top-k rows are streamed whole)
  TopkSeg* tk_seg;     // [B, G+1, 2, kTopkSegs] per (item, target/draft row, segment)
  float* tk_val;       // [B, G+1, 2, kTopkSegs, kTopkSegCap] raw logits at or above each segment's cut
  int32_t* tk_ids;     // same shape: their token ids
  // left-to-right verification (the walk stops at the first rejection; rows after it are not read)
  int ltr;             // the decision follows the walk: accept_prob and NONFINITE only up to it
  int phase_cap;       // > 0: the first streaming pass takes positions 0 .. phase_cap - 1 only
  int k_base;          // the streaming pass's first position (derived work lists)
  int32_t* npos;       // [B] positions whose rows were streamed (written between the two passes)
  int32_t* nwalk;      // [1] the second pass's item count (cleared by the first pass's list, summed by
                       //     the walk)
};

// Index of the TopkSeg record of (request i, position k, row `which` (0 target, 1 draft), segment 0).
__host__ __device__ inline size_t topk_slot(int G, int i, int k, int which) {
  return (((size_t)i * (G + 1) + k) * 2 + which) * kTopkSegs;
}

constexpr int kStreamThreads = 512;
constexpr int kMaxStreamSegs = 16;   // segments per row in the streaming kernel, at most
constexpr int kWorklistThreads = 1024;
constexpr int kPassThreads = 512;    // emit pass workgroup
constexpr int kEmitThreads = 256;    // emit final workgroup (x 8 tokens = one range)
constexpr int kFusedThreads = 1024;  // one workgroup per request doing the whole emit
constexpr int kFuseMinRequests = 256; // fuse when every compute unit gets a request (MI355X: 256 CUs)
constexpr int kTopkCap = 4096;   // top-k candidates kept in LDS per row
constexpr int kTopkPre = 4;      // vectors per thread sampled for the top-k lower bound

static constexpr double kLn2 = 0.69314718055994530942;
static constexpr double kLog2e = 1.44269504088896340736;

__host__ __device__ inline int num_ranges(int V) { return (V + kRangeElems - 1) / kRangeElems; }

// lse2 of a row from its nseg segment partials (NaN when a segment saw NaN/+inf or the kept set
// is empty): partial sums brought to the largest reference and added in fp64.
__device__ inline double combine_sum(const Partial* p, int nseg) {
  float Mr = -__builtin_inff();
  int bad = 0;
  for (int s = 0; s < nseg; ++s) {
    bad |= p[s].bad;
    if (p[s].v > 0.0) Mr = fmaxf(Mr, p[s].m);
  }
  double Sr = 0.0;
  for (int s = 0; s < nseg; ++s)
    if (p[s].v > 0.0) Sr += ldexp(p[s].v, (int)fmaxf(p[s].m - Mr, -2000.f));
  return (bad || !(Sr > 0.0)) ? __builtin_nan("") : (double)Mr + log2(Sr);
}

// First-occurrence argmax of a row from its segment partials (greedy rows); -1 when a segment
// saw NaN/+inf or no logit above -inf.
__device__ inline int combine_argmax(const Partial* p, int nseg) {
  float rb = -__builtin_inff();
  int ri = 0x7fffffff, bad = 0;
  for (int s = 0; s < nseg; ++s) {
    bad |= p[s].bad;
    const float v = (float)p[s].v;
    if (v > rb) {
      rb = v;
      ri = p[s].idx;
    } else if (v == rb) {
      ri = min(ri, p[s].idx);
    }
  }
  return (bad || !(rb > -__builtin_inff())) ? -1 : ri;
}

// Acceptance ratio r = min(1, p_t(x) / p_d(x)) from the raw logits at x, c = log2(e)/T, the rows'
// lse2 and kept-set thresholds: log p(x) = ln2 (z_x c - lse2), -inf outside the kept set;
// r = 0 when p_t(x) = 0, r = 1 when p_d(x) = 0 < p_t(x).
__device__ inline double acceptance_ratio(float zt, float zd, double c64, double l2t, float tht, double l2d,
                                          float thd) {
  const double lpt = (zt >= tht) ? kLn2 * ((double)zt * c64 - l2t) : -__builtin_inf();
  const double lpd = (zd >= thd) ? kLn2 * ((double)zd * c64 - l2d) : -__builtin_inf();
  if (lpt == -__builtin_inf()) return 0.0;
  if (lpd == -__builtin_inf()) return 1.0;
  return fmin(1.0, exp(lpt - lpd));
}

// Status and first rejection of request i.  Called by a whole wave (lane k looks at draft
// position k; gamma <= 64); every lane gets the result.
__device__ inline void request_decision(const VerifyArgs& a, int i, int* st_out, int* n_out) {
  const int G = a.G, V = a.V;
  const int lane = threadIdx.x & 63;
  const int L = a.lengths ? a.lengths[i] : G;
  int st = 0, n = 0;
  if (L < 0 || L > G) {
    st = SPEC_REQ_BAD_LENGTH;
  } else {
    const float T = a.greedy_only ? 0.f : a.temperature[i];
    const int K = (a.top_k && !a.greedy_only) ? a.top_k[i] : 0;
    if (!(T >= 0.f && T < __builtin_inff())) st |= SPEC_REQ_BAD_TEMPERATURE;
    if (K < 0) st |= SPEC_REQ_BAD_TOPK;
    int x = 0, acc = 1;
    if (lane < L) {
      x = a.tokens[(size_t)i * G + lane];
      acc = a.acc[(size_t)i * G + lane].accept;
    }
    if (__ballot(lane < L && (x < 0 || x >= V))) st |= SPEC_REQ_BAD_TOKEN;
    if (st == 0) st |= a.req_status[i];
    if (st == 0) {
      const unsigned long long rej = __ballot(lane < L && !acc);
      n = rej ? (int)__ffsll((long long)rej) - 1 : L;
    }
  }
  *st_out = st;
  *n_out = n;
}

// Row k of request i: the padded layout [B, G+1, V] (target) / [B, G, V] (draft), or, when
// a.flat is set, the flattened layout in which request i's rows start at t_off[i] / d_off[i].
template <int ES>
__device__ inline const char* target_row(const VerifyArgs& a, int i, int k) {
  const size_t r = a.flat ? (size_t)a.t_off[i] + k : (size_t)i * (a.G + 1) + k;
  return reinterpret_cast<const char*>(a.target) + r * (size_t)a.V * ES;
}

template <int ES>
__device__ inline const char* draft_row(const VerifyArgs& a, int i, int k) {
  const size_t r = a.flat ? (size_t)a.d_off[i] + k : (size_t)i * a.G + k;
  return reinterpret_cast<const char*>(a.draft) + r * (size_t)a.V * ES;
}

// Launch the emitted-token kernels (defined in emit.hip).
void launch_emit(const VerifyArgs& a, int bf16, hipStream_t s);

// Between the two streaming passes of a left-to-right call: the walk over the first pass's positions
// (defined in emit.hip).
void launch_ltr_walk(const VerifyArgs& a, hipStream_t s);

// Scratch of worklist_from_lengths.
struct WorklistShared {
  int cnt[kWorklistThreads / SPEC_WAVE][SPEC_MAX_GAMMA + 1];
  int ctot[SPEC_MAX_GAMMA + 1];
  int off[SPEC_MAX_GAMMA + 2];
  long long wsum[kWorklistThreads / SPEC_WAVE];
  long long wsum2[kWorklistThreads / SPEC_WAVE];   // a second scan's wave totals
};

constexpr int kWlPre = 16;   // draft tokens per request fetched ahead of the work list

// Request t's first min(gamma, kWlPre) draft tokens into thread t's registers (t < B; -1 elsewhere,
// and everywhere when the work list carries no tokens).  They do not depend on the lengths, so a
// caller issues these loads before it knows them.
__device__ inline void worklist_prefetch(const VerifyArgs& a, int (&xp)[kWlPre]) {
  const int tid = threadIdx.x;
  const bool want = a.tokens && !a.overlap_only && !a.derive_items && tid < a.B;
#pragma unroll
  for (int u = 0; u < kWlPre; ++u) xp[u] = (want && u < a.G) ? a.tokens[(size_t)tid * a.G + u] : -1;
}

// The position-major work list of a call with B <= kWorklistThreads (padded layout), by one
// workgroup of kWorklistThreads threads in which thread t holds request t's length L (its raw value,
// anything for t >= B) and the tokens of worklist_prefetch: items (i << 7 | k) for every k <= L_i
// (k < L_i for overlap_only), ordered by position, then request; each item's draft token (k < L_i);
// the item count; the request's cap mark (token cap a.max_items > 0: from the first request whose
// running sum of L_i + 1 passes the cap on, valid requests are marked SPEC_REQ_OVER_BUDGET and get
// no items) and its emit counter.
__device__ inline void worklist_from_lengths(WorklistShared& sh, const VerifyArgs& a, int L_raw,
                                             const int (&xp)[kWlPre]) {
  constexpr int NW = kWorklistThreads / SPEC_WAVE;   // the workgroup is kWorklistThreads wide
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int G = a.G, B = a.B;
  const bool want_x = a.tokens && !a.overlap_only;
  const int L = (tid < B) ? L_raw : -1;
  const bool valid = L >= 0 && L <= G;
  int drop = 0;
  if (a.max_items > 0) {
    const long long n = valid ? L + 1 : 0;
    const long long in = wave_inclusive_sum_i64(n, lane);
    if (lane == 63) sh.wsum[wave] = in;
    __syncthreads();
    long long before = 0;   // the earlier waves' totals (independent reads, no loop-carried wait)
#pragma unroll
    for (int w = 0; w < NW; ++w) before += (w < wave) ? sh.wsum[w] : 0;
    drop = (n > 0 && before + in > (long long)a.max_items);
  }
  if (tid < B) {
    a.req_status[tid] = drop ? SPEC_REQ_OVER_BUDGET : 0;
    a.ereq[tid].amb_n = 0;
  }
  const int last = (valid && !drop) ? (a.overlap_only ? L - 1 : L) : -1;
  if (a.derive_items) {
    // request-major: request tid's first item is the exclusive prefix of (last + 1) over the
    // requests before it (at most phase_cap items each in the first of two passes); the streaming
    // workgroups find their requests from these words
    const long long n = (a.phase_cap > 0) ? min(last + 1, a.phase_cap) : last + 1;
    const long long in = wave_inclusive_sum_i64(n, lane);
    if (lane == 63) sh.wsum2[wave] = in;
    __syncthreads();
    long long before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      before += (w < wave) ? sh.wsum2[w] : 0;
      total += sh.wsum2[w];
    }
    if (tid < B) a.items[tid] = (int)(before + in - n);
    if (tid == 0) {
      *a.nitems = (int)total;
      if (a.phase_cap > 0) *a.nwalk = 0;   // the walk between the passes adds the second's items
    }
    return;
  }
  for (int k = 0; k <= G; ++k) {
    const unsigned long long m = __ballot(last >= k);
    if (lane == 0) sh.cnt[wave][k] = __popcll(m);
  }
  __syncthreads();
  if (tid <= G) {
    // per-wave exclusive offsets within position tid, and its total c_k = #{i : last_i >= k}
    int c[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) c[w] = sh.cnt[w][tid];
    int run = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      sh.cnt[w][tid] = run;
      run += c[w];
    }
    sh.ctot[tid] = run;
  }
  __syncthreads();
  if (wave == 0) {
    // items of position k start at off[k] = c_0 + ... + c_{k-1}
    const long long c = (lane <= G) ? sh.ctot[lane] : 0;
    const long long incl = wave_inclusive_sum_i64(c, lane);
    if (lane <= G) sh.off[lane] = (int)(incl - c);
    const int total64 = (int)read_lane(incl, 63);
    if (lane == 0) {
      if (G == SPEC_WAVE) sh.off[SPEC_WAVE] = total64;   // position 64 (gamma = 64)
      const int nit = (G == SPEC_WAVE) ? total64 + sh.ctot[SPEC_WAVE] : total64;
      sh.off[G + 1] = nit;
      *a.nitems = nit;
    }
  }
  __syncthreads();
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // positions k0 .. k0 + 7 (at most G): x[u] is the draft token of position k0 + u; the
  // positions' offsets are read before the first ballot (independent reads, one wait)
  auto put8 = [&](int k0, const int (&x)[8]) {
    int base[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = min(k0 + u, G);
      base[u] = sh.off[k] + sh.cnt[wave][k];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int k = k0 + u;
      if (k > G) break;
      const unsigned long long m = __ballot(last >= k);
      if (last >= k) {
        const int idx = base[u] + __popcll(m & below);
        a.items[idx] = (tid << 7) | k;
        a.items_x[idx] = (k < L) ? x[u] : -1;
      }
    }
  };
  int x0[8], x1[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    x0[u] = xp[u];
    x1[u] = xp[8 + u];
  }
  put8(0, x0);
  if (G >= 8) put8(8, x1);
  static_assert(kWlPre == 16, "two groups of eight fetched ahead");
  for (int k0 = kWlPre; k0 <= G; k0 += 8) {
    int x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      x[u] = (want_x && valid && k0 + u < L) ? a.tokens[(size_t)tid * G + k0 + u] : -1;
    put8(k0, x);
  }
}

// Host steps shared by the entry points (defined in verify.hip).
bool shape_ok(int B, int G, int V, int dtype);
bool aligned16(const void* p);
// Point the workspace arrays of `a` into ws (after `extra_bytes` more for the caller at *extra,
// 256-byte aligned); SPEC_ERR_WORKSPACE when it is missing, short or misaligned.
int32_t bind_workspace(VerifyArgs& a, int dtype, void* ws, size_t ws_bytes, size_t extra_bytes, char** extra);
size_t workspace_bytes(int B, int G, int V, bool emit, bool topk);
// Work list (unless a.wl_ready), then the streaming statistics (events, when given, bracket the
// streaming kernel); item_bound > 0 caps the streaming grid's work items further.
void launch_statistics(const VerifyArgs& a, int dtype, hipStream_t s, void* ev0, void* ev1, size_t item_bound = 0);
// Statistics, acceptance and emit of a call whose workspace is bound (the verify kernels of
// spec_verify after the argument checks).
int32_t launch_verify_bound(VerifyArgs a, int dtype, hipStream_t s, void* ev0, void* ev1);
// The same for a left-to-right call (two streaming passes; see verify.hip).
int32_t launch_verify_ltr(VerifyArgs a, int dtype, hipStream_t s, void* ev0, void* ev1);
// Positions of every request that the first pass of a left-to-right call streams (at most, and at
// most what the walk kernel's wave holds: ltr_first_pass).
constexpr int kLtrFirstPass = 3;
int ltr_first_pass(int gamma, int nseg);
// Segment partials -> row records and (with draft tokens) the acceptance test.
void launch_combine(const VerifyArgs& a, hipStream_t s);

}  // namespace spec
