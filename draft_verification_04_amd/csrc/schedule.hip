// Confidence-scheduled verify lengths on gfx950.
//
// Follows the DSpark paper, §3.2.2 (survival a_{r,j} = product of c_{r,1..j};
// marginal gain of extending request r to j is a_{r,j}; admit candidates in
// descending survival; objective Theta = tau * SPS(batch tokens) read from a
// profiled cost table) and Algorithm 1 of the paper's Chinese translation
// (stop at the first admission that does not raise Theta); the global mode is
// the search without the break of §5.2.
//
// Exactness: survivals are float32 products taken left to right; tau is an
// int64 in fixed point with 47 fractional bits (each survival floored to a
// multiple of 2^-47; tau <= B + B*gamma <= 2^15 leaves room below 2^63), so the
// parallel prefix sum is exact and independent of its association;
// Theta(m) = fp64(tau(m)) * 2^-47 * sps[B + m].
//
// Candidates are ordered by the 32-bit key ~bits(a) (ascending key = descending
// survival), ties by index r * gamma + j (request, then position).  One CU retires
// only 64 lane operations per cycle, so the sort is spread over the chip.  Pools of at
// most 8192 candidates (and few enough requests) take one kernel for it:
//   runs_rank_kernel  every workgroup rebuilds all keys in LDS (each request's keys
//                 form an ascending run) and places 16 candidates, each by binary
//                 searches in the other requests' runs;
// larger pools take two:
//   keys_kernel   one wave per chunk of 64 candidates: survivals, and the chunk
//                 sorted by (key, index) in registers, each key stored with its index;
//   rank_kernel   one workgroup per chunk: each key's place in the whole pool is
//                 its place in its chunk plus, for every other chunk, the number of
//                 keys there that precede it (binary search in LDS), and the key and
//                 its index are written straight to that place;
//   final_kernel  one workgroup: exclusive int64 scan of the fixed-point
//                 survivals, Theta(m), first non-rise (early stop) or first maximum
//                 (global), and per-request counts of the first m* entries of the
//                 sorted pool, by their indices (LDS atomics); each thread reads its
//                 own positions of the sorted pool straight from memory.  In the combined
//                 schedule-and-verify call (B <= 1024) it also writes the verify work
//                 list from the lengths it holds, in place of the work-list kernel.
#include "common.hpp"
#include "spec_verify.h"
#include "verify_impl.hpp"

#include <math.h>

namespace spec {

constexpr int kChunk = SPEC_WAVE;                 // candidates per sorted chunk
constexpr int kKeysThreads = 256;                 // four chunks per keys workgroup
constexpr int kRankParts = 8;                     // waves sharing one chunk's searches
constexpr int kFinalThreads = 1024;
constexpr int kFinalWaves = kFinalThreads / SPEC_WAVE;
constexpr long long kOne = 1ll << 47;
constexpr unsigned kNoCandidate = 0xffffffffu;

struct SchedArgs {
  int B, G, budget, mode;
  const float* conf;
  const double* sps;
  int32_t* lengths;
  double* theta;
  int32_t* status;
  unsigned* chunked;      // [N] keys, each chunk of 64 sorted
  unsigned* chunked_idx;  // [N] the candidate index r * gamma + j of each key of `chunked`
  unsigned* sorted;       // [N] keys, whole pool sorted
  unsigned* sorted_idx;   // [N] the candidate index of each key of `sorted`
  const int32_t* capacity_in;  // top-K mode: [1] device, the number of candidates to admit
  int32_t* capacity_out;       // [1] device or NULL: the number admitted (m*)
};

constexpr int kSchedTopK = 2;   // internal mode: admit the first K sorted candidates

__device__ __forceinline__ unsigned surv_key(float s) { return s > 0.f ? ~__float_as_uint(s) : kNoCandidate; }
__device__ __forceinline__ float key_surv(unsigned k) { return __uint_as_float(~k); }

__device__ __forceinline__ long long fixed_q(float a) {
  // floor(a * 2^47): a is a float32 in [0, 1]; the product is exact in fp64
  return (long long)floor((double)a * 0x1p47);
}

__device__ __forceinline__ double theta_of(long long tau, double sps) {
  return ((double)tau * 0x1p-47) * sps;
}

// ---- keys ----------------------------------------------------------------

__global__ __launch_bounds__(kKeysThreads) void keys_kernel(SchedArgs a) {
  __shared__ float cf[kKeysThreads + 2 * SPEC_MAX_GAMMA];  // confidences of the requests in reach
  const int B = a.B, G = a.G, N = B * G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int c0 = blockIdx.x * kKeysThreads;
  const int cend = min(c0 + kKeysThreads, N);
  const int f0 = (c0 / G) * G, f1 = ((cend - 1) / G + 1) * G;  // whole requests overlapping the block
  for (int x = tid; x < f1 - f0; x += kKeysThreads) cf[x] = a.conf[f0 + x];
  __syncthreads();

  const int p = c0 + tid;
  unsigned key = kNoCandidate;
  if (p < N) {
    const int r = p / G, j = p - r * G;
    const float* c = cf + (r * G - f0);
    bool bad = false;
    float s = 0.f;
    for (int t = 0; t < G; ++t) {
      const float v = c[t];
      bad |= !(v >= 0.f && v <= 1.f);
      if (t <= j) s = (t == 0) ? v : __fmul_rn(s, v);
    }
    key = bad ? kNoCandidate : surv_key(s);
    if (j == 0 && a.status) a.status[r] = bad ? SPEC_REQ_BAD_CONFIDENCE : 0;
  }
  // bitonic sort of the wave's 64 (key, index) pairs, one per lane; padding sorts last
  unsigned long long x = ((unsigned long long)key << 32) | (unsigned)(p < N ? p : 0x7fffffff);
  for (int size = 2; size <= SPEC_WAVE; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const unsigned long long y = __shfl_xor(x, stride, SPEC_WAVE);
      const bool up = (lane & size) == 0;
      const bool lower = (lane & stride) == 0;
      x = (lower == up) ? (x < y ? x : y) : (x < y ? y : x);
    }
  }
  if (p < N) {
    a.chunked[p] = (unsigned)(x >> 32);
    a.chunked_idx[p] = (unsigned)x;
  }
}

// ---- ranks -----------------------------------------------------------------

// For S chunks c[u] at once: the number of their keys that precede key k of chunk ck, i.e.
// keys not larger than k in a chunk before ck (index order on ties) and keys smaller than k
// in a chunk after it (a key v precedes k when v < k + [chunk before ck], compared in 64
// bits).  Chunks hold up to 64 ascending keys.  The S searches advance in lockstep with
// plain arithmetic, so their LDS reads are in flight together.
template <int S>
__device__ __forceinline__ int count_before(const unsigned* keys, const int (&c)[S], int ck, int N,
                                            unsigned k) {
  int base[S], len[S];
  unsigned long long lim[S];
#pragma unroll
  for (int u = 0; u < S; ++u) {
    base[u] = c[u] * kChunk;
    len[u] = min(kChunk, N - base[u]);
    lim[u] = (unsigned long long)k + (c[u] < ck ? 1ull : 0ull);
  }
#pragma unroll
  for (int it = 0; it < 7; ++it) {  // 7 halvings empty a range of 64
    unsigned v[S];
#pragma unroll
    for (int u = 0; u < S; ++u) v[u] = keys[min(base[u] + (len[u] >> 1), N - 1)];
#pragma unroll
    for (int u = 0; u < S; ++u) {
      const int half = len[u] >> 1;
      const int go = (int)(len[u] > 0) & (int)((unsigned long long)v[u] < lim[u]);
      base[u] += go * (half + 1);
      len[u] = go ? len[u] - half - 1 : half;
    }
  }
  int n = 0;
#pragma unroll
  for (int u = 0; u < S; ++u) n += (c[u] != ck) ? base[u] - c[u] * kChunk : 0;
  return n;
}

__global__ __launch_bounds__(kChunk * kRankParts) void rank_kernel(SchedArgs a) {
  __shared__ __align__(16) unsigned keys[SPEC_MAX_SCHED_CANDIDATES];
  __shared__ int part[kRankParts][kChunk];
  const int N = a.B * a.G;
  const int tid = threadIdx.x, part_id = tid >> 6, lane = tid & 63;
  constexpr int NT = kChunk * kRankParts;
  // stage the chunk-sorted pool (16-byte loads for the aligned bulk)
  const int n4 = N >> 2;
  for (int x = tid; x < n4; x += NT)
    reinterpret_cast<uint4*>(keys)[x] = reinterpret_cast<const uint4*>(a.chunked)[x];
  for (int x = (n4 << 2) + tid; x < N; x += NT) keys[x] = a.chunked[x];
  __syncthreads();
  const int ck = blockIdx.x, nch = (N + kChunk - 1) / kChunk;
  const int p = ck * kChunk + lane;
  const bool valid = p < N;
  const unsigned k = valid ? keys[p] : 0u;
  const unsigned idx = a.chunked_idx[min(p, N - 1)];
  int cnt = 0;
  // this wave's share of the other chunks, eight searches in flight; chunks past the end are
  // replaced by the own chunk, which counts nothing
  for (int c = part_id; c < nch; c += 8 * kRankParts) {
    int cs[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) cs[u] = (c + u * kRankParts < nch) ? c + u * kRankParts : ck;
    cnt += count_before<8>(keys, cs, ck, N, k);
  }
  part[part_id][lane] = cnt;
  __syncthreads();
  if (part_id == 0 && valid) {
    int rank = lane;
#pragma unroll
    for (int w = 0; w < kRankParts; ++w) rank += part[w][lane];
    a.sorted[rank] = k;
    a.sorted_idx[rank] = idx;
  }
}

// ---- keys and ranks in one kernel, for pools of at most kRunsMaxN ---------

// A request's survivals never rise from one position to the next (each is the one before times a
// factor in [0, 1], rounded to nearest, which cannot exceed it), so its keys form an ascending
// run; a request with a bad confidence has kNoCandidate throughout, and once a survival reaches
// 0 the rest of the run is kNoCandidate too.  The place of candidate p = (request rp, position jp)
// in the pool sorted by (key, index) is then jp (the keys of its own run before it, ties broken by
// position) plus, for every other request r, the number of r's keys below key(p) + [r < rp],
// found by binary search in r's run.  Every workgroup rebuilds all keys in LDS from the
// confidences (the same products as keys_kernel) and places kRunsCand candidates, each with
// kRunsLanes threads that share out the other requests' runs.
constexpr int kRunsThreads = 512;
constexpr int kRunsLanes = 32;                           // threads per candidate
constexpr int kRunsCand = kRunsThreads / kRunsLanes;     // candidates per workgroup
constexpr int kRunsMaxN = 8192;                          // LDS words for the runs

// Whether the one-kernel sort serves a pool of B runs of gamma keys: the keys fit in LDS (each run
// gamma + 1 words apart when gamma is even, so that the stride is odd and threads reading the same
// place of consecutive runs meet no bank conflict) and each thread's binary searches stay few
// (B / kRunsLanes runs, floor(log2 gamma) + 1 steps each).
inline bool runs_sort_fits(int B, int gamma) {
  const int steps = 32 - __builtin_clz((unsigned)gamma);
  return (long long)B * (gamma | 1) <= kRunsMaxN && (long long)B * steps <= 128ll * kRunsLanes;
}

__global__ __launch_bounds__(kRunsThreads) void runs_rank_kernel(SchedArgs a) {
  __shared__ unsigned keys[kRunsMaxN + 1];   // the last word: a spare slot for discarded keys
  const int B = a.B, G = a.G, N = B * G;
  const int RS = G | 1;   // LDS stride of a run: G, or G + 1 when G is even
  const int tid = threadIdx.x;
  // the confidences, every thread's loads in flight together; candidate x = r G + j goes to
  // r RS + j, with r = floor(x / G) as the high word of x * ceil(2^32 / G) (exact: x (G - 1) < 2^32;
  // odd G, G = 1 among them, keeps x in place)
  {
    constexpr int PER = kRunsMaxN / kRunsThreads;
    const unsigned magic = G > 1 ? (unsigned)((0x100000000ull + (unsigned)G - 1) / (unsigned)G) : 0u;
    float cv[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int x = tid + e * kRunsThreads;
      cv[e] = x < N ? a.conf[x] : 0.f;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int x = tid + e * kRunsThreads;
      const int r = (int)__umulhi((unsigned)x, magic);
      if (x < N) keys[x + r * (RS - G)] = __float_as_uint(cv[e]);
    }
  }
  __syncthreads();
  // each request's run of keys, in place, sixteen confidences at a time (without branches: reads
  // past the run repeat its last word, and keys past it go to a spare slot)
  for (int r = tid; r < B; r += kRunsThreads) {
    unsigned* run = keys + r * RS;
    bool bad = false;
    float sv = 0.f;
    for (int t0 = 0; t0 < G; t0 += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = __uint_as_float(run[min(t0 + u, G - 1)]);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const bool in = t0 + u < G;
        bad |= in && !(v[u] >= 0.f && v[u] <= 1.f);
        const float nx = (t0 + u == 0) ? v[u] : __fmul_rn(sv, v[u]);
        sv = in ? nx : sv;
        keys[in ? r * RS + t0 + u : kRunsMaxN] = surv_key(sv);
      }
    }
    if (bad)
      for (int t = 0; t < G; ++t) run[t] = kNoCandidate;
    if (blockIdx.x == 0 && a.status) a.status[r] = bad ? SPEC_REQ_BAD_CONFIDENCE : 0;
  }
  __syncthreads();
  const int c = tid / kRunsLanes, t = tid % kRunsLanes;
  const int p = blockIdx.x * kRunsCand + c;
  const bool valid = p < N;
  const int pc = valid ? p : 0;
  const int rp = pc / G, jp = pc - rp * G;
  const unsigned kp = keys[rp * RS + jp];
  // run r's keys that precede p: those <= kp when r < rp (ties go to the lower index), else those
  // < kp, i.e. <= kp - 1 (no key is 0: a key is ~bits of a positive float, or kNoCandidate)
  const unsigned lim_lo = kp, lim_hi = kp - 1u;
  // binary lifting: the count n of keys <= lim in a sorted run is built from the powers of two
  // below 2^steps > G, adding h when key n + h - 1 is still <= lim
  const int top = 1 << (31 - __clz(G));   // the largest power of two <= G
  constexpr int S = 8;                    // searches in flight per thread
  int cnt = 0;
  for (int r0 = t; r0 < B; r0 += kRunsLanes * S) {
    int base[S], n[S];
    unsigned lim[S];
#pragma unroll
    for (int u = 0; u < S; ++u) {
      // a run not to count searches run 0 with limit 0, which no key is at or below
      const int r = r0 + u * kRunsLanes;
      const bool on = r < B && r != rp;
      base[u] = on ? r * RS : 0;
      n[u] = 0;
      lim[u] = on ? (r < rp ? lim_lo : lim_hi) : 0u;
    }
    for (int h = top; h > 0; h >>= 1) {
      unsigned v[S];
#pragma unroll
      for (int u = 0; u < S; ++u) v[u] = keys[base[u] + min(n[u] + h, G) - 1];
#pragma unroll
      for (int u = 0; u < S; ++u) n[u] += (n[u] + h <= G && v[u] <= lim[u]) ? h : 0;
    }
#pragma unroll
    for (int u = 0; u < S; ++u) cnt += n[u];
  }
#pragma unroll
  for (int o = kRunsLanes / 2; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, SPEC_WAVE);
  const int rank = jp + cnt;   // below N: each run counts at most its G keys
  if (t == 0 && valid && rank < N) {
    a.sorted[rank] = kp;
    a.sorted_idx[rank] = (unsigned)p;
  }
}

// ---- Theta path and lengths -----------------------------------------------

template <int K>
struct FinalShared {
  unsigned cnt[K * kFinalThreads];      // per-request admitted counts (B <= N <= K * kFinalThreads)
  long long wsum[kFinalWaves];
  double wth[kFinalWaves];
  int wm[kFinalWaves];
  int wbm[kFinalWaves];
  int wn[kFinalWaves];
  int mstar;
};

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.  Called once per
// kernel (wsum is written without a barrier before it).
__device__ __forceinline__ long long block_exclusive_sum(long long x, long long* wsum, long long* total) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const long long incl = wave_inclusive_sum_i64(x, lane);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  long long before = 0, all = 0;
  for (int w = 0; w < kFinalWaves; ++w) {
    before += (w < wave) ? wsum[w] : 0;
    all += wsum[w];
  }
  *total = all;
  return before + incl - x;
}

// K consecutive words from src + p0 (p0 a multiple of K, src 256-byte aligned), as 16-byte loads
// when K >= 4; words at or past n read as `fill`.
template <int K>
__device__ __forceinline__ void load_words(const unsigned* src, int p0, int n, unsigned fill, unsigned (&w)[K]) {
  if (p0 + K <= n) {
    if constexpr (K >= 4) {
#pragma unroll
      for (int e = 0; e < K; e += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + p0 + e);
        w[e] = v.x; w[e + 1] = v.y; w[e + 2] = v.z; w[e + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < K; ++e) w[e] = src[p0 + e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < K; ++e) w[e] = (p0 + e < n) ? src[p0 + e] : fill;
  }
}

static_assert(kFinalThreads == kWorklistThreads, "one thread per request in the combined call");

// WL: also build the verify work list of v from the lengths (B <= kFinalThreads).
template <int K, bool WL>
__global__ __launch_bounds__(kFinalThreads) void final_kernel(SchedArgs a, VerifyArgs v) {
  __shared__ FinalShared<K> sh;
  __shared__ WorklistShared wsh;
  // the verify work list's draft tokens, fetched with the keys (the largest tile fetches them at
  // the end: its registers are taken)
  constexpr bool kEarlyTokens = WL && K <= 8;
  int xp[kWlPre];
  if constexpr (kEarlyTokens) worklist_prefetch(v, xp);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int B = a.B, G = a.G;
  const int N = B * G;
  // SPS entries of this thread's admissions, fetched with the keys
  int m_cap = a.budget - B;
  m_cap = m_cap < 0 ? 0 : (m_cap > N ? N : m_cap);
  const int p0 = tid * K;
  const bool topk = a.mode == kSchedTopK;   // no cost table: the capacity is given
  const double sps_B = topk ? 0.0 : a.sps[B];
  const double sps_p0 = (!topk && p0 <= m_cap) ? a.sps[B + p0] : 0.0;
  double sps_m[K];
#pragma unroll
  for (int e = 0; e < K; ++e) sps_m[e] = (!topk && p0 + e + 1 <= m_cap) ? a.sps[B + p0 + e + 1] : 0.0;
  // this thread's sorted positions p0 .. p0 + K - 1: keys, and candidate indices (fetched with the
  // keys up to four per thread; the larger tiles fetch them once m* is known: their registers are
  // taken)
  constexpr bool kEarlyIdx = K <= 4;
  unsigned key[K], idx[K];
  load_words<K>(a.sorted, p0, N, kNoCandidate, key);
  if constexpr (kEarlyIdx) load_words<K>(a.sorted_idx, p0, N, 0u, idx);
  int nvalid = 0;
#pragma unroll
  for (int e = 0; e < K; ++e) nvalid += key[e] != kNoCandidate;
  nvalid = wave_sum_i(nvalid);
  if (lane == 0) sh.wn[wave] = nvalid;
  for (int r = tid; r < B; r += kFinalThreads) sh.cnt[r] = 0;
  __syncthreads();
  int E = 0;   // candidates in the pool
#pragma unroll
  for (int w = 0; w < kFinalWaves; ++w) E += sh.wn[w];
  long long q[K];
  long long tau_p0 = 0;
  int mstar;
  if (topk) {
    if (tid == 0) {
      const int cap = *a.capacity_in;
      sh.mstar = cap < 0 ? 0 : (cap > E ? E : cap);
    }
#pragma unroll
    for (int e = 0; e < K; ++e) q[e] = 0;
    __syncthreads();
    mstar = sh.mstar;
  } else {
  int m_max = a.budget - B;
  if (m_max > E) m_max = E;
  if (m_max < 0) m_max = 0;

  // exclusive scan of q over sorted positions 0 .. m_max-1 (K per thread)
  long long local = 0;
#pragma unroll
  for (int e = 0; e < K; ++e) {
    q[e] = (p0 + e < m_max) ? fixed_q(key_surv(key[e])) : 0;
    local += q[e];
  }
  long long total;
  const long long before = block_exclusive_sum(local, sh.wsum, &total);
  long long tau = (long long)B * kOne + before;  // tau at m = p0
  tau_p0 = tau;

  // Theta along the path; admission m uses sorted position m-1
  const double th0 = theta_of((long long)B * kOne, sps_B);
  int brk = 0x7fffffff;           // first m >= 1 with Theta(m) <= Theta(m-1)
  double best = -INFINITY;        // global: max Theta over this thread's m
  int best_m = 0x7fffffff;
  double tp = (p0 < m_max) ? theta_of(tau, sps_p0) : 0.0;
#pragma unroll
  for (int e = 0; e < K; ++e) {
    const int m = p0 + e + 1;
    if (m <= m_max) {
      tau += q[e];
      const double tm = theta_of(tau, sps_m[e]);
      if (!(tm > tp) && m < brk) brk = m;
      if (tm > best) {
        best = tm;
        best_m = m;
      }
      tp = tm;
    }
  }
  // block reductions: the early stop needs the first break, the global search the first maximum
  // (arrays of their own, so no barrier separates them from the scan's); every thread then
  // reads the waves' results and finds m* itself
  if (a.mode == SPEC_SCHED_EARLY_STOP) {
    const int wb = wave_min_i(brk);
    if (lane == 0) sh.wm[wave] = wb;
  } else {
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
    if (lane == 0) {
      sh.wth[wave] = wbest;
      sh.wbm[wave] = wbm;
    }
  }
  __syncthreads();
  if (a.mode == SPEC_SCHED_EARLY_STOP) {
    int b = 0x7fffffff;
#pragma unroll
    for (int w = 0; w < kFinalWaves; ++w) b = min(b, sh.wm[w]);
    mstar = (b == 0x7fffffff) ? m_max : b - 1;
  } else {
    double bt = th0;
    int bm = 0;
#pragma unroll
    for (int w = 0; w < kFinalWaves; ++w) {
      const double t = sh.wth[w];
      const int m = sh.wbm[w];
      if (t > bt || (t == bt && m < bm)) {
        bt = t;
        bm = m;
      }
    }
    mstar = bm;
  }
  if (tid == 0 && mstar == 0 && a.theta) a.theta[0] = th0;
  }  // search for m*
  if (tid == 0 && a.capacity_out) a.capacity_out[0] = mstar;
  if (!a.lengths) return;
  // Theta at m*: the thread holding sorted position m*-1 recomputes tau from its chunk
  if (!topk && mstar > 0 && mstar - 1 >= p0 && mstar - 1 < p0 + K && a.theta) {
    long long t = tau_p0;
    double sp = 0.0;
#pragma unroll
    for (int e = 0; e < K; ++e) {
      if (p0 + e < mstar) t += q[e];
      if (p0 + e + 1 == mstar) sp = sps_m[e];
    }
    a.theta[0] = theta_of(t, sp);
  }
  // The admitted candidates are the first m* of the pool sorted by (key, index): each request's
  // length is its count among them.
  if constexpr (!kEarlyIdx) load_words<K>(a.sorted_idx, p0, N, 0u, idx);
#pragma unroll
  for (int e = 0; e < K; ++e) {
    const int p = p0 + e;
    if (p < mstar) atomicAdd(&sh.cnt[idx[e] / (unsigned)G], 1u);
  }
  __syncthreads();
  int my_len = 0;   // request tid's length (B <= kFinalThreads)
  for (int r = tid; r < B; r += kFinalThreads) {
    const int len = (int)sh.cnt[r];
    a.lengths[r] = len;
    if (r == tid) my_len = len;
  }
  if constexpr (WL) {
    if constexpr (!kEarlyTokens) worklist_prefetch(v, xp);
    // the schedule admits at most budget - B candidates, so with budget >= B the lengths keep
    // sum (L_i + 1) within the budget and the work list's token cap drops nothing: it is skipped
    VerifyArgs vw = v;
    if (!topk && a.budget >= B) vw.max_items = 0;
    worklist_from_lengths(wsh, vw, my_len, xp);
  }
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

template <bool WL>
void launch_final(const SchedArgs& a, const VerifyArgs& v, int n, hipStream_t s) {
  const dim3 g(1), b(kFinalThreads);
  if (n <= 1 * kFinalThreads) hipLaunchKernelGGL((final_kernel<1, WL>), g, b, 0, s, a, v);
  else if (n <= 2 * kFinalThreads) hipLaunchKernelGGL((final_kernel<2, WL>), g, b, 0, s, a, v);
  else if (n <= 4 * kFinalThreads) hipLaunchKernelGGL((final_kernel<4, WL>), g, b, 0, s, a, v);
  else if (n <= 8 * kFinalThreads) hipLaunchKernelGGL((final_kernel<8, WL>), g, b, 0, s, a, v);
  else hipLaunchKernelGGL((final_kernel<16, WL>), g, b, 0, s, a, v);
}

}  // namespace spec

using namespace spec;

extern "C" size_t spec_schedule_workspace_size(int32_t B, int32_t gamma) {
  if (B < 1 || gamma < 1) return 0;
  const size_t n = (size_t)B * (size_t)gamma;
  return 4 * align256(n * sizeof(unsigned));
}

// v: the bound arguments of a verify call whose work list the final kernel writes, or NULL.
static int32_t launch_schedule(SchedArgs a, void* workspace, size_t workspace_bytes, hipStream_t s,
                               const VerifyArgs* v = nullptr) {
  const int B = a.B, gamma = a.G;
  if (!workspace || workspace_bytes < spec_schedule_workspace_size(B, gamma) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return SPEC_ERR_WORKSPACE;
  const int n = B * gamma;
  char* ws = static_cast<char*>(workspace);
  const size_t seg = align256((size_t)n * sizeof(unsigned));
  a.chunked = reinterpret_cast<unsigned*>(ws);
  a.chunked_idx = reinterpret_cast<unsigned*>(ws + seg);
  a.sorted = reinterpret_cast<unsigned*>(ws + 2 * seg);
  a.sorted_idx = reinterpret_cast<unsigned*>(ws + 3 * seg);
  if (runs_sort_fits(B, gamma)) {
    hipLaunchKernelGGL(runs_rank_kernel, dim3((n + kRunsCand - 1) / kRunsCand), dim3(kRunsThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(keys_kernel, dim3((n + kKeysThreads - 1) / kKeysThreads), dim3(kKeysThreads), 0, s, a);
    hipLaunchKernelGGL(rank_kernel, dim3((n + kChunk - 1) / kChunk), dim3(kChunk * kRankParts), 0, s, a);
  }
  if (v) launch_final<true>(a, *v, n, s);
  else launch_final<false>(a, VerifyArgs{}, n, s);
  return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

static int32_t check_search_args(int32_t B, int32_t gamma, const float* conf, const double* sps, int32_t sps_len,
                                 int32_t budget_tokens) {
  if (B < 1 || gamma < 1 || gamma > SPEC_MAX_GAMMA) return SPEC_ERR_INVALID_ARG;
  if ((long long)B * gamma > SPEC_MAX_SCHED_CANDIDATES) return SPEC_ERR_UNSUPPORTED;
  if (!conf || !sps) return SPEC_ERR_INVALID_ARG;
  long long m_cap = (long long)budget_tokens - B;
  if (m_cap < 0) m_cap = 0;
  if (m_cap > (long long)B * gamma) m_cap = (long long)B * gamma;
  if ((long long)sps_len <= (long long)B + m_cap) return SPEC_ERR_INVALID_ARG;
  return SPEC_OK;
}

extern "C" int32_t spec_schedule_lengths(int32_t B, int32_t gamma, const float* conf, const double* sps,
                                         int32_t sps_len, int32_t budget_tokens, int32_t mode,
                                         int32_t* lengths_out, double* theta_out, int32_t* status,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  const int32_t rc = check_search_args(B, gamma, conf, sps, sps_len, budget_tokens);
  if (rc != SPEC_OK) return rc;
  if (mode != SPEC_SCHED_EARLY_STOP && mode != SPEC_SCHED_GLOBAL) return SPEC_ERR_INVALID_ARG;
  if (!lengths_out) return SPEC_ERR_INVALID_ARG;
  SchedArgs a{B, gamma, budget_tokens, mode, conf, sps, lengths_out, theta_out, status,
              nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  return launch_schedule(a, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int32_t spec_schedule_capacity(int32_t B, int32_t gamma, const float* conf, const double* sps,
                                          int32_t sps_len, int32_t budget_tokens, int32_t* capacity_out,
                                          double* theta_out, int32_t* status, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  const int32_t rc = check_search_args(B, gamma, conf, sps, sps_len, budget_tokens);
  if (rc != SPEC_OK) return rc;
  if (!capacity_out) return SPEC_ERR_INVALID_ARG;
  SchedArgs a{B, gamma, budget_tokens, SPEC_SCHED_GLOBAL, conf, sps, nullptr, theta_out, status,
              nullptr, nullptr, nullptr, nullptr, nullptr, capacity_out};
  return launch_schedule(a, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int32_t spec_schedule_topk(int32_t B, int32_t gamma, const float* conf, const int32_t* capacity,
                                      int32_t* lengths_out, int32_t* status, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (B < 1 || gamma < 1 || gamma > SPEC_MAX_GAMMA) return SPEC_ERR_INVALID_ARG;
  if ((long long)B * gamma > SPEC_MAX_SCHED_CANDIDATES) return SPEC_ERR_UNSUPPORTED;
  if (!conf || !capacity || !lengths_out) return SPEC_ERR_INVALID_ARG;
  SchedArgs a{B, gamma, 0, kSchedTopK, conf, nullptr, lengths_out, nullptr, status,
              nullptr, nullptr, nullptr, nullptr, capacity, nullptr};
  return launch_schedule(a, workspace, workspace_bytes, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int32_t spec_schedule_verify(int32_t B, int32_t gamma, int32_t V, int32_t dtype, const float* conf,
                                        const double* sps, int32_t sps_len, int32_t budget_tokens, int32_t mode,
                                        const void* target_logits, const void* draft_logits,
                                        const int32_t* draft_tokens, const float* temperature,
                                        const int32_t* top_k, const uint64_t* seed, int32_t* lengths_out,
                                        double* theta_out, int32_t* sched_status, int32_t* num_accepted,
                                        int32_t* out_tokens, float* accept_prob, int32_t* status,
                                        void* sched_workspace, size_t sched_workspace_bytes,
                                        void* verify_workspace, size_t verify_workspace_bytes, void* stream,
                                        void* event_before, void* event_after) {
  int32_t rc = check_search_args(B, gamma, conf, sps, sps_len, budget_tokens);
  if (rc != SPEC_OK) return rc;
  const bool ltr = (mode & SPEC_VERIFY_LEFT_TO_RIGHT) != 0;
  mode &= ~SPEC_VERIFY_LEFT_TO_RIGHT;
  if (mode != SPEC_SCHED_EARLY_STOP && mode != SPEC_SCHED_GLOBAL) return SPEC_ERR_INVALID_ARG;
  if (budget_tokens < 1 || !lengths_out) return SPEC_ERR_INVALID_ARG;
  if (!shape_ok(B, gamma, V, dtype)) return SPEC_ERR_INVALID_ARG;
  if (!target_logits || !draft_logits || !draft_tokens || !temperature || !seed || !num_accepted || !out_tokens)
    return SPEC_ERR_INVALID_ARG;
  if (!aligned16(target_logits) || !aligned16(draft_logits)) return SPEC_ERR_INVALID_ARG;
  const bool fuse = B <= kFinalThreads;
  // batches the fused emit serves (every compute unit gets a request) and a streaming workgroup's
  // threads can cover (two requests each): no work list at all, the streaming workgroups derive
  // their items from the lengths and the status words the scheduler's last kernel writes
  const bool derive = fuse && B >= kFuseMinRequests && B <= 2 * kStreamThreads && gamma < SPEC_WAVE;
  // the left-to-right walk runs where the request-major work list and the fused emit do, on rows
  // without top-k; a budget below B (requests dropped by the token cap) is left out too
  if (ltr && (!derive || top_k || budget_tokens < B)) return SPEC_ERR_UNSUPPORTED;
  VerifyArgs v{};
  v.B = B; v.G = gamma; v.V = V; v.greedy_only = 0;
  v.target = target_logits; v.draft = draft_logits; v.tokens = draft_tokens; v.lengths = lengths_out;
  v.temperature = temperature; v.top_k = top_k; v.seed = seed;
  v.num_accepted = num_accepted; v.out_tokens = out_tokens; v.accept_prob = accept_prob; v.status = status;
  v.max_items = budget_tokens;   // the schedule keeps sum (L_i + 1) within it unless the budget is below B
  rc = bind_workspace(v, dtype, verify_workspace, verify_workspace_bytes, 0, nullptr);
  if (rc != SPEC_OK) return rc;
  SchedArgs a{B, gamma, budget_tokens, mode, conf, sps, lengths_out, theta_out, sched_status,
              nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  v.derive_items = derive ? 1 : 0;
  if (ltr) {
    v.ltr = 1;
    v.phase_cap = ltr_first_pass(gamma, v.nseg);
  }
  rc = launch_schedule(a, sched_workspace, sched_workspace_bytes, s, fuse ? &v : nullptr);
  if (rc != SPEC_OK) return rc;
  v.wl_ready = fuse ? 1 : 0;
  if (ltr) return launch_verify_ltr(v, dtype, s, event_before, event_after);
  return launch_verify_bound(v, dtype, s, event_before, event_after);
}
