/*
 * spec_verify.h -- C ABI of libspecverify, lossless draft verification and
 * confidence-scheduled verify lengths on AMD Instinct MI355X (gfx950).
 *
 * The operations are those of speculative decoding as stated in the DSpark
 * paper ("DSpark: Confidence-Scheduled Speculative Decoding with
 * Semi-Autoregressive Generation"):
 *   - spec_verify            -- rejection-sampling verification of a block of
 *                               gamma draft tokens per request against target
 *                               logits (paper §2.1), plus the token the target
 *                               appends after the accepted prefix (paper §1),
 *                               a fresh target token when nothing is verified
 *                               (paper appendix counterexample);
 *   - spec_verify_greedy     -- the same block verified by the argmax rule;
 *   - spec_schedule_lengths  -- survival products of per-position confidences
 *                               and the budgeted length selector (paper
 *                               §3.2.2; Algorithm 1 of the paper's Chinese
 *                               translation; the no-break search of §5.2);
 *   - spec_draft_markov      -- the draft block itself: the Markov-head
 *                               sequential sampler and the confidence head
 *                               (paper §3.1, §3.2.1);
 *   - spec_sts_fit / _apply  -- Sequential Temperature Scaling of the
 *                               confidences (paper §3.2.1).
 *
 * Conventions shared by every entry point
 *   - Every array argument is a DEVICE pointer (hipMalloc'd or a torch CUDA
 *     tensor's storage).  Scalars are passed by value.  The caller owns all
 *     memory; the library keeps no state between calls and never allocates
 *     (spec_verify_static alone keeps its workspace in a device array of the
 *     library, see there).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it asynchronously; nothing synchronises the host.
 *   - Return value: SPEC_OK, or an error code returned synchronously before
 *     anything is enqueued (bad pointer, shape, dtype, alignment, workspace)
 *     -- or SPEC_ERR_HIP if a launch itself failed.
 *   - Bad DATA (a draft token outside [0,V), a NaN/+inf logit in a needed
 *     row, a bad temperature, length or confidence) is not an error of the
 *     call: it is reported per request in `status` (SPEC_REQ_* bits) and
 *     that request gets num_accepted = 0, out_tokens = -1, accept_prob = NaN.
 *   - Two calls may run concurrently when they use different workspaces.
 *
 * Shapes (row-major, contiguous; B requests, gamma draft positions, vocabulary V):
 *   target_logits [B, gamma+1, V]  row k < gamma: target distribution at draft
 *                                   position k; row L: the row the appended
 *                                   token is drawn from when all L drafts pass
 *   draft_logits  [B, gamma, V]     draft distribution at position k
 *   draft_tokens  [B, gamma] int32  x_k, the draft token at position k
 *   lengths       [B] int32         verify length L_i in [0, gamma] (NULL = gamma)
 * Logits are fp32 or bf16 (spec_dtype); the base pointers must be 16-byte
 * aligned; any V >= 1 is accepted.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 3

/* Call status (return value of every entry point). */
enum {
    SPEC_OK = 0,
    SPEC_ERR_INVALID_ARG = 1, /* null pointer, size out of range, misalignment, bad enum */
    SPEC_ERR_WORKSPACE = 2,   /* workspace missing or smaller than the size query returned */
    SPEC_ERR_UNSUPPORTED = 3, /* a valid request this library does not support (e.g. V too large) */
    SPEC_ERR_HIP = 4          /* a HIP launch reported an error */
};

/* Logit element type. */
enum { SPEC_F32 = 0, SPEC_BF16 = 1 };

/* Scheduler mode. */
enum {
    SPEC_SCHED_EARLY_STOP = 0, /* admit while Theta rises strictly; stop at the first
                                  candidate that does not raise it (paper §3.2.2, Alg. 1) */
    SPEC_SCHED_GLOBAL = 1      /* smallest admitted count maximising Theta over the whole
                                  budget (the no-break search of paper §5.2) */
};

/* Verification order, OR-ed into the mode of spec_schedule_verify (DSpark paper §2.1: positions
   are verified left to right and the first rejection discards every later draft token). */
#define SPEC_VERIFY_LEFT_TO_RIGHT 0x100

/* Per-request data status bits (the `status` outputs). */
#define SPEC_REQ_BAD_TOKEN 1        /* a needed draft token outside [0, V) */
#define SPEC_REQ_BAD_TEMPERATURE 2  /* temperature negative, NaN or infinite */
#define SPEC_REQ_NONFINITE 4        /* NaN or +inf in a needed logit row */
#define SPEC_REQ_BAD_LENGTH 8       /* lengths[i] outside [0, gamma] */
#define SPEC_REQ_BAD_TOPK 16        /* top_k[i] < 0 */
#define SPEC_REQ_BAD_CONFIDENCE 32  /* scheduler: a confidence outside [0, 1] or NaN */
#define SPEC_REQ_OVER_BUDGET 64     /* spec_verify_bounded: the request's rows did not fit the token cap */
#define SPEC_REQ_BAD_ROWS 128      /* spec_verify_flat: the request's rows lie past the row counts passed */

/* Limits of this library. */
#define SPEC_MAX_GAMMA 64
#define SPEC_MAX_V 524288           /* bf16; fp32 rows are limited to SPEC_MAX_V / 2 */
#define SPEC_MAX_SCHED_CANDIDATES 16384 /* B * gamma for spec_schedule_lengths */

int32_t spec_abi_version(void);
const char* spec_status_string(int32_t status);

/*
 * spec_verify -- lossless rejection-sampling verification (paper §2.1).
 *
 * For request i with length L = lengths[i] (gamma if NULL), temperature
 * T = temperature[i], top-k K = top_k[i] (0 if NULL), seed s = seed[i]:
 *   p_t,k = softmax(target row k / T), p_d,k = softmax(draft row k / T), both
 *   restricted to the kept set when K > 0 (every v whose raw logit is >= the
 *   K-th largest raw logit of that row; ties kept; K >= V keeps all);
 *   for k = 0 .. L-1 in order: accept x_k iff u_acc(k) < min(1, p_t,k(x_k) /
 *   p_d,k(x_k)); the first rejection n ends the block (n = L if none);
 *   the emitted token is drawn by inverse CDF (ascending token id, smallest
 *   v with C(v) > u_emit(n) * W) from w = max(0, p_t,n - p_d,n) after a
 *   rejection, or from w = p_t,L (target row L) when all L drafts passed
 *   (with L = 0 this is a fresh token from target row 0).
 *   T = 0 selects the greedy rule of spec_verify_greedy for that request.
 * Draws: Philox4x64-10 (Salmon et al., SC'11), key (s, 0), block counter
 * (k + 1, i, 0, 0); u_acc(k) = word0 >> 11 scaled by 2^-53, u_emit(k) = word1
 * likewise.  The same seed and inputs give bitwise-identical outputs.
 *
 * Arguments
 *   B >= 1, 1 <= gamma <= SPEC_MAX_GAMMA, 1 <= V <= SPEC_MAX_V (fp32: V/2)
 *   dtype            SPEC_F32 or SPEC_BF16
 *   target_logits    [B, gamma+1, V]  (only rows k <= L_i are read)
 *   draft_logits     [B, gamma, V]    (only rows k < L_i are read)
 *   draft_tokens     [B, gamma] int32 (only k < L_i are read)
 *   lengths          [B] int32 or NULL
 *   temperature      [B] float32 (>= 0; 0 = greedy rule)
 *   top_k            [B] int32 or NULL
 *   seed             [B] uint64
 * Outputs (written for every request)
 *   num_accepted     [B] int32: n_i
 *   out_tokens       [B, gamma+1] int32: x_0 .. x_{n-1}, the emitted token, then -1
 *   accept_prob      [B, gamma] float32 or NULL: min(1, p_t/p_d) at x_k for every
 *                    k < L_i (also after the first rejection), NaN for k >= L_i;
 *                    greedy requests get 1 (match) or 0
 *   status           [B] int32 or NULL: SPEC_REQ_* bits, 0 when the data were valid
 * Workspace
 *   workspace        device scratch of at least spec_verify_workspace_size(B, gamma, V)
 *                    bytes, 256-byte aligned; owned by the caller; must not be used
 *                    by another call in flight.
 * Size limit
 *   SPEC_ERR_UNSUPPORTED (before anything is enqueued) when a launch would pass
 *   2^32 work-items: the row-streaming kernel runs one 512-thread workgroup per
 *   (row pair, segment of about 48 KB), so B * (gamma + 1) * max(1, V * elem /
 *   49152, at most 16) must stay below 2^23 (e.g. B = 500000, gamma = 16,
 *   V = 1000 fp32 is refused), and B below 2^22.
 */
size_t spec_verify_workspace_size(int32_t B, int32_t gamma, int32_t V);

int32_t spec_verify(int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                    const void* target_logits, const void* draft_logits,
                    const int32_t* draft_tokens, const int32_t* lengths,
                    const float* temperature, const int32_t* top_k, const uint64_t* seed,
                    int32_t* num_accepted, int32_t* out_tokens, float* accept_prob,
                    int32_t* status, void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_static -- spec_verify for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments, outputs, status words and results as
 * spec_verify, without the workspace arguments.  The workspace is a
 * file-scope device array of SPEC_STATIC_SCRATCH_BYTES bytes inside the
 * library; each GPU holds its own copy until the process ends.  The call
 * allocates nothing (no hipMalloc, no library allocation).
 *   - It runs on the calling thread's current device, which must be the
 *     device of `stream` and of every pointer.  The first call with a device
 *     current looks up that device's copy of the array (hipGetSymbolAddress)
 *     and keeps its address.
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (other streams, other threads) race and give wrong
 *     results.  Calls on one stream are ordered and safe.  The array keeps
 *     the last call's contents; the kernels write every word they read, so
 *     nothing needs clearing between calls.
 *   - SPEC_ERR_WORKSPACE, before any HIP call, when the shape needs more than
 *     SPEC_STATIC_SCRATCH_BYTES of workspace (spec_verify_workspace_size(B,
 *     gamma, V) > SPEC_STATIC_SCRATCH_BYTES; e.g. B = 256, gamma = 16,
 *     V = 151936 needs 30.2 MiB and B = 1024, gamma = 8, V = 129280 65 MiB).
 */
#define SPEC_STATIC_SCRATCH_BYTES (128u << 20)

int32_t spec_verify_static(int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                           const void* target_logits, const void* draft_logits,
                           const int32_t* draft_tokens, const int32_t* lengths,
                           const float* temperature, const int32_t* top_k, const uint64_t* seed,
                           int32_t* num_accepted, int32_t* out_tokens, float* accept_prob,
                           int32_t* status, void* stream);

/*
 * spec_verify_profiled -- spec_verify, with two caller-created hipEvent_t
 * (passed as void*) that take the start and end times of the dispatch of the
 * row-streaming kernel that reads the logits (hipExtLaunchKernel's events: no
 * separate marker is enqueued).  Either event may be NULL.  For measurement
 * only; results are identical to spec_verify.
 */
int32_t spec_verify_profiled(int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                             const void* target_logits, const void* draft_logits,
                             const int32_t* draft_tokens, const int32_t* lengths,
                             const float* temperature, const int32_t* top_k, const uint64_t* seed,
                             int32_t* num_accepted, int32_t* out_tokens, float* accept_prob,
                             int32_t* status, void* workspace, size_t workspace_bytes, void* stream,
                             void* event_before, void* event_after);

/*
 * spec_verify_bounded -- spec_verify under a token cap, with the optional events
 * of spec_verify_profiled.
 *   max_tokens  >= 1: the batch's token budget.  Requests are taken in index
 *               order, each with a valid length adding L_i + 1 to a running
 *               sum; the first one that takes the sum past max_tokens, and
 *               every later one with a valid length, get status
 *               SPEC_REQ_OVER_BUDGET (when no other SPEC_REQ_* bit applies) and
 *               the outputs of a failed request (num_accepted 0, out_tokens -1,
 *               accept_prob NaN); their rows are not read.  Lengths from spec_schedule_lengths with
 *               the same budget always fit, and then every output equals
 *               spec_verify's.  The cap sizes the grid of the row-streaming
 *               kernel, which otherwise holds B * (gamma + 1) items, most of
 *               them empty under a tight budget.
 * Everything else as for spec_verify_profiled; SPEC_ERR_INVALID_ARG when
 * max_tokens < 1.
 */
int32_t spec_verify_bounded(int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                            const void* target_logits, const void* draft_logits,
                            const int32_t* draft_tokens, const int32_t* lengths,
                            const float* temperature, const int32_t* top_k, const uint64_t* seed,
                            int32_t* num_accepted, int32_t* out_tokens, float* accept_prob,
                            int32_t* status, void* workspace, size_t workspace_bytes, void* stream,
                            int32_t max_tokens, void* event_before, void* event_after);

/*
 * spec_verify_flat -- spec_verify on the flattened variable-length layout in
 * which only the verified rows are stored, request after request (DSpark
 * paper, §5.3: every verified token of every request is one flat row):
 *   target_rows [sum_i (L_i + 1), V]: target rows 0 .. L_i of request i start
 *               at row T_i = sum_{j<i} (L_j + 1);
 *   draft_rows  [sum_i L_i, V]: draft rows 0 .. L_i - 1 of request i start at
 *               row D_i = sum_{j<i} L_j.
 * `lengths` is required (it defines the layout); a length outside [0, gamma]
 * makes that request BAD_LENGTH and counts as no rows.  The row offsets are
 * derived on the device.  target_row_count and draft_row_count (>= 0) are the
 * numbers of rows the two buffers hold: a request whose rows would lie past
 * either is not read and gets SPEC_REQ_BAD_ROWS (the lengths live on the
 * device, so the library cannot refuse the call up front without a sync).
 * Everything else -- arguments, outputs, status, workspace
 * (spec_verify_workspace_size), errors -- as for spec_verify, and the results
 * equal spec_verify's on the padded layout holding the same rows.
 */
int32_t spec_verify_flat(int32_t B, int32_t gamma, int32_t V, int32_t dtype, const void* target_rows,
                         int64_t target_row_count, const void* draft_rows, int64_t draft_row_count,
                         const int32_t* draft_tokens, const int32_t* lengths,
                         const float* temperature, const int32_t* top_k, const uint64_t* seed,
                         int32_t* num_accepted, int32_t* out_tokens, float* accept_prob, int32_t* status,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_greedy -- greedy verification, the argmax rule the DSpark paper
 * names beside rejection sampling in its related work (§6, parallel generation:
 * a drafter without exact per-token probabilities is limited to it).
 * a_k = argmax of raw target row k (lowest token id on ties); n = first
 * k < L_i with x_k != a_k, else L_i; out_tokens = x_0 .. x_{n-1}, a_n, then -1.
 * Draft logits are never read.  Arguments and outputs as for spec_verify (no
 * temperature, top-k or seed); the workspace is sized by
 * spec_verify_greedy_workspace_size.
 */
size_t spec_verify_greedy_workspace_size(int32_t B, int32_t gamma);

int32_t spec_verify_greedy(int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                           const void* target_logits, const int32_t* draft_tokens,
                           const int32_t* lengths, int32_t* num_accepted, int32_t* out_tokens,
                           int32_t* status, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * spec_schedule_lengths -- confidence-scheduled verify lengths (paper §3.2.2).
 *
 *   a_{i,j} = c_{i,0} * ... * c_{i,j} (float32, left to right);
 *   candidates (i, j) with a_{i,j} > 0, sorted by a descending, then i, then j;
 *   admitting the first m gives batch tokens B + m and expected accepted tokens
 *   tau(m) = B + sum of their survivals, held in fixed point with 47 fractional
 *   bits (each survival floored to a multiple of 2^-47; tau < 2^16 always fits);
 *   Theta(m) = fp64(tau(m)) * 2^-47 * sps[B + m];
 *   m ranges over 0 .. min(#candidates, budget_tokens - B);
 *   EARLY_STOP: m* = last m before the first Theta(m+1) <= Theta(m);
 *   GLOBAL: m* = the smallest m maximising Theta.
 *   lengths_out[i] = number of request i's candidates among the first m*.
 *
 * Arguments
 *   B >= 1, 1 <= gamma <= SPEC_MAX_GAMMA, B * gamma <= SPEC_MAX_SCHED_CANDIDATES
 *   conf          [B, gamma] float32 device, each in [0, 1]
 *   sps           [sps_len] float64 device: engine throughput in steps/s for a
 *                 forward batch of b tokens at index b (the profiled cost table)
 *   sps_len       must exceed min(budget_tokens, B * (gamma + 1))
 *   budget_tokens cap on batch tokens B + m (values below B admit nothing)
 *   mode          SPEC_SCHED_EARLY_STOP or SPEC_SCHED_GLOBAL
 * Outputs
 *   lengths_out   [B] int32 device
 *   theta_out     [1] float64 device or NULL: Theta(m*)
 *   status        [B] int32 device or NULL: SPEC_REQ_BAD_CONFIDENCE when a
 *                 confidence of that request is outside [0, 1] or NaN; such a
 *                 request contributes no candidate (its length is 0)
 *   workspace     at least spec_schedule_workspace_size(B, gamma) bytes (16 per
 *                 candidate, rounded up), 256-byte aligned, owned by the caller; it
 *                 carries the sort keys and their candidate indices between the
 *                 call's kernels and must not be
 *                 touched by other work until they finish on `stream`
 * Errors (nothing is launched): SPEC_ERR_INVALID_ARG for the conditions above,
 *   SPEC_ERR_UNSUPPORTED beyond SPEC_MAX_SCHED_CANDIDATES, SPEC_ERR_WORKSPACE for a
 *   missing, short or misaligned workspace.
 */
size_t spec_schedule_workspace_size(int32_t B, int32_t gamma);

int32_t spec_schedule_lengths(int32_t B, int32_t gamma, const float* conf, const double* sps,
                              int32_t sps_len, int32_t budget_tokens, int32_t mode,
                              int32_t* lengths_out, double* theta_out, int32_t* status,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_schedule_verify -- one step of the scheduled path (paper §3.2.2, then
 * §2.1): spec_schedule_lengths followed by spec_verify_bounded on the lengths
 * it selects, with the budget as the token cap, enqueued as one call.
 *   Scheduler arguments (conf, sps, sps_len, budget_tokens, mode) and outputs
 *   (lengths_out [B] required, theta_out or NULL, sched_status [B] or NULL) as
 *   for spec_schedule_lengths; budget_tokens >= 1.  Verify arguments (V, dtype,
 *   target_logits, draft_logits, draft_tokens, temperature, top_k, seed) and
 *   outputs (num_accepted, out_tokens, accept_prob, status) as for spec_verify,
 *   with lengths = lengths_out; event_before / event_after as for
 *   spec_verify_profiled.
 *   Workspaces: sched_workspace of spec_schedule_workspace_size(B, gamma) bytes
 *   and verify_workspace of spec_verify_workspace_size(B, gamma, V) bytes, both
 *   256-byte aligned, distinct, owned by the caller.
 *   Every output equals that of the two calls made one after the other on the
 *   same stream.  With B <= 1024 the scheduler's last kernel also writes the
 *   verify work list (one kernel fewer).
 * Left to right (mode | SPEC_VERIFY_LEFT_TO_RIGHT; DSpark paper §2.1: positions
 *   are verified in order and the first rejection discards every later draft):
 *   each request's verification is the walk k = 0, 1, ... that stops at the
 *   first rejection n, so rows after n are never examined.  num_accepted,
 *   out_tokens and the drawn tokens are those of the call without the flag;
 *   accept_prob is min(1, p_t/p_d) for k <= n (k < L) and NaN after n; status
 *   NONFINITE is raised only for a bad row the walk reaches (target and draft
 *   rows 0 .. n, target row L when every draft passed).  The argument checks
 *   (length, temperature, every draft token k < L) stay up front.  The rows are
 *   streamed in two passes: positions 0 .. c-1 of every request (c = 3, at most
 *   gamma, and 2 when a row spans more than 8 of the streaming kernel's ~48 KB
 *   segments), then positions c .. L of the requests whose walk passed all of
 *   them; rows after an earlier rejection are not read.  Supported for 256 <= B <= 1024, gamma < 64,
 *   top_k == NULL and budget_tokens >= B; else SPEC_ERR_UNSUPPORTED before
 *   anything is enqueued.
 * Errors: those of the two calls, checked before anything is enqueued.
 */
int32_t spec_schedule_verify(int32_t B, int32_t gamma, int32_t V, int32_t dtype, const float* conf,
                             const double* sps, int32_t sps_len, int32_t budget_tokens, int32_t mode,
                             const void* target_logits, const void* draft_logits,
                             const int32_t* draft_tokens, const float* temperature, const int32_t* top_k,
                             const uint64_t* seed, int32_t* lengths_out, double* theta_out,
                             int32_t* sched_status, int32_t* num_accepted, int32_t* out_tokens,
                             float* accept_prob, int32_t* status, void* sched_workspace,
                             size_t sched_workspace_bytes, void* verify_workspace,
                             size_t verify_workspace_bytes, void* stream, void* event_before,
                             void* event_after);

/*
 * Asynchronous scheduling (DSpark paper, §5.2): the admission capacity of a
 * step is fixed from confidences predicted two steps earlier (the global
 * search, without the early-stop break), and the step then admits its current
 * candidates, sorted by their up-to-date survival, up to that capacity -- a
 * rank-preserving top-K selection.  The capacity never sees the current
 * tokens, so admission stays non-anticipating.
 *
 * spec_schedule_capacity -- the global search of spec_schedule_lengths
 *   (mode SPEC_SCHED_GLOBAL) on `conf` (the earlier step's confidences);
 *   writes K = m*, the number of candidates it admits, to capacity_out [1]
 *   int32 device, and Theta(m*) to theta_out [1] or NULL.  Arguments, status
 *   and errors as for spec_schedule_lengths (no lengths are written).
 *
 * spec_schedule_topk -- lengths_out [B] int32 device: request i's share of
 *   the first min(K, #candidates) candidates of `conf` in sorted order (the
 *   order of spec_schedule_lengths), K = capacity [1] int32 device (written
 *   by an earlier spec_schedule_capacity, or by the caller; negative = 0).
 *   No cost table and no budget: the capacity carries both.  status [B] or
 *   NULL as for spec_schedule_lengths.  Workspace:
 *   spec_schedule_workspace_size(B, gamma) bytes for either call.
 */
int32_t spec_schedule_capacity(int32_t B, int32_t gamma, const float* conf, const double* sps,
                               int32_t sps_len, int32_t budget_tokens, int32_t* capacity_out,
                               double* theta_out, int32_t* status, void* workspace,
                               size_t workspace_bytes, void* stream);

int32_t spec_schedule_topk(int32_t B, int32_t gamma, const float* conf, const int32_t* capacity,
                           int32_t* lengths_out, int32_t* status, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * spec_philox_uniforms -- the library's draws, exposed for checking:
 * for t < n, (u_accept[t], u_emit[t]) = the two uniforms used for request
 * request[t] at draft position position[t] under seed[t] (see spec_verify).
 * All arrays device, length n.
 */
int32_t spec_philox_uniforms(int32_t n, const uint64_t* seed, const int32_t* request,
                             const int32_t* position, double* u_accept, double* u_emit,
                             void* stream);

/*
 * spec_overlap_mass -- per draft position, the overlap of the target and draft
 * distributions, c*_{i,k} = sum_v min(p_t,i,k(v), p_d,i,k(v)) (DSpark paper,
 * §3.2.1, Eq. 8: the probability that position k is accepted once it is
 * reached; the confidence head's label).  p = softmax(z / T_i) over the kept
 * set, exactly as in spec_verify.
 *
 * Arguments as for spec_verify (target [B, gamma+1, V] with row gamma unused,
 * draft [B, gamma, V], lengths or NULL, temperature, top_k or NULL); no draft
 * tokens and no seeds.
 * Outputs
 *   overlap_out [B, gamma] float64 device: c*_{i,k} for k < L_i; NaN for
 *               k >= L_i, for greedy requests (T_i = 0) and for requests with
 *               bad data.  Computed with fp32 probabilities summed in fp64:
 *               relative error ~1e-6.
 *   status      [B] int32 device or NULL: the spec_verify status bits (no token
 *               check).
 *   workspace   at least spec_overlap_workspace_size(B, gamma, V) bytes,
 *               256-byte aligned, owned by the caller, busy until the call's
 *               kernels finish on `stream`.
 * Cost: every row pair (target k, draft k), k < L_i, is read twice (row
 * statistics, then the overlap); the bonus rows are not read.
 * Errors as for spec_verify.
 */
size_t spec_overlap_workspace_size(int32_t B, int32_t gamma, int32_t V);

int32_t spec_overlap_mass(int32_t B, int32_t gamma, int32_t V, int32_t dtype, const void* target_logits,
                          const void* draft_logits, const int32_t* lengths, const float* temperature,
                          const int32_t* top_k, double* overlap_out, int32_t* status, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * spec_draft_markov -- the Markov-head sequential draft sampler and the
 * confidence head (DSpark paper, §3.1, Eq. 4 and Eq. 5; §3.2.1, Eq. 7).
 *
 * For each request i and k = 0 .. gamma-1 in order (x_{-1} = anchor[i]):
 *   z_k = U_k + W1[x_{k-1}] W2                  (Eq. 5: the Markov head's
 *         transition bias; the product is accumulated in fp32 from the bf16
 *         weights, U_k added in fp32, the sum rounded once to `dtype`, ties
 *         to even);
 *   x_k ~ softmax(z_k / T_i) over the whole vocabulary (Eq. 4): the smallest
 *         token v whose running sum of exp(z / T) in ascending token order
 *         exceeds u * total, u = word 0 of the Philox4x64-10 block at counter
 *         (k + 1, i, 1, 0) under key (seed_i, 0), as (w >> 11) * 2^-53 (the
 *         verifier's draws use counter word 2 = 0, so one seed may key both);
 *         T_i = 0: the first-occurrence argmax of z_k;
 *   conf_k = sigmoid(w . [h_k ; W1[x_{k-1}]] / tau_k)  (Eq. 7; tau_k the
 *         per-position temperature of Sequential Temperature Scaling, §3.2.1,
 *         1 without conf_tau), when `conf` is given.
 * The stored draft_logits rows ARE the draft distribution: hand them to
 * spec_verify (with the same temperatures and top_k = 0) and the pair is
 * lossless.  Sums are fp64 (exponentials evaluated in fp64 against exact
 * power-of-two references), so the drawn token is that of an exact
 * computation on the stored row except within ~1e-15 of a CDF boundary.
 *
 * Arguments
 *   B >= 1, 1 <= gamma <= SPEC_MAX_GAMMA, 1 <= V <= SPEC_MAX_V (fp32: V/2),
 *   r in {16, 32, ..., 256} (the paper's default is 256), d >= 0
 *   dtype         SPEC_BF16 or SPEC_F32: base_logits, draft_logits, hidden
 *   base_logits   [B, gamma, V] device: U_k from the parallel stage
 *   W1            [V, r] bf16 device: the Markov embedding table
 *   W2t           [V, r] bf16 device: the projection W2 (r x V) stored token-
 *                 major, row v = column v of W2
 *   anchor        [B] int32 device: x_{-1}, the last token of the previous
 *                 verification cycle
 *   temperature   [B] float32 device (0 = greedy)
 *   seed          [B] uint64 device, or NULL for all 0
 *   hidden        [B, gamma, d] device (dtype) or NULL when d = 0; conf_w
 *                 [d + r] float32 device: the confidence head's weight, the
 *                 first d entries against h_k; conf_tau [gamma] float64
 *                 device or NULL (spec_sts_fit's output); all ignored when
 *                 conf = NULL
 * Outputs (device)
 *   tokens        [B, gamma] int32: x_k (all -1 for a request with a status)
 *   draft_logits  [B, gamma, V] dtype: the stored z_k (may be base_logits
 *                 itself: each element is read before it is overwritten);
 *                 rows of a request with a status are not defined
 *   conf          [B, gamma] float32 or NULL: conf_k (NaN for a request with
 *                 a status), evaluated in fp64 and rounded
 *   status        [B] int32: SPEC_REQ_BAD_TEMPERATURE, SPEC_REQ_BAD_TOKEN
 *                 (anchor outside [0, V)), SPEC_REQ_NONFINITE (a stored row
 *                 with a NaN or +inf, or with no finite value)
 *   workspace     at least spec_draft_workspace_size(B, gamma, V) bytes,
 *                 256-byte aligned, owned by the caller, busy until the
 *                 call's kernels finish on `stream`.
 * base_logits, draft_logits, W1 and W2t must be 16-byte aligned.  The call
 * enqueues 2 gamma + 1 kernels; it never synchronises the host.
 * Errors: SPEC_ERR_INVALID_ARG (shape, r, dtype, null or misaligned pointer,
 * conf without conf_w or without hidden when d > 0), SPEC_ERR_WORKSPACE.
 */
size_t spec_draft_workspace_size(int32_t B, int32_t gamma, int32_t V);

int32_t spec_draft_markov(int32_t B, int32_t gamma, int32_t V, int32_t r, int32_t dtype,
                          const void* base_logits, const void* W1, const void* W2t,
                          const int32_t* anchor, const float* temperature, const uint64_t* seed,
                          int32_t d, const void* hidden, const float* conf_w, const double* conf_tau,
                          int32_t* tokens,
                          void* draft_logits, float* conf, int32_t* status, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * spec_sts_fit -- Sequential Temperature Scaling of the confidence head (DSpark
 * paper, §3.2.1, post-hoc calibration).  Per position k = 0 .. gamma-1 in
 * order, tau_k = the first grid value minimising the Expected Calibration
 * Error of the survival product a_k = prod_{i<=k} sigmoid(t_i / tau_i) over
 * the N held-out instances, the temperatures of earlier positions fixed.
 * ECE = (1/N) sum over `bins` equal-width bins of |sum_{n in bin} (a_n - y_n)|,
 * a value a falling in bin min(floor(a * bins), bins - 1).  Sums are fp64 in a
 * fixed order (the result does not depend on scheduling).
 *
 * Arguments (device pointers)
 *   1 <= N <= 2^26, 1 <= gamma <= SPEC_MAX_GAMMA, 1 <= ntau <= 4096, 1 <= bins <= 32
 *   conf_logits [N, gamma] float32: the head's logits t (before the sigmoid)
 *   labels      [N, gamma] uint8: nonzero when draft positions 0 .. k of the
 *               instance were all accepted (the event a_k predicts)
 *   taus        [ntau] float64: the grid (any values; a NaN result never wins)
 * Outputs (device)
 *   tau_out     [gamma] float64: tau_k (NaN when every ECE of position k is
 *               NaN -- a NaN logit makes its position's ECE NaN)
 *   index_out   [gamma] int32 or NULL: the grid index (-1 for NaN)
 *   ece_out     [gamma, ntau] float64 or NULL: the ECE of every grid value
 *   workspace   at least spec_sts_workspace_size(N, ntau, bins) bytes,
 *               256-byte aligned, owned by the caller.
 * Enqueues 4 gamma + 1 kernels on `stream`.  Errors: SPEC_ERR_INVALID_ARG,
 * SPEC_ERR_WORKSPACE.
 */
size_t spec_sts_workspace_size(int32_t N, int32_t ntau, int32_t bins);

int32_t spec_sts_fit(int32_t N, int32_t gamma, const float* conf_logits, const uint8_t* labels, int32_t ntau,
                     const double* taus, int32_t bins, double* tau_out, int32_t* index_out, double* ece_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_sts_apply -- calibrated confidences conf_out[i, k] = sigmoid(t[i, k] /
 * tau[k]) (fp64, rounded to float32) for B x gamma logits t (device float32),
 * tau [gamma] float64 device; the scheduler's input.  (spec_draft_markov
 * applies the same temperatures itself through conf_tau.)
 */
int32_t spec_sts_apply(int32_t B, int32_t gamma, const float* conf_logits, const double* tau, float* conf_out,
                       void* stream);

/*
 * spec_read_ceiling -- measurement aid, not part of verification: reads
 * floor(bytes / 16) 16-byte vectors starting at `data` once (nontemporal,
 * grid-stride over `grid` workgroups of 512 threads) so that a caller can time
 * the device's achievable HBM read rate on the same number of bytes the
 * streaming kernel reads.  `data` device, 16-byte aligned, at least `bytes`
 * long; `sink` [1] uint32 device, written only in a case that does not arise in
 * practice.  Asynchronous on `stream`.  SPEC_ERR_INVALID_ARG for a null or
 * misaligned pointer, bytes < 16 or grid outside [1, 2^20].
 */
int32_t spec_read_ceiling(const void* data, size_t bytes, int32_t grid, uint32_t* sink, void* stream);

/*
 * spec_left_to_right_first_pass -- the number of positions c that the first
 * streaming pass of a left-to-right spec_schedule_verify call (mode |
 * SPEC_VERIFY_LEFT_TO_RIGHT) reads for every request, for rows of V logits of
 * `dtype`: 3, at most gamma, and 2 when a row spans more than 8 of the
 * streaming kernel's ~48 KB segments.  A host-side query with no device work,
 * for callers that account for the rows a call reads (the second pass reads
 * positions c .. L of the requests whose walk passed all c).  0 for arguments
 * spec_verify would refuse.
 */
int32_t spec_left_to_right_first_pass(int32_t gamma, int32_t V, int32_t dtype);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
