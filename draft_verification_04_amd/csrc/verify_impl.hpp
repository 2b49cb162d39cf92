// Internal layout shared by the verification kernels and their host launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

struct VerifyArgs {
  int B, G, V;
  int greedy_only;
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
  int32_t* nitems;     // [1]
  int32_t* req_status; // [B] SPEC_REQ_* bits raised while streaming
};

constexpr int kStreamThreads = 512;
constexpr int kFinishThreads = 1024;
constexpr int kWorklistThreads = 1024;
constexpr int kTopkCap = 4096;   // top-k candidates kept in LDS per row
constexpr int kTopkPre = 4;      // vectors per thread sampled for the top-k lower bound

}  // namespace spec
