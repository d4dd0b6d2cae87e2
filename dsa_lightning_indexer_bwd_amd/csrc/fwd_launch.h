// Host-side description of the indexer forward-score and top-k launches.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ibwd {

// I[b,t,s] = sum_h w[b,t,h] * relu(q[b,t,h,:] . k[b,s,:]) for every key; with
// causal set, keys s > t + q_offset score -inf.
struct FwdProblem {
  const uint16_t* q;  // [B,S_q,H,D] bf16 bits
  const uint16_t* k;  // [B,S_k,D] bf16 bits
  const float* w;     // [B,S_q,H]
  float* scores;      // [B,S_q,S_k]
  int64_t B, S_q, S_k, H, D;
  bool causal;
  int64_t q_offset;
};

// Per row of scores: the min(topk, finite) largest finite scores, ties to the
// lower key id, listed by ascending key id; id -1 / value -inf after them.
struct TopkProblem {
  const float* scores;  // [rows, S_k]
  int32_t* ids;         // [rows, topk]
  float* vals;          // [rows, topk] or nullptr
  int64_t rows, S_k, topk;
};

hipError_t launch_fwd_scores(const FwdProblem& P, hipStream_t stream);
hipError_t launch_topk(const TopkProblem& P, hipStream_t stream);

}  // namespace ibwd
