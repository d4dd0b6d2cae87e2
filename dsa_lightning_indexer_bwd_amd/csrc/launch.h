// Internal interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace ibwd {

constexpr int64_t kMaxHeads = 64;

// One validated backward call.  Pointers are device pointers; shapes follow
// the public header.  For the dense variant ids == nullptr and row_len == S_k.
struct Problem {
  const uint16_t* q;    // [B,S_q,H,D] bf16 bits
  const uint16_t* k;    // [B,S_k,D] bf16 bits
  const float* w;       // [B,S_q,H]
  const int32_t* ids;   // [B,S_q,row_len] (sparse) or nullptr (dense)
  const float* I;       // [B,S_q,row_len]
  const float* p;       // [B,S_q,row_len]
  float* dq;            // [B,S_q,H,D]
  float* dw;            // [B,S_q,H]
  float* dk;            // [B,S_k,D]
  int64_t B, S_q, S_k, H, D, row_len;
  bool dense;
  int64_t q_offset;
  float sm_scale, grad_loss;
  bool deterministic;
  void* workspace;
};

// Workspace of the deterministic route: a 256-byte header (the magnitude
// bound) followed by one int64 fixed-point accumulator per d_k element.
constexpr size_t kDetHeaderBytes = 256;
inline size_t det_workspace_bytes(int64_t B, int64_t S_k, int64_t D) {
  return kDetHeaderBytes + size_t(B) * size_t(S_k) * size_t(D) * sizeof(int64_t);
}

// Enqueue the whole backward on `stream`.  Returns the first HIP error.
hipError_t launch(const Problem& P, hipStream_t stream);

// The MFMA main kernel (one wave per query row); d_k must already be zeroed
// (or the deterministic workspace prepared).
hipError_t launch_mfma(const Problem& P, hipStream_t stream);

}  // namespace ibwd
