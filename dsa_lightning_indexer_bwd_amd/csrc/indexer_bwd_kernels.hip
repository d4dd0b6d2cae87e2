// Kernels of the lightning-indexer backward for gfx950.
//
// Per query row t (NVIDIA/cudnn-frontend PR #730, harness `ref_grads` and the
// kernel-1 score-gradient contract):
//   dI_j   = grad_loss*sm_scale*(softmax_V(sm_scale*I)_j - p_j), 0 on padding
//   S[h,j] = q[t,h,:].k[id_j,:];  G[h,j] = dI_j*w[t,h]*[S>0]
//   dW[t,h] = sum_j dI_j*relu(S[h,j]);  dQ[t,h,:] = sum_j G[h,j]*k[id_j,:]
//   dK[id_j,:] += sum_h G[h,j]*q[t,h,:]
//
// This file holds the row-wise kernel: one workgroup per query row, the row's
// softmax statistics reduced in the workgroup, then 32-slot chunks of the row
// staged in LDS (K rows, G), dQ accumulated in registers in a fixed order, dW
// reduced across lanes in a fixed order, and dK scattered with fp32 atomics
// (or, on the deterministic route, int64 fixed-point atomics).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "launch.h"

namespace ibwd {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 32;  // slots per LDS chunk
constexpr int kMaxAcc = (kMaxHeads * 128) / kThreads;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Fixed-order workgroup reductions (4 waves).
__device__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wid] = v;
  __syncthreads();
  float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}
__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wid] = v;
  __syncthreads();
  float r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

struct RowView {
  const float* I;
  const float* p;
  const int32_t* ids;
  int64_t n;      // slots to visit
  int64_t t;
  __device__ int64_t key(const Problem& P, int64_t j) const {
    if (P.dense) return j;  // j < n already enforces j <= t + q_offset
    const int32_t id = ids[j];
    return (id >= 0 && id < P.S_k) ? int64_t(id) : int64_t(-1);
  }
};

__device__ RowView row_view(const Problem& P, int64_t r) {
  RowView v;
  v.t = r % P.S_q;
  v.I = P.I + r * P.row_len;
  v.p = P.p + r * P.row_len;
  v.ids = P.dense ? nullptr : P.ids + r * P.row_len;
  if (P.dense) {
    const int64_t last = v.t + P.q_offset;
    v.n = last < 0 ? 0 : (last + 1 < P.S_k ? last + 1 : P.S_k);
  } else {
    v.n = P.row_len;
  }
  return v;
}

// Fixed-point scale exponent of the deterministic route, from the bound that
// the bound kernel left in the workspace header: every partial sum of a d_k
// element stays below 2^62 in magnitude.
__device__ __forceinline__ int det_exponent(const void* ws, int64_t S_q) {
  const float rmax = __uint_as_float(*static_cast<const volatile uint32_t*>(ws));
  const double bound = 2.0 * double(rmax) * double(S_q);
  if (!(bound > 0.0)) return 62;
  int e = 0;
  frexp(bound, &e);  // bound < 2^e
  int F = 62 - e;
  return F < -100 ? -100 : (F > 100 ? 100 : F);
}

template <bool DET>
__global__ __launch_bounds__(kThreads) void rowwise_bwd_kernel(Problem P) {
  extern __shared__ float smem[];
  const int H = int(P.H), D = int(P.D);
  float* q_s = smem;                     // [H*D]
  float* k_s = q_s + H * D;              // [kChunk*D]
  float* g_s = k_s + kChunk * D;         // [H*kChunk]
  float* dI_s = g_s + H * kChunk;        // [kChunk]
  int64_t* key_s = reinterpret_cast<int64_t*>(dI_s + kChunk);  // [kChunk]
  float* dw_s = reinterpret_cast<float*>(key_s + kChunk);      // [H]
  float* red = dw_s + kMaxHeads;                               // [8]

  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const int64_t b = r / P.S_q;
  const RowView row = row_view(P, r);

  // ---- softmax statistics of the row over its valid slots -----------------
  float m = -INFINITY;
  for (int64_t j = tid; j < row.n; j += kThreads)
    if (row.key(P, j) >= 0) m = fmaxf(m, P.sm_scale * row.I[j]);
  m = block_max(m, red);
  float Z = 0.f;
  if (m > -INFINITY)
    for (int64_t j = tid; j < row.n; j += kThreads)
      if (row.key(P, j) >= 0) Z += expf(P.sm_scale * row.I[j] - m);
  Z = block_sum(Z, red);
  const float invZ = Z > 0.f ? 1.f / Z : 0.f;
  const float coef = P.grad_loss * P.sm_scale;

  const uint16_t* qrow = P.q + r * P.H * P.D;
  for (int e = tid; e < H * D; e += kThreads) q_s[e] = bf16_bits_to_f32(qrow[e]);
  for (int h = tid; h < kMaxHeads; h += kThreads) dw_s[h] = 0.f;
  const float* wrow = P.w + r * P.H;
  const uint16_t* kb = P.k + b * P.S_k * P.D;

  int F = 0;
  double fx_scale = 0.0;
  unsigned long long* acc64 = nullptr;
  if (DET) {
    F = det_exponent(P.workspace, P.S_q);
    fx_scale = ldexp(1.0, F);
    acc64 = reinterpret_cast<unsigned long long*>(static_cast<char*>(P.workspace) +
                                                  kDetHeaderBytes);
  }

  float acc[kMaxAcc];
#pragma unroll
  for (int i = 0; i < kMaxAcc; ++i) acc[i] = 0.f;

  for (int64_t j0 = 0; j0 < row.n; j0 += kChunk) {
    const int cnt = int(row.n - j0 < kChunk ? row.n - j0 : kChunk);
    __syncthreads();  // previous chunk fully consumed
    if (tid < kChunk) {
      const int64_t kk = tid < cnt ? row.key(P, j0 + tid) : -1;
      key_s[tid] = kk;
      float dI = 0.f;
      if (kk >= 0) dI = coef * (expf(P.sm_scale * row.I[j0 + tid] - m) * invZ - row.p[j0 + tid]);
      dI_s[tid] = dI;
    }
    __syncthreads();
    for (int e = tid; e < kChunk * D; e += kThreads) {
      const int jj = e / D, d = e % D;
      const int64_t kk = key_s[jj];
      k_s[e] = kk >= 0 ? bf16_bits_to_f32(kb[kk * P.D + d]) : 0.f;
    }
    __syncthreads();
    // S, G and the dW terms: lanes jj = 0..31 of a half-wave share one head
    for (int e = tid; e < H * kChunk; e += kThreads) {
      const int h = e / kChunk, jj = e % kChunk;
      float S = 0.f;
      for (int d = 0; d < D; ++d) S = fmaf(q_s[h * D + d], k_s[jj * D + d], S);
      const bool valid = key_s[jj] >= 0;
      const float dI = dI_s[jj];
      g_s[e] = (valid && S > 0.f) ? dI * wrow[h] : 0.f;
      float term = valid ? dI * fmaxf(S, 0.f) : 0.f;
      for (int o = 16; o > 0; o >>= 1) term += __shfl_xor(term, o, 64);
      if (jj == 0) dw_s[h] += term;  // one writer per head per chunk
    }
    __syncthreads();
    // dQ[h,d] += sum_jj G[h,jj] * K[jj,d], fixed order
#pragma unroll
    for (int i = 0; i < kMaxAcc; ++i) {
      const int e = tid + i * kThreads;
      if (e < H * D) {
        const int h = e / D, d = e % D;
        float a = acc[i];
        for (int jj = 0; jj < cnt; ++jj) a = fmaf(g_s[h * kChunk + jj], k_s[jj * D + d], a);
        acc[i] = a;
      }
    }
    // dK[id_jj, d] += sum_h G[h,jj] * q[h,d]
    for (int e = tid; e < cnt * D; e += kThreads) {
      const int jj = e / D, d = e % D;
      const int64_t kk = key_s[jj];
      if (kk < 0) continue;
      float c = 0.f;
      for (int h = 0; h < H; ++h) c = fmaf(g_s[h * kChunk + jj], q_s[h * D + d], c);
      const int64_t off = (b * P.S_k + kk) * P.D + d;
      if (DET) {
        const long long v = llrint(double(c) * fx_scale);
        atomicAdd(acc64 + off, static_cast<unsigned long long>(v));
      } else {
        unsafeAtomicAdd(P.dk + off, c);
      }
    }
  }
  __syncthreads();
  float* dqrow = P.dq + r * P.H * P.D;
#pragma unroll
  for (int i = 0; i < kMaxAcc; ++i) {
    const int e = tid + i * kThreads;
    if (e < H * D) dqrow[e] = acc[i];
  }
  for (int h = tid; h < H; h += kThreads) P.dw[r * P.H + h] = dw_s[h];
}

__global__ void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

// Deterministic route, pass 0: per row R = |grad_loss*sm_scale| * (1 + sum_V |p|)
// * max_d sum_h |w[h]*q[h,d]| bounds that row's contribution to any d_k element
// (sum_V |dI| <= |grad_loss*sm_scale| * (sum_V P + sum_V |p|)).  The maximum
// over rows goes to the workspace header (atomicMax on non-negative float bits
// is order independent).
__global__ __launch_bounds__(kThreads) void det_bound_kernel(Problem P) {
  __shared__ float red[8];
  __shared__ float colmax[128];
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const RowView row = row_view(P, r);
  float ps = 0.f;
  for (int64_t j = tid; j < row.n; j += kThreads)
    if (row.key(P, j) >= 0) ps += fabsf(row.p[j]);
  ps = block_sum(ps, red);
  const uint16_t* qrow = P.q + r * P.H * P.D;
  const float* wrow = P.w + r * P.H;
  if (tid < P.D) {
    float s = 0.f;
    for (int h = 0; h < P.H; ++h) s += fabsf(wrow[h] * bf16_bits_to_f32(qrow[h * P.D + tid]));
    colmax[tid] = s;
  }
  __syncthreads();
  if (tid == 0) {
    float mx = 0.f;
    for (int d = 0; d < P.D; ++d) mx = fmaxf(mx, colmax[d]);
    float R = fabsf(P.grad_loss * P.sm_scale) * (1.f + ps) * mx;
    if (!(R <= 3.0e38f)) R = 3.0e38f;  // inf / nan -> huge finite
    atomicMax(static_cast<uint32_t*>(P.workspace), __float_as_uint(R));
  }
}

// Deterministic route, last pass: d_k = acc * 2^-F.
__global__ void det_finalize_kernel(Problem P, int64_t n) {
  const int F = det_exponent(P.workspace, P.S_q);
  const double inv = ldexp(1.0, -F);
  const long long* acc = reinterpret_cast<const long long*>(
      static_cast<const char*>(P.workspace) + kDetHeaderBytes);
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    P.dk[i] = float(double(acc[i]) * inv);
}

size_t rowwise_smem_bytes(const Problem& P) {
  return sizeof(float) * size_t(P.H * P.D + kChunk * P.D + P.H * kChunk + kChunk) +
         sizeof(int64_t) * kChunk + sizeof(float) * (kMaxHeads + 8);
}

}  // namespace

hipError_t launch(const Problem& P, hipStream_t stream) {
  const int64_t rows = P.B * P.S_q;
  const int64_t dk_elems = P.B * P.S_k * P.D;
  const int fill_blocks = 1024;
  hipError_t err;
  if (P.deterministic) {
    const int64_t words = int64_t(det_workspace_bytes(P.B, P.S_k, P.D) / 4);
    zero_u32_kernel<<<fill_blocks, 256, 0, stream>>>(static_cast<uint32_t*>(P.workspace), words);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    det_bound_kernel<<<dim3(unsigned(rows)), kThreads, 0, stream>>>(P);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = launch_mfma(P, stream)) != hipSuccess) return err;
    det_finalize_kernel<<<fill_blocks, 256, 0, stream>>>(P, dk_elems);
    return hipGetLastError();
  }
  zero_u32_kernel<<<fill_blocks, 256, 0, stream>>>(reinterpret_cast<uint32_t*>(P.dk), dk_elems);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return launch_mfma(P, stream);
}

}  // namespace ibwd
