// MFMA kernel of the lightning-indexer backward for gfx950 (one wave per
// query row).
//
// Math per query row t (NVIDIA/cudnn-frontend PR #730: the harness' fp64
// `ref_grads` and the kernel-1 score-gradient contract; PR #549: dK is an fp32
// atomic scatter-add):
//   dI_j    = grad_loss*sm_scale*(softmax_V(sm_scale*I)_j - p_j)   (0 on padding)
//   S[h,j]  = q[t,h,:] . k[id_j,:]
//   G'[h,j] = dI_j * [S[h,j] > 0]          (G = w[t,h] * G')
//   dW[t,h] = sum_j G'[h,j] * S[h,j]       (= sum_j dI_j * relu(S))
//   dQ[t,h,:] = w[t,h] * sum_j G'[h,j] * k[id_j,:]
//   dK[id_j,:] += sum_h G'[h,j] * (w[t,h] * q[t,h,:])
//
// Work decomposition: a wave owns one query row; the row's slots are walked in
// chunks of 32.  Per chunk three bf16 MFMA products run on v_mfma_f32_32x32x16_bf16:
//   GEMM1  S^T[j,h]  = K_g[j,:] . Q[h,:]          M=j(32)  N=h  K=d
//   GEMM2  dQ'[h,d] += G'[h,j] K_g[j,d]           M=h      N=d  K=j(32)
//   GEMM3  C[j,d]    = G'[h,j] Q'[h,d]            M=j(32)  N=d  K=h
// GEMM1's output layout (lane = h, registers = j) is exactly GEMM2's A-operand
// layout, so G' never leaves registers for GEMM2.  GEMM2 needs K_g with j as
// the register axis and GEMM3 needs G' with h as the register axis; both are
// read back transposed from wave-private LDS tiles.  Q (and Q' = w*q rounded to
// bf16) are per-row register-resident operands.  dQ' accumulates in registers
// across all chunks; C goes straight from the accumulators to dK with fp32
// atomics, 32 consecutive floats (one 128-byte line) per half-wave.
//
// MFMA 32x32x16 bf16 lane layouts (verified on the device):
//   A[m][k]: lane l holds m = l%32, k = 8*(l/32) + e, e = 0..7
//   B[k][n]: lane l holds n = l%32, k = 8*(l/32) + e
//   D[m][n]: lane l holds n = l%32, m = 8*i + 4*(l/32) + r at register 4*i + r
// The reduction index may be permuted freely as long as A and B agree.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "launch.h"

namespace ibwd {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSlots = 32;  // slots per chunk (the MFMA M/K extent)

__device__ __forceinline__ f32x16_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;  // round to nearest even
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// ds_read_b64_tr_b16 (gfx950 LDS transpose read).  Within each 16-lane group,
// source lane s reads 4 consecutive bf16 at its own address; the result of lane
// i, element e is source lane (4e + i/4)'s element (i%4) (measured on the
// device).  So if source lane s points at row (row0 + s/4), columns
// col0 + 4*(s%4) .. +3 of a row-major bf16 tile, lane i receives the column
// col0 + i of rows row0 .. row0+3: a 4 x 16 block read transposed.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_tr4(const unsigned char* tile, int pitch, int row0, int col0) {
  const int s = threadIdx.x & 15;
  const unsigned char* a = tile + (row0 + (s >> 2)) * pitch + (col0 + 4 * (s & 3)) * 2;
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(a));
  return __builtin_bit_cast(uint2, v);
}
// B/A operand of 8 consecutive k (rows k0 .. k0+3 and k0+4 .. k0+7, split as
// rows [r0, r0+4) and [r1, r1+4)) at column col0 + (lane % 16).
__device__ __forceinline__ u32x4_t lds_tr8(const unsigned char* tile, int pitch, int r0, int r1,
                                           int col0) {
  const uint2 x = lds_tr4(tile, pitch, r0, col0);
  const uint2 y = lds_tr4(tile, pitch, r1, col0);
  return u32x4_t{x.x, x.y, y.x, y.y};
}

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// Order the wave's own LDS traffic: the compiler must not move LDS accesses
// across this point (lanes exchange data through LDS; the hardware keeps one
// wave's LDS operations in order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int det_exponent_mfma(const void* ws, int64_t S_q) {
  const float rmax = __uint_as_float(*static_cast<const volatile uint32_t*>(ws));
  const double bound = 2.0 * double(rmax) * double(S_q);
  if (!(bound > 0.0)) return 62;
  int e = 0;
  frexp(bound, &e);
  int F = 62 - e;
  return F < -100 ? -100 : (F > 100 ? 100 : F);
}

template <int D>
struct Lds {
  static constexpr int kPitch = D * 2 + 16;        // bytes per K / Q row (bank spread)
  static constexpr int kGPitch = kSlots * 2 + 8;   // bytes per G' row
  static constexpr int kKBuf = kSlots * kPitch;     // one K chunk
  static constexpr int kQBuf = 64 * kPitch;         // Q staging at row start (aliases K)
  static constexpr int kKArea = (2 * kKBuf > kQBuf) ? 2 * kKBuf : kQBuf;
  static constexpr int kGOff = kKArea;
  static constexpr int kStageOff = kGOff + 64 * kGPitch;
  static constexpr int kStages = 4;
  static constexpr int kStageBytes = kSlots * 8;    // dI (fp32) + key (int32)
  static constexpr int kBytes = kStageOff + kStages * kStageBytes;
};

// One query row per wave.  NH: 32-head tiles (H padded to 32*NH), D: head dim.
template <int NH, int D, bool DENSE, bool DET>
__global__ __launch_bounds__(64, 1) void mfma_row_kernel(Problem P) {
  constexpr int ND = D / 32;   // 32-wide d tiles (GEMM2/3 N)
  constexpr int KD = D / 16;   // 16-deep d steps (GEMM1 K)
  constexpr int KH = NH * 2;   // 16-deep h steps (GEMM3 K)
  using L = Lds<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[L::kBytes];

  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int H = int(P.H);

  // rows are visited longest-first for the dense variant
  const int64_t r = DENSE ? (P.B * P.S_q - 1 - int64_t(blockIdx.x)) : int64_t(blockIdx.x);
  const int64_t b = r / P.S_q;
  const int64_t t = r % P.S_q;
  int64_t n = P.row_len;
  if (DENSE) {
    const int64_t last = t + P.q_offset;
    n = last < 0 ? 0 : (last + 1 < P.S_k ? last + 1 : P.S_k);
  }
  const float* Irow = P.I + r * P.row_len;
  const float* prow = P.p + r * P.row_len;
  const int32_t* idrow = DENSE ? nullptr : P.ids + r * P.row_len;
  const uint16_t* kb = P.k + b * P.S_k * D;
  float* dkb = P.dk + b * P.S_k * D;
  const int S_k = int(P.S_k);

  auto key_of = [&](int64_t j) -> int {
    if (j >= n) return -1;
    if (DENSE) return int(j);
    const int id = idrow[j];
    return (id >= 0 && id < S_k) ? id : -1;
  };

  // ---- softmax statistics over the valid slots (online max / sum) ----------
  float m = -INFINITY, z = 0.f;
  for (int64_t j = lane; j < n; j += 64) {
    if (key_of(j) < 0) continue;
    const float v = P.sm_scale * Irow[j];
    if (v > m) {
      z = z * expf(m - v) + 1.f;
      m = v;
    } else {
      z += expf(v - m);
    }
  }
  {
    const float mw = wave_max(m);
    z = (m > -INFINITY) ? z * expf(m - mw) : 0.f;
    z = wave_sum(z);
    m = mw;
  }
  const float invZ = z > 0.f ? 1.f / z : 0.f;
  const float coef = P.grad_loss * P.sm_scale;

  // ---- per-row operands ------------------------------------------------------
  // w for the heads this lane owns in GEMM1's output (h = l32 + 32*nt)
  const float* wrow = P.w + r * P.H;
  float wv[NH];
#pragma unroll
  for (int nt = 0; nt < NH; ++nt) {
    const int h = l32 + 32 * nt;
    wv[nt] = h < H ? wrow[h] : 0.f;
  }
  // GEMM1 B operand: Q^T, lane holds q[h = l32+32nt][d = 8*half + 16*kd + e]
  u32x4_t qb1[NH][KD];
  const uint16_t* qrow = P.q + r * P.H * D;
#pragma unroll
  for (int nt = 0; nt < NH; ++nt) {
    const int h = l32 + 32 * nt;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      if (h < H) {
        qb1[nt][kd] = *reinterpret_cast<const u32x4_t*>(qrow + h * D + 8 * half + 16 * kd);
      } else {
        qb1[nt][kd] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }
  // GEMM3 B operand: Q'[h][d] = bf16(w_h*q[h][d]), lane holds d = l32 + 32*nd and
  // h = 16*ks + 8*half + e.  Staged through LDS (rows h, pitch kPitch).
  u32x4_t qb3[ND][KH];
  {
    unsigned char* qs = lds;
#pragma unroll
    for (int nt = 0; nt < NH; ++nt) {
      const int h = l32 + 32 * nt;
#pragma unroll
      for (int kd = 0; kd < KD; ++kd) {
        const u32x4_t v = qb1[nt][kd];
        u32x4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = pack_bf16(wv[nt] * bf16_lo(v[e]), wv[nt] * bf16_hi(v[e]));
        *reinterpret_cast<u32x4_t*>(qs + h * L::kPitch + (8 * half + 16 * kd) * 2) = o;
      }
    }
    wave_lds_sync();
    // lane: d = 32*nd + l32 (16-lane group g: columns 32*nd + 16*(g%2) + i),
    // h = 16*ks + 8*half + e
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      const int col0 = 32 * nd + 16 * ((lane >> 4) & 1);
#pragma unroll
      for (int ks = 0; ks < KH; ++ks) {
        const int r0 = 16 * ks + 8 * half;
        qb3[nd][ks] = lds_tr8(qs, L::kPitch, r0, r0 + 4, col0);
      }
    }
    wave_lds_sync();
  }

  // deterministic route: fixed-point scale
  float fx_scale = 0.f;
  if (DET) fx_scale = ldexpf(1.f, det_exponent_mfma(P.workspace, P.S_q));
  unsigned long long* acc64 =
      DET ? reinterpret_cast<unsigned long long*>(static_cast<char*>(P.workspace) +
                                                  kDetHeaderBytes) + b * P.S_k * D
          : nullptr;

  // ---- per-chunk staging: dI and key of 32 slots -> LDS ring ----------------
  const int nchunks = int((n + kSlots - 1) / kSlots);
  auto stage_ptr = [&](int c) -> unsigned char* {
    return lds + L::kStageOff + (c & (L::kStages - 1)) * L::kStageBytes;
  };
  auto stage_chunk = [&](int c) {
    if (c >= nchunks) return;
    if (lane < kSlots) {
      const int64_t j = int64_t(c) * kSlots + lane;
      const int key = key_of(j);
      float dI = 0.f;
      if (key >= 0) dI = coef * (expf(P.sm_scale * Irow[j] - m) * invZ - prow[j]);
      float* sd = reinterpret_cast<float*>(stage_ptr(c));
      int* sk = reinterpret_cast<int*>(stage_ptr(c) + kSlots * 4);
      sd[lane] = dI;
      sk[lane] = key;
    }
  };
  // K rows of one chunk: lane holds row j = l32, d = 8*half + 16*kd + e
  auto gather = [&](int c, u32x4_t (&kr)[KD]) {
    const int* sk = reinterpret_cast<const int*>(stage_ptr(c) + kSlots * 4);
    const int key = sk[l32];
    const uint16_t* src = kb + int64_t(key < 0 ? 0 : key) * D + 8 * half;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + 16 * kd);
      kr[kd] = key < 0 ? u32x4_t{0u, 0u, 0u, 0u} : v;
    }
  };
  auto kbuf = [&](int c) -> unsigned char* { return lds + (c & 1) * L::kKBuf; };
  auto store_k = [&](int c, const u32x4_t (&kr)[KD]) {
    unsigned char* kbp = kbuf(c);
#pragma unroll
    for (int kd = 0; kd < KD; ++kd)
      *reinterpret_cast<u32x4_t*>(kbp + l32 * L::kPitch + (8 * half + 16 * kd) * 2) = kr[kd];
  };

  f32x16_t dqacc[NH][ND];
#pragma unroll
  for (int nt = 0; nt < NH; ++nt)
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) dqacc[nt][nd] = f32x16_t{};
  float dw_acc[NH];
#pragma unroll
  for (int nt = 0; nt < NH; ++nt) dw_acc[nt] = 0.f;

  u32x4_t kcur[KD];
  if (nchunks > 0) {
    stage_chunk(0);
    stage_chunk(1);
    wave_lds_sync();
    gather(0, kcur);
    store_k(0, kcur);
    wave_lds_sync();
  }

  unsigned char* gs = lds + L::kGOff;
  for (int c = 0; c < nchunks; ++c) {
    // prefetch: rows of chunk c+1 (keys staged one chunk ahead), slots of c+2
    u32x4_t knext[KD];
    const bool more = c + 1 < nchunks;
    if (more) gather(c + 1, knext);
    stage_chunk(c + 2);

    const unsigned char* kc = kbuf(c);
    // ---- GEMM1: S^T[j][h] over d --------------------------------------------
    f32x16_t s[NH];
#pragma unroll
    for (int nt = 0; nt < NH; ++nt) s[nt] = f32x16_t{};
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      const u32x4_t a =
          *reinterpret_cast<const u32x4_t*>(kc + l32 * L::kPitch + (8 * half + 16 * kd) * 2);
#pragma unroll
      for (int nt = 0; nt < NH; ++nt) s[nt] = mfma(a, qb1[nt][kd], s[nt]);
    }

    // ---- G' = dI*[S>0], dW, bf16 packing ------------------------------------
    // lane: h = l32 + 32*nt; register 4*i + rr <-> slot j = 8*i + 4*half + rr
    const float* sd = reinterpret_cast<const float*>(stage_ptr(c));
    const int* sk = reinterpret_cast<const int*>(stage_ptr(c) + kSlots * 4);
    float dIv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(sd + 8 * i + 4 * half);
      dIv[i][0] = v.x;
      dIv[i][1] = v.y;
      dIv[i][2] = v.z;
      dIv[i][3] = v.w;
    }
    uint32_t gp[NH][4][2];
#pragma unroll
    for (int nt = 0; nt < NH; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float g[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float sv = s[nt][4 * i + rr];
          g[rr] = sv > 0.f ? dIv[i][rr] : 0.f;
          dw_acc[nt] = fmaf(g[rr], sv, dw_acc[nt]);
        }
        gp[nt][i][0] = pack_bf16(g[0], g[1]);
        gp[nt][i][1] = pack_bf16(g[2], g[3]);
        // G' tile in LDS: row h, slots 8*i + 4*half .. +3
        *reinterpret_cast<uint2*>(gs + (l32 + 32 * nt) * L::kGPitch + (8 * i + 4 * half) * 2) =
            make_uint2(gp[nt][i][0], gp[nt][i][1]);
      }
    }

    // ---- GEMM2: dQ'[h][d] += G'[h][j] K[j][d] --------------------------------
    // k-step ks covers slots 16*ks + {0..15}; register e of lane (half) is slot
    // 16*ks + 8*(e/4) + 4*half + e%4 (GEMM1's output order).
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        // lane: d = 32*nd + l32, slots 16*ks + 4*half + {0..3} and +8
        const int col0 = 32 * nd + 16 * ((lane >> 4) & 1);
        const int r0 = 16 * ks + 4 * half;
        const u32x4_t bop = lds_tr8(kc, L::kPitch, r0, r0 + 8, col0);
#pragma unroll
        for (int nt = 0; nt < NH; ++nt) {
          const u32x4_t aop = u32x4_t{gp[nt][2 * ks][0], gp[nt][2 * ks][1], gp[nt][2 * ks + 1][0],
                                      gp[nt][2 * ks + 1][1]};
          dqacc[nt][nd] = mfma(aop, bop, dqacc[nt][nd]);
        }
      }
    }

    wave_lds_sync();  // G' tile complete

    // ---- GEMM3: C[j][d] = G'^T[j][h] Q'[h][d], then the dK scatter ------------
    // A operand: lane j = l32, h = 16*ks + 8*half + e (the order qb3 was built in)
    u32x4_t ga[KH];
#pragma unroll
    for (int ks = 0; ks < KH; ++ks) {
      const int r0 = 16 * ks + 8 * half;
      ga[ks] = lds_tr8(gs, L::kGPitch, r0, r0 + 4, 16 * ((lane >> 4) & 1));
    }
    int keys[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int4 v = *reinterpret_cast<const int4*>(sk + 8 * i + 4 * half);
      keys[i][0] = v.x;
      keys[i][1] = v.y;
      keys[i][2] = v.z;
      keys[i][3] = v.w;
    }
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      f32x16_t cacc = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < KH; ++ks) cacc = mfma(ga[ks], qb3[nd][ks], cacc);
      const int d = l32 + 32 * nd;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int key = keys[i][rr];
          if (key >= 0) {
            const float v = cacc[4 * i + rr];
            if (DET) {
              const long long fx = __float2ll_rn(v * fx_scale);
              atomicAdd(acc64 + key * D + d, static_cast<unsigned long long>(fx));
            } else {
              unsafeAtomicAdd(dkb + key * D + d, v);
            }
          }
        }
      }
    }

    // ---- next chunk's K rows into the other LDS buffer -----------------------
    if (more) store_k(c + 1, knext);
    wave_lds_sync();
  }

  // ---- row epilogue: dQ = w * dQ', dW ---------------------------------------
  float* dqrow = P.dq + r * P.H * D;
#pragma unroll
  for (int nt = 0; nt < NH; ++nt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int h = 32 * nt + 8 * i + 4 * half + rr;
        if (h < H) {
          const float wh = wrow[h];
#pragma unroll
          for (int nd = 0; nd < ND; ++nd) dqrow[h * D + l32 + 32 * nd] = wh * dqacc[nt][nd][4 * i + rr];
        }
      }
    }
  }
#pragma unroll
  for (int nt = 0; nt < NH; ++nt) {
    const float tot = dw_acc[nt] + __shfl_xor(dw_acc[nt], 32, 64);
    const int h = l32 + 32 * nt;
    if (half == 0 && h < H) P.dw[r * P.H + h] = tot;
  }
}

template <int NH, int D>
hipError_t launch_mfma_t(const Problem& P, hipStream_t stream) {
  const dim3 grid(unsigned(P.B * P.S_q));
  if (P.dense) {
    if (P.deterministic)
      mfma_row_kernel<NH, D, true, true><<<grid, 64, 0, stream>>>(P);
    else
      mfma_row_kernel<NH, D, true, false><<<grid, 64, 0, stream>>>(P);
  } else {
    if (P.deterministic)
      mfma_row_kernel<NH, D, false, true><<<grid, 64, 0, stream>>>(P);
    else
      mfma_row_kernel<NH, D, false, false><<<grid, 64, 0, stream>>>(P);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma(const Problem& P, hipStream_t stream) {
  const bool two = P.H > 32;
  switch (P.D) {
    case 32:
      return two ? launch_mfma_t<2, 32>(P, stream) : launch_mfma_t<1, 32>(P, stream);
    case 64:
      return two ? launch_mfma_t<2, 64>(P, stream) : launch_mfma_t<1, 64>(P, stream);
    case 128:
      return two ? launch_mfma_t<2, 128>(P, stream) : launch_mfma_t<1, 128>(P, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace ibwd
