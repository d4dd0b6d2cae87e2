// Row kernel of the lightning-indexer backward for gfx950: one wave per query
// row, bf16 MFMA for the score recompute and dQ.
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
// The wave walks its row in chunks of 32 slots:
//   GEMM1  S^T[j,h]  = K_g[j,:] . Q[h,:]     v_mfma 32x32x16, M=j N=h K=d
//   GEMM2  dQ'[h,d] += G'[h,j] K_g[j,d]      M=h N=d K=j
// GEMM1's accumulator layout (lane = h, registers = j) is GEMM2's A-operand
// layout, so G' stays in registers; GEMM2's B operand (K_g with j on the
// register axis) is read transposed from a wave-private LDS tile with
// ds_read_b64_tr_b16.  dQ' accumulates in registers over the whole row.
//
// dK (this file is the atomic route): GEMM3  C[j,d] = G'[h,j] Q'[h,d]
// (M=j N=d K=h, G' read transposed from LDS) and an fp32 atomic add of every C
// row into dK.  The two-pass route has its own row kernel.
//
// Loads are software-pipelined one chunk ahead: the slot data (ids, I, p) of
// chunk c+2 and the K rows of chunk c+1 are in flight while chunk c computes.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "device_common.h"
#include "launch.h"

namespace ibwd {
namespace {


template <int D>
struct RowLds {
  static constexpr int kPitch = D * 2 + 16;       // bytes per K / Q' row (bank spread)
  static constexpr int kGPitch = kSlots * 2 + 8;  // bytes per G' row
  static constexpr int kKBuf = kSlots * kPitch;   // one K chunk
  static constexpr int kQBuf = 64 * kPitch;       // Q' staging at row start (aliases K)
  static constexpr int kKArea = (2 * kKBuf > kQBuf) ? 2 * kKBuf : kQBuf;
  static constexpr int kGOff = kKArea;
  static constexpr int kStageOff = kGOff + 64 * kGPitch;
  static constexpr int kStageBytes = kSlots * 8;  // dI (fp32) + key (int32)
  static constexpr int kBytes = kStageOff + 2 * kStageBytes;
};

// Slot data of one chunk as loaded (lane l holds slot l%32).
struct Raw {
  int id;
  float I;
  float p;
};

template <int NH, int D, bool DENSE>
__global__ __launch_bounds__(64, 1) void row_kernel(Problem P) {
  constexpr int ND = D / 32;  // 32-wide d tiles
  constexpr int KD = D / 16;  // 16-deep d steps (GEMM1 K)
  constexpr int KH = NH * 2;  // 16-deep h steps (GEMM3 K)
  using L = RowLds<D>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[L::kBytes];

  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int H = int(P.H);

  // dense rows are visited longest first
  const int64_t r = DENSE ? (P.B * P.S_q - 1 - int64_t(blockIdx.x)) : int64_t(blockIdx.x);
  const int64_t b = r / P.S_q;
  const int64_t t = r % P.S_q;
  const int row_len = int(P.row_len);
  int n = row_len;
  if (DENSE) {
    const int64_t last = t + P.q_offset;
    n = last < 0 ? 0 : int(last + 1 < P.S_k ? last + 1 : P.S_k);
  }
  const float* Irow = P.I + r * P.row_len;
  const float* prow = P.p + r * P.row_len;
  const int32_t* idrow = DENSE ? nullptr : P.ids + r * P.row_len;
  const uint16_t* kb = P.k + b * P.S_k * D;
  const int S_k = int(P.S_k);
  const int id_base = int(b) * P.id_batch_stride;

  auto key_of = [&](int j, int id) -> int {
    if (j >= n) return -1;
    if (DENSE) return j;
    return local_key(id, id_base, S_k);
  };

  // ---- softmax statistics over the valid slots ---------------------------------
  const float c2 = P.sm_scale * 1.4426950408889634f;  // base-2 logit scale
  const float2 st = row_softmax_stats(
      n, Irow, c2, [&](int j) { return DENSE ? 0 : idrow[j]; }, key_of, [](int, int, int) {});
  const float m2 = st.x, invZ = st.y;
  const float coef = P.grad_loss * P.sm_scale;

  // ---- per-row operands ------------------------------------------------------
  const float* wrow = P.w + r * P.H;
  float wv[NH];
#pragma unroll
  for (int nt = 0; nt < NH; ++nt) {
    const int h = l32 + 32 * nt;
    wv[nt] = h < H ? wrow[h] : 0.f;
  }
  // GEMM1 B operand: lane holds q[h = l32+32nt][d = 8*half + 16*kd + e]
  u32x4_t qb1[NH][KD];
  const uint16_t* qrow = P.q + r * P.H * D;
#pragma unroll
  for (int nt = 0; nt < NH; ++nt) {
    const int h = l32 + 32 * nt;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      qb1[nt][kd] = h < H ? *reinterpret_cast<const u32x4_t*>(qrow + h * D + 8 * half + 16 * kd)
                          : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  // Q'[h][d] = bf16(w_h * q[h][d]) staged in LDS rows h; read back transposed
  // (lane d = 32*nd + l32, h = 16*ks + 8*half + e) as GEMM3's B operand.
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
        for (int e = 0; e < 4; ++e) o[e] = pack_bf16(wv[nt] * bf16_lo(v[e]), wv[nt] * bf16_hi(v[e]));
        *reinterpret_cast<u32x4_t*>(qs + h * L::kPitch + (8 * half + 16 * kd) * 2) = o;
      }
    }
    wave_lds_sync();
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

  // ---- chunk pipeline ---------------------------------------------------------
  const int nchunks = (n + kSlots - 1) / kSlots;
  auto stage_ptr = [&](int c) -> unsigned char* {
    return lds + L::kStageOff + (c & 1) * L::kStageBytes;
  };
  auto load_raw = [&](int c) -> Raw {
    const int j = c * kSlots + l32;
    const int jc = j < row_len ? j : row_len - 1;
    Raw v;
    v.id = DENSE ? 0 : idrow[jc];
    v.I = Irow[jc];
    v.p = prow[jc];
    return v;
  };
  // dI and key of the lane's slot; lanes < 32 publish them to the stage ring
  auto finalize = [&](int c, const Raw& v, float& dI) -> int {
    const int j = c * kSlots + l32;
    const int key = key_of(j, v.id);
    dI = key >= 0 ? slot_dI(v.I, v.p, c2, m2, invZ, coef) : 0.f;
    // lanes l and l+32 hold the same slot and store the same values: no branch
    reinterpret_cast<float*>(stage_ptr(c))[l32] = dI;
    reinterpret_cast<int*>(stage_ptr(c) + kSlots * 4)[l32] = key;
    return key;
  };
  // K rows: lane holds row j = l32, d = 8*half + 16*kd + e (GEMM1's A layout)
  auto gather = [&](int key, u32x4_t (&kr)[KD]) {
    const uint16_t* src = kb + int64_t(key < 0 ? 0 : key) * D + 8 * half;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) kr[kd] = *reinterpret_cast<const u32x4_t*>(src + 16 * kd);
  };
  auto kbuf = [&](int c) -> unsigned char* { return lds + (c & 1) * L::kKBuf; };
  auto store_k = [&](int c, const u32x4_t (&kr)[KD], int key) {
    unsigned char* kbp = kbuf(c);
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      const u32x4_t v = key < 0 ? u32x4_t{0u, 0u, 0u, 0u} : kr[kd];
      *reinterpret_cast<u32x4_t*>(kbp + l32 * L::kPitch + (8 * half + 16 * kd) * 2) = v;
    }
  };

  f32x16_t dqacc[NH][ND];
#pragma unroll
  for (int nt = 0; nt < NH; ++nt)
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) dqacc[nt][nd] = f32x16_t{};
  float dw_acc[NH];
#pragma unroll
  for (int nt = 0; nt < NH; ++nt) dw_acc[nt] = 0.f;

  Raw raw_next;
  if (nchunks > 0) {
    const Raw raw0 = load_raw(0);
    float dI0;
    const int key0 = finalize(0, raw0, dI0);
    u32x4_t k0[KD];
    gather(key0, k0);
    raw_next = load_raw(1);
    store_k(0, k0, key0);
    wave_lds_sync();
  }

  unsigned char* gs = lds + L::kGOff;
  float* dkb = P.dk + b * P.S_k * D;

  for (int c = 0; c < nchunks; ++c) {
    // slot data of chunk c+1 (loaded one chunk ago) -> stage ring; its K rows
    // and the slot data of chunk c+2 go in flight
    float dIn;
    const int key_n = finalize(c + 1, raw_next, dIn);
    u32x4_t knext[KD];
    gather(key_n, knext);
    raw_next = load_raw(c + 2);
    wave_lds_sync();

    const unsigned char* kc = kbuf(c);
    // ---- GEMM1: S^T[j][h] over d ----------------------------------------------
    f32x16_t s[NH];
#pragma unroll
    for (int nt = 0; nt < NH; ++nt) s[nt] = f32x16_t{};
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      const u32x4_t a =
          *reinterpret_cast<const u32x4_t*>(kc + l32 * L::kPitch + (8 * half + 16 * kd) * 2);
#pragma unroll
      for (int nt = 0; nt < NH; ++nt) s[nt] = mfma32(a, qb1[nt][kd], s[nt]);
    }

    // ---- G' = dI*[S>0], dW, bf16 packing, sign-mask ballots -------------------
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
          const bool pos = sv > 0.f;
          g[rr] = pos ? dIv[i][rr] : 0.f;
          dw_acc[nt] = fmaf(g[rr], sv, dw_acc[nt]);
        }
        gp[nt][i][0] = pack_bf16(g[0], g[1]);
        gp[nt][i][1] = pack_bf16(g[2], g[3]);
        // G' tile in LDS: row h, slots 8*i + 4*half .. +3
        *reinterpret_cast<uint2*>(gs + (l32 + 32 * nt) * L::kGPitch + (8 * i + 4 * half) * 2) =
            make_uint2(gp[nt][i][0], gp[nt][i][1]);
      }
    }

    // ---- GEMM2: dQ'[h][d] += G'[h][j] K[j][d] ----------------------------------
    // k-step ks covers slots 16*ks + {0..15}; register e of lane (half) is slot
    // 16*ks + 8*(e/4) + 4*half + e%4 (GEMM1's output order)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const int col0 = 32 * nd + 16 * ((lane >> 4) & 1);
        const int r0 = 16 * ks + 4 * half;
        const u32x4_t bop = lds_tr8(kc, L::kPitch, r0, r0 + 8, col0);
#pragma unroll
        for (int nt = 0; nt < NH; ++nt) {
          const u32x4_t aop = u32x4_t{gp[nt][2 * ks][0], gp[nt][2 * ks][1], gp[nt][2 * ks + 1][0],
                                      gp[nt][2 * ks + 1][1]};
          dqacc[nt][nd] = mfma32(aop, bop, dqacc[nt][nd]);
        }
      }
    }

    {
      wave_lds_sync();  // G' tile complete
      // ---- GEMM3: C[j][d] = G'^T[j][h] Q'[h][d], then the dK scatter ----------
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
        for (int ks = 0; ks < KH; ++ks)
          cacc = mfma32(ga[ks], qb3[nd][ks], cacc);
        const int d = l32 + 32 * nd;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            // padding slots add +0 to row 0: no branch in the scatter
            const int key = keys[i][rr];
            const float v = key >= 0 ? cacc[4 * i + rr] : 0.f;
            unsafeAtomicAdd(dkb + (key >= 0 ? key : 0) * D + d, v);
          }
        }
      }
    }

    // ---- next chunk's K rows into the other LDS buffer -------------------------
    store_k(c + 1, knext, key_n);
    wave_lds_sync();
  }

  // ---- row epilogue: dQ = w * dQ', dW -----------------------------------------
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
          for (int nd = 0; nd < ND; ++nd)
            dqrow[h * D + l32 + 32 * nd] = wh * dqacc[nt][nd][4 * i + rr];
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

template <int NH, int D, bool DENSE>
hipError_t launch_rows_t(const Problem& P, hipStream_t stream) {
  const dim3 grid(unsigned(P.B * P.S_q));
  row_kernel<NH, D, DENSE><<<grid, 64, 0, stream>>>(P);
  return hipGetLastError();
}

template <int NH, int D>
hipError_t launch_rows_d(const Problem& P, hipStream_t stream) {
  return P.dense ? launch_rows_t<NH, D, true>(P, stream) : launch_rows_t<NH, D, false>(P, stream);
}

}  // namespace

hipError_t launch_rows(const Problem& P, hipStream_t stream) {
  const bool two = P.H > 32;
  switch (P.D) {
    case 32:
      return two ? launch_rows_d<2, 32>(P, stream) : launch_rows_d<1, 32>(P, stream);
    case 64:
      return two ? launch_rows_d<2, 64>(P, stream) : launch_rows_d<1, 64>(P, stream);
    case 128:
      return two ? launch_rows_d<2, 128>(P, stream) : launch_rows_d<1, 128>(P, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace ibwd
