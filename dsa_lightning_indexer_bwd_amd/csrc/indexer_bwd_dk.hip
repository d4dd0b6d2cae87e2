// Two-pass dK of the lightning-indexer backward for gfx950.
//
// dK[s,:] = sum over every (t, slot j) with id_j = s of C[t,j,:], where
//   C[t,j,:] = dI_j * sum_h [S[t,h,j] > 0] * (w[t,h] * q[t,h,:])
// (NVIDIA/cudnn-frontend PR #730 harness `ref_grads`, the `contrib` /
// `index_add_` step, with G = dI * w * [S > 0]).
//
// Scattering C with fp32 global atomics costs one atomic per (slot, d): 1.05e9
// at the 8192 x 1024 workload, and gfx950 sustains about 3.3e11 fp32 atomic
// adds per second whatever the access pattern (LDS float atomics are no
// faster), so the scatter alone would take milliseconds.  Instead the row
// kernel exports one record per valid slot {key, dI, the 64 sign bits
// [S > 0] over h}, grouped by key range, plus (w*q)^T per row; this kernel
// rebuilds C with bf16 MFMA and reduces it with plain LDS read-modify-write:
//
//   workgroup (key range R of 256 keys, query block, batch): an fp32 slab
//   [256][D] in LDS.  Each wave owns D/NW columns, so no two waves ever touch
//   the same LDS word; all waves walk the same stream of 16-slot tiles:
//     C^T tile [16 d x 16 slots] = (w*q)^T[16 d x HP] . M[HP x 16 slots]
//   on v_mfma 16x16x32, with M[h][slot] = [S > 0] in bf16 (0 or 1) looked up
//   per byte of the sign bits in a 256-entry table, and dI scaling the slot in
//   fp32.  A lane then holds 4 consecutive d of one slot and adds them into the
//   slab row of the slot's key with one 16-byte read and one 16-byte write.
//   Within a tile the 16 keys are distinct unless a row repeats an id; such a
//   tile takes an ordered one-slot-at-a-time path, so duplicates stay exact.
//   The next tile's records and the next query's (w*q)^T are loaded while the
//   current tile computes.
// The slab of every (range, query block) goes to global memory, and a last
// kernel sums the query-block slabs in a fixed order: the result does not
// depend on scheduling, so d_k is bitwise reproducible.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "launch.h"

namespace ibwd {
namespace {

constexpr int kTile = 16;  // slots per MFMA tile (N of 16x16x32)

template <int D>
struct DkShape {
  static constexpr int NW = D >= 64 ? 4 : 2;  // waves; each owns DW columns
  static constexpr int DW = D / NW;
  static constexpr int MT = DW / 16;          // 16-row m tiles of d per wave
  static constexpr int RK = kRangeKeys;
  static constexpr int kPitch = D + 4;        // floats per slab row (bank spread)
  static constexpr int kSlabBytes = RK * kPitch * 4;
  static constexpr int kLutOff = kSlabBytes;
  static constexpr int kStampOff = kLutOff + 256 * 16;
  static constexpr int kListOff = kStampOff + NW * RK * 4;
  static constexpr int kBytes = kListOff + kMaxQueryBlock * 16;
  static_assert(kSlabBytes >= 2 * kMaxQueryBlock * 4, "slab doubles as scan scratch");
};

// Exclusive prefix sum over a[0..n) in LDS by one wave, in place; returns the total.
__device__ int wave_exclusive_scan(int* a, int n) {
  const int lane = threadIdx.x & 63;
  const int per = (n + 63) / 64;
  const int s0 = lane * per < n ? lane * per : n;
  const int s1 = s0 + per < n ? s0 + per : n;
  int s = 0;
  for (int i = s0; i < s1; ++i) s += a[i];
  int incl = s;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  int run = incl - s;
  wave_lds_sync();
  for (int i = s0; i < s1; ++i) {
    const int v = a[i];
    a[i] = run;
    run += v;
  }
  wave_lds_sync();
  return __shfl(incl, 63, 64);
}

template <int NH, int D>
__global__ __launch_bounds__(64 * DkShape<D>::NW, 1) void dk_range_kernel(Problem P) {
  using S = DkShape<D>;
  constexpr int HP = NH * 32;
  constexpr int NTH = 64 * S::NW;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  float* slab = reinterpret_cast<float*>(lds);
  u32x4_t* lut = reinterpret_cast<u32x4_t*>(lds + S::kLutOff);
  int4* list = reinterpret_cast<int4*>(lds + S::kListOff);
  __shared__ int nne_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int R = blockIdx.x;
  const int qb = blockIdx.y;
  const int64_t b = blockIdx.z;
  const int RK = S::RK;
  const int R0 = R * RK;
  const int nkeys = int(P.S_k - R0 < RK ? P.S_k - R0 : RK);
  const int64_t t0 = int64_t(qb) * P.QBS;
  const int nq = int((t0 + P.QBS < P.S_q ? t0 + P.QBS : P.S_q) - t0);

  // ---- the block's queries that have slots in this range, with tile offsets
  {
    int* flag = reinterpret_cast<int*>(lds);  // scratch in the slab area
    int4 mine[(kMaxQueryBlock + NTH - 1) / NTH];
#pragma unroll
    for (int u = 0; u < (kMaxQueryBlock + NTH - 1) / NTH; ++u) {
      const int i = tid + u * NTH;
      if (i < nq) {
        const int64_t row = b * P.S_q + t0 + i;
        const int* offrow = P.off + row * (P.NR + 1);
        const int rb = offrow[R], re = offrow[R + 1];
        const int nt = (re - rb + kTile - 1) / kTile;
        mine[u] = make_int4(int(row), rb, re, nt);
        flag[i] = nt > 0 ? 1 : 0;
      }
    }
    __syncthreads();
    if (wv == 0) {
      const int nne = wave_exclusive_scan(flag, nq);  // flag := compacted index
      if (lane == 0) nne_s = nne;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < (kMaxQueryBlock + NTH - 1) / NTH; ++u) {
      const int i = tid + u * NTH;
      if (i < nq && mine[u].w > 0) list[flag[i]] = mine[u];
    }
    __syncthreads();
    if (wv == 0) {
      const int nne = nne_s;
      for (int i = lane; i < nne; i += 64) flag[i] = list[i].w;
      wave_lds_sync();
      wave_exclusive_scan(flag, nne);
      for (int i = lane; i < nne; i += 64) list[i].w = flag[i];  // w := first tile
    }
    __syncthreads();
  }
  const int nne = nne_s;

  for (int i = tid; i < RK * S::kPitch; i += NTH) slab[i] = 0.f;
  // byte -> 8 bf16: bit e of the byte is 1.0 (0x3f80) or 0
  for (int e = tid; e < 256; e += NTH) {
    uint32_t wd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wd[i] = (((e >> (2 * i)) & 1) ? 0x3f80u : 0u) | (((e >> (2 * i + 1)) & 1) ? 0x3f800000u : 0u);
    lut[e] = u32x4_t{wd[0], wd[1], wd[2], wd[3]};
  }
  __syncthreads();

  int* stamp = reinterpret_cast<int*>(lds + S::kStampOff) + wv * RK;
  const int d0 = wv * S::DW;

  // A operand: (w*q)^T, lane holds d = d0 + 16*mt + l16, h = 32*ks + 8*grp + e
  auto load_qt = [&](int row, u32x4_t (&a)[S::MT][NH]) {
    const uint16_t* qtrow = P.qt + int64_t(row) * D * HP;
#pragma unroll
    for (int mt = 0; mt < S::MT; ++mt)
#pragma unroll
      for (int ks = 0; ks < NH; ++ks)
        a[mt][ks] = *reinterpret_cast<const u32x4_t*>(qtrow + (d0 + 16 * mt + l16) * HP + 32 * ks +
                                                      8 * grp);
  };
  // record of slot l16 of a tile; index past the range end reads a row-tail entry
  auto load_rec = [&](int row, int idx, int end, bool& valid) -> int4 {
    valid = idx < end;
    const int i = valid ? idx : int(P.row_len);
    return P.rec[int64_t(row) * P.rec_stride + i];
  };

  // one 16-slot tile: the lane's record r (slot l16), valid flag vm, A operand qa
  auto process = [&](const int4& r, bool vm, const u32x4_t (&qa)[S::MT][NH]) {
    const int key = r.x;
    const float dI = __int_as_float(r.y);
    u32x4_t bop[NH];
#pragma unroll
    for (int ks = 0; ks < NH; ++ks) {
      const uint32_t word = vm ? uint32_t(ks == 0 ? r.z : r.w) : 0u;
      bop[ks] = lut[(word >> (8 * grp)) & 0xffu];
    }
    // are the tile's keys pairwise distinct?
    if (lane < kTile && vm) stamp[key - R0] = lane;
    wave_lds_sync();
    const bool clash = lane < kTile && vm && stamp[key - R0] != lane;
    const bool distinct = ballot(clash) == 0;

    f32x4_t acc[S::MT];
#pragma unroll
    for (int mt = 0; mt < S::MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NH; ++ks)
#pragma unroll
      for (int mt = 0; mt < S::MT; ++mt) acc[mt] = mfma16(qa[mt][ks], bop[ks], acc[mt]);

    // lane holds slot l16, d = d0 + 16*mt + 4*grp + (0..3)
    float* rowp = slab + (key - R0) * S::kPitch + d0 + 4 * grp;
    if (distinct) {
      if (vm) {
        float4 old[S::MT];
#pragma unroll
        for (int mt = 0; mt < S::MT; ++mt) old[mt] = *reinterpret_cast<const float4*>(rowp + 16 * mt);
#pragma unroll
        for (int mt = 0; mt < S::MT; ++mt) {
          float4 v = old[mt];
          v.x = fmaf(dI, acc[mt][0], v.x);
          v.y = fmaf(dI, acc[mt][1], v.y);
          v.z = fmaf(dI, acc[mt][2], v.z);
          v.w = fmaf(dI, acc[mt][3], v.w);
          *reinterpret_cast<float4*>(rowp + 16 * mt) = v;
        }
      }
    } else {
      // ordered path: one slot of the tile at a time
      for (int m = 0; m < kTile; ++m) {
        if (l16 == m && vm) {
#pragma unroll
          for (int mt = 0; mt < S::MT; ++mt) {
            float4 v = *reinterpret_cast<const float4*>(rowp + 16 * mt);
            v.x = fmaf(dI, acc[mt][0], v.x);
            v.y = fmaf(dI, acc[mt][1], v.y);
            v.z = fmaf(dI, acc[mt][2], v.z);
            v.w = fmaf(dI, acc[mt][3], v.w);
            *reinterpret_cast<float4*>(rowp + 16 * mt) = v;
          }
        }
        wave_lds_sync();
      }
    }
    wave_lds_sync();
  };
  // all tiles of one query; f/fv is the record of its first tile, loaded a
  // query earlier.  Records are prefetched one tile ahead with the loop
  // unrolled by two so that no loaded register is copied (a copy would wait
  // for the load).
  auto run_query = [&](const int4& e, const u32x4_t (&qa)[S::MT][NH], const int4& f, bool fv) {
    const int ntl = (e.z - e.y + kTile - 1) / kTile;
    bool vb;
    int4 rb = load_rec(e.x, e.y + kTile + l16, e.z, vb);
    process(f, fv, qa);
    for (int tt = 1; tt < ntl; tt += 2) {
      bool va;
      const int4 ra = load_rec(e.x, e.y + kTile * (tt + 1) + l16, e.z, va);
      process(rb, vb, qa);
      rb = load_rec(e.x, e.y + kTile * (tt + 2) + l16, e.z, vb);
      if (tt + 1 < ntl) process(ra, va, qa);
    }
  };

  if (nne > 0) {
    // queries alternate between two operand sets, each loaded one query ahead
    u32x4_t qa0[S::MT][NH], qa1[S::MT][NH];
    int4 f0, f1;
    bool fv0, fv1;
    {
      const int4 e0 = list[0];
      const int4 e1 = list[nne > 1 ? 1 : 0];
      load_qt(e0.x, qa0);
      f0 = load_rec(e0.x, e0.y + l16, e0.z, fv0);
      load_qt(e1.x, qa1);
      f1 = load_rec(e1.x, e1.y + l16, nne > 1 ? e1.z : 0, fv1);
    }
    for (int qi = 0; qi < nne; qi += 2) {
      run_query(list[qi], qa0, f0, fv0);
      {
        const int4 e2 = list[qi + 2 < nne ? qi + 2 : nne - 1];
        load_qt(e2.x, qa0);
        f0 = load_rec(e2.x, e2.y + l16, qi + 2 < nne ? e2.z : 0, fv0);
      }
      if (qi + 1 < nne) run_query(list[qi + 1], qa1, f1, fv1);
      {
        const int4 e3 = list[qi + 3 < nne ? qi + 3 : nne - 1];
        load_qt(e3.x, qa1);
        f1 = load_rec(e3.x, e3.y + l16, qi + 3 < nne ? e3.z : 0, fv1);
      }
    }
  }
  __syncthreads();
  // slab -> global partial of this (range, query block)
  float* dst = P.slab + ((b * P.NQB + qb) * (P.NR * RK) + R0) * D;
  for (int i = tid; i < nkeys * (D / 4); i += NTH) {
    const int kr = i / (D / 4), c4 = i % (D / 4);
    const float4 v = *reinterpret_cast<const float4*>(slab + kr * S::kPitch + 4 * c4);
    *reinterpret_cast<float4*>(dst + kr * D + 4 * c4) = v;
  }
}

// d_k[b][s][:] = sum over query blocks (in order) of the slabs.
__global__ __launch_bounds__(256) void dk_sum_kernel(Problem P) {
  const int64_t D4 = P.D / 4;
  const int64_t n = P.B * P.S_k * D4;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t span = P.NR * P.RK * D4;  // float4s per slab
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t b = i / (P.S_k * D4);
    const int64_t rest = i % (P.S_k * D4);
    const float4* src = reinterpret_cast<const float4*>(P.slab) + b * P.NQB * span + rest;
    float4 a = src[0];
    for (int64_t qb = 1; qb < P.NQB; ++qb) {
      const float4 v = src[qb * span];
      a.x += v.x;
      a.y += v.y;
      a.z += v.z;
      a.w += v.w;
    }
    reinterpret_cast<float4*>(P.dk)[i] = a;
  }
}

template <int NH, int D>
hipError_t launch_dk_t(const Problem& P, hipStream_t stream) {
  using S = DkShape<D>;
  const dim3 grid(unsigned(P.NR), unsigned(P.NQB), unsigned(P.B));
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&dk_range_kernel<NH, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::kBytes);
  if (err != hipSuccess) return err;
  dk_range_kernel<NH, D><<<grid, 64 * S::NW, S::kBytes, stream>>>(P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const int64_t n4 = P.B * P.S_k * P.D / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  dk_sum_kernel<<<unsigned(blocks), 256, 0, stream>>>(P);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dk(const Problem& P, hipStream_t stream) {
  const bool two = P.H > 32;
  switch (P.D) {
    case 32:
      return two ? launch_dk_t<2, 32>(P, stream) : launch_dk_t<1, 32>(P, stream);
    case 64:
      return two ? launch_dk_t<2, 64>(P, stream) : launch_dk_t<1, 64>(P, stream);
    case 128:
      return two ? launch_dk_t<2, 128>(P, stream) : launch_dk_t<1, 128>(P, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace ibwd
