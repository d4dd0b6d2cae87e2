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
//   workgroup (key range of 256 keys, query block, batch): an fp32 slab
//   [256 + 1][D] in LDS (the extra row absorbs the writes of empty tile rows).
//   Wave w owns the columns 32w .. 32w+31, so no two waves touch the same LDS
//   word; all waves walk the same stream of 32-slot tiles:
//     C tile [32 slots x 32 d] = M[32 slots x HP] . (w*q)^T[HP x 32 d]
//   on v_mfma 32x32x16, with M[slot][h] = [S > 0] in bf16 (0 or 1.0) expanded
//   from the sign words by two VALU operations per pair of heads, and dI
//   scaling each slot in fp32.  In the accumulator layout a half-wave holds 32
//   consecutive columns of one slot, so every LDS read-modify-write touches
//   32 consecutive words of one slab row per half-wave: with a row pitch of D
//   words no two lanes of a half-wave share a bank, whatever the keys.
//   A tile's 32 keys are distinct unless a row repeats an id; a tile with a
//   repeated key takes an ordered one-row-at-a-time path, so duplicates stay
//   exact.  The next tile's records and the next query's (w*q)^T are loaded
//   while the current tile computes.
// The slab of every (range, query block) goes to global memory, and a last
// kernel sums the query-block slabs in a fixed order: the result does not
// depend on scheduling, so d_k is bitwise reproducible.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "launch.h"

namespace ibwd {
namespace {

constexpr int kTile = 32;  // slots per MFMA tile (M of 32x32x16)
constexpr int kXcds = 8;   // accelerator dies of the chip, each with its own L2

template <int D>
struct DkShape {
  static constexpr int NW = D >= 32 ? D / 32 : 1;  // waves; wave w owns columns 32w..32w+31
  static constexpr int RK = kRangeKeys;
  static constexpr int kSlabBytes = (RK + 1) * D * 4;  // row RK: sink of empty tile rows
  static constexpr int kStampOff = kSlabBytes;
  static constexpr int kStampStride = RK + 4;  // per wave; entry RK takes inactive lanes
  static constexpr int kStageOff = kStampOff + NW * kStampStride * 4;  // per wave: 32 int2
  static constexpr int kListOff = kStageOff + NW * kTile * 8;
  static constexpr int kBytes = kListOff + kMaxQueryBlock * 16;
  static_assert(kSlabBytes >= kMaxQueryBlock * 4, "slab doubles as scan scratch");
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

// Records of one 32-slot tile.  MFMA row m (the A operand's lane m = l32)
// takes record base + pi(m), pi(8i + 4h + r) = 16h + 4i + r, so that
// accumulator register 4i + r of a lane in half h is the record
// base + 16h + 4i + r.  A lane loads only the record of its MFMA row (lanes l
// and l+32 the same one); the keys and dI of its 16 accumulator rows come
// from a per-wave LDS stage, where the 32 records of the tile are four
// 16-byte broadcast reads per half-wave away.  (Loading them from global
// memory per lane would move 16 times the tile's bytes through the vector
// memory path.)
// Entries past a range's end are sinks (key one past the range), so a tile
// needs no bounds checks: sink rows land in the slab's scratch row RK.
struct Tile {
  uint2 w;   // sign words of record base + pi(l32)
  int2 kd;   // {key, dI bits} of record base + pi(l32)
};

template <int NH, int D>
__global__ __launch_bounds__(64 * DkShape<D>::NW, 2) void dk_range_kernel(Problem P) {
  using S = DkShape<D>;
  constexpr int KS = NH * 2;  // 16-deep k-steps over the heads
  constexpr int HP = NH * 32;
  constexpr int NTH = 64 * S::NW;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  float* slab = reinterpret_cast<float*>(lds);
  int4* list = reinterpret_cast<int4*>(lds + S::kListOff);
  __shared__ int nne_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int wv = tid >> 6;
  // Workgroup i is dispatched to XCD i % 8.  Consecutive logical ids (the key
  // ranges of one query block) are given to workgroups of one XCD, so the
  // (w*q)^T rows that every range of the block reads are fetched into that
  // XCD's L2 once and hit there for the other ranges.
  int R, qb;
  int64_t b;
  {
    const int n = int(gridDim.x);
    const int i = int(blockIdx.x);
    const int x = i % kXcds, k = i / kXcds;
    const int per = n / kXcds, rem = n % kXcds;
    const int logical = x * per + (x < rem ? x : rem) + k;
    R = logical % int(P.NR);
    qb = (logical / int(P.NR)) % int(P.NQB);
    b = logical / int(P.NR * P.NQB);
  }
  const int RK = S::RK;
  const int R0 = R * RK;
  const int nkeys = int(P.S_k - R0 < RK ? P.S_k - R0 : RK);
  const int64_t t0 = int64_t(qb) * P.QBS;
  const int nq = int((t0 + P.QBS < P.S_q ? t0 + P.QBS : P.S_q) - t0);

  // ---- the block's queries that have records in this range ------------------
  {
    int* flag = reinterpret_cast<int*>(lds);  // scratch in the slab area
    int4 mine[(kMaxQueryBlock + NTH - 1) / NTH];
#pragma unroll
    for (int u = 0; u < (kMaxQueryBlock + NTH - 1) / NTH; ++u) {
      const int i = tid + u * NTH;
      if (i < nq) {
        const int64_t row = b * P.S_q + t0 + i;
        const int2 fe = reinterpret_cast<const int2*>(P.offs)[row * P.NR + R];
        mine[u] = make_int4(int(row), fe.x, fe.y, 0);
        flag[i] = fe.y > fe.x ? 1 : 0;
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
      if (i < nq && mine[u].z > mine[u].y) list[flag[i]] = mine[u];
    }
    __syncthreads();
  }
  const int nne = nne_s;

  for (int i = tid; i < (RK + 1) * D; i += NTH) slab[i] = 0.f;
  int* stamp = reinterpret_cast<int*>(lds + S::kStampOff) + wv * S::kStampStride;
  for (int i = lane; i < S::kStampStride; i += 64) stamp[i] = 0;
  __syncthreads();

  const int col = 32 * wv + l32;  // the lane's slab column
  // A-operand expansion: element pair j of k-step ks sits at bits q and q + 16
  // of the sign word shifted right by 8*(ks & 1), q = 4*half + j
  uint32_t emask[4], emul[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    emask[j] = 0x10001u << (4 * half + j);
    emul[j] = 0x3f80u >> (4 * half + j);
  }
  const int pim = 16 * ((l32 >> 2) & 1) + 4 * (l32 >> 3) + (l32 & 3);

  // B operand: (w*q)^T, lane holds d = col, h = 16*ks + 8*half + e
  // Query-level values (list entries) are wave-uniform: moving them to scalar
  // registers makes every record and (w*q)^T address a scalar row base plus a
  // 32-bit per-lane offset.
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  const uint32_t qt_lane = uint32_t((col * HP + 8 * half) * 2);
  auto load_qt = [&](int row, u32x4_t (&a)[KS]) {
    const char* qtrow = reinterpret_cast<const char*>(P.qt) + size_t(uni(row)) * (D * HP * 2);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      a[ks] = *reinterpret_cast<const u32x4_t*>(qtrow + qt_lane + 32 * ks);
  };
  // records of the tile starting at `base` (at most 31 entries past the
  // range's end: inside its sink entries)
  auto load_tile = [&](int row, int base) -> Tile {
    Tile tl;
    const size_t rb = size_t(uni(row)) * size_t(P.rec_stride) * 8;
    const uint32_t ia = uint32_t(uni(base) + pim) * 8;
    tl.w = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(P.rmask) + rb + ia);
    tl.kd = *reinterpret_cast<const int2*>(reinterpret_cast<const char*>(P.rkd) + rb + ia);
    return tl;
  };
  int2* stage = reinterpret_cast<int2*>(lds + S::kStageOff) + wv * kTile;

  // one tile of records tl with B operand qa
  auto process = [&](const Tile& tl, const u32x4_t (&qa)[KS]) {
    // are the tile's keys pairwise distinct?  Each lane of the lower half
    // writes its lane number at its key's stamp and reads it back (one wave's
    // LDS accesses run in order): lanes that share a key read the one lane
    // number that won, so all but one of them see a clash.  Lanes of the upper
    // half and sinks (key - R0 == RK) use the spare entry RK and do not count.
    // Stamps are per wave.
    const int ka = tl.kd.x;
    const bool active = half == 0 && ka - R0 < RK;
    int* sp = &stamp[active ? ka - R0 : RK];
    *sp = lane;
    if (half == 0) stage[pim] = tl.kd;
    wave_lds_sync();
    const int stamp_old = *sp;
    // keys and dI of the lane's accumulator rows base + 16*half + 4i + (0..3)
    int4 key[4];
    float4 di[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int4 a = *reinterpret_cast<const int4*>(stage + 16 * half + 4 * i);
      const int4 c = *reinterpret_cast<const int4*>(stage + 16 * half + 4 * i + 2);
      key[i] = make_int4(a.x, a.z, c.x, c.z);
      di[i] = make_float4(__int_as_float(a.y), __int_as_float(a.w), __int_as_float(c.y),
                          __int_as_float(c.w));
    }

    f32x16_t acc = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t word = (ks < 2 ? tl.w.x : tl.w.y) >> (8 * (ks & 1));
      u32x4_t av;
#pragma unroll
      for (int j = 0; j < 4; ++j) av[j] = __umul24(word & emask[j], emul[j]);
      acc = mfma32(av, qa[ks], acc);
    }

    // accumulator register 4i + r: record base + 16*half + 4i + r, column col;
    // byte offsets into the slab (the sink key R0 + RK lands on row RK)
    const int cbase = (col - R0 * D) * 4;
    int addr[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      addr[4 * i + 0] = key[i].x * (D * 4) + cbase;
      addr[4 * i + 1] = key[i].y * (D * 4) + cbase;
      addr[4 * i + 2] = key[i].z * (D * 4) + cbase;
      addr[4 * i + 3] = key[i].w * (D * 4) + cbase;
    }
    auto at = [&](int k) -> float& { return *reinterpret_cast<float*>(lds + addr[k]); };
    const float dv[16] = {di[0].x, di[0].y, di[0].z, di[0].w, di[1].x, di[1].y, di[1].z, di[1].w,
                          di[2].x, di[2].y, di[2].z, di[2].w, di[3].x, di[3].y, di[3].z, di[3].w};
    const bool clash = active && stamp_old != lane;
    if (ballot(clash) == 0) {
      float old[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) old[k] = at(k);
#pragma unroll
      for (int k = 0; k < 16; ++k) at(k) = fmaf(dv[k], acc[k], old[k]);
    } else {
      // ordered path: one slab row (one register of one half-wave) at a time
      for (int k = 0; k < 16; ++k) {
        for (int hh = 0; hh < 2; ++hh) {
          if (half == hh) at(k) = fmaf(dv[k], acc[k], at(k));
          wave_lds_sync();
        }
      }
    }
  };
  // all tiles of one query; f is its first tile, loaded a query earlier.
  // Tiles are prefetched one ahead with the loop unrolled by two so that no
  // loaded register is copied (a copy would wait for the load).
  auto run_query = [&](const int4 el, const u32x4_t (&qa)[KS], const Tile& f) {
    // the entry in scalar registers: no LDS read (and no wait behind the
    // previous tile's slab writes) inside the tile loop
    const int4 e = make_int4(uni(el.x), uni(el.y), uni(el.z), 0);
    const int ntl = (e.z - e.y + kTile - 1) / kTile;
    const int last = e.y + kTile * (ntl - 1);
    auto tbase = [&](int tt) { return e.y + kTile * tt < last ? e.y + kTile * tt : last; };
    Tile tb = load_tile(e.x, tbase(1));
    process(f, qa);
    for (int tt = 1; tt < ntl; tt += 2) {
      const Tile ta = load_tile(e.x, tbase(tt + 1));
      process(tb, qa);
      tb = load_tile(e.x, tbase(tt + 2));
      if (tt + 1 < ntl) process(ta, qa);
    }
  };

  if (nne > 0) {
    // queries alternate between two operand sets, each loaded one query ahead
    u32x4_t qa0[KS], qa1[KS];
    Tile f0, f1;
    {
      const int4 e0 = list[0];
      const int4 e1 = list[nne > 1 ? 1 : 0];
      load_qt(e0.x, qa0);
      f0 = load_tile(e0.x, e0.y);
      load_qt(e1.x, qa1);
      f1 = load_tile(e1.x, e1.y);
    }
    for (int qi = 0; qi < nne; qi += 2) {
      run_query(list[qi], qa0, f0);
      {
        const int4 e2 = list[qi + 2 < nne ? qi + 2 : nne - 1];
        load_qt(e2.x, qa0);
        f0 = load_tile(e2.x, e2.y);
      }
      if (qi + 1 < nne) run_query(list[qi + 1], qa1, f1);
      {
        const int4 e3 = list[qi + 3 < nne ? qi + 3 : nne - 1];
        load_qt(e3.x, qa1);
        f1 = load_tile(e3.x, e3.y);
      }
    }
  }
  __syncthreads();
  // slab -> global partial of this (range, query block)
  float* dst = P.slab + ((b * P.NQB + qb) * (P.NR * RK) + R0) * D;
  for (int i = tid; i < nkeys * (D / 4); i += NTH) {
    const int kr = i / (D / 4), c4 = i % (D / 4);
    const float4 v = *reinterpret_cast<const float4*>(slab + kr * D + 4 * c4);
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
  const dim3 grid(unsigned(P.NR * P.NQB * P.B));
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&dk_range_kernel<NH, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::kBytes);
  if (err != hipSuccess) return err;
  dk_range_kernel<NH, D><<<grid, 64 * S::NW, S::kBytes, stream>>>(P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  stage_done(1, "dk_range_kernel");
  const int64_t n4 = P.B * P.S_k * P.D / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  dk_sum_kernel<<<unsigned(blocks), 256, 0, stream>>>(P);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  stage_done(2, "dk_sum_kernel");
  return hipSuccess;
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
