// The step before the backward: indexer scores over every key, and the
// per-query top-k selection that turns them into the backward's ids and
// index_score.
//
//   fwd_scores_kernel  one workgroup of 8 waves per 8 queries of a batch, one
//                      query per wave: S = q.k^T on bf16 MFMA (32x32x16) with
//                      the query's q in registers and 256-key K tiles in LDS
//                      shared by the 8 waves, then I = sum_h w * relu(S)
//   topk_kernel        one workgroup per query row: radix select of the k-th
//                      largest finite score (8-bit passes over an order-
//                      preserving key, from the highest bit in which the
//                      row's keys differ), then an id-ordered compaction
//
// The score is the one whose gradients the fp64 reference of the
// NVIDIA/cudnn-frontend PR #730 benchmark harness computes (its dW is the sum
// of g * relu(S)); the top-k step is named there only by its test module.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "fwd_launch.h"
#include "launch.h"

namespace ibwd {
namespace {

constexpr int kFwdWaves = 8;
constexpr int kFwdThreads = 64 * kFwdWaves;
constexpr int kFwdQB = kFwdWaves;  // queries per workgroup, one per wave
constexpr int kFwdNK = 256;        // keys per LDS tile

// LDS K tile [kFwdNK][D] bf16.  A B-operand read has 16 lanes fetch the same
// 16-byte chunk of 16 consecutive key rows; the chunk index is XORed with the
// row's position among the rows that share a 256-byte bank window, so those
// 16 reads land in 16 different 16-byte bank groups.
template <int D>
struct FwdTile {
  static constexpr int C = D / 8;   // 16-byte chunks per key row
  static constexpr int R = 16 / C;  // key rows per 256 bytes
  static constexpr int kBytes = kFwdNK * D * 2;
  __device__ static int off(int row, int chunk) {
    return row * (D * 2) + ((chunk ^ ((row / R) % C)) * 16);
  }
};

template <int D, int NMT>
__global__ __launch_bounds__(kFwdThreads) void fwd_scores_kernel(FwdProblem P) {
  using T = FwdTile<D>;
  constexpr int KS = D / 16;  // MFMA k-steps over D
  constexpr int NCH = kFwdNK * T::C;                              // 16-byte chunks per tile
  constexpr int NL = (NCH + kFwdThreads - 1) / kFwdThreads;      // of them per thread
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* tiles = smem;                                    // two K tiles
  float* wl = reinterpret_cast<float*>(smem + 2 * T::kBytes);     // [kFwdQB][NMT*32]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int64_t nqb = (P.S_q + kFwdQB - 1) / kFwdQB;
  const int64_t b = int64_t(blockIdx.x) / nqb;
  const int64_t t0 = (int64_t(blockIdx.x) % nqb) * kFwdQB;
  const int H = int(P.H);
  const int S_k = int(P.S_k);
  const int64_t t_end = (t0 + kFwdQB < P.S_q) ? t0 + kFwdQB : P.S_q;
  // keys any query of the workgroup sees
  int nk = S_k;
  if (P.causal) {
    const int64_t lim = (t_end - 1) + P.q_offset + 1;
    nk = lim <= 0 ? 0 : (lim < S_k ? int(lim) : S_k);
  }

  for (int i = tid; i < kFwdQB * NMT * 32; i += kFwdThreads) {
    const int qi = i / (NMT * 32);
    const int h = i % (NMT * 32);
    const int64_t t = t0 + qi;
    wl[i] = (h < H && t < P.S_q) ? P.w[(b * P.S_q + t) * P.H + h] : 0.f;
  }

  // A operand: the wave's query's q rows (heads x D), held for the whole key loop
  const int64_t tq = t0 + wave;
  u32x4_t a[NMT][KS];
  {
    const int64_t t = tq < P.S_q ? tq : P.S_q - 1;  // a tail wave computes a duplicate, stores nothing
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int h = 32 * mt + l32;
      const uint16_t* qrow = P.q + ((b * P.S_q + t) * P.H + (h < H ? h : 0)) * D + 8 * half;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        a[mt][ks] = h < H ? *reinterpret_cast<const u32x4_t*>(qrow + 16 * ks) : u32x4_t{0, 0, 0, 0};
    }
  }

  const uint16_t* kb = P.k + b * P.S_k * D;
  uint4 stage[NL];
  auto load_tile = [&](int s0) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = tid + kFwdThreads * u;
      const int s = s0 + idx / T::C;
      stage[u] = (idx < NCH && s < nk)
                     ? *reinterpret_cast<const uint4*>(kb + int64_t(s) * D + (idx % T::C) * 8)
                     : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int idx = tid + kFwdThreads * u;
      if (idx < NCH)
        *reinterpret_cast<uint4*>(tiles + buf * T::kBytes + T::off(idx / T::C, idx % T::C)) = stage[u];
    }
  };

  const int ntiles = (nk + kFwdNK - 1) / kFwdNK;
  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();  // tile 0 and w

  float* srow = P.scores + (b * P.S_q + (tq < P.S_q ? tq : 0)) * P.S_k;
  const int64_t vis = P.causal ? tq + P.q_offset : int64_t(S_k) - 1;  // last visible key
  const bool store = tq < P.S_q && half == 0;
  const float* wq = wl + wave * NMT * 32 + 4 * half;
  float4 wr[NMT][4];  // w of this lane's heads 32mt + 8i + 4*half + (0..3)
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) wr[mt][i] = *reinterpret_cast<const float4*>(wq + 32 * mt + 8 * i);

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntiles) load_tile((it + 1) * kFwdNK);  // in flight during the MFMAs
    const unsigned char* tile = tiles + buf * T::kBytes;
#pragma unroll
    for (int nt = 0; nt < kFwdNK / 32; ++nt) {
      f32x16_t acc[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) acc[mt] = f32x16_t{};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t bk = *reinterpret_cast<const u32x4_t*>(tile + T::off(32 * nt + l32, 2 * ks + half));
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) acc[mt] = mfma32(a[mt][ks], bk, acc[mt]);
      }
      __builtin_amdgcn_s_setprio(0);
      // I = sum over heads of w * relu(S): this lane holds heads 8i + 4*half + r
      // of each 32-head tile for key column l32; the other half-wave holds the rest
      float v = 0.f;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 w4 = wr[mt][i];
          v += w4.x * fmaxf(acc[mt][4 * i + 0], 0.f);
          v += w4.y * fmaxf(acc[mt][4 * i + 1], 0.f);
          v += w4.z * fmaxf(acc[mt][4 * i + 2], 0.f);
          v += w4.w * fmaxf(acc[mt][4 * i + 3], 0.f);
        }
      const float tot = v + __shfl_xor(v, 32, 64);
      const int s = it * kFwdNK + 32 * nt + l32;
      if (store && s < S_k) srow[s] = s <= vis ? tot : -INFINITY;
    }
    if (it + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }
  // keys past every query's causal bound
  if (P.causal) {
    for (int qi = 0; qi < kFwdQB; ++qi) {
      const int64_t t = t0 + qi;
      if (t >= P.S_q) break;
      float* row = P.scores + (b * P.S_q + t) * P.S_k;
      for (int s = ntiles * kFwdNK + tid; s < S_k; s += kFwdThreads) row[s] = -INFINITY;
    }
  }
}

template <int D, int NMT>
hipError_t launch_fwd_t(const FwdProblem& P, hipStream_t stream) {
  const size_t lds = 2 * FwdTile<D>::kBytes + kFwdQB * NMT * 32 * sizeof(float);
  const int64_t nqb = (P.S_q + kFwdQB - 1) / kFwdQB;
  const dim3 grid(unsigned(P.B * nqb));
  const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_scores_kernel<D, NMT>),
                                              hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((fwd_scores_kernel<D, NMT>), grid, dim3(kFwdThreads), lds, stream, P);
  return hipGetLastError();
}

// ---- top-k selection -------------------------------------------------------------

// Order-preserving unsigned key of a finite float (larger float, larger key;
// -0 ranks with +0); every finite float maps to at least 0x00800000, so 0
// marks a score that is not a candidate (+-inf, NaN).
__device__ __forceinline__ uint32_t cand_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup per row.  E > 0: the row (at most 256*E scores) is read once
// into registers, thread tid holding ids tid + 256u; E == 0: every pass reads
// the row again.
template <int E>
__global__ __launch_bounds__(256) void topk_kernel(TopkProblem P) {
  __shared__ int hist[4][256];  // one histogram per wave
  __shared__ uint32_t part[3][4];
  __shared__ uint32_t s_sel[2];  // digit found, count of candidates above it
  __shared__ int4 cnt[E > 0 ? E : 1][2];  // per 256-id round: above / equal counts of each wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t r = blockIdx.x;
  const int S_k = int(P.S_k);
  const int topk = int(P.topk);
  const float* row = P.scores + r * P.S_k;
  int32_t* ids = P.ids + r * P.topk;
  float* vals = P.vals ? P.vals + r * P.topk : nullptr;

  uint32_t kreg[E > 0 ? E : 1];   // keys
  float freg[E > 0 ? E : 1];      // the scores themselves, for the output values
  if (E > 0) {
#pragma unroll
    for (int u = 0; u < E; ++u) {
      const int s = tid + 256 * u;
      freg[u] = s < S_k ? row[s] : 0.f;
      kreg[u] = s < S_k ? cand_key(freg[u]) : 0u;
    }
  }
  // f(s, key) for each of this thread's ids s = tid + 256u (key 0: not a candidate)
  auto for_each = [&](auto f) {
    if (E > 0) {
#pragma unroll
      for (int u = 0; u < (E > 0 ? E : 1); ++u) f(tid + 256 * u, kreg[u]);
    } else {
      for (int s = tid; s < S_k; s += 256) f(s, cand_key(row[s]));
    }
  };

  // candidates, and the smallest and largest candidate key
  uint32_t kmin = 0xffffffffu, kmax = 0u, nfin = 0u;
  for_each([&](int, uint32_t key) {
    if (key) {
      ++nfin;
      kmin = key < kmin ? key : kmin;
      kmax = key > kmax ? key : kmax;
    }
  });
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    nfin += uint32_t(__shfl_xor(int(nfin), o, 64));
    const uint32_t a = uint32_t(__shfl_xor(int(kmin), o, 64));
    const uint32_t c = uint32_t(__shfl_xor(int(kmax), o, 64));
    kmin = a < kmin ? a : kmin;
    kmax = c > kmax ? c : kmax;
  }
  if (lane == 0) {
    part[0][wave] = nfin;
    part[1][wave] = kmin;
    part[2][wave] = kmax;
  }
  __syncthreads();
  nfin = part[0][0] + part[0][1] + part[0][2] + part[0][3];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    kmin = part[1][w] < kmin ? part[1][w] : kmin;
    kmax = part[2][w] > kmax ? part[2][w] : kmax;
  }
  __syncthreads();
  const int keff = int(nfin) < topk ? int(nfin) : topk;

  // radix select of the keff-th largest key over the bits below the highest
  // bit in which the candidates differ (all candidates share the bits above)
  int krem = keff;  // then: how many keys equal to the threshold to take
  uint32_t prefix = kmax;
  if (keff > 0 && kmin != kmax) {
    int lo = 32 - __builtin_clz(kmin ^ kmax);  // undecided low bits
    prefix = lo == 32 ? 0u : (kmax >> lo) << lo;
    while (lo > 0) {
      const int shift = lo > 8 ? lo - 8 : 0;
      const int width = lo - shift;
      for (int i = tid; i < 4 * 256; i += 256) (&hist[0][0])[i] = 0;
      __syncthreads();
      for_each([&](int, uint32_t key) {
        if (key && (lo == 32 || (key >> lo) == (prefix >> lo)))
          atomicAdd(&hist[wave][(key >> shift) & ((1u << width) - 1u)], 1);
      });
      __syncthreads();
      // digits in descending order: thread i holds digit (2^width - 1 - i); inclusive scan
      const int digit = (1 << width) - 1 - tid;
      const int c = digit >= 0 ? hist[0][digit] + hist[1][digit] + hist[2][digit] + hist[3][digit] : 0;
      int incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      if (lane == 63) part[0][wave] = uint32_t(incl);
      __syncthreads();
      for (int w = 0; w < wave; ++w) incl += int(part[0][w]);
      if (c > 0 && incl >= krem && incl - c < krem) {
        s_sel[0] = uint32_t(digit);
        s_sel[1] = uint32_t(incl - c);
      }
      __syncthreads();
      prefix |= s_sel[0] << shift;
      krem -= int(s_sel[1]);
      lo = shift;
      __syncthreads();
    }
  }

  // prefix is the keff-th largest key: write every larger key and the first
  // krem keys equal to it, in ascending id order
  int nsel = 0;
  if (keff > 0) {
    const uint32_t thr = prefix;
    const int keq = krem;
    int gt_run = 0, eq_run = 0;
    // ids 256u .. 256u + 255 in one step: thread tid holds id s = 256u + tid
    auto step = [&](int s, uint32_t key) {
      const bool gt = key > thr;
      const bool eq = key != 0u && key == thr;
      const uint64_t mg = ballot(gt);
      const uint64_t me = ballot(eq);
      if (lane == 0) {
        part[0][wave] = uint32_t(__popcll(mg));
        part[1][wave] = uint32_t(__popcll(me));
      }
      __syncthreads();
      int gb = gt_run, eb = eq_run, gtot = 0, etot = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        if (w < wave) {
          gb += int(part[0][w]);
          eb += int(part[1][w]);
        }
        gtot += int(part[0][w]);
        etot += int(part[1][w]);
      }
      __syncthreads();
      gb += bits_below(mg);
      eb += bits_below(me);
      if (gt || (eq && eb < keq)) {
        const int pos = gb + (eb < keq ? eb : keq);
        ids[pos] = s;
        if (vals) vals[pos] = row[s];
      }
      gt_run += gtot;
      eq_run += etot;
    };
    const int rounds = (S_k + 255) / 256;
    if (E > 0) {
      // the row is in registers: every round's per-wave counts first, then one
      // barrier, then each thread's output positions from those counts (no
      // load and no barrier between the stores)
      const uint64_t lt = lanemask_lt();
#pragma unroll
      for (int u = 0; u < (E > 0 ? E : 1); ++u) {
        const uint64_t mg = ballot(kreg[u] > thr);
        const uint64_t me = ballot(kreg[u] != 0u && kreg[u] == thr);
        if (lane == 0) {
          reinterpret_cast<int*>(&cnt[u][0])[wave] = __popcll(mg);
          reinterpret_cast<int*>(&cnt[u][1])[wave] = __popcll(me);
        }
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < (E > 0 ? E : 1); ++u) {
        if (u >= rounds) break;
        const int4 g4 = cnt[u][0];
        const int4 e4 = cnt[u][1];
        const uint32_t key = kreg[u];
        const bool gt = key > thr;
        const bool eq = key != 0u && key == thr;
        const uint64_t mg = ballot(gt);
        const uint64_t me = ballot(eq);
        const int gb = gt_run + (wave > 0 ? g4.x : 0) + (wave > 1 ? g4.y : 0) + (wave > 2 ? g4.z : 0) +
                       __popcll(mg & lt);
        const int eb = eq_run + (wave > 0 ? e4.x : 0) + (wave > 1 ? e4.y : 0) + (wave > 2 ? e4.z : 0) +
                       __popcll(me & lt);
        if (gt || (eq && eb < keq)) {
          const int pos = gb + (eb < keq ? eb : keq);
          ids[pos] = tid + 256 * u;
          if (vals) vals[pos] = freg[u];
        }
        gt_run += g4.x + g4.y + g4.z + g4.w;
        eq_run += e4.x + e4.y + e4.z + e4.w;
      }
    } else {
      for (int u = 0; u < rounds; ++u) {
        const int s = tid + 256 * u;
        step(s, s < S_k ? cand_key(row[s]) : 0u);
      }
    }
    nsel = gt_run + (eq_run < keq ? eq_run : keq);
  }
  for (int j = nsel + tid; j < topk; j += 256) {
    ids[j] = -1;
    if (vals) vals[j] = -INFINITY;
  }
}

}  // namespace

hipError_t launch_fwd_scores(const FwdProblem& P, hipStream_t stream) {
  hipError_t err;
  const bool two = P.H > 32;
  switch (P.D) {
    case 32: err = two ? launch_fwd_t<32, 2>(P, stream) : launch_fwd_t<32, 1>(P, stream); break;
    case 64: err = two ? launch_fwd_t<64, 2>(P, stream) : launch_fwd_t<64, 1>(P, stream); break;
    case 128: err = two ? launch_fwd_t<128, 2>(P, stream) : launch_fwd_t<128, 1>(P, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (err == hipSuccess) stage_done(0, "fwd_scores_kernel");
  return err;
}

hipError_t launch_topk(const TopkProblem& P, hipStream_t stream) {
  const dim3 grid(unsigned(P.rows));
  if (P.S_k <= 1024)
    hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(256), 0, stream, P);
  else if (P.S_k <= 2048)
    hipLaunchKernelGGL(topk_kernel<8>, grid, dim3(256), 0, stream, P);
  else if (P.S_k <= 4096)
    hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, stream, P);
  else
    hipLaunchKernelGGL(topk_kernel<0>, grid, dim3(256), 0, stream, P);
  const hipError_t err = hipGetLastError();
  if (err == hipSuccess) stage_done(0, "topk_kernel");
  return err;
}

}  // namespace ibwd
