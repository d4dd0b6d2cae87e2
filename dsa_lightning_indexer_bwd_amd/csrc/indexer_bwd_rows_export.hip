// Row kernel of the two-pass route for gfx950: one wave per (query row, group
// of 32 heads), two waves per SIMD.
//
// Math per query row t (NVIDIA/cudnn-frontend PR #730: the harness' fp64
// `ref_grads` and the kernel-1 score-gradient contract):
//   dI_j    = grad_loss*sm_scale*(softmax_V(sm_scale*I)_j - p_j)   (0 on padding)
//   S[h,j]  = q[t,h,:] . k[id_j,:]
//   G'[h,j] = dI_j * [S[h,j] > 0]          (G = w[t,h] * G')
//   dW[t,h] = sum_j G'[h,j] * S[h,j]
//   dQ[t,h,:] = w[t,h] * sum_j G'[h,j] * k[id_j,:]
// and, for the range kernel that finishes dK, per valid slot a record
// {key, dI, the sign bits [S[h,j] > 0] of every h} grouped by key range, and
// (w*q)^T of the row.  For the slot-row route the kernel instead writes, per
// valid slot, its key and its dK row
//   C[j,:] = sum_h G'[h,j] (w*q)[h,:] = dI_j * sum_h [S[h,j] > 0] (w*q)[h,:]
// computed on the matrix cores from the same sign bits and rounded to bf16
// (see crow_pass).
//
// The 64 heads are split over the two waves of a workgroup (one row per
// workgroup).  Each wave then needs half the registers (dQ' accumulators, Q,
// the score tile), so it fits in 256 registers and two waves share each SIMD:
// one wave's VALU work (mask, G', dW) overlaps the other's MFMA work.  The
// softmax statistics, the record layout and every slot's dI and record
// position come from a prep kernel that runs first (one wave per row, many
// rows in flight per CU, so its dependent global round trips overlap across
// rows instead of stalling the MFMA work of this kernel).  The per-slot work
// that does not depend on the heads is split between the two waves instead of
// repeated: wave 1 stages dI and key, wave 0 the record position and stores
// the records; each wave gathers and stores half the rows of the shared K
// tile.  One barrier per chunk.  With H <= 32 a single wave does all of it.
//
// Per chunk of 32 slots:
//   GEMM1  S^T[j,h]  = K_g[j,:] . Q[h,:]     v_mfma 32x32x16, M=j N=h K=d; K_g
//          read from the shared LDS tile (16-byte reads), Q in registers
//   GEMM2  dQ'[h,d] += G'[h,j] K_g[j,d]      M=h N=d K=j; G' from GEMM1's
//          accumulators, K_g^T read transposed from the same tile
// The head of lane l32 in GEMM1's N dimension is 32*g + rotl5(l32), so the
// ballot of [S > 0] over the wave is directly the record's sign word in the
// bit order the range kernel expands with three VALU operations per pair.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "device_common.h"
#include "launch.h"

namespace ibwd {
namespace {

// Buffers per ring of the row kernel: K tiles, slot stages, wave 1's sign
// words.  Gathers, stages and sign words are written a fixed number of chunks
// ahead whatever the depth, so a build with IBWD_DEEP_BUFFERS (deeper rings, no
// buffer reused within its window) must produce the same bits as this one;
// the GPU tests compare the two builds.
#ifdef IBWD_DEEP_BUFFERS
constexpr int kKTiles = 4, kRowStages = 8, kW1Ring = 4;
#else
constexpr int kKTiles = 2, kRowStages = 4, kW1Ring = 2;
#endif
static_assert(kKTiles >= 2 && kRowStages >= 4 && kW1Ring >= 2, "rings cover the pipeline distances");
static_assert((kKTiles & (kKTiles - 1)) == 0 && (kRowStages & (kRowStages - 1)) == 0 &&
                  (kW1Ring & (kW1Ring - 1)) == 0,
              "ring positions are masks of the chunk index");

template <int D>
struct ExportLds {
  // K / Q' rows are stored unpadded with their 16-byte chunks permuted by an
  // XOR of the row (D >= 64): eight rows read or written at one chunk (16
  // bytes per lane) and the four rows x 32 bytes of a transposed read then
  // fall on distinct LDS banks.  D = 32 rows (four chunks) are padded instead.
  static constexpr bool kSwz = D >= 64;
  static constexpr int kPitch = kSwz ? D * 2 : D * 2 + 32;
  static constexpr int kTile = kSlots * kPitch;  // one K chunk
  // byte offset of byte `byte` of row `row` (16-byte accesses stay whole)
  __device__ static int at(int row, int byte) {
    const int f = kSwz ? (((row & 3) << 1) | ((row >> 2) & 1)) : 0;
    return row * kPitch + (((byte >> 4) ^ f) << 4) + (byte & 15);
  }
  // ds_read_b64_tr_b16 of a 4 x 16 block (rows row0.., bf16 columns col0..):
  // source lane s of each 16-lane group points at row row0 + s/4, columns
  // col0 + 4*(s%4) .. +3
  __device__ static uint2 tr4(const unsigned char* tile, int row0, int col0) {
    const int s = threadIdx.x & 15;
    const unsigned char* a = tile + at(row0 + (s >> 2), (col0 + 4 * (s & 3)) * 2);
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)(a));
    return __builtin_bit_cast(uint2, v);
  }
  // an MFMA operand of 8 k-values: rows [r0, r0+4) then [r1, r1+4)
  __device__ static u32x4_t tr8(const unsigned char* tile, int r0, int r1, int col0) {
    const uint2 x = tr4(tile, r0, col0);
    const uint2 y = tr4(tile, r1, col0);
    return u32x4_t{x.x, x.y, y.x, y.y};
  }
  // K tiles (chunks c, c+1, ...); at row start each wave stages its Q' in one
  static constexpr int kStageOff = kKTiles * kTile;
  // dI (fp32), key, record position, dI - bf16(dI) (fp32); ring of kRowStages
  static constexpr int kStageBytes = kSlots * 16;
  static constexpr int kW1Off = kStageOff + kRowStages * kStageBytes;  // sign words of wave 1
  static constexpr int kBytes = kW1Off + kW1Ring * kSlots * 4;
};

// LDS of the slot-row variant (CROWS): the row kernel's layout, then wave 0's
// sign words (a ring like wave 1's) and (w*q)^T of the row, [D][HP] bf16, kept
// for the whole row as the A operand of C^T.
template <int D, int NG, bool CROWS>
struct RowLds {
  using L = ExportLds<D>;
  static constexpr int HP = 32 * NG;
  static constexpr int kW0Off = L::kBytes;
  static constexpr int kQtOff = kW0Off + (CROWS ? kW1Ring * kSlots * 4 : 0);
  static constexpr int kQtPitch = HP * 2;
  static constexpr int kBytes = kQtOff + (CROWS ? D * kQtPitch : 0);
  static_assert(L::kBytes % 16 == 0, "16-byte aligned Q' rows");
  // byte offset of 16-byte chunk c (heads 8c .. 8c+7) of row d: chunks XORed by
  // the row's place within its 256-byte line, so that 16 consecutive rows at
  // one chunk (the A-operand reads) fall on distinct banks
  __device__ static int qt_at(int d, int c) {
    constexpr int rpb = 256 / kQtPitch;  // rows per 256 bytes
    constexpr int cpr = kQtPitch / 16;   // chunks per row
    return d * kQtPitch + ((c ^ ((d / rpb) & (cpr - 1))) << 4);
  }
};

struct Raw {
  int id;
  int2 pd;  // {record position (-1: padding), dI bits} from the prep kernel
};

__device__ __forceinline__ int rotl5(int b) { return ((b << 1) | (b >> 4)) & 31; }

constexpr int kPrepGroups = 16;  // 64-slot groups whose range masks the prep kernel keeps

// Lanes of the wave whose range equals this lane's (valid lanes only), from
// nbits ballots of the range bits: each lane keeps the ballot of bit b where
// its own bit b is set and the complement where it is clear (an XNOR with the
// bit spread over a word).
__device__ __forceinline__ uint64_t same_range_lanes(bool valid, int r, int nbits) {
  const uint64_t vm = ballot(valid);
  uint32_t lo = uint32_t(vm), hi = uint32_t(vm >> 32);
  for (int b = 0; b < nbits; ++b) {
    const uint32_t x = uint32_t(int(uint32_t(r) << (31 - b)) >> 31);  // all ones where bit b of r is set
    const uint64_t bb = ballot(x != 0u) & vm;
    lo &= ~(uint32_t(bb) ^ x);
    hi &= ~(uint32_t(bb >> 32) ^ x);
  }
  return uint64_t(hi) << 32 | lo;
}

// Per query row, before the row kernel: the softmax statistics over the valid
// slots, the slot count of every 128-key range, the row's record layout
// (ranges in key order, each starting at a multiple of 4 entries, slots in
// slot order within a range) and, for every slot, its record position and its
// dI.  One wave per row and no MFMA work, so many rows are in flight per CU and
// the dependent global round trips of these passes overlap across rows.
//   pass 1: statistics and range counts (ballots of the range bits; no LDS
//           atomics: gfx950 runs those at about 190 cycles per instruction for
//           the CU)
//   scan:   range starts; {first, end} of every range to `offs`
//   pass 2: positions (range start + earlier slots of the range, from the
//           same ballots) and dI, as {position or -1, dI} per slot
// PACKED (slot-row route): ranges follow each other without alignment.
// MAXG > 0: rows of at most 64*MAXG slots; pass 1's range masks stay in
// registers for pass 2, which then matches no ranges itself.
template <bool DENSE, bool PACKED, int MAXG>
__global__ __launch_bounds__(64) void row_prep_kernel(Problem P) {
  extern __shared__ int cursor[];  // one int per key range
  const int lane = threadIdx.x;
  const int64_t r = int64_t(blockIdx.x);
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
  int2* slot = reinterpret_cast<int2*>(P.slot) + r * P.row_len;
  int2* offrow = reinterpret_cast<int2*>(P.offs) + r * P.NR;
  const int S_k = int(P.S_k);
  const int id_base = int(r / P.S_q) * P.id_batch_stride;
  constexpr int RK = kRangeKeys;  // power of two: divisions are shifts
  const int NR = int(P.NR);
  auto key_of = [&](int j, int id) -> int {
    if (j >= n) return -1;
    if (DENSE) return j;
    return local_key(id, id_base, S_k);
  };
  int nbits = 0;
  while ((1 << nbits) < NR) ++nbits;
  const float c2 = P.sm_scale * 1.4426950408889634f;  // base-2 logit scale
  const float coef = P.grad_loss * P.sm_scale;

  // ---- pass 1: statistics, range counts ----------------------------------------
  if (!DENSE) {
    for (int i = lane; i < NR; i += 64) cursor[i] = 0;
    lds_order();
  }
  uint64_t sm[MAXG > 0 ? MAXG : 1];  // pass 1's range mask of each 64-slot group
  const float2 st = row_softmax_stats<64 * MAXG>(
      n, Irow, c2, [&](int j) { return DENSE ? 0 : idrow[j]; }, key_of, [&](int g, int, int key) {
        if (!DENSE) {
          const bool valid = key >= 0;
          const int rg = valid ? key / RK : 0;
          const uint64_t same = same_range_lanes(valid, rg, nbits);
          if (MAXG > 0) sm[g] = same;
          if (valid && bits_below(same) == 0) cursor[rg] += __popcll(same);
          lds_order();
        }
      });

  // ---- range starts and {first, end} -------------------------------------------
  if (DENSE) {
    // record of slot j at j: ranges are already in key order, 128 apart
    for (int i = lane; i < NR; i += 64) {
      const int cnt = n - i * RK < 0 ? 0 : (n - i * RK < RK ? n - i * RK : RK);
      offrow[i] = cnt > 0 ? make_int2(i * RK, i * RK + cnt) : make_int2(0, 0);
    }
  } else {
    const int per = (NR + 63) / 64;
    const int s0 = lane * per < NR ? lane * per : NR;
    const int s1 = s0 + per < NR ? s0 + per : NR;
    int sum = 0;
    for (int i = s0; i < s1; ++i) sum += PACKED ? cursor[i] : (cursor[i] + 3) & ~3;
    int incl = sum;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int run = incl - sum;
    lds_order();
    for (int i = s0; i < s1; ++i) {
      const int cnt = cursor[i];
      cursor[i] = run;
      offrow[i] = make_int2(run, run + cnt);
      run += PACKED ? cnt : (cnt + 3) & ~3;
    }
    lds_order();
  }

  // ---- pass 2: record position and dI of every slot ------------------------------
  constexpr int kU = 4;  // loads in flight per lane and array
  auto batch = [&](int j0) {
    int idv[kU];
    float iv[kU], pv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j0 + 64 * u + lane;
      const int jc = j < n ? j : n - 1;
      idv[u] = DENSE ? 0 : idrow[jc];
      iv[u] = Irow[jc];
      pv[u] = prow[jc];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (j0 + 64 * u < n) {
        const int j = j0 + 64 * u + lane;
        const int key = key_of(j, idv[u]);
        const bool valid = key >= 0;
        int pos = j;
        if (!DENSE) {
          const int rg = valid ? key / RK : 0;
          const uint64_t same = MAXG > 0 ? sm[(j0 >> 6) + u] : same_range_lanes(valid, rg, nbits);
          const int base = valid ? cursor[rg] : 0;
          const int below = bits_below(same);
          pos = base + below;
          lds_order();
          if (valid && below == 0) cursor[rg] = base + __popcll(same);
          lds_order();
        }
        const float dI = valid ? slot_dI(iv[u], pv[u], c2, st.x, st.y, coef) : 0.f;
        if (j < n) slot[j] = make_int2(valid ? pos : -1, __float_as_int(dI));
      }
    }
  };
  if constexpr (MAXG > 0) {
#pragma unroll
    for (int j0 = 0; j0 < 64 * MAXG; j0 += 64 * kU)
      if (j0 < n) batch(j0);
  } else {
    for (int j0 = 0; j0 < n; j0 += 64 * kU) batch(j0);
  }
}

// SPLIT: GEMM2 takes G' as two bf16 terms, bf16(G') and bf16(G' - bf16(G')),
// so that dQ carries only fp32 accumulation error (for bf16 outputs, whose own
// rounding would otherwise add to that of G').
// CROWS: the slot-row route's outputs (keys and dK rows) instead of records and
// (w*q)^T.
template <int D, bool DENSE, int NG, bool SPLIT, bool CROWS>
__global__ __launch_bounds__(64 * NG) __attribute__((amdgpu_waves_per_eu(2))) void row_export_kernel(
    Problem P) {
  constexpr int KD = D / 16;  // GEMM1 k-steps over d
  constexpr int ND = D / 32;  // GEMM2 32-wide d tiles
  using L = ExportLds<D>;
  using RL = RowLds<D, NG, CROWS>;
  static_assert(!(CROWS && DENSE), "the dense call keeps the key-range route");
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  // head group of this wave (wave-uniform: readfirstlane keeps it in a scalar)
  const int g = NG == 2 ? __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6)) : 0;
  // roles: the dI wave (stages each slot's dI and key) and the record wave
  // (stages record positions, stores the records); one wave holds both when
  // NG == 1
  const bool dI_wave = NG == 1 || g == 1;
  const bool rec_wave = g == 0;
  const int H = int(P.H);
  const int HP = int(P.HP);
  const int64_t ridx = int64_t(blockIdx.x);
  // dense rows are visited longest first
  const int64_t r = DENSE ? (P.B * P.S_q - 1 - ridx) : ridx;
  const int64_t b = r / P.S_q;
  const int64_t t = r % P.S_q;
  const int row_len = int(P.row_len);
  int n = row_len;
  if (DENSE) {
    const int64_t last = t + P.q_offset;
    n = last < 0 ? 0 : int(last + 1 < P.S_k ? last + 1 : P.S_k);
  }
  const int32_t* idrow = DENSE ? nullptr : P.ids + r * P.row_len;
  const int2* slotrow = reinterpret_cast<const int2*>(P.slot) + r * P.row_len;
  const uint16_t* kb = P.k + b * P.S_k * D;
  const int S_k = int(P.S_k);
  const int id_base = int(b) * P.id_batch_stride;

  auto key_of = [&](int j, int id) -> int {
    if (j >= n) return -1;
    if (DENSE) return j;
    return local_key(id, id_base, S_k);
  };
  int2* rkd = reinterpret_cast<int2*>(P.rkd) + r * P.rec_stride;
  uint2* rmask = reinterpret_cast<uint2*>(P.rmask) + r * P.rec_stride;

  // ---- per-row operands: this wave's heads -----------------------------------
  const int hl = 32 * g + rotl5(l32);  // head of lane l32 in GEMM1's N dimension
  const float wv = hl < H ? P.w[r * P.H + hl] : 0.f;
  // GEMM1 B operand: lane holds q[hl][d = 8*half + 16*kd + e]
  u32x4_t qb1[KD];
  const uint16_t* qrow = P.q + r * P.H * D;
#pragma unroll
  for (int kd = 0; kd < KD; ++kd)
    qb1[kd] = hl < H ? *reinterpret_cast<const u32x4_t*>(qrow + hl * D + 8 * half + 16 * kd)
                     : u32x4_t{0u, 0u, 0u, 0u};
  // the first two chunks' slot loads, issued now so that their latency
  // overlaps the (w*q)^T work below
  auto load_raw = [&](int c) -> Raw {
    const int j = c * kSlots + l32;
    const int jc = j < row_len ? j : row_len - 1;
    Raw v;
    v.id = DENSE ? 0 : idrow[jc];
    v.pd = slotrow[jc];
    return v;
  };
  const Raw raw0 = load_raw(0), raw1 = load_raw(1);
  // (w*q)^T: Q' rows staged in LDS (K tile g of this wave) at the natural head
  // offset rotl5(l32), read back transposed (lane d = 32*nd + l32, 8 heads
  // from 16*ks + 8*half)
  {
    unsigned char* qs = lds + g * L::kTile;
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      const u32x4_t v = qb1[kd];
      u32x4_t o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf16(wv * bf16_lo(v[e]), wv * bf16_hi(v[e]));
      *reinterpret_cast<u32x4_t*>(qs + L::at(rotl5(l32), (8 * half + 16 * kd) * 2)) = o;
    }
    wave_lds_sync();
    uint16_t* qtrow = P.qt + r * D * HP + 32 * g;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      const int col0 = 32 * nd + 16 * ((lane >> 4) & 1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int r0 = 16 * ks + 8 * half;
        const u32x4_t v = L::tr8(qs, r0, r0 + 4, col0);
        if (CROWS)  // row d, heads 32g + r0 .. +7: chunk 4g + 2ks + half
          *reinterpret_cast<u32x4_t*>(lds + RL::kQtOff + RL::qt_at(32 * nd + l32, 4 * g + 2 * ks + half)) = v;
        else
          *reinterpret_cast<u32x4_t*>(qtrow + (32 * nd + l32) * HP + r0) = v;
      }
    }
    __syncthreads();  // both Q' tiles read before the K tiles take their place
  }

  // ---- chunk pipeline ---------------------------------------------------------
  // Iteration c runs GEMM1 and GEMM2 of chunk c from its LDS tile, writes the
  // K rows of chunk c+1 (gathered during iteration c-1) into its tile
  // and gathers those of chunk c+2; the gathers thus have a whole iteration to
  // land.  Each wave gathers and writes half the rows of a tile.  Slot data
  // (dI, key) live in a ring of kRowStages stages written by the dI wave.  The barrier
  // at the top of an iteration publishes the tile and the stage, and the
  // record wave's view of wave 1's sign words of the previous chunk.
  const int nchunks = (n + kSlots - 1) / kSlots;
  auto ktile = [&](int c) -> unsigned char* { return lds + (c & (kKTiles - 1)) * L::kTile; };
  auto stage_ptr = [&](int c) -> unsigned char* {
    return lds + L::kStageOff + (c & (kRowStages - 1)) * L::kStageBytes;
  };
  uint32_t* w1x = reinterpret_cast<uint32_t*>(lds + L::kW1Off);
  uint32_t* w0x = reinterpret_cast<uint32_t*>(lds + RL::kW0Off);  // CROWS only
  // key of the lane's slot; the dI wave also publishes dI and key, the record
  // wave the position of the slot's record (lanes l and l+32 write the same
  // values)
  auto finalize = [&](int c, const Raw& v) -> int {
    const int j = c * kSlots + l32;
    const int key = key_of(j, v.id);
    if (dI_wave) {
      const float dI = key >= 0 ? __int_as_float(v.pd.y) : 0.f;
      reinterpret_cast<float*>(stage_ptr(c))[l32] = dI;
      reinterpret_cast<int*>(stage_ptr(c) + kSlots * 4)[l32] = key;
      // the part of dI that bf16(dI) drops (exact in fp32)
      if (SPLIT) reinterpret_cast<float*>(stage_ptr(c) + kSlots * 12)[l32] = dI - bf16_lo(pack_bf16(dI, 0.f));
    }
    // slots past the row (j >= row_len) load a clamped copy of the last slot's
    // entry: their position is -1 like that of every other padding slot
    if (rec_wave) reinterpret_cast<int*>(stage_ptr(c) + kSlots * 8)[l32] = key >= 0 ? v.pd.x : -1;
    return key;
  };
  // Each wave gathers only its RW rows of a chunk's K tile (all 32 when it is
  // alone): lane L holds row grow = 16g + L % RW, 16-byte chunks
  // L / RW + LPR*k.  Padding slots read row 0; their dI is 0, so they add
  // nothing.  GEMM1 then reads its A operand (lane: row l32, d = 8*half +
  // 16*kd + e) for all 32 rows from the shared tile.
  constexpr int RW = kSlots / NG;   // K rows gathered by this wave
  constexpr int LPR = 64 / RW;      // lanes per row
  constexpr int NCH = D / 8 / LPR;  // 16-byte chunks per lane
  const int grow = (NG == 2 ? 16 * g : 0) + lane % RW;
  const int gch0 = lane / RW;
  // key: the lane's slot key (lane l32 holds slot l32)
  auto gather = [&](int key, u32x4_t (&kr)[NCH]) {
    const int kr_key = __shfl(key, grow, 64);
    const uint16_t* src = kb + int64_t(kr_key < 0 ? 0 : kr_key) * D;
#pragma unroll
    for (int k = 0; k < NCH; ++k)
      kr[k] = *reinterpret_cast<const u32x4_t*>(src + 8 * (gch0 + LPR * k));
  };
  auto store_ktile = [&](int c, const u32x4_t (&kr)[NCH]) {
#pragma unroll
    for (int k = 0; k < NCH; ++k)
      *reinterpret_cast<u32x4_t*>(ktile(c) + L::at(grow, (gch0 + LPR * k) * 16)) = kr[k];
  };
  auto gemm1 = [&](int c) -> f32x16_t {
    f32x16_t s = f32x16_t{};
#pragma unroll
    for (int kd = 0; kd < KD; ++kd) {
      const u32x4_t a =
          *reinterpret_cast<const u32x4_t*>(ktile(c) + L::at(l32, (8 * half + 16 * kd) * 2));
      s = mfma32(a, qb1[kd], s);
    }
    return s;
  };

  f32x16_t dqacc[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) dqacc[nd] = f32x16_t{};
  float dw_acc = 0.f;

  // Records of chunk c are stored by the record wave in iteration c+1, after
  // the iteration's one wait and before its loads (gfx9's vmcnt counts stores
  // too, and a store issued after a load that is waited for later turns that
  // wait into a full drain).  Only lanes of valid slots store.  The validity
  // comes from the dI wave's stage (its key) and the position from the prep
  // kernel, which marks exactly the same slots (same ids, same key rule) with
  // -1; the store still checks the position itself, so that no slot can
  // address memory before the row's records.
  int prev_pos = 0;
  bool prev_valid = false;
  int2 prev_kd = make_int2(-1, 0);
  uint32_t prev_mask = 0u;
  auto store_records = [&](int c_prev) {
    if (rec_wave && prev_valid && prev_pos >= 0) {
      if (CROWS) {
        P.skey[r * P.rec_stride + prev_pos] = prev_kd.x;
      } else {
        const uint32_t w1 = NG == 2 ? w1x[(c_prev & (kW1Ring - 1)) * kSlots + l32] : 0u;
        rkd[prev_pos] = prev_kd;
        rmask[prev_pos] = make_uint2(prev_mask, w1);
      }
    }
  };

  // ---- slot-row route: C^T[d][j] = sum_h (w*q)^T[d][h] G'[h][j] of chunk cc --
  // M = d (the wave's 32-column blocks: wave g takes a contiguous half of D,
  // at D = 32 wave 0 takes it all), N = slot j, K = heads.  The A operand
  // (lane: row d, heads 16ks + 8half .. +7) is read from the LDS copy of
  // (w*q)^T; the B operand (lane: slot l32, the same eight heads) is expanded
  // from the slot's two sign words: head 16ks + 8half + e is bit
  // 8(ks&1) + 4half + e/2 + 16(e&1) of word ks/2 (bit b of word g is head
  // 32g + rotl5(b)), so a pair of heads is one shift, one AND and one 24-bit
  // multiply by bf16(dI).  Lane (slot l32, half) then holds C[l32][d] for
  // d = 32mb + 8i + 4half + 0..3, rounded to bf16 (nearest even).  For D >= 64
  // the wave stages its columns of the 32 rows in LDS, in the rows of the K
  // tile of chunk cc+2 that it gathers itself (free until it writes them later
  // in the iteration), and stores each row's piece as contiguous 16-byte lanes;
  // at D = 32 each lane stores its 8-byte pieces directly.  Padding slots
  // (position -1, dI 0) write the row after the last record.
  constexpr int MBT = D / 32;                                     // 32-column blocks
  constexpr int MPW = NG == 1 ? MBT : (MBT >= 2 ? MBT / 2 : 1);  // blocks per wave
  constexpr int SP = MPW * 64;                                    // staged row pitch, bytes
  constexpr int SCPR = SP / 16;                                   // 16-byte chunks per staged row
  constexpr int SRPB = SP >= 256 ? 1 : 256 / SP;                  // staged rows per 256 bytes
  static_assert(D < 64 || 32 * SP <= (kSlots / NG) * L::kPitch, "staging fits the wave's rows of a K tile");
  auto stg_at = [](int row, int ch) { return row * SP + ((ch ^ ((row / SRPB) & (SCPR - 1))) << 4); };
  auto crow_pass = [&](int cc) {
    const int mlo = NG == 1 ? 0 : g * MPW;  // first block of this wave
    if (mlo >= MBT) return;                 // wave 1 at D = 32
    const unsigned char* st = stage_ptr(cc);
    const float dIj = reinterpret_cast<const float*>(st)[l32];
    const uint32_t dib = pack_bf16(dIj, 0.f) & 0xffffu;
    const uint32_t wd0 = w0x[(cc & (kW1Ring - 1)) * kSlots + l32];
    const uint32_t wd1 = NG == 2 ? w1x[(cc & (kW1Ring - 1)) * kSlots + l32] : 0u;
    const unsigned char* qtl = lds + RL::kQtOff;
    unsigned char* stg = ktile(cc + 2) + (NG == 2 ? RW * g * L::kPitch : 0);
    auto rec_of = [&](int pos) -> int64_t {
      return pos >= 0 ? r * P.rec_stride + pos : P.B * P.S_q * P.rec_stride;
    };
#pragma unroll
    for (int kp = 0; kp < MPW; kp += 2) {
      const bool two = kp + 1 < MPW;
      const int mb0 = mlo + kp;
      f32x16_t ca = f32x16_t{}, cb = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 2 * NG; ++ks) {
        const uint32_t word = (ks < 2 ? wd0 : wd1) >> (8 * (ks & 1) + 4 * half);
        u32x4_t bx;
#pragma unroll
        for (int j = 0; j < 4; ++j) bx[j] = __umul24((word >> j) & 0x10001u, dib);
        const u32x4_t a0 = *reinterpret_cast<const u32x4_t*>(qtl + RL::qt_at(32 * mb0 + l32, 2 * ks + half));
        ca = mfma32(a0, bx, ca);
        if (two) {
          const u32x4_t a1 = *reinterpret_cast<const u32x4_t*>(qtl + RL::qt_at(32 * mb0 + 32 + l32, 2 * ks + half));
          cb = mfma32(a1, bx, cb);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint2 va = make_uint2(pack_bf16(ca[4 * i], ca[4 * i + 1]), pack_bf16(ca[4 * i + 2], ca[4 * i + 3]));
        const uint2 vb = make_uint2(pack_bf16(cb[4 * i], cb[4 * i + 1]), pack_bf16(cb[4 * i + 2], cb[4 * i + 3]));
        if (D >= 64) {
          // local column 32k + 8i + 4half: 16-byte chunk 4k + i, bytes 8half..
          *reinterpret_cast<uint2*>(stg + stg_at(l32, 4 * kp + i) + 8 * half) = va;
          if (two) *reinterpret_cast<uint2*>(stg + stg_at(l32, 4 * kp + 4 + i) + 8 * half) = vb;
        } else {
          const int pos = reinterpret_cast<const int*>(st + kSlots * 8)[l32];
          uint16_t* dst = P.crow + rec_of(pos) * D;
          *reinterpret_cast<uint2*>(dst + 32 * mb0 + 8 * i + 4 * half) = va;
          if (two) *reinterpret_cast<uint2*>(dst + 32 * mb0 + 32 + 8 * i + 4 * half) = vb;
        }
      }
    }
    if (D >= 64) {
      wave_lds_sync();
      constexpr int kRowsPer = 64 / SCPR;  // staged rows per 16-byte-lane pass
      // fully unrolled, except for one wave at D = 128 (eight passes), where
      // hoisting every read would spill
      constexpr int kUnroll = kSlots / kRowsPer > 4 ? 2 : kSlots / kRowsPer;
#pragma unroll kUnroll
      for (int it = 0; it < kSlots / kRowsPer; ++it) {
        const int row = it * kRowsPer + lane / SCPR;
        const int ch = lane % SCPR;
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + stg_at(row, ch));
        const int pos = reinterpret_cast<const int*>(st + kSlots * 8)[row];
        // read once, by the next kernel: streamed past the caches
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(P.crow + rec_of(pos) * D + 32 * mlo + 8 * ch));
      }
      wave_lds_sync();  // staging read before the wave's K rows take its place
    }
  };

  u32x4_t kr[NCH];
  Raw raw;
  if (nchunks > 0) {
    gather(finalize(0, raw0), kr);
    store_ktile(0, kr);
    gather(finalize(1, raw1), kr);
    raw = load_raw(2);
  }

  // one pipeline step: chunk c (its K tile complete), the K rows of chunk c+1
  // into its tile, gathers of chunk c+2
  auto step = [&](int c) {
    __syncthreads();  // K tile and stage of chunk c complete; chunk c-1 done by both waves
    // chunk c-1's dK rows: both waves' sign words are visible now, and the
    // stores go out before this iteration's loads
    if (CROWS && c > 0) crow_pass(c - 1);
    // raised priority while this wave issues its MFMAs, so that the other wave
    // of the SIMD fills the gaps with its VALU work
    __builtin_amdgcn_s_setprio(1);
    const f32x16_t s_cur = gemm1(c);
    __builtin_amdgcn_s_setprio(0);
    store_ktile(c + 1, kr);
    const int key_n2 = finalize(c + 2, raw);
    store_records(c - 1);
    gather(key_n2, kr);
    raw = load_raw(c + 3);

    // ---- G' = dI*[S>0], dW, bf16 packing, sign words --------------------------
    // lane: head hl; register 4*i + rr <-> slot 8*i + 4*half + rr
    const float* sd = reinterpret_cast<const float*>(stage_ptr(c));
    const int* sk = reinterpret_cast<const int*>(stage_ptr(c) + kSlots * 4);
    float dIv[4][4], dIl[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(sd + 8 * i + 4 * half);
      dIv[i][0] = v.x;
      dIv[i][1] = v.y;
      dIv[i][2] = v.z;
      dIv[i][3] = v.w;
      if (SPLIT) {
        const float4 u = *reinterpret_cast<const float4*>(sd + 3 * kSlots + 8 * i + 4 * half);
        dIl[i][0] = u.x;
        dIl[i][1] = u.y;
        dIl[i][2] = u.z;
        dIl[i][3] = u.w;
      }
    }
    uint32_t gp[4][2], gl[4][2];
    uint32_t maskword = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float gv[4], lv[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float sv = s_cur[4 * i + rr];
        const bool pos = sv > 0.f;
        gv[rr] = pos ? dIv[i][rr] : 0.f;
        if (SPLIT) lv[rr] = pos ? dIl[i][rr] : 0.f;
        dw_acc = fmaf(gv[rr], sv, dw_acc);
        // low half of the ballot: slot 8*i + rr, high half: slot 8*i + 4 + rr;
        // lane j of maskword takes the sign word of slot j
        const uint64_t bal = ballot(pos);
        maskword = write_lane(maskword, uint32_t(bal), 8 * i + rr);
        maskword = write_lane(maskword, uint32_t(bal >> 32), 8 * i + 4 + rr);
      }
      gp[i][0] = pack_bf16(gv[0], gv[1]);
      gp[i][1] = pack_bf16(gv[2], gv[3]);
      if (SPLIT) {
        gl[i][0] = pack_bf16(lv[0], lv[1]);
        gl[i][1] = pack_bf16(lv[2], lv[3]);
      }
    }
    if (NG == 2 && g == 1 && lane < kSlots) w1x[(c & (kW1Ring - 1)) * kSlots + lane] = maskword;
    if (CROWS && g == 0 && lane < kSlots) w0x[(c & (kW1Ring - 1)) * kSlots + lane] = maskword;

    // ---- GEMM2: dQ'[h][d] += G'[h][j] K[j][d] ----------------------------------
    // k-step ks covers slots 16*ks + {0..15}; register e of lane (half) is slot
    // 16*ks + 8*(e/4) + 4*half + e%4 (GEMM1's output order)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4_t aop = u32x4_t{gp[2 * ks][0], gp[2 * ks][1], gp[2 * ks + 1][0], gp[2 * ks + 1][1]};
      const u32x4_t alo = u32x4_t{gl[2 * ks][0], gl[2 * ks][1], gl[2 * ks + 1][0], gl[2 * ks + 1][1]};
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const int col0 = 32 * nd + 16 * ((lane >> 4) & 1);
        const int r0 = 16 * ks + 4 * half;
        const u32x4_t kt = L::tr8(ktile(c), r0, r0 + 8, col0);
        dqacc[nd] = mfma32(aop, kt, dqacc[nd]);
        if (SPLIT) dqacc[nd] = mfma32(alo, kt, dqacc[nd]);
      }
    }
    __builtin_amdgcn_s_setprio(0);

    // ---- record wave: this chunk's records, stored in the next iteration -----
    if (rec_wave) {
      const int key = sk[l32];
      const bool valid = lane < kSlots && key >= 0;
      prev_pos = reinterpret_cast<const int*>(stage_ptr(c) + kSlots * 8)[l32];
      prev_valid = valid;
      prev_kd = make_int2(key, __float_as_int(sd[l32]));
      prev_mask = maskword;
    }
  };
  for (int c = 0; c < nchunks; ++c) step(c);
  __syncthreads();  // the last chunk's sign words of wave 1
  if (CROWS && nchunks > 0) crow_pass(nchunks - 1);
  store_records(nchunks - 1);

  // ---- row epilogue: dQ = w * dQ', dW -----------------------------------------
  // dQ' register 4*i + rr of lane (half) is GEMM2's row m = 8*i + 4*half + rr,
  // i.e. head 32*g + rotl5(m).  bf16 outputs round the same fp32 values.  No
  // later kernel of the call reads dQ: its stores are non-temporal, so that
  // its lines do not sit dirty in the caches that the next kernels read through.
  const float tot = dw_acc + __shfl_xor(dw_acc, 32, 64);
  auto epilogue = [&](auto* dq, auto* dw, auto cvt) {
    auto* dqrow = dq + r * P.H * D;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int mrow = 8 * i + 4 * half + rr;
        const int h = 32 * g + rotl5(mrow);
        const float wh = __shfl(wv, mrow, 64);  // lane mrow holds w of that head
        if (h < H) {
#pragma unroll
          for (int nd = 0; nd < ND; ++nd)
            __builtin_nontemporal_store(cvt(wh * dqacc[nd][4 * i + rr]), &dqrow[h * D + l32 + 32 * nd]);
        }
      }
    }
    if (half == 0 && hl < H) dw[r * P.H + hl] = cvt(tot);
  };
  if (P.bf16_out)
    epilogue(reinterpret_cast<uint16_t*>(P.dq), reinterpret_cast<uint16_t*>(P.dw),
             [](float v) { return bf16_bits(v); });
  else
    epilogue(P.dq, P.dw, [](float v) { return v; });
}

template <int D, bool DENSE, int NG, bool CROWS>
void launch_export(const Problem& P, hipStream_t stream) {
  const dim3 grid(unsigned(P.B * P.S_q));
  constexpr int kLds = RowLds<D, NG, CROWS>::kBytes;
  // bf16 outputs take G' in two bf16 terms (the dQ rounding then stays the
  // only one of note); fp32 outputs keep one
  if (P.bf16_out)
    row_export_kernel<D, DENSE, NG, true, CROWS><<<grid, 64 * NG, kLds, stream>>>(P);
  else
    row_export_kernel<D, DENSE, NG, false, CROWS><<<grid, 64 * NG, kLds, stream>>>(P);
}

template <int D, bool DENSE, bool CROWS>
hipError_t launch_t(const Problem& P, hipStream_t stream) {
  const dim3 grid(unsigned(P.B * P.S_q));
  // rows of up to 1024 slots keep pass 1's range masks in registers
  if (!DENSE && P.row_len <= 64 * kPrepGroups)
    row_prep_kernel<DENSE, CROWS, kPrepGroups><<<grid, 64, size_t(P.NR) * 4, stream>>>(P);
  else
    row_prep_kernel<DENSE, CROWS, 0><<<grid, 64, size_t(P.NR) * 4, stream>>>(P);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  stage_done(0, "row_prep_kernel");
  if (P.HP > 32)
    launch_export<D, DENSE, 2, CROWS>(P, stream);
  else
    launch_export<D, DENSE, 1, CROWS>(P, stream);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  stage_done(1, "row_export_kernel");
  return hipSuccess;
}

template <int D>
hipError_t launch_d(const Problem& P, hipStream_t stream) {
  if (P.dense) return launch_t<D, true, false>(P, stream);
  return P.route == kDkSlotRows ? launch_t<D, false, true>(P, stream) : launch_t<D, false, false>(P, stream);
}

}  // namespace

hipError_t launch_rows_export(const Problem& P, hipStream_t stream) {
  switch (P.D) {
    case 32:
      return launch_d<32>(P, stream);
    case 64:
      return launch_d<64>(P, stream);
    case 128:
      return launch_d<128>(P, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace ibwd
