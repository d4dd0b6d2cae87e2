// Two-pass dK of the lightning-indexer backward for gfx950.
//
// dK[s,:] = sum over every (t, slot j) with id_j = s of C[t,j,:], where
//   C[t,j,:] = dI_j * sum_h [S[t,h,j] > 0] * (w[t,h] * q[t,h,:])
// (NVIDIA/cudnn-frontend PR #730 harness `ref_grads`, the `contrib` /
// `index_add_` step, with G = dI * w * [S > 0]).
//
// Scattering C with fp32 global atomics costs one atomic per (slot, d): 1.05e9
// at the 8192 x 1024 workload, and gfx950 sustains about 3.3e11 fp32 atomic
// adds per second whatever the access pattern, so the scatter alone would take
// milliseconds.  Instead the row kernel exports one record per valid slot
// {key, dI, the 64 sign bits [S > 0] over h}, grouped by key range, plus
// (w*q)^T per row, and this kernel computes dK of one key range as a GEMM
// whose accumulators never leave the matrix cores:
//
//   dK[key][d] = sum over queries t, heads h of A_t[key][h] * Q'_t[h][d],
//   A_t[key][h] = dI of t's record of key  *  its sign bit of head h
//                 (0 when t has no record of key),  Q'_t = (w*q)^T of row t.
//
//   workgroup (key range of 128 keys, query block, batch): four MMA waves and
//   a producer wave.  MMA wave kh owns keys 32kh .. 32kh+31 and all D columns
//   of the range, as v_mfma 32x32x16 accumulators (64 fp32 registers per lane
//   at D = 128), so each A fragment it expands serves D/32 MFMAs.  Per query with records in the range the producer
//   copies the query's records and Q'_t into LDS (global_load_lds, 16 bytes
//   per lane; Q' rows XOR-swizzled so the 16-byte B-operand reads are
//   bank-conflict free) and scatters the records into a key table ({dI, sign
//   words, tag}; entries of other queries are told apart by the tag, so the
//   table is never cleared); after one barrier every MMA wave expands its A
//   fragments from the table (bf16 dI where the sign bit is set, three VALU
//   operations per pair of heads) and issues its MFMAs.  Q' tiles are copied
//   two queries ahead (three tiles), record stages three ahead (four stages)
//   and key tables built one ahead (two tables), so the next queries' copies
//   and scatter run while the current one computes; the MMA waves issue no
//   memory operation but their B reads and table reads.
//   A key that a row selects twice (duplicate ids) keeps one record in the
//   table; the producer notices the other by reading the tags back, and after the
//   query loop the workgroup adds every such record in a pass of its own, in
//   a fixed order, so the result stays deterministic.
//   The MFMA work is 2*H*D per (query, key of the range) whether the query
//   selected the key or not: at 1024 of 4096 keys per query that is four
//   times the flops of the selected slots, traded for an instruction stream
//   that is almost all MFMA (a per-slot scatter spends ~60 instructions per
//   MFMA on LDS read-modify-writes and address arithmetic).
// The accumulators of every (range, query block) go to global memory, and a
// last kernel sums the query-block partials in a fixed order: the result does
// not depend on scheduling, so d_k is bitwise reproducible.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"
#include "launch.h"

namespace ibwd {
namespace {

constexpr int kXcds = 8;  // accelerator dies of the chip, each with its own L2

// Buffers per ring: Q' tiles, key tables, record stages.  The copies are issued
// a fixed number of queries ahead whatever the depth (Q' two, records three,
// tables one), so a build with IBWD_DEEP_BUFFERS (deeper rings, no buffer
// reused within a copy's window, one workgroup per CU) must produce the same
// bits as this one; the GPU tests compare the two builds.
#ifdef IBWD_DEEP_BUFFERS
constexpr int kQTiles = 4, kTables = 4, kStages = 8;
#else
constexpr int kQTiles = 3, kTables = 2, kStages = 4;
#endif
static_assert(kQTiles >= 3 && kTables >= 2 && kStages >= 4, "rings cover the copy distances");

template <int D, int HP>
struct DkShape {
  static constexpr int RK = kRangeKeys;        // keys per range (4 blocks of 32)
  static constexpr int NCB = D / 32;           // 32-column blocks
  static constexpr int NWC = 1;                // column groups of waves
  static constexpr int NWK = 4;                // key groups of waves (one 32-key block each)
  static constexpr int NW = NWK * NWC;         // MMA waves (plus one producer wave)
  static constexpr int NTH = 64 * (NW + 1);
  static constexpr int KBW = RK / 32 / NWK;    // key blocks per wave
  static constexpr int CBW = NCB / NWC;        // column blocks per wave
  static constexpr int KS = HP / 16;           // 16-deep k-steps over the heads
  static constexpr int kRowBytes = HP * 2;     // one d row of (w*q)^T
  static constexpr int kCpr = kRowBytes / 16;  // 16-byte chunks per row
  static constexpr int kQBytes = D * kRowBytes;
  static constexpr int kTOff = kQTiles * kQBytes;      // Q' tiles, then key tables,
  static constexpr int kStOff = kTOff + kTables * RK * 16;  // then record stages {kd, w}
  static constexpr int kStBytes = 2 * kRecBlock * 8;
  static constexpr int kListOff = kStOff + kStages * kStBytes;
  static constexpr int kFlagOff = kListOff + kMaxQueryBlock * 16;
  static constexpr int kBytes = kFlagOff + 16;
  static constexpr int kDmaQ = kQBytes / 1024;  // copies of 64 lanes x 16 B per Q' tile
  static constexpr int kFbTag = 16382;         // pass id of the duplicate passes
  // (query passes use 0 .. kMaxQueryBlock-1; 16383 marks a never-written entry)
  static_assert(kDmaQ * 1024 == kQBytes, "Q' tile splits into whole copies");
  static_assert(kDmaQ + 2 < 64, "one iteration's copies fit a vmcnt immediate");
  static_assert(kQTiles * kQBytes >= kMaxQueryBlock * 4, "Q' tiles double as scan scratch");
  static_assert(kRecBlock * 8 == 1024, "one DMA moves a record block of one array");
  static_assert(KBW == 1 && 32 * NWK == RK, "one 32-key block per MMA wave");
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

// s_waitcnt vmcnt(n) (n < 16), leaving the other counters alone.  Vector
// memory operations of a wave complete in issue order, so this waits for all
// but the last n the wave issued.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt immediate");  // bits 3:0 and 15:14
  __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
}

// 64 lanes x 16 bytes from global memory (gbase + voff per lane) straight into
// LDS bytes lds_addr + 16*lane (global_load_lds_dwordx4; the LDS base goes in
// M0).  Written as assembly so that the compiler neither inserts waits for it
// (it would wait for the copy before every later LDS read, the copy's own
// destination or not) nor counts it: the kernel waits for these copies itself,
// and the compiler's own vmcnt waits stay correct, only more conservative.
// M0 is saved and restored inside the statement, so the compiler's view of it
// never changes; one wait state separates the SALU write of M0 from the copy
// that reads it (a gfx9 hazard).
__device__ __forceinline__ void dma16(uint32_t lds_addr, const void* gbase, uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(gbase)
      : "memory");
}

// Four such copies of consecutive KiBs: global gbase + voff + 1024k into LDS
// lds_addr + 16*lane + 1024k, k = 0..3, under one M0 (the instruction offset
// moves the global address and the LDS destination alike).
__device__ __forceinline__ void dma16x4(uint32_t lds_addr, const void* gbase, uint32_t voff) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "global_load_lds_dwordx4 %2, %3 offset:1024\n\t"
      "global_load_lds_dwordx4 %2, %3 offset:2048\n\t"
      "global_load_lds_dwordx4 %2, %3 offset:3072\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_addr), "v"(voff), "s"(gbase)
      : "memory");
}

// Byte offset of chunk (16 bytes) c of row d of a Q' tile in LDS: the chunk
// index is XORed with bits of the row so that eight consecutive rows read at
// one chunk (one 16-byte B-operand read of eight lanes) hit distinct banks.
template <int HP>
__device__ __forceinline__ int qt_swz(int d, int c) {
  constexpr int kCpr = HP / 8;
  const int f = ((d * HP * 2) >> 7) & (kCpr - 1);
  return d * HP * 2 + ((c ^ f) << 4);
}

// SKIP: an MMA wave passes over a query that has no record among its 32 keys
// (worth it only when a query averages at most about one record per 32 keys:
// the test delays the wave's B reads behind its table read).
template <int NH, int D, bool SKIP>
// Two workgroups of NW + 1 waves share a CU (three waves on two of the SIMDs,
// two on the others), but the kernel is held to 128 registers per lane, the
// budget of four waves per SIMD: measured at the 8192 x 1024 workload, the
// same code given 136 registers runs 30% slower.
__global__ __launch_bounds__((DkShape<D, NH * 32>::NTH)) __attribute__((amdgpu_waves_per_eu(4))) void
dk_range_kernel(Problem P) {
  constexpr int HP = NH * 32;
  using S = DkShape<D, HP>;
  constexpr int KS = S::KS;
  constexpr int NTH = S::NTH;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  int4* list = reinterpret_cast<int4*>(lds + S::kListOff);
  int* flags = reinterpret_cast<int*>(lds + S::kFlagOff);  // count, duplicates, losers

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // waves 0 .. NW-1 own keys 32kh .. 32kh+31 x all columns;
  // wave NW copies the records and Q' tiles, builds the key tables (scatters
  // the records, checks for duplicate keys) and does no MMA
  const bool prod = wv == S::NW;
  const int kh = wv % S::NWK, ch = (wv / S::NWK) % S::NWC;
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
  const int64_t t0 = int64_t(qb) * P.QBS;
  const int nq = int((t0 + P.QBS < P.S_q ? t0 + P.QBS : P.S_q) - t0);

  // key tables: no entry carries a pass id of this launch yet
  for (int i = tid; i < kTables * RK; i += NTH)
    reinterpret_cast<uint4*>(lds + S::kTOff)[i] = make_uint4(0, 0, 0, 0xffffffffu);

  // ---- the block's queries that have records in this range ------------------
  {
    int* flag = reinterpret_cast<int*>(lds);  // scratch in the Q' tiles
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
      if (lane == 0) {
        flags[0] = nne;
        flags[1] = 0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < (kMaxQueryBlock + NTH - 1) / NTH; ++u) {
      const int i = tid + u * NTH;
      if (i < nq && mine[u].z > mine[u].y) list[flag[i]] = mine[u];
    }
    __syncthreads();
  }
  const int nne = __builtin_amdgcn_readfirstlane(flags[0]);

  // ---- operand helpers --------------------------------------------------------
  auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  const uint32_t lds0 = uint32_t(uintptr_t((__attribute__((address_space(3))) unsigned char*)(lds)));
  auto qtile = [&](int buf) { return lds + buf * S::kQBytes; };
  auto table = [&](int buf) { return reinterpret_cast<uint4*>(lds + S::kTOff + buf * RK * 16); };
  auto stage_kd = [&](int buf) { return reinterpret_cast<const int2*>(lds + S::kStOff + buf * S::kStBytes); };
  auto stage_w = [&](int buf) {
    return reinterpret_cast<const uint2*>(lds + S::kStOff + buf * S::kStBytes + kRecBlock * 8);
  };
  // lane i of each copy of a Q' tile fills LDS bytes 16i.. of its KiB with the
  // global chunk the XOR swizzle puts there (the swizzle term depends on the
  // lane only)
  uint32_t dma_lane;
  {
    const int pl = 16 * lane;
    const int c = (pl & (S::kRowBytes - 1)) >> 4;
    const int f = (pl >> 7) & (S::kCpr - 1);
    dma_lane = uint32_t((pl & ~(S::kRowBytes - 1)) | ((c ^ f) << 4));
  }
  // producer: KiBs k0 .. k1-1 of Q'_t of row `row` into tile `buf`, four KiB
  // per M0 setting
  auto dma_qt_part = [&](int row, int buf, int k0, int k1) {
    const unsigned char* src =
        reinterpret_cast<const unsigned char*>(P.qt) + size_t(uni(row)) * S::kQBytes;
    const uint32_t dst = lds0 + uint32_t(buf * S::kQBytes);
    int kib = k0;
#pragma unroll
    for (; kib + 4 <= k1; kib += 4) dma16x4(dst + uint32_t(kib * 1024), src + kib * 1024, dma_lane);
#pragma unroll
    for (; kib < k1; ++kib) dma16(dst + uint32_t(kib * 1024), src + kib * 1024, dma_lane);
  };
  auto dma_qt = [&](int row, int buf) { dma_qt_part(row, buf, 0, S::kDmaQ); };
  // the loop issues a tile's copies in two parts (a multiple of four KiB first)
  constexpr int kQSplit = S::kDmaQ >= 8 ? (S::kDmaQ / 2) & ~3 : S::kDmaQ / 2;
  // producer: records first .. first+kRecBlock-1 of row `row` into stage `buf`
  // (two DMAs: {key, dI} and the sign words; records past the range's end are
  // read and ignored)
  auto dma_recs = [&](int row, int first, int buf) {
    const size_t r0 = size_t(uni(row)) * size_t(P.rec_stride) + size_t(uni(first));
    const uint32_t st = lds0 + uint32_t(S::kStOff + buf * S::kStBytes);
    dma16(st, reinterpret_cast<const char*>(P.rkd) + r0 * 8, uint32_t(16 * lane));
    dma16(st + kRecBlock * 8, reinterpret_cast<const char*>(P.rmask) + r0 * 8, uint32_t(16 * lane));
  };
  auto rec_kd = [&](int row, int r) {
    return reinterpret_cast<const int2*>(P.rkd)[size_t(row) * size_t(P.rec_stride) + r];
  };
  auto rec_w = [&](int row, int r) {
    return reinterpret_cast<const uint2*>(P.rmask)[size_t(row) * size_t(P.rec_stride) + r];
  };
  auto tag_of = [](int pid, int r) { return uint32_t(pid) << 18 | uint32_t(r); };

  // accumulators: key block kb (keys 32*(KBW*kh + kb) + 8i + 4half + r in
  // register 4i + r; KBW = 1), column block cb (column 32*(CBW*ch + cb) + l32)
  f32x16_t acc[S::KBW][S::CBW];
#pragma unroll
  for (int kb = 0; kb < S::KBW; ++kb)
#pragma unroll
    for (int cb = 0; cb < S::CBW; ++cb) acc[kb][cb] = f32x16_t{};

  // one query's (or one duplicate record's) contribution: A from key table
  // `tb` (entries tagged with pass `pid`), B = Q' tile `qbuf`.  The wave's A
  // fragment of a k-step (its 32 keys x 16 heads) serves all its column blocks.
  auto mfma_pass = [&](int tb, int qbuf, int pid) {
    const uint4 e = table(tb)[32 * kh + l32];
    const unsigned char* Q = qtile(qbuf);
    const bool valid = (e.w >> 18) == uint32_t(pid);
    // bf16 dI where the sign bit is set: ((word >> p) & 0x10001) * dI_bf16
    // puts dI in both halves of a pair of heads at once
    // (a 24-bit multiply by 0 or 1, not a select: the compiler turns such a
    // select into a branch around a second read of the entry's dI, a
    // dependent LDS round trip in the middle of the pass)
    const uint32_t dib = __umul24(pack_bf16(__uint_as_float(e.x), 0.f) & 0xffffu, uint32_t(valid));
    if (SKIP && ballot(valid) == 0) return;  // no record of this query among the wave's keys
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t b[S::CBW];
#pragma unroll
      for (int cb = 0; cb < S::CBW; ++cb)
        b[cb] = *reinterpret_cast<const u32x4_t*>(Q + qt_swz<HP>(32 * (S::CBW * ch + cb) + l32, 2 * ks + half));
      const uint32_t word = (ks < 2 ? e.y : e.z) >> (8 * (ks & 1) + 4 * half);
      u32x4_t a;
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = __umul24((word >> j) & 0x10001u, dib);
#pragma unroll
      for (int cb = 0; cb < S::CBW; ++cb) acc[0][cb] = mfma32(a, b[cb], acc[0][cb]);
    }
  };

  // (Keys of records of range R lie in [R0, R0 + RK); the table index is
  // masked anyway, so that no record can address LDS outside the table.)
  // producer: scatter the records of list entry e (staged in `sbuf`) into table
  // tb, tagged pid, in record order (so a key written twice keeps the later
  // record, the same way in every scatter of these records).  Records past
  // the staged block (only with duplicate keys) come from global memory.
  auto scatter = [&](int4 e, int sbuf, int tb, int pid, int (&key)[2]) {
    uint4* T = table(tb);
    const int n = uni(e.z) - uni(e.y);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 64 * h + lane;
      key[h] = R0;
      if (r < n) {
        const int2 kd = stage_kd(sbuf)[r];
        const uint2 w = stage_w(sbuf)[r];
        key[h] = kd.x;
        T[(kd.x - R0) & (RK - 1)] = make_uint4(uint32_t(kd.y), w.x, w.y, tag_of(pid, r));
      }
    }
    for (int c0 = kRecBlock; c0 < n; c0 += 64) {
      wave_lds_sync();
      if (c0 + lane < n) {
        const int2 kd = rec_kd(e.x, e.y + c0 + lane);
        const uint2 w = rec_w(e.x, e.y + c0 + lane);
        T[(kd.x - R0) & (RK - 1)] = make_uint4(uint32_t(kd.y), w.x, w.y, tag_of(pid, c0 + lane));
      }
    }
  };
  // producer: did a record of a query with n records (keys key[], as the
  // scatter returned them) lose its entry of table tb (pass pid) to a later
  // record of the same key?
  auto lost_any = [&](int n, const int (&key)[2], int tb, int pid) {
    const uint4* T = table(tb);
    bool lost = false;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = 64 * h + lane;
      if (r < n) lost = lost || T[(key[h] - R0) & (RK - 1)].w != tag_of(pid, r);
    }
    return ballot(lost) != 0 || n > kRecBlock;  // more records than keys: duplicates
  };

  // ---- query loop ---------------------------------------------------------------
  // Query qi: Q' tile qi % kQTiles (copied two queries ahead), record stage
  // qi % kStages (copied three queries ahead), key table qi % kTables (built
  // right after the barrier of query qi-1, from the staged records), all by
  // the producer.  The producer issues its copies and no other vector-memory
  // operation in the loop (except its loads of records past a staged block,
  // which the compiler waits for at once), so "all but the previous
  // iteration's copies" is one vmcnt immediate.  The two roles run separate
  // loops (so that their registers need not be live at once), each with one
  // barrier per query.
  bool dup = false;  // producer: some record lost its table entry to a duplicate key
  if (prod) {
    // Iteration j copies Q'(j+2) and then records(j+3); at the top of
    // iteration qi every copy but those of iteration qi-1 must have landed
    // (Q'(qi) and records(qi+1) among them).
    auto wait_prev = [&](int qi) {
      if (qi + 2 < nne)
        wait_vm<S::kDmaQ + 2>();
      else if (qi + 1 < nne)
        wait_vm<S::kDmaQ>();
      else
        wait_vm<0>();
    };
    int key[2];  // keys of the last scattered query's records
    if (nne > 0) {
      const int4 e0 = list[0];
      dma_recs(e0.x, e0.y, 0);
      wait_vm<0>();
      scatter(e0, 0, 0, 0, key);
      // the copies of "iterations" -2 and -1
      dma_qt(e0.x, 0);
      if (nne > 1) dma_recs(uni(list[1].x), uni(list[1].y), 1);
      if (nne > 1) dma_qt(uni(list[1].x), 1);
      if (nne > 2) dma_recs(uni(list[2].x), uni(list[2].y), 2);
    }
    // list entries are read one iteration before they are needed
    int4 e_cur = nne > 0 ? list[0] : make_int4(0, 0, 0, 0);
    int4 e_n1 = nne > 1 ? list[1] : e_cur;
    int4 e_n2 = nne > 2 ? list[2] : e_cur;
    int4 e_n3 = nne > 3 ? list[3] : e_cur;
    int q2 = 2 % kQTiles;  // (qi+2) % kQTiles
    for (int qi = 0; qi < nne; ++qi) {
      wait_prev(qi);
      __syncthreads();  // Q'(qi) and table qi % kTables are complete; query qi-1 is done
      const int4 e1 = e_n1, e2 = e_n2, e3 = e_n3;
      const int n = uni(e_cur.z) - uni(e_cur.y);
      e_cur = e1;
      e_n1 = e2;
      e_n2 = e3;
      if (qi + 4 < nne) e_n3 = list[qi + 4];
      // duplicates of query qi: read its table entries back (its table stays
      // intact until the scatter of query qi+2, one iteration later)
      const int kq[2] = {key[0], key[1]};
      // table of query qi+1: its last readers finished query qi-1
      // the MMA waves wait for this table at the next barrier: the producer's
      // work of the iteration runs at the highest priority of the CU's waves
      __builtin_amdgcn_s_setprio(2);
      // The scatter and the tag check are chains of LDS round trips; the copies
      // are issued around the tag check, where they wait on the copy queue
      // while those round trips are in flight.
      if (qi + 1 < nne) scatter(e1, (qi + 1) % kStages, (qi + 1) % kTables, qi + 1, key);
      // Q' tile (qi+2) % kQTiles was last read in query qi-1 at the latest
      if (qi + 2 < nne) dma_qt_part(e2.x, q2, 0, kQSplit);
      dup = dup || lost_any(n, kq, qi % kTables, qi);
      if (qi + 2 < nne) dma_qt_part(e2.x, q2, kQSplit, S::kDmaQ);
      q2 = q2 == kQTiles - 1 ? 0 : q2 + 1;
      // stage (qi+3) % kStages was last read at the latest by the scatter of query
      // qi-1, whose table writes waited for those reads
      if (qi + 3 < nne) dma_recs(uni(e3.x), uni(e3.y), (qi + 3) % kStages);
      __builtin_amdgcn_s_setprio(0);
    }
  } else {
    int q0 = 0;  // qi % kQTiles
    for (int qi = 0; qi < nne; ++qi) {
      __syncthreads();  // Q'(qi) and table qi % kTables are complete
      // raised priority while this wave expands and issues its MFMAs, so that
      // the other MMA wave of the SIMD fills the gaps with its own work
      __builtin_amdgcn_s_setprio(1);
      mfma_pass(qi % kTables, q0, qi);
      __builtin_amdgcn_s_setprio(0);
      q0 = q0 == kQTiles - 1 ? 0 : q0 + 1;
    }
  }

  // ---- records that lost their table entry to a duplicate key --------------------
  // Rare (a row that selects one key more than once).  Per query: rebuild its
  // table the same way (same winners), list the losers, and add each in a pass
  // of its own through the spare table, in record order.
  if (prod && lane == 0 && dup) flags[1] = 1;
  __syncthreads();
  if (flags[1] != 0) {
    int* losers = reinterpret_cast<int*>(qtile(1));  // 64 record indices per round
    for (int i = tid; i < 2 * RK; i += NTH) table(0)[i] = make_uint4(0, 0, 0, 0xffffffffu);
    for (int qi = 0; qi < nne; ++qi) {
      __syncthreads();
      // the entry's fields in scalar registers: they stay live across the passes
      const int4 el = list[qi];
      const int ex = uni(el.x), ey = uni(el.y), n = uni(el.z) - ey;
      if (prod) {
        dma_recs(ex, ey, 0);
        dma_qt(ex, 0);
        wait_vm<0>();
        int kq[2];
        scatter(make_int4(ex, ey, ey + n, 0), 0, 0, S::kFbTag, kq);
      }
      __syncthreads();
      for (int c0 = 0; c0 < n; c0 += 64) {
        if (prod) {
          bool lost = false;
          if (c0 + lane < n) {
            const int2 kd = rec_kd(ex, ey + c0 + lane);
            lost = table(0)[(kd.x - R0) & (RK - 1)].w != tag_of(S::kFbTag, c0 + lane);
          }
          const uint64_t m = ballot(lost);
          // (position among the lost lanes below this one)
          const int pos = int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32),
                                                        __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
          if (lost) losers[pos] = c0 + lane;
          if (lane == 0) flags[2] = __popcll(m);
        }
        __syncthreads();
        const int nl = uni(flags[2]);
        for (int li = 0; li < nl; ++li) {
          const int r = uni(losers[li]);
          if (prod && lane == 0) {
            const int2 kd = rec_kd(ex, ey + r);
            const uint2 w = rec_w(ex, ey + r);
            table(1)[(kd.x - R0) & (RK - 1)] =
                make_uint4(uint32_t(kd.y), w.x, w.y, tag_of(S::kFbTag, r));
          }
          __syncthreads();
          if (!prod) mfma_pass(1, 0, S::kFbTag);
          __syncthreads();
          if (prod && lane == 0)
            table(1)[(rec_kd(ex, ey + r).x - R0) & (RK - 1)] = make_uint4(0, 0, 0, 0xffffffffu);
        }
        __syncthreads();
      }
    }
  }

  // ---- accumulators -> this (range, query block)'s partial dK ------------------
  if (prod) return;
  float* dst = P.slab + ((b * P.NQB + qb) * (P.NR * RK) + R0) * D;
#pragma unroll
  for (int kb = 0; kb < S::KBW; ++kb)
#pragma unroll
    for (int cb = 0; cb < S::CBW; ++cb) {
      const int col = 32 * (S::CBW * ch + cb) + l32;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kl = 32 * (S::KBW * kh + kb) + 8 * i + 4 * half + r;
          if (R0 + kl < P.S_k) dst[size_t(kl) * D + col] = acc[kb][cb][4 * i + r];
        }
    }
}

// d_k[b][s][:] = sum over query blocks (in order) of the slabs; stored as fp32,
// or rounded to bf16 (nearest even) for bf16 outputs.
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
    if (P.bf16_out)
      reinterpret_cast<uint2*>(P.dk)[i] = make_uint2(pack_bf16(a.x, a.y), pack_bf16(a.z, a.w));
    else
      reinterpret_cast<float4*>(P.dk)[i] = a;
  }
}

// Slot-row route: one workgroup of four waves per (key range, query block,
// batch); wave s owns keys 32s .. 32s+31 of the range.  The row kernel left,
// for every valid slot, its key and its dK row C = dI * sum_h [S > 0] (w*q) in
// bf16 at its record position (the prep kernel groups a row's records by key
// range, slot order within a range).  The range's records of the query block
// form one sequence: query by query, each query's run [first, end) of its row;
// the workgroup numbers it once (a prefix sum of the run lengths, in LDS).
// Rounds of 1024 records: wave w reads the keys of records 256w .. 256w+255 of
// the round (the query of a record by a binary search over the run starts),
// and queues them in LDS by key block, in record order.  After a barrier wave
// s takes its block's records from the queues of waves 0..3 in turn, that is
// in record order, 16 at a time: their rows are copied from global memory
// straight into LDS (global_load_lds, three batches in flight), and the batch
// is added with one v_mfma 32x32x16 per 32 columns,
//   acc[key][d] += sum_k onehot[key][k] * row_k[d],
// the one-hot A operand (1.0 where record k is of the key) read from a small
// LDS table, the rows read transposed as the B operand.  The products are
// exact and the sums run in the matrix cores' fixed order, so d_k does not
// depend on scheduling.  Each wave reads the keys of the next round before it
// adds the rows of the current one.  The partial dK then goes to the query
// block's slab.
constexpr int kRowWaves = kRangeKeys / 32;  // key blocks of 32 per range
template <int D>
__global__ __launch_bounds__(64 * kRowWaves) void dk_rows_kernel(Problem P) {
  constexpr int kScan = 4;             // 64-record chunks a wave scans per round
  constexpr int kRound = 64 * kScan * kRowWaves;
  static_assert(2 * 64 * kRowWaves >= kMaxQueryBlock, "two queries per thread cover a query block");
  __shared__ int ex_s[kMaxQueryBlock];      // start of each query's run in the sequence
  __shared__ int base_s[kMaxQueryBlock];    // record index of each run's first record
  __shared__ int2 queue[2][kRowWaves][64 * kScan];  // {record, key - 32s}, by block, in order
  __shared__ int qoff[2][kRowWaves][kRowWaves];      // [buf][scanning wave][block] start
  __shared__ int qcnt[2][kRowWaves][kRowWaves];
  __shared__ int wsum[kRowWaves];
  // staged rows of a batch, [16][D] bf16, 16-byte chunks XORed by the row so
  // that the four rows of a transposed read fall on distinct banks
  constexpr int RP = 2 * D;       // row pitch, bytes
  constexpr int CPR = RP / 16;    // 16-byte chunks per row
  constexpr int RPB = 256 / RP;   // rows per 256 bytes
  constexpr int kDmaB = CPR / 4;  // 1 KiB copies per batch
  constexpr int kStages = 3;      // batches in flight
  constexpr int ND = D / 32;      // 32-column blocks
  __shared__ __attribute__((aligned(16))) unsigned char stage_s[kRowWaves][kStages][16 * RP];
  __shared__ __attribute__((aligned(16))) uint16_t onehot_s[kRowWaves][32 * 16];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int rg = int(blockIdx.x);
  const int qb = int(blockIdx.y);
  const int64_t b = blockIdx.z;
  const int R0 = rg * kRangeKeys;
  const int64_t t0 = int64_t(qb) * P.QBS;
  const int nq = int((t0 + P.QBS < P.S_q ? t0 + P.QBS : P.S_q) - t0);
  const int2* offs = reinterpret_cast<const int2*>(P.offs);

  // ---- the sequence: run starts of the block's queries ---------------------
  // thread i takes queries 2i, 2i+1 (nq <= 512)
  int n2[2], f2[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = 2 * int(threadIdx.x) + u;
    const int2 fe = q < nq ? offs[(b * P.S_q + t0 + q) * P.NR + rg] : make_int2(0, 0);
    n2[u] = fe.y - fe.x;
    f2[u] = fe.x;
  }
  int incl = n2[0] + n2[1];
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kRowWaves; ++w) {
    const int v = wsum[w];
    before += w < wv ? v : 0;
    total += v;
  }
  {
    const int ex = before + incl - n2[0] - n2[1];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = 2 * int(threadIdx.x) + u;
      if (q < nq) {
        ex_s[q] = ex + (u ? n2[0] : 0);
        base_s[q] = int((b * P.S_q + t0 + q) * P.rec_stride) + f2[u];
      }
    }
  }
  __syncthreads();
  const int T = __builtin_amdgcn_readfirstlane(total);

  // record f of the sequence: its global record index (or 0) and key (or -1)
  auto locate = [&](int f, int& rec) -> int {
    int lo = 0;
#pragma unroll
    for (int st = kMaxQueryBlock / 2; st > 0; st >>= 1)
      if (lo + st < nq && ex_s[lo + st] <= f) lo += st;  // a query without records shares its start with the next
    rec = f < T ? base_s[lo] + (f - ex_s[lo]) : 0;
    return f < T ? P.skey[rec] : -1;
  };
  f32x16_t acc[ND];  // lane: column 32nb + l32, registers 4i + rr: key 8i + 4half + rr
#pragma unroll
  for (int nb = 0; nb < ND; ++nb) acc[nb] = f32x16_t{};
  const int l32 = lane & 31, half = lane >> 5;
  for (int i = lane; i < 32 * 16; i += 64) onehot_s[wv][i] = 0;
  auto st_at = [](int r, int byte) {
    return r * RP + (((byte >> 4) ^ (((r / RPB) & 3) * (CPR / 4))) << 4) + (byte & 15);
  };
  const uint32_t stage0 =
      uint32_t(uintptr_t((__attribute__((address_space(3))) unsigned char*)(&stage_s[wv][0][0])));
  int recs[kScan], keys[kScan];
  auto scan_issue = [&](int round) {
#pragma unroll
    for (int c = 0; c < kScan; ++c) keys[c] = locate(round * kRound + (kScan * wv + c) * 64 + lane, recs[c]);
  };
  // this wave's records of the round, by key block, into queue[buf][wv]
  auto scan_queue = [&](int buf) {
    uint64_t m[kScan][kRowWaves];
    int cnt[kRowWaves];
#pragma unroll
    for (int s2 = 0; s2 < kRowWaves; ++s2) cnt[s2] = 0;
#pragma unroll
    for (int c = 0; c < kScan; ++c) {
      const int blk = keys[c] >= 0 ? (keys[c] - R0) >> 5 : -1;
#pragma unroll
      for (int s2 = 0; s2 < kRowWaves; ++s2) {
        m[c][s2] = ballot(blk == s2);
        cnt[s2] += __popcll(m[c][s2]);
      }
    }
    int run[kRowWaves];
    int o = 0;
#pragma unroll
    for (int s2 = 0; s2 < kRowWaves; ++s2) {
      run[s2] = o;
      if (lane == 0) {
        qoff[buf][wv][s2] = o;
        qcnt[buf][wv][s2] = cnt[s2];
      }
      o += cnt[s2];
    }
#pragma unroll
    for (int c = 0; c < kScan; ++c) {
      const int blk = keys[c] >= 0 ? (keys[c] - R0) >> 5 : -1;
#pragma unroll
      for (int s2 = 0; s2 < kRowWaves; ++s2) {
        if (blk == s2)
          queue[buf][wv][run[s2] + bits_below(m[c][s2])] =
              make_int2(recs[c], keys[c] - R0 - 32 * s2);
        run[s2] += __popcll(m[c][s2]);
      }
    }
  };
  // this wave's block from the four queues of a round, in record order
  auto consume = [&](int buf) {
    int seg[kRowWaves + 1], off[kRowWaves];
    seg[0] = 0;
#pragma unroll
    for (int w = 0; w < kRowWaves; ++w) {
      off[w] = __builtin_amdgcn_readfirstlane(qoff[buf][w][wv]);
      seg[w + 1] = seg[w] + __builtin_amdgcn_readfirstlane(qcnt[buf][w][wv]);
    }
    const int n = seg[kRowWaves];
    if (n == 0) return;
    // entry j of the block's sequence ({0, -1} past the end: record 0, no key)
    auto entry = [&](int j) -> int2 {
      int w = 0;
#pragma unroll
      for (int w2 = 1; w2 < kRowWaves; ++w2) w += j >= seg[w2] ? 1 : 0;
      int o2 = 0, s0 = 0;
#pragma unroll
      for (int w2 = 0; w2 < kRowWaves; ++w2)
        if (w2 == w) o2 = off[w2], s0 = seg[w2];
      return j < n ? queue[buf][w][o2 + j - s0] : make_int2(0, -1);
    };
    // batch bi's rows into stage bi % kStages: copy i, lane L fills 16-byte
    // slot 64i + L (row r = slot / CPR, stored chunk slot % CPR)
    auto issue = [&](int bi) {
      const uint32_t dst = stage0 + uint32_t((bi % kStages) * 16 * RP);
#pragma unroll
      for (int i = 0; i < kDmaB; ++i) {
        const int slot = 64 * i + lane;
        const int r = slot / CPR;
        const int c = (slot % CPR) ^ (((r / RPB) & 3) * (CPR / 4));
        const int rec = entry(16 * bi + r).x;
        dma16(dst + uint32_t(1024 * i), P.crow, uint32_t(rec) * uint32_t(RP) + uint32_t(16 * c));
      }
    };
    const int nbat = (n + 15) / 16;
    // every copy is issued (batches past the end copy record 0 and add
    // nothing), so the wait before each batch counts exactly the two newer ones
    issue(0);
    issue(1);
    for (int bi = 0; bi < nbat; ++bi) {
      issue(bi + 2);
      const int2 eu = entry(16 * bi + (lane & 15));  // lane u < 16: entry u of the batch
      if (lane < 16 && eu.y >= 0) onehot_s[wv][eu.y * 16 + lane] = 0x3f80;  // bf16 1.0
      wave_lds_sync();
      const u32x4_t a = *reinterpret_cast<const u32x4_t*>(&onehot_s[wv][l32 * 16 + 8 * half]);
      wait_vm<2 * kDmaB>();  // this batch's rows are in LDS
      const unsigned char* st = &stage_s[wv][bi % kStages][0];
#pragma unroll
      for (int nb = 0; nb < ND; ++nb) {
        const int col0 = 32 * nb + 16 * ((lane >> 4) & 1);
        u32x4_t bv;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int s16 = lane & 15;
          const unsigned char* ad = st + st_at(8 * half + 4 * h + (s16 >> 2), (col0 + 4 * (s16 & 3)) * 2);
          const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                        (__attribute__((address_space(3))) i16x4_t*)(ad)));
          bv[2 * h] = v.x;
          bv[2 * h + 1] = v.y;
        }
        acc[nb] = mfma32(a, bv, acc[nb]);
      }
      wave_lds_sync();
      if (lane < 16 && eu.y >= 0) onehot_s[wv][eu.y * 16 + lane] = 0;
    }
    wait_vm<0>();  // the copies past the end have landed before their stages are reused
  };

  const int rounds = (T + kRound - 1) / kRound;
  if (rounds > 0) {
    scan_issue(0);
    scan_queue(0);
  }
  __syncthreads();
  for (int i = 0; i < rounds; ++i) {
    // keys in flight while this round's rows are added (issued unconditionally:
    // past the last round no record is found and nothing is read, and the
    // compiler's waits in consume stay exact)
    scan_issue(i + 1);
    consume(i & 1);
    if (i + 1 < rounds) scan_queue((i + 1) & 1);
    __syncthreads();  // round i's queues read by every wave; round i+1's written
  }

  float* dst = P.slab + ((b * P.NQB + qb) * (P.NR * kRangeKeys) + R0 + 32 * wv) * D;
#pragma unroll
  for (int nb = 0; nb < ND; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int k = 8 * i + 4 * half + rr;
        if (R0 + 32 * wv + k < P.S_k) dst[k * D + 32 * nb + l32] = acc[nb][4 * i + rr];
      }
}

hipError_t launch_sum(const Problem& P, hipStream_t stream) {
  const int64_t n4 = P.B * P.S_k * P.D / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  dk_sum_kernel<<<unsigned(blocks), 256, 0, stream>>>(P);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  stage_done(3, "dk_sum_kernel");
  return hipSuccess;
}

template <int D>
hipError_t launch_rows_t(const Problem& P, hipStream_t stream) {
  const dim3 grid(unsigned(P.NR), unsigned(P.NQB), unsigned(P.B));
  dk_rows_kernel<D><<<grid, 64 * kRowWaves, 0, stream>>>(P);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  stage_done(2, "dk_rows_kernel");
  return launch_sum(P, stream);
}

template <int NH, int D, bool SKIP>
hipError_t launch_range(const Problem& P, hipStream_t stream) {
  using S = DkShape<D, NH * 32>;
  const dim3 grid(unsigned(P.NR * P.NQB * P.B));
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(&dk_range_kernel<NH, D, SKIP>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::kBytes);
  if (err != hipSuccess) return err;
  dk_range_kernel<NH, D, SKIP><<<grid, S::NTH, S::kBytes, stream>>>(P);
  return hipGetLastError();
}

template <int NH, int D>
hipError_t launch_dk_t(const Problem& P, hipStream_t stream) {
  // skipping pays when a row averages at most one slot per 32 keys
  const bool skip = !P.dense && P.row_len * 32 <= P.S_k;
  hipError_t err = skip ? launch_range<NH, D, true>(P, stream) : launch_range<NH, D, false>(P, stream);
  if (err != hipSuccess) return err;
  stage_done(2, "dk_range_kernel");
  return launch_sum(P, stream);
}

}  // namespace

hipError_t launch_dk_rows(const Problem& P, hipStream_t stream) {
  switch (P.D) {
    case 32:
      return launch_rows_t<32>(P, stream);
    case 64:
      return launch_rows_t<64>(P, stream);
    case 128:
      return launch_rows_t<128>(P, stream);
    default:
      return hipErrorInvalidValue;
  }
}

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
