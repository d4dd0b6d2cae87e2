// Internal interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace ibwd {

constexpr int64_t kMaxHeads = 64;
constexpr int kSlots = 32;          // slots per chunk in the row kernel
constexpr int kRangeKeys = 128;     // keys per range of the two-pass dK route
constexpr int kMaxRanges = 2048;    // ranges a row can be bucketed into (S_k <= 262144)
constexpr int kMaxQueryBlock = 512;  // queries per range-kernel workgroup
constexpr int kRecBlock = 128;       // records the range kernel stages per DMA

enum DkRoute : int {
  kDkTwoPass = 0,  // masks + records exported, range-major LDS reduction (deterministic)
  kDkAtomic = 1,   // fp32 global atomics straight from the row kernel
  kDkSlotRows = 2,  // per-slot dK rows from the row kernel, summed per key range (deterministic)
};

// Route of a deterministic call.  The key-range GEMM multiplies, per query and
// 128-key range, every key of the range whether selected or not, and copies the
// query's (w*q)^T into the range's workgroup: its cost follows (queries x
// ranges).  Per-slot dK rows cost one fp32 row of D per selected slot, written
// and read once: they win when a row selects few keys per range.
// The slot-row sum copies rows with 32-bit byte offsets, so the route needs
// all rows in 4 GiB.  force: 0 = by density, 1 = key ranges, 2 = slot rows.
inline bool slot_rows_fit(int64_t B, int64_t S_q, int64_t D, int64_t row_len) {
  return (B * S_q * row_len + 1) * D * 2 < (int64_t(1) << 32);
}
inline bool use_slot_rows(int64_t B, int64_t S_q, int64_t S_k, int64_t D, int64_t row_len, bool dense,
                          int force) {
  if (dense || !slot_rows_fit(B, S_q, D, row_len)) return false;
  if (force) return force == 2;
  return row_len * 8 <= S_k;
}

// Workspace layout of the two-pass dK route.  A row's valid slots are stored
// as records grouped by key range (range r = key / RK), slot order within a
// range; range r occupies [first_r, end_r), and every range starts at a
// multiple of 4 entries (key-range route; the slot-row route packs the ranges).
//   rkd   [rows][rec_stride] int2   {key, dI bits} of the record
//   rmask [rows][rec_stride][2] u32 sign bits [S > 0] of heads 0..31, 32..63
//         (bit b of word g is head 32g + rotl5(b), rotl5 = 5-bit rotate left)
//   offs  [rows][NR] int2           {first, end} record of each range
//   slot  [rows][row_len] int2      {record position or -1, dI bits} of every
//                                   slot (written by the prep kernel)
//   qt    [rows][D][HP] bf16        (w*q)^T of every row, heads padded to HP
//   slab  [B][NQB][NR*RK][D] fp32   per query block partial dK
// rec_stride = row_len + 3*NR (alignment of the ranges), rounded up to a
// multiple of 4.
// The slot-row route keeps offs, slot and slab, and replaces rkd, rmask and qt by
//   skey  [rows][row_len] int        key of the record at each position
//   crow  [rows][row_len][D] bf16    the slot's dK row C = dI * sum_h [S>0] (w*q)
//         plus one row that padding slots write and nothing reads
// with rec_stride = row_len (ranges packed without alignment).
struct Layout {
  int64_t rows, row_len, rec_stride, HP, RK, NR, NQB, QBS, nchunk;
  bool slot_rows;
  size_t off_rkd, off_rmask, off_offs, off_slot, off_qt, off_slab, off_skey, off_crow, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline Layout make_layout(int64_t B, int64_t S_q, int64_t S_k, int64_t H, int64_t D,
                          int64_t row_len, bool slot_rows) {
  Layout L{};
  L.rows = B * S_q;
  L.row_len = row_len;
  L.slot_rows = slot_rows;
  L.HP = H > 32 ? 64 : 32;
  L.RK = kRangeKeys;
  L.NR = (S_k + L.RK - 1) / L.RK;
  L.rec_stride = slot_rows ? row_len : (row_len + 3 * L.NR + 3) & ~int64_t(3);  // 16-byte aligned rows
  // about 512 range-kernel workgroups (two per CU), at most kMaxQueryBlock
  // queries each
  int64_t nqb = (512 + L.NR * B - 1) / (L.NR * B);
  if (nqb < (S_q + kMaxQueryBlock - 1) / kMaxQueryBlock) nqb = (S_q + kMaxQueryBlock - 1) / kMaxQueryBlock;
  if (nqb > S_q) nqb = S_q;
  if (nqb < 1) nqb = 1;
  L.QBS = (S_q + nqb - 1) / nqb;
  L.NQB = (S_q + L.QBS - 1) / L.QBS;
  L.nchunk = (row_len + kSlots - 1) / kSlots;
  const size_t recs = size_t(L.rows) * size_t(L.rec_stride);
  size_t o = 0;
  if (slot_rows) {
    L.off_offs = o;
    o = align256(o + size_t(L.rows) * size_t(L.NR) * 8);
    L.off_slot = o;
    o = align256(o + recs * 8);
    L.off_skey = o;
    o = align256(o + recs * 4);
    L.off_crow = o;
    o = align256(o + (recs + 1) * size_t(D) * 2);
    L.off_slab = o;
    o = align256(o + size_t(B) * size_t(L.NQB) * size_t(L.NR * L.RK) * size_t(D) * 4);
    L.total = o;
    return L;
  }
  // the range kernel moves records in blocks of kRecBlock, which may run past
  // the last row's records: each record array is followed by one block of slack
  L.off_rkd = o;
  o = align256(o + recs * 8 + kRecBlock * 8);
  L.off_rmask = o;
  o = align256(o + recs * 8 + kRecBlock * 8);
  L.off_offs = o;
  o = align256(o + size_t(L.rows) * size_t(L.NR) * 8);
  L.off_slot = o;
  o = align256(o + size_t(L.rows) * size_t(row_len) * 8);
  L.off_qt = o;
  o = align256(o + size_t(L.rows) * size_t(D) * size_t(L.HP) * 2);
  L.off_slab = o;
  o = align256(o + size_t(B) * size_t(L.NQB) * size_t(L.NR * L.RK) * size_t(D) * 4);
  L.total = o;
  return L;
}

// One validated backward call.  Pointers are device pointers; shapes follow
// the public header.  For the dense variant ids == nullptr and row_len == S_k.
struct Problem {
  const uint16_t* q;    // [B,S_q,H,D] bf16 bits
  const uint16_t* k;    // [B,S_k,D] bf16 bits
  const float* w;       // [B,S_q,H]
  const int32_t* ids;   // [B,S_q,row_len] (sparse) or nullptr (dense)
  const float* I;       // [B,S_q,row_len]
  const float* p;       // [B,S_q,row_len]
  float* dq;            // [B,S_q,H,D]  (bf16 bits when bf16_out)
  float* dw;            // [B,S_q,H]    (bf16 bits when bf16_out)
  float* dk;            // [B,S_k,D]    (bf16 bits when bf16_out)
  int64_t B, S_q, S_k, H, D, row_len;
  bool dense;
  bool bf16_out;            // outputs rounded to bf16 (nearest even) instead of fp32
  int32_t id_batch_stride;  // 0: ids are batch-local; S_k: ids index the flattened [B*S_k] keys
  int64_t q_offset;
  float sm_scale, grad_loss;
  int route;            // DkRoute
  // two-pass exports (carved from the workspace)
  int* rkd;  // int2 pairs {key, dI bits}
  uint32_t* rmask;
  int* offs;  // int2 pairs
  int* slot;  // int2 pairs
  uint16_t* qt;
  float* slab;
  int* skey;    // slot-row route: key of each record
  uint16_t* crow;  // slot-row route: bf16 dK row of each record; row rows*rec_stride takes padding

  int64_t rec_stride, RK, NR, NQB, QBS, nchunk, HP;
};

// Profiling hook of the C ABI (indexer_bwd_set_stage_hook); the launch code
// reports every enqueued kernel through stage_done.
typedef void (*StageHook)(void* user, int stage, const char* kernel);
void set_stage_hook(StageHook hook, void* user);
void stage_done(int stage, const char* kernel);

// Enqueue the whole backward on `stream`.  Returns the first HIP error.
hipError_t launch(Problem P, void* workspace, hipStream_t stream);

// Size of the library-owned scratch array of the allocation-free entry point,
// and its device address on the current device (resolved once per device).
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
hipError_t noalloc_scratch(void** ptr);

// Row kernel of the atomic route (one wave per query row): dQ, dW and the fp32
// atomic dK scatter.
hipError_t launch_rows(const Problem& P, hipStream_t stream);
// Prep kernel (statistics, record layout, per-slot position and dI) and row
// kernel of the two-pass route (one wave per query row and group of 32 heads):
// dQ, dW, the slot records and (w*q)^T.
hipError_t launch_rows_export(const Problem& P, hipStream_t stream);
// Two-pass dK: range-major reduction into per query-block slabs, then the
// fixed-order sum of the slabs into d_k.
hipError_t launch_dk(const Problem& P, hipStream_t stream);
// Slot-row dK: the records' dK rows summed per (32 keys, query block) in a
// fixed order into the slabs, then the same slab sum.
hipError_t launch_dk_rows(const Problem& P, hipStream_t stream);

}  // namespace ibwd
