// C ABI of the lightning-indexer backward: argument validation, the device
// check, and the launch sequence.  Every check runs before the first write or
// launch, so an invalid call leaves the outputs untouched.
#include "dsa_indexer_bwd.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "fwd_launch.h"
#include "launch.h"

static_assert(IBWD_NOALLOC_SCRATCH_BYTES == ibwd::kNoAllocScratchBytes,
              "the header states the scratch size of the allocation-free entry point");

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];

int device_status() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return IBWD_ERR_HIP;
  if (dev >= kMaxDevices) return IBWD_ERR_UNSUPPORTED_DEVICE;
  std::call_once(g_dev_once[dev], [dev] {
    hipDeviceProp_t prop;
    g_dev_ok[dev] = 0;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      g_dev_ok[dev] = -1;
      return;
    }
    g_dev_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  });
  if (g_dev_ok[dev] < 0) return IBWD_ERR_HIP;
  return g_dev_ok[dev] ? IBWD_OK : IBWD_ERR_UNSUPPORTED_DEVICE;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;

bool fits(int64_t a, int64_t b) { return a > 0 && b > 0 && a <= kMaxElems / b; }
bool fits(int64_t a, int64_t b, int64_t c) { return fits(a, b) && fits(a * b, c); }
bool fits(int64_t a, int64_t b, int64_t c, int64_t d) { return fits(a, b, c) && fits(a * b * c, d); }

// Shape and pointer checks common to both entry points.
int check_common(const void* q, const void* k, const float* w, const float* I, const float* p,
                 void* d_q, void* d_w, void* d_k, int64_t B, int64_t S_q, int64_t S_k,
                 int64_t H, int64_t D, int64_t row_len, uint32_t flags) {
  if (!q || !k || !w || !I || !p || !d_q || !d_w || !d_k) return IBWD_ERR_INVALID_ARGUMENT;
  if (B < 1 || S_q < 1 || S_k < 1 || H < 1 || D < 1 || row_len < 1) return IBWD_ERR_INVALID_ARGUMENT;
  if (H > ibwd::kMaxHeads) return IBWD_ERR_INVALID_ARGUMENT;
  if (D != 32 && D != 64 && D != 128) return IBWD_ERR_INVALID_ARGUMENT;
  if (!fits(B, S_q, H, D) || !fits(B, S_k, D) || !fits(B, S_q, row_len))
    return IBWD_ERR_INVALID_ARGUMENT;
  if ((flags & ~(IBWD_FLAG_DETERMINISTIC | IBWD_FLAG_ATOMIC_DK | IBWD_FLAG_GLOBAL_IDS |
                 IBWD_FLAG_BF16_OUT | IBWD_FLAG_DK_KEY_RANGES | IBWD_FLAG_DK_SLOT_ROWS)) != 0)
    return IBWD_ERR_INVALID_ARGUMENT;
  if ((flags & IBWD_FLAG_DETERMINISTIC) && (flags & IBWD_FLAG_ATOMIC_DK)) return IBWD_ERR_INVALID_ARGUMENT;
  // the route flags choose between the deterministic routes
  if ((flags & IBWD_FLAG_DK_KEY_RANGES) && (flags & IBWD_FLAG_DK_SLOT_ROWS)) return IBWD_ERR_INVALID_ARGUMENT;
  if ((flags & IBWD_FLAG_ATOMIC_DK) && (flags & (IBWD_FLAG_DK_KEY_RANGES | IBWD_FLAG_DK_SLOT_ROWS)))
    return IBWD_ERR_INVALID_ARGUMENT;
  // the atomic route accumulates dK in d_k itself, which needs fp32
  if ((flags & IBWD_FLAG_BF16_OUT) && (flags & IBWD_FLAG_ATOMIC_DK)) return IBWD_ERR_INVALID_ARGUMENT;
  // the row kernel buckets a row's slots into at most kMaxRanges key ranges
  if ((S_k + ibwd::kRangeKeys - 1) / ibwd::kRangeKeys > ibwd::kMaxRanges)
    return IBWD_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(d_q, 16) || !aligned(d_k, 16))
    return IBWD_ERR_INVALID_ARGUMENT;
  if (!aligned(w, 4) || !aligned(I, 4) || !aligned(p, 4) || !aligned(d_w, 4))
    return IBWD_ERR_INVALID_ARGUMENT;
  return IBWD_OK;
}

int route_force(uint32_t flags) {
  return (flags & IBWD_FLAG_DK_SLOT_ROWS) ? 2 : (flags & IBWD_FLAG_DK_KEY_RANGES) ? 1 : 0;
}

bool slot_rows(int64_t B, int64_t S_q, int64_t S_k, int64_t D, int64_t row_len, bool dense,
               uint32_t flags) {
  return ibwd::use_slot_rows(B, S_q, S_k, D, row_len, dense, route_force(flags));
}

size_t workspace_bytes(int64_t B, int64_t S_q, int64_t S_k, int64_t H, int64_t D,
                       int64_t row_len, bool dense, uint32_t flags) {
  if (flags & IBWD_FLAG_ATOMIC_DK) return 0;
  return ibwd::make_layout(B, S_q, S_k, H, D, row_len, slot_rows(B, S_q, S_k, D, row_len, dense, flags))
      .total;
}

// Both sparse entry points: every check first, then the launch.  noalloc: the
// scratch is the library's per-device array (no workspace argument).
int sparse_call(const void* q, const void* k, const float* w, const int32_t* topk_ids,
                const float* index_score, const float* attn_score, void* d_q, void* d_w, void* d_k,
                int64_t B, int64_t S_q, int64_t S_k, int64_t H, int64_t D, int64_t topk,
                float sm_scale, float grad_loss, uint32_t flags, void* workspace, size_t ws_bytes,
                hipStream_t stream, bool noalloc) {
  int st = check_common(q, k, w, index_score, attn_score, d_q, d_w, d_k, B, S_q, S_k, H, D, topk,
                        flags);
  if (st != IBWD_OK) return st;
  if (!topk_ids || !aligned(topk_ids, 4)) return IBWD_ERR_INVALID_ARGUMENT;
  if (topk > S_k) return IBWD_ERR_INVALID_ARGUMENT;  // more slots than keys
  // the slot-row route keeps all dK rows within 4 GiB
  if ((flags & IBWD_FLAG_DK_SLOT_ROWS) && !ibwd::slot_rows_fit(B, S_q, D, topk))
    return IBWD_ERR_INVALID_ARGUMENT;
  const size_t need = workspace_bytes(B, S_q, S_k, H, D, topk, false, flags);
  if (noalloc) {
    if (need > ibwd::kNoAllocScratchBytes) return IBWD_ERR_INVALID_ARGUMENT;
  } else if (need > 0 && (ws_bytes < need || !workspace || !aligned(workspace, 256))) {
    return IBWD_ERR_INVALID_ARGUMENT;
  }
  st = device_status();
  if (st != IBWD_OK) return st;
  if (noalloc && need > 0 && ibwd::noalloc_scratch(&workspace) != hipSuccess) return IBWD_ERR_HIP;
  ibwd::Problem P{};
  P.q = static_cast<const uint16_t*>(q);
  P.k = static_cast<const uint16_t*>(k);
  P.w = w;
  P.ids = topk_ids;
  P.I = index_score;
  P.p = attn_score;
  P.dq = static_cast<float*>(d_q);
  P.dw = static_cast<float*>(d_w);
  P.dk = static_cast<float*>(d_k);
  P.bf16_out = (flags & IBWD_FLAG_BF16_OUT) != 0;
  P.B = B;
  P.S_q = S_q;
  P.S_k = S_k;
  P.H = H;
  P.D = D;
  P.row_len = topk;
  P.dense = false;
  // a global id of batch b is offset by b*S_k; B*S_k < 2^31 was checked above
  P.id_batch_stride = (flags & IBWD_FLAG_GLOBAL_IDS) ? int32_t(S_k) : 0;
  P.q_offset = 0;
  P.sm_scale = sm_scale;
  P.grad_loss = grad_loss;
  P.route = (flags & IBWD_FLAG_ATOMIC_DK)         ? ibwd::kDkAtomic
            : slot_rows(B, S_q, S_k, D, topk, false, flags) ? ibwd::kDkSlotRows
                                                 : ibwd::kDkTwoPass;
  return ibwd::launch(P, workspace, stream) == hipSuccess ? IBWD_OK : IBWD_ERR_HIP;
}

}  // namespace

extern "C" {

int indexer_bwd_sparse(const void* q, const void* k, const float* w, const int32_t* topk_ids,
                       const float* index_score, const float* attn_score, void* d_q, void* d_w,
                       void* d_k, int64_t B, int64_t S_q, int64_t S_k, int64_t H, int64_t D,
                       int64_t topk, float sm_scale, float grad_loss, uint32_t flags,
                       void* workspace, size_t ws_bytes, hipStream_t stream) {
  return sparse_call(q, k, w, topk_ids, index_score, attn_score, d_q, d_w, d_k, B, S_q, S_k, H, D,
                     topk, sm_scale, grad_loss, flags, workspace, ws_bytes, stream, false);
}

int indexer_bwd_sparse_noalloc(const void* q, const void* k, const float* w,
                               const int32_t* topk_ids, const float* index_score,
                               const float* attn_score, void* d_q, void* d_w, void* d_k, int64_t B,
                               int64_t S_q, int64_t S_k, int64_t H, int64_t D, int64_t topk,
                               float sm_scale, float grad_loss, uint32_t flags,
                               hipStream_t stream) {
  return sparse_call(q, k, w, topk_ids, index_score, attn_score, d_q, d_w, d_k, B, S_q, S_k, H, D,
                     topk, sm_scale, grad_loss, flags, nullptr, 0, stream, true);
}

int indexer_bwd_dense(const void* q, const void* k, const float* w, const float* index_score,
                      const float* attn_score, void* d_q, void* d_w, void* d_k, int64_t B,
                      int64_t S_q, int64_t S_k, int64_t H, int64_t D, int64_t q_offset,
                      float sm_scale, float grad_loss, uint32_t flags, void* workspace,
                      size_t ws_bytes, hipStream_t stream) {
  int st = check_common(q, k, w, index_score, attn_score, d_q, d_w, d_k, B, S_q, S_k, H, D, S_k,
                        flags);
  if (st != IBWD_OK) return st;
  if (q_offset < -(int64_t(1) << 40) || q_offset > (int64_t(1) << 40))
    return IBWD_ERR_INVALID_ARGUMENT;
  if (flags & IBWD_FLAG_GLOBAL_IDS) return IBWD_ERR_INVALID_ARGUMENT;  // the dense call has no ids
  if (flags & IBWD_FLAG_DK_SLOT_ROWS) return IBWD_ERR_INVALID_ARGUMENT;  // every key selected
  size_t need = workspace_bytes(B, S_q, S_k, H, D, S_k, true, flags);
  if (need > 0 && (ws_bytes < need || !workspace || !aligned(workspace, 256)))
    return IBWD_ERR_INVALID_ARGUMENT;
  st = device_status();
  if (st != IBWD_OK) return st;
  ibwd::Problem P{};
  P.q = static_cast<const uint16_t*>(q);
  P.k = static_cast<const uint16_t*>(k);
  P.w = w;
  P.ids = nullptr;
  P.I = index_score;
  P.p = attn_score;
  P.dq = static_cast<float*>(d_q);
  P.dw = static_cast<float*>(d_w);
  P.dk = static_cast<float*>(d_k);
  P.bf16_out = (flags & IBWD_FLAG_BF16_OUT) != 0;
  P.B = B;
  P.S_q = S_q;
  P.S_k = S_k;
  P.H = H;
  P.D = D;
  P.row_len = S_k;
  P.dense = true;
  P.id_batch_stride = 0;
  P.q_offset = q_offset;
  P.sm_scale = sm_scale;
  P.grad_loss = grad_loss;
  P.route = (flags & IBWD_FLAG_ATOMIC_DK) ? ibwd::kDkAtomic : ibwd::kDkTwoPass;
  return ibwd::launch(P, workspace, stream) == hipSuccess ? IBWD_OK : IBWD_ERR_HIP;
}

size_t indexer_bwd_workspace_bytes(int dense, int64_t B, int64_t S_q, int64_t S_k, int64_t H,
                                   int64_t D, int64_t topk, uint32_t flags) {
  const int64_t row_len = dense ? S_k : topk;
  if (B < 1 || S_q < 1 || S_k < 1 || H < 1 || H > ibwd::kMaxHeads || row_len < 1) return 0;
  if (row_len > S_k) return 0;
  if (D != 32 && D != 64 && D != 128) return 0;
  if (!fits(B, S_q, H, D) || !fits(B, S_k, D) || !fits(B, S_q, row_len)) return 0;
  if (dense && (flags & IBWD_FLAG_DK_SLOT_ROWS)) return 0;
  if (!dense && (flags & IBWD_FLAG_DK_SLOT_ROWS) && !ibwd::slot_rows_fit(B, S_q, D, row_len)) return 0;
  return workspace_bytes(B, S_q, S_k, H, D, row_len, dense != 0, flags);
}

int indexer_fwd_scores(const void* q, const void* k, const float* w, float* scores, int64_t B,
                       int64_t S_q, int64_t S_k, int64_t H, int64_t D, int causal,
                       int64_t q_offset, hipStream_t stream) {
  if (!q || !k || !w || !scores) return IBWD_ERR_INVALID_ARGUMENT;
  if (B < 1 || S_q < 1 || S_k < 1 || H < 1 || H > ibwd::kMaxHeads) return IBWD_ERR_INVALID_ARGUMENT;
  if (D != 32 && D != 64 && D != 128) return IBWD_ERR_INVALID_ARGUMENT;
  if (!fits(B, S_q, H, D) || !fits(B, S_k, D) || !fits(B, S_q, S_k)) return IBWD_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 4) || !aligned(scores, 4))
    return IBWD_ERR_INVALID_ARGUMENT;
  if (q_offset < -(int64_t(1) << 40) || q_offset > (int64_t(1) << 40)) return IBWD_ERR_INVALID_ARGUMENT;
  const int st = device_status();
  if (st != IBWD_OK) return st;
  ibwd::FwdProblem P{};
  P.q = static_cast<const uint16_t*>(q);
  P.k = static_cast<const uint16_t*>(k);
  P.w = w;
  P.scores = scores;
  P.B = B;
  P.S_q = S_q;
  P.S_k = S_k;
  P.H = H;
  P.D = D;
  P.causal = causal != 0;
  P.q_offset = q_offset;
  return ibwd::launch_fwd_scores(P, stream) == hipSuccess ? IBWD_OK : IBWD_ERR_HIP;
}

int indexer_topk(const float* scores, int32_t* topk_ids, float* topk_scores, int64_t rows,
                 int64_t S_k, int64_t topk, hipStream_t stream) {
  if (!scores || !topk_ids) return IBWD_ERR_INVALID_ARGUMENT;
  if (rows < 1 || S_k < 1 || topk < 1 || topk > S_k) return IBWD_ERR_INVALID_ARGUMENT;
  if (!fits(rows, S_k) || !fits(rows, topk)) return IBWD_ERR_INVALID_ARGUMENT;
  if (!aligned(scores, 4) || !aligned(topk_ids, 4) || !aligned(topk_scores, 4))
    return IBWD_ERR_INVALID_ARGUMENT;
  const int st = device_status();
  if (st != IBWD_OK) return st;
  ibwd::TopkProblem P{};
  P.scores = scores;
  P.ids = topk_ids;
  P.vals = topk_scores;
  P.rows = rows;
  P.S_k = S_k;
  P.topk = topk;
  return ibwd::launch_topk(P, stream) == hipSuccess ? IBWD_OK : IBWD_ERR_HIP;
}

const char* indexer_bwd_strerror(int status) {
  switch (status) {
    case IBWD_OK:
      return "ok";
    case IBWD_ERR_INVALID_ARGUMENT:
      return "invalid argument (null pointer, unsupported shape, misaligned pointer, bad flags "
             "or workspace too small)";
    case IBWD_ERR_UNSUPPORTED_DEVICE:
      return "unsupported device (gfx950 / MI355X required)";
    case IBWD_ERR_HIP:
      return "HIP runtime or launch error";
    default:
      return "unknown status";
  }
}

int indexer_bwd_set_stage_hook(indexer_bwd_stage_hook_t hook, void* user) {
  ibwd::set_stage_hook(hook, user);
  return IBWD_OK;
}

}  // extern "C"
