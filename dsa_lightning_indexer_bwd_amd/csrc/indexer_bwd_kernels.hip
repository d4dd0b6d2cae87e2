// Launch sequence of the lightning-indexer backward on gfx950.
//
//   two-pass route (default, bitwise deterministic):
//     row_prep_kernel   one wave per query row: softmax statistics, record
//                       layout by key range, per-slot record position and dI
//     row_export_kernel one wave per (query row, 32 heads): dQ, dW, slot records
//                     (key, dI, sign mask of S over h), (w*q)^T
//     dk_range_kernel one workgroup per (key range, query block): dK slabs in LDS
//     dk_sum_kernel   d_k = fixed-order sum of the query-block slabs
//   slot-row route (deterministic, for rows that select few keys per range):
//     row_prep_kernel   as above, ranges packed without alignment
//     row_export_kernel dQ, dW, and per valid slot its key and its dK row
//                       C = dI * sum_h [S>0] (w*q) (an MFMA product per chunk)
//     dk_rows_kernel    one wave per (32 keys, query block): the rows of its
//                       keys added in LDS in record order, into the slabs
//     dk_sum_kernel     as above
//   atomic route:
//     fill d_k with zeros, then row_kernel with fp32 atomic dK scatter
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "launch.h"

namespace {

// Scratch of the allocation-free entry point: one array per GPU, held until
// the process ends.  Host code never passes `scratch` itself to a kernel (in
// host code it names a host-side stand-in); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[ibwd::kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::once_flag g_scratch_once[kMaxScratchDevices];
void* g_scratch_ptr[kMaxScratchDevices];
hipError_t g_scratch_err[kMaxScratchDevices];

}  // namespace

namespace ibwd {

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    // with device `dev` current: its copy of the array
    g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

__global__ void zero_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

StageHook g_hook = nullptr;
void* g_hook_user = nullptr;

}  // namespace

void set_stage_hook(StageHook hook, void* user) {
  g_hook = hook;
  g_hook_user = user;
}

void stage_done(int stage, const char* kernel) {
  if (g_hook) g_hook(g_hook_user, stage, kernel);
}

hipError_t launch(Problem P, void* workspace, hipStream_t stream) {
  hipError_t err;
  const Layout L = make_layout(P.B, P.S_q, P.S_k, P.H, P.D, P.row_len, P.route == kDkSlotRows);
  P.rec_stride = L.rec_stride;
  P.RK = L.RK;
  P.NR = L.NR;
  P.NQB = L.NQB;
  P.QBS = L.QBS;
  P.nchunk = L.nchunk;
  P.HP = L.HP;
  if (P.route == kDkAtomic) {
    const int64_t n = P.B * P.S_k * P.D;
    zero_u32_kernel<<<1024, 256, 0, stream>>>(reinterpret_cast<uint32_t*>(P.dk), n);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    stage_done(0, "zero_u32_kernel");
    if ((err = launch_rows(P, stream)) != hipSuccess) return err;
    stage_done(1, "row_kernel");
    return hipSuccess;
  }
  char* ws = static_cast<char*>(workspace);
  if (P.route == kDkSlotRows) {
    P.offs = reinterpret_cast<int*>(ws + L.off_offs);
    P.slot = reinterpret_cast<int*>(ws + L.off_slot);
    P.skey = reinterpret_cast<int*>(ws + L.off_skey);
    P.crow = reinterpret_cast<uint16_t*>(ws + L.off_crow);
    P.slab = reinterpret_cast<float*>(ws + L.off_slab);
    if ((err = launch_rows_export(P, stream)) != hipSuccess) return err;  // stages 0, 1
    return launch_dk_rows(P, stream);  // stages 2, 3
  }
  P.rkd = reinterpret_cast<int*>(ws + L.off_rkd);
  P.rmask = reinterpret_cast<uint32_t*>(ws + L.off_rmask);
  P.offs = reinterpret_cast<int*>(ws + L.off_offs);
  P.slot = reinterpret_cast<int*>(ws + L.off_slot);
  P.qt = reinterpret_cast<uint16_t*>(ws + L.off_qt);
  P.slab = reinterpret_cast<float*>(ws + L.off_slab);
  if ((err = launch_rows_export(P, stream)) != hipSuccess) return err;  // stages 0, 1
  return launch_dk(P, stream);  // stages 2, 3
}

}  // namespace ibwd
