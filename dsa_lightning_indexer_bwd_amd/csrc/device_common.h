// Device helpers shared by the gfx950 kernels: MFMA wrappers, bf16 packing,
// LDS transpose reads and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ibwd {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

// v_mfma_f32_32x32x16_bf16.  Lane layouts (checked on the device):
//   A[m][k]: lane l holds m = l%32, k = 8*(l/32) + e   (e = 0..7)
//   B[k][n]: lane l holds n = l%32, k = 8*(l/32) + e
//   D[m][n]: lane l holds n = l%32, m = 8*i + 4*(l/32) + r in register 4*i + r
__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16.  Lane layouts (checked on the device):
//   A[m][k]: lane l holds m = l%16, k = 8*(l/16) + e
//   B[k][n]: lane l holds n = l%16, k = 8*(l/16) + e
//   D[m][n]: lane l holds n = l%16, m = 4*(l/16) + r in register r
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}
// One float -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint16_t bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (__bf16)v);
}
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

// ds_read_b64_tr_b16 (gfx950 LDS transpose read).  Within each 16-lane group,
// source lane s reads 4 consecutive bf16 at its own address; the result of lane
// i, element e is source lane (4e + i/4)'s element (i%4) (measured on the
// device).  With source lane s pointing at row (row0 + s/4), columns
// col0 + 4*(s%4) .. +3 of a row-major bf16 tile, lane i receives column
// col0 + i of rows row0 .. row0+3: a 4 x 16 block read transposed.
__device__ __forceinline__ uint2 lds_tr4(const unsigned char* tile, int pitch, int row0, int col0) {
  const int s = threadIdx.x & 15;
  const unsigned char* a = tile + (row0 + (s >> 2)) * pitch + (col0 + 4 * (s & 3)) * 2;
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(a));
  return __builtin_bit_cast(uint2, v);
}
// An MFMA operand of 8 k-values: rows [r0, r0+4) then [r1, r1+4) of a tile,
// at column col0 + (lane % 16).
__device__ __forceinline__ u32x4_t lds_tr8(const unsigned char* tile, int pitch, int r0, int r1,
                                           int col0) {
  const uint2 x = lds_tr4(tile, pitch, r0, col0);
  const uint2 y = lds_tr4(tile, pitch, r1, col0);
  return u32x4_t{x.x, x.y, y.x, y.y};
}

// Keep the compiler from moving LDS accesses across this point.  One wave's
// LDS operations execute in issue order, so this is all that lanes exchanging
// data through LDS inside one wave need.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The same ordering for the compiler only.  A wavefront-scope fence also
// waits for every outstanding global memory operation of the wave (gfx9
// counts loads and stores in one counter); lanes that exchange data through
// LDS within one wave need just the issue order, which this keeps, so loads
// in flight and stores just issued are not waited for.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// v_writelane_b32 through the compiler intrinsic, so that the backend knows
// the instruction and inserts the wait states it needs after the VALU write of
// the scalar source (a hand-written asm statement gets none).
extern "C" __device__ int __ibwd_writelane_i32(int val, int lane, int old) __asm(
    "llvm.amdgcn.writelane.i32");
// Lane `lane` of the result takes the wave-uniform `val`.
__device__ __forceinline__ uint32_t write_lane(uint32_t old, uint32_t val, int lane) {
  return uint32_t(__ibwd_writelane_i32(int(val), lane, int(old)));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }

// Key of a top-k id within its batch, or -1 for a padding slot.  base is 0
// for batch-local ids and b*S_k for ids into the flattened [B*S_k] keys of
// batch b.  With base + S_k <= 2^31 the unsigned difference lands in
// [0, S_k) exactly when base <= id < base + S_k: a negative id, or one below
// base, wraps to at least 2^31 - base >= S_k.
__device__ __forceinline__ int local_key(int id, int base, int S_k) {
  const uint32_t local = uint32_t(id) - uint32_t(base);
  return local < uint32_t(S_k) ? int(local) : -1;
}

// Softmax statistics of one query row over its valid slots, in base 2: with
// c2 = sm_scale*log2(e), m2 = max_j c2*I_j and invZ = 1 / sum_j 2^(c2*I_j - m2)
// over the slots j < n whose key_of(j, id_at(j)) >= 0.  One pass: each lane
// keeps a running max and a sum rescaled to it, then the wave combines them.
// c2*I is rounded before any max is subtracted (no contraction into a
// multiply-add), so the largest logit contributes 2^0 = 1 exactly.
// on_group(g, j, key) is called by every lane, in uniform control flow, once per
// slot position j = 64g + lane (key < 0 for padding and positions past n).  With
// MAXN > 0 (rows of at most MAXN slots) the loop is unrolled and g is a constant.
// Both row kernels use this and slot_dI, so their dI agree bit for bit.
template <int MAXN = 0, typename IdAt, typename KeyOf, typename OnGroup>
__device__ __forceinline__ float2 row_softmax_stats(int n, const float* __restrict__ Irow, float c2,
                                                    IdAt id_at, KeyOf key_of, OnGroup on_group) {
#pragma clang fp contract(off)
  constexpr int kU = 8;  // loads in flight per lane
  const int lane = threadIdx.x & 63;
  float m2 = -INFINITY, z = 0.f;
  auto batch = [&](int j0) {
    int idv[kU];
    float iv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = j0 + 64 * u + lane;
      const int jc = j < n ? j : n - 1;
      idv[u] = id_at(jc);
      iv[u] = Irow[jc];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int key = key_of(j0 + 64 * u + lane, idv[u]);
      if (key >= 0) {
        const float v = c2 * iv[u];
        const float mn = fmaxf(m2, v);
        z = z * __builtin_amdgcn_exp2f(m2 - mn) + __builtin_amdgcn_exp2f(v - mn);
        m2 = mn;
      }
      if (j0 + 64 * u < n) on_group((j0 >> 6) + u, j0 + 64 * u + lane, key);
    }
  };
  if constexpr (MAXN > 0) {
    // n <= MAXN: unrolled, so that on_group's group index is a constant
#pragma unroll
    for (int j0 = 0; j0 < MAXN; j0 += 64 * kU)
      if (j0 < n) batch(j0);
  } else {
    for (int j0 = 0; j0 < n; j0 += 64 * kU) batch(j0);
  }
  const float mw = wave_max(m2);
  z = m2 > -INFINITY ? z * __builtin_amdgcn_exp2f(m2 - mw) : 0.f;
  z = wave_sum(z);
  return make_float2(mw, z > 0.f ? 1.f / z : 0.f);
}

// dI of one valid slot: coef * (softmax - p), coef = grad_loss * sm_scale.
__device__ __forceinline__ float slot_dI(float I, float p, float c2, float m2, float invZ,
                                         float coef) {
#pragma clang fp contract(off)
  return coef * (__builtin_amdgcn_exp2f(c2 * I - m2) * invZ - p);
}
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = threadIdx.x & 63;
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}
// Set bits of m at lanes below this one (v_mbcnt; m may differ per lane).
__device__ __forceinline__ int bits_below(uint64_t m) {
  return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
}

}  // namespace ibwd
