// device_common.h -- device-side helpers shared by the prefill kernels (gfx950): vector
// types, buffer-descriptor loads, MFMA and exp2 wrappers, the work order of the grid.
#pragma once

#include <hip/hip_runtime.h>

namespace mixer {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int BN = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
// The reference max moves only when a score beats it by more than this many powers of two.
constexpr float kRescaleLog2Gap = 8.0f;
// 2^kRescaleLog2Gap: where the exponentials are taken before the reference is checked, a
// row's sum over one tile above this bound (which any probability above it forces) sends
// the tile back for a reference move.
constexpr float kTileSumBound = 256.0f;
// s_waitcnt immediate (gfx9 encoding): vmcnt = 0, expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVm0 = 0x0F70;

// ------------------------------------------------------------------ buffer access

// A raw buffer descriptor over `bytes` bytes at `base`; loads at offsets >= bytes return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes,
                                           0x00020000);
}

// Eight consecutive elements starting at element `e` as bf16 (fp32 is rounded to nearest
// even).
template <typename T>
__device__ __forceinline__ bf16x8 bload8(__amdgpu_buffer_rsrc_t r, int e);
template <>
__device__ __forceinline__ bf16x8 bload8<__bf16>(__amdgpu_buffer_rsrc_t r, int e) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, e * 2, 0, 0));
}
template <>
__device__ __forceinline__ bf16x8 bload8<float>(__amdgpu_buffer_rsrc_t r, int e) {
  const floatx4 a = __builtin_bit_cast(floatx4,
                                       __builtin_amdgcn_raw_buffer_load_b128(r, e * 4, 0, 0));
  const floatx4 b = __builtin_bit_cast(
      floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, e * 4 + 16, 0, 0));
  bf16x8 x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = (__bf16)a[i];
    x[i + 4] = (__bf16)b[i];
  }
  return x;
}

// Four consecutive elements.
template <typename T>
__device__ __forceinline__ bf16x4 bload4(__amdgpu_buffer_rsrc_t r, int e);
template <>
__device__ __forceinline__ bf16x4 bload4<__bf16>(__amdgpu_buffer_rsrc_t r, int e) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, e * 2, 0, 0));
}
template <>
__device__ __forceinline__ bf16x4 bload4<float>(__amdgpu_buffer_rsrc_t r, int e) {
  const floatx4 a = __builtin_bit_cast(floatx4,
                                       __builtin_amdgcn_raw_buffer_load_b128(r, e * 4, 0, 0));
  bf16x4 x;
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = (__bf16)a[i];
  return x;
}

// Four consecutive outputs.
__device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
  bf16x4 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  r[2] = (__bf16)c;
  r[3] = (__bf16)d;
  *reinterpret_cast<bf16x4*>(p) = r;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  floatx4 r;
  r[0] = a;
  r[1] = b;
  r[2] = c;
  r[3] = d;
  *reinterpret_cast<floatx4*>(p) = r;
}

// ------------------------------------------------------------------ math helpers

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// (batch*head, query tile) of workgroup `bid`. Workgroups are dealt to the 8 XCDs
// round-robin; when the head count is a multiple of 8, XCD (bid mod 8) takes a contiguous
// block of BH/8 heads, all their query tiles, so that a head's K/V (and that of query heads
// sharing one K/V head) is served from one L2.
// Causal layers go heaviest query tile first (the last tiles see the most keys), so that
// the light tiles fill the end. With `ascending` (the sliding window, where every tile past
// the first window costs the same) the short first-window tiles go first: the two
// workgroups that share a CU then start and end at different times, and one's prologue and
// epilogue overlap the other's key loop instead of coinciding with it. The workgroups in
// flight on an XCD then also hold neighbouring query tiles, whose windows share all but a
// few K/V tiles, so each K/V tile comes from HBM about once.
__device__ __forceinline__ void map_unit(int bid, int BH, int nq, int* bh, int* qt,
                                         bool ascending = false) {
  int rank;
  if ((BH & 7) == 0) {
    const int x = bid & 7, j = bid >> 3, hpx = BH >> 3;
    rank = j / hpx;
    *bh = x * hpx + j % hpx;
  } else {
    *bh = bid % BH;
    rank = bid / BH;
  }
  *qt = ascending ? rank : nq - 1 - rank;
}

// The same units, head by head: an XCD's (or, when the head count is not a multiple of 8,
// the grid's) heads one after another, each heaviest query tile first. Taken from a work
// queue in this order, the units in flight at once mostly belong to one head, whose K/V
// (4 MiB at L=8192, d=128) fits one L2, so fewer K/V tiles are fetched from HBM again.
__device__ __forceinline__ void map_unit_head_major(int bid, int BH, int nq, int* bh,
                                                    int* qt) {
  int head, rank;
  if ((BH & 7) == 0) {
    const int x = bid & 7, j = bid >> 3, hpx = BH >> 3;
    head = x * hpx + j / nq;
    rank = j % nq;
  } else {
    head = bid / nq;
    rank = bid % nq;
  }
  *bh = head;
  *qt = nq - 1 - rank;
}

}  // namespace mixer
