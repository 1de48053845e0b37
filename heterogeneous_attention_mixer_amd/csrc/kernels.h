// kernels.h -- internal interface between the host API (mixer_api.cpp) and the gfx950
// kernels (attn_prefill.hip). Not installed; the public ABI is include/mixer.h.
#pragma once

#include <hip/hip_runtime.h>

namespace mixer {

enum Variant { kFull = 0, kSliding = 1, kDifferential = 2 };

// One validated layer launch. Pointers are device pointers to bf16 (f32 == false) or fp32
// (f32 == true) tensors: q and out [B, H, L, d], k and v [B, Hkv, L, d]. Query head h of
// batch b reads K/V head b * Hkv + h / (H / Hkv), i.e. (b * H + h) / (H / Hkv).
struct PrefillLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int variant;
  int window;
  float lambda;
  int B, H, Hkv, L, d;
  bool f32;
};

// Enqueues the layer on `stream`; returns the launch status. bf16 layers run the LDS-DMA
// kernel (attn_prefill_dma.hip), fp32 layers the register-staged kernel (attn_prefill.hip),
// which splits q and k into bf16 high and low parts and rounds v to bf16 as it stages.
hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream);
hipError_t launch_prefill_dma(const PrefillLaunch& a, hipStream_t stream);
hipError_t launch_prefill_regstage(const PrefillLaunch& a, hipStream_t stream);

// An upper bound on the query tiles per (batch, head) of any kernel for a sequence of L
// tokens (every kernel's query tile holds at least 32 rows); host-side grid-size checks.
inline int max_grid_units(int L) { return (L + 31) / 32; }

// The matrix-core ceiling measurement (mfma_ceiling.hip): `blocks` workgroups of 4 waves,
// `iters` (a multiple of 4) instructions per accumulator chain, fragment sets of 8 x 64 x 8
// bf16 at `frags`, 4 x 16 x 64 floats per wave written to `sink`. Arguments are validated by
// the caller.
hipError_t launch_mfma_ceiling(const void* frags, int nsets, float* sink, int blocks, int iters,
                               hipStream_t stream);

}  // namespace mixer
