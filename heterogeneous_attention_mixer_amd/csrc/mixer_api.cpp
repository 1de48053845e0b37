// mixer_api.cpp -- the C ABI of libmixer.so (declared in include/mixer.h): argument
// validation (host only, before any HIP call), kernel dispatch, the Latin-square scheduler
// and error strings.
//
// Latin squares follow sec. 1 and sec. 3.2 of "Placement Is Free, Composition Is Not: The
// Latin Square as a Provably-Balanced Construction for Heterogeneous Sequence-Mixer Stacks":
// N types over N*N layers, each type once per row and once per column; Table 7 prints the
// 4x4 cyclic instance row by row.
#include <math.h>
#include <stdint.h>

#include <vector>

#include "../../include/mixer.h"
#include "kernels.h"

namespace {

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

// Host-only checks of one layer (q and out [B, H, L, d], k and v [B, Hkv, L, d]); fills
// `out` on success.
int validate(const void* q, const void* k, const void* v, void* o, int variant, int window,
             float lambda, int B, int H, int Hkv, int L, int d, bool f32,
             mixer::PrefillLaunch* out) {
  if (!q || !k || !v || !o) return MIXER_EINVAL;
  // The kernels move 16-byte vectors: every tensor must start on a 16-byte boundary.
  for (const void* p : {q, k, v, static_cast<const void*>(o)})
    if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return MIXER_EINVAL;
  if (B < 1 || H < 1 || Hkv < 1 || L < 1 || d < 1) return MIXER_EINVAL;
  if (H % Hkv != 0) return MIXER_EINVAL;
  if (variant != MIXER_FULL && variant != MIXER_SLIDING && variant != MIXER_DIFFERENTIAL)
    return MIXER_EINVAL;
  if (variant == MIXER_SLIDING && window < 1) return MIXER_EINVAL;
  if (variant == MIXER_DIFFERENTIAL && !isfinite(lambda)) return MIXER_EINVAL;
  // Element count and byte size must fit comfortably in 64-bit indexing.
  const unsigned __int128 elems = (unsigned __int128)B * H * L * d;
  const size_t esz = f32 ? 4 : 2;
  if (elems * esz >= ((unsigned __int128)1 << 62)) return MIXER_EINVAL;
  if (d != 64 && d != 128) return MIXER_EUNSUPPORTED;
  // One head's L x d slice is addressed with 32-bit byte offsets.
  if ((unsigned __int128)L * d * esz >= ((unsigned __int128)1 << 31)) return MIXER_EUNSUPPORTED;
  // One workgroup of 256 threads per (batch, head, query tile): the grid must fit in 32 bits
  // of threads.
  const unsigned __int128 wgs = (unsigned __int128)B * H * mixer::max_grid_units(L);
  if (wgs * 256 >= ((unsigned __int128)1 << 32)) return MIXER_EUNSUPPORTED;
  const size_t bytes = (size_t)elems * esz;
  const size_t kv_bytes = bytes / H * Hkv;
  if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, kv_bytes) ||
      overlaps(o, bytes, v, kv_bytes))
    return MIXER_EINVAL;
  out->q = q;
  out->k = k;
  out->v = v;
  out->out = o;
  out->variant = variant;
  out->window = variant == MIXER_SLIDING ? window : 0;
  out->lambda = variant == MIXER_DIFFERENTIAL ? lambda : 0.0f;
  out->B = B;
  out->H = H;
  out->Hkv = Hkv;
  out->L = L;
  out->d = d;
  out->f32 = f32;
  return MIXER_OK;
}

int launch(const mixer::PrefillLaunch& a, void* stream) {
  const hipError_t e = mixer::launch_prefill(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MIXER_OK : MIXER_EHIP;
}

}  // namespace

extern "C" {

int mixer_prefill_async(const void* q, const void* k, const void* v, void* out, int variant,
                        int window, float lambda, int B, int H, int L, int d, void* stream) {
  mixer::PrefillLaunch a;
  const int rc = validate(q, k, v, out, variant, window, lambda, B, H, H, L, d, false, &a);
  if (rc != MIXER_OK) return rc;
  return launch(a, stream);
}

int mixer_prefill_gqa_async(const void* q, const void* k, const void* v, void* out, int variant,
                            int window, float lambda, int B, int H, int Hkv, int L, int d,
                            void* stream) {
  mixer::PrefillLaunch a;
  const int rc = validate(q, k, v, out, variant, window, lambda, B, H, Hkv, L, d, false, &a);
  if (rc != MIXER_OK) return rc;
  return launch(a, stream);
}

int mixer_prefill(const void* q, const void* k, const void* v, void* out, int variant,
                  int window, float lambda, int B, int H, int L, int d) {
  return mixer_prefill_async(q, k, v, out, variant, window, lambda, B, H, L, d, nullptr);
}

int mixer_prefill_f32_async(const float* q, const float* k, const float* v, float* out,
                            int variant, int window, float lambda, int B, int H, int L, int d,
                            void* stream) {
  mixer::PrefillLaunch a;
  const int rc = validate(q, k, v, out, variant, window, lambda, B, H, H, L, d, true, &a);
  if (rc != MIXER_OK) return rc;
  return launch(a, stream);
}

// Largest order accepted by the scheduler calls (N*N must not overflow an int).
constexpr int kMaxOrder = 46340;

int mixer_latin_build(int N, const int* base, int* sched) {
  if (N < 1 || N > kMaxOrder || !base || !sched) return MIXER_EINVAL;
  for (int r = 0; r < N; ++r)
    for (int c = 0; c < N; ++c) sched[r * N + c] = base[(r + c) % N];
  return MIXER_OK;
}

int mixer_latin_check(int N, const int* sched) {
  if (N < 1 || N > kMaxOrder || !sched) return MIXER_EINVAL;
  // The N distinct types of the grid, in order of first appearance.
  std::vector<int> types;
  for (int i = 0; i < N * N; ++i) {
    bool seen = false;
    for (int t : types) seen = seen || (t == sched[i]);
    if (!seen) {
      if ((int)types.size() == N) return 0;  // more than N types
      types.push_back(sched[i]);
    }
  }
  if ((int)types.size() != N) return 0;
  // With exactly N types, each type appearing once in every row is the same as no repeat
  // within a row (same for columns).
  for (int r = 0; r < N; ++r)
    for (int c = 0; c < N; ++c)
      for (int c2 = c + 1; c2 < N; ++c2)
        if (sched[r * N + c] == sched[r * N + c2]) return 0;
  for (int c = 0; c < N; ++c)
    for (int r = 0; r < N; ++r)
      for (int r2 = r + 1; r2 < N; ++r2)
        if (sched[r * N + c] == sched[r2 * N + c]) return 0;
  return 1;
}

int mixer_layers_prefill(int n, const int* variants, const void* const* q,
                         const void* const* k, const void* const* v, void* const* out,
                         int window, float lambda, int B, int H, int L, int d, void* stream,
                         void* const* layer_events) {
  if (n < 1 || !variants || !q || !k || !v || !out) return MIXER_EINVAL;
  std::vector<mixer::PrefillLaunch> layers((size_t)n);
  for (int l = 0; l < n; ++l) {
    const int rc = validate(q[l], k[l], v[l], out[l], variants[l], window, lambda, B, H, H, L,
                            d, false, &layers[(size_t)l]);
    if (rc != MIXER_OK) return rc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Records event i where the caller asked for one (a NULL entry records nothing).
  auto mark = [&](int i) {
    return !layer_events || !layer_events[i] ||
           hipEventRecord(static_cast<hipEvent_t>(layer_events[i]), s) == hipSuccess;
  };
  if (!mark(0)) return MIXER_EHIP;
  for (int l = 0; l < n; ++l) {
    const int rc = launch(layers[(size_t)l], stream);
    if (rc != MIXER_OK) return rc;
    if (!mark(l + 1)) return MIXER_EHIP;
  }
  return MIXER_OK;
}

int mixer_stack_prefill(int N, const int* sched, const void* const* q, const void* const* k,
                        const void* const* v, void* const* out, int window, float lambda,
                        int B, int H, int L, int d, void* stream, void* const* layer_events) {
  if (N < 1 || N > kMaxOrder || !sched || !q || !k || !v || !out) return MIXER_EINVAL;
  const int lc = mixer_latin_check(N, sched);
  if (lc < 0) return lc;
  if (lc == 0) return MIXER_ENOTLATIN;
  return mixer_layers_prefill(N * N, sched, q, k, v, out, window, lambda, B, H, L, d, stream,
                              layer_events);
}

int mixer_mfma_ceiling_async(const void* frags, int nsets, float* sink, int blocks, int iters,
                             void* stream) {
  if (!frags || !sink) return MIXER_EINVAL;
  if ((reinterpret_cast<uintptr_t>(frags) | reinterpret_cast<uintptr_t>(sink)) & 15)
    return MIXER_EINVAL;
  if (nsets < 1 || nsets > (1 << 20) || blocks < 1 || blocks > (1 << 20)) return MIXER_EINVAL;
  if (iters < 4 || iters % 4 != 0) return MIXER_EINVAL;
  const size_t frag_bytes = (size_t)nsets * 8 * 64 * 16;
  const size_t sink_bytes = (size_t)blocks * 4 * 4 * 16 * 64 * sizeof(float);
  if (overlaps(frags, frag_bytes, sink, sink_bytes)) return MIXER_EINVAL;
  return mixer::launch_mfma_ceiling(frags, nsets, sink, blocks, iters,
                                    static_cast<hipStream_t>(stream)) == hipSuccess
             ? MIXER_OK
             : MIXER_EHIP;
}

const char* mixer_strerror(int status) {
  switch (status) {
    case MIXER_OK: return "success";
    case MIXER_EINVAL: return "invalid argument";
    case MIXER_EUNSUPPORTED: return "unsupported configuration (head dim must be 64 or 128)";
    case MIXER_ENOTLATIN: return "schedule is not a Latin square";
    case MIXER_EHIP: return "HIP runtime error at launch";
    default: return "unknown mixer status";
  }
}

}  // extern "C"
