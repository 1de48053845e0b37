// Exercises libmixer's host code (built with host_stubs.cpp in place of the kernels) under
// AddressSanitizer and UndefinedBehaviorSanitizer: every validation path, size overflow
// guards, the Latin-square build and check (sec. 1, sec. 3.2 and Table 7 of "Placement Is
// Free, Composition Is Not"), the layer runner's launch order and its all-or-nothing
// validation, and the ceiling entry point. Prints "OK <checks>" and exits 0 when every check
// holds.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "kernels.h"
#include "mixer.h"

extern std::vector<mixer::PrefillLaunch> g_launches;
extern long g_fail_launch_at, g_launch_calls, g_fail_event_at;
extern int g_ceiling_calls;
extern int g_events;

static int g_checks = 0, g_fail = 0;
#define CHECK(cond)                                                        \
  do {                                                                     \
    ++g_checks;                                                            \
    if (!(cond)) {                                                         \
      ++g_fail;                                                            \
      std::printf("FAILED line %d: %s\n", __LINE__, #cond);                \
    }                                                                      \
  } while (0)

// Fake, never-dereferenced, 16-byte aligned device addresses far apart.
static void* P(int i) { return reinterpret_cast<void*>((uintptr_t)(0x100000000ull * (i + 1))); }

static int call(int variant, int window, float lam, int B, int H, int L, int d,
                void* q = P(0), void* k = P(1), void* v = P(2), void* o = P(3)) {
  return mixer_prefill_async(q, k, v, o, variant, window, lam, B, H, L, d, nullptr);
}

static void test_prefill_validation() {
  const size_t n0 = g_launches.size();
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 2, 64, 128) == MIXER_OK);
  CHECK(g_launches.size() == n0 + 1);
  const mixer::PrefillLaunch& a = g_launches.back();
  CHECK(a.variant == MIXER_FULL && a.window == 0 && a.lambda == 0.f && a.B == 1 && a.H == 2 &&
        a.Hkv == 2 && a.L == 64 && a.d == 128 && !a.f32 && a.q == P(0) && a.out == P(3));
  // window and lambda only reach the kernel for the variant that uses them
  CHECK(call(MIXER_FULL, 77, 0.5f, 1, 1, 8, 64) == MIXER_OK);
  CHECK(g_launches.back().window == 0 && g_launches.back().lambda == 0.f);
  CHECK(call(MIXER_SLIDING, 77, 0.5f, 1, 1, 8, 64) == MIXER_OK);
  CHECK(g_launches.back().window == 77 && g_launches.back().lambda == 0.f);
  CHECK(call(MIXER_DIFFERENTIAL, 77, 0.5f, 1, 1, 8, 64) == MIXER_OK);
  CHECK(g_launches.back().window == 0 && g_launches.back().lambda == 0.5f);

  const size_t n1 = g_launches.size();
  char* base = static_cast<char*>(P(5));
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, 8, 64, nullptr) == MIXER_EINVAL);
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, 8, 64, P(0), nullptr) == MIXER_EINVAL);
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, 8, 64, P(0), P(1), nullptr) == MIXER_EINVAL);
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, 8, 64, P(0), P(1), P(2), nullptr) == MIXER_EINVAL);
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, 8, 64, base + 8) == MIXER_EINVAL);  // unaligned
  CHECK(call(MIXER_FULL, 0, 0.f, 0, 1, 8, 64) == MIXER_EINVAL);
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 0, 8, 64) == MIXER_EINVAL);
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, 0, 64) == MIXER_EINVAL);
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, 8, 0) == MIXER_EINVAL);
  CHECK(call(MIXER_FULL, 0, 0.f, -1, 1, 8, 64) == MIXER_EINVAL);
  CHECK(call(3, 0, 0.f, 1, 1, 8, 64) == MIXER_EINVAL);
  CHECK(call(-1, 0, 0.f, 1, 1, 8, 64) == MIXER_EINVAL);
  CHECK(call(MIXER_SLIDING, 0, 0.f, 1, 1, 8, 64) == MIXER_EINVAL);
  CHECK(call(MIXER_SLIDING, -5, 0.f, 1, 1, 8, 64) == MIXER_EINVAL);
  CHECK(call(MIXER_DIFFERENTIAL, 0, NAN, 1, 1, 8, 64) == MIXER_EINVAL);
  CHECK(call(MIXER_DIFFERENTIAL, 0, INFINITY, 1, 1, 8, 64) == MIXER_EINVAL);
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, 8, 96) == MIXER_EUNSUPPORTED);
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, 8, 32) == MIXER_EUNSUPPORTED);
  // sizes whose products overflow 32 and 64 bits must be rejected without overflow
  CHECK(call(MIXER_FULL, 0, 0.f, INT_MAX, INT_MAX, INT_MAX, INT_MAX) == MIXER_EINVAL);
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, INT_MAX, 128) == MIXER_EUNSUPPORTED);
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1 << 20, 1 << 12, 64) == MIXER_EUNSUPPORTED);
  // out overlapping an input (same base, or a tail overlap)
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, 8, 64, P(0), P(1), P(2), P(0)) == MIXER_EINVAL);
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, 8, 64, P(0), P(1), P(2),
             static_cast<char*>(P(1)) + 512) == MIXER_EINVAL);
  // adjacent but disjoint (8 x 64 bf16 = 1 KiB per tensor)
  CHECK(call(MIXER_FULL, 0, 0.f, 1, 1, 8, 64, P(0), P(1), P(2),
             static_cast<char*>(P(2)) + 1024) == MIXER_OK);
  CHECK(g_launches.size() == n1 + 1);
}

static void test_gqa_and_f32() {
  const size_t n0 = g_launches.size();
  CHECK(mixer_prefill_gqa_async(P(0), P(1), P(2), P(3), MIXER_FULL, 0, 0.f, 2, 16, 4, 128, 128,
                                nullptr) == MIXER_OK);
  CHECK(g_launches.back().H == 16 && g_launches.back().Hkv == 4 && g_launches.back().B == 2);
  CHECK(mixer_prefill_gqa_async(P(0), P(1), P(2), P(3), MIXER_FULL, 0, 0.f, 1, 16, 3, 128, 128,
                                nullptr) == MIXER_EINVAL);
  CHECK(mixer_prefill_gqa_async(P(0), P(1), P(2), P(3), MIXER_FULL, 0, 0.f, 1, 16, 0, 128, 128,
                                nullptr) == MIXER_EINVAL);
  CHECK(mixer_prefill_gqa_async(P(0), P(1), P(2), P(3), MIXER_FULL, 0, 0.f, 1, 4, 8, 128, 128,
                                nullptr) == MIXER_EINVAL);
  CHECK(mixer_prefill_f32_async(static_cast<const float*>(P(0)), static_cast<const float*>(P(1)),
                                static_cast<const float*>(P(2)), static_cast<float*>(P(3)),
                                MIXER_SLIDING, 3, 0.f, 1, 2, 100, 64, nullptr) == MIXER_OK);
  CHECK(g_launches.back().f32 && g_launches.back().window == 3);
  CHECK(g_launches.size() == n0 + 2);
}

static void test_latin() {
  for (int N = 1; N <= 11; ++N) {
    std::vector<int> base(N), sched(N * N);
    for (int i = 0; i < N; ++i) base[i] = (N - 1 - i) * 3 + 1;  // any distinct labels
    CHECK(mixer_latin_build(N, base.data(), sched.data()) == MIXER_OK);
    bool cyc = true;
    for (int r = 0; r < N; ++r)
      for (int c = 0; c < N; ++c) cyc = cyc && sched[r * N + c] == base[(r + c) % N];
    CHECK(cyc);
    CHECK(mixer_latin_check(N, sched.data()) == 1);
    if (N >= 2) {
      std::vector<int> periodic(N * N);
      for (int i = 0; i < N * N; ++i) periodic[i] = base[i % N];  // columns constant
      CHECK(mixer_latin_check(N, periodic.data()) == 0);
      std::vector<int> block(N * N);
      for (int i = 0; i < N * N; ++i) block[i] = base[i / N];  // rows constant
      CHECK(mixer_latin_check(N, block.data()) == 0);
    }
  }
  int s[4] = {0, 1, 1, 0};
  CHECK(mixer_latin_check(0, s) == MIXER_EINVAL);
  CHECK(mixer_latin_check(2, nullptr) == MIXER_EINVAL);
  CHECK(mixer_latin_build(2, nullptr, s) == MIXER_EINVAL);
  CHECK(mixer_latin_build(2, s, nullptr) == MIXER_EINVAL);
  CHECK(mixer_latin_build(INT_MAX, s, s) == MIXER_EINVAL);
  CHECK(mixer_latin_check(INT_MAX, s) == MIXER_EINVAL);
  int dup[2] = {4, 4};  // repeated labels cannot form a Latin square
  int out[4];
  const int rc = mixer_latin_build(2, dup, out);
  CHECK(rc == MIXER_EINVAL || (rc == MIXER_OK && mixer_latin_check(2, out) == 0));
}

static void test_layers() {
  const int N = 3;
  int base[3] = {MIXER_FULL, MIXER_SLIDING, MIXER_DIFFERENTIAL};
  int sched[9];
  CHECK(mixer_latin_build(N, base, sched) == MIXER_OK);
  std::vector<void*> q(9), k(9), v(9), o(9), ev(10);
  for (int l = 0; l < 9; ++l) {
    q[l] = P(10 + 4 * l);
    k[l] = P(11 + 4 * l);
    v[l] = P(12 + 4 * l);
    o[l] = P(13 + 4 * l);
  }
  for (int e = 0; e < 10; ++e) ev[e] = P(100 + e);
  const size_t n0 = g_launches.size();
  const int e0 = g_events;
  CHECK(mixer_stack_prefill(N, sched, q.data(), k.data(), v.data(), o.data(), 16, 0.8f, 1, 2, 64,
                            128, nullptr, ev.data()) == MIXER_OK);
  CHECK(g_launches.size() == n0 + 9);
  CHECK(g_events == e0 + 10);
  for (int l = 0; l < 9 && g_launches.size() == n0 + 9; ++l) {
    const mixer::PrefillLaunch& a = g_launches[n0 + l];
    CHECK(a.variant == sched[l] && a.q == q[l] && a.out == o[l]);
  }
  // not Latin: nothing launched
  int periodic[9] = {0, 1, 2, 0, 1, 2, 0, 1, 2};
  const size_t n1 = g_launches.size();
  CHECK(mixer_stack_prefill(N, periodic, q.data(), k.data(), v.data(), o.data(), 16, 0.8f, 1, 2,
                            64, 128, nullptr, nullptr) == MIXER_ENOTLATIN);
  // the general runner takes it, in order
  CHECK(mixer_layers_prefill(9, periodic, q.data(), k.data(), v.data(), o.data(), 16, 0.8f, 1, 2,
                             64, 128, nullptr, nullptr) == MIXER_OK);
  CHECK(g_launches.size() == n1 + 9);
  // one bad layer: nothing launched
  const size_t n2 = g_launches.size();
  q[5] = nullptr;
  CHECK(mixer_layers_prefill(9, periodic, q.data(), k.data(), v.data(), o.data(), 16, 0.8f, 1, 2,
                             64, 128, nullptr, nullptr) == MIXER_EINVAL);
  q[5] = P(30);
  int bad_variant[9] = {0, 1, 2, 0, 7, 2, 0, 1, 2};
  CHECK(mixer_layers_prefill(9, bad_variant, q.data(), k.data(), v.data(), o.data(), 16, 0.8f,
                             1, 2, 64, 128, nullptr, nullptr) == MIXER_EINVAL);
  CHECK(g_launches.size() == n2);
  // NULL entries record nothing there: only the first and the last event here
  for (int e = 1; e < 9; ++e) ev[e] = nullptr;
  const int e1 = g_events;
  CHECK(mixer_layers_prefill(9, periodic, q.data(), k.data(), v.data(), o.data(), 16, 0.8f, 1, 2,
                             64, 128, nullptr, ev.data()) == MIXER_OK);
  CHECK(g_launches.size() == n2 + 9);
  CHECK(g_events == e1 + 2);
  for (int e = 1; e < 9; ++e) ev[e] = P(100 + e);
  CHECK(mixer_layers_prefill(0, periodic, q.data(), k.data(), v.data(), o.data(), 16, 0.8f, 1, 2,
                             64, 128, nullptr, nullptr) == MIXER_EINVAL);
  // A launch the runtime refuses part-way (layer 4): MIXER_EHIP, the layers before it stay
  // enqueued, none after it is launched.
  const size_t n3 = g_launches.size();
  g_fail_launch_at = g_launch_calls + 4;
  CHECK(mixer_stack_prefill(N, sched, q.data(), k.data(), v.data(), o.data(), 16, 0.8f, 1, 2, 64,
                            128, nullptr, ev.data()) == MIXER_EHIP);
  g_fail_launch_at = -1;
  CHECK(g_launches.size() == n3 + 4);
  for (int l = 0; l < 4 && g_launches.size() == n3 + 4; ++l)
    CHECK(g_launches[n3 + l].q == q[l] && g_launches[n3 + l].variant == sched[l]);
  // An event record refused after layer 2: MIXER_EHIP with layers 0..2 enqueued.
  const size_t n4 = g_launches.size();
  g_fail_event_at = g_events + 3;  // event 0 (before layer 0), then after layers 0, 1, 2
  CHECK(mixer_layers_prefill(9, periodic, q.data(), k.data(), v.data(), o.data(), 16, 0.8f, 1, 2,
                             64, 128, nullptr, ev.data()) == MIXER_EHIP);
  g_fail_event_at = -1;
  CHECK(g_launches.size() == n4 + 3);
  // The single-layer call reports a refused launch as MIXER_EHIP and records nothing.
  const size_t n5 = g_launches.size();
  g_fail_launch_at = g_launch_calls;
  CHECK(mixer_prefill_async(P(40), P(41), P(42), P(43), MIXER_FULL, 0, 0.f, 1, 2, 64, 128,
                            nullptr) == MIXER_EHIP);
  g_fail_launch_at = -1;
  CHECK(g_launches.size() == n5);
  CHECK(mixer_stack_prefill(INT_MAX, sched, q.data(), k.data(), v.data(), o.data(), 16, 0.8f, 1,
                            2, 64, 128, nullptr, nullptr) == MIXER_EINVAL);
}

static void test_ceiling() {
  const int c0 = g_ceiling_calls;
  float* sink = static_cast<float*>(P(200));
  CHECK(mixer_mfma_ceiling_async(P(199), 4, sink, 8, 16, nullptr) == MIXER_OK);
  CHECK(mixer_mfma_ceiling_async(nullptr, 4, sink, 8, 16, nullptr) == MIXER_EINVAL);
  CHECK(mixer_mfma_ceiling_async(P(199), 0, sink, 8, 16, nullptr) == MIXER_EINVAL);
  CHECK(mixer_mfma_ceiling_async(P(199), 4, sink, 0, 16, nullptr) == MIXER_EINVAL);
  CHECK(mixer_mfma_ceiling_async(P(199), 4, sink, 8, 18, nullptr) == MIXER_EINVAL);
  CHECK(mixer_mfma_ceiling_async(P(199), INT_MAX, sink, INT_MAX, 16, nullptr) == MIXER_EINVAL);
  CHECK(mixer_mfma_ceiling_async(P(199), 4, static_cast<float*>(P(199)), 8, 16, nullptr) ==
        MIXER_EINVAL);
  CHECK(g_ceiling_calls == c0 + 1);
}

int main() {
  test_prefill_validation();
  test_gqa_and_f32();
  test_latin();
  test_layers();
  test_ceiling();
  for (int code = -6; code <= 2; ++code) CHECK(mixer_strerror(code) != nullptr);
  if (g_fail) {
    std::printf("%d of %d checks failed\n", g_fail, g_checks);
    return 1;
  }
  std::printf("OK %d\n", g_checks);
  return 0;
}
