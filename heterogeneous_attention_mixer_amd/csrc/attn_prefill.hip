// attn_prefill.hip -- flash-style causal prefill of one sequence-mixer layer for gfx950, for
// fp32 inputs and outputs. K and V are staged through registers (an LDS DMA cannot convert).
// Q and K are split into bf16 high and low parts, and each score is Khi Qhi + Khi Qlo +
// Klo Qhi on the matrix cores, so the scores keep nearly fp32 accuracy whatever their
// magnitude; V is rounded to bf16, as the probabilities are. The rest follows the bf16
// kernel in attn_prefill_dma.hip. Only the small fp32 workload uses it, so it is not tuned.
//
// Variants (Table 1, sec. 3.1 of "Placement Is Free, Composition Is Not: The Latin Square as
// a Provably-Balanced Construction for Heterogeneous Sequence-Mixer Stacks"):
//   full          causal softmax attention, scale 1/sqrt(d);
//   sliding       the same inside a causal window of W keys (query included);
//   differential  two causal softmax maps over the two halves of the head dimension, scale
//                 1/sqrt(d/2), combined as (P1 - lambda * P2) V with full-width V.
//
// Design (one workgroup = one (batch, head) and a block of query rows, 32 rows per wave):
//   * The scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K is
//     the A operand (read from LDS), Q the B operand (kept in registers for the whole
//     kernel). In the 32x32 accumulator a lane owns one query column and 16 key rows, so the
//     row max and row sum of the softmax are in-lane except for one exchange with lane^32.
//   * The same accumulator registers, rounded to bf16, are exactly the B operand of
//     O^T += V^T P^T: P never leaves the registers. V is staged into LDS transposed (V^T,
//     head-dim rows, key columns) with the key order permuted to match the accumulator
//     layout, so each A operand is one 16-byte LDS read.
//   * Online softmax in fp32 with exp2 (the scale is folded with log2(e)). The reference max
//     of a row is only moved when a new score exceeds it by more than 2^8 in probability
//     units, so the accumulator rescale (64 multiplies per lane) runs a few times per row
//     instead of on most tiles; probabilities stay below 256, far from fp32/bf16 limits.
//     The row sums are taken over the bf16-rounded probabilities (v_dot2 against ones), the
//     exact weights the value product uses.
//   * The differential variant gives each of its two softmax maps its own wave: the two
//     waves of a row block read the same K/V tiles (scores on their half of the head dim,
//     values on all of it) and meet once, at the end, through LDS. Each wave then carries
//     one accumulator set, so it fits the register budget of two waves per SIMD.
//   * Key tiles of 64 keys, double-buffered in LDS (one barrier per tile); the next tile's
//     K/V is fetched with buffer loads while the current tile is computed. Each head's
//     tensors get their own buffer descriptor, so reads past the sequence end return zeros
//     and need no clamping. Tiles no query of the workgroup can see are never loaded, tiles
//     a wave cannot see are skipped by that wave, and the element mask is applied only on
//     tiles that cross the diagonal or the window edge.
//   * Work order: the heaviest query tiles (most visible keys) are dispatched first, and when
//     the head count allows, all query tiles of a head land on the same XCD (workgroups are
//     dealt to the 8 XCDs round-robin), so a head's K/V is served from one L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace mixer {

// One softmax map of one wave over one key tile.
//   s     raw scores of the lane's query against its 32 keys of the tile (masked = -inf);
//         on return, the probabilities exp2(c * (s - m)) rounded to bf16 are in `pf`;
//   m     the row's reference max (raw score units), equal in lanes lane and lane^32;
//   l     the lane's partial row sum (the other half lives in lane^32);
//   o     the accumulators, rescaled when the reference max moves.
template <int DB>
__device__ __forceinline__ void softmax_step(floatx16 (&s)[2], float& m, float& l,
                                             floatx16 (&o)[DB], bf16x8 (&pf)[2][2], float c,
                                             float gap) {
  float tmax = s[0][0];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[kb][r]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  // Move the reference (and rescale) only if some row of the wave needs it. A row that has
  // seen no visible key yet has m = -inf and moves as soon as it sees one.
  if (__any(tmax > m + gap)) {
    const float m_new = fmaxf(m, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2((m - m_new) * c);
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    m = m_new;
  }
  const float mc = (m == -INFINITY) ? 0.0f : m * c;
  bf16x2 ones;
  ones[0] = (__bf16)1.0f;
  ones[1] = (__bf16)1.0f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        bf16x2 pp;
        pp[0] = (__bf16)fast_exp2(__builtin_fmaf(s[kb][h * 8 + e], c, -mc));
        pp[1] = (__bf16)fast_exp2(__builtin_fmaf(s[kb][h * 8 + e + 1], c, -mc));
        pf[kb][h][e] = pp[0];
        pf[kb][h][e + 1] = pp[1];
        l = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, l, false);
      }
}

// Eight fp32 values as two bf16 vectors: hi = x rounded to bf16, lo = (x - hi) rounded to
// bf16. hi + lo equals x to within 2^-16 of |x|, so products of split operands carry scores
// to nearly fp32 accuracy on the bf16 matrix cores.
__device__ __forceinline__ void split8(const floatx4& a, const floatx4& b, bf16x8& hi,
                                       bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = (__bf16)a[i];
    lo[i] = (__bf16)(a[i] - (float)hi[i]);
    hi[i + 4] = (__bf16)b[i];
    lo[i + 4] = (__bf16)(b[i] - (float)hi[i + 4]);
  }
}

__device__ __forceinline__ floatx4 fload4(__amdgpu_buffer_rsrc_t r, int e) {
  return __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, e * 4, 0, 0));
}

// ------------------------------------------------------------------ the kernel

// Per-variant launch shape. A workgroup covers `rows` blocks of 32 query rows of one
// (batch, head). Full and sliding: one wave per row block. Differential: two waves per row
// block, one per softmax map (map 0 on head-dim channels [0, d/2), map 1 on [d/2, d)); both
// stream the same K/V tiles from LDS and combine their outputs through LDS at the end, so
// each wave holds one accumulator set, like a full-attention wave with half-width scores.
template <int VAR>
struct Shape {
  static constexpr int maps = (VAR == kDifferential) ? 2 : 1;
  static constexpr int rows = 4;
  static constexpr int waves = rows * maps;
  static constexpr int threads = waves * kWave;
  static constexpr int bm = 32 * rows;  // query rows per workgroup
};
// Waves per SIMD the register allocation targets. At d=128 the split K tiles take 104 KiB
// of LDS, one workgroup per CU: one wave per SIMD for full and sliding (4 waves), two for
// the differential (8 waves). At d=64 (54 KiB) two workgroups fit.
template <int D, int VAR>
constexpr int kOccupancy = (D == 128 && VAR != kDifferential) ? 1 : 2;

template <int D, int VAR>
__global__ void __attribute__((amdgpu_flat_work_group_size(Shape<VAR>::threads,
                                                           Shape<VAR>::threads),
                               amdgpu_waves_per_eu(kOccupancy<D, VAR>, kOccupancy<D, VAR>)))
prefill_kernel(const float* __restrict__ qg, const float* __restrict__ kg,
               const float* __restrict__ vg, float* __restrict__ og, int L, int BH, int G,
               int nq, int window, float lambda) {
  constexpr bool kDiff = (VAR == kDifferential);
  constexpr bool kSlide = (VAR == kSliding);
  constexpr int kThreads = Shape<VAR>::threads;
  constexpr int kRows = Shape<VAR>::rows;
  constexpr int BM = Shape<VAR>::bm;
  constexpr int KSTEPS = D / 16;          // MFMA steps over the head dim
  constexpr int NQ = KSTEPS / Shape<VAR>::maps;  // ... over one map's score channels
  constexpr int DB = D / 32;              // 32-row blocks of the head dim in O^T
  constexpr int KP = D + 8;               // K tile row pitch (elements), 16 B pad
  constexpr int VP = BN + 8;              // V^T tile row pitch (elements), 16 B pad
  constexpr int KCH = BN * D / 8;         // 16-byte chunks of a K tile
  constexpr int KPT = KCH / kThreads;     // ... per thread
  // V is staged in units of 4 keys x VC channels, transposed in registers: VC = 8 when that
  // gives every thread a unit, else 4.
  constexpr int VC = ((BN / 4) * (D / 8) >= kThreads) ? 8 : 4;
  constexpr int VUN = (BN / 4) * (D / VC);
  constexpr int VPT = (VUN + kThreads - 1) / kThreads;
  static_assert(KCH % kThreads == 0, "K tile staging");
  typedef __bf16 vcvec __attribute__((ext_vector_type(VC)));

  // LDS: two buffers each of the K tile's high parts, its low parts and the V^T tile (tile
  // kt is computed from buffer kt & 1 while tile kt + 1 is written into the other one);
  // after the key loop the differential reuses the space to pass map 1's scaled output to
  // map 0.
  constexpr int kKsElems = BN * KP, kVtElems = D * VP;
  constexpr int kTileBytes = 2 * (2 * kKsElems + kVtElems) * 2;
  constexpr int kXchBytes = kDiff ? kRows * 64 * (DB * 16) * 4 : 0;
  constexpr int kSmemBytes = kTileBytes > kXchBytes ? kTileBytes : kXchBytes;
  __shared__ __attribute__((aligned(16))) char smem[kSmemBytes];
  __bf16* const Ks0 = reinterpret_cast<__bf16*>(smem);
  __bf16* const Vt0 = Ks0 + 2 * kKsElems;
  __bf16* const Kl0 = Vt0 + 2 * kVtElems;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rb = wave % kRows;            // row block of this wave
  const int map = wave / kRows;           // softmax map of this wave (differential)
  const int lr = lane & 31;  // query column owned in the accumulators
  const int lg = lane >> 5;  // lane half

  int bh, qt;
  map_unit(blockIdx.x, BH, nq, &bh, &qt);
  const int q0 = qt * BM;
  const int qw = q0 + rb * 32;    // first query row of this wave
  const int qi = qw + lr;         // this lane's query row
  const size_t head = (size_t)bh * (size_t)L * D;         // q and out
  const size_t kv_head = (size_t)(bh / G) * (size_t)L * D;  // k and v: G query heads each
  const int head_bytes = L * D * (int)sizeof(float);
  const __amdgpu_buffer_rsrc_t Qr = make_rsrc(qg + head, head_bytes);
  const __amdgpu_buffer_rsrc_t Kr = make_rsrc(kg + kv_head, head_bytes);
  const __amdgpu_buffer_rsrc_t Vr = make_rsrc(vg + kv_head, head_bytes);

  const float c = kLog2e / __builtin_sqrtf(kDiff ? (float)(D / 2) : (float)D);
  const float gap = kRescaleLog2Gap / c;
  // First score channel of this wave's map.
  const int ch0 = kDiff ? map * (D / 2) : 0;

  // Q fragments (B operand of S^T = K Q^T), high and low bf16 parts: lane holds row qi,
  // channels ch0 + kk*16 + lg*8 + [0,8). Rows past L read zeros and are never stored.
  bf16x8 qf[NQ], ql[NQ];
#pragma unroll
  for (int kk = 0; kk < NQ; ++kk) {
    const int e = qi * D + ch0 + kk * 16 + lg * 8;
    split8(fload4(Qr, e), fload4(Qr, e + 4), qf[kk], ql[kk]);
  }
  // Wait for Q here, once: otherwise the wait-count insertion cannot prove inside the key
  // loop that Q has arrived, and makes every tile's first score products wait for all
  // vector loads in flight, the next tile's prefetch included.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // Key tiles this workgroup can see.
  const int q_last = min(q0 + BM, L) - 1;
  int kt_lo = 0;
  if (kSlide) {
    const int lo = q0 - window + 1;
    kt_lo = lo > 0 ? lo / BN : 0;
  }
  const int kt_hi = q_last / BN;

  // Accumulators and softmax state of this wave's map.
  floatx16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;

  // Register staging of one K/V tile (element offsets within the head; keys past L read 0).
  // K stays fp32 until it is split into LDS; V is rounded to bf16 as it loads.
  floatx4 kreg[KPT][2];
  vcvec vreg[VPT][4];
  auto fetch = [&](int kt) {
    const int k0 = kt * BN;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / (D / 8), ch = idx % (D / 8);
      kreg[i][0] = fload4(Kr, (k0 + row) * D + ch * 8);
      kreg[i][1] = fload4(Kr, (k0 + row) * D + ch * 8 + 4);
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int u = tid + i * kThreads;
      if (VUN % kThreads == 0 || u < VUN) {
        const int a4 = u % (BN / 4), cc = u / (BN / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int off = (k0 + a4 * 4 + r) * D + cc * VC;
          if constexpr (VC == 8)
            vreg[i][r] = bload8<float>(Vr, off);
          else
            vreg[i][r] = bload4<float>(Vr, off);
        }
      }
    }
  };
  auto stage = [&](int buf) {
    __bf16* const Ks = Ks0 + buf * kKsElems;
    __bf16* const Kl = Kl0 + buf * kKsElems;
    __bf16* const Vt = Vt0 + buf * kVtElems;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / (D / 8), ch = idx % (D / 8);
      bf16x8 hi, lo;
      split8(kreg[i][0], kreg[i][1], hi, lo);
      *reinterpret_cast<bf16x8*>(&Ks[row * KP + ch * 8]) = hi;
      *reinterpret_cast<bf16x8*>(&Kl[row * KP + ch * 8]) = lo;
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int u = tid + i * kThreads;
      if (VUN % kThreads == 0 || u < VUN) {
        const int a4 = u % (BN / 4), cc = u / (BN / 4);
        // Keys 4*a4 .. 4*a4+3 go to column group (a4/4)*16 + perm(a4 % 4)*4 of V^T, with
        // perm = {0, 2, 1, 3}: the order in which the accumulator layout hands out keys.
        const int grp = a4 & 3;
        const int col = (a4 >> 2) * 16 + ((grp == 1) ? 2 : (grp == 2) ? 1 : grp) * 4;
#pragma unroll
        for (int e = 0; e < VC; ++e) {
          bf16x4 t;
          t[0] = vreg[i][0][e];
          t[1] = vreg[i][1][e];
          t[2] = vreg[i][2][e];
          t[3] = vreg[i][3][e];
          *reinterpret_cast<bf16x4*>(&Vt[(cc * VC + e) * VP + col]) = t;
        }
      }
    }
  };

  fetch(kt_lo);
  stage(kt_lo & 1);
  __syncthreads();
  for (int kt = kt_lo; kt <= kt_hi; ++kt) {
    const int buf = kt & 1;
    if (kt < kt_hi) fetch(kt + 1);  // in flight while this tile is computed

    const int k0 = kt * BN;
    // Does this wave see any key of the tile? (rows qw..qw+31 see keys
    // [qw - W + 1, qw + 31] together.)
    bool any = (qw < L) && (k0 <= qw + 31);
    if (kSlide) any = any && (k0 + BN - 1 >= qw - window + 1);
    if (any) {
      // Does every row of the wave see every key of the tile?
      bool full_tile = (k0 + BN - 1 <= qw);
      if (kSlide) full_tile = full_tile && (qw + 31 - k0 < window);
      const __bf16* const Ks = Ks0 + buf * kKsElems;
      const __bf16* const Kl = Kl0 + buf * kKsElems;
      const __bf16* const Vt = Vt0 + buf * kVtElems;

      // ---- scores S^T = K Q^T for 64 keys x 32 queries (two 32x32 blocks) over this
      // wave's score channels, from the split operands: Khi Qhi + Khi Qlo + Klo Qhi (the
      // dropped Klo Qlo term is below 2^-16 of each product)
      floatx16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
        const int koff = (kb * 32 + lr) * KP + ch0 + lg * 8;
#pragma unroll
        for (int kk = 0; kk < NQ; ++kk) {
          const bf16x8 khi = *reinterpret_cast<const bf16x8*>(&Ks[koff + kk * 16]);
          const bf16x8 klo = *reinterpret_cast<const bf16x8*>(&Kl[koff + kk * 16]);
          s[kb] = mfma32(khi, qf[kk], s[kb]);
          s[kb] = mfma32(khi, ql[kk], s[kb]);
          s[kb] = mfma32(klo, qf[kk], s[kb]);
        }
      }
      // ---- mask on tiles that cross the diagonal or the window edge
      if (!full_tile) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kj = k0 + kb * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
            bool vis = kj <= qi;
            if (kSlide) vis = vis && (qi - kj < window);
            if (!vis) s[kb][r] = -INFINITY;
          }
      }
      // ---- online softmax, then O^T += V^T P^T
      bf16x8 p[2][2];
      softmax_step<DB>(s, m, l, o, p, c, gap);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const __bf16* vrow = &Vt[(db * 32 + lr) * VP + lg * 8];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            o[db] = mfma32(*reinterpret_cast<const bf16x8*>(vrow + kb * 32 + h * 16),
                           p[kb][h], o[db]);
      }
    }
    if (kt < kt_hi) stage(buf ^ 1);  // that buffer was released by the previous barrier
    __syncthreads();
  }

  // ---- epilogue: out = O / l; differential: out = O1 / l1 - lambda * O2 / l2, with map 1's
  // term passed to map 0 through LDS (the key loop ended with a barrier, so the tile buffers
  // are free). Lanes lane and lane^32 hold the same query row. Element (db, r) of a lane is
  // head-dim channel db*32 + 8*(r/4) + 4*lg + r%4 of query qi.
  const float lsum = l + __shfl_xor(l, 32);
  if constexpr (kDiff) {
    float* const xch = reinterpret_cast<float*>(smem) + rb * 64 * (DB * 16);
    if (map == 1) {
      const float sc = lambda / lsum;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[(db * 16 + r) * 64 + lane] = o[db][r] * sc;
    }
    __syncthreads();
    if (map == 1) return;
  }
  if (qi < L) {
    const float inv = 1.0f / lsum;
    const float* const xch = reinterpret_cast<const float*>(smem) + rb * 64 * (DB * 16);
    float* orow = og + head + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = o[db][r4 * 4 + e] * inv;
          if constexpr (kDiff) x[e] -= xch[(db * 16 + r4 * 4 + e) * 64 + lane];
        }
        store4(orow + db * 32 + 8 * r4 + 4 * lg, x[0], x[1], x[2], x[3]);
      }
  }
}

// ------------------------------------------------------------------ launch

template <int D, int VAR>
static hipError_t launch_t(const PrefillLaunch& a, hipStream_t stream) {
  constexpr int BM = Shape<VAR>::bm;
  const int nq = (a.L + BM - 1) / BM;
  const int BH = a.B * a.H;
  const dim3 grid((unsigned)(BH * nq));
  hipLaunchKernelGGL((prefill_kernel<D, VAR>), grid, dim3(Shape<VAR>::threads), 0, stream,
                     static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                     static_cast<const float*>(a.v), static_cast<float*>(a.out), a.L, BH,
                     a.H / a.Hkv, nq, a.window, a.lambda);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_v(const PrefillLaunch& a, hipStream_t stream) {
  switch (a.variant) {
    case kFull: return launch_t<D, kFull>(a, stream);
    case kSliding: return launch_t<D, kSliding>(a, stream);
    default: return launch_t<D, kDifferential>(a, stream);
  }
}

hipError_t launch_prefill_regstage(const PrefillLaunch& a, hipStream_t stream) {
  return a.d == 64 ? launch_v<64>(a, stream) : launch_v<128>(a, stream);
}


}  // namespace mixer
