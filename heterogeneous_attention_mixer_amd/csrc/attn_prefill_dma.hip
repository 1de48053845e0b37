// attn_prefill_dma.hip -- bf16 causal prefill of one sequence-mixer layer for gfx950, with
// K/V tiles moved HBM -> LDS by the buffer unit (no register staging) and the softmax of
// each tile overlapped with matrix products: within a wave (the pipelined kernel) or between
// the two waves of a SIMD (the phase-separated kernel).
//
// Variants (Table 1, sec. 3.1 of "Placement Is Free, Composition Is Not: The Latin Square as
// a Provably-Balanced Construction for Heterogeneous Sequence-Mixer Stacks"):
//   full          causal softmax attention, scale 1/sqrt(d);
//   sliding       the same inside a causal window of W keys (query included);
//   differential  two causal softmax maps over the two halves of the head dimension, scale
//                 1/sqrt(d/2), combined as (P1 - lambda * P2) V with full-width V.
//
// Design (one workgroup = one (batch, head) and a block of query rows, 32 rows per wave):
//   * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16 (K from LDS
//     as the A operand, Q held in registers as the B operand). A lane owns one query column
//     and 16 keys of each 32-key block, so row max and row sum are in-lane plus one
//     permlane32 swap with lane^32.
//   * Those accumulators, rounded to bf16, are the B operand of O^T += V^T P^T. The V^T
//     operand is read from the row-major V tile with ds_read_b64_tr_b16: a 16-lane group
//     reading 4 key rows x 16 channels receives, per lane, one channel across the 4 keys.
//     The keys are taken in the order the score accumulator hands them out, so P never
//     moves between lanes.
//   * K and V tiles (64 keys) are written into LDS by buffer loads with the LDS flag: each
//     wave instruction moves 1 KiB (64 lanes x 16 B) straight from HBM, with no VGPRs and no
//     VALU work; keys past the end of the sequence are outside the head's buffer range and
//     arrive as zeros. Each 256 B (d=128) row is stored with its 16 B chunks permuted by an
//     XOR of the row index, which keeps both the K reads (16 rows, one chunk each) and the
//     transposed V reads (4 rows, 4 chunks each per 32 lanes) free of bank conflicts.
//   * Pipelined kernel (sliding; full on grids of at most one 256-row workgroup per CU):
//     K runs two tiles ahead of V. Iteration j issues the loads of K[j+2] and V[j],
//     then computes O += V[j-1] P[j-1] together with the row max of S[j], and the
//     exponentials of S[j] together with S[j+1] = K[j+1] Q^T; the matrix core and the vector
//     ALU work on independent data in each half. Two K and two V buffers, one barrier per
//     tile. Consecutive matrix instructions alternate between independent accumulators, and
//     the tile's probabilities are pinned inside the block (see the comments at qk_into and
//     at the end of the iteration).
//   * Online softmax in fp32 with exp2 (scale folded with log2 e); the reference max moves
//     only when a score beats it by more than 2^8 (probabilities stay below 256), so the
//     accumulator rescale is rare. Row sums are taken over the bf16-rounded probabilities,
//     the exact weights of the value product: by v_dot2 in the pipelined kernel, by four
//     small MFMAs per tile in the phase-separated one (whose registers leave room for them).
//   * Phase-separated kernel (prefill_phase_kernel, below; the differential, and full on
//     larger grids): eight waves, two per SIMD, alternate between a matrix phase and a
//     vector phase one phase apart. For the differential each softmax map gets its own wave
//     (scores on its half of the head dim, values on all of it) and the two maps of a row
//     block meet once, at the end, through LDS; for full every wave is a row block of its
//     own, 256 rows per workgroup, which halves the K/V tile bytes per flop. The vector
//     phase takes the exponentials against the current reference and leaves the row max to
//     a rare path at the start of the next matrix phase, taken only while a row has no
//     reference or when a row's tile sum exceeds 2^8.
//   * Work order: heaviest query tiles first (sliding: the short first-window tiles first);
//     all tiles of a head on one XCD when B*H is a multiple of 8. The phase-separated
//     kernel launches persistent when it has more units than CUs: one workgroup per CU takes
//     units from per-XCD queues in that order and steals from the other queues at the end.
//     Full causal in the key split (at most one workgroup per CU) pairs 64-row query tile t
//     with its mirror n-1-t in one workgroup, so that every workgroup holds the same work.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <thread>
#include <type_traits>
#include <vector>

#include "device_common.h"
#include "kernels.h"

namespace mixer {

namespace dma {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// Launch shape of the full and sliding kernel: 4 row blocks of 32 query rows per workgroup,
// each served by SPL waves. SPL = 1: 4 waves, two workgroups per CU (two waves per SIMD).
// SPL = 2 (key split, for grids of at most one workgroup per CU): 8 waves, the two waves of
// a row block take alternate key tiles and merge their softmax states at the end; one
// workgroup per CU, two waves per SIMD. The register budget is two waves per SIMD either way.
template <int SPL>
struct DShape {
  static constexpr int rows = 4;  // 32-row blocks
  static constexpr int waves = rows * SPL;
  static constexpr int threads = waves * kWave;
  static constexpr int bm = 32 * rows;
};

// Chunk swizzle of a tile row: the 16-byte chunk c of row r is stored at chunk c ^ swz(r).
// d = 128 (16 chunks per 256 B row): swaps the two 2-bit halves of r mod 16, a bijection
// on any 16 aligned rows, and gives 4 consecutive rows 4 different 4-chunk groups.
// d = 64 (8 chunks per 128 B row, two rows per bank sweep): the same two properties for
// rows of equal parity.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128)
    return ((r & 3) << 2) | ((r >> 2) & 3);
  else
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Buffer descriptor words (base, stride 0, num_records = bytes, raw-buffer flags): loads
// at byte offsets >= bytes return zeros.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 rsrc_words(unsigned long long base, int bytes) {
  u32x4 r;
  r[0] = (unsigned)base;
  r[1] = (unsigned)(base >> 32) & 0xffffu;
  r[2] = (unsigned)(bytes > 0 ? bytes : 0);
  r[3] = 0x00020000u;
  return r;
}

// 16 bytes per lane from offset `voff` of buffer `r` into LDS at lds_base + 16 * lane
// (lds_base wave-uniform, in M0); offsets outside the buffer write zeros. Written as
// assembly so that the compiler does not see an LDS store: it would otherwise order every
// later LDS read of the block after these loads and wait for them. Completion is the
// kernel's business: every tile is read only after an s_waitcnt and a barrier that follow its
// loads (vmcnt(0) in the pipelined kernel; in the phase-separated one a count that leaves out
// only the loads of later tiles, which complete in issue order), and no compiler-visible
// vector load is in flight inside the key loop.
// `voff` must be a register that is never rewritten while loads are in flight (the
// per-tile step lives in the descriptor): the address operand of a load inside inline
// assembly gets no hazard protection from the compiler.
// M0 (which the load reads as its LDS base) is saved and restored around it: the compiler
// reserves M0 and may rely on its value, so it must not change across the statement.
__device__ __forceinline__ void lds_load16(const u32x4& r, unsigned lds_base, int voff) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0"
      : "=&s"(saved)
      : "s"(lds_base), "v"(voff), "s"(r)
      : "memory");
}

// max(a, b, c): one v_max3_f32. This file is compiled with -fno-honor-nans (no NaN reaches
// a value the kernel uses: scores are finite or masked to -inf), so fmaxf needs no input
// canonicalization. (Not inline assembly: a vector read of an MFMA result needs wait states
// that the compiler inserts only for instructions it can see.)
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  return __builtin_fmaxf(a, __builtin_fmaxf(b, c));
}

// Value of lane ^ 32 next to the lane's own: returns (own, other) combined by `op`.
__device__ __forceinline__ float xhalf_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __builtin_fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int D, int VAR, int SPL, bool PAIR>
__global__ void __attribute__((amdgpu_flat_work_group_size(DShape<SPL>::threads,
                                                           DShape<SPL>::threads),
                               amdgpu_waves_per_eu(2, 2)))
prefill_dma_kernel(const __bf16* __restrict__ qg, const __bf16* __restrict__ kg,
                   const __bf16* __restrict__ vg, __bf16* __restrict__ og, int L, int BH,
                   int G, int nq, int window) {
  static_assert(VAR == kFull || VAR == kSliding, "the differential runs the phase kernel");
  static_assert(SPL == 1 || SPL == 2, "one or two waves per row block");
  static_assert(!PAIR || (SPL == 2 && VAR == kFull), "paired query tiles: full, key split");
  constexpr bool kSlide = (VAR == kSliding);
  constexpr int kWaves = DShape<SPL>::waves;
  constexpr int kRows = DShape<SPL>::rows;
  constexpr int BM = DShape<SPL>::bm;
  constexpr int NQ = D / 16;                      // MFMA steps over the head dim
  constexpr int DB = D / 32;                      // 32-channel blocks of O^T
  constexpr int ROWB = D * 2;                     // bytes per K/V row
  constexpr int TILEB = BN * ROWB;                // bytes per K/V tile
  constexpr int NI = TILEB / 1024;                // 1 KiB load instructions per tile
  constexpr int NIW = NI / kWaves;                // ... per wave
  constexpr int CPR = D / 8;                      // 16-byte chunks per row
  static_assert(NI % kWaves == 0, "tile loads must split evenly over the waves");

  // LDS: K buffers 0, 1 then V buffers 0, 1; buffer b of a kind holds the SPL tiles of
  // iterations of parity b (tile s of the iteration at s * TILEB). With SPL = 2 the same
  // memory passes the second wave's softmax state to the first at the end.
  __shared__ __attribute__((aligned(1024))) char smem[4 * SPL * TILEB];
  lds_char* const lds = (lds_char*)(smem);
  const unsigned lds_addr = (unsigned)(uintptr_t)lds;  // LDS byte address of smem
  // Byte offset of the K (V) buffer of parity b within smem.
  constexpr int kKBuf[2] = {0, SPL * TILEB};
  constexpr int kVBuf[2] = {2 * SPL * TILEB, 3 * SPL * TILEB};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // the same value, in an SGPR
  // Row block of this wave and its tile of each iteration. Paired tiles: waves 2r and 2r + 1
  // split row block r, so that each SIMD (waves w and w + 4) holds a wave of the light tile
  // and one of the heavy tile.
  const int rb = SPL == 1 ? wave : (PAIR ? wave >> 1 : wave % kRows);
  const int half = SPL == 1 ? 0 : (PAIR ? wave & 1 : wave / kRows);
  const int rb_s = SPL == 1 ? wave_s : (PAIR ? wave_s >> 1 : wave_s % kRows);  // in SGPRs
  const int half_s = SPL == 1 ? 0 : (PAIR ? wave_s & 1 : wave_s / kRows);
  const int lr = lane & 31;
  const int lg = lane >> 5;

  int bh, qt;
  map_unit(blockIdx.x, BH, nq, &bh, &qt, kSlide);
  // Paired tiles (an even number of 64-row query tiles, nq pairs): row blocks 0 and 1 are the
  // light tile qt, row blocks 2 and 3 the heavy tile 2 nq - 1 - qt, so that every workgroup
  // holds the same causal work. q0 is the heavy tile's first row.
  const int q0 = PAIR ? (2 * nq - 1 - qt) * 64 : qt * BM;
  auto row0 = [&](int r) { return PAIR ? (r < 2 ? qt * 64 + r * 32 : q0 + (r - 2) * 32)
                                       : q0 + r * 32; };
  const int qw = row0(rb);
  const int qi = qw + lr;
  const size_t head = (size_t)bh * (size_t)L * D;         // q and out
  const size_t kv_head = (size_t)(bh / G) * (size_t)L * D;  // k and v: G query heads each
  const int head_bytes = L * ROWB;
  const __amdgpu_buffer_rsrc_t Qr = make_rsrc(qg + head, head_bytes);
  const unsigned long long Kbase = reinterpret_cast<unsigned long long>(kg + kv_head);
  const unsigned long long Vbase = reinterpret_cast<unsigned long long>(vg + kv_head);

  const float c = kLog2e / __builtin_sqrtf((float)D);
  const float gap = kRescaleLog2Gap / c;

  // Q fragments: lane holds row qi, channels kk*16 + lg*8 + [0, 8).
  bf16x8 qf[NQ];
#pragma unroll
  for (int kk = 0; kk < NQ; ++kk) qf[kk] = bload8<__bf16>(Qr, qi * D + kk * 16 + lg * 8);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // ---- per-lane address parts, fixed for the whole kernel
  // Tile loads: instruction i of this wave covers rows [R0, R0 + 1024/ROWB) of the tile;
  // lane `lane` fills chunk slot lane % CPR of row R0 + lane / CPR, i.e. logical chunk
  // (lane % CPR) ^ swz(row).
  int ld_off[NIW];
#pragma unroll
  for (int t = 0; t < NIW; ++t) {
    const int i = wave + t * kWaves;
    const int r = i * (1024 / ROWB) + lane / CPR;
    ld_off[t] = r * ROWB + (((lane % CPR) ^ swz<D>(r)) << 4);
  }
  // K operand reads: row kb*32 + lr (the swizzle depends on the row mod 16 only), chunk
  // 2*kk + lg.
  const int k_sw = swz<D>(lr);
  // The wave's tile within its iteration's buffer is folded into the per-lane offsets.
  int k_off[NQ];
#pragma unroll
  for (int kk = 0; kk < NQ; ++kk)
    k_off[kk] = half * TILEB + lr * ROWB + (((2 * kk + lg) ^ k_sw) << 4);
  // V^T operand reads (transposed, 8 bytes per lane): for the 16-key half h of key block kb
  // and read rr, lane (group g = lane/16, s = lane%16) reads key row
  // kb*32 + 16h + 8rr + 4*lg + s/4, channels db*32 + 16*(g%2) + 4*(s%4) + [0, 4).
  // With SPL = 2 the V region starts at 64 KiB (d = 128), past what a DS instruction's
  // offset field holds: its base goes into the per-lane offsets, so that every immediate
  // stays below 64 KiB. With SPL = 1 the whole V buffer offset is an immediate.
  constexpr int kVOffBase = SPL == 1 ? 0 : kVBuf[0];
  constexpr int kVImm[2] = {kVBuf[0] - kVOffBase, kVBuf[1] - kVOffBase};
  const int vs = lane & 15, vdh = (lane >> 4) & 1;
  int v_off[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int r = 8 * rr + 4 * lg + (vs >> 2);
      const int chunk = 4 * db + 2 * vdh + ((vs & 3) >> 1);
      v_off[db][rr] = kVOffBase + half * TILEB + r * ROWB + ((chunk ^ swz<D>(r)) << 4) +
                      (vs & 1) * 8;
    }

  // ---- key tiles the workgroup can see: [lo, hi]. Iteration it takes tiles
  // lo + SPL*it + s (s < SPL), the one at s = half for this wave; with SPL = 2 the second
  // wave's tile of the last iteration may be hi + 1, which no row sees (it is masked).
  const int q_last = min(q0 + (PAIR ? 64 : BM), L) - 1;
  const int lo = kSlide ? max(0, q0 - window + 1) / BN : 0;
  const int hi = q_last / BN;
  const int n_it = (hi - lo) / SPL + 1;

  // LDS byte offsets of the K and V buffers holding tile j.
  // Tile j of K (v = false) or V (v = true) into the LDS buffer at byte offset `dst`.
  // The descriptor starts at the tile (scalar arithmetic), so the per-lane offsets ld_off
  // stay the same for every tile.
  auto load_tile = [&](bool v, int dst, int j) {
    const u32x4 r = rsrc_words((v ? Vbase : Kbase) + (unsigned long long)j * TILEB,
                               head_bytes - j * TILEB);
#pragma unroll
    for (int t = 0; t < NIW; ++t)
      lds_load16(r, (unsigned)(lds_addr + dst + (wave_s + t * kWaves) * 1024), ld_off[t]);
  };
  // The SPL tiles of iteration it into the buffer at byte offset `dst`.
  auto load_it = [&](bool v, int dst, int it) {
#pragma unroll
    for (int s = 0; s < SPL; ++s) load_tile(v, dst + s * TILEB, lo + SPL * it + s);
  };
  // Does every row of the wave see every key of tile j?
  auto full_tile = [&](int j) {
    const int k0 = j * BN;
    bool f = (k0 + BN - 1 <= qw);
    if (kSlide) f = f && (qw + 31 - k0 < window);
    return f;
  };

  floatx16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  // Scores and probabilities, double-buffered by tile parity: iteration j reads the scores
  // S[j] from sc[j & 1] and P[j-1] from pr[(j-1) & 1], and writes P[j] into pr[j & 1] and
  // S[j+1] into sc[(j+1) & 1]. With the parity a compile-time constant (the key loop is
  // unrolled by two), the roles swap without register copies and every LDS buffer offset
  // is an instruction immediate.
  floatx16 sc[2][2];
  bf16x8 pr[2][2][2];

  // The matrix instructions below alternate between independent accumulators: an MFMA that
  // accumulates into the result of the one just before it waits for that result (about 44
  // cycles instead of the 32 the pipe needs), so a wave issuing one chain leaves the pipe
  // idle between instructions. Each accumulator still sums its terms in the same order.
  // S^T = K Q^T from the K buffer at byte offset KOFF, into `d`: the two 32-key blocks
  // alternate.
  auto qk_into = [&](auto koff_c, floatx16(&d)[2]) {
    constexpr int KOFF = decltype(koff_c)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) d[kb][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
            lds + k_off[kk] + (KOFF + kb * 32 * ROWB));
        d[kb] = mfma32(a, qf[kk], d[kb]);
      }
  };
  // O^T += V^T P^T from the V buffer at byte offset VOFF: the DB channel blocks take turns.
  auto pv = [&](auto voff_c, const bf16x8(&p)[2][2]) {
    constexpr int VOFF = decltype(voff_c)::value;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const shortx4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<__attribute__((address_space(3))) shortx4*>(
                  lds + v_off[db][0] + (VOFF + (kb * 32 + 16 * h) * ROWB)));
          const shortx4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              reinterpret_cast<__attribute__((address_space(3))) shortx4*>(
                  lds + v_off[db][1] + (VOFF + (kb * 32 + 16 * h) * ROWB)));
          // One whole-vector shuffle and one bit cast: assembling the operand element by
          // element (bf16 from 16-bit integers) was lowered to a wrong byte permutation.
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = mfma32(a, p[kb][h], o[db]);
        }
  };
  // Element (kb, r) of a lane holds key j*BN + c + 4*lg, with c = kb*32 + 8*(r/4) + r%4 a
  // compile-time constant. With t = qi - j*BN - 4*lg the key is causal-visible when c <= t,
  // and inside the window as well when 0 <= t - c < window, one unsigned compare (window >= 1).
  auto mask = [&](int j, floatx16(&x)[2]) {
    const int t = qi - j * BN - 4 * lg;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int c = kb * 32 + 8 * (r >> 2) + (r & 3);
        const bool vis = kSlide ? (unsigned)(t - c) < (unsigned)window : c <= t;
        if (!vis) x[kb][r] = -INFINITY;
      }
  };
  auto row_max = [&](const floatx16(&x)[2]) {
    float t0 = vmax3(x[0][0], x[0][1], x[0][2]);
    float t1 = vmax3(x[1][0], x[1][1], x[1][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) {
      t0 = vmax3(t0, x[0][r], x[0][r + 1]);
      t1 = vmax3(t1, x[1][r], x[1][r + 1]);
    }
    t0 = vmax3(t0, x[0][15], t1);
    t0 = vmax3(t0, x[1][15], x[1][15]);
    return xhalf_max(t0);
  };
  // Probabilities exp2(c (s - m)) rounded to bf16 into `p`; their sum added to l.
  auto exps = [&](const floatx16(&x)[2], bf16x8(&p)[2][2]) {
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
          bf16x2 q2;
          q2[0] = (__bf16)fast_exp2(__builtin_fmaf(x[kb][h * 8 + e], c, -mc));
          q2[1] = (__bf16)fast_exp2(__builtin_fmaf(x[kb][h * 8 + e + 1], c, -mc));
          p[kb][h][e] = q2[0];
          p[kb][h][e + 1] = q2[1];
          l = __builtin_amdgcn_fdot2_f32_bf16(q2, ones, l, false);
        }
  };
  auto scale_o = [&](float f) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= f;
  };

  // ---- prologue: zero the V buffer of parity 1 (iteration 0 multiplies P = 0 by it, which
  // must hold finite values); the K tiles of iterations 0 and 1 into LDS; S = K Q^T of the
  // wave's tile of iteration 0 and its row max.
  {
    const floatx4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    floatx4* const vz = reinterpret_cast<floatx4*>(smem + kVBuf[1]);
#pragma unroll
    for (int i = tid; i < SPL * TILEB / 16; i += kWaves * kWave) vz[i] = z;
  }
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) pr[t][kb][h][e] = (__bf16)0.0f;
  load_it(false, kKBuf[0], 0);
  if (n_it > 1) load_it(false, kKBuf[1], 1);
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  // The first tile's scores, unless no row of this wave sees any of its keys (a wave below
  // the window of the workgroup's first rows, or a second wave's tile past its rows): then
  // zeros stand in, and the mask of the first iteration turns every one of them into -inf.
  const int j0_s = lo + half_s;
  const int qw_s = row0(rb_s);  // the wave's first row, as a scalar
  const bool see_first = (half_s == 0 || j0_s * BN <= qw_s + 31) &&
                         (!kSlide || j0_s * BN + BN - 1 >= qw_s - window + 1);
  float tmax_n;  // row max of the scores of the next tile (unmasked)
  if (see_first) {
    qk_into(std::integral_constant<int, kKBuf[0]>{}, sc[0]);
  } else {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[0][kb][r] = 0.0f;
  }
  tmax_n = row_max(sc[0]);
  __syncthreads();

  // ---- key loop. Every wave runs the same sequence on every iteration of the workgroup's
  // range: keys a wave cannot see are masked (probability 0, softmax state unchanged), so
  // the loop body is one straight path and the register allocation stays within two waves
  // per SIMD.
  float alpha_p = 1.0f;  // pending rescale of O, decided on the previous tile
  bool moved_p = false;
  // Iteration it, with PAR = it & 1, on this wave's tile j = lo + SPL*it + half; LAST marks
  // the last iteration, which has no next tile to score.
  auto iter = [&](auto par_c, auto last_c, int it) {
    constexpr int PAR = decltype(par_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
    const int j = lo + SPL * it + half;
    // Loads for the next iteration, issued first: the K tiles of iteration it+2 into K's
    // buffer PAR (those of iteration it were read during it-1), while it+2 is in the range,
    // and the V tiles of iteration it into V's buffer PAR (those of it-2 were read during
    // it-1).
    if ((PAIR || !LAST) && it + 2 < n_it) load_it(false, kKBuf[PAR], it + 2);
    load_it(true, kVBuf[PAR], it);
    // Rescale decided on the previous tile: O holds the tiles before that one here, and the
    // value product of the previous tile below is already on its reference.
    if (moved_p) scale_o(alpha_p);
    // Row max of tile j: taken during the previous iteration, again here after the mask
    // on tiles that cross the diagonal or the window edge.
    float tmax = tmax_n;
    if (!full_tile(j)) {
      mask(j, sc[PAR]);
      tmax = row_max(sc[PAR]);
    }
    // Reference move for tile j (rare): m and l follow at once, O at the next iteration.
    float alpha = 1.0f;
    const bool moved = __any(tmax > m + gap);
    if (moved) {
      const float m_new = __builtin_fmaxf(m, tmax);
      alpha = (m_new == -INFINITY) ? 1.0f : fast_exp2((m - m_new) * c);
      l *= alpha;
      m = m_new;
    }
    // One straight block: the next tile's S = K Q^T first (not in the last iteration), then
    // O += V P of the previous tile; beside them the exponentials of tile j and, once the
    // next S is in, its row max. The group barriers fix the issue order so that vector work
    // sits between the matrix instructions: a wave issues in order, and an MFMA waiting for
    // the busy matrix pipe holds up everything behind it.
    if constexpr (!LAST)
      qk_into(std::integral_constant<int, kKBuf[1 - PAR]>{}, sc[1 - PAR]);
    pv(std::integral_constant<int, kVImm[1 - PAR]>{}, pr[1 - PAR]);
    exps(sc[PAR], pr[PAR]);
    if constexpr (!LAST) tmax_n = row_max(sc[1 - PAR]);
    // Matrix instructions in the block, and vector instructions between two of them (about
    // 110 per block). The last block is left to the compiler's own order: every fixed
    // spacing tried there pushed the register pressure past the budget.
    constexpr int kMfma = LAST ? 0 : DB * 4 + 2 * NQ;
    constexpr int kValu = 110 / (DB * 4 + 2 * NQ) + 1;
    if constexpr (!LAST) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
#pragma unroll
    for (int i = 0; i < kMfma / 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);      // DS reads
      __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
    }
    // The probabilities and the row sum are consumed only by the next iteration, so the
    // compiler may sink their computation past the barrier, out of the block where it hides
    // under the matrix work: empty statements that read and write them keep it here.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) asm volatile("" : "+v"(pr[PAR][kb][h]));
    asm volatile("" : "+v"(l));
    alpha_p = alpha;
    moved_p = moved;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
  };
  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  using Inner = std::integral_constant<bool, false>;
  using Last = std::integral_constant<bool, true>;
  // Paired tiles: a wave's loop ends with the last tile of its own that any of its rows sees
  // (run as the last iteration: no next scores; its value product follows the loop). Its
  // remaining iterations only issue its share of the tile loads and meet the barriers.
  const int jl_w = (qw_s + 31) / BN - lo;  // the wave's last visible tile, from lo
  const int n_run = PAIR ? min(n_it, jl_w >= half_s ? (jl_w - half_s) / SPL + 1 : 1) : n_it;
  int it = 0;
  for (; it + 2 < n_run; it += 2) {  // it even; it and it + 1 both before the last
    iter(Even{}, Inner{}, it);
    iter(Odd{}, Inner{}, it + 1);
  }
  if (it + 1 < n_run) iter(Even{}, Inner{}, it++);  // it was n_run - 2
  if (it & 1)
    iter(Odd{}, Last{}, it);
  else
    iter(Even{}, Last{}, it);
  if (moved_p) scale_o(alpha_p);
  // The last value product, unless no row of this wave sees a key of its last tile (the
  // first rows of a workgroup whose last tile lies past them): its probabilities are all
  // zero.
  const int jl_s = lo + SPL * it + half_s;
  if (jl_s * BN <= qw_s + 31) {
    if (it & 1)
      pv(std::integral_constant<int, kVImm[1]>{}, pr[1]);
    else
      pv(std::integral_constant<int, kVImm[0]>{}, pr[0]);
  }
  // Paired tiles: a wave whose loop ended early meets the remaining iterations' barriers with
  // its share of their tile loads. Its last value product above read the V tile of its last
  // iteration, which the loads of the iteration two later (after the next barrier) replace.
  if constexpr (PAIR) {
    for (int t = it + 1; t < n_it; ++t) {
      const int par = t & 1;
      if (t + 2 < n_it) load_it(false, par ? kKBuf[1] : kKBuf[0], t + 2);
      load_it(true, par ? kVBuf[1] : kVBuf[0], t);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
    }
  }

  // ---- epilogue: out = O / l. Element (db, r) of a lane is channel
  // db*32 + 8*(r/4) + 4*lg + r%4 of query qi. The lane's indices are taken afresh here (the
  // lane number from mbcnt, the rest from scalars), so nothing but O, l and m has to stay
  // live through the key loop for it.
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int lg_e = lane_e >> 5;
  const int qi_e = row0(rb_s) + (lane_e & 31);
  float lsum = xhalf_sum(l);
  if constexpr (SPL == 2) {
    // The second wave of each row block hands its state (reference m, row sum, O) to the
    // first through LDS; the first rescales both to the larger reference and adds them.
    constexpr int kXch = 64 * (DB * 16 + 2);  // floats per row block
    static_assert(kRows * kXch * 4 <= 4 * SPL * TILEB, "exchange fits the tile buffers");
    __syncthreads();  // every wave is done reading the tiles
    float* const xch = reinterpret_cast<float*>(smem) + rb_s * kXch;
    if (half_s == 1) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[(db * 16 + r) * 64 + lane_e] = o[db][r];
      xch[DB * 16 * 64 + lane_e] = m;
      xch[(DB * 16 + 1) * 64 + lane_e] = lsum;
    }
    __syncthreads();
    if (half_s == 1) return;
    const float m1 = xch[DB * 16 * 64 + lane_e];
    const float l1 = xch[(DB * 16 + 1) * 64 + lane_e];
    const float mm = __builtin_fmaxf(m, m1);  // finite: every row sees its own key
    const float a0 = (m == -INFINITY) ? 0.0f : fast_exp2((m - mm) * c);
    const float a1 = (m1 == -INFINITY) ? 0.0f : fast_exp2((m1 - mm) * c);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        o[db][r] = o[db][r] * a0 + xch[(db * 16 + r) * 64 + lane_e] * a1;
    lsum = lsum * a0 + l1 * a1;
  }
  if (qi_e < L) {
    const float inv = 1.0f / lsum;
    __bf16* orow = og + head + (size_t)qi_e * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        store4(orow + db * 32 + 8 * r4 + 4 * lg_e, o[db][r4 * 4] * inv,
               o[db][r4 * 4 + 1] * inv, o[db][r4 * 4 + 2] * inv, o[db][r4 * 4 + 3] * inv);
  }
}

// ---------------------------------------------------------------- the phase-separated kernel
//
// The differential, and full causal on grids of more than one 256-row workgroup per CU.
// Eight waves, two per SIMD, in two phase groups: waves w and w + 4 share a SIMD, and the
// group of waves 4..7 runs one phase behind the group of waves 0..3.
//   * Differential: row block rb's two maps are waves rb (map 0) and rb + 4 (map 1). Each
//     wave has one map's softmax over half of the head dim and the value product over all
//     of it; the two maps of a row block meet once, at the end, through LDS. 128 rows.
//   * Full: every wave is a row block of its own, scores over the whole head dim. 256 rows,
//     so each K/V tile brought into LDS serves twice the rows of the pipelined kernel's.
// Per key tile k a wave runs an M phase (matrix work only: S[k] = K[k] Q^T, then
// O += V[k-1] P[k-1]) and
// a V phase (vector work: the exponentials of S[k] into P[k] against the current
// reference, the loads of later tiles, and four small MFMAs for the row sums of P[k]). The
// reference test for tile k (no reference yet, or a row's tile sum above 2^8: then the row
// max, the move with l and O, and the exponentials again) runs at the start of the M phase
// of tile k+1, before S is overwritten; it is rare. So on every SIMD one wave feeds the matrix
// core while its partner does the softmax, and a barrier ends every phase. The M phase runs
// at raised wave priority, so the arbiter favours the matrix instructions. Within a wave the
// phases strictly alternate, so one set of score and probability registers is enough.
// K[k] and V[k-1] (the pair of tile k) live in LDS buffer pair k mod 4; the loads of pair
// k+3 are issued in the V phase of tile k.

// Work queues of the persistent launch. A slot holds one counter per XCD queue (each on a
// 64-byte line of its own) and a count of the workgroups that have finished; the last
// workgroup to finish sets them all back to zero, so a slot is clean between launches. The
// host gives each stream a slot of its own: launches on one stream run one after another,
// and launches that may overlap never share a slot.
constexpr int kQueueSlots = 256;
constexpr int kQueues = 8;
constexpr int kSlotWords = (kQueues + 1) * 16;
__device__ unsigned g_unit_queue[kQueueSlots * kSlotWords];

// What the phase kernel keeps in LDS between units.
struct UnitArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float lambda;
  int BH, G, nq, slot, grid;
  int ux, ut;  // queue and ticket of the current unit (ux < 0: no more units)
};
// A wave-uniform value read from LDS, as a scalar.
__device__ __forceinline__ int rfl(int x) { return __builtin_amdgcn_readfirstlane(x); }
template <typename T>
__device__ __forceinline__ T* rfl_ptr(T* p) {
  const unsigned long long u = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)u);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(u >> 32));
  return reinterpret_cast<T*>(((unsigned long long)hi << 32) | lo);
}

template <int VAR>
struct PhaseShape {
  static constexpr int maps = VAR == kDifferential ? 2 : 1;
  static constexpr int rows = 8 / maps;  // 32-row blocks
  static constexpr int waves = rows * maps;
  static constexpr int threads = waves * kWave;
  static constexpr int bm = 32 * rows;
};

template <int D, int VAR>
__global__ void __attribute__((amdgpu_flat_work_group_size(PhaseShape<VAR>::threads,
                                                           PhaseShape<VAR>::threads),
                               amdgpu_waves_per_eu(2, 2)))
prefill_phase_kernel(const __bf16* __restrict__ qg, const __bf16* __restrict__ kg,
                     const __bf16* __restrict__ vg, __bf16* __restrict__ og, int L, int BH,
                     int G, int nq, float lambda, int slot) {
  static_assert(VAR == kFull || VAR == kDifferential, "full or differential");
  constexpr bool kDiff = VAR == kDifferential;
  constexpr int kWaves = PhaseShape<VAR>::waves;
  constexpr int kRows = PhaseShape<VAR>::rows;
  constexpr int BM = PhaseShape<VAR>::bm;
  constexpr int NQ = kDiff ? D / 32 : D / 16;  // MFMA steps over a map's score channels
  constexpr int DB = D / 32;
  constexpr int ROWB = D * 2;
  constexpr int TILEB = BN * ROWB;
  constexpr int NI = TILEB / 1024;
  constexpr int NIW = NI / kWaves;
  constexpr int CPR = D / 8;
  static_assert(NI % kWaves == 0, "tile loads must split evenly over the waves");
  // LDS: K buffers 0..3, then V buffers 0..3; reused after the key loop to pass map 1's
  // output to map 0 (differential).
  constexpr int kXchBytes = kDiff ? kRows * 64 * (DB * 16) * 4 : 0;
  constexpr int kSmem = (8 * TILEB > kXchBytes) ? 8 * TILEB : kXchBytes;
  // At the end of an M phase every load but those issued in the wave's last V phase is in.
  constexpr int kWaitOlder = 0x0F70 | (2 * NIW);
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];
  lds_char* const lds = (lds_char*)(smem);
  const unsigned lds_addr = (unsigned)(uintptr_t)lds;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int grp = wave_s >> 2;     // phase group (waves w and w + 4 share a SIMD)
  const int rb = wave % kRows;     // row block of this wave
  const int map = wave / kRows;    // softmax map (differential; 0 for full)
  const int lr = lane & 31;
  const int lg = lane >> 5;
  const float c = kLog2e / __builtin_sqrtf((float)(kDiff ? D / 2 : D));
  const int ch0 = map * (D / 2);  // first score channel of this wave's map
  const int head_bytes = L * ROWB;

  // Per-lane address parts (the same chunk swizzle and read patterns as the pipelined
  // kernel; V offsets carry the V region's base).
  int ld_off[NIW];
#pragma unroll
  for (int t = 0; t < NIW; ++t) {
    const int i = wave + t * kWaves;
    const int r = i * (1024 / ROWB) + lane / CPR;
    ld_off[t] = r * ROWB + (((lane % CPR) ^ swz<D>(r)) << 4);
  }
  const int k_sw = swz<D>(lr);
  int k_off[NQ];
#pragma unroll
  for (int kk = 0; kk < NQ; ++kk)
    k_off[kk] = lr * ROWB + (((ch0 / 8 + 2 * kk + lg) ^ k_sw) << 4);
  const int vs = lane & 15, vdh = (lane >> 4) & 1;
  int v_off[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int r = 8 * rr + 4 * lg + (vs >> 2);
      const int chunk = 4 * db + 2 * vdh + ((vs & 3) >> 1);
      v_off[db][rr] = 4 * TILEB + r * ROWB + ((chunk ^ swz<D>(r)) << 4) + (vs & 1) * 8;
    }
  // Row sums on the matrix core: v_mfma_f32_16x16x32_bf16 with a 0/1 selector as A and a
  // probability register as B. As B, lane l's register is k-group l/16 of column l%16; it
  // holds 8 probabilities of query l%32, so query n (< 16) fills k-groups 0 and 2 of column
  // n and query n+16 k-groups 1 and 3. Selector rows 0 and 8 take k-groups 0 and 2, rows 4
  // and 12 take 1 and 3, and the result's element 0 in lane l is row 4*(l/16) of column
  // l%16: the whole row sum of query l%32, in both lanes of the query. Four of these
  // (16 cycles each on the matrix pipe) replace 16 v_dot2c, each of which holds the matrix
  // pipe for about 10 cycles, out of the vector phase that runs beside the partner's MFMAs.
  bf16x8 rsel;
  {
    const int sr = lane & 15, sg = (lane >> 4) & 1;
    const bool one = ((sr == 0 || sr == 8) && sg == 0) || ((sr == 4 || sr == 12) && sg == 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) rsel[e] = one ? (__bf16)1.0f : (__bf16)0.0f;
  }

  // Units: (batch x head, query tile) pairs. With B*H a multiple of 8 there is one queue
  // per XCD, holding that XCD's heads heaviest tile first (full: the heads interleaved, as
  // map_unit deals them; the differential: head by head, as map_unit_head_major does);
  // otherwise one queue. Workgroup b starts on ticket b / nQ of queue b % nQ (its XCD's, as
  // the hardware deals workgroups to the XCDs round-robin). With a slot (the persistent
  // launch, one workgroup per CU), it then takes the next ticket of that queue, and once
  // that queue is empty, tickets of the others; without one (one workgroup per unit) it
  // stops after its first unit.
  // The launch's arguments and the current unit live in LDS between units, read back where
  // they are used: kept in scalar registers across the key loop they would not fit.
  __shared__ UnitArgs ua;
  if (tid == 0) {
    const int nQ = ((BH & 7) == 0) ? kQueues : 1;
    ua = UnitArgs{qg, kg, vg, og, lambda, BH, G, nq, slot, (int)gridDim.x,
                  (int)blockIdx.x % nQ, (int)blockIdx.x / nQ};
  }
  __syncthreads();
  for (;;) {
    int bh, qt;
    {
      const int BHu = rfl(ua.BH), nqu = rfl(ua.nq);
      const int nQ = ((BHu & 7) == 0) ? kQueues : 1;
      // The differential's queues hold their units head by head (its HBM traffic falls by
      // about 40 % and its time does not move); full keeps the heads interleaved, which is
      // faster for it.
      if constexpr (kDiff)
        map_unit_head_major(rfl(ua.ut) * nQ + rfl(ua.ux), BHu, nqu, &bh, &qt);
      else
        map_unit(rfl(ua.ut) * nQ + rfl(ua.ux), BHu, nqu, &bh, &qt);
    }
    const int q0 = qt * BM;
    const int qw = q0 + rb * 32;
    const int qi = qw + lr;
    const size_t head = (size_t)bh * (size_t)L * D;
    const size_t kv_head = (size_t)(bh / rfl(ua.G)) * (size_t)L * D;
    const __amdgpu_buffer_rsrc_t Qr = make_rsrc(rfl_ptr(ua.q) + head, head_bytes);
    const unsigned long long Kbase = reinterpret_cast<unsigned long long>(rfl_ptr(ua.k) + kv_head);
    const unsigned long long Vbase = reinterpret_cast<unsigned long long>(rfl_ptr(ua.v) + kv_head);

    bf16x8 qf[NQ];
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) qf[kk] = bload8<__bf16>(Qr, qi * D + ch0 + kk * 16 + lg * 8);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);

    const int q_last = min(q0 + BM, L) - 1;
    const int lo = 0;
    const int hi = q_last / BN;

    auto load_tile = [&](bool v, int dst, int j) {
      const u32x4 r = rsrc_words((v ? Vbase : Kbase) + (unsigned long long)j * TILEB,
                                 head_bytes - j * TILEB);
      // The LDS destination is formed here, behind an empty statement: left visible, the
      // compiler keeps every buffer pair's destinations live across the unrolled key loop and
      // runs out of scalar registers.
      unsigned m0b = lds_addr + (unsigned)wave_s * 1024u + (unsigned)dst;
      asm volatile("" : "+s"(m0b));
#pragma unroll
      for (int t = 0; t < NIW; ++t)
        lds_load16(r, m0b + (unsigned)(t * kWaves * 1024), ld_off[t]);
    };
    // Does every row of the wave see every key of tile j?
    auto full_tile = [&](int j) { return j * BN + BN - 1 <= qw; };

    floatx16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float m = -INFINITY, l = 0.0f;
    float lt = 0.0f;  // the row's sum of the last tile's probabilities, not yet in l
    floatx16 s[2];
    bf16x8 p[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) p[kb][h][e] = (__bf16)0.0f;

    // Probabilities exp2(c (s - m)) of the tile against the current reference, rounded to
    // bf16 into p; the row's sum of the rounded values into lt, on the matrix core.
    auto take_exps = [&]() {
      const float mc = (m == -INFINITY) ? 0.0f : m * c;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            p[kb][h][e] = (__bf16)fast_exp2(__builtin_fmaf(s[kb][h * 8 + e], c, -mc));
      // The partner wave is in its M phase at raised priority, so at the base priority these
      // four would wait for gaps in its matrix stream (about 240 cycles of the V phase): they
      // take the same priority and interleave with it instead.
      floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rsel, p[kb][h], acc, 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
      lt = acc[0];
    };
    // Reference test for the tile whose probabilities the V phase just took (S still holds
    // its masked scores). While a row has no reference yet, or when a row's tile sum says a
    // probability may exceed 2^gap, the row max moves the reference, l and O follow (O holds
    // the tiles before this one), and the probabilities are taken again. Then l takes lt.
    auto settle = [&]() {
      if (__any((lt > kTileSumBound) | (m == -INFINITY))) {
        float t0 = vmax3(s[0][0], s[0][1], s[0][2]);
        float t1 = vmax3(s[1][0], s[1][1], s[1][2]);
#pragma unroll
        for (int r = 3; r < 15; r += 2) {
          t0 = vmax3(t0, s[0][r], s[0][r + 1]);
          t1 = vmax3(t1, s[1][r], s[1][r + 1]);
        }
        const float tmax = xhalf_max(vmax3(vmax3(t0, s[0][15], t1), s[1][15], s[1][15]));
        const float m_new = __builtin_fmaxf(m, tmax);
        if (m_new != m) {
          const float alpha = (m == -INFINITY) ? 0.0f : fast_exp2((m - m_new) * c);
          l *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
          m = m_new;
          take_exps();
        }
      }
      l += lt;
    };
    // M phase of tile k (pair buffer `pb`, a compile-time constant, so that every operand
    // read's LDS offset is an instruction immediate): S = K[k] Q^T; O += V[k-1] P.
    auto m_phase = [&](auto pb_c) {
      constexpr int pb = decltype(pb_c)::value;
      constexpr int kbase = pb * TILEB;
      int ka[NQ], va[DB][2];
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk) ka[kk] = k_off[kk] + kbase;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) va[db][rr] = v_off[db][rr] + kbase;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < NQ; ++kk)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
              lds + ka[kk] + kb * 32 * ROWB);
          s[kb] = mfma32(a, qf[kk], s[kb]);
        }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int roff = (kb * 32 + 16 * h) * ROWB;
            const shortx4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                reinterpret_cast<__attribute__((address_space(3))) shortx4*>(
                    lds + va[db][0] + roff));
            const shortx4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                reinterpret_cast<__attribute__((address_space(3))) shortx4*>(
                    lds + va[db][1] + roff));
            const bf16x8 a = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
            o[db] = mfma32(a, p[kb][h], o[db]);
          }
      // Operand reads ahead of the matrix instructions that use them. A score MFMA reads one
      // K operand, a value MFMA two V reads: kEarly reads after each score MFMA (three for the
      // differential's 8 score MFMAs, two for full's 16) put the value product's reads well
      // ahead when it starts, and one read after each of its first value MFMAs keeps them
      // ahead to the end of the phase (an even 1.5 reads per MFMA let the lead fall to one
      // MFMA, less than the LDS latency).
      constexpr int kEarly = kDiff ? 3 : 2;
      constexpr int kLate = 2 * NQ + 8 * DB - 4 - 2 * NQ * kEarly;  // reads for value MFMAs
      static_assert(kLate >= 0 && kLate <= 4 * DB, "read schedule");
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 2 * NQ; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kEarly, 0);
      }
#pragma unroll
      for (int i = 0; i < kLate; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * DB - kLate, 0);
    };
    // V phase of tile k: loads of pair k+3, then the probabilities of S (masked on tiles
    // that cross the diagonal) against the current reference.
    auto v_phase = [&](int k) {
      const int nb = ((k + 3 - lo) & 3) * TILEB;
      load_tile(false, nb, k + 3);
      load_tile(true, 4 * TILEB + nb, k + 2);
      if (!full_tile(k)) {
        // Element (kb, r) holds key k*BN + cc + 4*lg with cc a compile-time constant: visible
        // when cc <= qi - k*BN - 4*lg.
        const int t = qi - k * BN - 4 * lg;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 8 * (r >> 2) + (r & 3) > t) s[kb][r] = -INFINITY;
      }
      // The first tile's rows have no reference yet, so the next M phase's test always takes
      // its rare path, which takes the exponentials and sums again: none here.
      if (k > lo) take_exps();
    };

    // ---- prologue (lo is tile 0): pair 0 = (K[0], zeros), pair 1 = (K[1], V[0]),
    // pair 2 = (K[2], V[1]).
    {
      const floatx4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      floatx4* const vz = reinterpret_cast<floatx4*>(smem + 4 * TILEB);
#pragma unroll
      for (int i = tid; i < TILEB / 16; i += kWaves * kWave) vz[i] = z;
    }
    load_tile(false, 0 * TILEB, lo);
    load_tile(false, 1 * TILEB, lo + 1);
    load_tile(true, 5 * TILEB, lo);
    load_tile(false, 2 * TILEB, lo + 2);
    load_tile(true, 6 * TILEB, lo + 1);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();

    // ---- key loop: group 1 runs one phase behind group 0; both run the same number of
    // barriers. The last M phase (tile hi+1) only adds V[hi] P[hi]; its scores are discarded.
    if (grp == 1) __syncthreads();
    // The loop is unrolled by the four buffer pairs (tile k uses pair k mod 4; lo is 0 here).
    auto step = [&](auto pb_c, int k) {
      if (k > lo) settle();  // tile k-1
      __builtin_amdgcn_s_setprio(1);
      m_phase(pb_c);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_s_waitcnt(kWaitOlder);
      __syncthreads();
      if (k <= hi) v_phase(k);
      __syncthreads();
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    int k = lo;
    for (; k + 3 <= hi + 1; k += 4) {
      step(P0{}, k);
      step(P1{}, k + 1);
      step(P2{}, k + 2);
      step(P3{}, k + 3);
    }
    if (k <= hi + 1) step(P0{}, k++);
    if (k <= hi + 1) step(P1{}, k++);
    if (k <= hi + 1) step(P2{}, k++);
    // The last M phase's scores are discarded; reading them here keeps the compiler from
    // dropping them only where it can prove which step comes last (every workgroup then
    // issues the same matrix work for its tile range).
    asm volatile("" ::"v"(s[0]), "v"(s[1]));
    // Group 0 ends its key loop one phase before group 1. Once its own tile loads are in, wave
    // 0 asks for the next unit, so that the answer comes back while the workgroup finishes:
    // lane 0 takes the next ticket of the current queue, and lanes 32.. read every queue's
    // counter in the same round trip, for when the current queue turns out empty. With no
    // tile load of the wave in flight, the key loop's counted waits are not disturbed.
    unsigned tk_next = 0;
    unsigned q_seen = 0;
    if (grp == 0) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      if (wave_s == 0 && ua.slot >= 0) {
        unsigned* const qs = g_unit_queue + ua.slot * kSlotWords;
        const int nQ = ((ua.BH & 7) == 0) ? kQueues : 1;
        if (lane == 0)
          tk_next = __hip_atomic_fetch_add(qs + 16 * ua.ux, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
        else if (lane >= 32 && lane < 32 + nQ)
          q_seen = __hip_atomic_load(qs + 16 * (lane - 32), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }

    // ---- epilogue. Element (db, r) of a lane is channel db*32 + 8*(r/4) + 4*lg + r%4 of
    // query qi.
    const float lsum = l;  // the row-sum MFMAs already add the two lanes of a query
    if constexpr (!kDiff) {  // out = O / l
      if (qi < L) {
        const float inv = 1.0f / lsum;
        __bf16* orow = rfl_ptr(ua.o) + head + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            store4(orow + db * 32 + 8 * r4 + 4 * lg, o[db][r4 * 4] * inv,
                   o[db][r4 * 4 + 1] * inv, o[db][r4 * 4 + 2] * inv, o[db][r4 * 4 + 3] * inv);
      }
    } else {
      // Differential: out = O1 / l1 - lambda * O2 / l2, map 1's term passed to map 0 through LDS.
      __syncthreads();  // every wave is done reading the tiles
      {
        float* const xch = reinterpret_cast<float*>(smem) + rb * 64 * (DB * 16);
        if (map == 1) {
          const float sc = ua.lambda / lsum;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) xch[(db * 16 + r) * 64 + lane] = o[db][r] * sc;
        }
      }
      __syncthreads();
      if (map == 0 && qi < L) {
        const float inv = 1.0f / lsum;
        const float* const xch = reinterpret_cast<const float*>(smem) + rb * 64 * (DB * 16);
        __bf16* orow = rfl_ptr(ua.o) + head + (size_t)qi * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[e] = o[db][r4 * 4 + e] * inv;
              x[e] -= xch[(db * 16 + r4 * 4 + e) * 64 + lane];
            }
            store4(orow + db * 32 + 8 * r4 + 4 * lg, x[0], x[1], x[2], x[3]);
          }
      }
    }

    if (rfl(ua.slot) < 0) break;
    // Wave 0 settles the next unit. When the current queue is empty it takes a ticket from the
    // queue with the most left, by the counters read with the request (lanes 32..) and read
    // again after every miss; a queue found empty stays empty, so this ends after at most nQ
    // misses.
    if (wave_s == 0) {
      const int nQ = ((rfl(ua.BH) & 7) == 0) ? kQueues : 1;
      const int Ux = rfl(ua.BH) * rfl(ua.nq) / nQ;
      unsigned* const qslot = g_unit_queue + rfl(ua.slot) * kSlotWords;
      // Tickets below this were dealt to the workgroups as their first units.
      auto first_dyn = [&](int x) { return (rfl(ua.grid) - x + nQ - 1) / nQ; };
      const int ux = rfl(ua.ux);
      int nx = ux;
      int nt = first_dyn(ux) + __builtin_amdgcn_readfirstlane((int)tk_next);
      bool reread = false;
      while (nt >= Ux) {
        if (reread && lane >= 32 && lane < 32 + nQ)
          q_seen = __hip_atomic_load(qslot + 16 * (lane - 32), __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        reread = true;
        nx = -1;
        int most = 0;
        for (int x = 0; x < nQ; ++x) {
          const int v = Ux - first_dyn(x) - (int)__builtin_amdgcn_readlane(q_seen, 32 + x);
          if (v > most) {
            most = v;
            nx = x;
          }
        }
        if (nx < 0) break;
        unsigned t = 0;
        if (lane == 0)
          t = __hip_atomic_fetch_add(qslot + 16 * nx, 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        nt = first_dyn(nx) + __builtin_amdgcn_readfirstlane((int)t);
      }
      if (lane == 0) {
        ua.ux = nx;
        ua.ut = nt;
      }
    }
    __syncthreads();
    if (rfl(ua.ux) < 0) break;
  }  // units

  // The last workgroup to finish returns the slot's counters to zero for the next launch.
  // The counters are only ever touched by device-scope atomics, and every workgroup's ticket
  // requests have returned before it counts itself here, so no ordering beyond that of the
  // atomics themselves is needed (and none that would flush the L2).
  if (tid == 0 && ua.slot >= 0) {
    unsigned* const qslot = g_unit_queue + ua.slot * kSlotWords;
    if (__hip_atomic_fetch_add(qslot + 16 * kQueues, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) == (unsigned)ua.grid - 1) {
      for (int x = 0; x <= kQueues; ++x)
        __hip_atomic_store(qslot + 16 * x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int D, int VAR, int SPL, bool PAIR = false>
hipError_t launch_dma_s(const PrefillLaunch& a, int nq, hipStream_t stream) {
  const int BH = a.B * a.H;
  hipLaunchKernelGGL((prefill_dma_kernel<D, VAR, SPL, PAIR>), dim3((unsigned)(BH * nq)),
                     dim3(DShape<SPL>::threads), 0, stream, static_cast<const __bf16*>(a.q),
                     static_cast<const __bf16*>(a.k), static_cast<const __bf16*>(a.v),
                     static_cast<__bf16*>(a.out), a.L, BH, a.H / a.Hkv, nq, a.window);
  return hipGetLastError();
}

// Full and sliding: the key split (SPL = 2) when the grid holds at most one workgroup per
// CU, where the 4-wave workgroups would leave one wave per SIMD and the longest query tile
// alone would set the time; otherwise two 4-wave workgroups per CU. Full causal with an even
// number of 64-row query tiles pairs them in the key split, light with heavy, so that every
// workgroup holds the same work and the heaviest no longer sets the time alone.
template <int D, int VAR>
hipError_t launch_dma_t(const PrefillLaunch& a, hipStream_t stream) {
  constexpr int BM = DShape<1>::bm;
  static_assert(DShape<2>::bm == BM, "both shapes tile the rows alike");
  const int nq = (a.L + BM - 1) / BM;
  const long long wgs = (long long)a.B * a.H * nq;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (wgs > cus) return launch_dma_s<D, VAR, 1>(a, nq, stream);
  const int nt64 = (a.L + 63) / 64;
  if (VAR == kFull && (nt64 & 1) == 0)
    return launch_dma_s<D, kFull, 2, true>(a, nt64 / 2, stream);
  return launch_dma_s<D, VAR, 2>(a, nq, stream);
}

// The queue slot of (device, stream): the stream's rank among the streams of that device
// that have launched the persistent kernel, or -1 once every slot has an owner. Launches on
// one stream run in order, so they share its slot safely; a slot never passes to another
// stream. The per-thread default stream is one handle for a different stream in every host
// thread, so it is told apart by thread. A graph captured from a stream keeps that stream's
// slot.
int queue_slot(int dev, hipStream_t stream) {
  struct Owner {
    int dev;
    hipStream_t stream;
    std::thread::id thread;
  };
  static std::mutex mu;
  static std::vector<Owner> owners;
  const std::thread::id thread =
      stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id();
  std::lock_guard<std::mutex> hold(mu);
  int n = 0;
  for (const Owner& o : owners) {
    if (o.dev != dev) continue;
    if (o.stream == stream && o.thread == thread) return n;
    ++n;
  }
  if (n >= kQueueSlots) return -1;
  owners.push_back(Owner{dev, stream, thread});
  return n;
}

template <int D, int VAR>
hipError_t launch_phase(const PrefillLaunch& a, int nq, hipStream_t stream) {
  const int BH = a.B * a.H;
  const long long units = (long long)BH * nq;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // One workgroup holds a CU (its LDS). With more units than CUs the launch is persistent:
  // one workgroup per CU, taking units from the stream's queue slot; otherwise (or with
  // every slot taken) one workgroup per unit.
  const int slot = units > cus ? queue_slot(dev, stream) : -1;
  const unsigned grid = slot >= 0 ? (unsigned)cus : (unsigned)units;
  hipLaunchKernelGGL((prefill_phase_kernel<D, VAR>), dim3(grid), dim3(PhaseShape<VAR>::threads),
                     0, stream, static_cast<const __bf16*>(a.q), static_cast<const __bf16*>(a.k),
                     static_cast<const __bf16*>(a.v), static_cast<__bf16*>(a.out), a.L, BH,
                     a.H / a.Hkv, nq, a.lambda, slot);
  return hipGetLastError();
}

// Full causal takes the phase-separated kernel (256-row units, one workgroup per CU) when it
// has more units than CUs, so that the later, lighter units fill in behind the heavy first
// ones; with fewer, the pipelined kernel's two 128-row workgroups per CU (or its key split)
// balance the causal work better.
template <int D>
hipError_t launch_full(const PrefillLaunch& a, hipStream_t stream) {
  constexpr int BM = PhaseShape<kFull>::bm;
  const int nq = (a.L + BM - 1) / BM;
  const long long wgs = (long long)a.B * a.H * nq;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  return wgs > cus ? launch_phase<D, kFull>(a, nq, stream) : launch_dma_t<D, kFull>(a, stream);
}

template <int D>
hipError_t launch_dma_v(const PrefillLaunch& a, hipStream_t stream) {
  switch (a.variant) {
    case kFull: return launch_full<D>(a, stream);
    case kSliding: return launch_dma_t<D, kSliding>(a, stream);
    default: {
      constexpr int BM = PhaseShape<kDifferential>::bm;
      return launch_phase<D, kDifferential>(a, (a.L + BM - 1) / BM, stream);
    }
  }
}

}  // namespace dma

hipError_t launch_prefill_dma(const PrefillLaunch& a, hipStream_t stream) {
  return a.d == 64 ? dma::launch_dma_v<64>(a, stream) : dma::launch_dma_v<128>(a, stream);
}

hipError_t launch_prefill(const PrefillLaunch& a, hipStream_t stream) {
  return a.f32 ? launch_prefill_regstage(a, stream) : launch_prefill_dma(a, stream);
}

}  // namespace mixer
