/*
 * mixer.h -- C ABI of libmixer.so: causal prefill of one sequence-mixer layer on an MI355X
 * (gfx950) GPU, in its full, sliding-window and differential variants, plus a Latin-square
 * layer scheduler.
 *
 * Source: "Placement Is Free, Composition Is Not: The Latin Square as a Provably-Balanced
 * Construction for Heterogeneous Sequence-Mixer Stacks" (arXiv 2609.20269).
 *
 * Conventions shared by every entry point
 *   - Tensors are contiguous row-major [B, H, L, d] device pointers (one head's L x d slice
 *     is contiguous), each starting on a 16-byte boundary. q, k, v and out have the same
 *     shape; H counts query heads and key/value heads alike (multi-head attention), except
 *     in mixer_prefill_gqa_async, whose k and v have Hkv heads.
 *   - Ownership: the caller allocates and owns every buffer. The library allocates no device
 *     memory and never synchronises the device. Its only state is a set of work-queue
 *     counters for the persistent launch of full causal (on grids of more 256-row query
 *     tiles than CUs) and of the differential: 256 slots per device in the library's own
 *     device memory (set up, zeroed, when the library is loaded), one slot per stream that
 *     makes such a launch, back at zero when each launch ends. Launches on one stream share
 *     its slot; launches on different streams never share one. A HIP graph captured from a
 *     stream keeps that stream's slot: a replay must not run while another launch made on
 *     that stream, or another replay of the graph, may be running. A stream that finds
 *     every slot taken gets the one-workgroup-per-tile launch, with the same results.
 *   - Asynchrony: the *_async calls and mixer_stack_prefill enqueue work on `stream` (a
 *     hipStream_t passed as void*, NULL = the legacy default stream) and return. Launch
 *     errors come back as MIXER_EHIP; a fault during execution surfaces at the caller's next
 *     synchronisation. Calls on different streams may run from different threads.
 *   - Validation is host-only and happens before any HIP call: a call that returns
 *     MIXER_EINVAL, MIXER_EUNSUPPORTED or MIXER_ENOTLATIN has not touched the device.
 *     MIXER_EHIP means the runtime refused a launch or an event record; the single-layer
 *     calls have then enqueued nothing, the multi-layer runners may have enqueued the layers
 *     before the failing one (see mixer_layers_prefill).
 *   - Scores are scaled by 1/sqrt(d) (full, sliding) or 1/sqrt(d/2) (differential); there
 *     is no scale argument.
 *   - Arithmetic: bf16 operands on the matrix cores with fp32 accumulation; softmax in fp32;
 *     the probabilities are rounded to bf16 before the value product; outputs are rounded
 *     once (round-to-nearest-even). Results are bitwise reproducible run to run.
 */
#ifndef MIXER_H
#define MIXER_H

#ifdef __cplusplus
extern "C" {
#endif

/* Mixer variants, named as in Table 1 (sec. 3.1) of the paper. */
typedef enum {
    MIXER_FULL = 0,         /* exact causal attention: key j visible to query i iff j <= i   */
    MIXER_SLIDING = 1,      /* causal window: visible iff 0 <= i - j <= window - 1            */
    MIXER_DIFFERENTIAL = 2  /* two half-head-dim maps: out = (P1 - lambda * P2) V             */
} mixer_variant;

typedef enum {
    MIXER_OK = 0,
    MIXER_EINVAL = -1,       /* bad argument: null or unaligned pointer, size < 1, unknown
                                variant, window < 1 for SLIDING, non-finite lambda for
                                DIFFERENTIAL, out overlapping q/k/v, size overflow, bad
                                schedule entry, Hkv not dividing H                         */
    MIXER_EUNSUPPORTED = -2, /* valid but not built: d not in {64, 128}, one head's L x d
                                slice of 2 GiB or more, grid too large                     */
    MIXER_ENOTLATIN = -3,    /* mixer_stack_prefill: schedule is not a Latin square          */
    MIXER_EHIP = -4          /* the HIP runtime reported an error at launch                  */
} mixer_status;

/*
 * mixer_prefill_async -- one causal-prefill mixer layer, bf16 in and out.
 *
 * Defines (Table 1, sec. 3.1; causality as audited in sec. 8), for every b, h and query i:
 *   FULL          out_i = sum_{j <= i} softmax_j(q_i . k_j / sqrt(d)) v_j
 *   SLIDING       as FULL over the keys i - window + 1 <= j <= i (the query counts toward
 *                 the window; window >= L equals FULL; window = 1 returns v)
 *   DIFFERENTIAL  two maps over the two halves of the head dimension: q1, k1 are
 *                 channels [0, d/2), q2, k2 channels [d/2, d); P1, P2 are the causal
 *                 softmax maps of q1 k1^T / sqrt(d/2) and q2 k2^T / sqrt(d/2); the second
 *                 map, weighted by lambda, is taken from the first:
 *                 out_i = sum_{j <= i} (P1_ij - lambda * P2_ij) v_j, v full width d.
 *
 * q, k, v   [B, H, L, d] bfloat16 device pointers (read only).
 * out       [B, H, L, d] bfloat16 device pointer (written); must not overlap q, k or v.
 * variant   a mixer_variant.
 * window    SLIDING only, >= 1 (ignored otherwise).
 * lambda    DIFFERENTIAL only, any finite value (ignored otherwise).
 * B, H, L   >= 1.   d: 64 or 128.
 * stream    hipStream_t, or NULL for the legacy default stream.
 * Returns MIXER_OK or a negative mixer_status.
 */
int mixer_prefill_async(const void *q, const void *k, const void *v, void *out,
                        int variant, int window, float lambda,
                        int B, int H, int L, int d, void *stream);

/*
 * mixer_prefill_gqa_async -- the same layer with grouped key/value heads: Hkv key/value heads
 * shared by H query heads, H / Hkv query heads per key/value head. This is the attention
 * shape of the model the paper builds (Table 2, sec. 4.1: 16 heads, 4 KV heads, head_dim
 * 128). Query head h of batch b attends with key/value head b * Hkv + h / (H / Hkv); every
 * other definition is mixer_prefill_async's (Hkv = H gives exactly that call).
 *
 * q, out    [B, H, L, d] bfloat16 device pointers (out written, must not overlap q, k, v).
 * k, v      [B, Hkv, L, d] bfloat16 device pointers (read only).
 * Hkv       >= 1 and dividing H; otherwise MIXER_EINVAL.
 * Other arguments and the return value as for mixer_prefill_async.
 */
int mixer_prefill_gqa_async(const void *q, const void *k, const void *v, void *out,
                            int variant, int window, float lambda,
                            int B, int H, int Hkv, int L, int d, void *stream);

/* The same layer on the legacy default stream. */
int mixer_prefill(const void *q, const void *k, const void *v, void *out,
                  int variant, int window, float lambda, int B, int H, int L, int d);

/*
 * mixer_prefill_f32_async -- the same layer for fp32 inputs and output. q and k are split
 * into bf16 high and low parts and the scores are the sum of three products (hi*hi, hi*lo,
 * lo*hi), so they carry nearly fp32 accuracy; v is rounded to bf16 (nearest-even) as it is
 * loaded; the rest is the bf16 entry point's arithmetic, and the fp32 result is stored
 * without rounding. Same arguments and errors as
 * mixer_prefill_async, with float pointers.
 */
int mixer_prefill_f32_async(const float *q, const float *k, const float *v, float *out,
                            int variant, int window, float lambda,
                            int B, int H, int L, int d, void *stream);

/*
 * mixer_latin_build -- the cyclic Latin square of order N (sec. 1, sec. 3.2; the 4x4
 * schedule of Table 7 is this construction): sched[r * N + c] = base[(r + c) mod N],
 * written row-major, so layer l = r * N + c runs type sched[l]. Pure host.
 * N >= 1; base: N ints; sched: N*N ints (written). Returns MIXER_OK or MIXER_EINVAL.
 */
int mixer_latin_build(int N, const int *base, int *sched);

/*
 * mixer_latin_check -- 1 if the row-major N x N schedule holds exactly N distinct types and
 * no type repeats within any row or any column (sec. 1, sec. 3.2),
 * 0 if not, MIXER_EINVAL for N < 1 or a null pointer. Pure host.
 */
int mixer_latin_check(int N, const int *sched);

/*
 * mixer_stack_prefill -- runs the N*N layers of a Latin-square schedule back to back on one
 * stream (layer l runs variant sched[l] on q[l], k[l], v[l] into out[l]); the host never
 * waits between layers.
 *
 * sched           N*N mixer_variant values, row-major; must pass mixer_latin_check.
 * q, k, v, out    host arrays of N*N device pointers, one [B, H, L, d] bf16 tensor each.
 * window, lambda  used by the SLIDING and DIFFERENTIAL layers respectively.
 * layer_events    NULL, or a host array of N*N + 1 hipEvent_t (passed as void*): event 0
 *                 is recorded before layer 0 and event l + 1 after layer l; a NULL entry
 *                 records nothing there (each record costs the stream a few microseconds).
 * Every layer's arguments are validated before the first launch. Returns MIXER_OK,
 * MIXER_ENOTLATIN (schedule not Latin; nothing launched), the first invalid layer's
 * validation error (nothing launched), or MIXER_EHIP as mixer_layers_prefill reports it.
 */
int mixer_stack_prefill(int N, const int *sched,
                        const void *const *q, const void *const *k, const void *const *v,
                        void *const *out, int window, float lambda,
                        int B, int H, int L, int d, void *stream, void *const *layer_events);

/*
 * mixer_layers_prefill -- n layers of any variants back to back on one stream, with no
 * Latin-square check: the runner mixer_stack_prefill uses after its check. It also runs the
 * other depth orders of one layer multiset, the placement arms of Table 7 (sec. 6.1):
 * periodic (the same row repeated), block (each type in one band) and the homogeneous
 * all-FULL reference.
 *
 * variants        n mixer_variant values; layer l runs variants[l].
 * q, k, v, out    host arrays of n device pointers, one [B, H, L, d] bf16 tensor each.
 * window, lambda, layer_events   as for mixer_stack_prefill (layer_events: n + 1 events).
 * Every layer's arguments are validated before the first launch. Returns MIXER_OK, the
 * first invalid layer's validation error (nothing launched then), or MIXER_EHIP when the
 * runtime refuses a launch or an event record part-way: layers 0 .. l-1 before the failing
 * one (and their events) may then already be enqueued on `stream` and will run; the
 * caller synchronises the stream before reusing their outputs.
 */
int mixer_layers_prefill(int n, const int *variants,
                         const void *const *q, const void *const *k, const void *const *v,
                         void *const *out, int window, float lambda,
                         int B, int H, int L, int d, void *stream, void *const *layer_events);

/* ---- Measurement aid (not part of the method) ------------------------------------------
 * The bf16 matrix-core rate the GPU sustains under its power cap when it runs nothing but
 * v_mfma_f32_32x32x16_bf16, used to rate the prefill kernels beside the data-sheet peak.
 * `blocks` workgroups of 4 waves; each wave keeps 4 independent accumulator chains of
 * `iters` instructions each (32*32*16*2 flops per instruction), so one call executes
 * blocks * 16 * iters * 32768 flops.
 *
 * frags   device, bf16, nsets fragment sets of 8 x 64 lanes x 8 elements (8 KiB per set):
 *         fragments 0-3 are A operands (lane l: row l % 32, k = 8*(l/32) + [0, 8) of a
 *         32 x 16 matrix), fragments 4-7 are B operands (lane l: column l % 32, the same k).
 *         Wave w (w = 4 * workgroup + wave) reads set w % nsets. Not written.
 * sink    device, fp32, blocks * 4 * 4 * 16 * 64 floats, written: chain c of wave w ends
 *         holding (iters/4) * sum_{u=0..3} A[(u+c)%4] B[(u+2c)%4] (a 32 x 32 matrix); its
 *         element (i, j) is at sink[((w*4 + c)*16 + r)*64 + lane] with lane = j + 32*((i/4)%2)
 *         and r = 4*(i/8) + i%4.
 * Both pointers 16-byte aligned and not overlapping; 1 <= nsets, blocks <= 2^20; iters a
 * positive multiple of 4. Returns MIXER_OK, MIXER_EINVAL or MIXER_EHIP; asynchronous on
 * `stream` like the *_async calls.
 */
int mixer_mfma_ceiling_async(const void *frags, int nsets, float *sink, int blocks, int iters,
                             void *stream);

/* A static, human-readable description of a mixer_status (never NULL). */
const char *mixer_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* MIXER_H */
