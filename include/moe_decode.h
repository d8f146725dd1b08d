/*
 * moe_decode.h -- C ABI of the MI355X (gfx950) small-row MoE decode library.
 *
 * One call runs the decode / verify step of a top-8 routed mixture-of-experts
 * layer for 1..8 token rows, entirely in hand-written HIP kernels on the
 * caller's stream:
 *   RMSNorm folded into the router logits -> top-8 (ties to the lower expert
 *   ID) -> softmax gates -> expert dedup table -> FP8 activation blocks ->
 *   up/gate GEMV over low-bit weights -> SiLU * gate, mid re-quantised to FP8
 *   per 1x128 block -> down GEMV -> gate-weighted combine with a shared expert.
 * A second entry point, lowbit_gemv, is a dense decode GEMV over 1-bit
 * group-128 weights or, for the LM head after the last layer, FP8 weights.
 *
 * Sources.  The operations follow the body of sgl-amd-mono PR #85 ("...MoE
 * expert dedup and weight loads, kernarg reload, LM-head loads"), quoted on the
 * GitHub page of sglang PR #47324 (cited below as "#85", with "Mod. row N" for
 * row N of its Modifications table), the README page "SGLang 1-Bit Turbo"
 * (section "PrismML 1-Bit GGUF Model Support (Q1_0_G128)"), and the page of
 * sglang PR #31683 "[ROCm][MI35X] Enable GLM-5.2-MXFP4 MTP speculative
 * decoding" for MXFP4 experts.
 *
 * Conventions for every function below:
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or copies device memory on its own; all scratch
 *    lives in the caller's workspace.  Host objects (the context) are the only
 *    allocations it makes.
 *  - Layouts are row-major; "[N, K]" is N rows of K contiguous elements.
 *    Every pointer must be 16-byte aligned.
 *  - bf16 values are passed as uint16_t bit patterns.
 *  - Validation is synchronous and happens before anything is enqueued; on an
 *    error nothing is launched.  Device faults surface at the caller's next
 *    synchronisation of the stream.  No C++ exception crosses the ABI.
 *  - Work is enqueued on `stream` in stream order; the functions do not
 *    synchronise.  One context per stream: two steps that overlap on one
 *    workspace race.
 */
#ifndef MOE_DECODE_H
#define MOE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null / misaligned pointer, rows out of range, aliasing */
  MOE_ERR_UNSUPPORTED = 2, /* shape or format outside what the kernels implement */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than moe_decode_workspace_size */
  MOE_ERR_DEVICE = 4       /* a HIP launch error (hipGetLastError) */
} moe_status;

/* Weight formats. */
typedef enum {
  /* FP8 E4M3 (OCP E4M3FN, largest finite 448) codes uint8 [N, K] with one fp32
   * scale per 128x128 block, scales float [N/128, K/128] (#85 Mod. rows 18, 21:
   * FP8 expert weights; also lowbit_gemv's FP8 form). */
  MOE_FMT_FP8_E4M3_B128 = 1,
  /* MXFP4: E2M1 codes packed two per byte, element 2i in the low nibble,
   * uint8 [N, K/2], with one E8M0 exponent per 32 elements along K, uint8
   * [N, K/32] (MXFP4 page; #85 Mod. row 1: MXFP4 experts).  Routed experts
   * only; their mid is kept in fp32 (not re-quantised).  Needs hidden % 256
   * == 0 and inter <= 4096. */
  MOE_FMT_MXFP4 = 2,
  /* 1-bit group-128: [N, K/128] blocks of 18 bytes, an fp16 scale d
   * (little-endian) then 16 bytes of sign bits; bit i of byte b is element
   * 8b+i; bit 1 means -d, bit 0 means +d (1-Bit Turbo, Q1_0_G128).
   * lowbit_gemv, and routed experts of the decode step: their scales
   * pointers are unused (may be NULL), their mid is re-quantised to FP8 per
   * 1x128 block as for FP8 experts; needs hidden % 512 == 0, inter % 256 ==
   * 0, inter <= 4096 and FP8 activations. */
  MOE_FMT_Q1_G128 = 3,
  /* bf16 weights [N, K], no scales.  lowbit_gemv only (the tail's LM head
   * kept in bf16). */
  MOE_FMT_BF16 = 4
} moe_wfmt;

/* The experts' input (the up/gate activation). */
typedef enum {
  /* FP8 E4M3 per 1x128 block of u = bf16(x * gamma), scale amax/448 in fp32,
   * rstd applied after the dot (#85 Mod. row 10: FP8 activation blocks).  The
   * default (0, so a zero-initialised config gets it). */
  MOE_ACT_FP8_B128 = 0,
  /* u itself (bf16), rstd applied after the dot: no activation rounding, for
   * measuring what the FP8 blocks cost.  FP8 routed experts only (with
   * MXFP4 routed experts the config is MOE_ERR_UNSUPPORTED). */
  MOE_ACT_BF16 = 1
} moe_afmt;

/* flags */
enum {
  /* Skip the dedup: every (row, pick) streams its expert separately.  For the
   * bitwise A/B check that dedup changes no output bit (#85 Mod. row 16: a
   * row adds its units up in the order it would alone). */
  MOE_F_NO_DEDUP = 1u << 1
};

typedef struct {
  int32_t hidden;       /* H: multiple of 128, at most 16384 */
  int32_t inter;        /* I of a routed expert: multiple of 128, at most 16384 */
  int32_t n_experts;    /* E: multiple of 16, 16..1024 */
  int32_t top_k;        /* must be 8 */
  int32_t shared_inter; /* I of the shared expert: 0 for none, else equal to inter */
  int32_t max_rows;     /* 1..8: the widest step this context will run */
  float rms_eps;        /* RMSNorm epsilon */
  int32_t routed_fmt;   /* MOE_FMT_FP8_E4M3_B128, MOE_FMT_MXFP4 or MOE_FMT_Q1_G128 */
  int32_t shared_fmt;   /* MOE_FMT_FP8_E4M3_B128 */
  uint32_t flags;       /* MOE_F_* */
  int32_t act_fmt;      /* moe_afmt: MOE_ACT_FP8_B128 (0) or MOE_ACT_BF16 */
} moe_decode_config;

/* One stored matrix: codes and scales in the layout its format fixes. */
typedef struct {
  const void* codes;
  const void* scales;
} moe_tensor;

typedef struct {
  const uint16_t* rms_gamma; /* bf16 [H] */
  const uint16_t* router_w;  /* bf16 [E, H] */
  moe_tensor gate, up;       /* routed, expert-major stacks of [I, H] */
  moe_tensor down;           /* routed, expert-major stack of [H, I] */
  moe_tensor sh_gate, sh_up; /* shared expert [Is, H] (unused when Is == 0) */
  moe_tensor sh_down;        /* shared expert [H, Is] */
} moe_decode_weights;

typedef struct moe_decode_ctx moe_decode_ctx;

/* Bytes of device workspace a context with this config needs, or 0 when the
 * config is not supported. */
size_t moe_decode_workspace_size(const moe_decode_config* cfg);

/* Validate cfg, bind the caller's workspace (device, >= the size above) and
 * create a context.  Enqueues one small kernel on `stream` that clears the
 * workspace (so debug views read before the first step are defined); later
 * steps on the same stream are ordered after it.  The workspace must be
 * 256-byte aligned.
 * Returns MOE_ERR_UNSUPPORTED for configs the kernels do not implement,
 * MOE_ERR_WORKSPACE for a missing or short workspace. */
moe_status moe_decode_init(const moe_decode_config* cfg, void* workspace, size_t ws_bytes,
                           hipStream_t stream, moe_decode_ctx** out);

/* One decode step (#85: the MoE part of a decoder-layer launch).
 *  x    bf16 [rows, H] token rows (device)
 *  rows 0..max_rows; 0 enqueues nothing and returns MOE_OK (zero-work
 *       launches are skipped)
 *  w    weights; every pointer it holds is a device pointer
 *  out  bf16 [rows, H] (device); must not overlap x
 * The output is the MoE branch only: sum_j g_j * expert_{e_j}(x) + shared(x),
 * with no residual.  Selection, gates, dedup table, activation blocks and mid
 * of the last step stay readable through moe_decode_debug_view until the next
 * step on this context. */
moe_status moe_decode_step(moe_decode_ctx* ctx, const uint16_t* x, int32_t rows,
                           const moe_decode_weights* w, uint16_t* out, hipStream_t stream);

/* The decode step without a context or workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same validation, kernels and result
 * as moe_decode_step with a context created from `cfg`, but the step's
 * intermediates live in a static device array of the library
 * (MOE_DECODE_NOALLOC_MAX_WORKSPACE bytes, one per GPU, held until the
 * process ends).  It calls no hipMalloc, hipFree or other allocating routine;
 * the first call on a device looks up that array's device address.
 *  cfg  as for moe_decode_init; its workspace (moe_decode_workspace_size) must
 *       be at most MOE_DECODE_NOALLOC_MAX_WORKSPACE bytes, else
 *       MOE_ERR_WORKSPACE (a GLM-scale layer at 8 rows needs about 2.6 MB)
 *  x, rows, w, out, stream  as for moe_decode_step
 * Every call on one GPU shares that GPU's array, and the array keeps the
 * last call's intermediates: two calls that overlap on one GPU (other
 * streams, other threads) race and may corrupt each other's output.  No
 * debug view, timing or relaunch is available for these steps. */
#define MOE_DECODE_NOALLOC_MAX_WORKSPACE ((size_t)8 << 20)
moe_status moe_decode_step_noalloc(const moe_decode_config* cfg, const uint16_t* x,
                                   int32_t rows, const moe_decode_weights* w, uint16_t* out,
                                   hipStream_t stream);

/* Device pointers into the workspace holding the last step's intermediates. */
typedef struct {
  const float* logits;       /* [max_rows, E]: the fp32 values the top-8 compared */
  const float* rstd;         /* [max_rows] */
  const int32_t* ids;        /* [max_rows, 8] picks in top-8 order */
  const float* gates;        /* [max_rows, 8] softmax of the 8 picked logits */
  const int32_t* n_groups;   /* [1] D, the number of distinct routed experts */
  const int32_t* grp_expert; /* [max_groups] expert of group g (slot-major first use) */
  const uint8_t* grp_owner;  /* [max_groups, 2] (slot, row) of the group's first use */
  const uint8_t* grp_mask;   /* [max_groups] bit r set when row r uses the group */
  const uint8_t* grp_slot;   /* [max_groups, 8] slot where row r picked it, 0xFF if none */
  const uint8_t* act_q;      /* [max_rows, H] FP8 activation codes (zero with MOE_ACT_BF16) */
  const float* act_s;        /* [max_rows, H/128] their block scales (zero with MOE_ACT_BF16) */
  /* mid, per (row r, pick j) with j = 8 for the shared expert, at index
   * r * 9 + j, with stride mid_stride elements (a deduplicated expert's mid
   * appears under every (row, pick) that uses it): */
  const float* mid;          /* [max_rows, 9, mid_stride] fp32, before quantisation */
  const uint8_t* midq;       /* [max_rows, 9, mid_stride] FP8 codes */
  const float* midqs;        /* [max_rows, 9, mid_stride/128] block scales */
  const float* y;            /* [max_rows, 9, H] fp32 down output per (row, pick), before
                                the gate-weighted combine; same indexing as mid */
  int32_t max_groups;        /* min(8 * max_rows, E), or 8 * max_rows with MOE_F_NO_DEDUP */
  int32_t mid_stride;        /* max(I, Is) */
} moe_decode_debug;

moe_status moe_decode_debug_view(const moe_decode_ctx* ctx, moe_decode_debug* view);

/* Optional per-kernel timing: when `events` is non-null, every later step
 * records events[0] before its first kernel and events[i+1] after kernel i
 * (MOE_DECODE_N_KERNELS kernels), on the step's stream.  The caller owns the
 * events (hipEventCreate) and must keep them alive; pass NULL to stop. */
#define MOE_DECODE_N_KERNELS 5 /* router, routing (with the up/gate of the shared and the
                                  routed experts + mid), up/gate + mid (an empty span when
                                  the routing launch ran it), down, combine */
moe_status moe_decode_set_timing(moe_decode_ctx* ctx, hipEvent_t* events);

/* Kernel timing without per-kernel events: enqueues `reps` more launches of
 * one kernel of the last step enqueued on this context (the up/gate or the
 * down GEMV), with that step's row count, router logits, routing table and
 * activations in the workspace, and the weights `w` -- which must hold the
 * same experts at
 * possibly other addresses, e.g. another copy of the layer, so that repeated
 * launches stream from HBM rather than from a cache.  The relaunched kernel
 * rewrites the same workspace values (mid, or the down outputs); the step's
 * output is not touched.  For measurement only (the caller brackets the
 * launches with its own events).
 * Returns MOE_ERR_INVALID_ARG without a previous step, for another kernel, for
 * reps < 0 or for weights that step validation rejects. */
/* MOE_DECODE_K_UPGATE relaunches the launch that ran the step's up/gate: the
 * routing launch, routing included, when the up/gate runs in it. */
#define MOE_DECODE_K_UPGATE 2
#define MOE_DECODE_K_DOWN 3
moe_status moe_decode_relaunch(moe_decode_ctx* ctx, int32_t kernel,
                               const moe_decode_weights* w, int32_t reps, hipStream_t stream);

/* The routing launch's waits (#85 Mod. row 3 and its `poll` section: the
 * routed experts' weights stream as soon as the routing has chosen them).
 * In steps of up to 4 rows the up/gate runs in the routing launch, whose
 * routed up/gate blocks each wait for a record that the routing block
 * publishes (wider steps run the routing alone and do not wait); a wait gives up after `cap_ticks` of the GPU's
 * 100 MHz real-time counter (0 restores the default, 10 ms), and a block that
 * gives up counts itself and skips its work, so that the step's output is then
 * wrong but every kernel ends.  withhold = 1 makes the routing block publish no
 * record, so that every routed block gives up: for tests of that path only.
 * Applies to later steps and relaunches of this context.
 * Returns MOE_ERR_INVALID_ARG for a null context or withhold not 0 or 1. */
moe_status moe_decode_set_wait(moe_decode_ctx* ctx, uint32_t cap_ticks, int32_t withhold);

/* The number of routed blocks that gave up waiting, summed over every step and
 * relaunch of this context's workspace since moe_decode_init (0 when every
 * routed block got its record).  Reads it on `stream`, after the work enqueued
 * there, and synchronizes that stream. */
moe_status moe_decode_wait_timeouts(moe_decode_ctx* ctx, uint32_t* count, hipStream_t stream);

void moe_decode_destroy(moe_decode_ctx* ctx);

const char* moe_status_string(moe_status s);

/* Dense decode GEMV, in one of three weight formats.
 *
 * MOE_FMT_Q1_G128 -- 1-bit group-128 weights (1-Bit Turbo, Q1_0_G128):
 *   y[n] = bf16( sum_g d[n,g] * sum_{k in g} sign[n,k] * x[k] ),
 * x used as bf16 directly, fp32 accumulation.  w->k a multiple of 128 (at
 * most 16384); w->codes points to the [N, K/128, 18] blocks (device);
 * w->scales is unused (the scales are in the blocks).  rows 1..8 (the
 * page's path was batch 1; several rows need K a multiple of 256 and are
 * computed together, each row as its batch-1 definition).  x bf16 [rows, K],
 * y bf16 [rows, N], both 16-byte aligned.
 *
 * MOE_FMT_FP8_E4M3_B128 -- FP8 weights with one fp32 scale per 128x128 block,
 * for the tail's LM-head GEMV after the last layer (#85 Mod. row 24: the tail
 * keeps its LM-head weight loads in flight across its tiles):
 *   y[r][n] = bf16( sum_k dec(W[n,k]) * s[n/128,k/128] * x[r][k] ),
 * x bf16 used directly (no activation quantisation), fp32 accumulation.
 * w->n and w->k multiples of 128; w->codes uint8 [N, K] (16-byte aligned),
 * w->scales float [N/128, K/128]; rows 1..8; x bf16 [rows, K] (16-byte
 * aligned), y bf16 [rows, N].
 *
 * MOE_FMT_BF16 -- bf16 weights, the same tail GEMV with the LM head kept in
 * bf16 (#85 Mod. row 24; the page names no weight format for the tail):
 *   y[r][n] = bf16( sum_k W[n,k] * x[r][k] ),
 * fp32 accumulation.  w->n a multiple of 128, w->k of 64; w->codes bf16
 * [N, K] (16-byte aligned); w->scales is unused; rows 1..8; x bf16 [rows, K]
 * (16-byte aligned), y bf16 [rows, N].
 *
 * All forms: all pointers are device memory owned by the caller; x and y must not
 * overlap; rows == 0 or N == 0 is a no-op.  Validation runs before anything
 * is enqueued: a null or misaligned pointer, negative sizes or overlap ->
 * MOE_ERR_INVALID_ARG; an unknown format, sizes off the form's grid or too
 * many rows -> MOE_ERR_UNSUPPORTED; a launch error -> MOE_ERR_DEVICE. */
typedef struct {
  int32_t fmt, n, k;
  const void* codes;
  const void* scales;
} lowbit_matrix;

moe_status lowbit_gemv(const lowbit_matrix* w, const uint16_t* x, int32_t rows, uint16_t* y,
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_DECODE_H */
