/*
 * boundary.h -- libboundary: the layer-boundary completion path on AMD
 * Instinct MI355X (gfx950).
 *
 * At a layer boundary each token row of the residual stream receives the
 * producer's outstanding contribution and is read by the consumer's norm:
 *   complete: s = sum of the P tensor-parallel partials (or the weighted
 *             gather-sum of a deferred MoE finalize),
 *   fold:     x = r + s, stored back into the bf16 residual,
 *   read:     y = x * w / sqrt(mean(x^2) + eps), as bf16, or as fp8 e4m3
 *             codes with one fp32 scale per token.
 * The semantics follow the SGLang developer guide "Layer boundaries"
 * (sections "Residual stream", "Residual update and input read", "Execute a
 * layer", "Enter and leave the layer stack", "Fusion providers and output
 * decisions") and the study note "SGLang flashinfer_allreduce_fusion精读"
 * (forward section, fusion diagram: all-reduce + residual add + RMSNorm in one
 * kernel, with all-reduce followed by add+norm as the fallback, and the
 * reduce-scatter variant that normalises only the rank's own row slice).
 * On one GPU the cross-rank sum is a sum over P partial buffers resident in
 * device memory.
 *
 * Conventions for every call:
 *   - Device pointers are caller-owned device memory; the library allocates
 *     no device memory and never synchronises, so every call can be
 *     captured into a HIP graph. A bnd_stream is a small host object.
 *   - bf16 tensors are row-major [rows, H] with a leading dimension `ld` in
 *     elements: row t starts at base + t*ld. Bases must be 16-byte aligned
 *     and ld a multiple of 8 with H <= ld <= BND_MAX_LD. H must be a
 *     multiple of 8 in [8, BND_MAX_HIDDEN]. Weights are fp32 [H], 16-byte
 *     aligned. T and the MoE expert-row count are at most BND_MAX_ROWS.
 *   - Reduced inputs (partials, expert index, gates) are indexed by GLOBAL
 *     token row 0..T-1. The residual and every output (y, q, scale, out,
 *     x of enter) are indexed by SLICE row: global row row_begin + i lives at
 *     base + i*ld. A stream over all rows has row_begin = 0, rows = T.
 *   - `hip_stream` is a hipStream_t (NULL = the null stream). Kernels run
 *     asynchronously on it; inputs must stay alive and unmodified until the
 *     consuming kernel has completed in stream order.
 *   - Outputs must not overlap the residual or any input (the norm weight
 *     included), and a residual the call writes must not overlap the weight.
 *   - Errors: every check happens on the host before any launch. On an error
 *     nothing is launched, no output byte changes and the stream's state is
 *     unchanged (a fusion candidate must refuse before touching its inputs,
 *     guide section "Fusion providers and output decisions"). A
 *     description of the last error of the calling thread is available from
 *     bnd_last_error().
 *   - Empty batches (rows == 0) launch nothing but still apply the state
 *     transition, as the final norm's skip_empty mode still completes owed
 *     work (guide section "Enter and leave the layer stack"). Pointers may
 *     then be NULL.
 *   - A bnd_stream is not thread-safe; interleaved microbatches each use
 *     their own stream (guide section "Enter and leave the layer stack",
 *     two-batch overlap).
 */
#ifndef LIBBOUNDARY_BOUNDARY_H
#define LIBBOUNDARY_BOUNDARY_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define BND_API __attribute__((visibility("default")))
#else
#define BND_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

#define BND_MAX_SOURCES 16        /* partials P and MoE picks k: 1..16 */
#define BND_MAX_HIDDEN 32768      /* H: multiple of 8 in [8, 32768] */
#define BND_MAX_ROWS 2147483647   /* T and expert rows: one launch grid, the int32 index range. A call's
                                   * launch also needs rows x threads per row <= 2^32 - 1 (a dispatch
                                   * counts work-items in 32 bits): at H = 4096 at least 8,388,607
                                   * rows fit; a call past its launch's limit returns NO_PATH. */
#define BND_MAX_LD 2147483647     /* leading dimensions, in elements */

/* Stream states, guide section "Residual stream" (state table). */
typedef enum bnd_state {
  BND_INITIAL = 0, /* neither residual nor contribution: the next read enters */
  BND_WRITTEN = 1, /* a residual and nothing pending: the next read applies no update */
  BND_PENDING = 2  /* a contribution, with or without a residual: complete, fold, read */
} bnd_state;

/* Kind of pending contribution. */
typedef enum bnd_kind {
  BND_KIND_NONE = 0,
  BND_KIND_PARTIALS = 1, /* P unreduced TP partial outputs */
  BND_KIND_MOE = 2       /* deferred MoE finalize handoff */
} bnd_kind;

/* Weight form of the consumer's RMSNorm. PLAIN: y = x * inv * w. GEMMA:
 * y = x * inv * (1 + w), the GemmaRMSNorm weight that the guide's fused
 * terminal finalize reads (section "Enter and leave the layer stack"); the
 * page does not spell the form out, this is the Gemma convention of a weight
 * stored as an offset from one. */
typedef enum bnd_norm_form { BND_NORM_PLAIN = 0, BND_NORM_GEMMA = 1 } bnd_norm_form;

typedef enum bnd_status {
  BND_OK = 0,
  BND_ERR_INVALID_ARG = -1,    /* null / misaligned pointer, bad ld, eps < 0, bad rows, overlap */
  BND_ERR_NOT_STARTED = -2,    /* a fold/complete on an Initial stream with nothing published */
  BND_ERR_FOREIGN_OUTPUT = -3, /* the owed token is not this stream's current one */
  BND_ERR_PENDING = -4,        /* enter/publish/take_output while a contribution is pending */
  BND_ERR_WRONG_KIND = -5,     /* the call does not complete this kind of contribution */
  BND_ERR_NO_PATH = -6,        /* H, P or k outside the supported range / launch shape */
  BND_ERR_UNAVAILABLE = -7,    /* fused completion switched off: use the unfused fallback */
  BND_ERR_HIP = -8             /* the HIP runtime refused the launch */
} bnd_status;

typedef struct bnd_stream bnd_stream;

/* Opaque handle of an unfinished output (guide: OwedOutput). Valid for one
 * stream and one publication; 0 means "nothing owed". */
typedef uint64_t bnd_owed;
#define BND_OWED_NONE ((bnd_owed)0)

/* ------------------------------------------------------------------------ */
/* Stream lifetime                                                          */
/* ------------------------------------------------------------------------ */

/* Start a stream over T token rows of hidden size H, holding rows
 * [row_begin, row_begin + rows) (the reduce-scatter share; 0, T for all rows),
 * in the Initial state (guide: residual_batch.start()). `residual` is the
 * storage of the stream's [rows, H] bf16 residual (slice rows, leading
 * dimension ld_res); it holds no value until a read enters or folds.
 * The first call in a process also reads, once, the current device's CU count
 * and the occupancy of the one-wavefront kernels, which the launch shapes are
 * chosen from on every device the process uses (the devices are taken to be
 * alike); no later call queries the device, so every hot call may run under
 * HIP graph capture.
 * Errors: INVALID_ARG (out == NULL, T < 0, bad slice, residual NULL with
 * rows > 0, misaligned, ld_res), NO_PATH (H, T > BND_MAX_ROWS). */
BND_API bnd_status bnd_stream_create(bnd_stream** out, int64_t T, int64_t H, int64_t row_begin,
                             int64_t rows, void* residual, int64_t ld_res);

/* Free the host object. The device buffers are the caller's. */
BND_API bnd_status bnd_stream_destroy(bnd_stream* s);

BND_API bnd_state bnd_stream_state(const bnd_stream* s);
BND_API bnd_kind bnd_stream_pending_kind(const bnd_stream* s);
/* 1 when the residual storage holds the stream's residual value. */
BND_API int bnd_stream_has_residual(const bnd_stream* s);

/* Weight form used by every later read on this stream (host only; the
 * default is BND_NORM_PLAIN). A model stack uses one norm class throughout,
 * so the form belongs to the stream rather than to each call.
 * Errors: INVALID_ARG (NULL stream, unknown form). */
BND_API bnd_status bnd_stream_set_norm_form(bnd_stream* s, bnd_norm_form form);

/* ------------------------------------------------------------------------ */
/* Publishing owed work (host only, nothing is launched)                    */
/* ------------------------------------------------------------------------ */

/* Record P unreduced partial outputs [T, H] bf16 (global rows, common ld) as
 * the stream's pending contribution (guide: finish() of an output that leaves
 * its sum to the next boundary; ResidualStream.leave()). The pointer array is
 * copied. From Initial the stream becomes Pending without a residual; from
 * Written, Pending with it. *owed receives the handle that the next read must
 * present.
 * Errors: PENDING, NO_PATH (P outside 1..16), INVALID_ARG. */
BND_API bnd_status bnd_publish_partials(bnd_stream* s, const void* const* partials, int P, int64_t ld,
                                bnd_owed* owed);

/* Record a deferred MoE finalize (guide: HandoffOutput): token t's
 * contribution is sum_j gate[t*k + j] * expert_rows[idx[t*k + j], :], over
 * the k picks. expert_rows is [n_rows, H] bf16 (leading dimension ld); idx is
 * int32 [T, k] in gather form (the row of expert_rows holding pick j of
 * token t); gate is fp32 [T, k], used as given. An index outside
 * [0, n_rows) contributes nothing, so a corrupt index cannot read outside the
 * buffer. Errors: PENDING, NO_PATH (k outside 1..16), INVALID_ARG. */
BND_API bnd_status bnd_publish_moe(bnd_stream* s, const void* expert_rows, int64_t n_rows, int64_t ld,
                           const int32_t* idx, const float* gate, int k, bnd_owed* owed);

/* ------------------------------------------------------------------------ */
/* The hot calls                                                            */
/* ------------------------------------------------------------------------ */

/* Read at stack entry (guide: the consumer's enter). From Initial: the
 * residual is initialised from x ([rows, H] bf16, slice rows; when x is the
 * residual storage itself, with the same ld, nothing is copied) and
 * y = norm(x). From Written the entry is skipped, x is ignored and
 * y = norm(residual) (a stack-entry boundary accepts a written stream).
 * The stream ends Written. Errors: PENDING, INVALID_ARG. */
BND_API bnd_status bnd_enter_norm(bnd_stream* s, const void* x, int64_t ld_x, const float* w, float eps,
                          void* y, int64_t ld_y, void* hip_stream);

/* The fused boundary (fusion points of the study note's diagram): from
 * Pending with partials, per row, s = sum_p c_p, x = r + s (r = 0 without a
 * residual), residual <- bf16(x), y <- bf16(x * w / sqrt(mean(x^2) + eps)),
 * the norm taken on the fp32 sum, not on the rounded residual. From Written
 * (owed must be BND_OWED_NONE) only the read runs: no second update. The
 * stream ends Written. Errors: NOT_STARTED (Initial), FOREIGN_OUTPUT,
 * WRONG_KIND (MoE pending), UNAVAILABLE (fusion off and P > 1),
 * INVALID_ARG, NO_PATH, HIP. */
BND_API bnd_status bnd_fold_norm(bnd_stream* s, bnd_owed owed, const float* w, float eps, void* y,
                         int64_t ld_y, void* hip_stream);

/* As bnd_fold_norm, with a quantised read (guide: prepare() may return
 * quantised input): per row, scale[i] = fp32(max_h |y_h| / 448) and
 * q[i, h] = e4m3fn(y_h / scale[i]) (OCP E4M3FN, round to nearest even,
 * saturating at +-448; a row with max |y| = 0 gets scale 0 and +0 codes).
 * q is [rows, H] uint8 (8-byte aligned, ld_q a multiple of 8, >= H), scale is
 * fp32 [rows]. The bf16 residual is written as in bnd_fold_norm. */
BND_API bnd_status bnd_fold_norm_quant_fp8(bnd_stream* s, bnd_owed owed, const float* w, float eps,
                                   uint8_t* q, int64_t ld_q, float* scale, void* hip_stream);

/* Finalize a deferred MoE handoff fused with the fold and the read (guide
 * section "Enter and leave the layer stack": finalize, all-reduce, residual
 * add and norm in one pass): s = sum_j gate * expert row, then as
 * bnd_fold_norm; the weighted sum is not rounded before the fold. From
 * Written only the read runs. Errors: NOT_STARTED, FOREIGN_OUTPUT,
 * WRONG_KIND (partials pending), UNAVAILABLE, INVALID_ARG, NO_PATH, HIP. */
BND_API bnd_status bnd_moe_finalize_fold_norm(bnd_stream* s, bnd_owed owed, const float* w, float eps,
                                      void* y, int64_t ld_y, void* hip_stream);

/* Complete the owed work only, leaving the update pending (guide:
 * complete_output()): out[i, :] = bf16(s) for the slice rows ([rows, H],
 * slice rows). The stream stays Pending, now with one partial that is `out`;
 * *new_owed receives its handle and the old one becomes stale. This and a
 * one-source bnd_fold_norm form the unfused fallback (all-reduce, then
 * add+norm). Errors: NOT_STARTED (Initial), WRONG_KIND (Written: nothing
 * owed), FOREIGN_OUTPUT, INVALID_ARG, NO_PATH, HIP. */
BND_API bnd_status bnd_complete_only(bnd_stream* s, bnd_owed owed, void* out, int64_t ld_out,
                             bnd_owed* new_owed, void* hip_stream);

/* Add an extra contribution exactly once (guide, section "Auxiliary capture
 * and extra contributions": add_to_output completes the contribution before
 * adding the extra once and keeps the residual update pending; the
 * integration checklist routes deepstack embeddings through it).
 * out[i, :] = bf16(s + extra[row_begin + i, :]) for the slice rows, where s is
 * the completed owed sum (partials, or the MoE finalize) and extra is
 * [T, H] bf16 indexed by global row like the partials. The stream stays
 * Pending, owing one partial that is `out`; *new_owed receives its handle.
 * Errors: as bnd_complete_only, and INVALID_ARG for a missing or
 * overlapping extra. */
BND_API bnd_status bnd_add_to_output(bnd_stream* s, bnd_owed owed, const void* extra, int64_t ld_extra,
                                     void* out, int64_t ld_out, bnd_owed* new_owed, void* hip_stream);

/* A plain residual snapshot that leaves the owed work in place (guide,
 * section "Auxiliary capture and extra contributions": snapshot() produces
 * an owned plain residual snapshot, the sum runs on a copy without consuming
 * the main contribution, and a producer-specific handoff is refused).
 * out[i, :] = bf16(r + s) for the slice rows (r = 0 on a Pending stream
 * without a residual; from Written, owed = BND_OWED_NONE and out is a copy of
 * the residual). The stream, its residual and its owed handle do not change.
 * Errors: NOT_STARTED (Initial), FOREIGN_OUTPUT, WRONG_KIND (MoE handoff
 * pending), INVALID_ARG, NO_PATH, HIP. */
BND_API bnd_status bnd_snapshot(bnd_stream* s, bnd_owed owed, void* out, int64_t ld_out, void* hip_stream);

/* Row share of rank r under a variable-size reduce-scatter (guide, section
 * "Choose a reduction policy": rsv, whose per-rank row counts come from the
 * batch metadata rather than an even split): rows
 * [sum_{i<r} counts[i], that + counts[r]) of a batch of T = sum(counts) rows,
 * for bnd_stream_create's row_begin and rows. Host only.
 * Errors: INVALID_ARG (NULL pointer, r outside [0, R), a negative count,
 * overflow). */
BND_API bnd_status bnd_rsv_share(const int64_t* counts, int R, int r, int64_t* row_begin, int64_t* rows,
                                 int64_t* T);

/* ------------------------------------------------------------------------ */
/* Host-only transitions (guide: the residual.batch helpers)                */
/* ------------------------------------------------------------------------ */

/* The stream becomes Written with `residual` ([rows, H] bf16, slice rows) as
 * its residual storage and value; a pending contribution is discarded.
 * Errors: INVALID_ARG. */
BND_API bnd_status bnd_written(bnd_stream* s, void* residual, int64_t ld_res);

/* Release the stream at a terminal exit whose output is written: it returns
 * to Initial (a later forward starts afresh). Errors: PENDING. */
BND_API bnd_status bnd_take_output(bnd_stream* s);

/* ------------------------------------------------------------------------ */
/* Diagnostics and options                                                  */
/* ------------------------------------------------------------------------ */

BND_API const char* bnd_status_str(bnd_status st);
/* Description of the calling thread's last error ("" if none). */
BND_API const char* bnd_last_error(void);
BND_API const char* bnd_version(void);

typedef enum bnd_option {
  /* 1: fused completion is unavailable (multi-source folds and MoE finalize
   * return BND_ERR_UNAVAILABLE, the caller completes and folds unfused).
   * Default 0, or 1 when the environment sets BND_DISABLE_FUSED=1. */
  BND_OPT_FUSED_UNAVAILABLE = 1,
  /* Launch-shape overrides for tuning; 0 = automatic (the library's measured
   * choice, which never changes a result: every shape gives the same bits).
   * Threads per row: a multiple of 64 in [64, 1024]. Vectors (of 8 elements)
   * per thread: 1, 2 or 4 for rows of several wavefronts; an even count
   * 6 .. 16 selects one wavefront (64 threads) per row with that many
   * vectors per lane, for calls that take owed partials or MoE picks only
   * (up to 14 for the reads, 16 for complete_only, add_to_output, snapshot).
   * A shape that cannot cover H, or that no kernel of the call has, fails
   * with NO_PATH. */
  BND_OPT_THREADS_PER_ROW = 2,
  BND_OPT_VECTORS_PER_THREAD = 3,
  /* One wavefront per row: BND_ONE_WAVEFRONT_AUTO (default) lets the library
   * choose; ALWAYS makes every call take its one-wavefront kernel (a forced
   * vector count then names its width, 2 and 4 included; the narrowest width
   * that covers H otherwise; NO_PATH where the call has none); NEVER keeps
   * every call on several wavefronts per row. */
  BND_OPT_ONE_WAVEFRONT = 4,
  /* Loads each one-wavefront row keeps in flight: 0 = automatic, 2, or the
   * deep ring of 4, 6 or 8 (every vector of a source in flight; only on a
   * one-wavefront launch of that many vectors per lane, NO_PATH otherwise). */
  BND_OPT_RING_DEPTH = 5
} bnd_option;

#define BND_ONE_WAVEFRONT_AUTO 0
#define BND_ONE_WAVEFRONT_ALWAYS 1
#define BND_ONE_WAVEFRONT_NEVER 2

/* Options are process-wide (every thread and stream sees the same values) and
 * are read when a call chooses its launch, so a change applies to the calls
 * that follow it. bnd_set_option returns BND_ERR_INVALID_ARG, and changes
 * nothing, for an unknown option or a value outside the ranges above;
 * bnd_get_option returns -1 for an unknown option. */
BND_API bnd_status bnd_set_option(bnd_option opt, int64_t value);
BND_API int64_t bnd_get_option(bnd_option opt);

/* The launch shape of the calling thread's last kernel launch through this
 * library: workgroups (one per row), threads per workgroup, 16-byte vectors
 * per thread, and 1 if the kernel was a one-wavefront-per-row kernel (0 if a
 * row had several wavefronts). All 0 before the thread's first launch; a call
 * that launches nothing (an error, zero rows) leaves the previous values. Any
 * pointer may be NULL. Always BND_OK. */
BND_API bnd_status bnd_last_launch_shape(int64_t* rows, int* threads, int* vectors_per_thread,
                                         int* one_wavefront);
/* The load ring depth of the calling thread's last launch through this
 * library: 2, 4, 6 or 8 for one wavefront per row, 0 for several wavefronts (and
 * before the thread's first launch). `depth` may be NULL. Always BND_OK. */
BND_API bnd_status bnd_last_launch_ring_depth(int* depth);

/* Timing: the calling thread's next kernel launch records `start_event` and
 * `stop_event` (hipEvent_t, created by the caller) from its own dispatch
 * (hipExtLaunchKernel), so hipEventElapsedTime between them is that
 * kernel's execution time without queue gaps. The events are used by exactly
 * one launch (a call that launches nothing leaves them armed); NULL, NULL
 * disarms. Not for use while a HIP graph is being captured. */
BND_API bnd_status bnd_time_next_launch(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* LIBBOUNDARY_BOUNDARY_H */
