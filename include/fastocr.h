/*
 * fastocr.h -- C ABI of the MI355X (gfx950) decode-step attention library for
 * FastOCR's Dynamic Visual Fixation.
 *
 * Source of the method: "FastOCR: Dynamic Visual Fixation via KV Cache Pruning
 * for Efficient Document Parsing" -- the technical summary (sections "Method",
 * "1. Focal-Guided Pruning" with "Focal Layer Selection" and "Cross-Layer
 * Propagation", "2. Cross-Step Fixation Reuse" with "Mechanism" and
 * "Implementation") and the paper's abstract.
 *
 * The library replaces the per-layer decode-attention call of a decoder.  The
 * caller keeps the full KV cache; the library never writes it (nothing is
 * evicted: Method).  Per decode step and layer it runs one of:
 *   - full attention (warm-up steps, focal layers, and the FULL baseline mode),
 *   - full attention + head-summed image-token scores + top-k(tau) on focal
 *     layers (Cross-Layer Propagation),
 *   - attention over the kept image tokens plus every text row on non-focal
 *     layers (Cross-Layer Propagation),
 * and carries the deepest focal layer's set into the next step on the device
 * (Cross-Step Fixation Reuse / Implementation).  A w-step warm-up picks the
 * focal layers from per-layer image-attention ratio (Focal Layer Selection).
 *
 * Conventions for every entry point:
 *   - Return value: FASTOCR_OK (0) or a negative FASTOCR_ERR_* code.  Nothing
 *     throws across the ABI and nothing aborts.
 *   - "device" pointers are HIP device memory on the handle's device; "host"
 *     pointers are ordinary host memory.  The caller owns every pointer it
 *     passes; the library keeps none of them past the call (kernels read them
 *     asynchronously on the handle's stream, so they must stay valid until
 *     that stream has passed the work).
 *   - Tensors are dense, row-major (last index fastest), 16-byte aligned.
 *   - The handle owns its scratch memory (allocated in fastocr_create; no
 *     allocation happens in fastocr_attend).  One handle = one stream; a
 *     handle is not thread-safe.
 *   - After FASTOCR_ERR_HIP the handle is poisoned: every later call except
 *     fastocr_destroy returns FASTOCR_ERR_STATE.
 *
 * Environment settings, read once by fastocr_create (for measurement and
 * tests; results do not depend on them beyond rounding order):
 *   FASTOCR_FULL_ROWS=R     rows per split of full passes (multiple of 16)
 *   FASTOCR_SPARSE_ROWS=R   kept-token passes: as many workgroups per (sequence,
 *                           KV head) pair as R rows each need at the longest
 *                           text the handle accepts (default: the workgroups
 *                           that fill one wave of the device); R at least that
 *                           length gives one workgroup per pair, which writes
 *                           the output (no merge)
 *   FASTOCR_KEPT_ALL_AS_FULL=0|1  with tau = 1, non-focal layers run the full
 *                           pass (default 1) or the kept-token pass over
 *                           every image token (0)
 *   FASTOCR_STREAM_ROWS=0|1 pruned steps' kept-token passes and focal-layer
 *                           passes load their K/V rows plainly (0) or
 *                           non-temporally (1); default:
 *                           non-temporally when one step's kept rows of the
 *                           non-focal layers, at the longest text, exceed the
 *                           256 MiB last-level cache
 *   FASTOCR_FOCAL_STAGE=0|1 focal passes never stage a split's image-token
 *                           logits in LDS (0: stored as they are computed), or
 *                           stage them whenever they fit (1); default: stage
 *                           them when they fit and a split has at least 512 rows
 *   FASTOCR_SKIP_DEAD_PICKS=0|1  a focal layer directly followed by another
 *                           focal layer skips its scores and top-k (default 1;
 *                           the outputs and the kept sets any layer uses are
 *                           the same either way)
 *   FASTOCR_TRACE=0|1       a named roctx range around every fastocr_attend
 *                           call ("fastocr step S layer L <kind>") and the
 *                           focal-layer profile, for rocprofv3 --marker-trace
 *                           (the roctx library is opened at run time; default 0)
 *   FASTOCR_VALU_FULL=0|1   full passes (warm-up, FULL mode, tau = 1 non-focal
 *                           layers) without MFMA: fp32 FMAs with 16-lane
 *                           shuffle reductions (bf16, head_dim 128, at most 8
 *                           query heads per KV head; default 0)
 */
#ifndef FASTOCR_H
#define FASTOCR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define FASTOCR_OK 0
#define FASTOCR_ERR_INVALID_ARG (-1) /* null pointer, bad shape, tau out of range, layer out of [0,L) */
#define FASTOCR_ERR_STATE (-2)       /* call out of order for the handle's state machine */
#define FASTOCR_ERR_HIP (-3)         /* HIP runtime failure (no device, launch error, ...) */
#define FASTOCR_ERR_OOM (-4)         /* scratch allocation failed */
#define FASTOCR_ERR_SCRATCH (-5)     /* fastocr_create_static: the configuration needs more scratch
                                        than the static array holds */

/* ---- element types of q, k_cache, v_cache and out ------------------------ */
#define FASTOCR_DTYPE_F32 0
#define FASTOCR_DTYPE_BF16 1

/* ---- modes --------------------------------------------------------------- */
#define FASTOCR_MODE_PRUNED 0 /* warm-up, then focal/non-focal pruning (the method) */
#define FASTOCR_MODE_FULL 1   /* full attention on every layer (unpruned baseline) */

/* ---- device status flags (fastocr_get_status) ---------------------------- */
#define FASTOCR_FLAG_LENS_CLAMPED 1 /* a lens entry was out of range and was clamped */
#define FASTOCR_FLAG_INDEX_CLAMPED 2 /* a selected index was out of range and was clamped */

/* ---- kernel classes timed by fastocr_get_timing -------------------------- */
#define FASTOCR_KC_FULL_SPLIT 0   /* split-K full attention (warm-up, FULL mode) */
#define FASTOCR_KC_FOCAL_SPLIT 1  /* the same with image-logit export (focal layers) */
#define FASTOCR_KC_SPARSE_SPLIT 2 /* split-K attention over gathered kept rows; writes the
                                     output itself when a sequence fits one split */
#define FASTOCR_KC_MERGE 3        /* split merge (+ head-summed image-token scores) */
#define FASTOCR_KC_TOPK 4         /* top-k selection of the kept set */
#define FASTOCR_KC_COUNT 5

typedef struct fastocr_config {
  double tau;             /* kept ratio of image tokens, 0 < tau <= 1 */
  float sm_scale;         /* logit scale; 0 selects 1/sqrt(head_dim) */
  int32_t num_layers;     /* L >= 1 */
  int32_t num_q_heads;    /* Hq, a multiple of num_kv_heads, Hq/Hkv <= 16, Hq <= 128 */
  int32_t num_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;       /* d: 64 or 128 */
  int32_t batch;          /* B >= 1 sequences, B * num_kv_heads <= 65535 */
  int32_t max_seq_len;    /* S: row stride of the KV cache (capacity per sequence) */
  int32_t max_img_tokens; /* upper bound on image tokens per sequence (<= S) */
  int32_t min_img_tokens; /* lower bound on image tokens per sequence, 0 if unknown;
                             only used to size launches (a sequence outside the
                             declared bounds is still attended in full) */
  int32_t dtype;          /* FASTOCR_DTYPE_* */
  int32_t num_focal;      /* |C|, 1 <= |C| <= L */
  int32_t warmup_steps;   /* w >= 1 */
  int32_t mode;           /* FASTOCR_MODE_* */
  int32_t max_text_tokens; /* upper bound on a sequence's text tokens len_b - n_img_b
                              (prompt + generated), 0 if unknown; only used to size
                              the kept-token launch (a sequence beyond it is still
                              attended in full) */
  int32_t reprofile_every; /* R >= 0: after every R pruned steps the next w steps are a new
                              warm-up window and the focal set is picked again from that
                              window alone (periodic re-selection; 0 = pick once) */
} fastocr_config;

typedef struct fastocr_info {
  int32_t step;           /* decode steps completed */
  int32_t next_layer;     /* layer the next fastocr_attend must name */
  int32_t phase;          /* 0 warm-up, 1 warm-up done (profile next), 2 pruned, 3 full */
  int32_t k_max;          /* capacity of the kept-set buffer per sequence */
  int32_t full_rows_per_split;
  int32_t full_max_splits;
  int32_t sparse_rows_per_split; /* kept-token pass: rows per workgroup at the longest text */
  int32_t sparse_max_splits;     /* kept-token pass: workgroups per (sequence, KV head) pair */
  int32_t sparse_direct;  /* 1: non-focal layers finish in one workgroup per (sequence, KV head)
                             pair (no merge launch) */
  int32_t focal_staged;   /* 1: focal passes keep a split's image-token logits in LDS and write
                             them once its rows are done (0: as they are computed) */
  int32_t stream_rows;    /* 1: pruned steps' kept-token and focal-layer passes load their K/V
                             rows non-temporally (one step's kept rows exceed the 256 MiB
                             last-level cache) */
  int32_t profiles;       /* focal-set picks so far (first warm-up and re-selections) */
  int64_t scratch_bytes;  /* device bytes owned by the handle */
} fastocr_info;

typedef struct fastocr_timing {
  double total_ms[FASTOCR_KC_COUNT]; /* summed time of the timed launches per class (HIP events) */
  int64_t launches[FASTOCR_KC_COUNT]; /* launches recorded */
  int64_t timed[FASTOCR_KC_COUNT];    /* ... of which timed (all but a batch's first) */
} fastocr_timing;

typedef struct fastocr_handle fastocr_handle;

/* fastocr_create: validate cfg, allocate the handle's scratch on the current
 * HIP device and bind the handle to hip_stream (a hipStream_t; NULL = the
 * null stream).  On success *out receives the handle.  Errors:
 * INVALID_ARG (cfg or out null, a field out of range), HIP (no device or
 * runtime failure), OOM (scratch allocation failed). */
int fastocr_create(const fastocr_config* cfg, void* hip_stream, fastocr_handle** out);

/* fastocr_create_static: fastocr_create without any device allocation, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops and harnesses that forbid hipMalloc).  The handle's scratch
 * is placed in a static device array of FASTOCR_STATIC_SCRATCH_MIB MiB that
 * the library holds on every GPU it runs on until the process ends, instead
 * of memory from hipMalloc; nothing else differs (same kernels, same
 * results).  Every static handle on a GPU shares that GPU's array, so at most
 * one is live per GPU at a time: a second fastocr_create_static on the same
 * device before fastocr_destroy of the first returns FASTOCR_ERR_STATE (two
 * handles using the array at once would race).  The array keeps the last
 * handle's contents; creation clears the part a handle uses.  fastocr_destroy
 * releases the array for the next static handle and frees nothing.  The host
 * handle object itself is ordinary host memory.  Errors: as fastocr_create,
 * and FASTOCR_ERR_SCRATCH when the configuration's scratch (fastocr_info
 * scratch_bytes, also given by fastocr_plan_launch) exceeds the array. */
#define FASTOCR_STATIC_SCRATCH_MIB 64
int fastocr_create_static(const fastocr_config* cfg, void* hip_stream, fastocr_handle** out);

/* fastocr_attend: decode attention of one layer at the current step
 * (Method / Focal-Guided Pruning / Cross-Layer Propagation; Cross-Step
 * Fixation Reuse / Implementation).
 *   layer    0..L-1; each step calls every layer once, in order; the step
 *            advances after layer L-1.
 *   q        device [B, Hq, d] of dtype; query of the current token.
 *   k_cache  device [B, Hkv, S, d] of dtype; keys of this layer (read only).
 *   v_cache  device [B, Hkv, S, d] of dtype; values of this layer (read only).
 *   lens     device int32 [B, 2]: (n_img_b, len_b).  Image tokens occupy rows
 *            [0, n_img_b), prompt and generated tokens [n_img_b, len_b); the
 *            current token's key/value is already at row len_b - 1.  n_img_b
 *            must not change over the handle's life.  Out-of-range entries
 *            are clamped on the device and latch FASTOCR_FLAG_LENS_CLAMPED.
 *   out      device [B, Hq, d] of dtype; attention output.
 * Query head h reads KV head h / (Hq / Hkv).  Which computation runs:
 *   FULL mode: full attention.
 *   PRUNED mode, warm-up window (the first w steps, and with reprofile_every
 *            = R > 0 the w steps after every R pruned steps): full
 *            attention; records each head's image mass and, at the window's
 *            last step, every layer's image-token scores.
 *   PRUNED mode, pruned step, layer in C: full attention, then per sequence
 *            the head-summed attention probability of every image token, then
 *            the k_b = clamp(ceil(tau*n_img_b - 1e-9), 1, n_img_b) highest
 *            (ties to the lower index) replace the kept set.  When layer + 1
 *            is in C too, that pick would be replaced before any layer
 *            attends with it, so only the full attention runs (set
 *            FASTOCR_SKIP_DEAD_PICKS=0 to compute it anyway).
 *   PRUNED mode, pruned step, layer not in C: attention over the kept set
 *            plus rows [n_img_b, len_b).
 * The first window ends with fastocr_profile_warmup.  A re-selection window
 * (R > 0) is profiled by the layer-0 call of the step after it, exactly as
 * fastocr_profile_warmup would (that call synchronises the stream); the new
 * focal set is read with fastocr_get_focal_layers.  The focal layers are
 * chosen as the summary's Focal Layer Selection describes; repeating the
 * choice periodically is this library's reading of the adaptive layer
 * selection that the summary's conclusion lists as future work.
 * Asynchronous otherwise: enqueues on the handle's stream and returns.
 * Errors: INVALID_ARG (null pointer, layer out of range), STATE (layer out
 * of order, a pruned step before the first fastocr_profile_warmup, poisoned
 * handle), HIP. */
int fastocr_attend(fastocr_handle* h, int32_t layer, const void* q, const void* k_cache,
                   const void* v_cache, const int32_t* lens, void* out);

/* fastocr_attend_append: fastocr_attend with the current token's key/value
 * appended by the same launches instead of by a separate kernel before the
 * call (the decode step appends the new token before attending: Method).
 *   k_new, v_new  device [B, Hkv, d] of dtype: the current token's key and
 *            value.  They are written into k_cache / v_cache at row len_b - 1
 *            (len_b after clamping; nothing for len_b = 0), and that row's
 *            attention uses them, so the row's previous content never
 *            matters.  The caches must be writable device memory; no other
 *            row is written.
 * Everything else, including outputs and the state machine, is exactly
 * fastocr_attend's: the results equal those of writing the row first and
 * calling fastocr_attend (same operations in the same order).  The cache
 * row is visible to later work on the handle's stream.  Errors: as
 * fastocr_attend, and INVALID_ARG for null k_new / v_new. */
int fastocr_attend_append(fastocr_handle* h, int32_t layer, const void* q, const void* k_new,
                          const void* v_new, void* k_cache, void* v_cache, const int32_t* lens,
                          void* out);

/* fastocr_profile_warmup: after a completed warm-up window (exactly w
 * steps), pick the focal layers (Focal Layer Selection): the |C| layers with
 * the largest mean image-attention mass over heads, sequences and the
 * window's steps (ties to the lower layer), written ascending to
 * focal_layers_out (host, |C| entries).  Initialises the kept set from the
 * window's last step's scores at the deepest focal layer and switches the
 * handle to pruned steps.  Synchronises the stream.  Errors: INVALID_ARG
 * (null), STATE (not exactly after a window), HIP. */
int fastocr_profile_warmup(fastocr_handle* h, int32_t* focal_layers_out);

/* fastocr_get_focal_layers: the current focal set C, ascending, into
 * layers_host (host int32, num_focal entries).  Errors: INVALID_ARG (null),
 * STATE (no focal set picked or set yet). */
int fastocr_get_focal_layers(fastocr_handle* h, int32_t* layers_host);

/* fastocr_destroy: synchronise the stream and free the handle's scratch.
 * NULL is accepted.  Returns HIP if the final synchronisation failed (the
 * memory is released regardless). */
int fastocr_destroy(fastocr_handle* h);

/* ---- inspection and conditioning (test and measurement harness) ---------- */

/* Synchronises; copies the device status flags (FASTOCR_FLAG_*) to *flags. */
int fastocr_get_status(fastocr_handle* h, int32_t* flags);

/* Enqueues device-to-device copies of the current kept set: idx_dev int32
 * [B, k_max] (ascending, first cnt entries valid) and cnt_dev int32 [B]. */
int fastocr_get_selection(fastocr_handle* h, int32_t* idx_dev, int32_t* cnt_dev);

/* Enqueues a device-to-device copy of the image-token scores of the last
 * focal layer that picked a kept set, float [B, max_img_tokens] (entries >=
 * n_img_b are unspecified). */
int fastocr_get_scores(fastocr_handle* h, float* scores_dev);

/* After fastocr_profile_warmup: the L per-layer mean image-attention ratios
 * (host double [L]). */
int fastocr_get_layer_ratios(fastocr_handle* h, double* ratios_host);

/* Replace the focal set C with count = num_focal distinct layers (host int32
 * [count], in [0, L)), at a step boundary.  On a handle whose warm-up window
 * is complete (the first one or a re-selection window) it ends the window
 * the way fastocr_profile_warmup does, with this set instead of the profiled
 * one: the kept set is initialised by top-k of the window's last-step
 * scores at the deepest given layer, and the handle switches to pruned
 * steps (the layer ratios are not computed).  During pruned steps it only
 * replaces C; the kept set carried to the next step is unchanged.
 * Synchronises the stream when it ends a window.  Errors: INVALID_ARG (null,
 * count != num_focal, a layer repeated or out of range), STATE (not at a step
 * boundary, warm-up window not complete, poisoned handle), HIP. */
int fastocr_set_focal_layers(fastocr_handle* h, const int32_t* layers_host, int32_t count);

/* Enqueues device-to-device copies into the kept set (same layout as
 * fastocr_get_selection).  Indices >= n_img_b are clamped by the kernels and
 * latch FASTOCR_FLAG_INDEX_CLAMPED. */
int fastocr_set_selection(fastocr_handle* h, const int32_t* idx_dev, const int32_t* cnt_dev);

int fastocr_get_info(fastocr_handle* h, fastocr_info* info);

/* fastocr_plan_launch: the launch geometry and scratch size fastocr_create
 * would choose for cfg on a device with num_cu compute units (the FASTOCR_*
 * environment overrides included), written to the plan fields of *info
 * (k_max, rows per split and splits of the full and kept-token passes,
 * sparse_direct, focal_staged, stream_rows, scratch_bytes; the state fields are those of
 * a new handle).  Host only: no device is used.  Errors:
 * INVALID_ARG (null, a configuration fastocr_create rejects, num_cu < 1). */
int fastocr_plan_launch(const fastocr_config* cfg, int32_t num_cu, fastocr_info* info);

/* Kernel timing with HIP events on the handle's stream.  enable != 0 makes
 * every launch record an event when its kernel completes (bound to the
 * dispatch: no extra packet is queued).  A launch is timed from the previous
 * timed launch's end to its own end, which is the kernel's duration when the
 * launches are queued back to back (the device never waits for the host, as
 * behind a long-running kernel) and also counts idle time otherwise; the first
 * launch after enabling, a reset or a fastocr_get_timing call is not counted.
 * fastocr_get_timing synchronises the stream and returns the per-class totals
 * since the last reset; fastocr_reset_timing clears them. */
int fastocr_set_timing(fastocr_handle* h, int32_t enable);
int fastocr_get_timing(fastocr_handle* h, fastocr_timing* out);
int fastocr_reset_timing(fastocr_handle* h);

/* ---- standalone operations ------------------------------------------------ */

/* Top-k selection (Cross-Layer Propagation: top-attended image tokens at kept
 * ratio tau) on caller buffers.  scores: device float [B, score_stride],
 * non-negative; lens: device int32 [B, 2] (n_img_b read, clamped to
 * score_stride); idx_out: device int32 [B, idx_stride] receives the k_b
 * indices ascending (k_b as in fastocr_attend, and at most idx_stride);
 * cnt_out: device int32 [B] receives k_b.  Ties go to the lower index.
 * hip_stream: hipStream_t.  Asynchronous.  Errors: INVALID_ARG, HIP. */
int fastocr_select_topk(const float* scores, int32_t score_stride, const int32_t* lens,
                        int32_t batch, double tau, int32_t* idx_out, int32_t idx_stride,
                        int32_t* cnt_out, void* hip_stream);

/* ---- decode state save / load ------------------------------------------- */

/* A decode can move to another handle (another process, another device)
 * between steps: the blob holds the step count and phase, the focal set and
 * ratios, the kept set carried to the next step (Cross-Step Fixation Reuse),
 * the current warm-up window's statistics, and the status flags.  It does
 * not hold the KV cache, which stays the caller's. */

/* fastocr_state_bytes: size in bytes of this handle's state blob. */
int fastocr_state_bytes(fastocr_handle* h, int64_t* bytes);

/* fastocr_save_state: at a step boundary (no layer of the current step
 * called yet), write the handle's decode state to host_buf (host memory of
 * at least fastocr_state_bytes bytes).  Synchronises the stream.  Errors:
 * INVALID_ARG (null, buffer too small), STATE (mid-step, poisoned handle),
 * HIP. */
int fastocr_save_state(fastocr_handle* h, void* host_buf, int64_t bytes);

/* fastocr_load_state: replace the decode state of a handle at a step
 * boundary with a blob from fastocr_save_state of a handle created with the
 * same configuration; the next fastocr_attend continues that decode exactly.
 * Synchronises the stream.  Errors: INVALID_ARG (null, short buffer, not a
 * blob of this configuration, inconsistent contents), STATE (mid-step,
 * poisoned handle), HIP. */
int fastocr_load_state(fastocr_handle* h, const void* host_buf, int64_t bytes);

/* ---- multi-span image layouts -------------------------------------------- */

/* The library's kernels take every sequence's image tokens as cache rows
 * [0, n_img_b).  A document whose image sits elsewhere in the cache (behind
 * a text prefix, or as several pages or images with text between them) is
 * brought into that layout once, after prefill, by a row permutation of each
 * layer's cache: softmax attention does not depend on the order of the keys
 * (positions are already encoded in the keys and values), so every output
 * of the method is unchanged (Method: only the set of attended tokens
 * changes).  Image token j of the method is then the j-th image row in
 * ascending row order, and the kept set is chosen over the tokens of all
 * spans together.  Rows decoded later are appended at row len_b - 1 as
 * before (the permutation leaves rows at and after the last prefill row in
 * place). */

/* fastocr_image_first_map: the permutation for one sequence.  spans: host
 * int32 [num_spans, 2] of (first row, row count), ascending and disjoint,
 * inside [0, rows).  map_out: host int32 [rows] receives the source row of
 * every destination row: the image rows in ascending order, then every other
 * row in ascending order.  Returns n_img (the summed counts), or
 * FASTOCR_ERR_INVALID_ARG for unsorted, overlapping or out-of-range spans. */
int32_t fastocr_image_first_map(const int32_t* spans, int32_t num_spans, int32_t rows, int32_t* map_out);

/* fastocr_pack_rows: dst[b, h, i, :] = src[b, h, row_map[b * S + i], :] for
 * every KV head h and i < rows_b.  src, dst: device [B, Hkv, S, head_dim] of
 * dtype, 16-byte aligned, not overlapping (INVALID_ARG otherwise); row_map:
 * device int32 [B, S]; rows: device int32 [B] (clamped to [0, S]); rows of
 * dst at or past rows_b are not written.  A map entry outside [0, S) is
 * clamped and, when status (device int32, may be NULL) is given, latches
 * FASTOCR_FLAG_INDEX_CLAMPED there.  hip_stream: hipStream_t.  Asynchronous.
 * Errors: INVALID_ARG, HIP. */
int fastocr_pack_rows(const void* src, void* dst, const int32_t* row_map, const int32_t* rows,
                      int32_t batch, int32_t num_kv_heads, int32_t max_seq_len, int32_t head_dim,
                      int32_t dtype, int32_t* status, void* hip_stream);

/* ---- measurement --------------------------------------------------------- */

/* fastocr_probe_read: stream `bytes` (a positive multiple of 16) of device
 * memory at buf (16-byte aligned) through the vector memory path with
 * `workgroups` workgroups of 256 threads, each thread folding what it reads
 * into one word; sink: device uint32 [64], written only if a fold hits a
 * sentinel value (not in practice).  Reads only; used to measure the HBM read
 * rate and the per-launch cost of reads the size of a kept-token pass.
 * hip_stream: hipStream_t.  Asynchronous.  Errors: INVALID_ARG, HIP. */
int fastocr_probe_read(const void* buf, int64_t bytes, int32_t workgroups, uint32_t* sink, void* hip_stream);

/* Host helpers (no device use). */
/* k = clamp(ceil(tau*n - 1e-9), 1, n) for n > 0; 0 for n <= 0; negative
 * FASTOCR_ERR_INVALID_ARG if tau is outside (0, 1]. */
int32_t fastocr_kept_count(double tau, int32_t n_img);

/* Focal layers from per-layer ratios (host double [num_layers]): the
 * num_focal largest, ties to the lower layer, ascending into out (host int32
 * [num_focal]). */
int fastocr_choose_focal_layers(const double* ratios, int32_t num_layers, int32_t num_focal,
                                int32_t* out);

/* Static text for a status code. */
const char* fastocr_error_string(int32_t code);

#ifdef __cplusplus
}
#endif

#endif /* FASTOCR_H */
