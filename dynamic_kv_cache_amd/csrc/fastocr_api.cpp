// Host runtime of the FastOCR decode-step attention library: handle, scratch
// arena, per-step/per-layer state machine, warm-up profiler finalisation and
// kernel dispatch.  The C ABI is declared in include/fastocr.h.
//
// Method source: "FastOCR: Dynamic Visual Fixation via KV Cache Pruning for
// Efficient Document Parsing", technical summary, Method / 1. Focal-Guided
// Pruning (Focal Layer Selection, Cross-Layer Propagation) and 2. Cross-Step
// Fixation Reuse (Implementation).

#include <dlfcn.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <numeric>
#include <vector>

#include "../../include/fastocr.h"
#include "internal.h"

using namespace fastocr;

namespace {

enum Phase : int { PHASE_WARMUP = 0, PHASE_WARMUP_DONE = 1, PHASE_PRUNED = 2, PHASE_FULL = 3 };

// Optional named ranges for profiler traces (FASTOCR_TRACE=1): the roctx
// library is opened at run time, so the library itself does not depend on it.
struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

Roctx open_roctx() {
  Roctx r;
  for (const char* name : {"librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so", "libroctx64.so.4"}) {
    void* lib = dlopen(name, RTLD_NOW | RTLD_LOCAL);
    if (!lib) continue;
    r.push = reinterpret_cast<int (*)(const char*)>(dlsym(lib, "roctxRangePushA"));
    r.pop = reinterpret_cast<int (*)()>(dlsym(lib, "roctxRangePop"));
    if (r.push && r.pop) return r;
    r = Roctx{};
  }
  return r;
}

// One named range for the lifetime of the object (no-op without roctx).
struct TraceRange {
  const Roctx* r;
  TraceRange(const Roctx* roctx, const char* msg) : r(roctx && roctx->push ? roctx : nullptr) {
    if (r) r->push(msg);
  }
  ~TraceRange() {
    if (r) r->pop();
  }
};

struct TimedLaunch {
  int cls;
  hipEvent_t end;  // recorded by the dispatch itself when the kernel completes
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

// Rows per split for a pass that visits at most `rows` rows per (sequence,
// KV head): whole rounds (kRowsPerRound rows, one tile group per wave),
// the fewest that still give about `target` workgroups, so a small batch
// spreads over many CUs (one CU streams only ~60 GB/s) and a large one
// reads long runs per workgroup.  At most max_splits splits.
int plan_rows_per_split(int64_t pairs, int rows, int target, int max_splits, const char* env) {
  int R = env_int(env, 0);
  if (R <= 0) {
    const int64_t want = (pairs * (int64_t)std::max(rows, 1) + target - 1) / target;
    R = (int)align_up((size_t)std::max<int64_t>(want, 1), kRowsPerRound);
  } else {
    R = (int)align_up((size_t)R, kTileRows);
  }
  while ((rows + R - 1) / R > max_splits) R += kRowsPerRound;
  return R;
}

// Launch geometry and scratch layout of a handle: a function of its
// configuration, the device's compute-unit count and the FASTOCR_*
// environment overrides alone (no device use).
struct Plan {
  int n_cap = 0, n_stride = 0, k_max = 0;
  int full_R = 0, full_splits = 0, full_sure = 0;  // sure: splits that hold rows for any accepted sequence
  int sparse_R = 0, sparse_splits = 0;  // kept-token pass: rows per workgroup at the longest
                                        // text the handle accepts, workgroups per pair
  bool keeps_all = false;        // tau = 1: non-focal layers run the full pass
  bool valu_full = false;        // full passes run the VALU variant (measurement override)
  bool skip_dead_picks = true;   // a focal layer followed by a focal layer picks nothing
  bool focal_staged = false;     // focal passes stage a split's logits in LDS
  bool stream_rows = false;      // pruned steps' kept-token and focal-layer passes stream their rows
  int max_splits = 0;            // merge states per head the scratch holds
  // scratch arena: byte offsets of each array, and the total
  size_t o_pstat = 0, o_po = 0, o_logits = 0, o_mz = 0, o_scores = 0, o_warm = 0, o_tm = 0, o_sel = 0,
         o_cnt = 0, o_status = 0, o_lens = 0, o_hist0 = 0, arena_bytes = 0;
};

bool config_ok(const fastocr_config& c);
int32_t kept_count_host(double tau, int32_t n_img);

// FASTOCR_OK, or FASTOCR_ERR_INVALID_ARG for a configuration whose launches
// cannot be planned.
int make_plan(const fastocr_config& c, int num_cu, Plan& p) {
  if (!config_ok(c) || num_cu < 1) return FASTOCR_ERR_INVALID_ARG;
  const int G = c.num_q_heads / c.num_kv_heads;
  p = Plan{};
  p.n_cap = c.max_img_tokens;
  p.n_stride = (int)align_up((size_t)std::max(c.max_img_tokens, 1), 4);
  p.k_max = std::max(kept_count_host(c.tau, c.max_img_tokens), 1);
  const int64_t pairs = (int64_t)c.batch * c.num_kv_heads;
  // about one wave of resident split workgroups per launch
  // A ragged batch (image counts between min_img_tokens and max_img_tokens)
  // is planned for the middle of that range, not for the longest sequence,
  // whose plan would leave most splits of the shorter sequences empty and
  // fill few CUs; each pair's last split is partly empty, so the plan keeps
  // half a workgroup per pair of the resident slots free (a launch just
  // over the slots runs a second wave).  7B-like B=16, 2169-6682 image
  // tokens, full step: 768-row splits (440 workgroups with rows) 1067 us,
  // 640 (516) 1247, 1024 (336) 1178, 1152 (304) 1224.
  int full_rows_est = c.max_seq_len;
  int full_target = kFullBlocksPerCU * num_cu;
  if (c.min_img_tokens > 0 && c.min_img_tokens < c.max_img_tokens) {
    full_rows_est = (c.min_img_tokens + c.max_img_tokens) / 2 + (c.max_seq_len - c.max_img_tokens);
    full_target = (int)std::max<int64_t>(full_target - pairs / 2, full_target / 2);
  }
  p.full_R = plan_rows_per_split(pairs, full_rows_est, full_target, kMaxMergeSplits, "FASTOCR_FULL_ROWS");
  while ((c.max_seq_len + p.full_R - 1) / p.full_R > kMaxMergeSplits) p.full_R += kRowsPerRound;
  p.full_splits = (c.max_seq_len + p.full_R - 1) / p.full_R;
  // rows of a kept-token pass at the longest text the handle accepts: kept
  // image rows + text rows
  int sparse_rows = c.max_seq_len;
  if (c.min_img_tokens > 0)
    sparse_rows = std::min(sparse_rows, p.k_max + c.max_seq_len - c.min_img_tokens);
  if (c.max_text_tokens > 0) sparse_rows = std::min(sparse_rows, p.k_max + c.max_text_tokens);
  const bool pruned = c.mode == FASTOCR_MODE_PRUNED;
  // Kept-token passes deal each pair's 16-row tiles round-robin to P
  // workgroups, as many as fill one wave of resident workgroups over all
  // pairs (a launch past one wave runs a second, mostly idle one: 72B-like
  // B=8, P = 12 (768 workgroups) 16.9 us against P = 16 19.6 us; 32B-like
  // B=4, P = 24 14.1 us against P = 25 16.4 us), but no more than the
  // pair's tiles at the longest text and at most kMaxKeptSplits (7B-like
  // B=1: P = 22-44 5.4 us, 64 5.5 us, 11 5.9 us).  FASTOCR_SPARSE_ROWS=R sets
  // P for R rows per workgroup at that length instead.
  if (pruned) {
    const int64_t slots = (int64_t)kKeptBlocksPerCU * num_cu;
    int P = (int)std::min<int64_t>(std::max<int64_t>(slots / pairs, 1), (sparse_rows + kTileRows - 1) / kTileRows);
    const int R_env = env_int("FASTOCR_SPARSE_ROWS", 0);
    if (R_env > 0) P = (sparse_rows + R_env - 1) / R_env;
    P = std::min(std::max(P, 1), kMaxKeptSplits);
    p.sparse_splits = P;
    p.sparse_R = (int)align_up((size_t)((sparse_rows + P - 1) / P), kTileRows);
    // In pruned steps the kept-token passes and the focal layers' passes load
    // their K/V rows non-temporally when the kept rows of one step's
    // non-focal layers (at the longest text) exceed the last-level cache: the
    // next step would not find them there anyway, and streaming keeps the
    // kept indices, the merge states and the focal logits cached.  Measured per step, streamed kept-token rows against
    // plain: 72B-like B=8 2115 against 2173-2178 us, 32B-like B=4 1396
    // against 1434, 7B-like B=16 500-501 against 505-506, but 7B-like B=1
    // (69 MB of kept rows a step) 259.3 against 257.6-258.3, where plain
    // loads find the previous step's rows in that cache; streamed focal-layer
    // rows on top, with the cache scrubbed before every step: 72B-like
    // 2053-2057 against 2083-2084 us for the focal passes (84.8 against 91.7
    // us each), 2020-2023 with the full passes of focal layers whose pick is
    // unused too; the others unchanged.  FASTOCR_STREAM_ROWS=0|1 overrides.
    const int64_t row_bytes = 2 * (int64_t)c.head_dim * (c.dtype == FASTOCR_DTYPE_BF16 ? 2 : 4);
    const int64_t step_bytes = (int64_t)(c.num_layers - c.num_focal) * pairs * sparse_rows * row_bytes;
    const int stream_env = env_int("FASTOCR_STREAM_ROWS", -1);
    p.stream_rows = stream_env < 0 ? step_bytes > kLastLevelCacheBytes : stream_env != 0;
  }
  p.skip_dead_picks = env_int("FASTOCR_SKIP_DEAD_PICKS", 1) != 0;
  // A focal pass with long splits keeps a split's image-token logits in LDS
  // and writes each head's run once the split's rows are done, when they fit.
  // Measured per focal pass, staged against stored as computed: 72B-like B=8
  // (1920-row splits) 91.2 us against 100.9 (82.9 with no export at all);
  // 32B-like B=4 (1408) 62.9 against 67.2; 7B-like B=16 (1152) 39.2 against
  // 41.1; but 7B-like B=1 (128-row splits, one round) 7.9 against 6.7, where
  // the write-out only lengthens the tail.  FASTOCR_FOCAL_STAGE=0 never
  // stages, =1 stages whenever the logits fit.
  const bool stage_fits = (int64_t)G * (p.full_R + kLogitStagePad) <= kLogitStageFloats;
  const int stage_env = env_int("FASTOCR_FOCAL_STAGE", -1);
  p.focal_staged = stage_fits && (stage_env < 0 ? p.full_R >= kLogitStageMinRows : stage_env != 0);
  // FASTOCR_VALU_FULL=1: full passes without MFMA (bf16, head_dim 128, groups
  // of at most kValuMaxGroup heads), to measure what the matrix cores buy
  p.valu_full = env_int("FASTOCR_VALU_FULL", 0) != 0 && c.dtype == FASTOCR_DTYPE_BF16 && c.head_dim == 128 &&
                G <= kValuMaxGroup;
  // k_b = n_b for every n_b exactly when tau = 1
  p.keeps_all = c.tau >= 1.0 && env_int("FASTOCR_KEPT_ALL_AS_FULL", 1) != 0;
  // state slots per head; the merge keeps one weight per state in LDS
  p.max_splits = std::max(p.full_splits, p.sparse_splits);
  if (p.max_splits > kMaxMergeSplits) return FASTOCR_ERR_INVALID_ARG;
  // Full passes: every sequence has at least min_img_tokens image rows and
  // the current token, so splits below that hold rows and load their K/V
  // ahead; the others (possibly empty for a short sequence of a ragged
  // batch) wait for the extent.
  const int min_full_rows = c.min_img_tokens + 1;
  p.full_sure = std::min((min_full_rows + p.full_R - 1) / p.full_R, p.full_splits);

  // scratch arena
  const size_t B = c.batch, Hq = c.num_q_heads, L = c.num_layers, D = c.head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  p.o_pstat = take(B * Hq * p.max_splits * sizeof(float4));
  p.o_po = take(B * Hq * p.max_splits * D * sizeof(float));
  p.o_logits = take(pruned ? B * Hq * p.n_stride * sizeof(float) : 0);
  p.o_mz = take(B * Hq * sizeof(float2));
  p.o_scores = take(pruned ? B * p.n_stride * sizeof(float) : 0);
  p.o_warm = take(pruned ? L * B * p.n_stride * sizeof(float) : 0);
  p.o_tm = take(pruned ? L * (size_t)c.warmup_steps * B * Hq * sizeof(float) : 0);
  p.o_sel = take(B * p.k_max * sizeof(int32_t));
  p.o_cnt = take(B * sizeof(int32_t));
  p.o_status = take(sizeof(int32_t));
  p.o_lens = take(B * 2 * sizeof(int32_t));
  p.o_hist0 = take(pruned ? B * 256 * sizeof(unsigned int) : 0);
  p.arena_bytes = off;
  return FASTOCR_OK;
}

}  // namespace

struct fastocr_handle {
  fastocr_config cfg{};
  hipStream_t stream = nullptr;
  int device = 0;
  int G = 0, D = 0, n_cap = 0, n_stride = 0, k_max = 0;
  int full_R = 0, full_splits = 0, sparse_R = 0, sparse_splits = 0, max_splits = 0;
  int full_sure = 0;                   // full-pass splits that hold rows for any accepted sequence
  bool keeps_all = false;              // tau = 1: non-focal layers run the full pass
  bool valu_full = false;              // full passes run the VALU variant (measurement override)
  bool skip_dead_picks = true;         // a focal layer followed by a focal layer picks nothing
  bool focal_staged = false;           // focal passes stage a split's logits in LDS
  bool stream_rows = false;            // pruned steps' kept-token and focal-layer passes stream their rows
  Roctx roctx;                         // FASTOCR_TRACE=1: a named range per call
  const void* app_k = nullptr;         // fastocr_attend_append: the current token's K/V
  const void* app_v = nullptr;

  float scale_log2 = 0.f;

  int step = 0, next_layer = 0, phase = PHASE_WARMUP;
  int warm_pos = 0;       // step index inside the current warm-up window
  int pruned_since = 0;   // pruned steps since the last profile
  int profiles = 0;       // completed profiles (first warm-up and re-selections)
  bool poisoned = false;
  std::vector<int32_t> focal;
  std::vector<char> is_focal;
  std::vector<double> ratios;

  void* arena = nullptr;
  size_t arena_bytes = 0;
  bool owns_arena = true;              // false: placed by the caller (fastocr_create_static)
  void (*on_destroy)(int device) = nullptr;
  float4* pstat = nullptr;
  float* po = nullptr;
  float* logits = nullptr;
  float2* mz = nullptr;
  float* scores = nullptr;
  float* warm_scores = nullptr;
  float* text_mass = nullptr;
  int32_t* sel = nullptr;
  int32_t* sel_cnt = nullptr;
  unsigned int* hist0 = nullptr;  // [B, 256] first-digit histograms, merge -> top-k, zero in between
  int32_t* status = nullptr;
  int32_t* lens_shadow = nullptr;  // [B, 2] lens of the last warm-up step

  bool timing = false;
  std::vector<TimedLaunch> events;
  size_t ev_used = 0;
  fastocr_timing timing_acc{};
};

namespace {

int fail_hip(fastocr_handle* h, hipError_t e) {
  if (e == hipSuccess) return FASTOCR_OK;
  if (h) h->poisoned = true;
  return FASTOCR_ERR_HIP;
}

// Launch helper: with timing on, the dispatch itself records an event when
// the kernel completes (no marker packet is queued).
template <typename F>
int timed(fastocr_handle* h, int cls, F&& launch) {
  LaunchTiming lt;
  if (h->timing) {
    if (h->ev_used == h->events.size()) {
      // timing-only event: no system-scope fence (cache write-back) on record
      TimedLaunch nl{cls, nullptr};
      if (hipEventCreateWithFlags(&nl.end, hipEventDisableSystemFence) != hipSuccess)
        return fail_hip(h, hipErrorOutOfMemory);
      h->events.push_back(nl);
    }
    TimedLaunch& tl = h->events[h->ev_used++];
    tl.cls = cls;
    lt.stop = tl.end;
  }
  return fail_hip(h, launch(lt));
}

SplitParams split_params(fastocr_handle* h, const void* q, const void* k, const void* v,
                         const int32_t* lens, void* out, bool sparse) {
  SplitParams p{};
  p.out = out;
  p.q = q;
  p.k = k;
  p.v = v;
  if (h->app_k) {  // fastocr_attend_append: the caches are the caller's writable buffers
    p.k_new = h->app_k;
    p.v_new = h->app_v;
    p.k_w = const_cast<void*>(k);
    p.v_w = const_cast<void*>(v);
  }
  p.lens = lens;
  p.sel = h->sel;
  p.sel_cnt = h->sel_cnt;
  p.logits = h->logits;
  p.pstat = h->pstat;
  p.po = h->po;
  p.status = h->status;
  p.B = h->cfg.batch;
  p.Hq = h->cfg.num_q_heads;
  p.Hkv = h->cfg.num_kv_heads;
  p.S = h->cfg.max_seq_len;
  p.n_cap = h->n_cap;
  p.n_stride = h->n_stride;
  p.k_stride = h->k_max;
  p.max_splits = h->max_splits;
  p.rows_per_split = sparse ? h->sparse_R : h->full_R;
  p.grid_splits = sparse ? h->sparse_splits : h->full_splits;
  p.sure_splits = sparse ? 0 : h->full_sure;
  p.stream_rows = (sparse && h->stream_rows) ? 1 : 0;  // (full passes: set by run_full)
  p.scale_log2 = h->scale_log2;
  return p;
}

int run_topk(fastocr_handle* h, const float* scores, const int32_t* lens, unsigned int* hist0) {
  TopkParams t{};
  t.hist0 = hist0;
  t.scores = scores;
  t.score_stride = h->n_stride;
  t.n_cap = h->n_cap;
  t.lens = lens;
  t.B = h->cfg.batch;
  t.tau = h->cfg.tau;
  t.idx = h->sel;
  t.idx_stride = h->k_max;
  t.cnt = h->sel_cnt;
  t.status = h->status;
  return timed(h, FASTOCR_KC_TOPK, [&](const LaunchTiming& lt) { return launch_topk(t, h->stream, lt); });
}

MergeParams merge_params(fastocr_handle* h, const int32_t* lens, void* out, bool sparse) {
  const fastocr_config& c = h->cfg;
  MergeParams m{};
  m.pstat = h->pstat;
  m.po = h->po;
  m.lens = lens;
  m.out = out;
  m.B = c.batch;
  m.Hq = c.num_q_heads;
  m.Hkv = c.num_kv_heads;
  m.n_cap = h->n_cap;
  m.max_splits = h->max_splits;
  m.grid_splits = sparse ? h->sparse_splits : h->full_splits;  // states per head
  m.n_stride = h->n_stride;
  return m;
}

// Full attention of one layer: split pass, then the merge (and optionally
// each head's text mass and, with `scores_dst`, the image-token scores),
// then with `topk` the selection of the kept set from those scores.  With
// `stream` the split pass loads its rows non-temporally.
int run_full(fastocr_handle* h, const void* q, const void* k, const void* v, const int32_t* lens,
             void* out, float* text_mass_dst, float* scores_dst, bool topk, bool stream) {
  const fastocr_config& c = h->cfg;
  const bool focal = scores_dst != nullptr;
  SplitParams sp = split_params(h, q, k, v, lens, out, false);
  sp.stream_rows = stream ? 1 : 0;
  sp.valu = (h->valu_full && !focal && !h->app_k) ? 1 : 0;
  sp.stage_logits = (focal && h->focal_staged) ? 1 : 0;
  int rc = timed(h, focal ? FASTOCR_KC_FOCAL_SPLIT : FASTOCR_KC_FULL_SPLIT, [&](const LaunchTiming& lt) {
    return launch_split(c.dtype, c.head_dim, focal ? KIND_FOCAL : KIND_FULL, sp, h->stream, lt);
  });
  if (rc) return rc;
  MergeParams mp = merge_params(h, lens, out, false);
  mp.text_mass = text_mass_dst;
  if (focal) {
    mp.logits = h->logits;
    mp.scores = scores_dst;
    mp.score_blocks = (h->n_stride + kMergeThreads - 1) / kMergeThreads;
    if (topk) mp.hist0 = h->hist0;  // the top-k below reads and clears it
  }
  rc = timed(h, FASTOCR_KC_MERGE,
             [&](const LaunchTiming& lt) { return launch_merge(c.dtype, c.head_dim, mp, h->stream, lt); });
  if (rc || !topk) return rc;
  return run_topk(h, scores_dst, lens, h->hist0);
}

// Non-focal layer: attention over the kept image rows and every text row.
// When every sequence fits one split the split kernel writes the outputs;
// otherwise every launched split writes a state and the merge combines them.
int run_sparse(fastocr_handle* h, const void* q, const void* k, const void* v, const int32_t* lens,
               void* out) {
  const fastocr_config& c = h->cfg;
  SplitParams sp = split_params(h, q, k, v, lens, out, true);
  int rc = timed(h, FASTOCR_KC_SPARSE_SPLIT, [&](const LaunchTiming& lt) {
    return launch_kept(c.dtype, c.head_dim, sp, h->stream, lt);
  });
  if (rc || h->sparse_splits <= 1) return rc;
  MergeParams mp = merge_params(h, lens, out, true);
  return timed(h, FASTOCR_KC_MERGE,
               [&](const LaunchTiming& lt) { return launch_kept_merge(c.dtype, c.head_dim, mp, h->stream, lt); });
}

void select_focal(const double* ratios, int L, int num_focal, int32_t* out) {
  std::vector<int> idx(L);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int a, int b) { return ratios[a] > ratios[b]; });
  std::vector<int> pick(idx.begin(), idx.begin() + num_focal);
  std::sort(pick.begin(), pick.end());
  for (int i = 0; i < num_focal; ++i) out[i] = pick[i];
}

// k = clamp(ceil(tau*n - 1e-9), 1, n) for n > 0 (tau in (0, 1]); each
// operation rounded on its own, as the device computes it.
int32_t kept_count_host(double tau, int32_t n_img) {
#pragma clang fp contract(off)
  if (n_img <= 0) return 0;
  const double prod = tau * (double)n_img;
  const double k = std::ceil(prod - 1e-9);
  int32_t ki = (int32_t)k;
  return std::min(std::max(ki, 1), n_img);
}

bool config_ok(const fastocr_config& c) {
  if (c.num_layers < 1 || c.num_kv_heads < 1 || c.num_q_heads < 1 || c.batch < 1) return false;
  if (c.num_q_heads % c.num_kv_heads != 0) return false;
  if ((int64_t)c.batch * c.num_kv_heads > 65535) return false;  // one grid dimension
  if (c.num_q_heads / c.num_kv_heads > 16 || c.num_q_heads > 128) return false;
  if (c.head_dim != 64 && c.head_dim != 128) return false;
  if (c.max_seq_len < 1) return false;
  if (c.max_img_tokens < 0 || c.max_img_tokens > c.max_seq_len) return false;
  if (c.min_img_tokens < 0 || c.min_img_tokens > c.max_img_tokens) return false;
  if (c.max_text_tokens < 0 || c.max_text_tokens > c.max_seq_len) return false;
  if (c.dtype != FASTOCR_DTYPE_F32 && c.dtype != FASTOCR_DTYPE_BF16) return false;
  if (c.mode != FASTOCR_MODE_PRUNED && c.mode != FASTOCR_MODE_FULL) return false;
  if (!(c.tau > 0.0 && c.tau <= 1.0)) return false;
  if (!(c.sm_scale >= 0.f) || !std::isfinite(c.sm_scale)) return false;
  if (c.mode == FASTOCR_MODE_PRUNED) {
    if (c.num_focal < 1 || c.num_focal > c.num_layers) return false;
    if (c.warmup_steps < 1) return false;
  }
  if (c.reprofile_every < 0) return false;
  // every cache index must fit comfortably in 64-bit byte offsets
  const double cache_elems = (double)c.batch * c.num_kv_heads * c.max_seq_len * c.head_dim;
  if (cache_elems > 4.0e15) return false;
  return true;
}

}  // namespace

// ---- decode state save / load --------------------------------------------

namespace {

constexpr uint32_t kStateMagic = 0x52434f46u;  // "FOCR"
constexpr uint32_t kStateVersion = 1;

// Everything a later step depends on, at a step boundary: the host state
// machine and the device arrays that persist across steps (kept set and
// counts, the warm-up window's statistics, the lens copy of its last step,
// the status word).  The configuration fields identify the handles a blob
// fits.
struct StateHeader {
  uint32_t magic, version;
  int32_t L, Hq, Hkv, D, B, S, n_cap, n_stride, k_max, w, num_focal, mode, dtype, reprofile_every;
  double tau;
  int32_t step, phase, warm_pos, pruned_since, profiles, n_focal, n_ratios, pad;
};

struct StateArray {
  void* dev;
  size_t bytes;
};

std::vector<StateArray> state_arrays(fastocr_handle* h) {
  const fastocr_config& c = h->cfg;
  const size_t B = c.batch, Hq = c.num_q_heads, L = c.num_layers;
  const bool pruned = c.mode == FASTOCR_MODE_PRUNED;
  return {
      {h->sel, B * h->k_max * sizeof(int32_t)},
      {h->sel_cnt, B * sizeof(int32_t)},
      {h->text_mass, pruned ? L * (size_t)c.warmup_steps * B * Hq * sizeof(float) : 0},
      {h->warm_scores, pruned ? L * B * h->n_stride * sizeof(float) : 0},
      {h->lens_shadow, B * 2 * sizeof(int32_t)},
      {h->status, sizeof(int32_t)},
  };
}

size_t state_bytes(fastocr_handle* h) {
  size_t n = sizeof(StateHeader) + (size_t)h->cfg.num_layers * (sizeof(int32_t) + sizeof(double));
  for (const StateArray& a : state_arrays(h)) n += a.bytes;
  return n;
}

StateHeader state_header(fastocr_handle* h) {
  const fastocr_config& c = h->cfg;
  StateHeader s{};
  s.magic = kStateMagic;
  s.version = kStateVersion;
  s.L = c.num_layers;
  s.Hq = c.num_q_heads;
  s.Hkv = c.num_kv_heads;
  s.D = c.head_dim;
  s.B = c.batch;
  s.S = c.max_seq_len;
  s.n_cap = h->n_cap;
  s.n_stride = h->n_stride;
  s.k_max = h->k_max;
  s.w = c.warmup_steps;
  s.num_focal = c.num_focal;
  s.mode = c.mode;
  s.dtype = c.dtype;
  s.reprofile_every = c.reprofile_every;
  s.tau = c.tau;
  s.step = h->step;
  s.phase = h->phase;
  s.warm_pos = h->warm_pos;
  s.pruned_since = h->pruned_since;
  s.profiles = h->profiles;
  s.n_focal = (int32_t)h->focal.size();
  s.n_ratios = (int32_t)h->ratios.size();
  return s;
}

}  // namespace

extern "C" {

int32_t fastocr_kept_count(double tau, int32_t n_img) {
  if (!(tau > 0.0 && tau <= 1.0)) return FASTOCR_ERR_INVALID_ARG;
  return kept_count_host(tau, n_img);
}

int fastocr_choose_focal_layers(const double* ratios, int32_t num_layers, int32_t num_focal,
                                int32_t* out) {
  if (!ratios || !out || num_layers < 1 || num_focal < 1 || num_focal > num_layers)
    return FASTOCR_ERR_INVALID_ARG;
  select_focal(ratios, num_layers, num_focal, out);
  return FASTOCR_OK;
}

const char* fastocr_error_string(int32_t code) {
  switch (code) {
    case FASTOCR_OK: return "ok";
    case FASTOCR_ERR_INVALID_ARG: return "invalid argument";
    case FASTOCR_ERR_STATE: return "call out of order for the handle state";
    case FASTOCR_ERR_HIP: return "HIP runtime error";
    case FASTOCR_ERR_OOM: return "device allocation failed";
    case FASTOCR_ERR_SCRATCH: return "configuration needs more scratch than the static array holds";
    default: return "unknown status";
  }
}

int fastocr_create(const fastocr_config* cfg, void* hip_stream, fastocr_handle** out) {
  return fastocr::create_handle(cfg, hip_stream, out, nullptr, 0, nullptr);
}

}  // extern "C"

// fastocr_create, with the scratch arena either allocated here (arena null)
// or placed at `arena` (device memory of arena_cap bytes that the caller
// keeps; `on_destroy(device)` is called when the handle is destroyed).
int fastocr::create_handle(const fastocr_config* cfg, void* hip_stream, fastocr_handle** out, void* arena,
                           size_t arena_cap, void (*on_destroy)(int)) {
  if (!cfg || !out) return FASTOCR_ERR_INVALID_ARG;
  *out = nullptr;
  if (!config_ok(*cfg)) return FASTOCR_ERR_INVALID_ARG;

  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) return FASTOCR_ERR_HIP;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FASTOCR_ERR_HIP;
  int num_cu = 256;
  {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess && prop.multiProcessorCount > 0)
      num_cu = prop.multiProcessorCount;
  }

  Plan plan;
  if (make_plan(*cfg, num_cu, plan) != FASTOCR_OK) return FASTOCR_ERR_INVALID_ARG;
  fastocr_handle* h = new (std::nothrow) fastocr_handle();
  if (!h) return FASTOCR_ERR_OOM;
  h->cfg = *cfg;
  h->stream = reinterpret_cast<hipStream_t>(hip_stream);
  h->device = dev;
  const fastocr_config& c = h->cfg;
  h->G = c.num_q_heads / c.num_kv_heads;
  h->D = c.head_dim;
  h->n_cap = plan.n_cap;
  h->n_stride = plan.n_stride;
  h->k_max = plan.k_max;
  const float scale = c.sm_scale > 0.f ? c.sm_scale : 1.0f / std::sqrt((float)c.head_dim);
  h->scale_log2 = scale * 1.4426950408889634f;
  h->phase = c.mode == FASTOCR_MODE_FULL ? PHASE_FULL : PHASE_WARMUP;
  h->full_R = plan.full_R;
  h->full_splits = plan.full_splits;
  h->full_sure = plan.full_sure;
  h->sparse_R = plan.sparse_R;
  h->sparse_splits = plan.sparse_splits;
  h->keeps_all = plan.keeps_all;
  h->valu_full = plan.valu_full;
  h->skip_dead_picks = plan.skip_dead_picks;
  h->focal_staged = plan.focal_staged;
  h->stream_rows = plan.stream_rows;
  h->max_splits = plan.max_splits;
  if (env_int("FASTOCR_TRACE", 0) != 0) h->roctx = open_roctx();
  const bool pruned = c.mode == FASTOCR_MODE_PRUNED;
  const size_t o_pstat = plan.o_pstat, o_po = plan.o_po, o_logits = plan.o_logits, o_mz = plan.o_mz,
               o_scores = plan.o_scores, o_warm = plan.o_warm, o_tm = plan.o_tm, o_sel = plan.o_sel,
               o_cnt = plan.o_cnt, o_status = plan.o_status, o_lens = plan.o_lens, o_hist0 = plan.o_hist0;
  h->arena_bytes = plan.arena_bytes;
  hipError_t e = hipSuccess;
  if (arena) {
    if (h->arena_bytes > arena_cap) {
      delete h;
      return FASTOCR_ERR_SCRATCH;
    }
    h->arena = arena;
    h->owns_arena = false;
    h->on_destroy = on_destroy;
  } else {
    e = hipMalloc(&h->arena, h->arena_bytes);
    if (e != hipSuccess) {
      delete h;
      return e == hipErrorOutOfMemory ? FASTOCR_ERR_OOM : FASTOCR_ERR_HIP;
    }
  }
  char* base = static_cast<char*>(h->arena);
  h->pstat = reinterpret_cast<float4*>(base + o_pstat);
  h->po = reinterpret_cast<float*>(base + o_po);
  h->logits = pruned ? reinterpret_cast<float*>(base + o_logits) : nullptr;
  h->mz = reinterpret_cast<float2*>(base + o_mz);
  h->scores = pruned ? reinterpret_cast<float*>(base + o_scores) : nullptr;
  h->warm_scores = pruned ? reinterpret_cast<float*>(base + o_warm) : nullptr;
  h->text_mass = pruned ? reinterpret_cast<float*>(base + o_tm) : nullptr;
  h->sel = reinterpret_cast<int32_t*>(base + o_sel);
  h->sel_cnt = reinterpret_cast<int32_t*>(base + o_cnt);
  h->status = reinterpret_cast<int32_t*>(base + o_status);
  h->lens_shadow = reinterpret_cast<int32_t*>(base + o_lens);
  h->hist0 = pruned ? reinterpret_cast<unsigned int*>(base + o_hist0) : nullptr;
  e = hipMemsetAsync(h->arena, 0, h->arena_bytes, h->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) {
    if (h->owns_arena) (void)hipFree(h->arena);
    delete h;
    return FASTOCR_ERR_HIP;
  }
  h->is_focal.assign(c.num_layers, 0);
  *out = h;
  return FASTOCR_OK;
}

extern "C" {

// Focal Layer Selection at the end of a warm-up window (the first one, or a
// periodic re-selection window): synchronises the stream.
static int profile_impl(fastocr_handle* h) {
  TraceRange range(&h->roctx, "fastocr profile");
  const fastocr_config& c = h->cfg;
  const size_t BH = (size_t)c.batch * c.num_q_heads;
  const size_t per_layer = (size_t)c.warmup_steps * BH;
  std::vector<float> tm((size_t)c.num_layers * per_layer);
  hipError_t e = hipStreamSynchronize(h->stream);
  if (e == hipSuccess)
    e = hipMemcpy(tm.data(), h->text_mass, tm.size() * sizeof(float), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail_hip(h, e);
  // Image-attention ratio of a layer: mean over the window's steps, sequences
  // and heads of the image probability mass, 1 - text mass (Focal Layer
  // Selection).
  h->ratios.assign(c.num_layers, 0.0);
  for (int l = 0; l < c.num_layers; ++l) {
    double s = 0.0;
    for (size_t i = 0; i < per_layer; ++i) s += 1.0 - (double)tm[l * per_layer + i];
    h->ratios[l] = s / (double)per_layer;
  }
  h->focal.assign(c.num_focal, 0);
  select_focal(h->ratios.data(), c.num_layers, c.num_focal, h->focal.data());
  h->is_focal.assign(c.num_layers, 0);
  for (int32_t l : h->focal) h->is_focal[l] = 1;
  // The first pruned step inherits the set picked from the window's last
  // step's scores at the deepest focal layer (Cross-Step Fixation Reuse /
  // Implementation).  The image-token counts come from the lens of that
  // step, copied aside when it ran.
  const int deepest = h->focal.back();
  int rc = run_topk(h, h->warm_scores + (size_t)deepest * c.batch * h->n_stride, h->lens_shadow, nullptr);
  if (rc) return rc;
  e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return fail_hip(h, e);
  h->phase = PHASE_PRUNED;
  h->pruned_since = 0;
  ++h->profiles;
  return FASTOCR_OK;
}

// One layer of the current step (fastocr_attend, fastocr_attend_append).
static int attend_impl(fastocr_handle* h, int32_t layer, const void* q, const void* k_cache,
                       const void* v_cache, const int32_t* lens, void* out) {
  if (h->poisoned) return FASTOCR_ERR_STATE;
  if (!q || !k_cache || !v_cache || !lens || !out) return FASTOCR_ERR_INVALID_ARG;
  const fastocr_config& c = h->cfg;
  if (layer < 0 || layer >= c.num_layers) return FASTOCR_ERR_INVALID_ARG;
  if (layer != h->next_layer) return FASTOCR_ERR_STATE;
  int rc = FASTOCR_OK;
  if (h->phase == PHASE_WARMUP_DONE) {
    // the first warm-up ends with an explicit fastocr_profile_warmup; a
    // re-selection window profiles itself here, before the step's first layer
    if (h->profiles == 0) return FASTOCR_ERR_STATE;
    rc = profile_impl(h);
    if (rc) return rc;
  }

  const size_t BH = (size_t)c.batch * c.num_q_heads;
  char label[96] = "";
  if (h->roctx.push) {
    const bool dead = h->skip_dead_picks && layer + 1 < c.num_layers && h->is_focal[layer + 1];
    const char* kind = h->phase == PHASE_FULL              ? "full"
                       : h->phase == PHASE_WARMUP          ? "warm-up"
                       : h->is_focal[layer] && dead        ? "focal-unused-pick"
                       : h->is_focal[layer]                ? "focal"
                       : h->keeps_all              ? "kept-all"
                                                   : "kept-token";
    std::snprintf(label, sizeof(label), "fastocr step %d layer %d %s", h->step, layer, kind);
  }
  TraceRange range(&h->roctx, label);
  switch (h->phase) {
    case PHASE_FULL:
      rc = run_full(h, q, k_cache, v_cache, lens, out, nullptr, nullptr, false, false);
      break;
    case PHASE_WARMUP: {
      float* tm = h->text_mass + ((size_t)layer * c.warmup_steps + h->warm_pos) * BH;
      float* sc = (h->warm_pos == c.warmup_steps - 1)
                      ? h->warm_scores + (size_t)layer * c.batch * h->n_stride
                      : nullptr;
      rc = run_full(h, q, k_cache, v_cache, lens, out, tm, sc, false, false);
      if (!rc && sc && layer == 0) {
        hipError_t e = hipMemcpyAsync(h->lens_shadow, lens, (size_t)c.batch * 2 * sizeof(int32_t),
                                      hipMemcpyDeviceToDevice, h->stream);
        if (e != hipSuccess) rc = fail_hip(h, e);
      }
      break;
    }
    case PHASE_PRUNED:
      if (h->is_focal[layer] && h->skip_dead_picks && layer + 1 < c.num_layers && h->is_focal[layer + 1]) {
        // the next layer is focal too and replaces this layer's pick before
        // any layer attends with it: the full pass alone gives every output
        rc = run_full(h, q, k_cache, v_cache, lens, out, nullptr, nullptr, false, h->stream_rows);
      } else if (h->is_focal[layer]) {
        rc = run_full(h, q, k_cache, v_cache, lens, out, nullptr, h->scores, true, h->stream_rows);
      } else if (h->keeps_all) {
        // tau = 1 keeps every image token: the kept set plus the text is the
        // whole sequence, which the full pass reads without the gather
        rc = run_full(h, q, k_cache, v_cache, lens, out, nullptr, nullptr, false, false);
      } else {
        rc = run_sparse(h, q, k_cache, v_cache, lens, out);
      }
      break;
    default:
      return FASTOCR_ERR_STATE;
  }
  if (rc) return rc;
  if (++h->next_layer == c.num_layers) {
    h->next_layer = 0;
    ++h->step;
    if (h->phase == PHASE_WARMUP && ++h->warm_pos == c.warmup_steps) h->phase = PHASE_WARMUP_DONE;
    if (h->phase == PHASE_PRUNED && ++h->pruned_since == c.reprofile_every) {
      // periodic re-selection: a new warm-up window of w full steps, whose
      // statistics alone pick the next focal set
      h->phase = PHASE_WARMUP;
      h->warm_pos = 0;
    }
  }
  return FASTOCR_OK;
}

int fastocr_attend(fastocr_handle* h, int32_t layer, const void* q, const void* k_cache,
                   const void* v_cache, const int32_t* lens, void* out) {
  if (!h) return FASTOCR_ERR_INVALID_ARG;
  h->app_k = h->app_v = nullptr;
  return attend_impl(h, layer, q, k_cache, v_cache, lens, out);
}

int fastocr_attend_append(fastocr_handle* h, int32_t layer, const void* q, const void* k_new,
                          const void* v_new, void* k_cache, void* v_cache, const int32_t* lens,
                          void* out) {
  if (!h) return FASTOCR_ERR_INVALID_ARG;
  if (!k_new || !v_new) return FASTOCR_ERR_INVALID_ARG;
  h->app_k = k_new;
  h->app_v = v_new;
  const int rc = attend_impl(h, layer, q, k_cache, v_cache, lens, out);
  h->app_k = h->app_v = nullptr;
  return rc;
}

int fastocr_profile_warmup(fastocr_handle* h, int32_t* focal_layers_out) {
  if (!h || !focal_layers_out) return FASTOCR_ERR_INVALID_ARG;
  if (h->poisoned || h->phase != PHASE_WARMUP_DONE) return FASTOCR_ERR_STATE;
  const int rc = profile_impl(h);
  if (rc) return rc;
  std::memcpy(focal_layers_out, h->focal.data(), sizeof(int32_t) * h->cfg.num_focal);
  return FASTOCR_OK;
}

int fastocr_get_focal_layers(fastocr_handle* h, int32_t* layers_host) {
  if (!h || !layers_host) return FASTOCR_ERR_INVALID_ARG;
  if (h->focal.empty()) return FASTOCR_ERR_STATE;
  std::memcpy(layers_host, h->focal.data(), sizeof(int32_t) * h->focal.size());
  return FASTOCR_OK;
}

int fastocr_destroy(fastocr_handle* h) {
  if (!h) return FASTOCR_OK;
  int rc = FASTOCR_OK;
  if (hipStreamSynchronize(h->stream) != hipSuccess) rc = FASTOCR_ERR_HIP;
  for (auto& ev : h->events) (void)hipEventDestroy(ev.end);
  if (h->owns_arena) {
    if (h->arena && hipFree(h->arena) != hipSuccess) rc = FASTOCR_ERR_HIP;
  } else if (h->on_destroy) {
    h->on_destroy(h->device);
  }
  delete h;
  return rc;
}

int fastocr_get_status(fastocr_handle* h, int32_t* flags) {
  if (!h || !flags) return FASTOCR_ERR_INVALID_ARG;
  if (h->poisoned) return FASTOCR_ERR_STATE;
  hipError_t e = hipStreamSynchronize(h->stream);
  if (e == hipSuccess) e = hipMemcpy(flags, h->status, sizeof(int32_t), hipMemcpyDeviceToHost);
  return fail_hip(h, e);
}

int fastocr_get_selection(fastocr_handle* h, int32_t* idx_dev, int32_t* cnt_dev) {
  if (!h || !idx_dev || !cnt_dev) return FASTOCR_ERR_INVALID_ARG;
  if (h->poisoned) return FASTOCR_ERR_STATE;
  const size_t B = h->cfg.batch;
  hipError_t e = hipMemcpyAsync(idx_dev, h->sel, B * h->k_max * sizeof(int32_t),
                                hipMemcpyDeviceToDevice, h->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(cnt_dev, h->sel_cnt, B * sizeof(int32_t), hipMemcpyDeviceToDevice, h->stream);
  return fail_hip(h, e);
}

int fastocr_set_selection(fastocr_handle* h, const int32_t* idx_dev, const int32_t* cnt_dev) {
  if (!h || !idx_dev || !cnt_dev) return FASTOCR_ERR_INVALID_ARG;
  if (h->poisoned) return FASTOCR_ERR_STATE;
  const size_t B = h->cfg.batch;
  hipError_t e = hipMemcpyAsync(h->sel, idx_dev, B * h->k_max * sizeof(int32_t),
                                hipMemcpyDeviceToDevice, h->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->sel_cnt, cnt_dev, B * sizeof(int32_t), hipMemcpyDeviceToDevice, h->stream);
  return fail_hip(h, e);
}

int fastocr_get_scores(fastocr_handle* h, float* scores_dev) {
  if (!h || !scores_dev) return FASTOCR_ERR_INVALID_ARG;
  if (h->poisoned || !h->scores) return FASTOCR_ERR_STATE;
  if (h->n_cap == 0) return FASTOCR_OK;
  hipError_t e = hipMemcpy2DAsync(scores_dev, (size_t)h->n_cap * sizeof(float), h->scores,
                                  (size_t)h->n_stride * sizeof(float), (size_t)h->n_cap * sizeof(float),
                                  h->cfg.batch, hipMemcpyDeviceToDevice, h->stream);
  return fail_hip(h, e);
}

int fastocr_get_layer_ratios(fastocr_handle* h, double* ratios_host) {
  if (!h || !ratios_host) return FASTOCR_ERR_INVALID_ARG;
  if ((int)h->ratios.size() != h->cfg.num_layers) return FASTOCR_ERR_STATE;
  std::memcpy(ratios_host, h->ratios.data(), sizeof(double) * h->ratios.size());
  return FASTOCR_OK;
}

int fastocr_set_focal_layers(fastocr_handle* h, const int32_t* layers_host, int32_t count) {
  if (!h || !layers_host) return FASTOCR_ERR_INVALID_ARG;
  const int L = h->cfg.num_layers;
  // exactly |C| layers: fastocr_get_focal_layers and fastocr_profile_warmup
  // write num_focal entries
  if (count != h->cfg.num_focal) return FASTOCR_ERR_INVALID_ARG;
  std::vector<char> seen(L, 0);
  for (int i = 0; i < count; ++i) {
    const int l = layers_host[i];
    if (l < 0 || l >= L || seen[l]) return FASTOCR_ERR_INVALID_ARG;
    seen[l] = 1;
  }
  if (h->poisoned || (h->phase != PHASE_WARMUP_DONE && h->phase != PHASE_PRUNED)) return FASTOCR_ERR_STATE;
  if (h->next_layer != 0) return FASTOCR_ERR_STATE;
  h->focal.clear();
  for (int l = 0; l < L; ++l)
    if (seen[l]) h->focal.push_back(l);
  h->is_focal = seen;
  if (h->phase == PHASE_WARMUP_DONE) {
    // ends the warm-up window as a profile does, with the given set: the
    // first pruned step inherits top-k of the window's last-step scores at
    // the deepest of these layers (Cross-Step Fixation Reuse /
    // Implementation); the layer ratios are not computed
    const int deepest = h->focal.back();
    int rc = run_topk(h, h->warm_scores + (size_t)deepest * h->cfg.batch * h->n_stride, h->lens_shadow, nullptr);
    if (rc) return rc;
    const hipError_t e = hipStreamSynchronize(h->stream);
    if (e != hipSuccess) return fail_hip(h, e);
    h->pruned_since = 0;
    ++h->profiles;
  }
  h->phase = PHASE_PRUNED;
  return FASTOCR_OK;
}

int fastocr_get_info(fastocr_handle* h, fastocr_info* info) {
  if (!h || !info) return FASTOCR_ERR_INVALID_ARG;
  info->step = h->step;
  info->next_layer = h->next_layer;
  info->phase = h->phase;
  info->k_max = h->k_max;
  info->full_rows_per_split = h->full_R;
  info->full_max_splits = h->full_splits;
  info->sparse_rows_per_split = h->sparse_R;
  info->sparse_max_splits = h->sparse_splits;
  info->sparse_direct = h->sparse_splits <= 1 ? 1 : 0;
  info->focal_staged = h->focal_staged ? 1 : 0;
  info->stream_rows = h->stream_rows ? 1 : 0;
  info->profiles = h->profiles;
  info->scratch_bytes = (int64_t)h->arena_bytes;
  return FASTOCR_OK;
}

int fastocr_plan_launch(const fastocr_config* cfg, int32_t num_cu, fastocr_info* info) {
  if (!cfg || !info) return FASTOCR_ERR_INVALID_ARG;
  Plan p;
  const int rc = make_plan(*cfg, num_cu, p);
  if (rc != FASTOCR_OK) return rc;
  *info = fastocr_info{};
  info->phase = cfg->mode == FASTOCR_MODE_FULL ? PHASE_FULL : PHASE_WARMUP;
  info->k_max = p.k_max;
  info->full_rows_per_split = p.full_R;
  info->full_max_splits = p.full_splits;
  info->sparse_rows_per_split = p.sparse_R;
  info->sparse_max_splits = p.sparse_splits;
  info->sparse_direct = p.sparse_splits <= 1 ? 1 : 0;
  info->focal_staged = p.focal_staged ? 1 : 0;
  info->stream_rows = p.stream_rows ? 1 : 0;
  info->scratch_bytes = (int64_t)p.arena_bytes;
  return FASTOCR_OK;
}

int fastocr_set_timing(fastocr_handle* h, int32_t enable) {
  if (!h) return FASTOCR_ERR_INVALID_ARG;
  h->timing = enable != 0;
  return FASTOCR_OK;
}

int fastocr_get_timing(fastocr_handle* h, fastocr_timing* out) {
  if (!h || !out) return FASTOCR_ERR_INVALID_ARG;
  if (h->poisoned) return FASTOCR_ERR_STATE;
  hipError_t e = hipStreamSynchronize(h->stream);
  if (e != hipSuccess) return fail_hip(h, e);
  // a launch's time: from the previous timed launch's end to its own end
  for (size_t i = 0; i < h->ev_used; ++i) {
    const int cls = h->events[i].cls;
    h->timing_acc.launches[cls] += 1;
    if (i == 0) continue;
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, h->events[i - 1].end, h->events[i].end);
    if (e != hipSuccess) return fail_hip(h, e);
    h->timing_acc.total_ms[cls] += ms;
    h->timing_acc.timed[cls] += 1;
  }
  h->ev_used = 0;
  *out = h->timing_acc;
  return FASTOCR_OK;
}

int fastocr_reset_timing(fastocr_handle* h) {
  if (!h) return FASTOCR_ERR_INVALID_ARG;
  if (hipStreamSynchronize(h->stream) != hipSuccess) return fail_hip(h, hipErrorUnknown);
  h->ev_used = 0;
  h->timing_acc = fastocr_timing{};
  return FASTOCR_OK;
}


int fastocr_state_bytes(fastocr_handle* h, int64_t* bytes) {
  if (!h || !bytes) return FASTOCR_ERR_INVALID_ARG;
  *bytes = (int64_t)state_bytes(h);
  return FASTOCR_OK;
}

int fastocr_save_state(fastocr_handle* h, void* host_buf, int64_t bytes) {
  if (!h || !host_buf) return FASTOCR_ERR_INVALID_ARG;
  if (bytes < (int64_t)state_bytes(h)) return FASTOCR_ERR_INVALID_ARG;
  if (h->poisoned || h->next_layer != 0) return FASTOCR_ERR_STATE;
  const int L = h->cfg.num_layers;
  char* p = static_cast<char*>(host_buf);
  const StateHeader s = state_header(h);
  std::memcpy(p, &s, sizeof(s));
  p += sizeof(s);
  std::vector<int32_t> focal(L, -1);
  std::copy(h->focal.begin(), h->focal.end(), focal.begin());
  std::vector<double> ratios(L, 0.0);
  std::copy(h->ratios.begin(), h->ratios.end(), ratios.begin());
  std::memcpy(p, focal.data(), L * sizeof(int32_t));
  p += L * sizeof(int32_t);
  std::memcpy(p, ratios.data(), L * sizeof(double));
  p += L * sizeof(double);
  hipError_t e = hipStreamSynchronize(h->stream);
  for (const StateArray& a : state_arrays(h)) {
    if (e == hipSuccess && a.bytes) e = hipMemcpy(p, a.dev, a.bytes, hipMemcpyDeviceToHost);
    p += a.bytes;
  }
  return e == hipSuccess ? FASTOCR_OK : fail_hip(h, e);
}

int fastocr_load_state(fastocr_handle* h, const void* host_buf, int64_t bytes) {
  if (!h || !host_buf) return FASTOCR_ERR_INVALID_ARG;
  if (bytes < (int64_t)sizeof(StateHeader) || bytes < (int64_t)state_bytes(h)) return FASTOCR_ERR_INVALID_ARG;
  if (h->poisoned || h->next_layer != 0) return FASTOCR_ERR_STATE;
  const int L = h->cfg.num_layers;
  const char* p = static_cast<const char*>(host_buf);
  StateHeader s;
  std::memcpy(&s, p, sizeof(s));
  p += sizeof(s);
  StateHeader mine = state_header(h);
  // the configuration must be the handle's own (the per-run fields may differ)
  mine.step = s.step;
  mine.phase = s.phase;
  mine.warm_pos = s.warm_pos;
  mine.pruned_since = s.pruned_since;
  mine.profiles = s.profiles;
  mine.n_focal = s.n_focal;
  mine.n_ratios = s.n_ratios;
  if (std::memcmp(&s, &mine, sizeof(s)) != 0) return FASTOCR_ERR_INVALID_ARG;
  const bool pruned = h->cfg.mode == FASTOCR_MODE_PRUNED;
  const int ph = s.phase;
  const bool phase_ok = pruned ? (ph == PHASE_WARMUP || ph == PHASE_WARMUP_DONE || ph == PHASE_PRUNED)
                               : ph == PHASE_FULL;
  if (!phase_ok || s.step < 0 || s.warm_pos < 0 || s.warm_pos > s.w || s.pruned_since < 0 ||
      s.profiles < 0 || s.n_focal < 0 || s.n_focal > L || s.n_ratios < 0 || s.n_ratios > L ||
      (ph == PHASE_PRUNED && s.n_focal == 0))
    return FASTOCR_ERR_INVALID_ARG;
  std::vector<int32_t> focal(L);
  std::memcpy(focal.data(), p, L * sizeof(int32_t));
  p += L * sizeof(int32_t);
  std::vector<char> is_focal(L, 0);
  for (int i = 0; i < s.n_focal; ++i) {
    if (focal[i] < 0 || focal[i] >= L || is_focal[focal[i]]) return FASTOCR_ERR_INVALID_ARG;
    is_focal[focal[i]] = 1;
  }
  std::vector<double> ratios(L);
  std::memcpy(ratios.data(), p, L * sizeof(double));
  p += L * sizeof(double);
  hipError_t e = hipStreamSynchronize(h->stream);
  for (const StateArray& a : state_arrays(h)) {
    if (e == hipSuccess && a.bytes) e = hipMemcpy(a.dev, p, a.bytes, hipMemcpyHostToDevice);
    p += a.bytes;
  }
  if (e != hipSuccess) return fail_hip(h, e);
  h->step = s.step;
  h->phase = s.phase;
  h->warm_pos = s.warm_pos;
  h->pruned_since = s.pruned_since;
  h->profiles = s.profiles;
  h->focal.assign(focal.begin(), focal.begin() + s.n_focal);
  h->is_focal = is_focal;
  h->ratios.assign(ratios.begin(), ratios.begin() + s.n_ratios);
  return FASTOCR_OK;
}

int32_t fastocr_image_first_map(const int32_t* spans, int32_t num_spans, int32_t rows, int32_t* map_out) {
  if ((!spans && num_spans > 0) || !map_out || num_spans < 0 || rows < 0) return FASTOCR_ERR_INVALID_ARG;
  std::vector<char> img((size_t)rows, 0);
  int64_t n = 0, prev_end = 0;
  for (int32_t i = 0; i < num_spans; ++i) {
    const int64_t a = spans[2 * i], c = spans[2 * i + 1];
    // ascending, disjoint, inside [0, rows)
    if (a < prev_end || c < 0 || a + c > rows) return FASTOCR_ERR_INVALID_ARG;
    for (int64_t r = a; r < a + c; ++r) img[(size_t)r] = 1;
    n += c;
    prev_end = a + c;
  }
  int32_t at = 0;
  for (int32_t r = 0; r < rows; ++r)
    if (img[(size_t)r]) map_out[at++] = r;
  for (int32_t r = 0; r < rows; ++r)
    if (!img[(size_t)r]) map_out[at++] = r;
  return (int32_t)n;
}

int fastocr_pack_rows(const void* src, void* dst, const int32_t* row_map, const int32_t* rows,
                      int32_t batch, int32_t num_kv_heads, int32_t max_seq_len, int32_t head_dim,
                      int32_t dtype, int32_t* status, void* hip_stream) {
  if (!src || !dst || !row_map || !rows) return FASTOCR_ERR_INVALID_ARG;
  if (batch < 1 || num_kv_heads < 1 || max_seq_len < 1) return FASTOCR_ERR_INVALID_ARG;
  if ((int64_t)batch * num_kv_heads > 65535) return FASTOCR_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return FASTOCR_ERR_INVALID_ARG;
  if (dtype != FASTOCR_DTYPE_F32 && dtype != FASTOCR_DTYPE_BF16) return FASTOCR_ERR_INVALID_ARG;
  const int row_bytes = head_dim * (dtype == FASTOCR_DTYPE_BF16 ? 2 : 4);
  const uintptr_t bytes = (uintptr_t)batch * num_kv_heads * max_seq_len * row_bytes;
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  if (s0 < d0 + bytes && d0 < s0 + bytes) return FASTOCR_ERR_INVALID_ARG;  // overlap
  if ((s0 | d0) % 16) return FASTOCR_ERR_INVALID_ARG;
  PackParams p{};
  p.src = src;
  p.dst = dst;
  p.map = row_map;
  p.rows = rows;
  p.status = status;
  p.B = batch;
  p.Hkv = num_kv_heads;
  p.S = max_seq_len;
  p.row_bytes = row_bytes;
  const hipError_t e = launch_pack(p, reinterpret_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? FASTOCR_OK : FASTOCR_ERR_HIP;
}

int fastocr_select_topk(const float* scores, int32_t score_stride, const int32_t* lens,
                        int32_t batch, double tau, int32_t* idx_out, int32_t idx_stride,
                        int32_t* cnt_out, void* hip_stream) {
  if (!scores || !lens || !idx_out || !cnt_out) return FASTOCR_ERR_INVALID_ARG;
  if (score_stride < 1 || batch < 1 || idx_stride < 1) return FASTOCR_ERR_INVALID_ARG;
  if (!(tau > 0.0 && tau <= 1.0)) return FASTOCR_ERR_INVALID_ARG;
  TopkParams t{};
  t.scores = scores;
  t.score_stride = score_stride;
  t.n_cap = score_stride;
  t.lens = lens;
  t.B = batch;
  t.tau = tau;
  t.idx = idx_out;
  t.idx_stride = idx_stride;
  t.cnt = cnt_out;
  t.status = nullptr;
  hipError_t e = launch_topk(t, reinterpret_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? FASTOCR_OK : FASTOCR_ERR_HIP;
}

}  // extern "C"
