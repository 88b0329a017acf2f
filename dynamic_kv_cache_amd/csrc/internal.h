// Internal interface between the host runtime (fastocr_api.cpp) and the
// gfx950 kernels (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fastocr.h"

namespace fastocr {

// Kinds of full-row split-K attention pass (kept-token passes run
// kept_attn_kernel).
enum SplitKind : int {
  KIND_FULL = 0,    // all rows [0, len_b)
  KIND_FOCAL = 1,   // all rows, and export the image-token logits
};

// Split kernel geometry: a wave consumes 16-row MFMA tiles and loads
// kTilesPerWave of them (one for fp32 rows of 128 elements) before computing
// any; a workgroup is kSplitWaves waves, so one round of a workgroup covers
// kRowsPerRound cache rows (half that for fp32 rows of 128; full-pass splits
// are whole multiples of kRowsPerRound either way).
constexpr int kTileRows = 16;
constexpr int kSplitWaves = 4;
constexpr int kTilesPerWave = 2;
constexpr int kRowsPerRound = kTileRows * kSplitWaves * kTilesPerWave;
constexpr int kSplitThreads = kSplitWaves * 64;
// Resident workgroups per CU the kernels are compiled for: full passes keep
// two rounds of K/V in registers, kept-token passes one.
constexpr int kFullBlocksPerCU = 2;
constexpr int kKeptBlocksPerCU = 3;
// Kept-token passes (non-focal layers) run kept_attn_kernel: each (sequence,
// KV head) pair's 16-row tiles are dealt round-robin to P workgroups
// (P <= kMaxKeptSplits), whose states the merge kernel combines.
constexpr int kMaxKeptSplits = 32;
// The chip's last-level (Infinity) cache, shared by all XCDs.  Kept-token
// and focal passes stream their K/V rows past the caches when one step's
// kept rows exceed it.
constexpr int64_t kLastLevelCacheBytes = int64_t(256) << 20;
// Focal passes stage a split's image-token logits in LDS (heads x
// (rows_per_split + kLogitStagePad) floats) when they fit in this many floats
// (66 KB, two workgroups per CU).
constexpr int kLogitStagePad = 16;
constexpr int kLogitStageFloats = 8 * (2048 + kLogitStagePad);
constexpr int kLogitStageMinRows = 512;  // shorter splits store the logits as computed
constexpr int kMergeThreads = 256;
constexpr int kMaxMergeSplits = 1024;  // split weights one merge workgroup keeps in LDS
constexpr int kMaxHeads = 128;
constexpr int kTopkThreads = 1024;
constexpr int kTopkRegKeys = 16;  // keys per thread the top-k holds in registers
constexpr int kTopkCand = 64;      // a k-th-key bin this small is ranked pairwise (one wave)

struct SplitParams {
  const void* q;          // [B, Hq, D]
  const void* k;          // [B, Hkv, S, D]
  const void* v;          // [B, Hkv, S, D]
  const int32_t* lens;    // [B, 2]
  const int32_t* sel;     // [B, k_stride]   kept set (kept-token pass)
  const int32_t* sel_cnt; // [B]
  float* logits;          // [B, Hq, n_stride] log2-domain scaled logits (focal)
  float4* pstat;          // [B, Hq, max_splits] (max, sum p, sum rounded p, text sum p) of
                          // each split
  float* po;              // [B, Hq, max_splits, D] unnormalised partial outputs
  void* out;              // [B, Hq, D] in the io dtype (a kept-token pass of one split per pair)
  int32_t* status;
  int32_t B, Hq, Hkv, S, n_cap, n_stride, k_stride, max_splits, rows_per_split;
  int32_t grid_splits;    // workgroups launched per (sequence, KV head)
  int32_t stream_rows;    // load the K/V rows non-temporally
  int32_t sure_splits;    // full pass: splits that hold rows for every accepted sequence
  const void* k_new;      // [B, Hkv, D] the current token's key and value, or null: when
  const void* v_new;      // set, cache row len-1 is read from here and written into the
  void* k_w;              // caches (k_w, v_w: the same buffers as k, v) by each pair's
  void* v_w;              // split 0
  float scale_log2;       // logit scale * log2(e)
  int32_t stage_logits;   // focal kind: stage the logits in LDS (G * (rows_per_split +
                          // kLogitStagePad) <= kLogitStageFloats) and write them after the
                          // split's rows; 0: store them as they are computed
  int32_t valu;           // full kind, bf16, D = 128, Hq/Hkv <= kValuMaxGroup: the VALU
                          // variant (fp32 FMAs and 16-lane shuffle reductions instead of
                          // MFMA; a measurement override, same states)
};
constexpr int kValuMaxGroup = 8;

// Merge of a split pass (one workgroup per head) and, for focal layers, the
// head-summed image-token scores (score_blocks workgroups per sequence).
struct MergeParams {
  const float4* pstat;
  const float* po;
  const int32_t* lens;
  void* out;              // [B, Hq, D] in the io dtype
  float* text_mass;       // [B, Hq] or null
  int32_t B, Hq, Hkv, n_cap, max_splits;
  int32_t grid_splits;    // states per head written by the split pass
  const float* logits;    // [B, Hq, n_stride]
  float* scores;          // [B, n_stride]
  int32_t n_stride;
  int32_t score_blocks;   // workgroups per sequence for scores (0: none)
  unsigned int* hist0;    // [B, 256] or null: add each image token's leading score
                          // byte to its sequence's histogram (the top-k's first pass)
};

struct TopkParams {
  const float* scores;
  int32_t score_stride;
  int32_t n_cap;          // image tokens are clamped to [0, min(len_b, n_cap)]
  const int32_t* lens;
  int32_t B;
  double tau;
  int32_t* idx;
  int32_t idx_stride;
  int32_t* cnt;
  int32_t* status;        // may be null
  unsigned int* hist0;    // [B, 256] leading-byte histograms of the scores, or null;
                          // read and cleared to zero
};

// Row gather of a cache: dst[b, h, i] = src[b, h, map[b, i]] for i < rows_b.
struct PackParams {
  const void* src;        // [B, Hkv, S, row_bytes]
  void* dst;              // same shape; must not overlap src
  const int32_t* map;     // [B, S] source row of each destination row
  const int32_t* rows;    // [B] destination rows to fill (clamped to [0, S])
  int32_t* status;        // may be null: FASTOCR_FLAG_INDEX_CLAMPED on a map entry outside [0, S)
  int32_t B, Hkv, S, row_bytes;  // row_bytes a multiple of 16
};
constexpr int kPackThreads = 256;
constexpr int kPackRowsPerBlock = 64;

// Optional timing: events recorded by the dispatch itself (start: when the
// dispatch is processed; stop: when the kernel completes).
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

hipError_t launch_split(int dtype, int head_dim, SplitKind kind, const SplitParams& p,
                        hipStream_t stream, const LaunchTiming& timing = LaunchTiming{});
hipError_t launch_kept(int dtype, int head_dim, const SplitParams& p, hipStream_t stream,
                       const LaunchTiming& timing = LaunchTiming{});
hipError_t launch_merge(int dtype, int head_dim, const MergeParams& p, hipStream_t stream,
                        const LaunchTiming& timing = LaunchTiming{});
// Merge of a kept-token pass (grid_splits <= 64, no scores, no text mass).
hipError_t launch_kept_merge(int dtype, int head_dim, const MergeParams& p, hipStream_t stream,
                             const LaunchTiming& timing = LaunchTiming{});
hipError_t launch_topk(const TopkParams& p, hipStream_t stream,
                       const LaunchTiming& timing = LaunchTiming{});
hipError_t launch_pack(const PackParams& p, hipStream_t stream);

// fastocr_create with the scratch arena allocated (arena null) or placed at
// `arena` (arena_cap bytes of device memory the caller keeps; a larger plan
// fails with FASTOCR_ERR_SCRATCH; on_destroy(device) runs at destroy).
int create_handle(const fastocr_config* cfg, void* hip_stream, fastocr_handle** out, void* arena,
                  size_t arena_cap, void (*on_destroy)(int));

}  // namespace fastocr
