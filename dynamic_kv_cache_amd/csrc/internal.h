// Internal interface between the host runtime (fastocr_api.cpp) and the
// gfx950 kernels (kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fastocr {

// Kinds of split-K attention pass.
enum SplitKind : int {
  KIND_FULL = 0,    // all rows [0, len_b)
  KIND_FOCAL = 1,   // all rows, and export the image-token logits
  KIND_SPARSE = 2,  // kept image rows (gathered by index) + rows [n_img_b, len_b)
};

// Rows a wave consumes per tile and waves per workgroup of the split kernel.
constexpr int kTileRows = 16;
constexpr int kSplitWaves = 4;
constexpr int kRowsPerPass = kTileRows * kSplitWaves;
// Upper bound on splits per (sequence, KV head); the combine kernel keeps one
// weight per split in LDS.
constexpr int kMaxSplits = 2048;

struct SplitParams {
  const void* q;          // [B, Hq, D]
  const void* k;          // [B, Hkv, S, D]
  const void* v;          // [B, Hkv, S, D]
  const int32_t* lens;    // [B, 2]
  const int32_t* sel;     // [B, k_stride]   (sparse)
  const int32_t* sel_cnt; // [B]             (sparse)
  float* logits;          // [B, Hq, n_stride] log2-domain scaled logits (focal)
  float4* pstat;          // [B, Hq, max_splits] (max, sum p, sum rounded p, text sum p)
  float* po;              // [B, Hq, max_splits, D] unnormalised partial outputs
  int32_t* status;
  int32_t B, Hq, Hkv, S, n_cap, n_stride, k_stride, max_splits, rows_per_split;
  int32_t grid_splits;    // workgroups launched per (sequence, KV head)
  float scale_log2;       // logit scale * log2(e)
};

struct CombineParams {
  const float4* pstat;
  const float* po;
  const int32_t* lens;
  const int32_t* sel_cnt; // non-null: sparse row count
  void* out;              // [B, Hq, D] in the io dtype
  float2* mz;             // [B, Hq] (max, 1 / sum p) or null
  float* text_mass;       // [B, Hq] text probability mass or null
  int32_t B, Hq, S, n_cap, k_stride, max_splits, rows_per_split;
  int32_t grid_splits;    // splits the matching split pass launched
  int32_t* status;
};

struct ScoreParams {
  const float* logits;    // [B, Hq, n_stride]
  const float2* mz;       // [B, Hq]
  const int32_t* lens;
  float* scores;          // [B, n_stride]
  int32_t B, Hq, S, n_cap, n_stride;
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
};

hipError_t launch_split(int dtype, int head_dim, SplitKind kind, const SplitParams& p,
                        hipStream_t stream);
hipError_t launch_combine(int dtype, int head_dim, const CombineParams& p, hipStream_t stream);
hipError_t launch_score(const ScoreParams& p, hipStream_t stream);
hipError_t launch_topk(const TopkParams& p, hipStream_t stream);

}  // namespace fastocr
