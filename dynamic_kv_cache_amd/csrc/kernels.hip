// gfx950 kernels of the FastOCR decode-step attention path.
//
// Method source: "FastOCR: Dynamic Visual Fixation via KV Cache Pruning for
// Efficient Document Parsing", technical summary, Method / 1. Focal-Guided
// Pruning (Focal Layer Selection, Cross-Layer Propagation) and 2. Cross-Step
// Fixation Reuse; the paper's abstract.
//
// Kernels
//   split_attn_kernel  split-K decode attention over one chunk of rows per
//                      workgroup, for one (sequence, KV head).  Three kinds:
//                      full rows, full rows + image-logit export (focal
//                      layers), and kept image rows gathered by index + every
//                      text row (non-focal layers).
//   combine_kernel     merges the per-split partial softmax states into the
//                      output; optionally exports each head's (max, 1/sum) and
//                      its text-probability mass.
//   score_kernel       head-summed probability of every image token.
//   topk_kernel        radix select of the k_b highest scores per sequence,
//                      ties to the lower index, ascending output.
//
// Matrix layout on the MFMA units.  A workgroup is 4 waves; a wave consumes
// 16 cache rows per tile.  The GQA query group of one KV head (up to 16
// heads, zero padded) is the N side of a 16x16 MFMA tile:
//   logits^T[16 rows x 16 heads]  = K_tile[16 x d] * Q^T[d x 16]
//   out^T   [16 d     x 16 heads] += V_tile^T[16 d x 16 rows] * P^T[16 rows x 16 heads]
// Because a contraction may visit its index in any order, the d index is
// permuted so every lane's operands come straight from global memory with
// no LDS transpose:
//   QK: lane (c = lane%16, g = lane/16) loads the contiguous slice
//       K[row c][g*d/4, (g+1)*d/4) and the same slice of its query head c;
//       MFMA number kk contracts elements kk*4..kk*4+3 of those slices (bf16
//       16x16x16) or element kk (fp32 16x16x4).
//   PV: lane (c, g) loads rows 4g..4g+3 of the tile, each the contiguous
//       slice [c*d/16, (c+1)*d/16); MFMA number db uses element db of each
//       row, so output lane (c, g) ends up holding head c's outputs for
//       d = (4g+i)*(d/16) + db, i.e. the contiguous range [g*d/4, (g+1)*d/4).
// The logits come out as lane (c, g) = head c, rows 4g..4g+3, which is
// exactly the P^T operand the PV product needs, so softmax stays in
// registers.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/fastocr.h"
#include "internal.h"

namespace fastocr {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

template <typename T>
__device__ __forceinline__ void store_out(T* p, float v);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float v) { *p = v; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float v) {
  *p = (uint16_t)f32_to_bf16(v);
}

// Clamp a sequence's (n_img, len) to the buffers; report whether it changed.
__device__ __forceinline__ bool seq_extent(const int32_t* lens, int b, int S, int n_cap, int& n,
                                           int& len) {
  const int n0 = lens[2 * b];
  const int l0 = lens[2 * b + 1];
  len = min(max(l0, 0), S);
  n = min(max(n0, 0), min(len, n_cap));
  return n != n0 || len != l0;
}

// Rows attended by one sequence in a split pass, in "virtual row" order:
// full kinds visit [0, len); the sparse kind visits the kept set first, then
// the text rows [n, len).
__device__ __forceinline__ int kept_rows(const int32_t* sel_cnt, int b, int n, int k_stride) {
  return min(max(sel_cnt[b], 0), min(n, k_stride));
}

template <typename T>
__device__ __forceinline__ void load_words(uint32_t* dst, const T* src, int nwords) {
  // nwords is a compile-time multiple of 2 or 4 at every call site.
  const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
  if ((nwords & 3) == 0) {
#pragma unroll
    for (int i = 0; i < nwords; i += 4) {
      uint4 v = *reinterpret_cast<const uint4*>(s + i);
      dst[i] = v.x; dst[i + 1] = v.y; dst[i + 2] = v.z; dst[i + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < nwords; i += 2) {
      uint2 v = *reinterpret_cast<const uint2*>(s + i);
      dst[i] = v.x; dst[i + 1] = v.y;
    }
  }
}

__device__ __forceinline__ float wave_max16_32(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float wave_sum16_32(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// ---------------------------------------------------------------------------
// split-K decode attention
// ---------------------------------------------------------------------------

template <typename T, int D, int KIND>
__global__ __launch_bounds__(256) void split_attn_kernel(SplitParams p) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int E = D / 4;                           // K/q elements per lane
  constexpr int KW = E * (int)sizeof(T) / 4;         // ... as 32-bit words
  constexpr int NDB = D / 16;                        // PV d-blocks = V elements per row per lane
  constexpr int VW = NDB * (int)sizeof(T) / 4;       // V words per row per lane
  constexpr int OST = D + 1;                         // padded LDS row of partial outputs

  __shared__ float s_stat[kSplitWaves][16][4];
  __shared__ float s_o[kSplitWaves][16][OST];

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int G = p.Hq / p.Hkv;

  int n, len;
  const bool clamped = seq_extent(p.lens, b, p.S, p.n_cap, n, len);
  if (clamped && split == 0 && kvh == 0 && threadIdx.x == 0)
    atomicOr(p.status, FASTOCR_FLAG_LENS_CLAMPED);
  const int kept = (KIND == KIND_SPARSE) ? kept_rows(p.sel_cnt, b, n, p.k_stride) : n;
  const int rows = (KIND == KIND_SPARSE) ? kept + (len - n) : len;
  const int begin = split * p.rows_per_split;
  if (begin >= rows) return;
  const int end = min(begin + p.rows_per_split, rows);

  const size_t row_base = ((size_t)b * p.Hkv + kvh) * (size_t)p.S;
  const T* __restrict__ Kb = reinterpret_cast<const T*>(p.k) + row_base * D;
  const T* __restrict__ Vb = reinterpret_cast<const T*>(p.v) + row_base * D;
  const int32_t* __restrict__ selb = (KIND == KIND_SPARSE) ? p.sel + (size_t)b * p.k_stride : nullptr;

  // virtual row -> cache row
  auto phys = [&](int r) -> int {
    if (KIND == KIND_SPARSE) {
      if (r < kept) {
        int j = selb[r];
        if (j < 0 || j >= n) {
          atomicOr(p.status, FASTOCR_FLAG_INDEX_CLAMPED);
          j = min(max(j, 0), max(n - 1, 0));
        }
        return j;
      }
      return n + (r - kept);
    }
    return r;
  };

  // Query operand of this lane: head (kvh*G + col), elements [grp*E, grp*E+E).
  uint32_t qw[KW];
  if (col < G) {
    const T* qp = reinterpret_cast<const T*>(p.q) + ((size_t)b * p.Hq + kvh * G + col) * D + grp * E;
    load_words(qw, qp, KW);
  } else {
#pragma unroll
    for (int i = 0; i < KW; ++i) qw[i] = 0u;
  }

  float m_run = -INFINITY, z = 0.f, lsum = 0.f, zt = 0.f;
  f32x4_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int tile = begin + wave * kTileRows; tile < end; tile += kRowsPerPass) {
    // ---- loads: K row (tile+col), slice grp; V rows tile+4grp+j, slice col
    uint32_t kw[KW];
    {
      const int pk = phys(min(tile + col, end - 1));
      load_words(kw, Kb + (size_t)pk * D + grp * E, KW);
    }
    uint32_t vw[4][VW];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pv = phys(min(tile + 4 * grp + j, end - 1));
      load_words(vw[j], Vb + (size_t)pv * D + col * NDB, VW);
    }

    // ---- logits^T = K_tile * Q^T
    f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if constexpr (BF) {
#pragma unroll
      for (int kk = 0; kk < E / 4; ++kk) {
        bf16x4_t a, bq;
        uint32_t a0 = kw[2 * kk], a1 = kw[2 * kk + 1];
        uint32_t b0 = qw[2 * kk], b1 = qw[2 * kk + 1];
        a = bf16x4_t{(short)(a0 & 0xffff), (short)(a0 >> 16), (short)(a1 & 0xffff), (short)(a1 >> 16)};
        bq = bf16x4_t{(short)(b0 & 0xffff), (short)(b0 >> 16), (short)(b1 & 0xffff), (short)(b1 >> 16)};
        s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, bq, s, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < E; ++kk)
        s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kw[kk]), __uint_as_float(qw[kk]), s,
                                                 0, 0, 0);
    }

    // ---- masked, scaled logits of rows tile+4grp+i for head col
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = tile + 4 * grp + i;
      x[i] = (r < end) ? s[i] * p.scale_log2 : -INFINITY;
    }
    if constexpr (KIND == KIND_FOCAL) {
      if (col < G) {
        float* lg = p.logits + ((size_t)b * p.Hq + kvh * G + col) * p.n_stride;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = tile + 4 * grp + i;
          if (r < end && r < n) lg[r] = x[i];
        }
      }
    }

    // ---- online softmax (per head; the 4 lane groups share a head)
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = wave_max16_32(mt);
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    float pr[4], pu[4];
    uint32_t pb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pr[i] = exp2f(x[i] - m_new);
      if constexpr (BF) {
        pb[i] = f32_to_bf16(pr[i]);
        pu[i] = bf16_to_f32(pb[i]);
      } else {
        pu[i] = pr[i];
      }
    }
    float ztile = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = tile + 4 * grp + i;
      const bool text = (KIND == KIND_SPARSE) ? (r >= kept) : (r >= n);
      ztile += text ? pr[i] : 0.f;
    }
    z = z * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
    lsum = lsum * alpha + ((pu[0] + pu[1]) + (pu[2] + pu[3]));
    zt = zt * alpha + ztile;
    m_run = m_new;

    // ---- out^T += V_tile^T * P^T
    if constexpr (BF) {
      const bf16x4_t pv = bf16x4_t{(short)pb[0], (short)pb[1], (short)pb[2], (short)pb[3]};
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int w = db >> 1;
        uint32_t e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) e[j] = (db & 1) ? (vw[j][w] >> 16) : (vw[j][w] & 0xffffu);
        const bf16x4_t a = bf16x4_t{(short)e[0], (short)e[1], (short)e[2], (short)e[3]};
        f32x4_t c = acc[db] * alpha;
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pv, c, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        f32x4_t c = acc[db] * alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vw[i][db]), pr[i], c, 0, 0, 0);
        acc[db] = c;
      }
    }
  }

  // ---- per-wave totals (lane groups of one head hold partial sums)
  z = wave_sum16_32(z);
  lsum = wave_sum16_32(lsum);
  zt = wave_sum16_32(zt);
  if (grp == 0) {
    s_stat[wave][col][0] = m_run;
    s_stat[wave][col][1] = z;
    s_stat[wave][col][2] = lsum;
    s_stat[wave][col][3] = zt;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[wave][col][(4 * grp + i) * NDB + db] = acc[db][i];
  __syncthreads();

  // ---- merge the 4 waves into this split's partial state
  const size_t slot0 = ((size_t)b * p.Hq + kvh * G) * p.max_splits + split;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = s_stat[0][h][0];
#pragma unroll
    for (int w = 1; w < kSplitWaves; ++w) M = fmaxf(M, s_stat[w][h][0]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) o += s_o[w][h][d] * exp2f(s_stat[w][h][0] - M);
    p.po[(slot0 + (size_t)h * p.max_splits) * D + d] = o;
  }
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = s_stat[0][h][0];
#pragma unroll
    for (int w = 1; w < kSplitWaves; ++w) M = fmaxf(M, s_stat[w][h][0]);
    float zz = 0.f, ll = 0.f, tt = 0.f;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
      const float e = exp2f(s_stat[w][h][0] - M);
      zz += s_stat[w][h][1] * e;
      ll += s_stat[w][h][2] * e;
      tt += s_stat[w][h][3] * e;
    }
    p.pstat[slot0 + (size_t)h * p.max_splits] = make_float4(M, zz, ll, tt);
  }
}

// ---------------------------------------------------------------------------
// split combine
// ---------------------------------------------------------------------------

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = fmaxf(r, red[w]);
  return r;
}

__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r += red[w];
  return r;
}

template <typename T, int D>
__global__ __launch_bounds__(128) void combine_kernel(CombineParams p) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[4];
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  int n, len;
  seq_extent(p.lens, b, p.S, p.n_cap, n, len);
  const int rows = p.sel_cnt ? kept_rows(p.sel_cnt, b, n, p.k_stride) + (len - n) : len;
  int nsplit = (rows + p.rows_per_split - 1) / p.rows_per_split;
  if (nsplit > p.grid_splits) {
    // more rows than the launch was sized for (a sequence below the declared
    // minimum image-token count): only the launched splits exist
    if (threadIdx.x == 0) atomicOr(p.status, FASTOCR_FLAG_ROWS_TRUNCATED);
    nsplit = p.grid_splits;
  }
  const size_t slot0 = ((size_t)b * p.Hq + h) * p.max_splits;
  T* out = reinterpret_cast<T*>(p.out) + ((size_t)b * p.Hq + h) * D;

  if (nsplit == 0) {
    for (int d = threadIdx.x; d < D; d += blockDim.x) store_out<T>(out + d, 0.f);
    if (threadIdx.x == 0) {
      if (p.mz) p.mz[b * p.Hq + h] = make_float2(-INFINITY, 0.f);
      if (p.text_mass) p.text_mass[b * p.Hq + h] = 0.f;
    }
    return;
  }

  float mloc = -INFINITY;
  for (int s = threadIdx.x; s < nsplit; s += blockDim.x) mloc = fmaxf(mloc, p.pstat[slot0 + s].x);
  const float M = block_reduce_max(mloc, s_red);
  float zl = 0.f, ll = 0.f, tl = 0.f;
  for (int s = threadIdx.x; s < nsplit; s += blockDim.x) {
    const float4 st = p.pstat[slot0 + s];
    const float w = exp2f(st.x - M);
    s_w[s] = w;
    zl += st.y * w;
    ll += st.z * w;
    tl += st.w * w;
  }
  const float Z = block_reduce_sum(zl, s_red);
  const float Lr = block_reduce_sum(ll, s_red);
  const float Zt = block_reduce_sum(tl, s_red);  // ends with a barrier: s_w is visible
  const float inv_l = 1.f / Lr;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float o = 0.f;
    const float* po = p.po + slot0 * D + d;
    for (int s = 0; s < nsplit; ++s) o += po[(size_t)s * D] * s_w[s];
    store_out<T>(out + d, o * inv_l);
  }
  if (threadIdx.x == 0) {
    if (p.mz) p.mz[b * p.Hq + h] = make_float2(M, 1.f / Z);
    if (p.text_mass) p.text_mass[b * p.Hq + h] = Zt / Z;
  }
}

// ---------------------------------------------------------------------------
// head-summed image-token scores
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void score_kernel(ScoreParams p) {
  __shared__ float2 s_mz[128];
  const int b = blockIdx.y;
  for (int h = threadIdx.x; h < p.Hq; h += blockDim.x) s_mz[h] = p.mz[b * p.Hq + h];
  __syncthreads();
  int n, len;
  seq_extent(p.lens, b, p.S, p.n_cap, n, len);
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  const float* lg = p.logits + (size_t)b * p.Hq * p.n_stride + j;
  float s = 0.f;
  for (int h = 0; h < p.Hq; ++h) s += exp2f(lg[(size_t)h * p.n_stride] - s_mz[h].x) * s_mz[h].y;
  p.scores[(size_t)b * p.n_stride + j] = s;
}

// ---------------------------------------------------------------------------
// top-k selection
// ---------------------------------------------------------------------------

// k = clamp(ceil(tau*n - 1e-9), 1, n); the products and differences are
// rounded one operation at a time so host and device agree bit for bit.
__device__ __forceinline__ int device_kept_count(double tau, int n) {
  if (n <= 0) return 0;
  const double prod = __dmul_rn(tau, (double)n);
  const double k = ceil(__dadd_rn(prod, -1e-9));
  int ki = (int)k;
  return min(max(ki, 1), n);
}

constexpr int kTopkThreads = 1024;

// Exclusive prefix count of `flag` over the workgroup in thread order, using
// wave ballots; returns the prefix and stores the workgroup total in *total.
__device__ __forceinline__ int block_exclusive_count(bool flag, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long m = __ballot(flag);
  const int below = __popcll(m & ((1ull << lane) - 1ull));
  __syncthreads();
  if (lane == 0) s_wave[wave] = __popcll(m);
  __syncthreads();
  int before = 0, all = 0;
  const int nw = blockDim.x >> 6;
  for (int w = 0; w < nw; ++w) {
    const int c = s_wave[w];
    before += (w < wave) ? c : 0;
    all += c;
  }
  *total = all;
  return before + below;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  __shared__ unsigned int s_hist[256];
  __shared__ unsigned int s_prefix;
  __shared__ int s_remaining;
  __shared__ int s_wave[kTopkThreads / 64];
  const int b = blockIdx.x;
  const int n0 = p.lens[2 * b];
  const int n = min(max(n0, 0), min(max(p.lens[2 * b + 1], 0), p.n_cap));
  if (n0 != n && threadIdx.x == 0 && p.status) atomicOr(p.status, FASTOCR_FLAG_LENS_CLAMPED);
  const int k = min(device_kept_count(p.tau, n), p.idx_stride);
  if (threadIdx.x == 0) p.cnt[b] = k;
  if (k == 0) return;
  const unsigned int* keys = reinterpret_cast<const unsigned int*>(p.scores) + (size_t)b * p.score_stride;
  int32_t* out = p.idx + (size_t)b * p.idx_stride;

  // Radix select of the k-th largest key, 8 bits per pass from the top.  For
  // non-negative floats the IEEE bit pattern orders like the value.
  unsigned int prefix = 0u, mask = 0u;
  int remaining = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = threadIdx.x; i < 256; i += blockDim.x) s_hist[i] = 0u;
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += blockDim.x) {
      const unsigned int key = keys[j];
      if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      const int lane = threadIdx.x;
      unsigned int c[4], sum = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = s_hist[255 - 4 * lane - i];
        sum += c[i];
      }
      unsigned int incl = sum;
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      unsigned int above = incl - sum;  // keys with a larger digit
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (above < (unsigned int)remaining && (unsigned int)remaining <= above + c[i]) {
          s_prefix = prefix | ((unsigned int)(255 - 4 * lane - i) << shift);
          s_remaining = remaining - (int)above;
        }
        above += c[i];
      }
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    mask |= 255u << shift;
    __syncthreads();
  }
  const unsigned int theta = prefix;  // k-th largest key
  const int need_eq = remaining;      // keys equal to theta to take, lowest index first

  int out_base = 0, eq_base = 0;
  for (int base = 0; base < n; base += blockDim.x) {
    const int j = base + threadIdx.x;
    const unsigned int key = (j < n) ? keys[j] : 0u;
    const bool gt = (j < n) && key > theta;
    const bool eq = (j < n) && key == theta;
    int eq_total, keep_total;
    const int eq_rank = eq_base + block_exclusive_count(eq, s_wave, &eq_total);
    const bool keep = gt || (eq && eq_rank < need_eq);
    const int pos = out_base + block_exclusive_count(keep, s_wave, &keep_total);
    if (keep) out[pos] = j;
    eq_base += eq_total;
    out_base += keep_total;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <typename T, int D>
static hipError_t launch_split_t(SplitKind kind, const SplitParams& p, hipStream_t stream) {
  dim3 grid(p.grid_splits, p.Hkv, p.B), block(kSplitWaves * 64);
  switch (kind) {
    case KIND_FULL: split_attn_kernel<T, D, KIND_FULL><<<grid, block, 0, stream>>>(p); break;
    case KIND_FOCAL: split_attn_kernel<T, D, KIND_FOCAL><<<grid, block, 0, stream>>>(p); break;
    case KIND_SPARSE: split_attn_kernel<T, D, KIND_SPARSE><<<grid, block, 0, stream>>>(p); break;
  }
  return hipGetLastError();
}

hipError_t launch_split(int dtype, int head_dim, SplitKind kind, const SplitParams& p,
                        hipStream_t stream) {
  if (dtype == FASTOCR_DTYPE_BF16)
    return head_dim == 128 ? launch_split_t<uint16_t, 128>(kind, p, stream)
                           : launch_split_t<uint16_t, 64>(kind, p, stream);
  return head_dim == 128 ? launch_split_t<float, 128>(kind, p, stream)
                         : launch_split_t<float, 64>(kind, p, stream);
}

hipError_t launch_combine(int dtype, int head_dim, const CombineParams& p, hipStream_t stream) {
  dim3 grid(p.Hq, p.B), block(128);
  if (dtype == FASTOCR_DTYPE_BF16) {
    if (head_dim == 128) combine_kernel<uint16_t, 128><<<grid, block, 0, stream>>>(p);
    else combine_kernel<uint16_t, 64><<<grid, block, 0, stream>>>(p);
  } else {
    if (head_dim == 128) combine_kernel<float, 128><<<grid, block, 0, stream>>>(p);
    else combine_kernel<float, 64><<<grid, block, 0, stream>>>(p);
  }
  return hipGetLastError();
}

hipError_t launch_score(const ScoreParams& p, hipStream_t stream) {
  dim3 grid((p.n_stride + 255) / 256, p.B), block(256);
  score_kernel<<<grid, block, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkParams& p, hipStream_t stream) {
  topk_kernel<<<dim3(p.B), dim3(kTopkThreads), 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace fastocr
