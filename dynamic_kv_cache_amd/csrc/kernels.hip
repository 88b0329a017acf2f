// gfx950 kernels of the FastOCR decode-step attention path.
//
// Method source: "FastOCR: Dynamic Visual Fixation via KV Cache Pruning for
// Efficient Document Parsing", technical summary, Method / 1. Focal-Guided
// Pruning (Focal Layer Selection, Cross-Layer Propagation) and 2. Cross-Step
// Fixation Reuse; the paper's abstract.
//
// Kernels
//   split_attn_kernel  split-K decode attention of one (sequence, KV head)
//                      over one chunk of consecutive rows per workgroup, in
//                      two kinds: all rows (warm-up, FULL mode, tau = 1), and
//                      all rows + the image-token logit export (focal
//                      layers; staged in LDS for long splits).  Writes one
//                      partial softmax state per split.
//   kept_attn_kernel   attention of one (sequence, KV head) over its kept
//                      image rows, gathered by index, and every text row
//                      (non-focal layers): the pair's 16-row tiles dealt
//                      round-robin to its workgroups.  Writes one state per
//                      workgroup, or the output when a pair has one.
//   merge_kernel       one workgroup per head merges the split states into
//                      the output (and the head's text-probability mass);
//                      for focal layers, score workgroups compute the
//                      head-summed probability of every image token.
//   kept_merge_kernel  the merge of a kept-token pass (at most 64 states per
//                      head, no text mass, no scores).
//   topk_kernel        the k_b highest scores per sequence, ties to the lower
//                      index, ascending output.
//   pack_rows_kernel   one-time image-first gather of a multi-span cache.
// Workgroups never wait on each other inside a kernel: on this GPU a device
// fence plus an arrival atomic, or the same chain kept inside one XCD's L2,
// costs as much as the next kernel launch or more.
//
// Placement and caching.  Block i runs on XCD i mod 8; the kept-token pass
// and its merge pad their pair dimension to a multiple of 8, so a pair's
// blocks and the merge of its heads share one XCD and its L2.  In pruned
// steps the kept-token and focal-layer passes load their K/V rows
// non-temporally when a step's kept rows exceed the last-level cache, which
// then keeps the kept indices, merge states and focal logits instead.
//
// Matrix layout on the MFMA units.  A wave consumes 16 cache rows per tile.
// The GQA query group of one KV head (up to 16 heads, zero padded) is the N
// side of a 16x16 MFMA tile:
//   logits^T[16 rows x 16 heads]  = K_tile[16 x d] * Q^T[d x 16]
//   out^T   [16 d     x 16 heads] += V_tile^T[16 d x 16 rows] * P^T[16 rows x 16 heads]
// Because a contraction may visit its index in any order, the d index is
// permuted so every lane's operands come straight from global memory with
// no LDS transpose:
//   QK: lane (c = lane%16, g = lane/16) loads the 16-byte pieces i*4 + g of
//       K[row c] (so the 4 lane groups read 64 contiguous bytes per load)
//       and the same pieces of its query head c; MFMA number kk contracts
//       elements kk*4..kk*4+3 of those slices (bf16 16x16x16) or element kk
//       (fp32 16x16x4).
//   PV: lane (c, g) loads rows 4g..4g+3 of the tile, each the contiguous
//       slice [c*d/16, (c+1)*d/16); MFMA number db uses element db of each
//       row, so output lane (c, g) ends up holding head c's outputs for
//       d = (4g+i)*(d/16) + db, i.e. the contiguous range [g*d/4, (g+1)*d/4).
// The logits come out as lane (c, g) = head c, rows 4g..4g+3, which is
// exactly the P^T operand the PV product needs, so softmax stays in
// registers.  A wave issues the loads of all its tiles of a round (up to 4)
// before computing any, and rescales its running softmax state once per
// round.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "../../include/fastocr.h"
#include "internal.h"

namespace fastocr {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Two 32-bit words holding bf16 pairs, as an MFMA bf16x4 operand (no data
// movement).
__device__ __forceinline__ bf16x4_t as_bf16x4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(bf16x4_t, u32x2_t{lo, hi});
}
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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

// This lane's slice of a K row (or of its query row): 16-byte pieces
// i*4 + grp of the row, i = 0 .. KW/4 - 1.  The four lane groups of a column
// therefore read 64 contiguous bytes per load instruction.
template <typename T, int KW>
__device__ __forceinline__ void load_slice(uint32_t* dst, const T* row, int grp) {
  constexpr int PIECE = 16 / (int)sizeof(T);  // elements per 16-byte piece
#pragma unroll
  for (int i = 0; i < KW / 4; ++i) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + (i * 4 + grp) * PIECE);
    dst[4 * i] = v.x;
    dst[4 * i + 1] = v.y;
    dst[4 * i + 2] = v.z;
    dst[4 * i + 3] = v.w;
  }
}

// Streaming forms of load_slice / load_words (non-temporal loads).
template <typename T, int KW>
__device__ __forceinline__ void load_slice_nt(uint32_t* dst, const T* row, int grp) {
  constexpr int PIECE = 16 / (int)sizeof(T);
#pragma unroll
  for (int i = 0; i < KW / 4; ++i) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + (i * 4 + grp) * PIECE));
    dst[4 * i] = v[0];
    dst[4 * i + 1] = v[1];
    dst[4 * i + 2] = v[2];
    dst[4 * i + 3] = v[3];
  }
}

template <typename T>
__device__ __forceinline__ void load_words_nt(uint32_t* dst, const T* src, int nwords) {
  const uint32_t* s = reinterpret_cast<const uint32_t*>(src);
  if ((nwords & 3) == 0) {
#pragma unroll
    for (int i = 0; i < nwords; i += 4) {
      const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(s + i));
      dst[i] = v[0]; dst[i + 1] = v[1]; dst[i + 2] = v[2]; dst[i + 3] = v[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < nwords; i += 2) {
      const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(s + i));
      dst[i] = v[0]; dst[i + 1] = v[1];
    }
  }
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

// ---------------------------------------------------------------------------
// wave and workgroup primitives (DPP row shifts and row broadcasts)
// ---------------------------------------------------------------------------
// These kernels run once per launch on CUs whose instruction cache is cold,
// so they are written as short loops rather than long unrolled sequences.

#define FASTOCR_DPP(old, x, ctrl, rmask) __builtin_amdgcn_update_dpp((old), (x), (ctrl), (rmask), 0xf, false)

// Inclusive prefix sum over the 64 lanes of a wave: scans within each
// 16-lane row (row_shr 1, 2, 4, 8), then carries row totals with
// row_bcast:15 (into rows 1 and 3) and row_bcast:31 (into rows 2 and 3).
__device__ __forceinline__ unsigned int wave_incl_scan(unsigned int x) {
  x += (unsigned int)FASTOCR_DPP(0, (int)x, 0x111, 0xf);
  x += (unsigned int)FASTOCR_DPP(0, (int)x, 0x112, 0xf);
  x += (unsigned int)FASTOCR_DPP(0, (int)x, 0x114, 0xf);
  x += (unsigned int)FASTOCR_DPP(0, (int)x, 0x118, 0xf);
  x += (unsigned int)FASTOCR_DPP(0, (int)x, 0x142, 0xa);
  x += (unsigned int)FASTOCR_DPP(0, (int)x, 0x143, 0xc);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  x += __int_as_float(FASTOCR_DPP(0, __float_as_int(x), 0x111, 0xf));
  x += __int_as_float(FASTOCR_DPP(0, __float_as_int(x), 0x112, 0xf));
  x += __int_as_float(FASTOCR_DPP(0, __float_as_int(x), 0x114, 0xf));
  x += __int_as_float(FASTOCR_DPP(0, __float_as_int(x), 0x118, 0xf));
  x += __int_as_float(FASTOCR_DPP(0, __float_as_int(x), 0x142, 0xa));
  x += __int_as_float(FASTOCR_DPP(0, __float_as_int(x), 0x143, 0xc));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

__device__ __forceinline__ float wave_max(float x) {
  int v = __float_as_int(x);
  x = fmaxf(x, __int_as_float(FASTOCR_DPP(v, v, 0x111, 0xf))); v = __float_as_int(x);
  x = fmaxf(x, __int_as_float(FASTOCR_DPP(v, v, 0x112, 0xf))); v = __float_as_int(x);
  x = fmaxf(x, __int_as_float(FASTOCR_DPP(v, v, 0x114, 0xf))); v = __float_as_int(x);
  x = fmaxf(x, __int_as_float(FASTOCR_DPP(v, v, 0x118, 0xf))); v = __float_as_int(x);
  x = fmaxf(x, __int_as_float(FASTOCR_DPP(v, v, 0x142, 0xa))); v = __float_as_int(x);
  x = fmaxf(x, __int_as_float(FASTOCR_DPP(v, v, 0x143, 0xc))); v = __float_as_int(x);
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
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

struct TopkShared {
  // keys staged from coalesced loads: thread t's keys [t*per, t*per + per)
  // at [t*(per+1), ...), padded so the per-thread reads hit distinct banks
  unsigned int stage[kTopkThreads * (kTopkRegKeys + 1)];
  unsigned int hist[kTopkThreads / 64][256];  // one histogram per wave
  alignas(16) unsigned int wave_sum[kTopkThreads / 64];
  alignas(16) unsigned int wave_sum2[kTopkThreads / 64];
  unsigned int cand_key[kTopkCand];
  int cand_idx[kTopkCand];
  unsigned int prefix;
  int remaining;
  int bin_count;
  int ncand;
  unsigned int theta;
  int need_eq;
};

// Append (key, index) to the candidate list if the key lies in the k-th
// key's bin (one LDS atomic per wave).
__device__ __forceinline__ void gather_key(unsigned int key, bool valid, int index, unsigned int mask,
                                           unsigned int prefix, TopkShared& sh, int lane) {
  const bool take = valid && (key & mask) == prefix;
  const unsigned long long tm = __ballot(take);
  if (tm == 0ull) return;
  const int leader = __ffsll((unsigned long long)tm) - 1;
  int slot0 = 0;
  if (lane == leader) slot0 = atomicAdd(&sh.ncand, __popcll(tm));
  slot0 = __builtin_amdgcn_readlane(slot0, leader);
  if (take) {
    const int slot = slot0 + __popcll(tm & ((1ull << lane) - 1ull));
    sh.cand_key[slot] = key;
    sh.cand_idx[slot] = index;
  }
}

// Count one key into this wave's histogram of digit (key >> shift) & 255,
// if its higher digits match `prefix` under `mask`.  Keys of one wave mostly
// share their leading digits, so lanes with the first pending lane's digit
// are counted by one atomic; the remaining lanes add one each.  (Repeating
// the aggregation for further digits measured slower.)
__device__ __forceinline__ void hist_key(unsigned int key, bool valid, int shift, unsigned int mask,
                                         unsigned int prefix, unsigned int* hist, int lane) {
  const unsigned int dig = (key >> shift) & 255u;
  const bool pending = valid && (key & mask) == prefix;
  const unsigned long long pm = __ballot(pending);
  if (pm != 0ull) {
    const int leader = __ffsll((unsigned long long)pm) - 1;
    const unsigned int ld = (unsigned int)__builtin_amdgcn_readlane((int)dig, leader);
    const bool same = pending && dig == ld;
    const unsigned long long sm = __ballot(same);
    if (lane == leader) atomicAdd(&hist[ld], (unsigned int)__popcll(sm));
    if (pending && !same) atomicAdd(&hist[dig], 1u);
  }
}

// Sum of the first `wave` entries of a per-wave array of kTopkThreads / 64
// values, read as 128-bit words.
__device__ __forceinline__ unsigned int sum_before(const unsigned int* v, int wave) {
  unsigned int acc = 0;
#pragma unroll
  for (int q = 0; q < kTopkThreads / 256; ++q) {
    const uint4 w = reinterpret_cast<const uint4*>(v)[q];
    acc += (4 * q + 0 < wave ? w.x : 0u) + (4 * q + 1 < wave ? w.y : 0u) + (4 * q + 2 < wave ? w.z : 0u) +
           (4 * q + 3 < wave ? w.w : 0u);
  }
  return acc;
}

// Top-k of the non-negative float keys[0, n) by one kTopkThreads workgroup.
// Thread t owns keys [t*per, t*per + per) of the row's capacity n_cap >= n.
// With PER > 0 they are held in registers (per = PER, a power of two up to
// kTopkRegKeys): loaded coalesced (key tid + i * kTopkThreads) before n and
// k are known, and moved to their owners through LDS when a pass first needs
// them.  With PER = 0 they are re-read from memory per pass.  A 4-pass
// radix select (8 bits per pass, most significant first; the IEEE bits of a
// non-negative float order like its value) finds the k-th largest key theta
// and how many keys equal to theta are kept; one workgroup prefix sum then
// places every kept index, so the output is in ascending index order and
// ties at theta go to the lowest indices.
template <int PER>
__device__ void block_topk(const unsigned int* __restrict__ keys, int per, int n, int k,
                           int32_t* __restrict__ out, TopkShared& sh, unsigned int (&reg)[PER > 0 ? PER : 1],
                           bool have_c0, unsigned int c0) {
  constexpr bool IN_REGS = PER > 0;
  constexpr int R = IN_REGS ? PER : 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (IN_REGS) per = PER;
  const int base = tid * per;
  const int mine = max(0, min(per, n - base));
  // in-register keys: load order -> owners (thread t's keys at
  // stage[t*(PER+1) ...], padded so the owners' reads hit distinct banks)
  bool staged = !IN_REGS;
  auto stage_write = [&]() {
    constexpr int LP = __builtin_ctz((unsigned int)R);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int j = tid + i * kTopkThreads;
      sh.stage[(j >> LP) * (R + 1) + (j & (R - 1))] = reg[i];
    }
  };
  auto stage_read = [&]() {  // after a barrier
#pragma unroll
    for (int i = 0; i < R; ++i) reg[i] = sh.stage[tid * (R + 1) + i];
    staged = true;
  };

  unsigned int prefix = 0u, mask = 0u;
  int remaining = k;
  bool ranked = false;
  if (tid == 0) sh.ncand = 0;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    // the first digit's counts may come with the scores (thread t < 256
    // holds digit 255 - t): then the first pass builds no histogram
    const bool from_c0 = pass == 0 && have_c0;
    if (!from_c0) {
      if (IN_REGS && !staged) stage_write();
      for (int i = tid; i < (kTopkThreads / 64) * 256; i += kTopkThreads) (&sh.hist[0][0])[i] = 0u;
      __syncthreads();
      if (IN_REGS && !staged) stage_read();
      if constexpr (IN_REGS) {
#pragma unroll
        for (int i = 0; i < R; ++i) hist_key(reg[i], i < mine, shift, mask, prefix, sh.hist[wave], lane);
      } else {
#pragma unroll 1
        for (int i = 0; i < per; ++i)
          hist_key(keys[min(base + i, n - 1)], i < mine, shift, mask, prefix, sh.hist[wave], lane);
      }
      __syncthreads();
    }
    // thread t < 256 owns digit 255 - t: inclusive count in descending digit order
    unsigned int c = 0, incl = 0;
    if (tid < 256) {
      if (from_c0) {
        c = c0;
      } else {
        for (int w = 0; w < kTopkThreads / 64; ++w) c += sh.hist[w][255 - tid];
      }
      incl = wave_incl_scan(c);
      if (lane == 63) sh.wave_sum[wave] = incl;
    }
    __syncthreads();
    if (tid < 256) {
      incl += sum_before(sh.wave_sum, wave);
      const unsigned int above = incl - c;  // keys with a larger digit
      if (above < (unsigned int)remaining && (unsigned int)remaining <= incl) {
        sh.prefix = prefix | ((unsigned int)(255 - tid) << shift);
        sh.remaining = remaining - (int)above;
        sh.bin_count = (int)c;
      }
    }
    __syncthreads();
    prefix = sh.prefix;
    remaining = sh.remaining;
    mask |= 255u << shift;
    if (pass < 3 && sh.bin_count <= kTopkCand) {
      ranked = true;
      break;
    }
  }

  if (IN_REGS && !staged) {
    stage_write();
    __syncthreads();
    stage_read();
  }
  if (ranked) {
    // The k-th key's bin is small: gather it and rank its keys pairwise by
    // (value descending, index ascending); the key of rank remaining - 1 is
    // theta.
    if constexpr (IN_REGS) {
#pragma unroll
      for (int i = 0; i < R; ++i) gather_key(reg[i], i < mine, base + i, mask, prefix, sh, lane);
    } else {
#pragma unroll 1
      for (int i = 0; i < per; ++i)
        gather_key(keys[min(base + i, n - 1)], i < mine, base + i, mask, prefix, sh, lane);
    }
    __syncthreads();
    // lane c of every wave holds candidate c; wave w compares it with
    // candidates [w*CPW, (w+1)*CPW) (broadcast LDS reads) and leaves the
    // two partial counts, packed, in the histogram area (free by now)
    constexpr int NWV = kTopkThreads / 64;
    constexpr int CPW = (kTopkCand + NWV - 1) / NWV;
    const int nc = sh.ncand;
    const unsigned int kc = lane < nc ? sh.cand_key[lane] : 0u;
    const int ic = lane < nc ? sh.cand_idx[lane] : 0;
    int greater = 0, before = 0;
#pragma unroll
    for (int jj = 0; jj < CPW; ++jj) {
      const int j = wave * CPW + jj;
      if (j < nc) {  // uniform over the wave
        const unsigned int kj = sh.cand_key[j];
        const int ij = sh.cand_idx[j];
        greater += kj > kc ? 1 : 0;
        before += (kj == kc && ij < ic) ? 1 : 0;
      }
    }
    unsigned int* part = &sh.hist[0][0];  // [NWV][64]
    part[wave * 64 + lane] = (unsigned int)greater | ((unsigned int)before << 16);
    __syncthreads();
    if (wave == 0 && lane < nc) {
      unsigned int acc = 0;
#pragma unroll
      for (int w = 0; w < NWV; ++w) acc += part[w * 64 + lane];
      const int g = (int)(acc & 0xffffu), bf = (int)(acc >> 16);
      if (g + bf == remaining - 1) {
        sh.theta = kc;
        sh.need_eq = remaining - g;
      }
    }
  } else if (tid == 0) {
    // every digit fixed: the remaining keys all equal theta
    sh.theta = prefix;
    sh.need_eq = remaining;
  }
  __syncthreads();
  const unsigned int theta = sh.theta;  // k-th largest key
  const int need_eq = sh.need_eq;       // keys equal to theta to keep, lowest index first

  unsigned int gt = 0, eq = 0;
  if constexpr (IN_REGS) {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      gt += (i < mine && reg[i] > theta) ? 1u : 0u;
      eq += (i < mine && reg[i] == theta) ? 1u : 0u;
    }
  } else {
#pragma unroll 1
    for (int i = 0; i < mine; ++i) {
      const unsigned int key = keys[base + i];
      gt += key > theta ? 1u : 0u;
      eq += key == theta ? 1u : 0u;
    }
  }
  // exclusive prefix sums of both counts over the workgroup (wave_sum was
  // last read before the barrier above)
  unsigned int gt_incl = wave_incl_scan(gt);
  unsigned int eq_incl = wave_incl_scan(eq);
  if (lane == 63) {
    sh.wave_sum[wave] = gt_incl;
    sh.wave_sum2[wave] = eq_incl;
  }
  __syncthreads();
  gt_incl += sum_before(sh.wave_sum, wave);
  eq_incl += sum_before(sh.wave_sum2, wave);
  int eq_seen = (int)(eq_incl - eq);
  int pos = (int)(gt_incl - gt) + min(eq_seen, need_eq);
  if constexpr (IN_REGS) {
    // kept indices land in LDS (the staging area, free by now) and leave in
    // one coalesced copy
    int* kept = reinterpret_cast<int*>(sh.stage);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const bool valid = i < mine;
      const bool gt_i = valid && reg[i] > theta;
      const bool eq_i = valid && reg[i] == theta;
      const bool keep = gt_i || (eq_i && eq_seen < need_eq);
      if (keep) kept[pos] = base + i;
      pos += keep ? 1 : 0;
      eq_seen += eq_i ? 1 : 0;
    }
    __syncthreads();
    for (int i = tid; i < k; i += kTopkThreads) out[i] = kept[i];
  } else {
#pragma unroll 1
    for (int i = 0; i < mine; ++i) {
      const unsigned int key = keys[base + i];
      if (key > theta) {
        out[pos++] = base + i;
      } else if (key == theta) {
        if (eq_seen < need_eq) out[pos++] = base + i;
        ++eq_seen;
      }
    }
  }
}

// Top-k of one sequence's scores.  The sequence extent is read first (no
// store precedes it, so it can come through the scalar cache), then the
// first digit's counts and the keys this thread loads, all before k is known.
template <int PER>
__device__ __forceinline__ void topk_sequence(const float* scores, int n_cap, const int32_t* lens, int b,
                                              double tau, int idx_stride, int32_t* out, int32_t* cnt,
                                              int32_t* status, unsigned int* hist0, TopkShared& sh) {
  constexpr int R = PER > 0 ? PER : 1;
  const unsigned int* keys = reinterpret_cast<const unsigned int*>(scores);
  const int tid = threadIdx.x;
  const int n0 = lens[2 * b];
  const int l0 = lens[2 * b + 1];
  // the first digit's counts (thread t < 256: digit 255 - t) are the first
  // thing the select needs; every thread issues one load (no branch, so the
  // wait for it does not also wait for the keys)
  const unsigned int* c0_src = hist0 ? hist0 + (255 - (tid & 255)) : keys;
  unsigned int c0 = *c0_src;
  unsigned int reg[R];
  if constexpr (PER > 0) {
#pragma unroll
    for (int i = 0; i < R; ++i) reg[i] = keys[min(tid + i * kTopkThreads, n_cap - 1)];
  }
  const int n = min(max(n0, 0), min(max(l0, 0), n_cap));
  if (n0 != n && tid == 0 && status) atomicOr(status, FASTOCR_FLAG_LENS_CLAMPED);
  const int k = min(device_kept_count(tau, n), idx_stride);
  if (tid == 0) *cnt = k;
  // cleared for the next focal layer (this thread's own load of it is older)
  if (hist0 && tid < 256) hist0[255 - tid] = 0u;
  if (k == 0) return;
  const int per = (n_cap + kTopkThreads - 1) / kTopkThreads;
  block_topk<PER>(keys, per, n, k, out, sh, reg, hist0 != nullptr, tid < 256 ? c0 : 0u);
}

// ---------------------------------------------------------------------------
// split-K decode attention
// ---------------------------------------------------------------------------

// Full-cache passes (warm-up, focal layers, the FULL baseline): each
// workgroup streams one split of rows_per_split consecutive rows of one
// (sequence, KV head) pair in 128-row rounds, double-buffered (the next
// round's loads are issued before the current round is computed), and
// writes one merge state per split.
// STREAM: the K/V rows are loaded non-temporally, which pruned steps do when
// one step's kept rows exceed the last-level cache (the logits written here
// and read by the merge, and the kept indices and states of the layers
// around, then stay cached).
template <typename T, int D, int KIND, int NW, int TPW, bool STREAM>
__global__ __launch_bounds__(NW * 64, 2) void split_attn_kernel(SplitParams p) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int NT = NW * 64;                   // threads
  constexpr int RPR = NW * TPW * kTileRows;     // rows per round
  constexpr int E = D / 4;                      // K/q elements per lane
  constexpr int KW = E * (int)sizeof(T) / 4;    // ... as 32-bit words
  constexpr int NDB = D / 16;                   // PV d-blocks = V elements per row per lane
  constexpr int VW = NDB * (int)sizeof(T) / 4;  // V words per row per lane
  constexpr int HH = 8;                         // heads per LDS merge round
  constexpr int OST = D + 4;                    // padded LDS row of partial outputs (16-byte aligned)

  __shared__ float s_stat[NW][16][4];
  // the wave combine's partial outputs, and before them (focal kind) the
  // split's staged image-token logits
  constexpr int ON = NW * HH * OST;
  constexpr int POOL = (KIND == KIND_FOCAL && kLogitStageFloats > ON) ? kLogitStageFloats : ON;
  __shared__ __align__(16) float s_pool[POOL];
  float (*s_o)[HH][OST] = reinterpret_cast<float (*)[HH][OST]>(s_pool);
  static_assert(KIND == KIND_FULL || KIND == KIND_FOCAL, "kept-token passes run kept_attn_kernel");

  // x = split, y = (sequence, KV head) pair, so workgroups dispatched
  // together stream neighbouring rows
  const int pair = blockIdx.y;
  const int split = blockIdx.x;
  const int kvh = pair % p.Hkv;
  const int b = pair / p.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: tile rows stay scalar
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int G = p.Hq / p.Hkv;

  const int begin = split * p.rows_per_split;
  const size_t row_base = ((size_t)b * p.Hkv + kvh) * (size_t)p.S;
  const T* __restrict__ Kb = reinterpret_cast<const T*>(p.k) + row_base * D;
  const T* __restrict__ Vb = reinterpret_cast<const T*>(p.v) + row_base * D;

  // Loads that do not depend on the sequence extent are issued before it is
  // read, so they are in flight together: the query slice and the first
  // round's K/V rows.  Any row below S lies inside the cache allocation; rows
  // past the extent get zero weight and their V values are zeroed once it is
  // known.
  uint32_t qw[KW];
  if (col < G) {
    const T* qp = reinterpret_cast<const T*>(p.q) + ((size_t)b * p.Hq + kvh * G + col) * D;
    load_slice<T, KW>(qw, qp, grp);
  } else {
#pragma unroll
    for (int i = 0; i < KW; ++i) qw[i] = 0u;
  }
  const int r_first = begin + wave * kTileRows;  // this wave's first tile row
  uint32_t kw[TPW][KW];
  uint32_t vw[TPW][4][VW];
  // Splits below sure_splits hold rows for every sequence the handle
  // accepts: they load ahead.  The others may be empty and learn that
  // from the extent before loading anything.
  // The first round's tiles all lie in the split's rows (a split is at least
  // one round), so they load without a condition (rows clamped to the cache;
  // a tile past its end is never weighted): a per-tile condition made the
  // compiler wait for one tile's K before issuing the next tile's loads.
  const bool ahead = split < p.sure_splits;
  if (ahead) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tile = r_first + u * NW * kTileRows;
      if constexpr (STREAM) load_slice_nt<T, KW>(kw[u], Kb + (size_t)min(tile + col, p.S - 1) * D, grp);
      else load_slice<T, KW>(kw[u], Kb + (size_t)min(tile + col, p.S - 1) * D, grp);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if constexpr (STREAM) load_words_nt(vw[u][j], Vb + (size_t)min(tile + 4 * grp + j, p.S - 1) * D + col * NDB, VW);
        else load_words(vw[u][j], Vb + (size_t)min(tile + 4 * grp + j, p.S - 1) * D + col * NDB, VW);
    }
  }

  int n, len;
  const bool clamped = seq_extent(p.lens, b, p.S, p.n_cap, n, len);
  const bool reporter = split == 0 && kvh == 0 && tid == 0;

  // Fused append: the current token (cache row len - 1) comes from k_new /
  // v_new in every load of this launch, and split 0 of the pair writes it
  // into the caches for later steps (no workgroup of this launch reads that
  // cache row).
  const int cur = len - 1;
  const bool app = p.k_new != nullptr && len > 0;
  const T* __restrict__ knew = app ? reinterpret_cast<const T*>(p.k_new) + ((size_t)b * p.Hkv + kvh) * D : nullptr;
  const T* __restrict__ vnew = app ? reinterpret_cast<const T*>(p.v_new) + ((size_t)b * p.Hkv + kvh) * D : nullptr;
  if (app && split == 0) {
    constexpr int C16 = D * (int)sizeof(T) / 16;  // 16-byte pieces per row
    T* kc = reinterpret_cast<T*>(p.k_w) + (row_base + cur) * D;
    T* vc = reinterpret_cast<T*>(p.v_w) + (row_base + cur) * D;
    if (tid < C16) reinterpret_cast<uint4*>(kc)[tid] = reinterpret_cast<const uint4*>(knew)[tid];
    else if (tid < 2 * C16) reinterpret_cast<uint4*>(vc)[tid - C16] = reinterpret_cast<const uint4*>(vnew)[tid - C16];
  }
  if (app && ahead) {
    // a full pass loaded this wave's first-round rows before the extent was
    // known: the current token's row, if among them, is reloaded from
    // k_new / v_new
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tile = r_first + u * NW * kTileRows;
      if (tile <= cur && cur < tile + kTileRows) {  // uniform over the wave
        if (tile + col == cur) load_slice<T, KW>(kw[u], knew, grp);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (tile + 4 * grp + j == cur) load_words(vw[u][j], vnew + col * NDB, VW);
      }
    }
  }
  if (clamped && reporter) atomicOr(p.status, FASTOCR_FLAG_LENS_CLAMPED);
  const int rows = len;
  if (begin >= rows) {
    // an empty split: a state that carries no weight in the merge
    for (int i = tid; i < G; i += NT)
      p.pstat[((size_t)b * p.Hq + kvh * G + i) * p.max_splits + split] = make_float4(-INFINITY, 0.f, 0.f, 0.f);
    return;
  }
  const int end = min(begin + p.rows_per_split, rows);

  const int lg_stride = p.rows_per_split + kLogitStagePad;  // staged logits per head (LDS)
  const bool stage = KIND == KIND_FOCAL && p.stage_logits && G * lg_stride <= kLogitStageFloats;
  float m_run = -INFINITY, z = 0.f, lsum = 0.f, zt = 0.f;
  f32x4_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // One round: rows [r0, r0 + RPR) of this wave's tiles, whose K/V words
  // are in kw / vw.
  auto round = [&](int r0, uint32_t (&kw)[TPW][KW], uint32_t (&vw)[TPW][4][VW]) {
    // V rows past the end of the split carry zero weight: zero them so that
    // whatever the cache holds there cannot turn 0 * v into NaN
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = r0 + u * NW * kTileRows + 4 * grp + j < end;
#pragma unroll
        for (int w = 0; w < VW; ++w) vw[u][j][w] = ok ? vw[u][j][w] : 0u;
      }

    // ---- logits^T = K_tile * Q^T for every tile of the round
    float x[TPW][4];
    float mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tile = r0 + u * NW * kTileRows;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[u][i] = -INFINITY;
      if (tile >= end) continue;
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (BF) {
#pragma unroll
        for (int kk = 0; kk < E / 4; ++kk) {
          s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_bf16x4(kw[u][2 * kk], kw[u][2 * kk + 1]),
                                                        as_bf16x4(qw[2 * kk], qw[2 * kk + 1]), s, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < E; ++kk)
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kw[u][kk]), __uint_as_float(qw[kk]), s,
                                                   0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = tile + 4 * grp + i;
        x[u][i] = (r < end) ? s[i] * p.scale_log2 : -INFINITY;
        mt = fmaxf(mt, x[u][i]);
      }
      if constexpr (KIND == KIND_FOCAL) {
        // this lane's 4 logits are consecutive image rows of one head: one
        // 16-byte store (rows are a multiple of 4, n_stride too), into LDS
        // when staged (rows past the image rows are never written out)
        if (col < G) {
          float* lg = p.logits + ((size_t)b * p.Hq + kvh * G + col) * p.n_stride;
          const int r = tile + 4 * grp;
          const int lim = min(end, n);
          if (stage) {
            if (r < lim)
              *reinterpret_cast<float4*>(&s_pool[col * lg_stride + (r - begin)]) =
                  make_float4(x[u][0], x[u][1], x[u][2], x[u][3]);
          } else if (r + 3 < lim) {
            *reinterpret_cast<float4*>(lg + r) = make_float4(x[u][0], x[u][1], x[u][2], x[u][3]);
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (r + i < lim) lg[r + i] = x[u][i];
          }
        }
      }
    }

    // ---- online softmax: one rescale per round (per head; the 4 lane
    // groups of a column share the head)
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    z *= alpha;
    lsum *= alpha;
    zt *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    m_run = m_new;

    // ---- out^T += V_tile^T * P^T (rows past `end` have p = 0)
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tile = r0 + u * NW * kTileRows;
      if (tile >= end) continue;
      float pr[4], pu[4];
      uint32_t pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(x[u][i] - m_new);
        if constexpr (BF) {
          pb[i] = f32_to_bf16(pr[i]);
          pu[i] = bf16_to_f32(pb[i]);
        } else {
          pu[i] = pr[i];
        }
        zt += (tile + 4 * grp + i >= n) ? pr[i] : 0.f;
      }
      z += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      lsum += (pu[0] + pu[1]) + (pu[2] + pu[3]);
      if constexpr (BF) {
        const bf16x4_t pv = as_bf16x4(pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          // element db of rows j = 0..3: the low (even db) or high (odd db)
          // halves of word db/2, packed pairwise with v_perm
          const int w = db >> 1;
          const uint32_t sel = (db & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t lo = __builtin_amdgcn_perm(vw[u][1][w], vw[u][0][w], sel);
          const uint32_t hi = __builtin_amdgcn_perm(vw[u][3][w], vw[u][2][w], sel);
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_bf16x4(lo, hi), pv, acc[db], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vw[u][i][db]), pr[i], acc[db],
                                                           0, 0, 0);
      }
    }
  };
  // The K/V loads of the round starting at row r0 (the K row of the lane's
  // column, and its four V rows, per tile).
  auto load_round = [&](int r0, uint32_t (&kw)[TPW][KW], uint32_t (&vw)[TPW][4][VW]) {
    int pk[TPW], pvr[TPW][4];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tile = r0 + u * NW * kTileRows;
      pk[u] = min(tile + col, p.S - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) pvr[u][j] = min(tile + 4 * grp + j, p.S - 1);
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (r0 + u * NW * kTileRows < end) {  // uniform over the wave
        const T* kr = app && pk[u] == cur ? knew : Kb + (size_t)pk[u] * D;
        if constexpr (STREAM) load_slice_nt<T, KW>(kw[u], kr, grp);
        else load_slice<T, KW>(kw[u], kr, grp);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const T* vr = (app && pvr[u][j] == cur ? vnew : Vb + (size_t)pvr[u][j] * D) + col * NDB;
          if constexpr (STREAM) load_words_nt(vw[u][j], vr, VW);
          else load_words(vw[u][j], vr, VW);
        }
      }
    }
  };
  // Round r covers rows [begin + r*RPR, +RPR); tile u of wave w in a round
  // starts at row (u*NW + w)*16, so neighbouring waves read neighbouring
  // tiles.  Rounds alternate between two register buffers; the next round's
  // loads are issued before the current round is computed (the first
  // round's loads are already in flight unless the split loaded nothing
  // ahead).
  if (r_first < end) {
    if (!ahead) load_round(r_first, kw, vw);
    uint32_t kw2[TPW][KW];
    uint32_t vw2[TPW][4][VW];
    for (int r0 = r_first; r0 < end; r0 += 2 * RPR) {
      if (r0 + RPR < end) load_round(r0 + RPR, kw2, vw2);
      round(r0, kw, vw);
      if (r0 + RPR >= end) break;
      if (r0 + 2 * RPR < end) load_round(r0 + 2 * RPR, kw, vw);
      round(r0 + RPR, kw2, vw2);
    }
  }

  if constexpr (KIND == KIND_FOCAL) {
    // staged logits: each head's image rows of the split leave as one
    // contiguous run (stored while K/V streamed in, the 64-byte pieces of
    // every head cost about twice as much)
    if (stage) {
      __syncthreads();
      const int lim = min(end, n) - begin;
      for (int h = 0; h < G; ++h) {
        float* lg = p.logits + ((size_t)b * p.Hq + kvh * G + h) * p.n_stride + begin;
        const float* sl = s_pool + h * lg_stride;
        for (int i = 4 * tid; i < lim; i += 4 * NT) {
          if (i + 3 < lim) {
            *reinterpret_cast<float4*>(lg + i) = *reinterpret_cast<const float4*>(sl + i);
          } else {
            for (int t = i; t < lim; ++t) lg[t] = sl[t];
          }
        }
      }
      __syncthreads();  // s_o reuses the staging buffer
    }
  }

  // ---- per-wave totals (the 4 lane groups of a head hold partial sums)
  z += __shfl_xor(z, 16);
  z += __shfl_xor(z, 32);
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  zt += __shfl_xor(zt, 16);
  zt += __shfl_xor(zt, 32);

  if (grp == 0) {
    s_stat[wave][col][0] = m_run;
    s_stat[wave][col][1] = z;
    s_stat[wave][col][2] = lsum;
    s_stat[wave][col][3] = zt;
  }

  // ---- merge the waves, in rounds of HH heads: every wave leaves its
  // unscaled accumulator in LDS, and the reducing threads weight wave w by
  // exp2(m_w - M) themselves, so one barrier per round suffices
  const size_t slot0 = ((size_t)b * p.Hq + kvh * G) * p.max_splits + split;
  for (int h0 = 0; h0 < G; h0 += HH) {
    if (h0 > 0) __syncthreads();  // the previous round has read s_o
    if (col >= h0 && col < h0 + HH) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_o[wave][col - h0][(4 * grp + i) * NDB + db] = acc[db][i];
    }
    __syncthreads();
    // thread t reduces the 4 consecutive outputs of float4 column t % (D/4)
    // of head t / (D/4) (+ NT/(D/4) heads per further pass)
    const int hn = min(HH, G - h0);
    constexpr int C4 = D / 4;
    for (int idx = tid; idx < hn * C4; idx += NT) {
      const int h = idx / C4;
      const int c4 = idx - h * C4;
      float mw[NW];
      float4 ov[NW];
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        mw[w] = s_stat[w][h0 + h][0];
        ov[w] = *reinterpret_cast<const float4*>(&s_o[w][h][4 * c4]);
        M = fmaxf(M, mw[w]);
      }
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float e = __builtin_amdgcn_exp2f(mw[w] - M);
        o.x += ov[w].x * e;
        o.y += ov[w].y * e;
        o.z += ov[w].z * e;
        o.w += ov[w].w * e;
      }
      *reinterpret_cast<float4*>(p.po + (slot0 + (size_t)(h0 + h) * p.max_splits) * D + 4 * c4) = o;
    }
  }
  if (tid < G) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_stat[w][tid][0]);
    float zz = 0.f, ll = 0.f, tt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float e = __builtin_amdgcn_exp2f(s_stat[w][tid][0] - M);
      zz += s_stat[w][tid][1] * e;
      ll += s_stat[w][tid][2] * e;
      tt += s_stat[w][tid][3] * e;
    }
    p.pstat[slot0 + (size_t)tid * p.max_splits] = make_float4(M, zz, ll, tt);
  }
}

// ---------------------------------------------------------------------------
// kept-token pass (non-focal layers)
// ---------------------------------------------------------------------------

// Attention of one (sequence, KV head) pair over its kept image rows
// (gathered by index) and its text rows, as virtual rows r = 0 .. rows - 1:
// r < kept is image token sel[r], the others are text row n + r - kept.  The
// pair's 16-row tiles are dealt round-robin to its P workgroups (grid y):
// workgroup s takes tiles s, s + P, s + 2P, ..., round j of it holding its
// tiles j*TPR .. j*TPR + TPR - 1 (wave w, slot u: tile j*TPR + u*NW + w).
// So at any step every workgroup of a pair has the same number of rows, to
// within one tile, and a tile's rows do not depend on the pair's row count:
// the kept indices of the first round load before the sequence extent is
// read, and each round loads the next round's with its K/V rows.  (Staging
// the workgroup's indices in LDS behind a barrier measured ~1 us slower per
// launch: every wave then waits for all of them; five indices per tile in
// registers spill at 3 workgroups per CU; one index per tile plus lane
// permutes fits.  Two more tiles per wave loaded straight to LDS, at 2
// workgroups per CU, measured slower at every size.)  Each workgroup
// combines its waves' softmax states in LDS.  With one workgroup per pair it
// writes the output; otherwise it writes its state for the merge kernel.  (A
// variant in which the pair's last workgroup merged the states itself,
// behind an arrival counter, measured no faster than the merge launch with
// device-coherent state stores, as slow or slower with the workgroups of a
// pair kept on one XCD and the exchange in its L2, and 3-4x slower with
// device-scope release/acquire fences, whose L2 write-back dominates.)
// STREAM: the K/V rows are loaded non-temporally, which the launch plan
// picks when one step's kept rows exceed the last-level cache (they would
// not be found there on the next step, and the kept indices and merge
// states then stay cached).  PAD: see the grid below.
template <typename T, int D, int NW, int TPW, bool PAD, bool STREAM>
__global__ __launch_bounds__(NW * 64, kKeptBlocksPerCU) void kept_attn_kernel(SplitParams p) {
  constexpr bool BF = sizeof(T) == 2;
  constexpr int NT = NW * 64;                   // threads
  constexpr int TPR = NW * TPW;                 // tiles per workgroup round
  constexpr int E = D / 4;                      // K/q elements per lane
  constexpr int KW = E * (int)sizeof(T) / 4;    // ... as 32-bit words
  constexpr int NDB = D / 16;                   // PV d-blocks = V elements per row per lane
  constexpr int VW = NDB * (int)sizeof(T) / 4;  // V words per row per lane
  constexpr int HH = 8;                         // heads per LDS combine round
  constexpr int OST = D + 4;                    // padded LDS row of partial outputs (16-byte aligned)

  __shared__ float s_stat[NW][16][4];
  __shared__ __align__(16) float s_o[NW][HH][OST];

  // Grid x is the pair count, rounded up to a multiple of 8 when it is not
  // one (PAD: the extra blocks exit at once), so block pair + gridDim.x *
  // split runs on XCD pair mod 8 for every split.  (The check waits for the
  // kernel arguments before the rest of them load, so only a padded grid
  // has it.)
  const int pair = blockIdx.x;
  if constexpr (PAD)
    if (pair >= p.B * p.Hkv) return;
  const int split = blockIdx.y;
  const int P = p.grid_splits;
  const int kvh = pair % p.Hkv;
  const int b = pair / p.Hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: tile rows stay scalar
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int G = p.Hq / p.Hkv;

  const size_t row_base = ((size_t)b * p.Hkv + kvh) * (size_t)p.S;
  const T* __restrict__ Kb = reinterpret_cast<const T*>(p.k) + row_base * D;
  const T* __restrict__ Vb = reinterpret_cast<const T*>(p.v) + row_base * D;
  const int32_t* __restrict__ selb = p.sel + (size_t)b * p.k_stride;
  // first virtual row of this wave's tile in slot u of round j
  auto tile_row = [&](int j, int u) { return (split + P * (j * TPR + u * NW + wave)) * kTileRows; };

  // A lane holds the kept index of row `col` of each of its tiles; the index
  // of V row 4*grp + jj is read from the lane of that column.  The first
  // round's indices and the query slice do not depend on the sequence extent
  // and load before it is read.
  auto load_idx = [&](int j, int (&jk)[TPW]) {
#pragma unroll
    for (int u = 0; u < TPW; ++u) jk[u] = selb[min(tile_row(j, u) + col, p.k_stride - 1)];
  };
  int jk[TPW];
  load_idx(0, jk);
  // the kept count loads here too: the stores below may alias it, so a load
  // written after them could not be issued before them
  const int sel_cnt_b = p.sel_cnt[b];
  uint32_t qw[KW];
  if (col < G) {
    const T* qp = reinterpret_cast<const T*>(p.q) + ((size_t)b * p.Hq + kvh * G + col) * D;
    load_slice<T, KW>(qw, qp, grp);
  } else {
#pragma unroll
    for (int i = 0; i < KW; ++i) qw[i] = 0u;
  }

  int n, len;
  const bool clamped = seq_extent(p.lens, b, p.S, p.n_cap, n, len);
  const bool reporter = split == 0 && kvh == 0 && tid == 0;
  if (clamped && reporter) atomicOr(p.status, FASTOCR_FLAG_LENS_CLAMPED);

  // Fused append: the current token (cache row len - 1, a text row) comes
  // from k_new / v_new in every load of this launch, and workgroup 0 of the
  // pair writes it into the caches for later steps.
  const int cur = len - 1;
  const bool app = p.k_new != nullptr && len > 0;
  const T* __restrict__ knew = app ? reinterpret_cast<const T*>(p.k_new) + ((size_t)b * p.Hkv + kvh) * D : nullptr;
  const T* __restrict__ vnew = app ? reinterpret_cast<const T*>(p.v_new) + ((size_t)b * p.Hkv + kvh) * D : nullptr;
  if (app && split == 0) {
    constexpr int C16 = D * (int)sizeof(T) / 16;  // 16-byte pieces per row
    T* kc = reinterpret_cast<T*>(p.k_w) + (row_base + cur) * D;
    T* vc = reinterpret_cast<T*>(p.v_w) + (row_base + cur) * D;
    if (tid < C16) reinterpret_cast<uint4*>(kc)[tid] = reinterpret_cast<const uint4*>(knew)[tid];
    else if (tid < 2 * C16) reinterpret_cast<uint4*>(vc)[tid - C16] = reinterpret_cast<const uint4*>(vnew)[tid - C16];
  }
  const int kept = min(max(sel_cnt_b, 0), min(n, p.k_stride));
  const int rows = kept + (len - n);

  // virtual row -> cache row, given the kept index j loaded for row r
  // (branch-free; an index outside [0, n) is clamped and reported once)
  bool bad_index = false;
  auto cache_row = [&](int r, int j) -> int {
    const bool img = r < kept;
    bad_index |= img & ((unsigned)j >= (unsigned)n);
    const int jc = min(max(j, 0), max(n - 1, 0));
    return img ? jc : min(n + (r - kept), p.S - 1);
  };

  float m_run = -INFINITY, z = 0.f, lsum = 0.f, zt = 0.f;
  f32x4_t acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // One round of this wave: tiles starting at virtual rows tb[u], whose K/V
  // words are in kw / vw.  Rows at or past `rows` carry no weight.
  auto round = [&](const int (&tb)[TPW], uint32_t (&kw)[TPW][KW], uint32_t (&vw)[TPW][4][VW]) {
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = tb[u] + 4 * grp + j < rows;
#pragma unroll
        for (int w = 0; w < VW; ++w) vw[u][j][w] = ok ? vw[u][j][w] : 0u;
      }
    float x[TPW][4];
    float mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) x[u][i] = -INFINITY;
      if (tb[u] >= rows) continue;  // uniform over the wave
      f32x4_t s = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (BF) {
#pragma unroll
        for (int kk = 0; kk < E / 4; ++kk)
          s = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_bf16x4(kw[u][2 * kk], kw[u][2 * kk + 1]),
                                                        as_bf16x4(qw[2 * kk], qw[2 * kk + 1]), s, 0, 0, 0);
      } else {
#pragma unroll
        for (int kk = 0; kk < E; ++kk)
          s = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kw[u][kk]), __uint_as_float(qw[kk]), s, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[u][i] = (tb[u] + 4 * grp + i < rows) ? s[i] * p.scale_log2 : -INFINITY;
        mt = fmaxf(mt, x[u][i]);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    z *= alpha;
    lsum *= alpha;
    zt *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    m_run = m_new;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (tb[u] >= rows) continue;
      float pr[4], pu[4];
      uint32_t pb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[i] = __builtin_amdgcn_exp2f(x[u][i] - m_new);
        if constexpr (BF) {
          pb[i] = f32_to_bf16(pr[i]);
          pu[i] = bf16_to_f32(pb[i]);
        } else {
          pu[i] = pr[i];
        }
        zt += (tb[u] + 4 * grp + i >= kept) ? pr[i] : 0.f;
      }
      z += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      lsum += (pu[0] + pu[1]) + (pu[2] + pu[3]);
      if constexpr (BF) {
        const bf16x4_t pv = as_bf16x4(pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16));
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int w = db >> 1;
          const uint32_t sel = (db & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t lo = __builtin_amdgcn_perm(vw[u][1][w], vw[u][0][w], sel);
          const uint32_t hi = __builtin_amdgcn_perm(vw[u][3][w], vw[u][2][w], sel);
          acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_bf16x4(lo, hi), pv, acc[db], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(vw[u][i][db]), pr[i], acc[db], 0, 0, 0);
      }
    }
  };
  // The K/V loads of a round (the K row of the lane's column and its four V
  // rows, per tile), given the kept indices jk of the round's tiles.
  auto load_round = [&](const int (&tb)[TPW], const int (&jk)[TPW], uint32_t (&kw)[TPW][KW],
                        uint32_t (&vw)[TPW][4][VW]) {
    int pk[TPW], pvr[TPW][4];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      pk[u] = cache_row(tb[u] + col, jk[u]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int jv = __builtin_amdgcn_ds_bpermute((grp << 4) + 4 * jj, jk[u]);
        pvr[u][jj] = cache_row(tb[u] + 4 * grp + jj, jv);
      }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      if (tb[u] < rows) {  // uniform over the wave
        const T* kr = app && pk[u] == cur ? knew : Kb + (size_t)pk[u] * D;
        if constexpr (STREAM) load_slice_nt<T, KW>(kw[u], kr, grp);
        else load_slice<T, KW>(kw[u], kr, grp);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const T* vr = (app && pvr[u][j] == cur ? vnew : Vb + (size_t)pvr[u][j] * D) + col * NDB;
          if constexpr (STREAM) load_words_nt(vw[u][j], vr, VW);
          else load_words(vw[u][j], vr, VW);
        }
      }
    }
  };
  // Each round issues its K/V loads, then the next round's kept indices, so
  // that the next round's K/V addresses are known when it starts.
  for (int j = 0; tile_row(j, 0) < rows; ++j) {
    int tb[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) tb[u] = tile_row(j, u);
    uint32_t kw[TPW][KW];
    uint32_t vw[TPW][4][VW];
    load_round(tb, jk, kw, vw);
    load_idx(j + 1, jk);  // (clamped to the index array past the last round)
    round(tb, kw, vw);
  }
  if (bad_index) atomicOr(p.status, FASTOCR_FLAG_INDEX_CLAMPED);

  // ---- combine the waves: per-wave totals, then rounds of HH heads (each
  // wave leaves its unscaled accumulator in LDS; the reducing threads weight
  // wave w by exp2(m_w - M)); a workgroup without rows has M = -inf
  z += __shfl_xor(z, 16);
  z += __shfl_xor(z, 32);
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  zt += __shfl_xor(zt, 16);
  zt += __shfl_xor(zt, 32);
  if (grp == 0) {
    s_stat[wave][col][0] = m_run;
    s_stat[wave][col][1] = z;
    s_stat[wave][col][2] = lsum;
    s_stat[wave][col][3] = zt;
  }
  const bool direct = P == 1;
  const size_t slot0 = ((size_t)b * p.Hq + kvh * G) * p.max_splits + split;
  T* out = reinterpret_cast<T*>(p.out) + ((size_t)b * p.Hq + kvh * G) * D;
  for (int h0 = 0; h0 < G; h0 += HH) {
    if (h0 > 0) __syncthreads();  // the previous round has read s_o
    if (col >= h0 && col < h0 + HH) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_o[wave][col - h0][(4 * grp + i) * NDB + db] = acc[db][i];
    }
    __syncthreads();
    // thread t reduces the 4 consecutive outputs (h, 4*c4 .. 4*c4 + 3) of
    // float4 column c4 = t % (D/4) of head h = t / (D/4) (+ NT/(D/4) per
    // further pass): one weight per wave and head, one 16-byte LDS read per
    // wave, one 16-byte store
    const int hn = min(HH, G - h0);
    constexpr int C4 = D / 4;
    for (int idx = tid; idx < hn * C4; idx += NT) {
      const int h = idx / C4;
      const int c4 = idx - h * C4;
      float mv[NW], lv[NW];
      float4 ov[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        mv[w] = s_stat[w][h0 + h][0];
        lv[w] = s_stat[w][h0 + h][2];
        ov[w] = *reinterpret_cast<const float4*>(&s_o[w][h][4 * c4]);
      }
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, mv[w]);
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float e = mv[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv[w] - M);
        o.x += ov[w].x * e;
        o.y += ov[w].y * e;
        o.z += ov[w].z * e;
        o.w += ov[w].w * e;
        L += lv[w] * e;
      }
      if (direct) {
        T* od = out + (size_t)(h0 + h) * D + 4 * c4;
        const bool none = M == -INFINITY;
        store_out<T>(od + 0, none ? 0.f : o.x / L);
        store_out<T>(od + 1, none ? 0.f : o.y / L);
        store_out<T>(od + 2, none ? 0.f : o.z / L);
        store_out<T>(od + 3, none ? 0.f : o.w / L);
      } else {
        *reinterpret_cast<float4*>(p.po + (slot0 + (size_t)(h0 + h) * p.max_splits) * D + 4 * c4) = o;
      }
    }
  }
  if (direct) return;
  if (tid < G) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_stat[w][tid][0]);
    float zz = 0.f, ll = 0.f, tt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = s_stat[w][tid][0];
      const float e = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      zz += s_stat[w][tid][1] * e;
      ll += s_stat[w][tid][2] * e;
      tt += s_stat[w][tid][3] * e;
    }
    p.pstat[slot0 + (size_t)tid * p.max_splits] = make_float4(M, zz, ll, tt);
  }
}

// ---------------------------------------------------------------------------
// VALU variant of the full split pass (measurement override)
// ---------------------------------------------------------------------------

// The same work and merge-state format as split_attn_kernel<.., KIND_FULL>,
// with the query-group x K-tile product and the probability x V product done
// as fp32 FMAs on the vector ALUs.  Lane (s, c) = (lane / 16, lane % 16) holds
// elements [8c, 8c + 8) of its rows and of the group's queries; a row's logit
// is the sum over the 16 lanes of a slot (four shuffle steps), and each slot
// keeps its own softmax state over the rows it visits, combined across slots
// and waves at the end.  bf16, D = 128, groups of at most GM heads.
template <int GM>
__global__ __launch_bounds__(256, 2) void split_valu_kernel(SplitParams p) {
  constexpr int D = 128, NW = 4, U = 4;  // U rows per lane per round
  constexpr int RND = NW * U * 4;        // rows per workgroup round
  __shared__ float s_acc[NW][GM][D];
  __shared__ float s_st[NW][GM][3];
  const int pair = blockIdx.y;
  const int split = blockIdx.x;
  const int kvh = pair % p.Hkv;
  const int b = pair / p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, slot = lane >> 4;
  const int G = p.Hq / p.Hkv;
  const int begin = split * p.rows_per_split;
  const size_t row_base = ((size_t)b * p.Hkv + kvh) * (size_t)p.S;
  const uint16_t* __restrict__ Kb = reinterpret_cast<const uint16_t*>(p.k) + row_base * D + 8 * c;
  const uint16_t* __restrict__ Vb = reinterpret_cast<const uint16_t*>(p.v) + row_base * D + 8 * c;

  float qf[GM][8];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (h < G)
      w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.q) +
                                          ((size_t)b * p.Hq + kvh * G + h) * D + 8 * c);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[h][2 * e] = __uint_as_float(ws[e] << 16) * p.scale_log2;
      qf[h][2 * e + 1] = __uint_as_float(ws[e] & 0xffff0000u) * p.scale_log2;
    }
  }
  int n, len;
  const bool clamped = seq_extent(p.lens, b, p.S, p.n_cap, n, len);
  if (clamped && split == 0 && kvh == 0 && tid == 0) atomicOr(p.status, FASTOCR_FLAG_LENS_CLAMPED);
  const size_t slot0 = ((size_t)b * p.Hq + kvh * G) * p.max_splits + split;
  if (begin >= len) {
    if (tid < G) p.pstat[slot0 + (size_t)tid * p.max_splits] = make_float4(-INFINITY, 0.f, 0.f, 0.f);
    return;
  }
  const int end = min(begin + p.rows_per_split, len);

  float m[GM], z[GM], zt[GM], acc[GM][8];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    m[h] = -INFINITY;
    z[h] = zt[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  for (int r0 = begin; r0 < end; r0 += RND) {
    int rr[U];
    uint4 kw[U], vw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      rr[u] = r0 + (u * NW + wave) * 4 + slot;
      const size_t rc = (size_t)min(rr[u], p.S - 1);
      kw[u] = *reinterpret_cast<const uint4*>(Kb + rc * D);
      vw[u] = *reinterpret_cast<const uint4*>(Vb + rc * D);
    }
    float kf[U][8], vf[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = rr[u] < end;
      const uint32_t ks[4] = {kw[u].x, kw[u].y, kw[u].z, kw[u].w};
      const uint32_t vs[4] = {vw[u].x, vw[u].y, vw[u].z, vw[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[u][2 * e] = __uint_as_float(ks[e] << 16);
        kf[u][2 * e + 1] = __uint_as_float(ks[e] & 0xffff0000u);
        // rows past the end carry zero weight: zero their values so that
        // whatever the cache holds there cannot turn 0 * v into NaN
        vf[u][2 * e] = ok ? __uint_as_float(vs[e] << 16) : 0.f;
        vf[u][2 * e + 1] = ok ? __uint_as_float(vs[e] & 0xffff0000u) : 0.f;
      }
    }
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      if (h >= G) break;  // uniform
      float x[U];
      float mt = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float sacc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sacc = fmaf(kf[u][e], qf[h][e], sacc);
        sacc += __shfl_xor(sacc, 1);
        sacc += __shfl_xor(sacc, 2);
        sacc += __shfl_xor(sacc, 4);
        sacc += __shfl_xor(sacc, 8);
        x[u] = rr[u] < end ? sacc : -INFINITY;
        mt = fmaxf(mt, x[u]);
      }
      const float m_new = fmaxf(m[h], mt);
      if (m_new == -INFINITY) continue;  // no rows for this slot yet
      const float alpha = __builtin_amdgcn_exp2f(m[h] - m_new);
      z[h] *= alpha;
      zt[h] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float pr = __builtin_amdgcn_exp2f(x[u] - m_new);
        z[h] += pr;
        zt[h] += rr[u] >= n ? pr : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pr, vf[u][e], acc[h][e]);
      }
      m[h] = m_new;
    }
  }

  // combine the four slots of a wave (lanes c, c + 16, c + 32, c + 48)
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h >= G) break;
    float M = fmaxf(m[h], __shfl_xor(m[h], 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    const float w = m[h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[h] - M);
    float zz = z[h] * w, tt = zt[h] * w;
    zz += __shfl_xor(zz, 16);
    zz += __shfl_xor(zz, 32);
    tt += __shfl_xor(tt, 16);
    tt += __shfl_xor(tt, 32);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float a = acc[h][e] * w;
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      if (slot == 0) s_acc[wave][h][8 * c + e] = a;
    }
    if (lane == 0) {
      s_st[wave][h][0] = M;
      s_st[wave][h][1] = zz;
      s_st[wave][h][2] = tt;
    }
  }
  __syncthreads();
  // combine the waves: one state per head (the normaliser is the fp32 sum)
  for (int i = tid; i < G * D; i += NW * 64) {
    const int h = i / D, d = i - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_st[w][h][0]);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (s_st[w][h][0] != -INFINITY) o += s_acc[w][h][d] * __builtin_amdgcn_exp2f(s_st[w][h][0] - M);
    p.po[(slot0 + (size_t)h * p.max_splits) * D + d] = o;
  }
  if (tid < G) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_st[w][tid][0]);
    float zz = 0.f, tt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (s_st[w][tid][0] != -INFINITY) {
        const float e = __builtin_amdgcn_exp2f(s_st[w][tid][0] - M);
        zz += s_st[w][tid][1] * e;
        tt += s_st[w][tid][2] * e;
      }
    p.pstat[slot0 + (size_t)tid * p.max_splits] = make_float4(M, zz, zz, tt);
  }
}

// ---------------------------------------------------------------------------
// merge of split states, and image-token scores
// ---------------------------------------------------------------------------

// Sum over groups of SL = 8 or 16 adjacent lanes; every lane of a group gets
// the group total.  Pairs lanes i and 15-i (row_mirror, SL = 16) and i and
// 7-i (row_half_mirror), then folds with the quad permutations 1,0,3,2 and
// 2,3,0,1.
template <int SL>
__device__ __forceinline__ float group_sum(float x) {
  if (SL == 16) x += __int_as_float(FASTOCR_DPP(0, __float_as_int(x), 0x140, 0xf));
  x += __int_as_float(FASTOCR_DPP(0, __float_as_int(x), 0x141, 0xf));
  x += __int_as_float(FASTOCR_DPP(0, __float_as_int(x), 0xb1, 0xf));
  x += __int_as_float(FASTOCR_DPP(0, __float_as_int(x), 0x4e, 0xf));
  return x;
}

// Max over each 16-lane row; every lane gets its row's result (the same
// mirror/quad folds as group_sum<16>).
__device__ __forceinline__ float row_max16(float x) {
  int v = __float_as_int(x);
  x = fmaxf(x, __int_as_float(FASTOCR_DPP(v, v, 0x140, 0xf))); v = __float_as_int(x);
  x = fmaxf(x, __int_as_float(FASTOCR_DPP(v, v, 0x141, 0xf))); v = __float_as_int(x);
  x = fmaxf(x, __int_as_float(FASTOCR_DPP(v, v, 0xb1, 0xf))); v = __float_as_int(x);
  x = fmaxf(x, __int_as_float(FASTOCR_DPP(v, v, 0x4e, 0xf)));
  return x;
}

// merge_head for up to 64 splits: every wave derives the head's softmax
// totals itself (lane s holds split s's state) and weights its partial
// outputs from their own maxima, so no workgroup barrier.  A thread uses
// NV = ceil(splits / SL) slots (the same count for the whole launch); the
// body is instantiated per count, so each thread issues exactly the loads
// it uses, all at once from indices clamped to the last split, with no
// branch between the loads and their use (a lane-conditional load, or an
// early exit, made the compiler wait for one load before issuing the next).
template <typename T, int D, int NV>
__device__ __forceinline__ void merge_head_small(const MergeParams& p, int b, int h) {
  constexpr int D4 = D / 4;
  constexpr int SL = kMergeThreads / D4;
  const int tid = threadIdx.x, lane = tid & 63;
  const size_t slot0 = ((size_t)b * p.Hq + h) * p.max_splits;
  const int d4 = tid / SL, sl = tid % SL;
  const float4* po = reinterpret_cast<const float4*>(p.po + slot0 * D) + d4;
  const int nsplit = p.grid_splits;
  T* out = reinterpret_cast<T*>(p.out) + ((size_t)b * p.Hq + h) * D;
  const int last = nsplit - 1;
  const float4 qr = p.pstat[slot0 + min(lane, last)];
  float4 pv[NV];
  float mxr[NV];  // maxima of the splits this thread accumulates
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int s = min(sl + i * SL, last);
    pv[i] = po[(size_t)s * D4];
    mxr[i] = p.pstat[slot0 + s].x;
  }
  __builtin_amdgcn_sched_barrier(0);  // all loads issue before the first use of any
  const bool mine = lane < nsplit;
  const float M = wave_max(mine ? qr.x : -INFINITY);
  const bool none = M == -INFINITY;  // no rows at all: zero output and no image mass
  // lanes past the last split and empty splits get weight 0; a state's sums
  // are finite (an empty split's are 0), so they add exactly 0
  const float w = (mine && qr.x != -INFINITY) ? __builtin_amdgcn_exp2f(qr.x - M) : 0.f;
  const float Z = wave_sum(qr.y * w);
  const float L = wave_sum(qr.z * w);
  const float Zt = wave_sum(qr.w * w);
  // branch-free sums: a split of weight 0 adds exactly 0 whatever its
  // partial output holds (an empty split's is not written this launch)
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float wsv = (sl + i * SL < nsplit && mxr[i] != -INFINITY) ? __builtin_amdgcn_exp2f(mxr[i] - M) : 0.f;
    const bool use = wsv != 0.f;
    a0 += use ? pv[i].x * wsv : 0.f;
    a1 += use ? pv[i].y * wsv : 0.f;
    a2 += use ? pv[i].z * wsv : 0.f;
    a3 += use ? pv[i].w * wsv : 0.f;
  }
  a0 = group_sum<SL>(a0);
  a1 = group_sum<SL>(a1);
  a2 = group_sum<SL>(a2);
  a3 = group_sum<SL>(a3);
  if (sl == 0) {
    const float inv = 1.f / L;
    store_out<T>(out + 4 * d4 + 0, none ? 0.f : a0 * inv);
    store_out<T>(out + 4 * d4 + 1, none ? 0.f : a1 * inv);
    store_out<T>(out + 4 * d4 + 2, none ? 0.f : a2 * inv);
    store_out<T>(out + 4 * d4 + 3, none ? 0.f : a3 * inv);
  }
  if (tid == 0 && p.text_mass) p.text_mass[b * p.Hq + h] = none ? 1.f : Zt / Z;  // image mass = 1 - this
}

template <typename T, int D, int NV>
__device__ __forceinline__ void merge_head_small_dispatch(const MergeParams& p, int b, int h, int nv) {
  if constexpr (NV > 1)
    if (nv < NV) return merge_head_small_dispatch<T, D, NV - 1>(p, b, h, nv);
  merge_head_small<T, D, NV>(p, b, h);
}

// Workgroups [0, Hq): merge head h's split states into its output.  Thread
// t covers float4 column t / SL of the output and splits s = t % SL (mod SL).
// Every launched split has written a state this launch (an empty split one
// with max -inf and no weight), so the merge does not read the sequence
// extent: all its loads are issued at once.
template <typename T, int D>
__device__ void merge_head(const MergeParams& p, int b, int h) {
  constexpr int D4 = D / 4;
  constexpr int SL = kMergeThreads / D4;
  constexpr int NST = kMaxMergeSplits / kMergeThreads;  // split states per thread
  constexpr int PF = 8;                                  // partial outputs per thread in registers
  __shared__ float s_w[kMaxMergeSplits];
  __shared__ float s_red[kMergeThreads / 64][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t slot0 = ((size_t)b * p.Hq + h) * p.max_splits;
  const int d4 = tid / SL, sl = tid % SL;
  const float4* po = reinterpret_cast<const float4*>(p.po + slot0 * D) + d4;
  const int nsplit = p.grid_splits;
  T* out = reinterpret_cast<T*>(p.out) + ((size_t)b * p.Hq + h) * D;
  if (nsplit <= 64) {
    merge_head_small_dispatch<T, D, 64 / SL>(p, b, h, (nsplit + SL - 1) / SL);
    return;
  }
  float4 st[NST];
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int s = tid + i * kMergeThreads;
    st[i] = s < nsplit ? p.pstat[slot0 + s] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 pv[PF];
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int s = sl + i * SL;
    pv[i] = s < nsplit ? po[(size_t)s * D4] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NST; ++i)
    if (tid + i * kMergeThreads < nsplit) m = fmaxf(m, st[i].x);
  m = wave_max(m);
  if (lane == 0) s_red[wave][0] = m;
  __syncthreads();
  float M = s_red[0][0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, s_red[w][0]);
  if (M == -INFINITY) {  // no rows at all: zero output and no image mass
    for (int d = tid; d < D; d += kMergeThreads) store_out<T>(out + d, 0.f);
    if (tid == 0 && p.text_mass) p.text_mass[b * p.Hq + h] = 1.f;  // image mass = 1 - this
    return;
  }
  float z = 0.f, l = 0.f, t = 0.f;
#pragma unroll
  for (int i = 0; i < NST; ++i) {
    const int s = tid + i * kMergeThreads;
    if (s < nsplit) {
      // empty splits get weight exactly 0 (and their partial outputs, not
      // written this launch, are never multiplied)
      const float w = st[i].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st[i].x - M);
      s_w[s] = w;
      z += st[i].y * w;
      l += st[i].z * w;
      t += st[i].w * w;
    }
  }
  z = wave_sum(z);
  l = wave_sum(l);
  t = wave_sum(t);
  if (lane == 0) {
    s_red[wave][1] = z;
    s_red[wave][2] = l;
    s_red[wave][3] = t;
  }
  __syncthreads();
  float Z = 0.f, L = 0.f, Zt = 0.f;
#pragma unroll
  for (int w = 0; w < kMergeThreads / 64; ++w) {
    Z += s_red[w][1];
    L += s_red[w][2];
    Zt += s_red[w][3];
  }
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int i = 0; i < PF; ++i) {
    const int s = sl + i * SL;
    const float w = s < nsplit ? s_w[s] : 0.f;
    if (w != 0.f) {
      a0 += pv[i].x * w;
      a1 += pv[i].y * w;
      a2 += pv[i].z * w;
      a3 += pv[i].w * w;
    }
  }
  for (int s = sl + PF * SL; s < nsplit; s += SL) {
    const float w = s_w[s];
    if (w != 0.f) {
      const float4 v = po[(size_t)s * D4];
      a0 += v.x * w;
      a1 += v.y * w;
      a2 += v.z * w;
      a3 += v.w * w;
    }
  }
  a0 = group_sum<SL>(a0);
  a1 = group_sum<SL>(a1);
  a2 = group_sum<SL>(a2);
  a3 = group_sum<SL>(a3);
  if (sl == 0) {
    const float inv = 1.f / L;
    store_out<T>(out + 4 * d4 + 0, a0 * inv);
    store_out<T>(out + 4 * d4 + 1, a1 * inv);
    store_out<T>(out + 4 * d4 + 2, a2 * inv);
    store_out<T>(out + 4 * d4 + 3, a3 * inv);
  }
  if (tid == 0 && p.text_mass) p.text_mass[b * p.Hq + h] = Zt / Z;
}

// Workgroups [Hq, Hq + score_blocks): head-summed probability of
// kMergeThreads image tokens each.  Each score workgroup derives every
// head's softmax max and sum from the split states itself (16 lanes per
// head), so it does not depend on the merge workgroups.  The token's logits
// of up to kScoreRegHeads heads are loaded before anything else, those of
// further heads 16 at a time.
constexpr int kScoreRegHeads = 64;
constexpr int kScorePrefetchPasses = 4;  // heads whose split states load up front: 4 x 16

__device__ void score_block(const MergeParams& p, int b, int sb) {
  __shared__ float2 s_mz[kMaxHeads];
  __shared__ unsigned int s_hist[256];
  const int tid = threadIdx.x;
  const int j = sb * kMergeThreads + tid;
  int n = 0;  // image tokens, clamped as the top-k clamps them
  if (p.hist0) {
    const int n0 = p.lens[2 * b], l0 = p.lens[2 * b + 1];
    n = min(max(n0, 0), min(max(l0, 0), p.n_cap));
    for (int i = tid; i < 256; i += kMergeThreads) s_hist[i] = 0u;
  }
  const float* lg = p.logits + (size_t)b * p.Hq * p.n_stride + min(j, p.n_stride - 1);
  float x[kScoreRegHeads];
#pragma unroll
  for (int h = 0; h < kScoreRegHeads; ++h) x[h] = h < p.Hq ? lg[(size_t)h * p.n_stride] : 0.f;

  // Every head's softmax max and 1/sum from the split states, 16 lanes per
  // head and 16 heads per pass; the states of the first kScorePrefetchPasses
  // passes are loaded before any is reduced.
  const int nsplit = p.grid_splits;
  const int hl = tid & 15;
  constexpr int HPP = kMergeThreads / 16;
  float4 st[kScorePrefetchPasses][4];
#pragma unroll
  for (int pass = 0; pass < kScorePrefetchPasses; ++pass) {
    const int h = pass * HPP + (tid >> 4);
    const float4* ps = p.pstat + ((size_t)b * p.Hq + min(h, p.Hq - 1)) * p.max_splits;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = hl + 16 * i;
      st[pass][i] = (h < p.Hq && s < nsplit) ? ps[s] : make_float4(-INFINITY, 0.f, 0.f, 0.f);
    }
  }
  auto head_totals = [&](int h, const float4 (&sv)[4]) {
    const bool hv = h < p.Hq;
    const float4* ps = p.pstat + ((size_t)b * p.Hq + (hv ? h : 0)) * p.max_splits;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, sv[i].x);
    if (hv)
      for (int s = hl + 64; s < nsplit; s += 16) m = fmaxf(m, ps[s].x);
    m = row_max16(m);
    float z = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (hl + 16 * i < nsplit && sv[i].x != -INFINITY) z += sv[i].y * __builtin_amdgcn_exp2f(sv[i].x - m);
    if (hv)
      for (int s = hl + 64; s < nsplit; s += 16) {
        const float4 q = ps[s];
        if (q.x != -INFINITY) z += q.y * __builtin_amdgcn_exp2f(q.x - m);
      }
    z = group_sum<16>(z);
    if (hv && hl == 0) s_mz[h] = make_float2(m, 1.f / z);
  };
#pragma unroll
  for (int pass = 0; pass < kScorePrefetchPasses; ++pass)
    if (pass * HPP < p.Hq) head_totals(pass * HPP + (tid >> 4), st[pass]);
  for (int h0 = kScorePrefetchPasses * HPP; h0 < p.Hq; h0 += HPP) {
    const int h = h0 + (tid >> 4);
    const float4* ps = p.pstat + ((size_t)b * p.Hq + min(h, p.Hq - 1)) * p.max_splits;
    float4 sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = hl + 16 * i;
      sv[i] = (h < p.Hq && s < nsplit) ? ps[s] : make_float4(-INFINITY, 0.f, 0.f, 0.f);
    }
    head_totals(h, sv);
  }
  // heads past Hq up to the register heads add exactly 0 (logit 0, weight 0)
  if (tid >= p.Hq && tid < kScoreRegHeads) s_mz[tid] = make_float2(0.f, 0.f);
  __syncthreads();
  // tokens past this sequence's image tokens get scores too (from stale
  // logits); nothing reads them
  float s = 0.f;
  if (j < p.n_stride) {
#pragma unroll
    for (int h = 0; h < kScoreRegHeads; ++h) s += __builtin_amdgcn_exp2f(x[h] - s_mz[h].x) * s_mz[h].y;
    for (int h0 = kScoreRegHeads; h0 < p.Hq; h0 += 16) {
      float y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) y[i] = h0 + i < p.Hq ? lg[(size_t)(h0 + i) * p.n_stride] : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (h0 + i < p.Hq) s += __builtin_amdgcn_exp2f(y[i] - s_mz[h0 + i].x) * s_mz[h0 + i].y;
    }
    p.scores[(size_t)b * p.n_stride + j] = s;
  }
  if (p.hist0) {
    // leading byte of the image tokens' scores, the top-k's first digit
    hist_key(__float_as_uint(s), j < n, 24, 0u, 0u, s_hist, tid & 63);
    __syncthreads();
    for (int i = tid; i < 256; i += kMergeThreads)
      if (s_hist[i]) atomicAdd(p.hist0 + (size_t)b * 256 + i, s_hist[i]);
  }
}

// The merge of a kept-token pass: at most 64 states per head (one per lane),
// no text mass and no scores.  The same arithmetic, in the same order, as
// merge_head's path for up to 64 splits, without its loads for longer
// passes, its per-split maxima (the weights come from the lanes holding the
// states) and its text-mass sums: 3.9 against 4.5 us per launch in a
// 72B-like B=8 graph, 2.9 against 3.3 at 7B-like B=1 (measured after a
// kernel writing the states, in isolation).
static_assert(kMaxKeptSplits <= 64, "a kept-token pass's states fit one wave's lanes");
// A thread uses NV = ceil(P / SL) state slots (the same count for the whole
// launch): the body is instantiated per count, so each thread issues exactly
// the loads it uses, all before the first use of any, and the compiler waits
// for them one by one.
template <typename T, int D, int NV>
__device__ __forceinline__ void kept_merge_body(const MergeParams& p) {
  constexpr int D4 = D / 4;
  constexpr int SL = kMergeThreads / D4;  // lanes sharing an output column
  // Workgroup (pair, g) is block pair + X * g, X = B * Hkv rounded up to a
  // multiple of 8.  Block i runs on XCD i mod 8, so it shares the XCD (and
  // its L2) of the pair's kept-token workgroups (blocks pair + X * split),
  // and a state line is only ever written and read there.  That measured
  // faster kept-token passes at 7B-like B=16 (9.3 against 9.5 us with the
  // heads in (head, sequence) order, 9.8 with every pair's merge one XCD
  // over) and made no difference at 32B- and 72B-like sizes.
  const int G = p.Hq / p.Hkv;
  const int b = blockIdx.x / p.Hkv, h = (blockIdx.x % p.Hkv) * G + blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int d4 = tid / SL, sl = tid % SL;
  const int P = p.grid_splits;
  const size_t slot0 = ((size_t)b * p.Hq + h) * p.max_splits;
  // lane s holds state s; thread (d4, sl) the partial outputs of states
  // sl, sl + SL, ... in column d4.  Every load is issued unconditionally from
  // an index clamped to the last state (dropped below): a load under a lane
  // condition, or before an early exit, made the compiler wait for it before
  // issuing the next ones.
  const float4 qr = p.pstat[slot0 + min(lane, P - 1)];
  const float4* po = reinterpret_cast<const float4*>(p.po + slot0 * D) + d4;
  float4 pv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) pv[i] = po[(size_t)min(sl + i * SL, P - 1) * D4];
  __builtin_amdgcn_sched_barrier(0);  // all loads issue before the first use of any
  T* out = reinterpret_cast<T*>(p.out) + ((size_t)b * p.Hq + h) * D;
  const bool mine = lane < P;
  const float M = wave_max(mine ? qr.x : -INFINITY);
  const bool none = M == -INFINITY;  // no rows at all: zero output
  // lanes past P and states without rows get weight 0 (and add 0 to L: a
  // state's sums are finite)
  const float w = (mine && qr.x != -INFINITY) ? __builtin_amdgcn_exp2f(qr.x - M) : 0.f;
  const float L = wave_sum(qr.z * w);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  {
    // products and sums rounded separately, as in the general merge; a state
    // not used (past P or of weight 0) is multiplied by 0 and adds exactly 0
    // (its partial outputs are finite), so every loaded value is used and no
    // load is moved under a condition
#pragma clang fp contract(off)
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int s = sl + i * SL;
      const float ws = __shfl(w, s);
      const float wu = (s < P && ws != 0.f) ? ws : 0.f;
      a0 += pv[i].x * wu;
      a1 += pv[i].y * wu;
      a2 += pv[i].z * wu;
      a3 += pv[i].w * wu;
    }
  }
  a0 = group_sum<SL>(a0);
  a1 = group_sum<SL>(a1);
  a2 = group_sum<SL>(a2);
  a3 = group_sum<SL>(a3);
  if (sl == 0) {
    const float inv = 1.f / L;
    store_out<T>(out + 4 * d4 + 0, none ? 0.f : a0 * inv);
    store_out<T>(out + 4 * d4 + 1, none ? 0.f : a1 * inv);
    store_out<T>(out + 4 * d4 + 2, none ? 0.f : a2 * inv);
    store_out<T>(out + 4 * d4 + 3, none ? 0.f : a3 * inv);
  }
}

template <typename T, int D, int NV>
__device__ __forceinline__ void kept_merge_dispatch(const MergeParams& p, int nv) {
  if constexpr (NV > 1)
    if (nv < NV) return kept_merge_dispatch<T, D, NV - 1>(p, nv);
  kept_merge_body<T, D, NV>(p);
}

template <typename T, int D, bool PAD>
__global__ __launch_bounds__(kMergeThreads) void kept_merge_kernel(MergeParams p) {
  constexpr int SL = kMergeThreads / (D / 4);
  constexpr int PF = 64 / SL;  // slots per thread for 64 states
  if constexpr (PAD)
    if ((int)blockIdx.x >= p.B * p.Hkv) return;  // (grid x rounded up to a multiple of 8)
  kept_merge_dispatch<T, D, PF>(p, (p.grid_splits + SL - 1) / SL);
}

template <typename T, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeParams p) {
  const int b = blockIdx.y;
  if ((int)blockIdx.x < p.Hq) merge_head<T, D>(p, b, blockIdx.x);
  else score_block(p, b, blockIdx.x - p.Hq);
}

// PER: keys per thread held in registers (a power of two up to
// kTopkRegKeys), or 0 for rows longer than kTopkRegKeys * kTopkThreads.
template <int PER>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  __shared__ TopkShared sh;
  const int b = blockIdx.x;
  unsigned int* hist0 = p.hist0 ? p.hist0 + (size_t)b * 256 : nullptr;
  if (p.n_cap < 1) {
    if (threadIdx.x == 0) p.cnt[b] = 0;
    if (hist0)
      for (int i = threadIdx.x; i < 256; i += kTopkThreads) hist0[i] = 0u;
    return;
  }
  topk_sequence<PER>(p.scores + (size_t)b * p.score_stride, p.n_cap, p.lens, b, p.tau, p.idx_stride,
                     p.idx + (size_t)b * p.idx_stride, p.cnt + b, p.status, hist0, sh);
}

// ---------------------------------------------------------------------------
// row gather (image-first packing of a multi-span cache)
// ---------------------------------------------------------------------------

// One workgroup per kPackRowsPerBlock destination rows of one (sequence, KV
// head): consecutive threads move consecutive 16-byte pieces of a row, so
// both the source row and the destination rows are read and written
// contiguously.
__global__ __launch_bounds__(kPackThreads) void pack_rows_kernel(PackParams p) {
  const int pair = blockIdx.y;
  const int b = pair / p.Hkv;
  const int rows = min(max(p.rows[b], 0), p.S);
  const int i0 = blockIdx.x * kPackRowsPerBlock;
  if (i0 >= rows) return;
  const int pieces = p.row_bytes / 16;
  const int n = min(kPackRowsPerBlock, rows - i0) * pieces;
  const size_t base = (size_t)pair * p.S;
  const char* src = reinterpret_cast<const char*>(p.src);
  char* dst = reinterpret_cast<char*>(p.dst);
  bool bad = false;
  for (int t = threadIdx.x; t < n; t += kPackThreads) {
    const int i = i0 + t / pieces;
    const int c = t - (t / pieces) * pieces;
    const int s0 = p.map[(size_t)b * p.S + i];
    const int s = min(max(s0, 0), p.S - 1);
    bad |= s != s0;
    const uint4 v = reinterpret_cast<const uint4*>(src + (base + s) * p.row_bytes)[c];
    reinterpret_cast<uint4*>(dst + (base + i) * p.row_bytes)[c] = v;
  }
  if (bad && p.status) atomicOr(p.status, FASTOCR_FLAG_INDEX_CLAMPED);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <typename P>
static hipError_t launch(void (*kernel)(P), dim3 grid, dim3 block, hipStream_t stream,
                         const LaunchTiming& timing, const P& p) {
  if (timing.start || timing.stop) {
    void* args[] = {const_cast<P*>(&p)};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, 0, stream,
                              timing.start, timing.stop, 0);
  }
  kernel<<<grid, block, 0, stream>>>(p);
  return hipGetLastError();
}

// Tiles a wave loads per round: fp32 rows of 128 elements take twice the
// registers of bf16 ones, and two tiles of them per wave would spill.
template <typename T, int D>
constexpr int tiles_per_wave() { return (sizeof(T) == 4 && D == 128) ? 1 : kTilesPerWave; }

template <typename T, int D>
static hipError_t launch_split_t(SplitKind kind, const SplitParams& p, hipStream_t stream,
                                 const LaunchTiming& timing) {
  const dim3 block(kSplitThreads), grid(p.grid_splits, p.Hkv * p.B);
  constexpr int TPW = tiles_per_wave<T, D>();
  switch (kind) {
    case KIND_FULL:
      if constexpr (sizeof(T) == 2 && D == 128)
        if (p.valu) return launch(split_valu_kernel<kValuMaxGroup>, grid, block, stream, timing, p);
      if (p.stream_rows)
        return launch(split_attn_kernel<T, D, KIND_FULL, kSplitWaves, TPW, true>, grid, block, stream, timing, p);
      return launch(split_attn_kernel<T, D, KIND_FULL, kSplitWaves, TPW, false>, grid, block, stream, timing, p);
    case KIND_FOCAL:
      if (p.stream_rows)
        return launch(split_attn_kernel<T, D, KIND_FOCAL, kSplitWaves, TPW, true>, grid, block, stream, timing, p);
      return launch(split_attn_kernel<T, D, KIND_FOCAL, kSplitWaves, TPW, false>, grid, block, stream, timing, p);
    default:
      return hipErrorInvalidValue;
  }
}

// Both kept-token kernels take grid x = the (sequence, KV head) pairs rounded
// up to a multiple of 8, so a pair's blocks all run on one XCD.
static int kept_grid_x(int pairs) { return (pairs + 7) / 8 * 8; }

template <typename T, int D>
static hipError_t launch_kept_t(const SplitParams& p, hipStream_t stream, const LaunchTiming& timing) {
  constexpr int TPW = tiles_per_wave<T, D>();
  const int pairs = p.Hkv * p.B;
  const dim3 block(kSplitThreads), grid(kept_grid_x(pairs), p.grid_splits);
  if (pairs % 8 != 0)
    return p.stream_rows ? launch(kept_attn_kernel<T, D, kSplitWaves, TPW, true, true>, grid, block, stream, timing, p)
                         : launch(kept_attn_kernel<T, D, kSplitWaves, TPW, true, false>, grid, block, stream, timing, p);
  return p.stream_rows ? launch(kept_attn_kernel<T, D, kSplitWaves, TPW, false, true>, grid, block, stream, timing, p)
                       : launch(kept_attn_kernel<T, D, kSplitWaves, TPW, false, false>, grid, block, stream, timing, p);
}

hipError_t launch_kept(int dtype, int head_dim, const SplitParams& p, hipStream_t stream,
                       const LaunchTiming& timing) {
  if (dtype == FASTOCR_DTYPE_BF16)
    return head_dim == 128 ? launch_kept_t<uint16_t, 128>(p, stream, timing)
                           : launch_kept_t<uint16_t, 64>(p, stream, timing);
  return head_dim == 128 ? launch_kept_t<float, 128>(p, stream, timing)
                         : launch_kept_t<float, 64>(p, stream, timing);
}

hipError_t launch_split(int dtype, int head_dim, SplitKind kind, const SplitParams& p, hipStream_t stream,
                        const LaunchTiming& timing) {
  if (dtype == FASTOCR_DTYPE_BF16)
    return head_dim == 128 ? launch_split_t<uint16_t, 128>(kind, p, stream, timing)
                           : launch_split_t<uint16_t, 64>(kind, p, stream, timing);
  return head_dim == 128 ? launch_split_t<float, 128>(kind, p, stream, timing)
                         : launch_split_t<float, 64>(kind, p, stream, timing);
}

hipError_t launch_kept_merge(int dtype, int head_dim, const MergeParams& p, hipStream_t stream,
                             const LaunchTiming& timing) {
  if (p.grid_splits < 1 || p.grid_splits > 64 || p.score_blocks != 0 || p.text_mass != nullptr ||
      p.Hkv < 1 || p.Hq % p.Hkv != 0)
    return hipErrorInvalidValue;
  const int pairs = p.B * p.Hkv;
  const dim3 grid(kept_grid_x(pairs), p.Hq / p.Hkv), block(kMergeThreads);
  if (pairs % 8 != 0) {
    if (dtype == FASTOCR_DTYPE_BF16)
      return head_dim == 128 ? launch(kept_merge_kernel<uint16_t, 128, true>, grid, block, stream, timing, p)
                             : launch(kept_merge_kernel<uint16_t, 64, true>, grid, block, stream, timing, p);
    return head_dim == 128 ? launch(kept_merge_kernel<float, 128, true>, grid, block, stream, timing, p)
                           : launch(kept_merge_kernel<float, 64, true>, grid, block, stream, timing, p);
  }
  if (dtype == FASTOCR_DTYPE_BF16)
    return head_dim == 128 ? launch(kept_merge_kernel<uint16_t, 128, false>, grid, block, stream, timing, p)
                           : launch(kept_merge_kernel<uint16_t, 64, false>, grid, block, stream, timing, p);
  return head_dim == 128 ? launch(kept_merge_kernel<float, 128, false>, grid, block, stream, timing, p)
                         : launch(kept_merge_kernel<float, 64, false>, grid, block, stream, timing, p);
}

hipError_t launch_merge(int dtype, int head_dim, const MergeParams& p, hipStream_t stream,
                        const LaunchTiming& timing) {
  const dim3 grid(p.Hq + p.score_blocks, p.B), block(kMergeThreads);
  if (dtype == FASTOCR_DTYPE_BF16)
    return head_dim == 128 ? launch(merge_kernel<uint16_t, 128>, grid, block, stream, timing, p)
                           : launch(merge_kernel<uint16_t, 64>, grid, block, stream, timing, p);
  return head_dim == 128 ? launch(merge_kernel<float, 128>, grid, block, stream, timing, p)
                         : launch(merge_kernel<float, 64>, grid, block, stream, timing, p);
}

hipError_t launch_topk(const TopkParams& p, hipStream_t stream, const LaunchTiming& timing) {
  const dim3 grid(p.B), block(kTopkThreads);
  const int per = (p.n_cap + kTopkThreads - 1) / kTopkThreads;
  if (per <= 1) return launch(topk_kernel<1>, grid, block, stream, timing, p);
  if (per <= 2) return launch(topk_kernel<2>, grid, block, stream, timing, p);
  if (per <= 4) return launch(topk_kernel<4>, grid, block, stream, timing, p);
  if (per <= 8) return launch(topk_kernel<8>, grid, block, stream, timing, p);
  if (per <= kTopkRegKeys) return launch(topk_kernel<kTopkRegKeys>, grid, block, stream, timing, p);
  return launch(topk_kernel<0>, grid, block, stream, timing, p);
}

hipError_t launch_pack(const PackParams& p, hipStream_t stream) {
  const dim3 grid((p.S + kPackRowsPerBlock - 1) / kPackRowsPerBlock, p.B * p.Hkv), block(kPackThreads);
  pack_rows_kernel<<<grid, block, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace fastocr
