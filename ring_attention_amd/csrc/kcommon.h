// kcommon.h -- device-side helpers shared by the forward kernels (HIP path only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ring_sched.h"

namespace rattn {

// Launch parameters common to the forward kernels.
struct FwdParams {
  int32_t B, Hq, Hkv;
  int32_t group;     // Hq / Hkv
  int64_t Nq;        // query rows in q (per batch)
  int64_t Nk;        // key/value rows in k, v (per batch)
  float c;           // scale * log2(e): scores are exponentiated with exp2
  // Split-KV: the live key tiles of every query tile are divided into
  // n_splits contiguous ranges, one workgroup each; split s writes its
  // normalised partial (fp32) at out + s * split_out_stride and its lse at
  // lse + s * split_lse_stride.  n_splits = 1: no split, strides unused.
  int32_t n_splits;
  int64_t split_out_stride;
  int64_t split_lse_stride;
  // Output rows: query row i of this call is row out_row_off + i of the
  // [B, out_rows, Hq] output.  merge_out = 1 (fp32 output only): log-sum-exp
  // merge this call's normalised result into the (out, lse) already there
  // instead of overwriting it.
  int64_t out_rows;
  int64_t out_row_off;
  int32_t merge_out;
};

// Merge of a normalised partial (lse_n) into a running normalised result
// (lse_r): out = f_r * out_r + f_n * out_n, lse = lse_out.  An empty side
// (lse = -inf) weighs 0; two empty sides give out 0, lse -inf.  This is the
// log-sum-exp correction applied after every ring step, in max-shifted form.
struct MergeW {
  float f_r, f_n, lse;
};
__device__ __forceinline__ MergeW merge_weights(float lse_r, float lse_n) {
  const float m = fmaxf(lse_r, lse_n);
  if (m == -__builtin_inff()) return MergeW{0.f, 0.f, m};
  const float wr = expf(lse_r - m), wn = expf(lse_n - m), z = wr + wn;
  return MergeW{wr / z, wn / z, m + logf(z)};
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

// 16-bit storage types and their MFMA operand vectors.
struct Bf16 {
  typedef __bf16 elem;
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  typedef __bf16 v4 __attribute__((ext_vector_type(4)));
  typedef __bf16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mfma32x32x16(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
struct F16 {
  typedef _Float16 elem;
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  typedef _Float16 v4 __attribute__((ext_vector_type(4)));
  typedef _Float16 v2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ f32x16 mfma32x32x16(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};
struct F32 {
  typedef float elem;
};

// Round-to-nearest-even conversion to the storage type (v_cvt_pk_bf16_f32 /
// v_cvt_f16_f32 on gfx950).
template <typename TT>
__device__ __forceinline__ typename TT::elem to_elem(float x) {
  return (typename TT::elem)x;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Lanes l and l^32 hold the two halves of one query's keys in the 32x32 MFMA
// accumulator layout.  v_permlane32_swap with both operands = x returns, in
// each lane, x of lane l%32 and x of lane l%32+32 (one per result, in an
// order that depends on the half); max and sum of the two are symmetric, so
// they do not depend on that order.  A VALU exchange: no LDS round trip.
__device__ __forceinline__ float pair_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Lazy rescaling threshold, in base-2 units of the scaled score.
constexpr float kRescaleSlack = 8.f;
constexpr float kRescaleBound = 256.f;  // 2^kRescaleSlack

// Number of leading keys of a key tile visible to one query: keys kk < limit
// are visible.  `rows` keys are present in the tile; under the causal rule
// key kk (at position kpos0 + kk) is visible iff kk <= qpos - kpos0 = rel.
__device__ __forceinline__ int visible_limit(int rows, int32_t causal, int64_t rel) {
  if (!causal) return rows;
  const int64_t n = rel + 1;
  return n <= 0 ? 0 : (n < rows ? (int)n : rows);
}

// XCD-aware placement of (batch, head) pairs: consecutive workgroups are
// dealt round-robin to the 8 XCDs, so workgroups b, b+8, b+16, ... share an
// XCD and its L2.  Remap so that those get adjacent heads (with GQA, the query
// heads of one key/value head), which then hit the same K/V lines in L2.
__device__ __forceinline__ int32_t xcd_head_swizzle(int32_t bh, int32_t BH) {
  return (BH & 7) == 0 ? (bh & 7) * (BH >> 3) + (bh >> 3) : bh;
}

// Cursor over the live key tiles of one query tile, in ring order.
struct TileCursor {
  int32_t v;   // visit index
  int32_t nv;  // number of visits
  int64_t t;   // tile within the visit
  int64_t nt;  // live tiles in the visit
  Run run;
};

template <int BC>
__device__ __forceinline__ void cursor_settle(TileCursor& c, const Sched& s, int32_t rank,
                                              int64_t qhi) {
  while (c.t >= c.nt) {
    ++c.v;
    if (c.v >= c.nv) return;
    c.run = visit(s, rank, c.v);
    c.nt = live_tiles(c.run, qhi, s.causal, BC);
    c.t = 0;
  }
}

template <int BC>
__device__ __forceinline__ TileCursor cursor_begin(const Sched& s, int32_t rank, int64_t qhi) {
  TileCursor c;
  c.nv = num_visits(s);
  c.v = -1;
  c.t = 0;
  c.nt = 0;
  c.run.row0 = c.run.len = c.run.pos0 = 0;
  cursor_settle<BC>(c, s, rank, qhi);
  return c;
}

// Number of live key tiles of one query tile (what a cursor walks).
template <int BC>
__device__ __forceinline__ int64_t count_live_tiles(const Sched& s, int32_t rank, int64_t qhi) {
  int64_t n = 0;
  const int32_t nv = num_visits(s);
  for (int32_t v = 0; v < nv; ++v) n += live_tiles(visit(s, rank, v), qhi, s.causal, BC);
  return n;
}

// Cursor on live tile number t (0-based) of a query tile, or past the end.
template <int BC>
__device__ __forceinline__ TileCursor cursor_at(const Sched& s, int32_t rank, int64_t qhi,
                                                int64_t t) {
  TileCursor c = cursor_begin<BC>(s, rank, qhi);
  while (c.v < c.nv && t >= c.nt - c.t) {
    t -= c.nt - c.t;
    c.t = c.nt;
    cursor_settle<BC>(c, s, rank, qhi);
  }
  if (c.v < c.nv) c.t += t;
  return c;
}

// Work item of this workgroup: (batch * head, query tile, key split); the
// (batch, head) index runs fastest, then the split, then the query tile.
struct WorkItem {
  int32_t bh, t_lin, split;
};
__device__ __forceinline__ WorkItem work_item_of(uint32_t id, int32_t BH, int32_t n_splits) {
  const uint32_t r = id / (uint32_t)BH;
  WorkItem w;
  w.bh = (int32_t)(id % (uint32_t)BH);
  w.t_lin = (int32_t)(r / (uint32_t)n_splits);
  w.split = (int32_t)(r % (uint32_t)n_splits);
  return w;
}
__device__ __forceinline__ WorkItem work_item(int32_t BH, int32_t n_splits) {
  return work_item_of(blockIdx.x, BH, n_splits);
}

// First live tile of this split and the number of tiles it takes: split s of
// n covers tiles [T s / n, T (s+1) / n) of the T live tiles.
template <int BC>
__device__ __forceinline__ TileCursor split_cursor(const Sched& s, int32_t rank, int64_t qhi,
                                                   int32_t split, int32_t n_splits,
                                                   int64_t* count) {
  const int64_t T = count_live_tiles<BC>(s, rank, qhi);
  if (n_splits == 1) {  // no split: skip the (software) 64-bit divisions
    *count = T;
    return cursor_begin<BC>(s, rank, qhi);
  }
  const int64_t b0 = T * split / n_splits, b1 = T * (split + 1) / n_splits;
  *count = b1 - b0;
  return cursor_at<BC>(s, rank, qhi, b0);
}

template <int BC>
__device__ __forceinline__ void cursor_next(TileCursor& c, const Sched& s, int32_t rank,
                                            int64_t qhi) {
  ++c.t;
  cursor_settle<BC>(c, s, rank, qhi);
}

}  // namespace rattn
