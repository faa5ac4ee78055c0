// bwd.h -- work description and launchers of the backward kernels (HIP path only).
//
// The backward of exact attention recomputes the probabilities from the
// forward's log-sum-exp instead of storing them, and needs, per query row,
// D = rowsum(dO * O) (youngju.dev "Ring Attention" analysis,
// ring_attention_backward):
//   P_ij  = exp(scale s_ij - lse_i)          (0 for a masked pair)
//   dV_j  = sum_i P_ij dO_i
//   dS_ij = P_ij (dO_i . v_j - D_i)
//   dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i
// Two kernels share the pair loop: one owns a tile of query rows and walks
// the visible keys (dQ), the other owns a tile of keys and walks the query
// rows that see them, over every query head of its GQA group (dK, dV).  No
// atomics: every output row is written by exactly one workgroup.
//
// A call covers query rows [q_off, q_off + Nq) of a [B, q_rows, Hq, d]
// tensor (q, dO, lse, D, dQ share that row space) and key rows
// [k_off, k_off + Nk) of a [B, k_rows, Hkv, d] tensor (k, v, dK, dV).  Each
// side is one or two runs of contiguous global positions (the ring layouts:
// a ZigZag shard is two chunks); the causal rule compares positions.
#pragma once
#include <hip/hip_runtime.h>

#include "kcommon.h"

namespace rattn {

struct BwdRun {
  int64_t row0;  // first row, relative to the call's row offset
  int64_t len;
  int64_t pos0;  // global position of row0
};

struct BwdParams {
  int32_t B, Hq, Hkv, group;
  int64_t q_rows, q_off;  // row space of q / dO / lse / D / dQ and this call's first row
  int64_t k_rows, k_off;  // row space of k / v / dK / dV and this call's first row
  float scale;            // multiplies dQ and dK
  float c;                // scale * log2(e): P = exp2(s c - lse log2(e))
  int32_t causal;
  int32_t nq, nk;         // runs in use (1 or 2 each)
  BwdRun q[2], k[2];
  int32_t accumulate;     // 1: fp32 outputs, added to; 0: outputs in the input type
  // Varlen (vl_nseq > 0; B = 1, offsets 0): sequence i owns query rows
  // [vl_q_start[i], +vl_q_len[i]) and key rows [vl_k_start[i], +vl_k_len[i])
  // (device arrays, clamped to q_rows / k_rows), key j at position j, query
  // i at k_len - q_len + i; the runs above are unused.  vl_max_q / vl_max_k
  // bound the lengths (tiles per sequence).
  const int32_t* vl_q_start;
  const int32_t* vl_q_len;
  const int32_t* vl_k_start;
  const int32_t* vl_k_len;
  int32_t vl_nseq;
  int64_t vl_max_q;
  int64_t vl_max_k;
};

// Tile of `br` rows number t over one side's runs (tiles do not straddle runs).
struct BwdTile {
  int64_t row0, rows, pos0;
};
__host__ __device__ __forceinline__ int64_t bwd_tiles(const BwdRun* r, int n, int br) {
  int64_t t = 0;
  for (int i = 0; i < n; ++i) t += (r[i].len + br - 1) / br;
  return t;
}
__host__ __device__ __forceinline__ BwdTile bwd_tile(const BwdRun* r, int n, int br, int64_t t) {
  BwdTile x{0, 0, 0};
  for (int i = 0; i < n; ++i) {
    const int64_t nt = (r[i].len + br - 1) / br;
    if (t < nt) {
      x.row0 = r[i].row0 + t * br;
      x.pos0 = r[i].pos0 + t * br;
      const int64_t rem = r[i].len - t * br;
      x.rows = rem < br ? rem : br;
      return x;
    }
    t -= nt;
  }
  return x;
}

// Work items of the query-stationary (dQ) and key-stationary (dK/dV)
// kernels: tiles of `br` rows of one side, numbered over the runs, or over
// (sequence, tile) in varlen mode.
__host__ __device__ __forceinline__ int64_t bwd_q_tiles(const BwdParams& p, int br) {
  return p.vl_nseq > 0 ? p.vl_nseq * ((p.vl_max_q + br - 1) / br) : bwd_tiles(p.q, p.nq, br);
}
__host__ __device__ __forceinline__ int64_t bwd_k_tiles(const BwdParams& p, int br) {
  return p.vl_nseq > 0 ? p.vl_nseq * ((p.vl_max_k + br - 1) / br) : bwd_tiles(p.k, p.nk, br);
}

// One work item: its tile (rows <= 0: nothing to do) and the runs of the
// other side it pairs with.
struct BwdItem {
  BwdTile tile;
  BwdRun other[2];
  int n_other;
};

#if defined(__HIPCC__)
__device__ __forceinline__ void bwd_seq(const BwdParams& p, int32_t i, int64_t* qs, int64_t* lq,
                                        int64_t* ks, int64_t* lk) {
  *qs = p.vl_q_start[i];
  *lq = p.vl_q_len[i];
  *ks = p.vl_k_start[i];
  *lk = p.vl_k_len[i];
  if (*qs < 0 || *qs > p.q_rows) *lq = 0;
  if (*lq > p.q_rows - *qs) *lq = p.q_rows - *qs;
  if (*lq < 0) *lq = 0;
  if (*ks < 0 || *ks > p.k_rows) *lk = 0;
  if (*lk > p.k_rows - *ks) *lk = p.k_rows - *ks;
  if (*lk < 0) *lk = 0;
}

__device__ __forceinline__ BwdItem bwd_q_item(const BwdParams& p, int br, int64_t t) {
  BwdItem it;
  if (p.vl_nseq <= 0) {
    it.tile = bwd_tile(p.q, p.nq, br, t);
    it.n_other = p.nk;
    it.other[0] = p.k[0];
    it.other[1] = p.k[1];
    return it;
  }
  const int64_t per = (p.vl_max_q + br - 1) / br;
  const int32_t i = (int32_t)(t / per);
  const int64_t lt = t - (int64_t)i * per;
  int64_t qs, lq, ks, lk;
  bwd_seq(p, i, &qs, &lq, &ks, &lk);
  const int64_t rem = lq - lt * br;
  it.tile = BwdTile{qs + lt * br, rem <= 0 ? 0 : (rem < br ? rem : br), lk - lq + lt * br};
  it.other[0] = BwdRun{ks, lk, 0};
  it.other[1] = BwdRun{0, 0, 0};
  it.n_other = lk > 0 ? 1 : 0;
  return it;
}

__device__ __forceinline__ BwdItem bwd_k_item(const BwdParams& p, int br, int64_t t) {
  BwdItem it;
  if (p.vl_nseq <= 0) {
    it.tile = bwd_tile(p.k, p.nk, br, t);
    it.n_other = p.nq;
    it.other[0] = p.q[0];
    it.other[1] = p.q[1];
    return it;
  }
  const int64_t per = (p.vl_max_k + br - 1) / br;
  const int32_t i = (int32_t)(t / per);
  const int64_t lt = t - (int64_t)i * per;
  int64_t qs, lq, ks, lk;
  bwd_seq(p, i, &qs, &lq, &ks, &lk);
  const int64_t rem = lk - lt * br;
  it.tile = BwdTile{ks + lt * br, rem <= 0 ? 0 : (rem < br ? rem : br), lt * br};
  it.other[0] = BwdRun{qs, lq, lk - lq};
  it.other[1] = BwdRun{0, 0, 0};
  it.n_other = lq > 0 ? 1 : 0;
  return it;
}
#endif

// D = rowsum(dO * O) in float32 for `rows` rows of d elements (input type).
hipError_t launch_bwd_delta(int dtype, int d, const void* out, const void* dout, float* delta,
                            int64_t rows, hipStream_t stream);

// dQ and dK/dV with the vector-ALU kernels (every dtype and d).
hipError_t launch_bwd_generic(int dtype, int d, const void* q, const void* k, const void* v,
                              const void* dout, const float* lse, const float* delta, void* dq,
                              void* dk, void* dv, const BwdParams& p, hipStream_t stream);

// dQ and dK/dV on the matrix cores: 16-bit inputs (dtype 1 or 2), d = 128.
hipError_t launch_bwd_mfma(int dtype, const void* q, const void* k, const void* v,
                           const void* dout, const float* lse, const float* delta, void* dq,
                           void* dk, void* dv, const BwdParams& p, hipStream_t stream);

}  // namespace rattn
