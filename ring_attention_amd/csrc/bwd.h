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
