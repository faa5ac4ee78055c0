// fwd_generic.hip -- plain vector-ALU forward kernel (any supported d and dtype).
//
// One wavefront per tile of 64 query rows, one lane per query row.  Key/value
// tiles of 32 rows are staged in LDS as float32 and read by broadcast.  Each
// lane runs the online softmax of its row over groups of 8 keys:
//   m' = max(m, max_j s_j),  alpha = exp(m - m'),  p_j = exp(s_j - m'),
//   l' = alpha l + sum_j p_j,  O' = alpha O + sum_j p_j v_j
// (youngju.dev "Ring Attention" analysis, blockwise_attention; guijiagi.com
// "ring-attention-explained", online softmax section), with the division by l
// deferred to the end (yz520gzy FlashAttention chapter, FlashAttention-2).
// Scores are exponentiated as exp2(s*scale*log2(e) - m) with m kept in that
// scaled base-2 unit.  For 16-bit inputs p is rounded to the input type before
// it multiplies V, as the Triton kernel of the yz520gzy chapter does; l keeps
// the unrounded p.  This kernel carries the float32 path; the MFMA kernels
// carry every 16-bit case (the 16-bit branches here are kept for completeness).
#include "kcommon.h"
#include "launch.h"

namespace rattn {

template <typename TT, int D, bool OUT_F32>
__global__ __launch_bounds__(64) void fwd_generic_kernel(
    const typename TT::elem* __restrict__ q, const typename TT::elem* __restrict__ k,
    const typename TT::elem* __restrict__ v, void* __restrict__ out, float* __restrict__ lse,
    FwdParams p, Sched s) {
  using E = typename TT::elem;
  constexpr int BC = 32;
  constexpr int G = 8;  // keys per online-softmax update
  __shared__ float k_lds[BC][D];
  __shared__ float v_lds[BC][D];

  const int lane = threadIdx.x;
  const int32_t BH = p.B * p.Hq;
  const WorkItem wi = work_item(BH, p.n_splits);
  const int32_t bh = wi.bh;
  const int32_t t_lin = wi.t_lin;
  const int32_t b = bh / p.Hq, hq = bh % p.Hq, hkv = hq / p.group;
  const QTile qt = query_tile(s, t_lin, kGenericBr);
  if (qt.rows <= 0) return;  // varlen: a tile past the end of its sequence

  const bool q_valid = lane < qt.rows;
  const int64_t q_pos = qt.pos0 + lane;
  const int64_t qhi = qt.pos0 + qt.rows - 1;

  float qv[D];
  float acc[D];
  const int64_t q_off = (((int64_t)b * p.Nq + qt.row0 + lane) * p.Hq + hq) * D;
#pragma unroll
  for (int t = 0; t < D; ++t) {
    qv[t] = q_valid ? (float)q[q_off + t] : 0.f;
    acc[t] = 0.f;
  }
  float m = kNegInf, l = 0.f;

  int64_t left;  // key tiles of this split still to visit
  TileCursor cur = split_cursor<BC>(s, qt.rank, qhi, wi.split, p.n_splits, &left);
  for (; left > 0; --left) {
    const int64_t krow0 = cur.run.row0 + cur.t * BC;
    const int64_t kpos0 = cur.run.pos0 + cur.t * BC;
    const int64_t rem = cur.run.len - cur.t * BC;
    const int krows = rem < BC ? (int)rem : BC;

    __syncthreads();
    for (int e = lane; e < BC * D; e += 64) {
      const int r = e / D, col = e % D;
      float kx = 0.f, vx = 0.f;
      if (r < krows) {
        const int64_t off = (((int64_t)b * p.Nk + krow0 + r) * p.Hkv + hkv) * D + col;
        kx = (float)k[off];
        vx = (float)v[off];
      }
      k_lds[r][col] = kx;
      v_lds[r][col] = vx;
    }
    __syncthreads();

    const int lim = visible_limit(krows, s.causal, q_pos - kpos0);
    for (int j0 = 0; j0 < BC; j0 += G) {
      float sc[G];
      float gmax = kNegInf;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int t = 0; t < D; ++t) dot = fmaf(qv[t], k_lds[j0 + j][t], dot);
        sc[j] = j0 + j < lim ? dot * p.c : kNegInf;
        gmax = fmaxf(gmax, sc[j]);
      }
      const float m_new = fmaxf(m, gmax);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = exp2f(m - m_use);
      l *= alpha;
#pragma unroll
      for (int t = 0; t < D; ++t) acc[t] *= alpha;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float pj = exp2f(sc[j] - m_use);
        l += pj;
        const float pv = (float)to_elem<TT>(pj);
#pragma unroll
        for (int t = 0; t < D; ++t) acc[t] = fmaf(pv, v_lds[j0 + j][t], acc[t]);
      }
      m = m_new;
    }
    cursor_next<BC>(cur, s, qt.rank, qhi);
  }

  if (!q_valid) return;
  const bool seen = l > 0.f;
  const float inv = seen ? 1.f / l : 0.f;
  const float lse_n = seen ? m * kLn2 + logf(l) : kNegInf;
  const int64_t orow = ((int64_t)b * p.out_rows + p.out_row_off + qt.row0 + lane) * p.Hq + hq;
  const int64_t o_off = orow * D;
  float* lse_w = lse + wi.split * p.split_lse_stride;
  const bool merging = OUT_F32 && p.merge_out;
  const MergeW mw = merging ? merge_weights(lse_w[orow], lse_n) : MergeW{0.f, 1.f, lse_n};
  if (OUT_F32) {
    float* o = (float*)out + wi.split * p.split_out_stride + o_off;
    const float f_n = mw.f_n * inv;
    if (merging) {
#pragma unroll
      for (int t = 0; t < D; ++t) o[t] = acc[t] * f_n + o[t] * mw.f_r;
    } else {
#pragma unroll
      for (int t = 0; t < D; ++t) o[t] = acc[t] * f_n;
    }
  } else {
    E* o = (E*)out + o_off;
#pragma unroll
    for (int t = 0; t < D; ++t) o[t] = to_elem<TT>(acc[t] * inv);
  }
  lse_w[orow] = mw.lse;
}

// Host-side launchers (declared in launch.h).
template <typename TT, int D>
static hipError_t launch_generic_t(const void* q, const void* k, const void* v, void* out,
                                   float* lse, bool out_f32, const FwdParams& p,
                                   const Sched& s, hipStream_t stream) {
  using E = typename TT::elem;
  const int64_t blocks = (int64_t)s.n_tiles * p.B * p.Hq * p.n_splits;
  if (blocks <= 0) return hipSuccess;
  if (out_f32)
    hipLaunchKernelGGL((fwd_generic_kernel<TT, D, true>), dim3((unsigned)blocks), dim3(64), 0,
                       stream, (const E*)q, (const E*)k, (const E*)v, out, lse, p, s);
  else
    hipLaunchKernelGGL((fwd_generic_kernel<TT, D, false>), dim3((unsigned)blocks), dim3(64), 0,
                       stream, (const E*)q, (const E*)k, (const E*)v, out, lse, p, s);
  return hipGetLastError();
}

template <typename TT>
static hipError_t launch_generic_d(int d, const void* q, const void* k, const void* v, void* out,
                                   float* lse, bool out_f32, const FwdParams& p,
                                   const Sched& s, hipStream_t stream) {
  switch (d) {
    case 16: return launch_generic_t<TT, 16>(q, k, v, out, lse, out_f32, p, s, stream);
    case 32: return launch_generic_t<TT, 32>(q, k, v, out, lse, out_f32, p, s, stream);
    case 64: return launch_generic_t<TT, 64>(q, k, v, out, lse, out_f32, p, s, stream);
    case 128: return launch_generic_t<TT, 128>(q, k, v, out, lse, out_f32, p, s, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_generic(int dtype, int d, const void* q, const void* k, const void* v,
                              void* out, float* lse, bool out_f32, const FwdParams& p,
                              const Sched& s, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_generic_d<F32>(d, q, k, v, out, lse, out_f32, p, s, stream);
    case 1: return launch_generic_d<F16>(d, q, k, v, out, lse, out_f32, p, s, stream);
    case 2: return launch_generic_d<Bf16>(d, q, k, v, out, lse, out_f32, p, s, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rattn
