// merge.hip -- log-sum-exp merge of two partial attention results (HBM-bound).
//
// For every row, (out, lse) <- (out, lse) (+) (blk_out, blk_lse):
//   m = max(lse, blk_lse);  w_a = exp(lse - m);  w_b = exp(blk_lse - m)
//   out' = (w_a out + w_b blk_out) / (w_a + w_b);  lse' = m + log(w_a + w_b)
// This is the log-sum-exp correction the Twinkle page ("Sequence parallel and
// Ring Attention", forward pass, update_out_and_lse) applies after each ring
// step, written in max-shifted form instead of its sigmoid form: both are the
// same function for finite inputs, and this one also covers an empty side
// (lse = -inf contributes weight 0; two empty sides give out 0, lse -inf),
// where the sigmoid form yields NaN.
//
// d/4 lanes of one wavefront share a row, each moving 16 bytes of out and of
// blk_out, so the read of lse and its in-place rewrite happen in the same
// wavefront instruction stream (no cross-wave race on lse).
#include "launch.h"

namespace rattn {

namespace {

template <int D>
__global__ __launch_bounds__(256) void merge_kernel(float* __restrict__ out,
                                                    float* __restrict__ lse,
                                                    const float* __restrict__ blk_out,
                                                    const float* __restrict__ blk_lse, int32_t H,
                                                    int64_t Nq, int64_t Nb, int64_t row_off,
                                                    int64_t total_rows) {
  constexpr int LPR = D / 4;  // lanes per row
  static_assert(64 % LPR == 0, "a row must not straddle wavefronts");
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = g / LPR;
  const int c4 = (int)(g % LPR);
  if (row >= total_rows) return;
  const int64_t h = row % H;
  const int64_t i = (row / H) % Nb;
  const int64_t b = row / ((int64_t)H * Nb);
  const int64_t orow = (b * Nq + row_off + i) * H + h;

  const float la = lse[orow];
  const float lb = blk_lse[row];
  const float m = fmaxf(la, lb);
  f32x4 o;
  float l_new;
  if (m == kNegInf) {
    o = f32x4{0.f, 0.f, 0.f, 0.f};
    l_new = kNegInf;
  } else {
    const float wa = expf(la - m), wb = expf(lb - m);
    const float z = wa + wb;
    const float fa = wa / z, fb = wb / z;
    const f32x4 oa = *(const f32x4*)(out + orow * D + 4 * c4);
    const f32x4 ob = *(const f32x4*)(blk_out + row * D + 4 * c4);
    o = oa * fa + ob * fb;
    l_new = m + logf(z);
  }
  *(f32x4*)(out + orow * D + 4 * c4) = o;
  if (c4 == 0) lse[orow] = l_new;
}

// n-way form for split-KV: rows = B*Nq*H; split s holds its normalised
// partial at ws_out + s*rows*D and its lse at ws_lse + s*rows.  out gets the
// merged result in the input type, lse the merged lse.
template <typename TT, int D>
__global__ __launch_bounds__(256) void split_reduce_kernel(void* __restrict__ out,
                                                           float* __restrict__ lse,
                                                           const float* __restrict__ ws_out,
                                                           const float* __restrict__ ws_lse,
                                                           int32_t n_splits, int64_t rows) {
  constexpr int LPR = D / 4;
  static_assert(64 % LPR == 0, "a row must not straddle wavefronts");
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = g / LPR;
  const int c4 = (int)(g % LPR);
  if (row >= rows) return;
  float m = kNegInf;
  for (int32_t s = 0; s < n_splits; ++s) m = fmaxf(m, ws_lse[s * rows + row]);
  f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
  float l_new = kNegInf;
  if (m != kNegInf) {
    float z = 0.f;
    for (int32_t s = 0; s < n_splits; ++s) {
      const float w = expf(ws_lse[s * rows + row] - m);
      z += w;
      o += *(const f32x4*)(ws_out + (s * rows + row) * D + 4 * c4) * w;
    }
    o *= 1.f / z;
    l_new = m + logf(z);
  }
  if constexpr (sizeof(typename TT::elem) == 4) {
    *(f32x4*)((float*)out + row * D + 4 * c4) = o;
  } else {
    typedef typename TT::elem E;
    typedef E e4 __attribute__((ext_vector_type(4)));
    e4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = to_elem<TT>(o[e]);
    *(e4*)((E*)out + row * D + 4 * c4) = v;
  }
  if (c4 == 0) lse[row] = l_new;
}

template <typename TT, int D>
hipError_t launch_reduce(void* out, float* lse, const float* ws_out, const float* ws_lse,
                         int n_splits, int64_t rows, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t blocks = (rows * (D / 4) + 255) / 256;
  hipLaunchKernelGGL((split_reduce_kernel<TT, D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     out, lse, ws_out, ws_lse, (int32_t)n_splits, rows);
  return hipGetLastError();
}

template <typename TT>
hipError_t launch_reduce_t(int d, void* out, float* lse, const float* ws_out,
                           const float* ws_lse, int n_splits, int64_t rows, hipStream_t stream) {
  switch (d) {
    case 16: return launch_reduce<TT, 16>(out, lse, ws_out, ws_lse, n_splits, rows, stream);
    case 32: return launch_reduce<TT, 32>(out, lse, ws_out, ws_lse, n_splits, rows, stream);
    case 64: return launch_reduce<TT, 64>(out, lse, ws_out, ws_lse, n_splits, rows, stream);
    case 128: return launch_reduce<TT, 128>(out, lse, ws_out, ws_lse, n_splits, rows, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_d(float* out, float* lse, const float* blk_out, const float* blk_lse, int B,
                    int H, int64_t Nq, int64_t Nb, int64_t row_off, hipStream_t stream) {
  const int64_t rows = (int64_t)B * Nb * H;
  if (rows == 0) return hipSuccess;
  const int64_t threads = rows * (D / 4);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, stream, out, lse,
                     blk_out, blk_lse, (int32_t)H, Nq, Nb, row_off, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_merge(float* out, float* lse, const float* blk_out, const float* blk_lse,
                        int B, int H, int64_t Nq, int64_t Nb, int64_t row_off, int d,
                        hipStream_t stream) {
  switch (d) {
    case 16: return launch_d<16>(out, lse, blk_out, blk_lse, B, H, Nq, Nb, row_off, stream);
    case 32: return launch_d<32>(out, lse, blk_out, blk_lse, B, H, Nq, Nb, row_off, stream);
    case 64: return launch_d<64>(out, lse, blk_out, blk_lse, B, H, Nq, Nb, row_off, stream);
    case 128: return launch_d<128>(out, lse, blk_out, blk_lse, B, H, Nq, Nb, row_off, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_split_reduce(int dtype, int d, void* out, float* lse, const float* ws_out,
                               const float* ws_lse, int n_splits, int64_t rows,
                               hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_reduce_t<F32>(d, out, lse, ws_out, ws_lse, n_splits, rows, stream);
    case 1: return launch_reduce_t<F16>(d, out, lse, ws_out, ws_lse, n_splits, rows, stream);
    case 2: return launch_reduce_t<Bf16>(d, out, lse, ws_out, ws_lse, n_splits, rows, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rattn
