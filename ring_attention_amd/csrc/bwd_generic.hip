// bwd_generic.hip -- D = rowsum(dO * O) and the vector-ALU backward kernels.
//
// The recomputation backward of the youngju.dev "Ring Attention" analysis
// (ring_attention_backward): P is rebuilt from the forward's log-sum-exp as
// exp2(scale log2(e) s - lse log2(e)), D = rowsum(dO * O) is formed once per
// query row, dS = P (dP - D), and the scale is applied to dQ and dK once at
// the end.  All arithmetic in float32.  These kernels carry every dtype and
// head dim; they are the float32 path (the 16-bit inputs at the sizes that
// matter run on the matrix-core kernels).
//
// A row of d values is spread over LP = max(1, d/32) neighbouring lanes (at
// most 32 values per lane, so q, dO and the dQ accumulator of a row stay in
// registers); dot products are summed across those lanes with xor shuffles.
#include "bwd.h"

namespace rattn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename E>
__device__ __forceinline__ float ld(const E* p) {
  return (float)*p;
}

// ---- D = rowsum(dO * O) --------------------------------------------------
// L = d / CH lanes per row, CH elements (16 bytes) per lane.
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const E* __restrict__ out,
                                                        const E* __restrict__ dout,
                                                        float* __restrict__ delta, int64_t rows) {
  constexpr int CH = 16 / sizeof(E);
  constexpr int L = D / CH;
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "lanes per row");
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / L;
  const int part = (int)(gid % L);
  float acc = 0.f;
  if (row < rows) {
    const E* o = out + row * D + part * CH;
    const E* g = dout + row * D + part * CH;
    E ov[CH], gv[CH];
    *(uint4*)ov = *(const uint4*)o;
    *(uint4*)gv = *(const uint4*)g;
#pragma unroll
    for (int e = 0; e < CH; ++e) acc = fmaf((float)ov[e], (float)gv[e], acc);
  }
#pragma unroll
  for (int o = 1; o < L; o <<= 1) acc += __shfl_xor(acc, o);
  if (row < rows && part == 0) delta[row] = acc;
}

template <int D>
struct RowSplit {
  static constexpr int LP = D >= 64 ? D / 32 : 1;  // lanes per row
  static constexpr int DL = D / LP;                // values per lane
  static constexpr int PAD = DL + 1;               // LDS stride of one lane's slice
};

// LDS tile of BC rows x D floats, each row split into LP slices of DL
// values with a one-float pad between slices (the LP lanes of a row read
// different banks).
template <int D, int BC>
struct RowTile {
  float x[BC][RowSplit<D>::LP][RowSplit<D>::PAD];
};

template <typename E, int D, int BC>
__device__ __forceinline__ void load_tile(RowTile<D, BC>& t, const E* base, int64_t row_stride,
                                          int rows) {
  using S = RowSplit<D>;
  for (int e = threadIdx.x; e < BC * D; e += blockDim.x) {
    const int r = e / D, col = e % D;
    t.x[r][col / S::DL][col % S::DL] = r < rows ? ld(base + r * row_stride + col) : 0.f;
  }
}

template <int LP>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int o = 1; o < LP; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// ---- dQ: one workgroup per tile of query rows ------------------------------
template <typename TT, int D, bool ACC>
__global__ __launch_bounds__(256) void bwd_dq_generic_kernel(
    const typename TT::elem* __restrict__ q, const typename TT::elem* __restrict__ k,
    const typename TT::elem* __restrict__ v, const typename TT::elem* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, void* __restrict__ dq,
    BwdParams p) {
  using E = typename TT::elem;
  using S = RowSplit<D>;
  constexpr int RQ = 256 / S::LP;
  constexpr int BC = 32;
  __shared__ RowTile<D, BC> kt, vt;

  const int32_t BH = p.B * p.Hq;
  const int32_t bh = blockIdx.x % BH;
  const int64_t tl = blockIdx.x / BH;
  const int32_t b = bh / p.Hq, hq = bh % p.Hq, hkv = hq / p.group;
  const BwdItem item = bwd_q_item(p, RQ, tl);
  if (item.tile.rows <= 0) return;  // varlen: a tile past the end of its sequence
  const BwdTile qt = item.tile;
  const int r = threadIdx.x / S::LP, part = threadIdx.x % S::LP;
  const bool valid = r < qt.rows;
  const int64_t qpos = qt.pos0 + r;
  const int64_t qhi = qt.pos0 + qt.rows - 1;
  const int64_t row = ((int64_t)b * p.q_rows + p.q_off + qt.row0 + (valid ? r : 0)) * p.Hq + hq;

  float qv[S::DL], gv[S::DL], acc[S::DL];
#pragma unroll
  for (int t = 0; t < S::DL; ++t) {
    qv[t] = valid ? ld(q + row * D + part * S::DL + t) : 0.f;
    gv[t] = valid ? ld(dout + row * D + part * S::DL + t) : 0.f;
    acc[t] = 0.f;
  }
  const float lse2 = valid ? lse[row] * kLog2e : kNegInf;
  const float dl = valid ? delta[row] : 0.f;
  const bool live = lse2 != kNegInf;  // a row that saw no key has P = 0 everywhere

  const int64_t kstride = (int64_t)p.Hkv * D;
  for (int ri = 0; ri < item.n_other; ++ri) {
    const BwdRun r = ri == 0 ? item.other[0] : item.other[1];  // no runtime-indexed array
    const Run run{r.row0, r.len, r.pos0};
    const int64_t nt = live_tiles(run, qhi, p.causal, BC);
    for (int64_t t = 0; t < nt; ++t) {
      const int64_t krow0 = p.k_off + run.row0 + t * BC;
      const int64_t kpos0 = run.pos0 + t * BC;
      const int64_t rem = run.len - t * BC;
      const int krows = rem < BC ? (int)rem : BC;
      const int64_t kbase = ((int64_t)b * p.k_rows + krow0) * kstride + (int64_t)hkv * D;
      __syncthreads();
      load_tile<E, D, BC>(kt, k + kbase, kstride, krows);
      load_tile<E, D, BC>(vt, v + kbase, kstride, krows);
      __syncthreads();
      const int lim = live ? visible_limit(krows, p.causal, qpos - kpos0) : 0;
      for (int j = 0; j < BC; ++j) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int t2 = 0; t2 < S::DL; ++t2) {
          s = fmaf(qv[t2], kt.x[j][part][t2], s);
          dp = fmaf(gv[t2], vt.x[j][part][t2], dp);
        }
        s = row_sum<S::LP>(s);
        dp = row_sum<S::LP>(dp);
        const float pr = j < lim ? exp2f(s * p.c - lse2) : 0.f;
        const float ds = pr * (dp - dl);
#pragma unroll
        for (int t2 = 0; t2 < S::DL; ++t2) acc[t2] = fmaf(ds, kt.x[j][part][t2], acc[t2]);
      }
    }
  }
  if (!valid) return;
  if (ACC) {
    float* o = (float*)dq + row * D + part * S::DL;
#pragma unroll
    for (int t = 0; t < S::DL; ++t) o[t] += acc[t] * p.scale;
  } else {
    E* o = (E*)dq + row * D + part * S::DL;
#pragma unroll
    for (int t = 0; t < S::DL; ++t) o[t] = (E)(acc[t] * p.scale);
  }
}

// ---- dK, dV: one workgroup per tile of keys --------------------------------
template <typename TT, int D, bool ACC>
__global__ __launch_bounds__(256) void bwd_dkv_generic_kernel(
    const typename TT::elem* __restrict__ q, const typename TT::elem* __restrict__ k,
    const typename TT::elem* __restrict__ v, const typename TT::elem* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, void* __restrict__ dk,
    void* __restrict__ dv, BwdParams p) {
  using E = typename TT::elem;
  using S = RowSplit<D>;
  constexpr int RK = 256 / S::LP;
  constexpr int BC = 32;
  __shared__ RowTile<D, BC> qt_l, gt_l;
  __shared__ float lse_l[BC], dl_l[BC];

  const int32_t BH = p.B * p.Hkv;
  const int32_t bh = blockIdx.x % BH;
  const int64_t tl = blockIdx.x / BH;
  const int32_t b = bh / p.Hkv, hkv = bh % p.Hkv;
  const BwdItem item = bwd_k_item(p, RK, tl);
  if (item.tile.rows <= 0) return;  // varlen: a tile past the end of its sequence
  const BwdTile kt = item.tile;
  const int r = threadIdx.x / S::LP, part = threadIdx.x % S::LP;
  const bool valid = r < kt.rows;
  const int64_t kpos = kt.pos0 + r;
  const int64_t krow = ((int64_t)b * p.k_rows + p.k_off + kt.row0 + (valid ? r : 0)) * p.Hkv + hkv;

  float kv[S::DL], vv[S::DL], ak[S::DL], av[S::DL];
#pragma unroll
  for (int t = 0; t < S::DL; ++t) {
    kv[t] = valid ? ld(k + krow * D + part * S::DL + t) : 0.f;
    vv[t] = valid ? ld(v + krow * D + part * S::DL + t) : 0.f;
    ak[t] = av[t] = 0.f;
  }

  const int64_t qstride = (int64_t)p.Hq * D;
  for (int g = 0; g < p.group; ++g) {
    const int32_t hq = hkv * p.group + g;
    for (int ri = 0; ri < item.n_other; ++ri) {
      const BwdRun run = ri == 0 ? item.other[0] : item.other[1];
      // query rows before the tile's first key position see none of its keys
      int64_t start = 0;
      if (p.causal) {
        start = kt.pos0 - run.pos0;
        start = start < 0 ? 0 : (start > run.len ? run.len : start);
      }
      for (int64_t i0 = start; i0 < run.len; i0 += BC) {
        const int64_t rem = run.len - i0;
        const int qrows = rem < BC ? (int)rem : BC;
        const int64_t qpos0 = run.pos0 + i0;
        const int64_t qrow0 = (int64_t)b * p.q_rows + p.q_off + run.row0 + i0;
        __syncthreads();
        load_tile<E, D, BC>(qt_l, q + qrow0 * qstride + (int64_t)hq * D, qstride, qrows);
        load_tile<E, D, BC>(gt_l, dout + qrow0 * qstride + (int64_t)hq * D, qstride, qrows);
        if (threadIdx.x < BC) {
          const int i = threadIdx.x;
          const int64_t lr = (qrow0 + i) * p.Hq + hq;
          lse_l[i] = i < qrows ? lse[lr] * kLog2e : kNegInf;
          dl_l[i] = i < qrows ? delta[lr] : 0.f;
        }
        __syncthreads();
        for (int i = 0; i < BC; ++i) {
          float s = 0.f, dp = 0.f;
#pragma unroll
          for (int t2 = 0; t2 < S::DL; ++t2) {
            s = fmaf(kv[t2], qt_l.x[i][part][t2], s);
            dp = fmaf(vv[t2], gt_l.x[i][part][t2], dp);
          }
          s = row_sum<S::LP>(s);
          dp = row_sum<S::LP>(dp);
          const float l2 = lse_l[i];
          const bool vis = l2 != kNegInf && (!p.causal || kpos <= qpos0 + i);
          const float pr = vis ? exp2f(s * p.c - l2) : 0.f;
          const float ds = pr * (dp - dl_l[i]);
#pragma unroll
          for (int t2 = 0; t2 < S::DL; ++t2) {
            ak[t2] = fmaf(ds, qt_l.x[i][part][t2], ak[t2]);
            av[t2] = fmaf(pr, gt_l.x[i][part][t2], av[t2]);
          }
        }
      }
    }
  }
  if (!valid) return;
  if (ACC) {
    float* ok = (float*)dk + krow * D + part * S::DL;
    float* ov = (float*)dv + krow * D + part * S::DL;
#pragma unroll
    for (int t = 0; t < S::DL; ++t) {
      ok[t] += ak[t] * p.scale;
      ov[t] += av[t];
    }
  } else {
    E* ok = (E*)dk + krow * D + part * S::DL;
    E* ov = (E*)dv + krow * D + part * S::DL;
#pragma unroll
    for (int t = 0; t < S::DL; ++t) {
      ok[t] = (E)(ak[t] * p.scale);
      ov[t] = (E)av[t];
    }
  }
}

template <typename E, int D>
hipError_t delta_t(const void* out, const void* dout, float* delta, int64_t rows,
                   hipStream_t stream) {
  constexpr int L = D / (16 / sizeof(E));
  const int64_t blocks = (rows * L + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_delta_kernel<E, D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const E*)out, (const E*)dout, delta, rows);
  return hipGetLastError();
}

template <typename E>
hipError_t delta_d(int d, const void* out, const void* dout, float* delta, int64_t rows,
                   hipStream_t stream) {
  switch (d) {
    case 16: return delta_t<E, 16>(out, dout, delta, rows, stream);
    case 32: return delta_t<E, 32>(out, dout, delta, rows, stream);
    case 64: return delta_t<E, 64>(out, dout, delta, rows, stream);
    case 128: return delta_t<E, 128>(out, dout, delta, rows, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename TT, int D, bool ACC>
hipError_t generic_acc(const void* q, const void* k, const void* v, const void* dout,
                       const float* lse, const float* delta, void* dq, void* dk, void* dv,
                       const BwdParams& p, hipStream_t stream) {
  using E = typename TT::elem;
  using S = RowSplit<D>;
  const int64_t qb = bwd_q_tiles(p, 256 / S::LP) * p.B * p.Hq;
  if (qb > 0) {
    hipLaunchKernelGGL((bwd_dq_generic_kernel<TT, D, ACC>), dim3((unsigned)qb), dim3(256), 0,
                       stream, (const E*)q, (const E*)k, (const E*)v, (const E*)dout, lse, delta,
                       dq, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t kb = bwd_k_tiles(p, 256 / S::LP) * p.B * p.Hkv;
  if (kb > 0) {
    hipLaunchKernelGGL((bwd_dkv_generic_kernel<TT, D, ACC>), dim3((unsigned)kb), dim3(256), 0,
                       stream, (const E*)q, (const E*)k, (const E*)v, (const E*)dout, lse, delta,
                       dk, dv, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename TT, int D>
hipError_t generic_t(const void* q, const void* k, const void* v, const void* dout,
                     const float* lse, const float* delta, void* dq, void* dk, void* dv,
                     const BwdParams& p, hipStream_t stream) {
  return p.accumulate
             ? generic_acc<TT, D, true>(q, k, v, dout, lse, delta, dq, dk, dv, p, stream)
             : generic_acc<TT, D, false>(q, k, v, dout, lse, delta, dq, dk, dv, p, stream);
}

template <typename TT>
hipError_t generic_d(int d, const void* q, const void* k, const void* v, const void* dout,
                     const float* lse, const float* delta, void* dq, void* dk, void* dv,
                     const BwdParams& p, hipStream_t stream) {
  switch (d) {
    case 16: return generic_t<TT, 16>(q, k, v, dout, lse, delta, dq, dk, dv, p, stream);
    case 32: return generic_t<TT, 32>(q, k, v, dout, lse, delta, dq, dk, dv, p, stream);
    case 64: return generic_t<TT, 64>(q, k, v, dout, lse, delta, dq, dk, dv, p, stream);
    case 128: return generic_t<TT, 128>(q, k, v, dout, lse, delta, dq, dk, dv, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_bwd_delta(int dtype, int d, const void* out, const void* dout, float* delta,
                            int64_t rows, hipStream_t stream) {
  switch (dtype) {
    case 0: return delta_d<float>(d, out, dout, delta, rows, stream);
    case 1: return delta_d<_Float16>(d, out, dout, delta, rows, stream);
    case 2: return delta_d<__bf16>(d, out, dout, delta, rows, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd_generic(int dtype, int d, const void* q, const void* k, const void* v,
                              const void* dout, const float* lse, const float* delta, void* dq,
                              void* dk, void* dv, const BwdParams& p, hipStream_t stream) {
  switch (dtype) {
    case 0: return generic_d<F32>(d, q, k, v, dout, lse, delta, dq, dk, dv, p, stream);
    case 1: return generic_d<F16>(d, q, k, v, dout, lse, delta, dq, dk, dv, p, stream);
    case 2: return generic_d<Bf16>(d, q, k, v, dout, lse, delta, dq, dk, dv, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rattn
