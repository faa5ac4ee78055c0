// fwd_mfma.hip -- 16-bit attention forward on gfx950 matrix cores.
//
// What it computes: for each query row, the online softmax over key tiles
// (guijiagi.com "ring-attention-explained", online softmax section; youngju.dev
// "Ring Attention" analysis, blockwise_attention):
//   m' = max(m, rowmax S), alpha = exp(m - m'), P = exp(S - m'),
//   l' = alpha l + rowsum P, O' = alpha O + P V,
// with O kept unnormalised and divided by l once at the end (yz520gzy
// FlashAttention chapter, FlashAttention-2 deferred normalisation) and P
// rounded to the input type before it multiplies V (the Triton kernel of the
// same chapter casts p to v's type before the second dot).
//
// How, on CDNA4:
//   * A workgroup of 4 wavefronts owns a tile of 128 query rows, 32 per wave;
//     d = 16 (the V^T operand is padded to 32 rows with zeros and only O^T
//     rows 0..15 are stored).  Larger d runs on fwd_mfma128.hip's kernel;
//     the template below is written for any d that is a multiple of 16, and
//     only d = 16 is instantiated.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{bf16,f16}: A = 32 keys x 16 dims read from LDS,
//     B = 16 dims x 32 queries held in registers for the whole tile.  In the
//     32x32 accumulator each lane then holds one query column and 16 key rows,
//     so a row maximum is an in-lane max3 chain plus one exchange with the
//     lane 32 apart, and each lane accumulates its share of the row sum l.
//   * O^T = V^T P^T uses P straight from the score registers as the B operand.
//     The key order of those registers is fixed by the accumulator layout
//     (register r of lane l holds key 8*(r/4) + 4*(l/32) + r%4 of the 32-key
//     block); V^T is stored in LDS with bits 2 and 3 of the key index swapped
//     so that each lane's 8 keys for one MFMA are one 16-byte LDS read.
//   * K and V^T tiles (64 keys) are double-buffered in LDS: the global loads of
//     tile i+1 are issued before the matrix work of tile i and written to the
//     other buffer after it; one barrier per tile.
//   * Exponentials use exp2 with scale*log2(e) folded into one FMA; the
//     running max is kept in that scaled base-2 unit.
//   * Fully masked key tiles are never visited (the schedule walks only the
//     live prefix of each ring block); a wave whose 32 queries all precede a
//     key tile skips its matrix work for that tile; element masks are applied
//     only on diagonal or ragged tiles.
#include "kcommon.h"
#include "launch.h"

namespace rattn {

namespace {

constexpr int kBc = 64;       // keys per tile
constexpr int kThreads = 256;

// Column of key `kk` (0..63) inside a V^T row: swap bits 2 and 3.
__device__ __forceinline__ int vt_col(int kk) {
  return (kk & ~12) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

template <typename TT, int D, bool OUT_F32>
__global__ __launch_bounds__(kThreads, 2) void fwd_mfma_kernel(
    const typename TT::elem* __restrict__ q, const typename TT::elem* __restrict__ k,
    const typename TT::elem* __restrict__ v, void* __restrict__ out, float* __restrict__ lse,
    FwdParams p, Sched s) {
  using E = typename TT::elem;
  using v8 = typename TT::v8;
  using v4 = typename TT::v4;
  constexpr int KP = D + 8;    // K row pitch in LDS (elements)
  constexpr int VP = kBc + 8;  // V^T row pitch in LDS (elements)
  constexpr int CPR = D / 8;   // 16-byte chunks per row
  constexpr int NCH = kBc * CPR;  // 16-byte chunks per tile per tensor
  constexpr int CH = (NCH + kThreads - 1) / kThreads;  // chunks per thread per tensor
  constexpr int KS = D / 16;   // MFMA k-steps for S
  // 32-row blocks of O^T; at d = 16 one block whose rows 16..31 are zero
  constexpr int DB = D >= 32 ? D / 32 : 1;
  constexpr int VROWS = 32 * DB;  // rows of V^T in LDS (>= D)
  static_assert(NCH % kThreads == 0 || NCH < kThreads, "tile/thread mismatch");

  // 16-bit patterns in LDS; read back as MFMA operand vectors.
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kBc * KP];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][VROWS * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;  // which half of the wavefront
  const int l32 = lane & 31;

  // ---- work item -------------------------------------------------------
  const int32_t BH = p.B * p.Hq;
  const WorkItem wi = work_item(BH, p.n_splits);
  const int32_t bh = xcd_head_swizzle(wi.bh, BH);
  const int32_t t_lin = wi.t_lin;
  const int32_t b = bh / p.Hq, hq = bh % p.Hq, hkv = hq / p.group;
  const QTile qt = query_tile(s, t_lin, kMfmaBr);
  if (qt.rows <= 0) return;  // varlen: a tile past the end of its sequence
  const int64_t qhi = qt.pos0 + qt.rows - 1;

  const int wq0 = 32 * wave;                 // first row of this wave in the tile
  const bool wave_active = wq0 < qt.rows;
  const int64_t wave_qlo = qt.pos0 + wq0;
  const int64_t wave_qhi = qt.pos0 + (wq0 + 31 < qt.rows ? wq0 + 31 : qt.rows - 1);
  const int my_q = wq0 + l32;
  const bool q_valid = my_q < qt.rows;
  const int64_t q_pos = qt.pos0 + my_q;

  // ---- Q fragments: B operand, 8 dims per lane per k-step ----------------
  v8 qf[KS];
  {
    const E* qp = q + (((int64_t)b * p.Nq + qt.row0 + my_q) * p.Hq + hq) * D + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (q_valid) {
        qf[ks] = *(const v8*)(qp + 16 * ks);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (E)0.f;
      }
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = kNegInf;  // running max of scaled base-2 scores
  float l_run = 0.f;      // this lane's share of the running sum

  const int64_t kv_stride = (int64_t)p.Hkv * D;
  const E* kbase = k + (int64_t)b * p.Nk * kv_stride + (int64_t)hkv * D;
  const E* vbase = v + (int64_t)b * p.Nk * kv_stride + (int64_t)hkv * D;

  // Per-thread byte offsets of its 16-byte chunks inside a tile, relative to
  // the tile's first row (the tile base is uniform, so every load is one
  // global_load with a scalar base and a 32-bit vector offset).  K chunks run
  // along rows (coalesced); V chunks give each lane one key (for the
  // transposed LDS store).
  uint32_t koff[CH], voff[CH];
  int krow_of[CH], vrow_of[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int ci = (tid + kThreads * i) % NCH;  // threads past NCH repeat a chunk
    krow_of[i] = ci / CPR;
    vrow_of[i] = ci % kBc;
    koff[i] = (uint32_t)((krow_of[i] * kv_stride + (ci % CPR) * 8) * sizeof(E));
    voff[i] = (uint32_t)((vrow_of[i] * kv_stride + (ci / kBc) * 8) * sizeof(E));
  }
  const uint32_t row_bytes = (uint32_t)(kv_stride * sizeof(E));

  uint4 kreg[CH], vreg[CH];

  auto load_tile = [&](const TileCursor& c) {
    const int64_t krow0 = c.run.row0 + c.t * kBc;
    const int64_t rem = c.run.len - c.t * kBc;
    const char* kt = (const char*)(kbase + krow0 * kv_stride);
    const char* vt = (const char*)(vbase + krow0 * kv_stride);
    if (rem >= kBc) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        kreg[i] = *(const uint4*)(kt + koff[i]);
        vreg[i] = *(const uint4*)(vt + voff[i]);
      }
    } else {
      // ragged last tile of a run: rows past its end read the last row
      // (in bounds) and are zeroed, so no score or value comes from them
      const int krows = (int)rem;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int kx = krow_of[i] < krows ? 0 : krow_of[i] - (krows - 1);
        const int vx = vrow_of[i] < krows ? 0 : vrow_of[i] - (krows - 1);
        const uint4 ka = *(const uint4*)(kt + koff[i] - (uint32_t)kx * row_bytes);
        const uint4 va = *(const uint4*)(vt + voff[i] - (uint32_t)vx * row_bytes);
        const uint32_t km = kx ? 0u : ~0u, vm = vx ? 0u : ~0u;
        kreg[i] = make_uint4(ka.x & km, ka.y & km, ka.z & km, ka.w & km);
        vreg[i] = make_uint4(va.x & vm, va.y & vm, va.z & vm, va.w & vm);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ci = tid + kThreads * i;
      if (NCH < kThreads && ci >= NCH) continue;
      const int kr = ci / CPR, kc = ci % CPR;
      *(uint4*)&k_lds[buf][kr * KP + kc * 8] = kreg[i];
      const int vr = ci % kBc, vc = ci / kBc;
      const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
      const int col = vt_col(vr);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        vt_lds[buf][(vc * 8 + e) * VP + col] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  };

  if (VROWS > D) {
    // d = 16: V^T rows D .. 31 of both buffers stay zero (O^T rows 16..31 = 0)
    for (int i = tid; i < 2 * (VROWS - D) * VP; i += kThreads)
      vt_lds[i / ((VROWS - D) * VP)][D * VP + i % ((VROWS - D) * VP)] = 0;
  }
  int64_t left;  // key tiles of this split still to visit
  TileCursor cur = split_cursor<kBc>(s, qt.rank, qhi, wi.split, p.n_splits, &left);
  if (left > 0) {
    load_tile(cur);
    store_tile(0);
  }
  int buf = 0;
  for (; left > 0; --left) {
    TileCursor nxt = cur;
    cursor_next<kBc>(nxt, s, qt.rank, qhi);
    const bool has_next = left > 1;
    if (has_next) load_tile(nxt);
    __syncthreads();

    const int64_t kpos0 = cur.run.pos0 + cur.t * kBc;
    const int64_t rem = cur.run.len - cur.t * kBc;
    const int krows = rem < kBc ? (int)rem : kBc;
    const bool wave_sees = wave_active && (!s.causal || kpos0 <= wave_qhi);
    if (wave_sees) {
      // S^T = K Q^T: two 32-key blocks
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
        const uint16_t* krow = &k_lds[buf][(kb * 32 + l32) * KP + 8 * hl];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sacc[kb] = TT::mfma32x32x16(*(const v8*)(krow + 16 * ks), qf[ks], sacc[kb]);
      }
      // element mask on diagonal / ragged tiles
      const bool need_mask =
          krows < kBc || (s.causal && kpos0 + krows - 1 > wave_qlo);
      if (need_mask) {
        // keys kk < lim of this tile are visible to this lane's query: one
        // clamped 32-bit bound per lane, then a select per score
        const int lim = visible_limit(krows, s.causal, q_pos - kpos0);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            sacc[kb][r] = kk < lim ? sacc[kb][r] : kNegInf;
          }
      }
      // online softmax.  The running max only moves when some row's tile
      // max exceeds it by more than kRescaleSlack (base-2 units); otherwise
      // scores are exponentiated against the stale max, so p <= 2^slack,
      // and the O/l rescale is skipped for the whole wave.  Exact in exact
      // arithmetic: O and l always share one reference max.
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[kb][r]);
      mt = pair_max(mt);
      const float m_cand = mt * p.c;
      if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kRescaleSlack) != 0) {
        const float m_new = fmaxf(m_run, m_cand);
        const float alpha = exp2_fast(m_run - (m_new == kNegInf ? 0.f : m_new));
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      const float m_use = m_run == kNegInf ? 0.f : m_run;
      float rs = 0.f;
      v8 pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = exp2_fast(fmaf(sacc[kb][r], p.c, -m_use));
          rs += pr;
          pf[2 * kb + (r >> 3)][r & 7] = to_elem<TT>(pr);
        }
      l_run += rs;
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vrow = &vt_lds[buf][(db * 32 + l32) * VP + 8 * hl];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          oacc[db] = TT::mfma32x32x16(*(const v8*)(vrow + 16 * u), pf[u], oacc[db]);
      }
    }
    if (has_next) store_tile(buf ^ 1);
    buf ^= 1;
    cur = nxt;
  }

  // ---- epilogue: O / l, LSE = m ln2 + ln l --------------------------------
  const float l_tot = pair_sum(l_run);
  if (!q_valid) return;
  const bool seen = l_tot > 0.f;
  const float inv = seen ? 1.f / l_tot : 0.f;
  const float lse_n = seen ? m_run * kLn2 + logf(l_tot) : kNegInf;
  const int64_t orow = ((int64_t)b * p.out_rows + p.out_row_off + qt.row0 + my_q) * p.Hq + hq;
  float* out_f = (float*)out + wi.split * p.split_out_stride;
  float* lse_w = lse + wi.split * p.split_lse_stride;
  const bool merging = OUT_F32 && p.merge_out;
  const MergeW mw = merging ? merge_weights(lse_w[orow], lse_n) : MergeW{0.f, 1.f, lse_n};
  const float f_n = mw.f_n * inv;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (32 * db + 8 * j >= D) continue;  // d = 16: only O^T rows 0..15 exist
      const int d0 = 32 * db + 8 * j + 4 * hl;
      if (OUT_F32) {
        f32x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = oacc[db][4 * j + e] * f_n;
        f32x4* dst = (f32x4*)(out_f + orow * D + d0);
        if (merging) o4 += *dst * mw.f_r;
        *dst = o4;
      } else {
        v4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = to_elem<TT>(oacc[db][4 * j + e] * inv);
        *(v4*)((E*)out + orow * D + d0) = o4;
      }
    }
  if (hl == 0) lse_w[orow] = mw.lse;
}

template <typename TT, int D>
hipError_t launch_t(const void* q, const void* k, const void* v, void* out, float* lse,
                    bool out_f32, const FwdParams& p, const Sched& s, hipStream_t stream) {
  using E = typename TT::elem;
  const int64_t blocks = (int64_t)s.n_tiles * p.B * p.Hq * p.n_splits;
  if (blocks <= 0) return hipSuccess;
  if (out_f32)
    hipLaunchKernelGGL((fwd_mfma_kernel<TT, D, true>), dim3((unsigned)blocks), dim3(kThreads),
                       0, stream, (const E*)q, (const E*)k, (const E*)v, out, lse, p, s);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<TT, D, false>), dim3((unsigned)blocks), dim3(kThreads),
                       0, stream, (const E*)q, (const E*)k, (const E*)v, out, lse, p, s);
  return hipGetLastError();
}

template <typename TT>
hipError_t launch_d(int d, const void* q, const void* k, const void* v, void* out, float* lse,
                    bool out_f32, const FwdParams& p, const Sched& s, hipStream_t stream) {
  if (d == 16) return launch_t<TT, 16>(q, k, v, out, lse, out_f32, p, s, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_mfma(int dtype, int d, const void* q, const void* k, const void* v,
                           void* out, float* lse, bool out_f32, const FwdParams& p,
                           const Sched& s, uint32_t* queues, hipStream_t stream) {
  if (d >= 32)
    return launch_fwd_mfma128(dtype, d, q, k, v, out, lse, out_f32, p, s, queues, stream);
  switch (dtype) {
    case 1: return launch_d<F16>(d, q, k, v, out, lse, out_f32, p, s, stream);
    case 2: return launch_d<Bf16>(d, q, k, v, out, lse, out_f32, p, s, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rattn
