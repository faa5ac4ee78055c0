// fwd_mfma128.hip -- the d = 128 attention forward on gfx950 matrix cores.
//
// Same method as fwd_mfma.hip (online softmax over key tiles with a running
// max m, running sum l and unnormalised O, P rounded to the input type before
// PV, O/l once at the end -- guijiagi.com "ring-attention-explained", online
// softmax section; yz520gzy FlashAttention chapter, FlashAttention-2 and its
// Triton kernel), with a data path built for head dimension 128:
//
//   * K and V tiles (64 keys x 128 dims, 16 KB each) move global -> LDS by
//     direct-to-LDS DMA (global_load_lds_dwordx4): each wave instruction
//     writes 1 KB = 4 rows, lane l to LDS byte 16*l of that block, so no
//     registers stage the tile and no LDS store instructions are issued.
//   * Each lane chooses which 16-byte chunk of its row it fetches, so rows
//     are stored with their chunks XOR-swizzled: K chunk c of row r sits at
//     slot c ^ (r % 16), V chunk c at slot c ^ 4*(r % 4).  Both tile reads
//     below then touch every LDS bank equally (no bank conflicts).
//   * S^T = K Q^T (v_mfma_f32_32x32x16): A = 16-byte K fragments (one
//     ds_read_b128 each), B = the query tile held in registers.
//   * O^T = V^T P^T: the V^T fragment (8 keys of one head dim per lane) comes
//     from two ds_read_b64_tr_b16 transposing loads of the row-major V tile:
//     in each group of 16 lanes, lane i receives element i%4 of the 8-byte
//     pieces addressed by lanes 4k + i/4, k = 0..3; lanes address a 4-key x
//     16-dim block so that lane i gets 4 consecutive keys of dim i.  The key
//     order matches the P registers taken straight from the score
//     accumulator (register r of lane l holds key 8(r/4) + 4(l/32) + r%4).
//   * Tiles are double-buffered in two separate LDS arrays, and the tile loop
//     is unrolled by two so that each step's buffers are known statically:
//     the DMA of tile j+1 is issued before the matrix work of tile j, and
//     the compiler can see that the reads of tile j do not touch the buffer
//     the DMA is filling, so it waits for the DMA only at the one barrier
//     per tile.
#include "kcommon.h"
#include "launch.h"

namespace rattn {

namespace {

constexpr int D = 128;
constexpr int kThreads = 256;  // 4 wavefronts x 32 query rows
constexpr int kRowBytes = D * 2;

// Keys per tile: 64 (two resident workgroups per CU) or 32 (three).
#ifndef RATTN_D128_BC
#define RATTN_D128_BC 64
#endif
constexpr int BC = RATTN_D128_BC;
static_assert(BC == 32 || BC == 64, "tile width");
// A K+V buffer holds 2*BC rows of 256 bytes; each wave moves BC/16 1-KB DMA
// blocks per tensor.
constexpr int kTileBytes = BC * kRowBytes;
constexpr int kBufBytes = 2 * kTileBytes;
constexpr int NKB = BC / 32;   // 32-key score blocks
constexpr int NU = BC / 16;    // 16-key PV steps
constexpr int NDMA = BC / 16;  // DMA blocks per wave per tensor
constexpr int kWavesPerEu = BC == 64 ? 2 : 3;

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ lds_void* lds_at(char* base, int byte_off) {
  return (lds_void*)(base + byte_off);
}

template <typename TT>
__device__ __forceinline__ typename TT::v8 read_k_frag(const char* lds, uint32_t off) {
  return *(const typename TT::v8*)(lds + off);
}

// 4 consecutive keys of one head dim via the transposing LDS read.
__device__ __forceinline__ v4s read_tr(const char* lds, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(
          (__attribute__((address_space(3))) char*)(lds_void*)(lds + off)));
}

static_assert(kThreads / 64 * 32 == kMfma128Br, "schedule built for this tile height");

template <typename TT, bool OUT_F32>
__global__ __launch_bounds__(kThreads, kWavesPerEu) void fwd_mfma128_kernel(
    const typename TT::elem* __restrict__ q, const typename TT::elem* __restrict__ k,
    const typename TT::elem* __restrict__ v, void* __restrict__ out, float* __restrict__ lse,
    FwdParams p, Sched s) {
  using E = typename TT::elem;
  using v8 = typename TT::v8;
  using v4 = typename TT::v4;
  constexpr int KS = D / 16;  // 8 k-steps of S
  constexpr int DB = D / 32;  // 4 row blocks of O^T
  constexpr int kBc = BC;

  __shared__ __attribute__((aligned(1024))) char smem0[kBufBytes];
  __shared__ __attribute__((aligned(1024))) char smem1[kBufBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int l16 = lane & 15;

  // ---- work item -------------------------------------------------------
  const int32_t BH = p.B * p.Hq;
  const int32_t bh = xcd_head_swizzle((int32_t)(blockIdx.x % BH), BH);
  const int32_t t_lin = blockIdx.x / BH;
  const int32_t b = bh / p.Hq, hq = bh % p.Hq, hkv = hq / p.group;
  const QTile qt = query_tile(s, t_lin);
  const int64_t qhi = qt.pos0 + qt.rows - 1;

  const int wq0 = 32 * wave;
  const bool wave_active = wq0 < qt.rows;
  const int64_t wave_qlo = qt.pos0 + wq0;
  const int64_t wave_qhi = qt.pos0 + (wq0 + 31 < qt.rows ? wq0 + 31 : qt.rows - 1);
  const int my_q = wq0 + l32;
  const bool q_valid = my_q < qt.rows;
  const int64_t q_pos = qt.pos0 + my_q;

  // ---- Q fragments (B operand), loaded once ------------------------------
  v8 qf[KS];
  {
    const E* qp = q + (((int64_t)b * p.Nq + qt.row0 + (q_valid ? my_q : 0)) * p.Hq + hq) * D +
                  8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *(const v8*)(qp + 16 * ks);
      if (!q_valid) qf[ks] = v8{};
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m_run = kNegInf;
  float l_run = 0.f;

  // ---- DMA addressing ----------------------------------------------------
  const int64_t kv_stride = (int64_t)p.Hkv * D;  // elements between rows
  const char* kbase = (const char*)(k + (int64_t)b * p.Nk * kv_stride + (int64_t)hkv * D);
  const char* vbase = (const char*)(v + (int64_t)b * p.Nk * kv_stride + (int64_t)hkv * D);
  const uint32_t row_bytes = (uint32_t)(kv_stride * sizeof(E));
  // Tile rows handled by this wave: DMA blocks n = NDMA*wave + i,
  // rows 4n + lane/16; lane l writes LDS slot l%16 of its row and fetches
  // the logical chunk that belongs there.  Per-lane byte offsets from the
  // tile's first row are fixed, so each DMA is one scalar tile base plus a
  // 32-bit lane offset.
  uint32_t kdma_off[NDMA], vdma_off[NDMA];
  int dma_row[NDMA];
#pragma unroll
  for (int i = 0; i < NDMA; ++i) {
    const int r = 4 * (NDMA * wave + i) + (lane >> 4);
    dma_row[i] = r;
    kdma_off[i] = (uint32_t)r * row_bytes + 16 * (l16 ^ (r & 15));
    vdma_off[i] = (uint32_t)r * row_bytes + 16 * (l16 ^ (4 * (r & 3)));
  }

  auto issue_tile = [&](const TileCursor& c, char* lk) {
    const int64_t krow0 = c.run.row0 + c.t * kBc;
    const int64_t rem = c.run.len - c.t * kBc;
    const char* kt = kbase + krow0 * (int64_t)row_bytes;
    const char* vt = vbase + krow0 * (int64_t)row_bytes;
    char* lv = lk + kTileBytes;
    if (rem >= kBc) {
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int n = NDMA * wave + i;
        __builtin_amdgcn_global_load_lds(kt + kdma_off[i], lds_at(lk, n * 1024), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vt + vdma_off[i], lds_at(lv, n * 1024), 16, 0, 0);
      }
    } else {
      // ragged last tile of a run: rows past its end repeat the last row
      // (finite values; their scores are masked, so p = 0 for them)
      const uint32_t back_unit = row_bytes;
      const int last = (int)rem - 1;
#pragma unroll
      for (int i = 0; i < NDMA; ++i) {
        const int n = NDMA * wave + i;
        const uint32_t back = dma_row[i] > last ? (uint32_t)(dma_row[i] - last) * back_unit : 0u;
        __builtin_amdgcn_global_load_lds(kt + (kdma_off[i] - back), lds_at(lk, n * 1024), 16,
                                         0, 0);
        __builtin_amdgcn_global_load_lds(vt + (vdma_off[i] - back), lds_at(lv, n * 1024), 16,
                                         0, 0);
      }
    }
  };

  // ---- fragment addressing: per-lane byte offsets inside one K+V buffer ----
  // K: row kb*32 + l32, logical chunk 2*ks + hl at slot chunk ^ (row % 16)
  uint32_t k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    k_off[ks] = (uint32_t)(l32 * kRowBytes + 16 * ((2 * ks + hl) ^ (l32 & 15)));
  // V (transposing read): lane i of 16-lane group g reads key row
  // 16u + 8h + 4*hl + i/4, dims 32*db + 16*(g%2) + 4*(i%4) .. +3
  uint32_t v_off[DB];
  {
    const int qrow = l16 >> 2;
    const int g2 = (lane >> 4) & 1;
    const int c_in = 2 * g2 + ((l16 & 3) >> 1);  // chunk within the 32-dim block
    const int half = (l16 & 1) * 8;              // byte within the 16-byte chunk
#pragma unroll
    for (int db = 0; db < DB; ++db)
      v_off[db] = (uint32_t)(kTileBytes + (4 * hl + qrow) * kRowBytes +
                             16 * ((4 * db + c_in) ^ (4 * qrow)) + half);
  }

  TileCursor cur = cursor_begin<kBc>(s, qt.rank, qhi);
  if (cur.v < cur.nv) issue_tile(cur, smem0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  auto step = [&](char* cur_buf, char* next_buf) {
    TileCursor nxt = cur;
    cursor_next<kBc>(nxt, s, qt.rank, qhi);
    const bool has_next = nxt.v < nxt.nv;
    if (has_next) issue_tile(nxt, next_buf);
    const int64_t kpos0 = cur.run.pos0 + cur.t * kBc;
    const int64_t rem = cur.run.len - cur.t * kBc;
    const int krows = rem < kBc ? (int)rem : kBc;
    const bool wave_sees = wave_active && (!s.causal || kpos0 <= wave_qhi);
    if (wave_sees) {
      const char* lb = cur_buf;
      // S^T = K Q^T.  All K fragments of the tile are requested before the
      // first MFMA so the LDS latency is paid once per tile, and the 32-key
      // accumulator chains alternate.
      v8 kf[NKB][KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          kf[kb][ks] = read_k_frag<TT>(lb, k_off[ks] + kb * 32 * kRowBytes);
      f32x16 sacc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          sacc[kb] = TT::mfma32x32x16(kf[kb][ks], qf[ks], sacc[kb]);
      const bool need_mask = krows < kBc || (s.causal && kpos0 + krows - 1 > wave_qlo);
      if (need_mask) {
        const int lim = visible_limit(krows, s.causal, q_pos - kpos0);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            sacc[kb][r] = kk < lim ? sacc[kb][r] : kNegInf;
          }
      }
      // online softmax with lazy rescaling (see fwd_mfma.hip)
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
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
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      }
      const float m_use = m_run == kNegInf ? 0.f : m_run;
      float rs = 0.f;
      v8 pf[NU];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = exp2_fast(fmaf(sacc[kb][r], p.c, -m_use));
          rs += pr;
          pf[2 * kb + (r >> 3)][r & 7] = to_elem<TT>(pr);
        }
      l_run += rs;
      // O^T += V^T P^T: MFMA u covers keys 16u .. 16u+15
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint32_t o = v_off[db] + 16 * u * kRowBytes;
          const v4s lo = read_tr(lb, o);
          const v4s hi = read_tr(lb, o + 8 * kRowBytes);
          const v8 a = __builtin_shufflevector(__builtin_bit_cast(v4, lo),
                                               __builtin_bit_cast(v4, hi), 0, 1, 2, 3, 4, 5,
                                               6, 7);
          oacc[db] = TT::mfma32x32x16(a, pf[u], oacc[db]);
        }
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    cur = nxt;
  };
  while (cur.v < cur.nv) {
    step(smem0, smem1);
    if (!(cur.v < cur.nv)) break;
    step(smem1, smem0);
  }
  // ---- epilogue: O / l, LSE = m ln2 + ln l --------------------------------
  const float l_tot = pair_sum(l_run);
  if (!q_valid) return;
  const bool seen = l_tot > 0.f;
  const float inv = seen ? 1.f / l_tot : 0.f;
  const int64_t orow = ((int64_t)b * p.Nq + qt.row0 + my_q) * p.Hq + hq;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * hl;
      if (OUT_F32) {
        f32x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = oacc[db][4 * j + e] * inv;
        *(f32x4*)((float*)out + orow * D + d0) = o4;
      } else {
        v4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = to_elem<TT>(oacc[db][4 * j + e] * inv);
        *(v4*)((E*)out + orow * D + d0) = o4;
      }
    }
  if (hl == 0) lse[orow] = seen ? m_run * kLn2 + logf(l_tot) : kNegInf;
}

template <typename TT>
hipError_t launch_t(const void* q, const void* k, const void* v, void* out, float* lse,
                    bool out_f32, const FwdParams& p, const Sched& s, hipStream_t stream) {
  using E = typename TT::elem;
  const int64_t blocks = (int64_t)s.n_tiles * p.B * p.Hq;
  if (blocks <= 0) return hipSuccess;
  if (out_f32)
    hipLaunchKernelGGL((fwd_mfma128_kernel<TT, true>), dim3((unsigned)blocks),
                       dim3(kThreads), 0, stream, (const E*)q, (const E*)k, (const E*)v, out, lse,
                       p, s);
  else
    hipLaunchKernelGGL((fwd_mfma128_kernel<TT, false>), dim3((unsigned)blocks),
                       dim3(kThreads), 0, stream, (const E*)q, (const E*)k, (const E*)v, out, lse,
                       p, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma128(int dtype, const void* q, const void* k, const void* v, void* out,
                              float* lse, bool out_f32, const FwdParams& p, const Sched& s,
                              hipStream_t stream) {
  switch (dtype) {
    case 1: return launch_t<F16>(q, k, v, out, lse, out_f32, p, s, stream);
    case 2: return launch_t<Bf16>(q, k, v, out, lse, out_f32, p, s, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rattn
