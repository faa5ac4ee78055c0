// fwd_short.hip -- the attention forward (16-bit, d = 32, 64, 128) for
// launches with few query rows per head, where 256-row work items leave most
// compute units idle (a single head of 4096 queries is 16 such items on 256
// compute units).
//
// Method (unchanged): online softmax over key tiles with a running max m,
// running sum l and unnormalised O, P rounded to the input type before PV,
// O/l once at the end (guijiagi.com "ring-attention-explained", online
// softmax section; yz520gzy FlashAttention chapter, FlashAttention-2 and its
// Triton kernel).  The partial results of disjoint key ranges are combined
// with the log-sum-exp correction of the ring steps (Twinkle "Sequence
// parallel and Ring Attention", forward pass, update_out_and_lse).
//
// Work division.  A workgroup owns 32 query rows of one (batch, head) and
// divides their live key tiles (32 keys each, in ring order) into 8
// contiguous ranges, one per wavefront.  Every wave holds the 32 query rows
// in registers and runs the online softmax over its own range; at the end
// the 8 partial states (m, l, O) go through LDS and are merged row by row
// (weights 2^(m_w - max m)).  The merge needs no memory beyond the
// workgroup's LDS, so the launch allocates nothing.
//
// Per wave and key tile j: an MFMA phase {PV of tile j-1, QK of tile j}
// (d/16 + d/16 v_mfma_f32_32x32x16, interleaved so that dependent MFMAs are
// two apart) and a softmax phase of tile j.  S^T = K Q^T: the K fragments (A
// operand, key row = lane mod 32) come straight from global memory into
// registers, one tile ahead; Q is the B operand held in registers.
// O^T = V^T P^T: V tiles move global -> LDS by direct-to-LDS DMA into two
// buffers per wave (16-byte chunk c of row r at slot c ^ 4 (r mod 4)) and
// are read transposed with ds_read_b64_tr_b16; P is packed from the score
// registers in place (register r of lane l holds key 8(r/4) + 4(l/32) + r%4),
// so it is the B operand as it stands.
#include <type_traits>

#include "kcommon.h"
#include "launch.h"
#include "lds_dma.h"

namespace rattn {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = kShortBr;  // 32 query rows per workgroup
constexpr int BC = 32;         // keys per tile
constexpr int NU = BC / 16;    // 16-key MFMA steps of PV
static_assert(kBr == 32, "one MFMA column block of queries per wave");

// Geometry of head dimension D (128, 64 or 32).  A K or V row is 2 D bytes,
// D / 8 chunks of 16 bytes; one 1 KB DMA request moves 512 / D rows.
// Chunk c of row r sits in LDS at slot
//   K: c ^ (r mod 16) (D = 128),  c ^ ((r / 2) mod 8) (D = 64),  c ^ ((r / 4) mod 4) (D = 32),
//   V: c ^ 4 (r mod 4) (D = 128), c ^ 4 ((r / 2) mod 2) (D = 64), c (D = 32),
// so that a 16-lane K fragment read (16 rows, one chunk each) and a 32-lane
// transposing V read (4 rows x 8 half-chunks) each touch every LDS bank once
// (the layout of the 256-row kernel).
template <int D_>
struct SGeo {
  static constexpr int D = D_;
  static_assert(D == 128 || D == 64 || D == 32, "head dimensions of this kernel");
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;
  static constexpr int kTileBytes = BC * kRowBytes;   // one K or V tile: 8, 4, 2 KB
  static constexpr int KS = D / 16;                   // 16-dim MFMA steps of QK
  static constexpr int DB = D / 32;                   // 32-dim output blocks
  static constexpr int kReq = kTileBytes / 1024;      // 1 KB requests per tile
  static constexpr int kReqRows = 1024 / kRowBytes;   // rows per request
  // the K swizzle of the row a lane lands in repeats every kPeriod requests
  // (the V swizzle is the same for every request)
  static constexpr int kPeriod = D / 32;
  // merge area: per wave 32 rows of D floats, padded by 4 floats a row
  static constexpr int kMergeRow = D + 4;
  static constexpr int kKVBytes = kWaves * 2 * kTileBytes;  // one K and one V tile per wave
  static constexpr int kMergeBytes = kWaves * kBr * kMergeRow * 4 + 2 * kWaves * kBr * 4;
  static constexpr int kSmemBytes = kKVBytes > kMergeBytes ? kKVBytes : kMergeBytes;
  static_assert(kSmemBytes <= 160 * 1024, "LDS of one workgroup");
  static_assert(KS == NU * DB, "QK and PV steps alternate one for one");
  __device__ static int kslot(int c, int r) {
    return D == 128 ? c ^ (r & 15) : (D == 64 ? c ^ ((r >> 1) & 7) : c ^ ((r >> 2) & 3));
  }
  __device__ static int vslot(int c, int r) {
    return D == 128 ? c ^ (4 * (r & 3)) : (D == 64 ? c ^ (4 * ((r >> 1) & 1)) : c);
  }
};

// eight waves, two per SIMD: at most 256 registers per wave
template <typename TT, int D, bool OUT_F32, bool BUF>
__global__ __launch_bounds__(kThreads, 2) void fwd_short_kernel(
    const typename TT::elem* __restrict__ q, const typename TT::elem* __restrict__ k,
    const typename TT::elem* __restrict__ v, void* __restrict__ out, float* __restrict__ lse,
    FwdParams p, Sched s) {
  using E = typename TT::elem;
  using v8 = typename TT::v8;
  using v4 = typename TT::v4;
  using E2 = typename TT::v2;
  using G = SGeo<D>;
  constexpr int kRowBytes = G::kRowBytes;
  constexpr int kTileBytes = G::kTileBytes;
  constexpr int KS = G::KS;
  constexpr int DB = G::DB;

  __shared__ __attribute__((aligned(1024))) char smem[G::kSmemBytes];
  const uint32_t smem_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int l16 = lane & 15;

  // ---- work item: 32 query rows of one (batch, head) -----------------------
  const int32_t BH = p.B * p.Hq;
  const WorkItem wi = work_item_of(blockIdx.x, BH, p.n_splits);
  const int32_t bh = xcd_head_swizzle(wi.bh, BH);
  const int32_t b = bh / p.Hq, hq = bh % p.Hq, hkv = hq / p.group;
  const QTile qt = query_tile(s, wi.t_lin, kBr);
  if (qt.rows <= 0) return;  // a tile past the end of its segment (whole workgroup)
  const int64_t qhi = qt.pos0 + qt.rows - 1;
  const bool q_valid = l32 < qt.rows;
  const int64_t q_pos = qt.pos0 + l32;

  v8 qf[KS];
  {
    const E* qp = q + (((int64_t)b * p.Nq + qt.row0 + (q_valid ? l32 : 0)) * p.Hq + hq) * D +
                  8 * hl;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *(const v8*)(qp + 16 * ks);
      if (!q_valid) qf[ks] = v8{};
    }
  }

  // ---- this wave's key tiles ------------------------------------------------
  // split s of n takes live tiles [A s / n, A (s+1) / n) of the A live tiles
  // (split-KV launches; n = 1 otherwise), and wave w of the workgroup takes
  // [b0 + T w / 8, b0 + T (w+1) / 8) of those T tiles
  const int64_t all = count_live_tiles<BC>(s, qt.rank, qhi);
  int64_t b0 = 0, b1 = all;
  if (p.n_splits > 1) {  // the 64-bit divisions run in software: only when split
    b0 = all * wi.split / p.n_splits;
    b1 = all * (wi.split + 1) / p.n_splits;
  }
  const int64_t T = b1 - b0;
  const int64_t t0 = b0 + ((T * wave) >> 3), t1 = b0 + ((T * (wave + 1)) >> 3);
  const int n = (int)(t1 - t0);
  TileCursor cur = cursor_at<BC>(s, qt.rank, qhi, t0);

  const int64_t kv_stride = (int64_t)p.Hkv * D;  // elements between key rows
  const char* kbase = (const char*)(k + (int64_t)b * p.Nk * kv_stride + (int64_t)hkv * D);
  const char* vbase = (const char*)(v + (int64_t)b * p.Nk * kv_stride + (int64_t)hkv * D);
  const uint32_t row_bytes = (uint32_t)(kv_stride * sizeof(E));
  const v4i krs = BUF ? head_rsrc(kbase) : v4i{}, vrs = BUF ? head_rsrc(vbase) : v4i{};

  // DMA: request j of a tile moves rows R j .. R j + R-1 (1 KB, R = 512 / D);
  // lane l lands in slot l mod (D/8) of row R j + l / (D/8) and so reads the
  // source chunk stored there (each swizzle is its own inverse).  The rows'
  // offsets go in the scalar offset; the lane parts repeat every kPeriod
  // requests (K) or not at all (V).
  const int dma_r = lane / G::kChunks;
  const int dma_c = lane % G::kChunks;
  uint32_t k_lane[G::kPeriod];
#pragma unroll
  for (int j = 0; j < G::kPeriod; ++j) {
    const int r = G::kReqRows * j + dma_r;
    k_lane[j] = (uint32_t)r * row_bytes + 16 * G::kslot(dma_c, r);
  }
  const uint32_t v_lane = (uint32_t)dma_r * row_bytes + 16 * G::vslot(dma_c, dma_r);
  const uint32_t kreg = smem_addr + (uint32_t)wave * 2 * kTileBytes;  // this wave's K buffer
  const uint32_t vreg = kreg + kTileBytes;                             // and its V buffer
  const char* kb_ptr = smem + (kreg - smem_addr);
  const char* vb_ptr = smem + (vreg - smem_addr);

  // fragment addressing: K rows (lane mod 32 = key) for the A operand of QK,
  // V^T by transposing reads (16-key step u adds 16 rows)
  uint32_t k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_off[ks] = (uint32_t)(l32 * kRowBytes + 16 * G::kslot(2 * ks + hl, l32));
  uint32_t v_off[DB];
  {
    const int qrow = l16 >> 2;
    const int g2 = (lane >> 4) & 1;
    const int c_in = 2 * g2 + ((l16 & 3) >> 1);
    const int half = (l16 & 1) * 8;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      v_off[db] = (uint32_t)((4 * hl + qrow) * kRowBytes + 16 * G::vslot(4 * db + c_in, 4 * hl + qrow) +
                             half);
  }

  // One tile of the cursor: first row, positions, rows present.
  struct TileRef {
    int64_t krow0, kpos0;
    int rows;
  };
  auto tile_of = [&](const TileCursor& c) {
    TileRef r;
    r.krow0 = c.run.row0 + c.t * BC;
    r.kpos0 = c.run.pos0 + c.t * BC;
    const int64_t rem = c.run.len - c.t * BC;
    r.rows = rem < BC ? (int)rem : BC;
    return r;
  };

  // One tile of K (is_v = false) or V into this wave's buffer.  Rows past a
  // ragged end repeat the last row (finite values; their scores are masked).
  // The last reader of the buffer (this wave's MFMA phase) has consumed its
  // LDS reads before the DMA overwrites them.
  auto dma_tile = [&](const TileRef& t, bool is_v) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const uint32_t dst = is_v ? vreg : kreg;
    const int64_t tb = t.krow0 * (int64_t)row_bytes;
#pragma unroll
    for (int j = 0; j < G::kReq; ++j) {
      // rows of request j before the lane's own: in the scalar offset
      const uint32_t rows_k = (uint32_t)(G::kReqRows * G::kPeriod * (j / G::kPeriod)) * row_bytes;
      const uint32_t rows_v = (uint32_t)(G::kReqRows * j) * row_bytes;
      const uint32_t lane_part = is_v ? v_lane : k_lane[j % G::kPeriod];
      const uint32_t rows_part = is_v ? rows_v : rows_k;
      if (BUF && t.rows == BC) {
        dma16(is_v ? vrs : krs, (uint32_t)tb + rows_part, lane_part, dst + 1024 * j);
        continue;
      }
      // ragged tile: rows past the end repeat the last one
      const int r = G::kReqRows * j + dma_r;
      const uint32_t back = r > t.rows - 1 ? (uint32_t)(r - (t.rows - 1)) * row_bytes : 0u;
      const uint32_t lane_off = rows_part + lane_part - back;
      if (BUF)
        dma16(is_v ? vrs : krs, (uint32_t)tb, lane_off, dst + 1024 * j);
      else
        dma16((is_v ? vbase : kbase) + tb + lane_off, dst + 1024 * j);
    }
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  f32x16 sacc = f32x16{};
  float pk[8];  // P of the last scored tile, packed: key pair (r, r+1) -> dword r/2
#pragma unroll
  for (int i = 0; i < 8; ++i) pk[i] = 0.f;
  float m_run = kNegInf;
  float l_run = 0.f;

  // MFMA phase: QK of the tile in the K buffer and PV of the tile in the V
  // buffer (P in pk).  All fragments are read into registers first, so the
  // buffers can take the next tiles' DMA (`refill`) while the 16 MFMAs run
  // (alternating QK and PV steps, dependent MFMAs two apart).
  auto m_phase = [&](auto pv_tag, auto qk_tag, auto refill) {
    constexpr bool PV = decltype(pv_tag)::value;
    constexpr bool QK = decltype(qk_tag)::value;
    v8 kfr[KS], vfr[NU * DB];
    if constexpr (QK) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kfr[ks] = *(const v8*)(kb_ptr + k_off[ks]);
    }
    if constexpr (PV) {
#pragma unroll
      for (int x = 0; x < NU * DB; ++x) {
        const uint32_t o = v_off[x % DB] + 16 * (x / DB) * kRowBytes;
        const v4s lo = read_tr(vb_ptr, o);
        const v4s hi = read_tr(vb_ptr, o + 8 * kRowBytes);
        vfr[x] = __builtin_shufflevector(__builtin_bit_cast(v4, lo), __builtin_bit_cast(v4, hi), 0,
                                         1, 2, 3, 4, 5, 6, 7);
      }
    }
    refill();  // waits for the reads above (lgkmcnt), then DMA into both buffers
#pragma unroll
    for (int i = 0; i < KS; ++i) {
      if constexpr (QK) sacc = TT::mfma32x32x16(kfr[i], qf[i], i == 0 ? f32x16{} : sacc);
      if constexpr (PV) {
        const int u = i / DB;
        const f32x4 pw = {pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]};
        oacc[i % DB] = TT::mfma32x32x16(vfr[i], __builtin_bit_cast(v8, pw), oacc[i % DB]);
      }
    }
  };

  // Softmax phase of the tile just scored: mask, lazy running max, P, sum.
  auto v_phase = [&](const TileRef& t) {
    const bool need_mask = t.rows < BC || (s.causal && t.kpos0 + BC - 1 > qt.pos0);
    bool sees_key = true;
    if (need_mask) {
      const int vis = visible_limit(t.rows, s.causal, q_pos - t.kpos0);
      sees_key = vis > 0;
      const int lim = vis - 4 * hl;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 8 * (r >> 2) + (r & 3);
        sacc[r] = kk < lim ? sacc[r] : kNegInf;
      }
    }
    float tsum;
    auto exps = [&](float m_use) {
      float rs[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = exp2_fast(fmaf(sacc[r], p.c, -m_use));
        const float p1 = exp2_fast(fmaf(sacc[r + 1], p.c, -m_use));
        const int i = (r >> 1) & 1;
        rs[i] = r < 4 ? p0 : rs[i] + p0;
        rs[i] += p1;
        const E2 pair = {to_elem<TT>(p0), to_elem<TT>(p1)};
        pk[r / 2] = __builtin_bit_cast(float, pair);
      }
      tsum = rs[0] + rs[1];
    };
    // Lazy rescaling (the rule of the 256-row kernel): m moves only when a
    // score exceeds it by more than kRescaleSlack base-2 units; a lane whose
    // p sum is at most 2^(slack-1) holds no such p, so the exact row max is
    // taken only when some lane's sum is larger or a row sees its first key.
    const bool no_max = m_run == kNegInf;
    exps(no_max ? 0.f : m_run);
    const bool slow = (tsum > 0.5f * kRescaleBound) | (no_max & sees_key);
    if (__builtin_amdgcn_ballot_w64(slow) != 0) {
      float mt = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[r]);
      mt = pair_max(mt);
      const float m_cand = mt * p.c;
      if (__builtin_amdgcn_ballot_w64(m_cand > m_run + kRescaleSlack) != 0) {
        const float m_new = fmaxf(m_run, m_cand);
        const float alpha = exp2_fast(m_run - (m_new == kNegInf ? 0.f : m_new));
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
        exps(m_run == kNegInf ? 0.f : m_run);
      }
    }
    l_run += tsum;
  };

  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;

  // One K and one V buffer per wave.  The MFMA phase {PV of tile j-1, QK
  // of tile j} reads both into registers and then requests tile j+1's K and
  // tile j's V into them; they land during that phase's MFMAs and the
  // softmax of tile j, and the next MFMA phase waits for them.
  if (n > 0) {
    TileRef t_j = tile_of(cur), t_j1 = t_j;
    dma_tile(t_j, false);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    m_phase(no{}, yes{}, [&] {
      if (n > 1) {
        cursor_next<BC>(cur, s, qt.rank, qhi);
        t_j1 = tile_of(cur);
        dma_tile(t_j1, false);
      }
      dma_tile(t_j, true);
    });
    for (int j = 0; j + 1 < n; ++j) {
      v_phase(t_j);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      m_phase(yes{}, yes{}, [&] {
        if (j + 2 < n) {
          cursor_next<BC>(cur, s, qt.rank, qhi);
          dma_tile(tile_of(cur), false);
        }
        dma_tile(t_j1, true);
      });
      t_j = t_j1;
      t_j1 = tile_of(cur);
    }
    v_phase(t_j);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    m_phase(yes{}, no{}, [] {});
  }

  // ---- merge of the 8 waves' partial results in LDS ------------------------
  const float l_tot = pair_sum(l_run);
  __syncthreads();  // every wave is done with its V buffers
  float* mo = (float*)smem;
  constexpr int kMergeRow = G::kMergeRow;
  float* mm = mo + kWaves * kBr * kMergeRow;
  float* ml = mm + kWaves * kBr;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * hl;
      f32x4 o4;
#pragma unroll
      for (int e = 0; e < 4; ++e) o4[e] = oacc[db][4 * j + e];
      *(f32x4*)(mo + (wave * kBr + l32) * kMergeRow + d0) = o4;
    }
  if (hl == 0) {
    mm[wave * kBr + l32] = m_run;
    ml[wave * kBr + l32] = l_tot;
  }
  __syncthreads();

  // thread t: row t / (D/8), dims 8 (t mod (D/8)) .. +7
  constexpr int TPR = D / 8;  // threads per row, all in one wave
  const int row = tid / TPR;
  const int c8 = (tid % TPR) * 8;
  if (row >= kBr || row >= qt.rows) return;
  float mx = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, mm[w * kBr + row]);
  float o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  float lsum = 0.f;
  if (mx != kNegInf) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = mm[w * kBr + row];
      const float a = mw == kNegInf ? 0.f : exp2_fast(mw - mx);
      lsum += a * ml[w * kBr + row];
      const f32x4 lo = *(const f32x4*)(mo + (w * kBr + row) * kMergeRow + c8);
      const f32x4 hi = *(const f32x4*)(mo + (w * kBr + row) * kMergeRow + c8 + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] += a * lo[e];
        o[4 + e] += a * hi[e];
      }
    }
  }
  const bool seen = lsum > 0.f;
  const float inv = seen ? 1.f / lsum : 0.f;
  const float lse_n = seen ? mx * kLn2 + logf(lsum) : kNegInf;
  const int64_t orow = ((int64_t)b * p.out_rows + p.out_row_off + qt.row0 + row) * p.Hq + hq;
  if constexpr (OUT_F32) {
    // split-KV: this split's plane of the partial results
    float* out_f = (float*)out + wi.split * p.split_out_stride;
    lse += wi.split * p.split_lse_stride;
    f32x4* dst = (f32x4*)(out_f + orow * D + c8);
    MergeW mw{0.f, 1.f, lse_n};
    f32x4 prev0 = f32x4{}, prev1 = f32x4{};
    if (p.merge_out) {
      prev0 = dst[0];
      prev1 = dst[1];
      mw = merge_weights(lse[orow], lse_n);
    }
    const float f_n = mw.f_n * inv;
    f32x4 r0, r1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r0[e] = o[e] * f_n;
      r1[e] = o[4 + e] * f_n;
    }
    if (p.merge_out) {
      r0 += prev0 * mw.f_r;
      r1 += prev1 * mw.f_r;
    }
    dst[0] = r0;
    dst[1] = r1;
    // the threads of a row are in one wave, which read the previous lse
    // (above, in program order) before this store replaces it
    if (tid % TPR == 0) lse[orow] = mw.lse;
  } else {
    v8 o8;
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] = to_elem<TT>(o[e] * inv);
    *(v8*)((E*)out + orow * D + c8) = o8;
    if (tid % TPR == 0) lse[orow] = lse_n;
  }
}

template <typename TT, int D>
hipError_t launch_t(const void* q, const void* k, const void* v, void* out, float* lse,
                    bool out_f32, const FwdParams& p, const Sched& s, hipStream_t stream) {
  using E = typename TT::elem;
  const int64_t blocks = (int64_t)s.n_tiles * p.B * p.Hq * p.n_splits;
  if (blocks <= 0) return hipSuccess;
  const bool buf = (uint64_t)p.Nk * (uint64_t)p.Hkv * D * sizeof(E) <= 0xFFFF0000ull;
  const dim3 g((unsigned)blocks), t(kThreads);
  const E *qe = (const E*)q, *ke = (const E*)k, *ve = (const E*)v;
  if (out_f32 && buf)
    hipLaunchKernelGGL((fwd_short_kernel<TT, D, true, true>), g, t, 0, stream, qe, ke, ve, out, lse, p, s);
  else if (out_f32)
    hipLaunchKernelGGL((fwd_short_kernel<TT, D, true, false>), g, t, 0, stream, qe, ke, ve, out, lse, p, s);
  else if (buf)
    hipLaunchKernelGGL((fwd_short_kernel<TT, D, false, true>), g, t, 0, stream, qe, ke, ve, out, lse, p, s);
  else
    hipLaunchKernelGGL((fwd_short_kernel<TT, D, false, false>), g, t, 0, stream, qe, ke, ve, out, lse, p, s);
  return hipGetLastError();
}

template <typename TT>
hipError_t launch_d(int d, const void* q, const void* k, const void* v, void* out, float* lse,
                    bool out_f32, const FwdParams& p, const Sched& s, hipStream_t stream) {
  if (d == 128) return launch_t<TT, 128>(q, k, v, out, lse, out_f32, p, s, stream);
  if (d == 64) return launch_t<TT, 64>(q, k, v, out, lse, out_f32, p, s, stream);
  if (d == 32) return launch_t<TT, 32>(q, k, v, out, lse, out_f32, p, s, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_fwd_short(int dtype, int d, const void* q, const void* k, const void* v,
                            void* out, float* lse, bool out_f32, const FwdParams& p,
                            const Sched& s, hipStream_t stream) {
  if (dtype == 1) return launch_d<F16>(d, q, k, v, out, lse, out_f32, p, s, stream);
  if (dtype == 2) return launch_d<Bf16>(d, q, k, v, out, lse, out_f32, p, s, stream);
  return hipErrorInvalidValue;
}

}  // namespace rattn
