// fwd_mfma128.hip -- the d = 128 attention forward on gfx950 matrix cores,
// two wave groups in ping-pong.
//
// Method (unchanged): online softmax over key tiles with a running max m,
// running sum l and unnormalised O, P rounded to the input type before PV,
// O/l once at the end (guijiagi.com "ring-attention-explained", online
// softmax section; yz520gzy FlashAttention chapter, FlashAttention-2 and its
// Triton kernel).
//
// Schedule.  A workgroup of 8 wavefronts owns 256 query rows, 32 per wave;
// waves w and w+4 share a SIMD.  Waves 0-3 form group A, waves 4-7 group B.
// Per key tile k each group runs an MFMA phase M_k = {PV of tile k-1, QK of
// tile k} (32 MFMAs) and a VALU phase V_k = {mask, exp, sum, P; the row max
// only when the sum shows it can move} of tile k.  Group B runs one phase behind group A, so one group's softmax runs
// next to the other group's matrix work on every SIMD:
//      window   0  |  1  |   2    |   3    |  ...
//      A        M0 | V0  | M1  V1 | M2  V2 |
//      B        -- | M0  | V0  M1 | V1  M2 |
// A workgroup barrier ends every window (A's after its V phase, B's after
// its M phase), one per key tile; inside a window the groups run unsynchronised.
//
// Every M phase inside the tile loop runs the same 32-MFMA stream (a single
// code path keeps the accumulators in place); a tile a wave does not score
// gets P = 0.  Group A's first phase skips the PV half and each group's
// last phase the QK half, whose results would be unused.  The
// stream reads each MFMA's LDS operand a few MFMAs ahead.  Scalar
// bookkeeping sits in the V phase, next to the VALU work; each M phase
// opens by issuing this wave's share of the DMA of a later tile.
//
// Data path.  K and V tiles (64 keys x 128 dims) move global -> LDS by
// direct-to-LDS DMA into a ring of 4 buffers; tile k is requested two
// windows before group A's QK reads it.  Rows
// are stored with XOR-swizzled 16-byte chunks (K chunk c of row r at slot
// c ^ (r%16), V at c ^ 4(r%4)) so the fragment reads below are conflict-free.
// S^T = K Q^T with v_mfma_f32_32x32x16 (A = K fragment, B = Q held in
// registers); O^T = V^T P^T with the V^T fragment from two ds_read_b64_tr_b16
// transposing reads and P packed from the score registers in place (register
// r of lane l holds key 8(r/4) + 4(l/32) + r%4 of a 32-key block), so it is
// the B operand as it stands.
// The DMA is issued from inline assembly and waited for explicitly
// (s_waitcnt vmcnt) before the barrier that precedes its first reader, so
// the compiler adds no conservative waits between a DMA and unrelated LDS
// reads.  The LDS address is an M0 operand of the asm, so the compiler
// writes M0 itself and knows the asm reads it.
#include <stdlib.h>

#include <type_traits>

#include "kcommon.h"
#include "launch.h"
#include "lds_dma.h"

namespace rattn {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBr = 32 * kWaves;    // 256 query rows per workgroup
constexpr int BC = 64;              // keys per tile
constexpr int kNBuf = 4;
constexpr int NKB = BC / 32;
constexpr int NU = BC / 16;

// Geometry of one head dimension D (128, 64 or 32).  A K or V row is 2 D
// bytes, D / 8 chunks of 16 bytes; one direct-to-LDS request moves 1 KB,
// 1024 / 2D rows.  Chunk c of row r sits in LDS at chunk slot
//   K: c ^ (r mod 16) (D = 128),  c ^ ((r / 2) mod 8) (D = 64),  c ^ ((r / 4) mod 4) (D = 32),
//   V: c ^ 4 (r mod 4) (D = 128), c ^ 4 ((r / 2) mod 2) (D = 64), c (D = 32),
// so that a K fragment read (16 lanes per cycle: 16 rows, one chunk each)
// and a transposing V read (32 lanes: 4 rows x 8 half-chunks) each touch
// every LDS bank once.
template <int D_>
struct Geo {
  static constexpr int D = D_;
  static_assert(D == 128 || D == 64 || D == 32, "head dimensions of this kernel");
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;
  static constexpr int kTileBytes = BC * kRowBytes;       // 16 KB, 8 KB
  static constexpr int kBufBytes = 2 * kTileBytes;        // K + V
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int kRowsPerDma = 1024 / kRowBytes;    // 4, 8
  static constexpr int kDmaBlocks = kBufBytes / 1024;     // per tile: 32, 16, 8
  static constexpr int kDmaPerWave = kDmaBlocks / kWaves; // 4, 2, 1
  static constexpr int kBlocksPerTensor = kDmaPerWave / 2;
  __device__ static int kslot(int c, int r) {
    return D == 128 ? c ^ (r & 15) : (D == 64 ? c ^ ((r >> 1) & 7) : c ^ ((r >> 2) & 3));
  }
  __device__ static int vslot(int c, int r) {
    return D == 128 ? c ^ (4 * (r & 3)) : (D == 64 ? c ^ (4 * ((r >> 1) & 1)) : c);
  }
};

static_assert(kBr == kMfma128Br, "schedule built for this tile height");

// N = this wave's DMA requests of one tile, which may stay in flight
template <int N>
__device__ __forceinline__ void wait_dma_but_one_tile() {
  static_assert(N == 4 || N == 2 || N == 1, "requests per wave per tile");
  if constexpr (N == 4)
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if constexpr (N == 2)
    asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
}
__device__ __forceinline__ void slot_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <typename TT>
__device__ __forceinline__ typename TT::v8 read_k_frag(const char* lds, uint32_t off) {
  return *(const typename TT::v8*)(lds + off);
}

// Cursor over the live key tiles of one query tile in ring order, with what
// the tile loop needs of the current run computed once per run, so that the
// per-tile tests are 32-bit scalar compares: a run holds fewer than 2^31 rows
// (the host rejects larger tensors), so its tile counts fit in 32 bits.
struct RunCursor {
  int32_t v, nv;     // visit (run) index, number of visits
  int32_t t, nt;     // tile within the run, live tiles of the run
  int32_t n_full;    // tiles of the run that hold BC rows
  int32_t t_live;    // this wave: tiles t < t_live hold a key visible to one of its rows
  int32_t t_nomask;  // this wave: tiles t < t_nomask are full and visible to all its rows
  int64_t row0, pos0, len;
};

struct RunCursorCtx {
  const Sched* s;
  int32_t rank;
  int64_t qhi;                // last query position of the work item
  int64_t wave_qlo, wave_qhi; // this wave's first and last query positions
  bool wave_active;
};

__device__ __forceinline__ int32_t clamp_tiles(int64_t x, int32_t hi) {
  return x < 0 ? 0 : (x > hi ? hi : (int32_t)x);
}

__device__ __forceinline__ void run_load(RunCursor& c, const RunCursorCtx& x) {
  const Run r = visit(*x.s, x.rank, c.v);
  c.row0 = r.row0;
  c.pos0 = r.pos0;
  c.len = r.len;
  c.nt = (int32_t)live_tiles(r, x.qhi, x.s->causal, BC);
  c.n_full = clamp_tiles(r.len / BC, c.nt);
  if (!x.wave_active) {
    c.t_live = c.t_nomask = 0;
  } else if (x.s->causal) {
    // floor division by BC of possibly negative positions: arithmetic shift
    c.t_live = clamp_tiles(((x.wave_qhi - r.pos0) >> 6) + 1, c.nt);
    c.t_nomask = clamp_tiles(((x.wave_qlo - r.pos0 - (BC - 1)) >> 6) + 1, c.n_full);
  } else {
    c.t_live = c.nt;
    c.t_nomask = c.n_full;
  }
  c.t = 0;
}

__device__ __forceinline__ void run_settle(RunCursor& c, const RunCursorCtx& x) {
  while (c.t >= c.nt) {
    ++c.v;
    if (c.v >= c.nv) return;
    run_load(c, x);
  }
}

// Cursor on live tile number t0 of the work item (0-based), or past the end.
__device__ __forceinline__ RunCursor run_cursor_at(const RunCursorCtx& x, int64_t t0) {
  RunCursor c;
  c.nv = num_visits(*x.s);
  c.v = 0;
  c.t = 0;
  c.nt = 0;
  c.row0 = c.pos0 = c.len = 0;
  c.n_full = c.t_live = c.t_nomask = 0;
  if (c.nv > 0) {
    run_load(c, x);
    run_settle(c, x);
  }
  while (c.v < c.nv && t0 >= c.nt - c.t) {
    t0 -= c.nt - c.t;
    c.t = c.nt;
    run_settle(c, x);
  }
  if (c.v < c.nv) c.t += (int32_t)t0;
  return c;
}

__device__ __forceinline__ void run_next(RunCursor& c, const RunCursorCtx& x) {
  ++c.t;
  if (c.t >= c.nt) run_settle(c, x);
}

// One work item (a query tile of a (batch, head), or one key split of it):
// work item `item` of the enumeration work_item_of describes.
// SERIAL: the debug form of the schedule (RATTN_SERIALIZE=1): one tile in
// flight, requested and waited for by every wave right before the phase that
// reads it, both wave groups in lockstep with a workgroup barrier around every
// phase.  Every wave performs the same arithmetic in the same order as in the
// pipelined schedule, so the two must agree bit for bit; a difference points
// at an LDS buffering hazard of the pipelined one.
template <typename TT, int D, bool OUT_F32, bool BUF, bool QUEUED, bool SERIAL = false>
__device__ __forceinline__ void fwd_item(const typename TT::elem* __restrict__ q,
                                         const typename TT::elem* __restrict__ k,
                                         const typename TT::elem* __restrict__ v,
                                         void* __restrict__ out, float* __restrict__ lse,
                                         const FwdParams& p, const Sched& s, uint32_t item) {
  using E = typename TT::elem;
  using v8 = typename TT::v8;
  using v4 = typename TT::v4;
  using E2 = typename TT::v2;
  using G = Geo<D>;
  constexpr int kRowBytes = G::kRowBytes;
  constexpr int kTileBytes = G::kTileBytes;
  constexpr int kBufBytes = G::kBufBytes;
  constexpr int KS = G::KS;
  constexpr int DB = G::DB;
  constexpr int kDmaPerWave = G::kDmaPerWave;
  // this wave's K (and V) blocks of a tile; D = 32: one block, wave w moves
  // block w mod 4 of K (w < 4) or of V
  constexpr bool kOnePart = kDmaPerWave == 1;
  constexpr int NBW = kOnePart ? 1 : G::kBlocksPerTensor;

  __shared__ __attribute__((aligned(1024))) char smem[kNBuf * kBufBytes];
  const uint32_t smem_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;  // 0: A, 1: B (one phase behind)
  const int hl = lane >> 5;
  const int l32 = lane & 31;
  const int l16 = lane & 15;

  // ---- work item -------------------------------------------------------
  const int32_t BH = p.B * p.Hq;
  const WorkItem wi = work_item_of(item, BH, p.n_splits);
  const int32_t bh = xcd_head_swizzle(wi.bh, BH);
  const int32_t t_lin = wi.t_lin;
  const int32_t b = bh / p.Hq, hq = bh % p.Hq, hkv = hq / p.group;
  const QTile qt = query_tile(s, t_lin, kBr);
  if (qt.rows <= 0) return;  // varlen: a tile past the end of its sequence
  const int64_t qhi = qt.pos0 + qt.rows - 1;

  const int wq0 = 32 * wave;
  const bool wave_active = wq0 < qt.rows;
  const int64_t wave_qlo = qt.pos0 + wq0;
  const int64_t wave_qhi = qt.pos0 + (wq0 + 31 < qt.rows ? wq0 + 31 : qt.rows - 1);
  const int my_q = wq0 + l32;
  const bool q_valid = my_q < qt.rows;
  const int64_t q_pos = qt.pos0 + my_q;

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

  // ---- DMA: wave w moves K blocks 2w, 2w+1 and V blocks 2w, 2w+1 ---------
  const int64_t kv_stride = (int64_t)p.Hkv * D;
  const char* kbase = (const char*)(k + (int64_t)b * p.Nk * kv_stride + (int64_t)hkv * D);
  const char* vbase = (const char*)(v + (int64_t)b * p.Nk * kv_stride + (int64_t)hkv * D);
  const uint32_t row_bytes = (uint32_t)(kv_stride * sizeof(E));
  // Block b of a tile's K (V) half is rows kRowsPerDma b .. +kRowsPerDma-1;
  // lane l lands in LDS slot l mod kChunks of row kRowsPerDma b + l / kChunks
  // and therefore reads the source chunk stored at that slot (the swizzles
  // are their own inverses).
  uint32_t kdma_off[NBW], vdma_off[NBW];
  int dma_row[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int slot = lane % G::kChunks;
    const int blk = kOnePart ? (wave & 3) : NBW * wave + i;
    const int r = G::kRowsPerDma * blk + lane / G::kChunks;
    dma_row[i] = r;
    kdma_off[i] = (uint32_t)r * row_bytes + 16 * G::kslot(slot, r);
    vdma_off[i] = (uint32_t)r * row_bytes + 16 * G::vslot(slot, r);
  }
  // This wave's four 16-byte-per-lane DMA parts of one tile: part 2i is K
  // block 2w+i, part 2i+1 is V block 2w+i.
  // BUF: the head's K and V rows as buffer resources, built once
  const v4i krs = BUF ? head_rsrc(kbase) : v4i{}, vrs = BUF ? head_rsrc(vbase) : v4i{};
  // One tile's request: its first row, whether it holds BC rows (else the
  // rows of the run from krow0 on) and its LDS buffer.  Lane offsets are the
  // precomputed kdma_off / vdma_off, except in the ragged last tile of a run,
  // whose rows past the end repeat the last row (finite values; their scores
  // are masked, so p = 0 for them).
  struct DmaPlan {
    int64_t krow0;
    int rem;       // rows from krow0 on, at most BC
    bool full;
    uint32_t lds;  // LDS address of the K half of the buffer
    bool on;
  };
  auto plan_tile = [&](const RunCursor& c, int buf) {
    DmaPlan dp;
    dp.krow0 = c.row0 + (int64_t)c.t * BC;
    dp.full = c.t < c.n_full;
    dp.rem = dp.full ? BC : (int)(c.len - (int64_t)c.t * BC);
    dp.lds = smem_addr + buf * kBufBytes;
    dp.on = true;
    return dp;
  };

  // ---- fragment addressing inside one K+V buffer --------------------------
  uint32_t k_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    k_off[ks] = (uint32_t)(l32 * kRowBytes + 16 * G::kslot(2 * ks + hl, l32));
  uint32_t v_off[DB];
  {
    const int qrow = l16 >> 2;
    const int g2 = (lane >> 4) & 1;
    const int c_in = 2 * g2 + ((l16 & 3) >> 1);
    const int half = (l16 & 1) * 8;
#pragma unroll
    for (int db = 0; db < DB; ++db)
      v_off[db] = (uint32_t)(kTileBytes + (4 * hl + qrow) * kRowBytes +
                             16 * G::vslot(4 * db + c_in, 4 * hl + qrow) + half);
  }

  // ---- tile bookkeeping ----------------------------------------------------
  int T;  // key tiles of this work item (of its split)
  const RunCursorCtx cx{&s, qt.rank, qhi, wave_qlo, wave_qhi, wave_active};
  RunCursor cdma;
  {
    // split s of n takes tiles [T s / n, T (s+1) / n) of the T live tiles
    const int64_t all = count_live_tiles<BC>(s, qt.rank, qhi);
    int64_t b0 = 0, b1 = all;
    if (p.n_splits > 1) {  // the 64-bit divisions run in software: only when split
      b0 = all * wi.split / p.n_splits;
      b1 = all * (wi.split + 1) / p.n_splits;
    }
    T = (int)(b1 - b0);
    cdma = run_cursor_at(cx, b0);
  }
  RunCursor cqk = cdma;  // next tile this group scores; cdma: next tile to request
  int n_req = 0;
  // plan the next tile's DMA (none once all T tiles are requested)
  auto plan_next = [&]() {
    DmaPlan dp;
    dp.on = false;
    if (n_req < T) {
      dp = plan_tile(cdma, n_req & (kNBuf - 1));
      run_next(cdma, cx);
      ++n_req;
    }
    return dp;
  };
  auto issue_all = [&](const DmaPlan& dp) {
    if (!dp.on) return;
    if constexpr (kOnePart) {
      const bool is_v = wave >= 4;
      const uint32_t dst = dp.lds + (is_v ? kTileBytes : 0) + (wave & 3) * 1024;
      const uint32_t off = is_v ? vdma_off[0] : kdma_off[0];
      const int last = dp.full ? BC - 1 : dp.rem - 1;
      const uint32_t back = dma_row[0] > last ? (uint32_t)(dma_row[0] - last) * row_bytes : 0u;
      const int64_t tb = dp.krow0 * (int64_t)row_bytes;
      if (BUF)
        dma16(is_v ? vrs : krs, (uint32_t)tb, off - back, dst);
      else
        dma16((is_v ? vbase : kbase) + tb + (off - back), dst);
      return;
    }
    if (BUF && dp.full) {
      // full tile: its byte offset in the scalar soffset, lane offsets as
      // precomputed (no per-tile vector work)
      const uint32_t t_off = (uint32_t)(dp.krow0 * (int64_t)row_bytes);
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        dma16(krs, t_off, kdma_off[i], dp.lds + (NBW * wave + i) * 1024);
        dma16(vrs, t_off, vdma_off[i], dp.lds + kTileBytes + (NBW * wave + i) * 1024);
      }
      return;
    }
    const int last = dp.rem - 1;
    const int64_t tb = dp.krow0 * (int64_t)row_bytes;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const uint32_t back = dma_row[i] > last ? (uint32_t)(dma_row[i] - last) * row_bytes : 0u;
      const uint32_t lk = dp.lds + (NBW * wave + i) * 1024;
      if (BUF) {
        dma16(krs, (uint32_t)tb, kdma_off[i] - back, lk);
        dma16(vrs, (uint32_t)tb, vdma_off[i] - back, lk + kTileBytes);
      } else {
        dma16(kbase + tb + (kdma_off[i] - back), lk);
        dma16(vbase + tb + (vdma_off[i] - back), lk + kTileBytes);
      }
    }
  };
  // Group B's first M phase runs the full MFMA stream (it sits in the tile
  // loop), so its PV reads the V half of buffer kNBuf-1 with P = 0: zero it
  // so that 0 * V stays 0 (no DMA targets that buffer before both groups'
  // first M phase).
  {
    uint4* z = (uint4*)(smem + (kNBuf - 1) * kBufBytes + kTileBytes);
    for (int i = tid; i < kTileBytes / 16; i += kThreads) z[i] = uint4{0, 0, 0, 0};
  }
  if constexpr (!SERIAL) {
    issue_all(plan_next());  // tile 0
    issue_all(plan_next());  // tile 1
    if (T > 1) wait_dma_but_one_tile<kDmaPerWave>(); else wait_dma_all();
  }
  __syncthreads();

  // per-group state carried between phases
  // sacc holds this wave's scores of the last scored tile; the V phase
  // writes their P in the input type, packed into pk (key pair (r, r+1) of
  // 32-key block kb -> dword 8 kb + r/2), which the next PV reads as its
  // B operand.  P = 0 when the wave did not score the tile.
  f32x16 sacc[NKB];
  f32x16 pk = f32x16{};
  static_assert(NKB == 2, "P of a 64-key tile fills exactly one accumulator");
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
  int64_t s_kpos0 = 0;   // positions of the scored tile (for the mask)
  int s_krows = 0;

  // One M phase as a flat stream of MFMAs, PV first (16: u-major, db-minor,
  // four independent accumulators), then QK (16: ks-major, kb-minor, two
  // accumulators).  Each MFMA's LDS operand is read kAhead MFMAs before it
  // is used, so the reads stream under the matrix work of the same wave.
  constexpr int kAhead = 3;  // measured: 3 beats 1, 2, 4, 6 and 8 by 0.6-1.5%
  auto mfma_stream = [&](auto pv_tag, auto qk_tag, const char* pvb, const char* qkb) {
    constexpr bool PV = decltype(pv_tag)::value;
    constexpr bool QK = decltype(qk_tag)::value;
    constexpr int NPV = PV ? NU * DB : 0;
    constexpr int N = NPV + (QK ? KS * NKB : 0);
    auto load = [&](int i) -> v8 {
      if (PV && i < NPV) {
        const uint32_t o = v_off[i % DB] + 16 * (i / DB) * kRowBytes;
        const v4s lo = read_tr(pvb, o);
        const v4s hi = read_tr(pvb, o + 8 * kRowBytes);
        return __builtin_shufflevector(__builtin_bit_cast(v4, lo), __builtin_bit_cast(v4, hi), 0,
                                       1, 2, 3, 4, 5, 6, 7);
      }
      const int j = i - NPV;
      return read_k_frag<TT>(qkb, k_off[j / NKB] + (j % NKB) * 32 * kRowBytes);
    };
    v8 fb[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i)
      if (i < N) fb[i] = load(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const v8 a = fb[i % kAhead];
      if (i + kAhead < N) fb[i % kAhead] = load(i + kAhead);
      if (PV && i < NPV) {
        const int u = i / DB;
        const f32x4 pw = {pk[4 * u], pk[4 * u + 1], pk[4 * u + 2], pk[4 * u + 3]};
        oacc[i % DB] = TT::mfma32x32x16(a, __builtin_bit_cast(v8, pw), oacc[i % DB]);
      } else {
        const int j = i - NPV;
        sacc[j % NKB] = TT::mfma32x32x16(a, qf[j / NKB], j < NKB ? f32x16{} : sacc[j % NKB]);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep this issue order
    }
  };

  // M phase kk: PV of tile kk-1 (P = 0 for a tile this wave did not score),
  // then QK of tile kk.
  // The DMA of tile kk+2 (if any) is issued first.  The wave runs this
  // phase at raised priority, so that on its SIMD the issue arbiter prefers
  // its MFMAs over the partner wave's softmax VALU (oldest-first would favour
  // group A in both phases).
  // pv, qk: which halves run (both, except in group A's first phase, whose
  // PV would multiply P = 0, and in each group's last, whose QK is unused).
  auto m_phase = [&](int kk, auto pv, auto qk) {
    const char* pvb = smem + ((kk - 1) & (kNBuf - 1)) * kBufBytes;
    const char* qkb = smem + (kk & (kNBuf - 1)) * kBufBytes;
    __builtin_amdgcn_s_setprio(1);
    issue_all(plan_next());
    mfma_stream(pv, qk, pvb, qkb);
    __builtin_amdgcn_s_setprio(0);
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;

  // V phase: mask, running max (lazy rescale), exp, row sum, P of the tile
  // scored in the last M phase.
  // The scalar bookkeeping (tile positions, cursor) runs here too, where it
  // issues between the VALU work instead of delaying the matrix stream.
  auto v_phase = [&]() {
    const int32_t t = cqk.t;
    const bool s_live = t < cqk.t_live;
    const bool need_mask = t >= cqk.t_nomask;
    s_kpos0 = cqk.pos0 + (int64_t)t * BC;
    s_krows = t < cqk.n_full ? BC : (int)(cqk.len - (int64_t)t * BC);
    run_next(cqk, cx);
    if (!s_live) {
      pk = f32x16{};  // P = 0
      return;
    }
    bool sees_key = true;  // this lane's query has a visible key in the tile
    if (need_mask) {
      // key index of register r of block kb is kb*32 + 8(r/4) + 4hl + r%4;
      // compare its lane-independent part against the limit shifted by 4hl
      const int vis = visible_limit(s_krows, s.causal, q_pos - s_kpos0);
      sees_key = vis > 0;
      const int lim = vis - 4 * hl;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk2 = kb * 32 + 8 * (r >> 2) + (r & 3);
          sacc[kb][r] = kk2 < lim ? sacc[kb][r] : kNegInf;
        }
    }
    // P = exp2(c s - m) into pk (input type, packed), its fp32 row sum into
    // four partial sums; the scores stay in sacc for the slow path below.
    float tsum;
    auto exps = [&](float m_use) {
      float rs[4];
      // D = 128, one workgroup per item: all shifted scores, then all
      // exponentials, then their uses, so that no use waits on a just-issued
      // exponential.  It takes 32 more registers, which the D = 64 and 32
      // budgets do not have, and which cost the queued kernel more (measured)
      // than the order gains.
      constexpr bool kSplitExp = D == 128 && !QUEUED;
      float x[NKB][16];
      if constexpr (kSplitExp) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) x[kb][r] = fmaf(sacc[kb][r], p.c, -m_use);
        __builtin_amdgcn_sched_barrier(0x4);  // only scalar work moves across
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) x[kb][r] = exp2_fast(x[kb][r]);
        __builtin_amdgcn_sched_barrier(0x4);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = kSplitExp ? x[kb][r] : exp2_fast(fmaf(sacc[kb][r], p.c, -m_use));
          const float p1 =
              kSplitExp ? x[kb][r + 1] : exp2_fast(fmaf(sacc[kb][r + 1], p.c, -m_use));
          const int i = (r >> 1) & 3;
          rs[i] = (kb == 0 && r < 8) ? p0 : rs[i] + p0;
          rs[i] += p1;
          const E2 pair = {to_elem<TT>(p0), to_elem<TT>(p1)};
          pk[8 * kb + r / 2] = __builtin_bit_cast(float, pair);
        }
      tsum = (rs[0] + rs[1]) + (rs[2] + rs[3]);
    };
    // Lazy rescaling: the running max m moves only when a score exceeds it
    // by more than kRescaleSlack (base-2 units), i.e. when some p would
    // exceed 2^kRescaleSlack.  Every p is >= 0, so a lane whose sum stays
    // within half that bound holds no such p, and the exact row max is
    // needed only when some lane's sum does not (or a row sees its first
    // key); the decisions, and so the results, are those of computing the
    // max for every tile.
    const bool no_max = m_run == kNegInf;
    exps(no_max ? 0.f : m_run);
    const bool slow = (tsum > 0.5f * kRescaleBound) | (no_max & sees_key);
    if (__builtin_amdgcn_ballot_w64(slow) != 0) {
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
        exps(m_run == kNegInf ? 0.f : m_run);
      }
    }
    l_run += tsum;
  };

  // Before the window in which the groups score tile j, tile j must have
  // landed on every wave; only tile j+1's requests may still be in flight.
  auto wait_tile = [&](int j) {
    if (j + 1 < T) wait_dma_but_one_tile<kDmaPerWave>(); else wait_dma_all();
  };

  // Windows.  Window 0 is group A's M0, window 1 A's V0 and B's M0; window
  // k >= 2 holds A's M_{k-1}, V_{k-1} and B's V_{k-2}, M_{k-1}.  Window k ends
  // with the barrier both groups pass after waiting for their part of tile k.
  // Each wave requests its share of tile m at the start of its M phase for
  // tile m-2, in window m-1 (group A's request of tile 2: window 0).  Buffer
  // m%4 last held tile m-4, whose last readers (the PV in both groups'
  // M_{m-3}, window m-2) finished at the barrier ending window m-2.  Tile m
  // is complete on every wave at the barrier ending window m, before any QK
  // of tile m (window m+1).  Both groups pass T+1 barriers.
  if constexpr (SERIAL) {
    // phase kk: tile kk lands, then {PV of tile kk-1, QK of tile kk}, then
    // the softmax of tile kk
    for (int kk = 0; kk <= T; ++kk) {
      if (kk < T) {
        issue_all(plan_next());
        wait_dma_all();
      }
      __syncthreads();
      const char* pvb = smem + ((kk - 1) & (kNBuf - 1)) * kBufBytes;
      const char* qkb = smem + (kk & (kNBuf - 1)) * kBufBytes;
      if (kk == 0) {
        if (T > 0) mfma_stream(no{}, yes{}, pvb, qkb);
      } else if (kk < T) {
        mfma_stream(yes{}, yes{}, pvb, qkb);
      } else {
        mfma_stream(yes{}, no{}, pvb, qkb);
      }
      __syncthreads();
      if (kk < T) v_phase();
      __syncthreads();
    }
  } else if (group == 0) {
    m_phase(0, no{}, yes{});
    slot_barrier();
    for (int j = 0; j + 1 < T; ++j) {
      v_phase();
      wait_tile(j + 1);
      slot_barrier();
      m_phase(j + 1, yes{}, yes{});  // requests tile j+3
    }
    if (T > 0) {
      v_phase();
      wait_tile(T);
      slot_barrier();
      m_phase(T, yes{}, no{});  // PV of the last tile
    }
  } else {
    slot_barrier();
    for (int j = 0; j < T; ++j) {
      m_phase(j, yes{}, yes{});  // requests tile j+2
      wait_tile(j + 1);
      slot_barrier();
      v_phase();
    }
    m_phase(T, yes{}, no{});  // PV of the last tile
  }
  // ---- epilogue: O / l, LSE = m ln2 + ln l --------------------------------
  const float l_tot = pair_sum(l_run);
  if constexpr (!OUT_F32 && !QUEUED) {
    // 16-bit output, one workgroup per item: the normalised rows go through
    // LDS, so that the global stores write whole rows, consecutive lanes
    // along a row, instead of 8 bytes in each of 32 rows per store
    // instruction.  A staged row is 2D bytes plus 16 of padding (16-byte
    // aligned; it spreads the rows of one fragment store over the banks).
    // The queued kernel keeps the direct stores: with staging its items
    // read twice the bytes from HBM (the run time unchanged).
    constexpr int kStageRow = 2 * D + 16;
    static_assert(kBr * kStageRow <= (kNBuf - 1) * kBufBytes + kTileBytes,
                  "staging stays clear of the zeroed V block");
    __syncthreads();  // both groups are done with the ring buffers
    if (q_valid) {
      const bool seen = l_tot > 0.f;
      const float inv = seen ? 1.f / l_tot : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = to_elem<TT>(oacc[db][4 * j + e] * inv);
          *(v4*)(smem + my_q * kStageRow + 2 * (32 * db + 8 * j + 4 * hl)) = o4;
        }
      if (hl == 0) {
        const int64_t orow = ((int64_t)b * p.out_rows + p.out_row_off + qt.row0 + my_q) * p.Hq + hq;
        lse[wi.split * p.split_lse_stride + orow] = seen ? fmaf(m_run, kLn2, logf(l_tot)) : kNegInf;
      }
    }
    __syncthreads();
    constexpr int kChunks = 2 * D / 16;  // 16-byte chunks per row
#pragma unroll 1
    for (int i = 0; i < kBr * kChunks / kThreads; ++i) {
      const int id = i * kThreads + tid;
      const int r = id / kChunks, c = id % kChunks;
      if (r < qt.rows) {
        const int64_t grow = ((int64_t)b * p.out_rows + p.out_row_off + qt.row0 + r) * p.Hq + hq;
        *(uint4*)((char*)out + grow * (2 * D) + 16 * c) = *(const uint4*)(smem + r * kStageRow + 16 * c);
      }
    }
    return;
  }
  // float32 output (ring steps, split-KV partials) and the queued kernel's
  // 16-bit output: each lane stores its own fragments
  if (!q_valid) return;
  const bool seen = l_tot > 0.f;
  const float inv = seen ? 1.f / l_tot : 0.f;
  // explicit fused forms, so that every instantiation (the serialized one
  // included) rounds the same way
  const float lse_n = seen ? fmaf(m_run, kLn2, logf(l_tot)) : kNegInf;
  const int64_t orow = ((int64_t)b * p.out_rows + p.out_row_off + qt.row0 + my_q) * p.Hq + hq;
  float* out_f = (float*)out + wi.split * p.split_out_stride;
  float* lse_w = lse + wi.split * p.split_lse_stride;
  const bool merging = OUT_F32 && p.merge_out;
  // The running result this step merges into: every load is issued before
  // the first use, so the row pays one memory latency, not one per chunk.
  f32x4 prev[OUT_F32 ? DB * 4 : 1];
  float lse_prev = kNegInf;
  if (merging) {
    lse_prev = lse_w[orow];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        prev[4 * db + j] = *(const f32x4*)(out_f + orow * D + 32 * db + 8 * j + 4 * hl);
  }
  const MergeW mw = merging ? merge_weights(lse_prev, lse_n) : MergeW{0.f, 1.f, lse_n};
  const float f_n = mw.f_n * inv;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * hl;
      if (OUT_F32) {
        f32x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = oacc[db][4 * j + e] * f_n;
        f32x4* dst = (f32x4*)(out_f + orow * D + d0);
        if (merging)
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = fmaf(prev[4 * db + j][e], mw.f_r, o4[e]);
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

// D = 64: 64 KB of LDS and at most 128 registers per wave, two workgroups per
// compute unit (four waves per SIMD); D = 128: one workgroup, two waves per SIMD.
template <typename TT, int D, bool OUT_F32, bool BUF>
__global__ __launch_bounds__(kThreads, D == 128 ? 2 : 4) void fwd_mfma128_kernel(
    const typename TT::elem* __restrict__ q, const typename TT::elem* __restrict__ k,
    const typename TT::elem* __restrict__ v, void* __restrict__ out, float* __restrict__ lse,
    FwdParams p, Sched s) {
  fwd_item<TT, D, OUT_F32, BUF, false>(q, k, v, out, lse, p, s, blockIdx.x);
}

// The serialized debug schedule of the same work items (RATTN_SERIALIZE=1).
template <typename TT, int D, bool OUT_F32, bool BUF>
__global__ __launch_bounds__(kThreads, D == 128 ? 2 : 4) void fwd_mfma128_serial_kernel(
    const typename TT::elem* __restrict__ q, const typename TT::elem* __restrict__ k,
    const typename TT::elem* __restrict__ v, void* __restrict__ out, float* __restrict__ lse,
    FwdParams p, Sched s) {
  fwd_item<TT, D, OUT_F32, BUF, false, true>(q, k, v, out, lse, p, s, blockIdx.x);
}

// The same work items taken from queues instead of one workgroup each: a grid
// of as many workgroups as the chip holds at once, where every workgroup
// repeatedly takes the next item of a queue.  Queue j (a counter in `queues`,
// zero at launch) hands out items j, j + 8, j + 16, ... in that order: the
// items a one-per-workgroup launch would run on XCD j (workgroups are dealt
// to the 8 XCDs round-robin), so each XCD keeps streaming the same heads'
// keys and values through its L2.  A workgroup serves its own XCD's queue
// and, once that is empty, takes the remaining items of the others: XCDs
// that run at a higher clock take on more of the work instead of idling at
// the end.  Every item is taken exactly once (each ticket of an atomic
// counter goes to one workgroup), so the results are those of the
// one-per-workgroup launch.
constexpr uint32_t kNoItem = 0xffffffffu;
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 7;
}
template <typename TT, int D, bool OUT_F32, bool BUF>
__global__ __launch_bounds__(kThreads, D == 128 ? 2 : 4) void fwd_mfma128_queue_kernel(
    const typename TT::elem* __restrict__ q, const typename TT::elem* __restrict__ k,
    const typename TT::elem* __restrict__ v, void* __restrict__ out, float* __restrict__ lse,
    FwdParams p, Sched s, uint32_t* __restrict__ queues, uint32_t n_items) {
  __shared__ uint32_t next;
  const uint32_t home = xcc_id();
  uint32_t skip = 0;  // queues this workgroup found empty (thread 0)
  for (;;) {
    if (threadIdx.x == 0) {
      uint32_t id = kNoItem;
      for (; skip < 8; ++skip) {
        const uint32_t j = (home + skip) & 7;
        const uint64_t cand = j + 8ull * atomicAdd(&queues[j], 1u);
        if (cand < n_items) {
          id = (uint32_t)cand;
          break;
        }
      }
      next = id;
    }
    __syncthreads();
    const uint32_t id = next;
    __syncthreads();  // every thread has read `next` before thread 0 writes it again
    if (id == kNoItem) return;
    fwd_item<TT, D, OUT_F32, BUF, true>(q, k, v, out, lse, p, s, id);
  }
}

__global__ void zero_queues_kernel(uint32_t* __restrict__ queues) {
  if (threadIdx.x < kFwdQueues) queues[threadIdx.x] = 0;
}

// Queue launch of kernel `kq` when the chip holds fewer than half of the
// `blocks` work items at once; returns false (nothing launched) otherwise.
template <typename KQ, typename E>
bool launch_queued(KQ kq, int64_t blocks, uint32_t* queues, hipStream_t stream, const E* q,
                   const E* k, const E* v, void* out, float* lse, const FwdParams& p,
                   const Sched& s, hipError_t* err) {
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kq, kThreads, 0);
  if (e != hipSuccess) {
    *err = e;
    return true;
  }
  if (cus <= 0 || per_cu <= 0) return false;
  const int64_t grid = (int64_t)cus * per_cu;
  if (blocks < 2 * grid) return false;
  hipLaunchKernelGGL(zero_queues_kernel, dim3(1), dim3(64), 0, stream, queues);
  hipLaunchKernelGGL(kq, dim3((unsigned)grid), dim3(kThreads), 0, stream, q, k, v, out, lse, p,
                     s, queues, (uint32_t)blocks);
  *err = hipGetLastError();
  return true;
}

template <typename TT, int D>
hipError_t launch_t(const void* q, const void* k, const void* v, void* out, float* lse,
                    bool out_f32, const FwdParams& p, const Sched& s, uint32_t* queues,
                    hipStream_t stream) {
  using E = typename TT::elem;
  const int64_t blocks = (int64_t)s.n_tiles * p.B * p.Hq * p.n_splits;
  if (blocks <= 0) return hipSuccess;
  // buffer-form DMA while one head's key/value rows span less than 4 GB
  // (32-bit lane offsets from the head's first row)
  const bool buf = (uint64_t)p.Nk * (uint64_t)p.Hkv * D * sizeof(E) <= 0xFFFF0000ull;
  const dim3 g((unsigned)blocks), t(kThreads);
  const E *qe = (const E*)q, *ke = (const E*)k, *ve = (const E*)v;
  // RATTN_SERIALIZE=1: the serialized debug schedule, one workgroup per item
  const char* ser = getenv("RATTN_SERIALIZE");
  if (ser && ser[0] == '1' && ser[1] == 0) {
    if (out_f32 && buf)
      hipLaunchKernelGGL((fwd_mfma128_serial_kernel<TT, D, true, true>), g, t, 0, stream, qe, ke, ve, out, lse, p, s);
    else if (out_f32)
      hipLaunchKernelGGL((fwd_mfma128_serial_kernel<TT, D, true, false>), g, t, 0, stream, qe, ke, ve, out, lse, p, s);
    else if (buf)
      hipLaunchKernelGGL((fwd_mfma128_serial_kernel<TT, D, false, true>), g, t, 0, stream, qe, ke, ve, out, lse, p, s);
    else
      hipLaunchKernelGGL((fwd_mfma128_serial_kernel<TT, D, false, false>), g, t, 0, stream, qe, ke, ve, out, lse, p, s);
    return hipGetLastError();
  }
  // queued launches at d = 128 only: at d = 64 and 32 the loop around the
  // item does not fit the register budget of two workgroups per compute unit
  if constexpr (D == 128) if (queues && blocks <= 0xFFFFFFF0ll) {
    hipError_t e = hipSuccess;
    bool done;
    if (out_f32 && buf)
      done = launch_queued(fwd_mfma128_queue_kernel<TT, D, true, true>, blocks, queues, stream,
                           qe, ke, ve, out, lse, p, s, &e);
    else if (out_f32)
      done = launch_queued(fwd_mfma128_queue_kernel<TT, D, true, false>, blocks, queues, stream,
                           qe, ke, ve, out, lse, p, s, &e);
    else if (buf)
      done = launch_queued(fwd_mfma128_queue_kernel<TT, D, false, true>, blocks, queues, stream,
                           qe, ke, ve, out, lse, p, s, &e);
    else
      done = launch_queued(fwd_mfma128_queue_kernel<TT, D, false, false>, blocks, queues, stream,
                           qe, ke, ve, out, lse, p, s, &e);
    if (done) return e;
  }
  if (out_f32 && buf)
    hipLaunchKernelGGL((fwd_mfma128_kernel<TT, D, true, true>), g, t, 0, stream, qe, ke, ve, out, lse, p, s);
  else if (out_f32)
    hipLaunchKernelGGL((fwd_mfma128_kernel<TT, D, true, false>), g, t, 0, stream, qe, ke, ve, out, lse, p, s);
  else if (buf)
    hipLaunchKernelGGL((fwd_mfma128_kernel<TT, D, false, true>), g, t, 0, stream, qe, ke, ve, out, lse, p, s);
  else
    hipLaunchKernelGGL((fwd_mfma128_kernel<TT, D, false, false>), g, t, 0, stream, qe, ke, ve, out, lse, p, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma128(int dtype, int d, const void* q, const void* k, const void* v,
                              void* out, float* lse, bool out_f32, const FwdParams& p,
                              const Sched& s, uint32_t* queues, hipStream_t stream) {
  if (d == 128) {
    if (dtype == 1) return launch_t<F16, 128>(q, k, v, out, lse, out_f32, p, s, queues, stream);
    if (dtype == 2) return launch_t<Bf16, 128>(q, k, v, out, lse, out_f32, p, s, queues, stream);
  } else if (d == 64) {
    if (dtype == 1) return launch_t<F16, 64>(q, k, v, out, lse, out_f32, p, s, queues, stream);
    if (dtype == 2) return launch_t<Bf16, 64>(q, k, v, out, lse, out_f32, p, s, queues, stream);
  } else if (d == 32) {
    if (dtype == 1) return launch_t<F16, 32>(q, k, v, out, lse, out_f32, p, s, queues, stream);
    if (dtype == 2) return launch_t<Bf16, 32>(q, k, v, out, lse, out_f32, p, s, queues, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace rattn
