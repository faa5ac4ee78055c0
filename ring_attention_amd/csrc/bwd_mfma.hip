// bwd_mfma.hip -- 16-bit attention backward at d = 128 on gfx950 matrix cores.
//
// What it computes: the recomputation backward of the youngju.dev "Ring
// Attention" analysis (ring_attention_backward).  From the forward's
// log-sum-exp and D = rowsum(dO * O):
//   P = exp2(S scale log2(e) - lse log2(e)),  dP = dO V^T,  dS = P (dP - D)
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K
// P and dS are rounded to the input type before they enter a matrix product
// (the forward does the same with P); dP - D is formed in float32.
//
// How, on CDNA4 (v_mfma_f32_32x32x16_{bf16,f16}, 8 wavefronts per workgroup):
//   * dK/dV kernel: a workgroup owns 128 keys; their K and V rows sit in LDS
//     and are the B operand of S = Q K^T and dP = dO V^T, whose 32x32
//     accumulators give each lane one key column and 16 query rows.  Tiles of
//     64 query rows (Q, dO, lse, D) stream through LDS; P and dS go straight
//     from the accumulator registers into the B operand of dV^T += dO^T P and
//     dK^T += Q^T dS, with the A operands dO^T and Q^T read by transposing
//     LDS reads (ds_read_b64_tr_b16).  The query rows of every head of the
//     key/value head's GQA group are streamed in turn, so dK and dV need no
//     reduction across workgroups.
//   * dQ kernel: a workgroup owns 256 query rows (Q, dO in registers) and
//     streams tiles of 64 keys (K, V): S^T = K Q^T and dP^T = V dO^T put one
//     query per lane, so lse and D are one register each; dQ^T += K^T dS^T
//     with K^T read transposed from the same LDS tile.  Its two wave groups
//     run in ping-pong, as in the forward (see the kernel).
//   * Tiles move global -> LDS by direct-to-LDS DMA (buffer_load ... lds):
//     double buffered in the dK/dV kernel, a ring of 4 buffers in the dQ
//     kernel.  One XOR swizzle serves both LDS read patterns of a tile:
//     16-byte chunk c of row r sits at chunk slot
//     c ^ (4 (r mod 4) + (r div 4) mod 4), so the 16 rows of a row-fragment
//     read and the 4 rows x 4 chunks of a transposing read land in distinct
//     banks.
//   * Causal: the dQ kernel visits the live prefix of key tiles (a tile none
//     of a wave's rows sees gets dS = 0); the dK/dV kernel starts each query
//     run at the first row that can see its keys and skips the matrix work
//     of a tile none of a wave's pairs sees.  Element masks only on diagonal
//     or ragged tiles.
#include <type_traits>

#include "bwd.h"

namespace rattn {

namespace {

constexpr int D = 128;
constexpr int KS = D / 16;                  // k-steps of a contraction over d
constexpr int DB = D / 32;                  // 32-row blocks of d
constexpr int kRowBytes = D * 2;
constexpr int kRows = 64;                   // rows of a streamed tile
constexpr int kTileBytes = kRows * kRowBytes;  // 16 KB
constexpr int kOwn = 128;                   // keys a dK/dV workgroup owns (32 per wave)
constexpr float kLog2e = 1.4426950408889634f;

typedef short v4s __attribute__((ext_vector_type(4)));

// Direct-to-LDS DMA (LDS address in M0).  Each asm block begins with 5 wait
// states: the compiler does not look inside inline asm for hazards, and on
// gfx950 a VMEM instruction that reads an SGPR (M0, the resource, the scalar
// offset) written by a VALU instruction must follow it by at least 5.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
__device__ __forceinline__ void dma4(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
// Buffer form of dma16: 16 bytes per lane from a raw buffer resource plus a
// 32-bit lane offset (buffer_load_dwordx4 ... lds); used while every input
// tensor is below 4 GB.
typedef int v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i tensor_rsrc(const void* base) {
  const uint64_t a = (uint64_t)base;
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffff));
  r[2] = -1;           // num_records 2^32 - 1
  r[3] = 0x00020000;   // 32-bit data format
  return r;
}
// soff: the wave-uniform part of the offset (scalar), voff: the lane part
__device__ __forceinline__ void dma16(v4i rsrc, uint32_t soff, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// chunk-slot swizzle of row r (see the file comment)
__device__ __forceinline__ int swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

__device__ __forceinline__ v4s read_tr(const char* lds, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(
          (__attribute__((address_space(3))) char*)(lds + off)));
}

// Per-lane byte offsets of the two LDS read patterns inside one tile.
//   row[ks]: 8 elements of row l%32, columns 16 ks + 8 (l/32) .. +7 (the A
//     operand X[32 rows, 16 cols]); add 32 b rows for row block b.
//   tr[db][s]: transposing read s of the A operand X^T[32 columns of d block
//     db, 16 rows]: lane l gets column 32 db + l%32 of rows 8 s + 4 (l/32)
//     .. +3, so the pair (s = 0, 1) covers rows {0..3, 8..11} + 4 (l/32), the
//     row order of the accumulator registers r = 0..7 (key 8 (r/4) +
//     4 (l/32) + r%4); add 16 u rows for row group u.
struct FragOff {
  uint32_t row[KS];
  uint32_t tr[DB][2];
};
__device__ __forceinline__ FragOff frag_offsets(int lane) {
  const int hl = lane >> 5, l32 = lane & 31, l16 = lane & 15;
  FragOff f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    f.row[ks] = (uint32_t)(l32 * kRowBytes + 16 * ((2 * ks + hl) ^ swz(l32)));
  const int qrow = l16 >> 2;
  const int c_in = 2 * ((lane >> 4) & 1) + ((l16 & 3) >> 1);
  const int half = (l16 & 1) * 8;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int r = 8 * s + 4 * hl + qrow;
      f.tr[db][s] = (uint32_t)(r * kRowBytes + 16 * ((4 * db + c_in) ^ swz(r)) + half);
    }
  return f;
}

template <typename TT>
__device__ __forceinline__ typename TT::v8 row_frag(const char* tile, const FragOff& f, int ks,
                                                    int row_block) {
  return *(const typename TT::v8*)(tile + f.row[ks] + row_block * 32 * kRowBytes);
}
template <typename TT>
__device__ __forceinline__ typename TT::v8 tr_frag(const char* tile, const FragOff& f, int db,
                                                   int row16) {
  typedef short v8s __attribute__((ext_vector_type(8)));
  const uint32_t o = (uint32_t)(row16 * 16 * kRowBytes);
  const v4s lo = read_tr(tile, f.tr[db][0] + o);
  const v4s hi = read_tr(tile, f.tr[db][1] + o);
  const v8s x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(typename TT::v8, x);
}

// Request one 64-row tile of a [.., d] tensor: rows row0 .. row0+rows-1 of
// the flattened row space (stride `stride` elements between rows); rows past
// `rows` repeat the last one (finite, masked by the caller).  This wave moves
// rows 16 w .. 16 w + 15, four 1 KB blocks.
// `tensor` + `col0` elements is the tile's first column (BUF: `rsrc` is the
// tensor as a buffer resource and the lane offsets are 32-bit).
template <bool BUF, typename E>
__device__ __forceinline__ void dma_tile(const E* tensor, v4i rsrc, int64_t col0, int64_t row0,
                                         int rows, int64_t stride, uint32_t lds_tile, int wave,
                                         int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * wave + 4 * i + (lane >> 4);
    const int rc = r < rows ? r : rows - 1;
    const uint32_t chunk = 16 * ((lane & 15) ^ swz(r));
    const uint32_t dst = lds_tile + (uint32_t)((16 * wave + 4 * i) * kRowBytes);
    if (BUF)
      dma16(rsrc, (uint32_t)((row0 * stride + col0) * (int64_t)sizeof(E)),
            (uint32_t)(rc * stride * (int64_t)sizeof(E)) + chunk, dst);
    else
      dma16((const char*)(tensor + (row0 + rc) * stride + col0) + chunk, dst);
  }
}

__device__ __forceinline__ float lse2_of(float lse) {
  // rows that saw no key (lse = -inf) get +inf: P = exp2(x - inf) = 0
  return lse == kNegInf ? __builtin_inff() : lse * kLog2e;
}

// Pack 16 float32 accumulator values (rows r = 0..15 of one 32-row block)
// into 8 dwords of input-type pairs, register pair (r, r+1) -> dword r/2.
template <typename TT>
__device__ __forceinline__ void pack_pair(float* dst, float a, float b) {
  using E2 = typename TT::v2;
  const E2 pr = {to_elem<TT>(a), to_elem<TT>(b)};
  *dst = __builtin_bit_cast(float, pr);
}
template <typename TT>
__device__ __forceinline__ typename TT::v8 packed_operand(const float* w, int u) {
  const f32x4 x = {w[4 * u], w[4 * u + 1], w[4 * u + 2], w[4 * u + 3]};
  return __builtin_bit_cast(typename TT::v8, x);
}

// Work order.  The dispatcher deals workgroups to the 8 XCDs round-robin
// (workgroup id % 8), and each XCD has its own L2.  Give every XCD whole
// (batch, head) pairs, their tiles consecutive in its sequence, so that the
// workgroups an XCD runs at the same time stream the same head's tiles
// (K/V, or Q/dO) through its L2.  heavy_last: a head's tiles are taken
// from the last one (causal dQ: later query tiles see more keys).
__device__ __forceinline__ void work_order(int32_t BH, int64_t n_tiles, bool heavy_last,
                                           int32_t* bh, int64_t* tl) {
  const uint32_t id = blockIdx.x;
  if ((BH & 7) == 0) {
    const uint32_t x = id & 7, j = id >> 3;
    const int64_t t = (int64_t)j % n_tiles;
    *bh = (int32_t)(x + 8 * (uint32_t)((int64_t)j / n_tiles));
    *tl = heavy_last ? n_tiles - 1 - t : t;
  } else {
    *bh = (int32_t)(id % (uint32_t)BH);
    const int64_t t = id / (uint32_t)BH;
    *tl = heavy_last ? n_tiles - 1 - t : t;
  }
}

// ---- dK, dV ------------------------------------------------------------------
// Eight wavefronts, 128 keys per workgroup.  K and V of the workgroup's keys
// sit in LDS (64 KB) and are read as the B operand of S = Q K^T and
// dP = dO V^T, so that a wave holds only its dK and dV accumulators and two
// waves fit per SIMD.  Wave w takes keys 32 (w % 4) .. +31 and query rows
// 32 (w / 4) .. +31 of every 64-row query tile; waves w and w + 4 add their
// dK and dV through LDS at the end.
constexpr int kThreadsKV = 512;

template <typename TT, bool ACC, bool BUF>
__global__ __launch_bounds__(kThreadsKV, 1) void bwd_dkv_mfma_kernel(
    const typename TT::elem* __restrict__ q, const typename TT::elem* __restrict__ k,
    const typename TT::elem* __restrict__ v, const typename TT::elem* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, void* __restrict__ dk,
    void* __restrict__ dv, BwdParams p) {
  using E = typename TT::elem;
  using v8 = typename TT::v8;
  constexpr int kKV = 2 * kOwn * kRowBytes;      // K, then V, of the owned keys: 64 KB
  constexpr int kStat = 2 * kTileBytes;          // in a query buffer: lse, then D, 64 floats each
  constexpr int kBufBytes = kStat + 2 * kRows * 4;
  constexpr int kSmem = kKV + 2 * kBufBytes;
  constexpr int kRed = 4 * 2 * DB * 16 * 64 * 4;  // dK, dV of waves 4..7
  static_assert(kRed <= kSmem, "the dK, dV hand-over fits in the tiles' LDS");
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];
  const uint32_t smem_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3;   // key group: keys 32 kg .. +31
  const int qh = wave >> 2;  // query half of every query tile
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  const int32_t BH = p.B * p.Hkv;
  int32_t bh;
  int64_t tl;
  work_order(BH, bwd_k_tiles(p, kOwn), false, &bh, &tl);
  const int32_t b = bh / p.Hkv, hkv = bh % p.Hkv;
  const BwdItem item = bwd_k_item(p, kOwn, tl);
  if (item.tile.rows <= 0) return;  // varlen: a tile past the end of its sequence
  const BwdTile kt = item.tile;
  // the (at most two) query runs as scalars: a runtime-indexed array would
  // live in scratch, and the compiler's wait for a scratch load would also
  // wait for the tile DMA issued before it
  const BwdRun qr0 = item.other[0], qr1 = item.other[1];
  const int wk0 = 32 * kg;
  const int wkrows = kt.rows - wk0 < 0 ? 0 : (kt.rows - wk0 > 32 ? 32 : (int)(kt.rows - wk0));
  const bool k_valid = l32 < wkrows;
  const int64_t wkpos = kt.pos0 + wk0;      // position of the wave's first key
  const int64_t kpos = wkpos + l32;         // this lane's key
  const int64_t krow0 = (int64_t)b * p.k_rows + p.k_off + kt.row0;  // first owned key row
  const int64_t krow = (krow0 + wk0 + (k_valid ? l32 : 0)) * p.Hkv + hkv;

  f32x16 dka[DB], dva[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dka[db] = dva[db] = f32x16{};

  // query tiles: every head of the group, each run from the first row that
  // can see one of this workgroup's keys
  auto run_start = [&](const BwdRun& r) {
    int64_t s0 = 0;
    if (p.causal) {
      s0 = kt.pos0 - r.pos0;
      s0 = s0 < 0 ? 0 : (s0 > r.len ? r.len : s0);
    }
    return s0;
  };
  const int64_t st0 = item.n_other > 0 ? run_start(qr0) : 0;
  const int64_t st1 = item.n_other > 1 ? run_start(qr1) : 0;
  const int64_t nt0 = item.n_other > 0 ? (qr0.len - st0 + kRows - 1) / kRows : 0;
  const int64_t nt1 = item.n_other > 1 ? (qr1.len - st1 + kRows - 1) / kRows : 0;
  const int64_t per_head = nt0 + nt1;
  const int64_t T = per_head * p.group;
  struct QT {
    int64_t row0;  // flattened row index in [B * q_rows]
    int64_t pos0;
    int32_t hq;
    int rows;
  };
  auto tile_of = [&](int64_t t) {
    QT x;
    // 32-bit: a workgroup walks far fewer than 2^31 tiles
    const int32_t g = (int32_t)((uint32_t)t / (uint32_t)per_head);
    int64_t r = t - (int64_t)g * per_head;
    const bool second = r >= nt0;
    if (second) r -= nt0;
    const int64_t i0 = (second ? st1 : st0) + r * kRows;
    const int64_t rem = (second ? qr1.len : qr0.len) - i0;
    x.rows = rem < kRows ? (int)rem : kRows;
    x.row0 = (int64_t)b * p.q_rows + p.q_off + (second ? qr1.row0 : qr0.row0) + i0;
    x.pos0 = (second ? qr1.pos0 : qr0.pos0) + i0;
    x.hq = hkv * p.group + (int32_t)g;
    return x;
  };
  const int64_t qstride = (int64_t)p.Hq * D;
  const v4i qrs = BUF ? tensor_rsrc(q) : v4i{}, grs = BUF ? tensor_rsrc(dout) : v4i{};
  // query tile t into buffer buf: waves 0-3 move Q, waves 4-7 dO (16 rows
  // each), wave 0 the lse and wave 4 the D values of its rows
  auto issue = [&](int64_t t, int buf) {
    const QT x = tile_of(t);
    const uint32_t base = smem_addr + kKV + buf * kBufBytes;
    if (qh == 0)
      dma_tile<BUF>(q, qrs, (int64_t)x.hq * D, x.row0, x.rows, qstride, base, kg, lane);
    else
      dma_tile<BUF>(dout, grs, (int64_t)x.hq * D, x.row0, x.rows, qstride, base + kTileBytes, kg,
                    lane);
    if (kg == 0) {
      const int rc = lane < x.rows ? lane : x.rows - 1;
      const float* src = (qh == 0 ? lse : delta) + (x.row0 + rc) * p.Hq + x.hq;
      dma4(src, base + kStat + qh * kRows * 4);
    }
  };

  const FragOff fo = frag_offsets(lane);
  const char* kb_l = smem;                      // K rows of the owned keys
  const char* vb_l = smem + kOwn * kRowBytes;   // V rows
  auto compute = [&](int64_t t, int buf) {
    const QT x = tile_of(t);
    const char* qb_l = smem + kKV + buf * kBufBytes;
    const char* gb_l = qb_l + kTileBytes;
    const float* lse_l = (const float*)(qb_l + kStat);
    const float* dl_l = lse_l + kRows;
    const int qb = qh;
    if (wkrows == 0 || 32 * qb >= x.rows) return;
    if (p.causal && x.pos0 + 32 * qb + 31 < wkpos) return;  // no row of the block sees a key
    const bool need_mask = x.rows < kRows || (p.causal && x.pos0 < wkpos + wkrows - 1);
    // S and dP over the 8 k-steps: the four operands of a step (Q, K, dO, V
    // fragments) are read two steps ahead, and the issue order is pinned, so
    // that the reads stay a bounded number of registers
    f32x16 s_acc = {}, dp_acc = {};
    v8 fq[2], fk[2], fg[2], fv[2];
    auto ld_s = [&](int ks, int slot) {
      fq[slot] = row_frag<TT>(qb_l, fo, ks, qb);
      fk[slot] = row_frag<TT>(kb_l, fo, ks, kg);
      fg[slot] = row_frag<TT>(gb_l, fo, ks, qb);
      fv[slot] = row_frag<TT>(vb_l, fo, ks, kg);
    };
    ld_s(0, 0);
    ld_s(1, 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int slot = ks & 1;
      s_acc = TT::mfma32x32x16(fq[slot], fk[slot], s_acc);
      dp_acc = TT::mfma32x32x16(fg[slot], fv[slot], dp_acc);
      if (ks + 2 < KS) ld_s(ks + 2, slot);
      __builtin_amdgcn_sched_barrier(0);
    }
    // query row of register r: 32 qb + 8 (r/4) + 4 hl + r%4
    f32x4 lv[4], dv4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lv[j] = *(const f32x4*)(lse_l + 32 * qb + 8 * j + 4 * hl);
      dv4[j] = *(const f32x4*)(dl_l + 32 * qb + 8 * j + 4 * hl);
    }
    // P and dS of the block, each step over all 16 registers at once so
    // that the independent chains overlap.  Register r of a lane holds
    // query row 32 qb + 8 (r/4) + 4 hl + r%4, visible iff the row exists
    // and (causal) the key is not after it: r2 = 8 (r/4) + r%4 in
    // [rel, rlim) with rel = kpos - (x.pos0 + 32 qb + 4 hl).
    float pr[16], ds[16];
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
      pr[rr] = fmaf(s_acc[rr], p.c, -lse2_of(lv[rr >> 2][rr & 3]));
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) pr[rr] = exp2_fast(pr[rr]);
    if (need_mask) {
      const int64_t rel64 = kpos - (x.pos0 + 32 * qb + 4 * hl);
      const int rel = p.causal ? (rel64 > 64 ? 64 : (rel64 < -64 ? -64 : (int)rel64)) : -64;
      const int rlim = x.rows - 32 * qb - 4 * hl;  // rows r2 < rlim exist
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int r2 = 8 * (rr >> 2) + (rr & 3);
        pr[rr] = ((r2 >= rel) & (r2 < rlim)) ? pr[rr] : 0.f;
      }
    }
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) ds[rr] = pr[rr] * (dp_acc[rr] - dv4[rr >> 2][rr & 3]);
    float pw[8], dw[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      pack_pair<TT>(&pw[r >> 1], pr[r], pr[r + 1]);
      pack_pair<TT>(&dw[r >> 1], ds[r], ds[r + 1]);
    }
    // dV^T += dO^T P and dK^T += Q^T dS over (u, db): the two transposed
    // operands of a step read two steps ahead, issue order pinned
    v8 tg[2], tq[2];
    auto ld_t = [&](int i, int slot) {
      tg[slot] = tr_frag<TT>(gb_l, fo, i % DB, 2 * qb + i / DB);
      tq[slot] = tr_frag<TT>(qb_l, fo, i % DB, 2 * qb + i / DB);
    };
    ld_t(0, 0);
    ld_t(1, 1);
#pragma unroll
    for (int i = 0; i < 2 * DB; ++i) {
      const int slot = i & 1, u = i / DB, db = i % DB;
      dva[db] = TT::mfma32x32x16(tg[slot], packed_operand<TT>(pw, u), dva[db]);
      dka[db] = TT::mfma32x32x16(tq[slot], packed_operand<TT>(dw, u), dka[db]);
      if (i + 2 < 2 * DB) ld_t(i + 2, slot);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (T > 0) {
    // the owned keys' K and V rows (rows past the last key repeat it: finite
    // values whose results are not stored), then query tile 0
    const int64_t kstride = (int64_t)p.Hkv * D;
    const v4i krs = BUF ? tensor_rsrc(k) : v4i{}, vrs = BUF ? tensor_rsrc(v) : v4i{};
    dma_tile<BUF>(k, krs, (int64_t)hkv * D, krow0, kt.rows, kstride, smem_addr, wave, lane);
    dma_tile<BUF>(v, vrs, (int64_t)hkv * D, krow0, kt.rows, kstride,
                  smem_addr + kOwn * kRowBytes, wave, lane);
    issue(0, 0);
    wait_dma();
    __syncthreads();
    for (int64_t t = 0; t < T; ++t) {
      if (t + 1 < T) issue(t + 1, (int)((t + 1) & 1));
      compute(t, (int)(t & 1));
      wait_dma();
      __syncthreads();
    }
  }

  // waves 4..7 hand their sums to waves 0..3 (every tile read is done: the
  // loop ends with a barrier; with no tile no DMA was issued)
  float* red = (float*)smem + (size_t)kg * (2 * DB * 16 * 64);
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[(db * 16 + r) * 64 + lane] = dka[db][r];
        red[((DB + db) * 16 + r) * 64 + lane] = dva[db][r];
      }
  }
  __syncthreads();
  if (qh == 1 || !k_valid) return;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dka[db][r] += red[(db * 16 + r) * 64 + lane];
      dva[db][r] += red[((DB + db) * 16 + r) * 64 + lane];
    }
  // lane: key l%32; register 4 j + e of block db: dim 32 db + 8 j + 4 hl + e
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * hl;
      f32x4 gk, gv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gk[e] = dka[db][4 * j + e] * p.scale;
        gv[e] = dva[db][4 * j + e];
      }
      if (ACC) {
        f32x4* ok = (f32x4*)((float*)dk + krow * D + d0);
        f32x4* ov = (f32x4*)((float*)dv + krow * D + d0);
        *ok = *ok + gk;
        *ov = *ov + gv;
      } else {
        typename TT::v4 ek, ev;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ek[e] = to_elem<TT>(gk[e]);
          ev[e] = to_elem<TT>(gv[e]);
        }
        *(typename TT::v4*)((E*)dk + krow * D + d0) = ek;
        *(typename TT::v4*)((E*)dv + krow * D + d0) = ev;
      }
    }
}

// ---- dQ, two wave groups in ping-pong -----------------------------------------
// Eight wavefronts own 256 query rows, 32 per wave (Q and dO rows in
// registers as the B operands of S^T = K Q^T and dP^T = V dO^T, one query
// per lane); waves w and w+4 share a SIMD.  Waves 0-3 form group A, waves
// 4-7 group B.  Per key tile k each group runs an MFMA phase
// M_k = {dQ^T += K^T dS^T of tile k-1, S^T and dP^T of tile k} (48 MFMAs)
// and a vector phase V_k = {P = exp2(S c - lse log2 e), mask, dS = P (dP - D),
// packed to the input type} of tile k.  Group B runs one phase behind group
// A, so on every SIMD one group's vector work runs next to the other
// group's matrix work:
//      window   0  |  1  |   2    |   3    |  ...
//      A        M0 | V0  | M1  V1 | M2  V2 |
//      B        -- | M0  | V0  M1 | V1  M2 |
// with one workgroup barrier per window.  Key tiles (K and V, 64 rows each)
// move global -> LDS by direct-to-LDS DMA into a ring of 4 buffers; each
// wave requests its share of tile m at the start of its M phase for tile
// m-2.  A tile a wave does not see gets dS = 0 (its S and dP are computed
// and dropped), so that every M phase runs the same MFMA stream.
constexpr int kPPWaves = 8;
constexpr int kThreadsPP = 64 * kPPWaves;
constexpr int kOwnPP = 32 * kPPWaves;  // query rows per workgroup
constexpr int kNBuf = 4;

__device__ __forceinline__ void wait_dma_but_one_tile4() {
  asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
}
__device__ __forceinline__ void slot_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <typename TT, bool ACC, bool BUF>
__global__ __launch_bounds__(kThreadsPP, 1) void bwd_dq_pp_kernel(
    const typename TT::elem* __restrict__ q, const typename TT::elem* __restrict__ k,
    const typename TT::elem* __restrict__ v, const typename TT::elem* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, void* __restrict__ dq,
    BwdParams p) {
  using E = typename TT::elem;
  using v8 = typename TT::v8;
  constexpr int kBufBytes = 2 * kTileBytes;  // K, then V
  __shared__ __attribute__((aligned(1024))) char smem[kNBuf * kBufBytes];
  const uint32_t smem_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;  // 0: A, 1: B (one phase behind)
  const int hl = lane >> 5;
  const int l32 = lane & 31;

  const int32_t BH = p.B * p.Hq;
  int32_t bh;
  int64_t tl;
  work_order(BH, bwd_q_tiles(p, kOwnPP), p.causal != 0, &bh, &tl);
  const int32_t b = bh / p.Hq, hq = bh % p.Hq, hkv = hq / p.group;
  const BwdItem item = bwd_q_item(p, kOwnPP, tl);
  if (item.tile.rows <= 0) return;  // varlen: a tile past the end of its sequence
  const BwdTile qt = item.tile;
  const BwdRun kr0 = item.other[0], kr1 = item.other[1];  // scalars, as in the dK/dV kernel
  const int wq0 = 32 * wave;
  const int wqrows = qt.rows - wq0 < 0 ? 0 : (qt.rows - wq0 > 32 ? 32 : (int)(qt.rows - wq0));
  const bool q_valid = l32 < wqrows;
  const int64_t wqlo = qt.pos0 + wq0;
  const int64_t wqhi = wqlo + wqrows - 1;
  const int64_t qpos = wqlo + l32;
  const int64_t qhi = qt.pos0 + qt.rows - 1;
  const int64_t qrow =
      ((int64_t)b * p.q_rows + p.q_off + qt.row0 + wq0 + (q_valid ? l32 : 0)) * p.Hq + hq;

  v8 qf[KS], gf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (q_valid) {  // a wave past the tile's last row has no row to read
      qf[ks] = *(const v8*)(q + qrow * D + 16 * ks + 8 * hl);
      gf[ks] = *(const v8*)(dout + qrow * D + 16 * ks + 8 * hl);
    } else {
      qf[ks] = gf[ks] = v8{};
    }
  }
  const float l2 = q_valid ? lse2_of(lse[qrow]) : __builtin_inff();
  const float dl = q_valid ? delta[qrow] : 0.f;
  f32x16 dqa[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dqa[db] = f32x16{};

  // key tiles: the live prefix of every key run (for the workgroup's last row)
  const int64_t nt0 =
      item.n_other > 0 ? live_tiles(Run{kr0.row0, kr0.len, kr0.pos0}, qhi, p.causal, kRows) : 0;
  const int64_t nt1 =
      item.n_other > 1 ? live_tiles(Run{kr1.row0, kr1.len, kr1.pos0}, qhi, p.causal, kRows) : 0;
  const int T = (int)(nt0 + nt1);  // a run holds fewer than 2^31 rows
  struct KT {
    int64_t row0;  // flattened row index in [B * k_rows]
    int64_t pos0;
    int rows;
  };
  auto tile_of = [&](int t) {
    KT x;
    const bool second = t >= nt0;
    const int64_t tt = second ? t - nt0 : t;
    const int64_t rem = (second ? kr1.len : kr0.len) - tt * kRows;
    x.rows = rem < kRows ? (int)rem : kRows;
    x.row0 = (int64_t)b * p.k_rows + p.k_off + (second ? kr1.row0 : kr0.row0) + tt * kRows;
    x.pos0 = (second ? kr1.pos0 : kr0.pos0) + tt * kRows;
    return x;
  };

  // ---- DMA: wave w moves rows 8w .. 8w+7 of a tile's K and of its V ---------
  const int64_t kstride = (int64_t)p.Hkv * D;
  const uint32_t row_bytes = (uint32_t)(kstride * (int64_t)sizeof(E));
  const v4i krs = BUF ? tensor_rsrc(k) : v4i{}, vrs = BUF ? tensor_rsrc(v) : v4i{};
  int dma_row[2];
  uint32_t dma_off[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * wave + 4 * i + (lane >> 4);
    dma_row[i] = r;
    dma_off[i] = (uint32_t)r * row_bytes + 16 * ((lane & 15) ^ swz(r));
  }
  int n_req = 0;
  // request the next tile (none once all T are requested); rows past the
  // end of a ragged tile repeat its last row (finite; their dS is 0)
  auto issue_next = [&]() {
    if (n_req >= T) return;
    const KT x = tile_of(n_req);
    const uint32_t lds = smem_addr + (n_req & (kNBuf - 1)) * kBufBytes + 8 * wave * kRowBytes;
    ++n_req;
    const int64_t tb = (x.row0 * kstride + (int64_t)hkv * D) * (int64_t)sizeof(E);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t back =
          dma_row[i] > x.rows - 1 ? (uint32_t)(dma_row[i] - (x.rows - 1)) * row_bytes : 0u;
      const uint32_t lk = lds + 4 * i * kRowBytes;
      if (BUF) {
        dma16(krs, (uint32_t)tb, dma_off[i] - back, lk);
        dma16(vrs, (uint32_t)tb, dma_off[i] - back, lk + kTileBytes);
      } else {
        dma16((const char*)k + tb + (dma_off[i] - back), lk);
        dma16((const char*)v + tb + (dma_off[i] - back), lk + kTileBytes);
      }
    }
  };
  // Group B's first M phase runs the full MFMA stream, so its dQ reads the K
  // half of buffer kNBuf-1 with dS = 0: zero it so that 0 * K stays 0 (no
  // DMA targets that buffer before both groups' first M phase).
  {
    uint4* z = (uint4*)(smem + (kNBuf - 1) * kBufBytes);
    for (int i = tid; i < kTileBytes / 16; i += kThreadsPP) z[i] = uint4{0, 0, 0, 0};
  }
  issue_next();  // tile 0
  issue_next();  // tile 1
  if (T > 1) wait_dma_but_one_tile4(); else wait_dma();
  __syncthreads();

  const FragOff fo = frag_offsets(lane);
  f32x16 sacc[2], dpacc[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) sacc[kb] = dpacc[kb] = f32x16{};
  float dw[16];  // dS of the last scored tile, packed (key pair (r, r+1) of block kb -> 8 kb + r/2)
#pragma unroll
  for (int i = 0; i < 16; ++i) dw[i] = 0.f;

  // One M phase as a flat stream: dQ (16 MFMAs, u-major, db-minor), then S
  // and dP (16 + 16, ks-major: S kb 0, S kb 1, dP kb 0, dP kb 1).  Each
  // MFMA's LDS operand is read kAhead MFMAs ahead.
  constexpr int kAhead = 3;
  auto mfma_stream = [&](auto dq_tag, auto sp_tag, const char* dqb, const char* spb) {
    constexpr bool DQ = decltype(dq_tag)::value;
    constexpr bool SP = decltype(sp_tag)::value;
    constexpr int NDQ = DQ ? 4 * DB : 0;
    constexpr int N = NDQ + (SP ? 4 * KS : 0);
    auto load = [&](int i) -> v8 {
      if (DQ && i < NDQ) return tr_frag<TT>(dqb, fo, i % DB, i / DB);
      const int j = i - NDQ;
      const int sel = j & 3;  // 0, 1: K rows of block 0, 1; 2, 3: V rows
      return row_frag<TT>(spb + (sel >> 1) * kTileBytes, fo, j >> 2, sel & 1);
    };
    v8 fb[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i)
      if (i < N) fb[i] = load(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const v8 a = fb[i % kAhead];
      if (i + kAhead < N) fb[i % kAhead] = load(i + kAhead);
      if (DQ && i < NDQ) {
        const int u = i / DB;
        dqa[i % DB] = TT::mfma32x32x16(a, packed_operand<TT>(dw, u), dqa[i % DB]);
      } else {
        const int j = i - NDQ, sel = j & 3, ks = j >> 2;
        if (sel < 2)
          sacc[sel] = TT::mfma32x32x16(a, qf[ks], ks == 0 ? f32x16{} : sacc[sel]);
        else
          dpacc[sel - 2] = TT::mfma32x32x16(a, gf[ks], ks == 0 ? f32x16{} : dpacc[sel - 2]);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep this issue order
    }
  };
  auto m_phase = [&](int kk, auto dq_tag, auto sp_tag) {
    const char* dqb = smem + ((kk - 1) & (kNBuf - 1)) * kBufBytes;
    const char* spb = smem + (kk & (kNBuf - 1)) * kBufBytes;
    __builtin_amdgcn_s_setprio(1);
    issue_next();
    mfma_stream(dq_tag, sp_tag, dqb, spb);
    __builtin_amdgcn_s_setprio(0);
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;

  // V phase of tile t: dS into dw (0 for a tile none of the wave's rows sees)
  int vt = 0;
  auto v_phase = [&]() {
    const KT x = tile_of(vt);
    ++vt;
    if (wqrows == 0 || (p.causal && x.pos0 > wqhi)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dw[i] = 0.f;
      return;
    }
    const bool need_mask = x.rows < kRows || (p.causal && x.pos0 + x.rows - 1 > wqlo);
    // key of register r of block kb: 32 kb + 8 (r/4) + 4 hl + r%4; keys
    // below lim are visible to this lane's query
    const int lim =
        (need_mask ? visible_limit(x.rows, p.causal, qpos - x.pos0) : kRows) - 4 * hl;
    float pr[2][16];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[kb][r] = fmaf(sacc[kb][r], p.c, -l2);
    __builtin_amdgcn_sched_barrier(0x4);  // only scalar work moves across
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[kb][r] = exp2_fast(pr[kb][r]);
    __builtin_amdgcn_sched_barrier(0x4);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk2 = 32 * kb + 8 * (r >> 2) + (r & 3);
          pr[kb][r] = kk2 < lim ? pr[kb][r] : 0.f;
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        pack_pair<TT>(&dw[8 * kb + (r >> 1)], pr[kb][r] * (dpacc[kb][r] - dl),
                      pr[kb][r + 1] * (dpacc[kb][r + 1] - dl));
  };

  // Before the window in which the groups score tile j, tile j must have
  // landed on every wave; only tile j+1's requests may still be in flight.
  auto wait_tile = [&](int j) {
    if (j + 1 < T) wait_dma_but_one_tile4(); else wait_dma();
  };
  // Windows as in the forward's ping-pong: buffer m%4 is written (tile m,
  // window m-1) after the barrier that ends window m-2, where its last
  // readers (the dQ of tile m-4 in both groups' M_{m-3}) are done; tile m is
  // complete on every wave at the barrier that ends window m, before its
  // first reader (M_m, window m+1).  Both groups pass T+1 barriers.
  if (group == 0) {
    m_phase(0, no{}, yes{});
    slot_barrier();
    for (int j = 0; j + 1 < T; ++j) {
      v_phase();
      wait_tile(j + 1);
      slot_barrier();
      m_phase(j + 1, yes{}, yes{});
    }
    if (T > 0) {
      v_phase();
      wait_tile(T);
      slot_barrier();
      m_phase(T, yes{}, no{});  // dQ of the last tile
    }
  } else {
    slot_barrier();
    for (int j = 0; j < T; ++j) {
      m_phase(j, yes{}, yes{});
      wait_tile(j + 1);
      slot_barrier();
      v_phase();
    }
    m_phase(T, yes{}, no{});  // dQ of the last tile
  }

  if (!q_valid) return;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int d0 = 32 * db + 8 * j + 4 * hl;
      f32x4 g;
#pragma unroll
      for (int e = 0; e < 4; ++e) g[e] = dqa[db][4 * j + e] * p.scale;
      if (ACC) {
        f32x4* o = (f32x4*)((float*)dq + qrow * D + d0);
        *o = *o + g;
      } else {
        typename TT::v4 eg;
#pragma unroll
        for (int e = 0; e < 4; ++e) eg[e] = to_elem<TT>(g[e]);
        *(typename TT::v4*)((E*)dq + qrow * D + d0) = eg;
      }
    }
}

template <typename TT, bool ACC>
hipError_t launch_acc(const void* q, const void* k, const void* v, const void* dout,
                      const float* lse, const float* delta, void* dq, void* dk, void* dv,
                      const BwdParams& p, hipStream_t stream) {
  using E = typename TT::elem;
  // buffer-form DMA while q, dO, k and v are each below 4 GB (32-bit offsets)
  const uint64_t lim = 0xFFFF0000ull;
  const bool buf = (uint64_t)p.B * p.q_rows * p.Hq * D * sizeof(E) <= lim &&
                   (uint64_t)p.B * p.k_rows * p.Hkv * D * sizeof(E) <= lim;
  const int64_t qb = bwd_q_tiles(p, kOwnPP) * p.B * p.Hq;
  if (qb > 0) {
    if (buf)
      hipLaunchKernelGGL((bwd_dq_pp_kernel<TT, ACC, true>), dim3((unsigned)qb),
                         dim3(kThreadsPP), 0, stream, (const E*)q, (const E*)k, (const E*)v,
                         (const E*)dout, lse, delta, dq, p);
    else
      hipLaunchKernelGGL((bwd_dq_pp_kernel<TT, ACC, false>), dim3((unsigned)qb),
                         dim3(kThreadsPP), 0, stream, (const E*)q, (const E*)k, (const E*)v,
                         (const E*)dout, lse, delta, dq, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t kb = bwd_k_tiles(p, kOwn) * p.B * p.Hkv;
  if (kb > 0) {
    if (buf)
      hipLaunchKernelGGL((bwd_dkv_mfma_kernel<TT, ACC, true>), dim3((unsigned)kb),
                         dim3(kThreadsKV), 0, stream, (const E*)q, (const E*)k, (const E*)v,
                         (const E*)dout, lse, delta, dk, dv, p);
    else
      hipLaunchKernelGGL((bwd_dkv_mfma_kernel<TT, ACC, false>), dim3((unsigned)kb),
                         dim3(kThreadsKV), 0, stream, (const E*)q, (const E*)k, (const E*)v,
                         (const E*)dout, lse, delta, dk, dv, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename TT>
hipError_t launch_t(const void* q, const void* k, const void* v, const void* dout,
                    const float* lse, const float* delta, void* dq, void* dk, void* dv,
                    const BwdParams& p, hipStream_t stream) {
  return p.accumulate ? launch_acc<TT, true>(q, k, v, dout, lse, delta, dq, dk, dv, p, stream)
                      : launch_acc<TT, false>(q, k, v, dout, lse, delta, dq, dk, dv, p, stream);
}

}  // namespace

hipError_t launch_bwd_mfma(int dtype, const void* q, const void* k, const void* v,
                           const void* dout, const float* lse, const float* delta, void* dq,
                           void* dk, void* dv, const BwdParams& p, hipStream_t stream) {
  switch (dtype) {
    case 1: return launch_t<F16>(q, k, v, dout, lse, delta, dq, dk, dv, p, stream);
    case 2: return launch_t<Bf16>(q, k, v, dout, lse, delta, dq, dk, dv, p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace rattn
