// ring_sched.h -- work description shared by the host scheduler and the kernels.
//
// The ring schedule is simulated on one GPU.  A launch covers a set of query
// rows split into segments; every segment belongs to one ring rank and has
// contiguous global positions.  For each query tile the kernel walks the
// key/value "visits" of its rank in ring order and classifies every key tile
// as skipped, fully visible or masked by comparing global positions.
//
// Ring order (ultralytics.com "Ring Attention", how-it-works section;
// youngju.dev "Ring Attention" analysis, ring forward): at step s rank r holds
// the key/value block of rank (r - s) mod W.
// ZigZag (Twinkle "Sequence parallel and Ring Attention", ZigZag section):
// rank r owns chunks r and 2W-1-r of the 2W equal chunks.
// Causal rule: a key is visible iff its position is not after the query's
// (youngju.dev causal step: the strict upper triangle of the diagonal block is
// masked; earlier blocks are fully visible, later ones skipped).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define RATTN_HD __host__ __device__ __forceinline__
#else
#define RATTN_HD inline
#endif

namespace rattn {

constexpr int kMaxQSeg = 64;  // 2W segments for a ZigZag launch over all ranks

enum VisitMode : int32_t {
  kVisitExplicit = 0,        // the launch lists its key/value runs (one ring step)
  kVisitContiguousRing = 1,  // rank r holds block r of W equal blocks
  kVisitZigZagRing = 2,      // rank r holds chunks r and 2W-1-r of 2W chunks
  kVisitVarlen = 3,          // independent sequences of a packed batch
};

// A contiguous run of rows of a tensor: rows [row0, row0+len) sit at global
// positions pos0, pos0+1, ...
struct Run {
  int64_t row0;
  int64_t len;
  int64_t pos0;
};

struct QSeg {
  int64_t row0;
  int64_t len;
  int64_t pos0;
  int32_t rank;        // ring rank owning these query rows (selects the visit order)
  int32_t tile_begin;  // first linear tile index of this segment
};

struct Sched {
  int32_t mode;       // VisitMode
  int32_t W;          // ring size
  int64_t blk;        // rows per block (contiguous) or per chunk (ZigZag)
  int32_t causal;
  int32_t reverse;    // enumerate tiles of a segment from the last one (longest first)
  int32_t n_kruns;    // explicit mode only
  int32_t n_qseg;
  int32_t n_tiles;    // query tiles per (batch, head)
  int32_t br;         // query rows per tile this schedule was built for
  Run kruns[2];
  QSeg qseg[kMaxQSeg];
  // Varlen mode: sequence i owns query rows [vl_q_start[i], +vl_q_len[i]) and
  // key/value rows [vl_k_start[i], +vl_k_len[i]) (device arrays of vl_nseq
  // int32, clamped to the vl_nq / vl_nk rows the tensors hold); query tile t
  // is tile t % vl_tiles of sequence t / vl_tiles.  Positions inside a
  // sequence: key j at j, query i at len_k - len_q + i (the last query
  // aligned with the last key).
  const int32_t* vl_q_start;
  const int32_t* vl_q_len;
  const int32_t* vl_k_start;
  const int32_t* vl_k_len;
  int32_t vl_nseq;
  int32_t vl_tiles;
  int64_t vl_nq;
  int64_t vl_nk;
};

RATTN_HD int32_t num_visits(const Sched& s) {
  if (s.mode == kVisitVarlen) return 1;
  return s.mode == kVisitExplicit ? s.n_kruns : (s.mode == kVisitContiguousRing ? s.W : 2 * s.W);
}

#if defined(__HIPCC__)
// Key/value rows of varlen sequence i, clamped to the rows k holds (device only).
__device__ __forceinline__ Run varlen_keys(const Sched& s, int32_t i) {
  const int64_t st = s.vl_k_start[i];
  int64_t len = s.vl_k_len[i];
  if (st < 0 || st > s.vl_nk) return Run{0, 0, 0};
  if (len > s.vl_nk - st) len = s.vl_nk - st;
  return Run{st, len < 0 ? 0 : len, 0};
}
#endif

// Key/value run visited at position v of rank's ring order.  Outside explicit
// mode the key/value tensor is in natural order, so row index == position.
// Ring modes take 0 <= rank < W and 0 <= v < num_visits, so the source rank
// (rank - step) mod W is rank - step, plus W when that is negative (no
// integer division, which the GPU does in software).
RATTN_HD Run visit(const Sched& s, int32_t rank, int32_t v) {
  Run r;
#if defined(__HIP_DEVICE_COMPILE__)
  if (s.mode == kVisitVarlen) return varlen_keys(s, rank);  // rank = sequence
#endif
  if (s.mode == kVisitExplicit) {
    r = s.kruns[v];
  } else if (s.mode == kVisitContiguousRing) {
    int32_t src = rank - v;
    if (src < 0) src += s.W;
    r.row0 = (int64_t)src * s.blk;
    r.len = s.blk;
    r.pos0 = r.row0;
  } else {
    int32_t step = v >> 1;
    int32_t src = rank - step;
    if (src < 0) src += s.W;
    int32_t chunk = (v & 1) ? (2 * s.W - 1 - src) : src;
    r.row0 = (int64_t)chunk * s.blk;
    r.len = s.blk;
    r.pos0 = r.row0;
  }
  return r;
}

// Number of key tiles of `run` that hold at least one key visible to a query
// at position <= qhi.  Under the causal rule the visible tiles of a run with
// increasing positions form a prefix.
RATTN_HD int64_t live_tiles(const Run& r, int64_t qhi, int32_t causal, int32_t bc) {
  if (r.len <= 0) return 0;
  int64_t n = (r.len + bc - 1) / bc;
  if (!causal) return n;
  if (r.pos0 > qhi) return 0;
  int64_t m = (qhi - r.pos0) / bc + 1;
  return m < n ? m : n;
}

// Query tile lookup: linear tile index -> (segment, rows, positions).
struct QTile {
  int64_t row0;  // first query row
  int64_t rows;  // rows in this tile (<= br)
  int64_t pos0;  // position of the first row
  int32_t rank;
};

// br: query rows per tile, the s.br the schedule was built with; kernels pass
// it as a compile-time constant, so that the divisions by it are shifts.
RATTN_HD QTile query_tile(const Sched& s, int32_t t, int32_t br) {
  QTile qt;
#if defined(__HIP_DEVICE_COMPILE__)
  if (s.mode == kVisitVarlen) {
    // rows <= 0: a tile past the end of its sequence (the kernel exits)
    const int32_t i = t / s.vl_tiles;
    int64_t lt = t % s.vl_tiles;
    const int64_t st = s.vl_q_start[i];
    int64_t lq = s.vl_q_len[i];
    if (st < 0 || st > s.vl_nq) lq = 0;
    if (lq > s.vl_nq - st) lq = s.vl_nq - st;
    const int64_t nt = (lq + br - 1) / br;
    if (s.reverse) lt = nt - 1 - lt;  // causal: latest (longest) tiles first
    qt.row0 = st + lt * br;
    const int64_t rem = lq - lt * br;
    qt.rows = (lt < 0 || lt >= nt) ? 0 : (rem < br ? rem : br);
    qt.pos0 = varlen_keys(s, i).len - lq + lt * br;
    qt.rank = i;
    return qt;
  }
#endif
  // segment i: the last one whose tile_begin <= t (binary search; tile_begin
  // increases with i and qseg[0].tile_begin = 0)
  int32_t i = 0, hi = s.n_qseg;
  while (hi - i > 1) {
    const int32_t mid = (i + hi) >> 1;
    if (t < s.qseg[mid].tile_begin) hi = mid; else i = mid;
  }
  const QSeg& g = s.qseg[i];
  int64_t nt = (g.len + br - 1) / br;
  int64_t lt = t - g.tile_begin;
  if (s.reverse) lt = nt - 1 - lt;
  qt.row0 = g.row0 + lt * br;
  int64_t rem = g.len - lt * br;
  qt.rows = rem < br ? rem : br;
  qt.pos0 = g.pos0 + lt * br;
  qt.rank = g.rank;
  return qt;
}

}  // namespace rattn
