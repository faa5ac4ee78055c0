// rattn_abi.hip -- the C ABI (include/rattn.h): argument checks, the ring
// scheduler that turns (W, zigzag, rank) or explicit segments into query
// segments and key/value visits, and kernel dispatch.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "bwd.h"
#include "launch.h"
#include "rattn.h"
#include "ring_sched.h"

namespace rattn {
namespace {

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

constexpr int kMaxSplits = 64;  // split-KV: most key splits per query tile

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

// a*b without signed overflow, for sizes that are all >= 0.
bool mul_ok(int64_t a, int64_t b, int64_t* r) {
  if (a != 0 && b > INT64_MAX / a) return false;
  *r = a * b;
  return true;
}

// Element count of a [B, N, H, d] tensor fits comfortably in 64-bit offsets,
// and N rows in 31 bits (the kernels count rows and tiles of a run in 32 bits).
bool tensor_ok(int64_t B, int64_t N, int64_t H, int64_t d) {
  int64_t x;
  return N < ((int64_t)1 << 31) && mul_ok(B, N, &x) && mul_ok(x, H, &x) && mul_ok(x, d, &x) &&
         x < ((int64_t)1 << 60);
}

// Fill tile_begin in longest-first order (causal: the segment with the latest
// positions first, and inside a segment the last tile first) and count tiles.
int finalize(Sched& s, QSeg* segs, int n, int br) {
  int m = 0;
  for (int i = 0; i < n; ++i)
    if (segs[i].len > 0) segs[m++] = segs[i];
  if (s.causal)
    std::stable_sort(segs, segs + m, [](const QSeg& a, const QSeg& b) {
      return a.pos0 + a.len > b.pos0 + b.len;
    });
  int64_t tiles = 0;
  for (int i = 0; i < m; ++i) {
    segs[i].tile_begin = (int32_t)tiles;
    tiles += (segs[i].len + br - 1) / br;
    if (tiles > INT32_MAX) return RATTN_EUNSUPPORTED;
    s.qseg[i] = segs[i];
  }
  s.n_qseg = m;
  s.n_tiles = (int32_t)tiles;
  s.reverse = s.causal ? 1 : 0;
  s.br = br;
  return RATTN_OK;
}

int check_dtype_d(int dtype, int d) {
  if (dtype < RATTN_F32 || dtype > RATTN_BF16) return RATTN_EINVAL;
  if (!supported_d(d)) return RATTN_EUNSUPPORTED;
  return RATTN_OK;
}

bool use_mfma(int dtype, int d) { return dtype != RATTN_F32 && d >= 16; }

// Query rows per tile of the kernel that will run (the schedule is built for it).
int tile_rows(int dtype, int d) {
  if (!use_mfma(dtype, d)) return kGenericBr;
  return d >= 32 ? kMfma128Br : kMfmaBr;
}

float resolve_scale(float scale, int d) {
  return (scale > 0.f && isfinite(scale)) ? scale : (float)(1.0 / sqrt((double)d));
}

FwdParams make_params(int B, int Hq, int Hkv, int64_t Nq, int64_t Nk, float scale) {
  FwdParams p;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.group = Hq / Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.c = (float)((double)scale * 1.4426950408889634074);  // scale * log2(e)
  p.n_splits = 1;
  p.split_out_stride = 0;
  p.split_lse_stride = 0;
  p.out_rows = Nq;
  p.out_row_off = 0;
  p.merge_out = 0;
  return p;
}

// The schedule with query tiles of br rows (same segments, same order).
bool retile(Sched& s, int br) {
  int64_t tiles = 0;
  for (int i = 0; i < s.n_qseg; ++i) {
    s.qseg[i].tile_begin = (int32_t)tiles;
    tiles += (s.qseg[i].len + br - 1) / br;
    if (tiles > INT32_MAX) return false;
  }
  s.n_tiles = (int32_t)tiles;
  s.br = br;
  return true;
}

// A 16-bit launch (d = 32, 64, 128) with few 256-row work items runs on the
// key-split kernel instead (32 query rows per workgroup, the key tiles
// divided among its 8 waves, merged in LDS).  That kernel moves each
// key/value byte for 32 query rows instead of 256, so it pays only where the
// 256-row items leave compute units idle.  Chosen when the items number at
// most a quarter of the compute units (uniform items), or half of them for
// causal items (whose lengths vary, so the 256-row launch waits for its
// longest) -- at d = 32 twice that, the narrow rows costing the key-split
// kernel less -- and when its items are long (the first query tile, the
// longest under the causal order, sees at least 24 key tiles of 64) or very
// few (at most a quarter of the compute units either way).
// Measured on MI355X (us per call, 256-row kernel -> key-split kernel):
// d = 128 bf16, one head of 4096 queries 86 -> 29, 8 causal heads of 4096
// 87 -> 69; 8 non-causal heads of 4096 stay on the 256-row kernel (93 against
// 117); d = 64 fp16 one head 64 -> 20, (B, N, H) = (2, 1024, 4) 22 -> 13;
// d = 32 one head 67 -> 15, 16 non-causal heads of 2048 39 -> 29.
// Split-KV launches decide on the same unsplit items; each split of a query
// tile is then one workgroup of the key-split kernel.
// The environment variable RATTN_FWD_SHORT overrides the choice for every
// eligible launch: "0" never takes the key-split kernel, "1" always does.
bool short_launch(int dtype, int d, const FwdParams& p, const Sched& s) {
  if (!use_mfma(dtype, d) || d < 32 || s.mode == kVisitVarlen) return false;
  const char* env = getenv("RATTN_FWD_SHORT");
  if (env && env[0] == '0' && env[1] == 0) return false;
  const char* ser = getenv("RATTN_SERIALIZE");  // the 256-row kernel's debug schedule
  if (ser && ser[0] == '1' && ser[1] == 0) return false;
  if (env && env[0] == '1' && env[1] == 0) return true;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;  // the regular launch reports the error
  const int64_t items = (int64_t)s.n_tiles * p.B * p.Hq;
  const int64_t room = (int64_t)cus * (d == 32 ? 2 : 1);
  if (items <= 0 || items * (s.causal ? 2 : 4) > room) return false;
  if (items * 4 <= (int64_t)cus) return true;
  const QTile qt = query_tile(s, 0, s.br);
  int64_t t64 = 0;
  for (int32_t v = 0; v < num_visits(s); ++v)
    t64 += live_tiles(visit(s, qt.rank, v), qt.pos0 + qt.rows - 1, s.causal, 64);
  return t64 >= 24;
}

int dispatch(int dtype, int d, const void* q, const void* k, const void* v, void* out,
             float* lse, bool out_f32, const FwdParams& p, const Sched& s, int64_t grid,
             void* stream, uint32_t* queues = nullptr) {
  if (grid > INT32_MAX) return RATTN_EUNSUPPORTED;
  hipError_t e;
  if (short_launch(dtype, d, p, s)) {
    Sched s32 = s;
    if (retile(s32, kShortBr) && (int64_t)s32.n_tiles * p.B * p.Hq * p.n_splits <= INT32_MAX) {
      e = launch_fwd_short(dtype, d, q, k, v, out, lse, out_f32, p, s32, (hipStream_t)stream);
      return e == hipSuccess ? RATTN_OK : RATTN_EHIP;
    }
  }
  if (use_mfma(dtype, d))
    e = launch_fwd_mfma(dtype, d, q, k, v, out, lse, out_f32, p, s, queues, (hipStream_t)stream);
  else
    e = launch_fwd_generic(dtype, d, q, k, v, out, lse, out_f32, p, s, (hipStream_t)stream);
  return e == hipSuccess ? RATTN_OK : RATTN_EHIP;
}

}  // namespace
}  // namespace rattn

using namespace rattn;

namespace rattn {
namespace {

// Checks of rattn_fwd's arguments and its schedule (shared with rattn_fwd_split).
int prepare_ring(const void* q, const void* k, const void* v, const void* out, const float* lse,
                 int B, int Hq, int Hkv, int64_t Nq, int64_t N, int d, int dtype, int causal,
                 int n_ring_steps, int zigzag, int rank, Sched* sched) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return RATTN_EINVAL;
  if (N < 0 || Nq < 0) return RATTN_EINVAL;
  // a pointer may be null only when its tensor is empty
  if ((Nq > 0 && (!q || !out || !lse)) || (N > 0 && (!k || !v))) return RATTN_EINVAL;
  int rc = check_dtype_d(dtype, d);
  if (rc != RATTN_OK) return rc;
  if ((causal != 0 && causal != 1) || (zigzag != 0 && zigzag != 1)) return RATTN_EINVAL;
  if (n_ring_steps < 1) return RATTN_EINVAL;
  if (n_ring_steps > kMaxQSeg / 2) return RATTN_EUNSUPPORTED;
  const int W = n_ring_steps;
  const int64_t parts = zigzag ? 2 * (int64_t)W : W;
  if (N % parts != 0) return RATTN_EINVAL;
  if (rank < -1 || rank >= W) return RATTN_EINVAL;
  if (rank == -1 ? Nq != N : Nq != N / W) return RATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(lse, 4))
    return RATTN_EINVAL;
  if (!tensor_ok(B, N, Hq > Hkv ? Hq : Hkv, d)) return RATTN_EUNSUPPORTED;

  const int br = tile_rows(dtype, d);
  Sched& s = *sched;
  memset(&s, 0, sizeof s);
  s.W = W;
  s.causal = causal;
  QSeg segs[kMaxQSeg];
  memset(segs, 0, sizeof segs);
  int n = 0;
  if (!zigzag) {
    s.mode = kVisitContiguousRing;
    s.blk = N / W;
    if (rank >= 0) {
      segs[n++] = QSeg{0, Nq, rank * s.blk, rank, 0};
    } else {
      for (int g = 0; g < W; ++g) segs[n++] = QSeg{g * s.blk, s.blk, g * s.blk, g, 0};
    }
  } else {
    s.mode = kVisitZigZagRing;
    const int64_t c = N / (2 * (int64_t)W);
    s.blk = c;
    if (rank >= 0) {
      segs[n++] = QSeg{0, c, rank * c, rank, 0};
      segs[n++] = QSeg{c, c, (2 * (int64_t)W - 1 - rank) * c, rank, 0};
    } else {
      for (int g = 0; g < 2 * W; ++g)
        segs[n++] = QSeg{g * c, c, g * c, g < W ? g : 2 * W - 1 - g, 0};
    }
  }
  return finalize(s, segs, n, br);
}

}  // namespace
}  // namespace rattn

extern "C" int rattn_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                         int B, int Hq, int Hkv, int64_t Nq, int64_t N, int d, int dtype,
                         float scale, int causal, int n_ring_steps, int zigzag, int rank,
                         void* stream) {
  Sched s;
  const int rc = prepare_ring(q, k, v, out, lse, B, Hq, Hkv, Nq, N, d, dtype, causal,
                              n_ring_steps, zigzag, rank, &s);
  if (rc != RATTN_OK || Nq == 0) return rc;
  const FwdParams p = make_params(B, Hq, Hkv, Nq, N, resolve_scale(scale, d));
  return dispatch(dtype, d, q, k, v, out, lse, false, p, s, (int64_t)s.n_tiles * B * Hq, stream);
}

extern "C" int rattn_fwd_queued(const void* q, const void* k, const void* v, void* out,
                                float* lse, int B, int Hq, int Hkv, int64_t Nq, int64_t N, int d,
                                int dtype, float scale, int causal, int n_ring_steps, int zigzag,
                                int rank, void* queue_ws, int64_t queue_ws_bytes, void* stream) {
  Sched s;
  const int rc = prepare_ring(q, k, v, out, lse, B, Hq, Hkv, Nq, N, d, dtype, causal,
                              n_ring_steps, zigzag, rank, &s);
  if (rc != RATTN_OK || Nq == 0) return rc;
  if (!queue_ws || queue_ws_bytes < RATTN_QUEUE_WS_BYTES || !aligned(queue_ws, 4))
    return RATTN_EINVAL;
  static_assert(kFwdQueues * sizeof(uint32_t) <= RATTN_QUEUE_WS_BYTES, "queue workspace");
  const FwdParams p = make_params(B, Hq, Hkv, Nq, N, resolve_scale(scale, d));
  return dispatch(dtype, d, q, k, v, out, lse, false, p, s, (int64_t)s.n_tiles * B * Hq, stream,
                  (uint32_t*)queue_ws);
}

extern "C" int rattn_fwd_varlen(const void* q, const void* k, const void* v, void* out,
                                float* lse, const int32_t* q_start, const int32_t* q_len,
                                const int32_t* k_start, const int32_t* k_len, int n_seq,
                                int64_t max_len_q, int64_t Nq, int64_t Nk, int Hq, int Hkv,
                                int d, int dtype, float scale, int causal, void* stream) {
  using namespace rattn;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return RATTN_EINVAL;
  if (n_seq < 0 || max_len_q < 0 || Nq < 0 || Nk < 0) return RATTN_EINVAL;
  int rc = check_dtype_d(dtype, d);
  if (rc != RATTN_OK) return rc;
  if (causal != 0 && causal != 1) return RATTN_EINVAL;
  if (n_seq == 0 || max_len_q == 0 || Nq == 0) return RATTN_OK;
  if (!q || !out || !lse || !q_start || !q_len || !k_start || !k_len || (Nk > 0 && (!k || !v)))
    return RATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(lse, 4) || !aligned(q_start, 4) || !aligned(q_len, 4) || !aligned(k_start, 4) ||
      !aligned(k_len, 4))
    return RATTN_EINVAL;
  if (!tensor_ok(1, std::max(Nq, Nk), Hq > Hkv ? Hq : Hkv, d)) return RATTN_EUNSUPPORTED;
  const int br = tile_rows(dtype, d);
  const int64_t tiles = (max_len_q + br - 1) / br;
  if (tiles > INT32_MAX || tiles * n_seq > INT32_MAX) return RATTN_EUNSUPPORTED;
  Sched s;
  memset(&s, 0, sizeof s);
  s.mode = kVisitVarlen;
  s.W = 1;
  s.causal = causal;
  s.reverse = causal ? 1 : 0;
  s.br = br;
  s.n_tiles = (int32_t)(tiles * n_seq);
  s.vl_q_start = q_start;
  s.vl_q_len = q_len;
  s.vl_k_start = k_start;
  s.vl_k_len = k_len;
  s.vl_nseq = n_seq;
  s.vl_tiles = (int32_t)tiles;
  s.vl_nq = Nq;
  s.vl_nk = Nk;
  const FwdParams p = make_params(1, Hq, Hkv, Nq, Nk, resolve_scale(scale, d));
  return dispatch(dtype, d, q, k, v, out, lse, false, p, s, (int64_t)s.n_tiles * Hq, stream);
}

extern "C" int rattn_fwd_split(const void* q, const void* k, const void* v, void* out,
                               float* lse, int B, int Hq, int Hkv, int64_t Nq, int64_t N, int d,
                               int dtype, float scale, int causal, int n_ring_steps, int zigzag,
                               int rank, int n_splits, float* ws, int64_t ws_floats,
                               void* stream) {
  if (n_splits < 1) return RATTN_EINVAL;
  if (n_splits > kMaxSplits) return RATTN_EUNSUPPORTED;
  Sched s;
  int rc = prepare_ring(q, k, v, out, lse, B, Hq, Hkv, Nq, N, d, dtype, causal, n_ring_steps,
                        zigzag, rank, &s);
  if (rc != RATTN_OK || Nq == 0) return rc;
  if (n_splits == 1)
    return rattn_fwd(q, k, v, out, lse, B, Hq, Hkv, Nq, N, d, dtype, scale, causal,
                     n_ring_steps, zigzag, rank, stream);
  const int64_t rows = (int64_t)B * Nq * Hq;
  int64_t need;
  if (!mul_ok(rows, (int64_t)d + 1, &need) || !mul_ok(need, n_splits, &need))
    return RATTN_EUNSUPPORTED;
  if (!ws || ws_floats < need || !aligned(ws, 16)) return RATTN_EINVAL;
  FwdParams p = make_params(B, Hq, Hkv, Nq, N, resolve_scale(scale, d));
  p.n_splits = n_splits;
  p.split_out_stride = rows * d;
  p.split_lse_stride = rows;
  float* ws_out = ws;
  float* ws_lse = ws + (int64_t)n_splits * rows * d;
  rc = dispatch(dtype, d, q, k, v, ws_out, ws_lse, true, p, s,
                (int64_t)s.n_tiles * B * Hq * n_splits, stream);
  if (rc != RATTN_OK) return rc;
  if ((rows * (d / 4) + 255) / 256 > INT32_MAX) return RATTN_EUNSUPPORTED;
  const hipError_t e = launch_split_reduce(dtype, d, out, lse, ws_out, ws_lse, n_splits, rows,
                                           (hipStream_t)stream);
  return e == hipSuccess ? RATTN_OK : RATTN_EHIP;
}

// ---- split-KV without allocation -------------------------------------------

// The partials of rattn_fwd_split_noalloc: one fixed array per GPU (each GPU
// that runs the library holds its own copy).  Host code never passes this
// name to a kernel: on the host it is a stand-in, not a device address; the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[RATTN_NOALLOC_SCRATCH_FLOATS];

namespace rattn {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The scratch of the calling thread's current device.
int device_scratch(float** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return RATTN_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return RATTN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return RATTN_EHIP;
    g_scratch_ptr[dev] = (float*)p;
  }
  *ptr = g_scratch_ptr[dev];
  return RATTN_OK;
}

}  // namespace
}  // namespace rattn

extern "C" int rattn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* out,
                                       float* lse, int B, int Hq, int Hkv, int64_t Nq,
                                       int64_t N, int d, int dtype, float scale, int causal,
                                       int n_ring_steps, int zigzag, int rank, int n_splits,
                                       void* stream) {
  if (n_splits < 1) return RATTN_EINVAL;
  if (n_splits > kMaxSplits) return RATTN_EUNSUPPORTED;
  Sched s;
  const int rc = prepare_ring(q, k, v, out, lse, B, Hq, Hkv, Nq, N, d, dtype, causal,
                              n_ring_steps, zigzag, rank, &s);
  if (rc != RATTN_OK || Nq == 0) return rc;
  if (n_splits == 1)
    return rattn_fwd(q, k, v, out, lse, B, Hq, Hkv, Nq, N, d, dtype, scale, causal,
                     n_ring_steps, zigzag, rank, stream);
  int64_t need;
  if (!mul_ok((int64_t)B * Nq * Hq, (int64_t)d + 1, &need) || !mul_ok(need, n_splits, &need) ||
      need > RATTN_NOALLOC_SCRATCH_FLOATS)
    return RATTN_ESCRATCH;
  float* ws = nullptr;
  const int sc = device_scratch(&ws);
  if (sc != RATTN_OK) return sc;
  return rattn_fwd_split(q, k, v, out, lse, B, Hq, Hkv, Nq, N, d, dtype, scale, causal,
                         n_ring_steps, zigzag, rank, n_splits, ws, RATTN_NOALLOC_SCRATCH_FLOATS,
                         stream);
}

extern "C" int rattn_split_hint(int B, int Hq, int64_t Nq, int64_t N, int d, int dtype,
                                int n_ring_steps, int zigzag, int rank, int n_cu) {
  (void)zigzag;
  (void)rank;
  if (B < 1 || Hq < 1 || Nq < 1 || N < 1 || n_cu < 1 || n_ring_steps < 1) return 1;
  if (check_dtype_d(dtype, d) != RATTN_OK) return 1;
  const int64_t br = tile_rows(dtype, d);
  const int64_t items = (Nq + br - 1) / br * B * Hq;
  // Launches this small run on the key-split kernel (32 query rows per
  // workgroup) unless RATTN_FWD_SHORT=0: aim at one of its workgroups per
  // compute unit, each wave keeping at least 4 key tiles of 32 (one head of
  // 4096 queries: 128 workgroups, 2 splits).
  const char* env = getenv("RATTN_FWD_SHORT");
  const bool short_off = env && env[0] == '0' && env[1] == 0;
  if (!short_off && dtype != RATTN_F32 && d >= 32 && items * 4 <= (int64_t)n_cu) {
    const int64_t groups = (Nq + kShortBr - 1) / kShortBr * B * Hq;
    int64_t n = (int64_t)n_cu / groups;
    const int64_t cap = ((N + 31) / 32) / (8 * 4);
    if (n > cap) n = cap;
    if (n > kMaxSplits) n = kMaxSplits;
    return n < 1 ? 1 : (int)n;
  }
  // Half as many workgroups as compute units already hides most of the
  // split's cost (partials written and merged); measured on 4096 x 4096,
  // one head: 8 splits (128 workgroups) beat 4, 16 and 32.
  const int64_t want = ((int64_t)n_cu + 1) / 2;
  if (items >= want) return 1;
  int64_t n = (want + items - 1) / items;
  const int64_t key_tiles = (N + 63) / 64;  // keep at least 8 key tiles per split
  if (n > key_tiles / 8) n = key_tiles / 8;
  if (n > kMaxSplits) n = kMaxSplits;
  return n < 1 ? 1 : (int)n;
}

namespace rattn {
namespace {

// rattn_fwd_step / rattn_fwd_step_merge: query rows [q_off, q_off + Nq) of a
// [B, q_rows, Hq, d] tensor over key/value rows [k_off, k_off + Nk) of
// [B, k_rows, Hkv, d] tensors; output rows [row_off, row_off + Nq) of a
// [B, Nq_out, Hq, d] fp32 output; merge = 1 merges into it.
int fwd_step_impl(const void* q, const void* k_blk, const void* v_blk, float* out,
                  float* lse, int B, int Hq, int Hkv, int64_t q_rows, int64_t q_off, int64_t Nq,
                  int64_t k_rows, int64_t k_off, int64_t Nk, int d, int dtype,
                  float scale, int causal, const int64_t* q_seg_start, const int64_t* q_seg_len,
                  const int64_t* k_seg_start, const int64_t* k_seg_len, int64_t Nq_out,
                  int64_t row_off, int merge, void* stream) {
  if (!q_seg_start || !q_seg_len || !k_seg_start || !k_seg_len) return RATTN_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return RATTN_EINVAL;
  if (Nq < 0 || Nk < 0 || row_off < 0 || Nq_out < 0) return RATTN_EINVAL;
  if (q_off < 0 || k_off < 0 || q_off > q_rows || Nq > q_rows - q_off || k_off > k_rows ||
      Nk > k_rows - k_off)
    return RATTN_EINVAL;
  if (row_off > Nq_out || Nq > Nq_out - row_off) return RATTN_EINVAL;
  // a pointer may be null only when its tensor is empty
  if ((Nq > 0 && (!q || !out || !lse)) || (Nk > 0 && (!k_blk || !v_blk))) return RATTN_EINVAL;
  int rc = check_dtype_d(dtype, d);
  if (rc != RATTN_OK) return rc;
  if (causal != 0 && causal != 1) return RATTN_EINVAL;
  for (int i = 0; i < 2; ++i)
    if (q_seg_len[i] < 0 || k_seg_len[i] < 0) return RATTN_EINVAL;
  if (q_seg_len[0] + q_seg_len[1] != Nq || k_seg_len[0] + k_seg_len[1] != Nk)
    return RATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(k_blk, 16) || !aligned(v_blk, 16) || !aligned(out, 16) ||
      !aligned(lse, 4))
    return RATTN_EINVAL;
  const int64_t rows_max = std::max(std::max(q_rows, k_rows), Nq_out);
  if (!tensor_ok(B, rows_max, Hq > Hkv ? Hq : Hkv, d)) return RATTN_EUNSUPPORTED;
  if (Nq == 0) return RATTN_OK;

  const int br = tile_rows(dtype, d);
  Sched s;
  memset(&s, 0, sizeof s);
  s.mode = kVisitExplicit;
  s.W = 1;
  s.causal = causal;
  s.n_kruns = 0;
  if (k_seg_len[0] > 0) s.kruns[s.n_kruns++] = Run{k_off, k_seg_len[0], k_seg_start[0]};
  if (k_seg_len[1] > 0)
    s.kruns[s.n_kruns++] = Run{k_off + k_seg_len[0], k_seg_len[1], k_seg_start[1]};
  QSeg segs[2] = {QSeg{q_off, q_seg_len[0], q_seg_start[0], 0, 0},
                  QSeg{q_off + q_seg_len[0], q_seg_len[1], q_seg_start[1], 0, 0}};
  rc = finalize(s, segs, 2, br);
  if (rc != RATTN_OK) return rc;
  // rows are addressed in the full [B, q_rows] / [B, k_rows] row spaces; the
  // kernels write query row r to output row out_row_off + r
  FwdParams p = make_params(B, Hq, Hkv, q_rows, k_rows, resolve_scale(scale, d));
  p.out_rows = Nq_out;
  p.out_row_off = row_off - q_off;
  p.merge_out = merge;
  return dispatch(dtype, d, q, k_blk, v_blk, out, lse, true, p, s,
                  (int64_t)s.n_tiles * B * Hq, stream);
}

}  // namespace
}  // namespace rattn

extern "C" int rattn_fwd_step(const void* q, const void* k_blk, const void* v_blk,
                              float* out_part, float* lse_part, int B, int Hq, int Hkv,
                              int64_t q_rows, int64_t q_off, int64_t Nq, int64_t k_rows,
                              int64_t k_off, int64_t Nk, int d, int dtype, float scale,
                              int causal, const int64_t* q_seg_start, const int64_t* q_seg_len,
                              const int64_t* k_seg_start, const int64_t* k_seg_len,
                              void* stream) {
  return fwd_step_impl(q, k_blk, v_blk, out_part, lse_part, B, Hq, Hkv, q_rows, q_off, Nq,
                       k_rows, k_off, Nk, d, dtype, scale, causal, q_seg_start, q_seg_len,
                       k_seg_start, k_seg_len, Nq, 0, 0, stream);
}

extern "C" int rattn_fwd_step_merge(const void* q, const void* k_blk, const void* v_blk,
                                    float* out, float* lse, int B, int Hq, int Hkv,
                                    int64_t q_rows, int64_t q_off, int64_t Nq, int64_t k_rows,
                                    int64_t k_off, int64_t Nk, int d, int dtype, float scale,
                                    int causal, const int64_t* q_seg_start,
                                    const int64_t* q_seg_len, const int64_t* k_seg_start,
                                    const int64_t* k_seg_len, int64_t Nq_out, int64_t row_off,
                                    void* stream) {
  return fwd_step_impl(q, k_blk, v_blk, out, lse, B, Hq, Hkv, q_rows, q_off, Nq, k_rows, k_off,
                       Nk, d, dtype, scale, causal, q_seg_start, q_seg_len, k_seg_start,
                       k_seg_len, Nq_out, row_off, 1, stream);
}

extern "C" int rattn_merge(float* out, float* lse, const float* blk_out, const float* blk_lse,
                           int B, int H, int64_t Nq, int64_t Nb, int64_t row_off, int d,
                           void* stream) {
  if (B < 1 || H < 1 || Nq < 0 || Nb < 0 || row_off < 0) return RATTN_EINVAL;
  // a pointer may be null only when no row is merged
  if (Nb > 0 && (!out || !lse || !blk_out || !blk_lse)) return RATTN_EINVAL;
  if (!supported_d(d)) return RATTN_EUNSUPPORTED;
  if (row_off > Nq || Nb > Nq - row_off) return RATTN_EINVAL;
  if (!aligned(out, 16) || !aligned(blk_out, 16) || !aligned(lse, 4) || !aligned(blk_lse, 4))
    return RATTN_EINVAL;
  if (!tensor_ok(B, Nq, H, d)) return RATTN_EUNSUPPORTED;
  const int64_t threads = (int64_t)B * Nb * H * (d / 4);
  if ((threads + 255) / 256 > INT32_MAX) return RATTN_EUNSUPPORTED;
  hipError_t e = launch_merge(out, lse, blk_out, blk_lse, B, H, Nq, Nb, row_off, d,
                              (hipStream_t)stream);
  return e == hipSuccess ? RATTN_OK : RATTN_EHIP;
}

// ---- backward ------------------------------------------------------------

namespace rattn {
namespace {

BwdParams make_bwd_params(int B, int Hq, int Hkv, float scale) {
  BwdParams p;
  memset(&p, 0, sizeof p);
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.group = Hq / Hkv;
  p.scale = scale;
  p.c = (float)((double)scale * 1.4426950408889634074);  // scale * log2(e)
  return p;
}

// Keep the non-empty runs (a run of length 0 contributes nothing).
void set_runs(BwdRun* dst, int32_t* n, const BwdRun* src, int m) {
  *n = 0;
  for (int i = 0; i < m; ++i)
    if (src[i].len > 0) dst[(*n)++] = src[i];
}

int bwd_dispatch(int dtype, int d, const void* q, const void* k, const void* v,
                 const void* dout, const float* lse, const float* delta, void* dq, void* dk,
                 void* dv, const BwdParams& p, void* stream) {
  const int64_t g1 = bwd_q_tiles(p, 64) * p.B * p.Hq;
  const int64_t g2 = bwd_k_tiles(p, 64) * p.B * p.Hkv;
  if (g1 > INT32_MAX || g2 > INT32_MAX) return RATTN_EUNSUPPORTED;
  hipError_t e =
      (dtype != RATTN_F32 && d == 128)
          ? launch_bwd_mfma(dtype, q, k, v, dout, lse, delta, dq, dk, dv, p, (hipStream_t)stream)
          : launch_bwd_generic(dtype, d, q, k, v, dout, lse, delta, dq, dk, dv, p,
                               (hipStream_t)stream);
  return e == hipSuccess ? RATTN_OK : RATTN_EHIP;
}

}  // namespace
}  // namespace rattn

extern "C" int rattn_bwd_delta(const void* out, const void* dout, float* delta, int64_t rows,
                               int d, int dtype, void* stream) {
  using namespace rattn;
  if (rows < 0) return RATTN_EINVAL;
  int rc = check_dtype_d(dtype, d);
  if (rc != RATTN_OK) return rc;
  if (rows == 0) return RATTN_OK;
  if (!out || !dout || !delta) return RATTN_EINVAL;
  if (!aligned(out, 16) || !aligned(dout, 16) || !aligned(delta, 4)) return RATTN_EINVAL;
  if (!tensor_ok(1, rows, 1, d) || rows * d / 4 / 256 + 1 > INT32_MAX) return RATTN_EUNSUPPORTED;
  hipError_t e = launch_bwd_delta(dtype, d, out, dout, delta, rows, (hipStream_t)stream);
  return e == hipSuccess ? RATTN_OK : RATTN_EHIP;
}

extern "C" int rattn_bwd(const void* q, const void* k, const void* v, const void* out,
                         const float* lse, const void* dout, void* dq, void* dk, void* dv,
                         float* delta_ws, int B, int Hq, int Hkv, int64_t Nq, int64_t N, int d,
                         int dtype, float scale, int causal, int n_ring_steps, int zigzag,
                         int rank, void* stream) {
  using namespace rattn;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return RATTN_EINVAL;
  if (N < 0 || Nq < 0) return RATTN_EINVAL;
  if ((Nq > 0 && (!q || !out || !lse || !dout || !dq || !delta_ws)) ||
      (N > 0 && (!k || !v || !dk || !dv)))
    return RATTN_EINVAL;
  int rc = check_dtype_d(dtype, d);
  if (rc != RATTN_OK) return rc;
  if ((causal != 0 && causal != 1) || (zigzag != 0 && zigzag != 1)) return RATTN_EINVAL;
  if (n_ring_steps < 1) return RATTN_EINVAL;
  if (n_ring_steps > kMaxQSeg / 2) return RATTN_EUNSUPPORTED;
  const int64_t W = n_ring_steps;
  const int64_t parts = zigzag ? 2 * W : W;
  if (N % parts != 0) return RATTN_EINVAL;
  if (rank < -1 || rank >= W) return RATTN_EINVAL;
  if (rank == -1 ? Nq != N : Nq != N / W) return RATTN_EINVAL;
  const void* p16[] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* x : p16)
    if (!aligned(x, 16)) return RATTN_EINVAL;
  if (!aligned(lse, 4) || !aligned(delta_ws, 4)) return RATTN_EINVAL;
  if (!tensor_ok(B, N, Hq > Hkv ? Hq : Hkv, d)) return RATTN_EUNSUPPORTED;

  BwdParams p = make_bwd_params(B, Hq, Hkv, resolve_scale(scale, d));
  p.causal = causal;
  p.q_rows = Nq;
  p.k_rows = N;
  // query runs: the positions of the rows q holds (the gradient does not
  // depend on the order the ring visits the key/value blocks in)
  BwdRun qr[2] = {BwdRun{0, Nq, 0}, BwdRun{0, 0, 0}};
  if (rank >= 0 && !zigzag) {
    qr[0].pos0 = rank * (N / W);
  } else if (rank >= 0) {
    const int64_t c = N / (2 * W);
    qr[0] = BwdRun{0, c, rank * c};
    qr[1] = BwdRun{c, c, (2 * W - 1 - rank) * c};
  }
  set_runs(p.q, &p.nq, qr, 2);
  const BwdRun kr = BwdRun{0, N, 0};
  set_runs(p.k, &p.nk, &kr, 1);
  if (Nq == 0 && N == 0) return RATTN_OK;
  if (Nq > 0) {
    hipError_t e = launch_bwd_delta(dtype, d, out, dout, delta_ws, (int64_t)B * Nq * Hq,
                                    (hipStream_t)stream);
    if (e != hipSuccess) return RATTN_EHIP;
  }
  return bwd_dispatch(dtype, d, q, k, v, dout, lse, delta_ws, dq, dk, dv, p, stream);
}

extern "C" int rattn_bwd_varlen(const void* q, const void* k, const void* v, const void* out,
                                const float* lse, const void* dout, void* dq, void* dk,
                                void* dv, float* delta_ws, const int32_t* q_start,
                                const int32_t* q_len, const int32_t* k_start,
                                const int32_t* k_len, int n_seq, int64_t max_len_q,
                                int64_t max_len_k, int64_t Nq, int64_t Nk, int Hq, int Hkv,
                                int d, int dtype, float scale, int causal, void* stream) {
  using namespace rattn;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return RATTN_EINVAL;
  if (n_seq < 0 || max_len_q < 0 || max_len_k < 0 || Nq < 0 || Nk < 0) return RATTN_EINVAL;
  int rc = check_dtype_d(dtype, d);
  if (rc != RATTN_OK) return rc;
  if (causal != 0 && causal != 1) return RATTN_EINVAL;
  if (n_seq == 0 || (Nq == 0 && Nk == 0)) return RATTN_OK;
  if ((Nq > 0 && (!q || !out || !lse || !dout || !dq || !delta_ws)) ||
      (Nk > 0 && (!k || !v || !dk || !dv)) || !q_start || !q_len || !k_start || !k_len)
    return RATTN_EINVAL;
  const void* p16[] = {q, k, v, out, dout, dq, dk, dv};
  for (const void* x : p16)
    if (!aligned(x, 16)) return RATTN_EINVAL;
  if (!aligned(lse, 4) || !aligned(delta_ws, 4) || !aligned(q_start, 4) ||
      !aligned(q_len, 4) || !aligned(k_start, 4) || !aligned(k_len, 4))
    return RATTN_EINVAL;
  if (!tensor_ok(1, std::max(Nq, Nk), Hq > Hkv ? Hq : Hkv, d)) return RATTN_EUNSUPPORTED;
  if (max_len_q > INT32_MAX || max_len_k > INT32_MAX) return RATTN_EUNSUPPORTED;
  BwdParams p = make_bwd_params(1, Hq, Hkv, resolve_scale(scale, d));
  p.causal = causal;
  p.q_rows = Nq;
  p.k_rows = Nk;
  p.vl_q_start = q_start;
  p.vl_q_len = q_len;
  p.vl_k_start = k_start;
  p.vl_k_len = k_len;
  p.vl_nseq = n_seq;
  p.vl_max_q = max_len_q;
  p.vl_max_k = max_len_k;
  if (Nq > 0) {
    hipError_t e = launch_bwd_delta(dtype, d, out, dout, delta_ws, Nq * Hq, (hipStream_t)stream);
    if (e != hipSuccess) return RATTN_EHIP;
  }
  return bwd_dispatch(dtype, d, q, k, v, dout, lse, delta_ws, dq, dk, dv, p, stream);
}

extern "C" int rattn_bwd_step(const void* q, const void* k, const void* v, const void* dout,
                              const float* lse, const float* delta, float* dq_acc,
                              float* dk_acc, float* dv_acc, int B, int Hq, int Hkv,
                              int64_t q_rows, int64_t q_off, int64_t Nq, int64_t k_rows,
                              int64_t k_off, int64_t Nk, int d, int dtype, float scale,
                              int causal, const int64_t* q_seg_start, const int64_t* q_seg_len,
                              const int64_t* k_seg_start, const int64_t* k_seg_len,
                              void* stream) {
  using namespace rattn;
  if (!q_seg_start || !q_seg_len || !k_seg_start || !k_seg_len) return RATTN_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return RATTN_EINVAL;
  if (Nq < 0 || Nk < 0 || q_off < 0 || k_off < 0 || q_rows < 0 || k_rows < 0)
    return RATTN_EINVAL;
  if (q_off > q_rows || Nq > q_rows - q_off || k_off > k_rows || Nk > k_rows - k_off)
    return RATTN_EINVAL;
  if ((Nq > 0 && (!q || !dout || !lse || !delta || !dq_acc)) ||
      (Nk > 0 && (!k || !v || !dk_acc || !dv_acc)))
    return RATTN_EINVAL;
  int rc = check_dtype_d(dtype, d);
  if (rc != RATTN_OK) return rc;
  if (causal != 0 && causal != 1) return RATTN_EINVAL;
  for (int i = 0; i < 2; ++i)
    if (q_seg_len[i] < 0 || k_seg_len[i] < 0) return RATTN_EINVAL;
  if (q_seg_len[0] + q_seg_len[1] != Nq || k_seg_len[0] + k_seg_len[1] != Nk)
    return RATTN_EINVAL;
  const void* p16[] = {q, k, v, dout, dq_acc, dk_acc, dv_acc};
  for (const void* x : p16)
    if (!aligned(x, 16)) return RATTN_EINVAL;
  if (!aligned(lse, 4) || !aligned(delta, 4)) return RATTN_EINVAL;
  const int64_t rows_max = std::max(q_rows, k_rows);
  if (!tensor_ok(B, rows_max, Hq > Hkv ? Hq : Hkv, d)) return RATTN_EUNSUPPORTED;
  if (Nq == 0 || Nk == 0) return RATTN_OK;  // no pair: nothing to add

  BwdParams p = make_bwd_params(B, Hq, Hkv, resolve_scale(scale, d));
  p.causal = causal;
  p.accumulate = 1;
  p.q_rows = q_rows;
  p.q_off = q_off;
  p.k_rows = k_rows;
  p.k_off = k_off;
  const BwdRun qr[2] = {BwdRun{0, q_seg_len[0], q_seg_start[0]},
                        BwdRun{q_seg_len[0], q_seg_len[1], q_seg_start[1]}};
  const BwdRun kr[2] = {BwdRun{0, k_seg_len[0], k_seg_start[0]},
                        BwdRun{k_seg_len[0], k_seg_len[1], k_seg_start[1]}};
  set_runs(p.q, &p.nq, qr, 2);
  set_runs(p.k, &p.nk, kr, 2);
  return bwd_dispatch(dtype, d, q, k, v, dout, lse, delta, dq_acc, dk_acc, dv_acc, p, stream);
}

extern "C" const char* rattn_status_string(int status) {
  switch (status) {
    case RATTN_OK: return "ok";
    case RATTN_EINVAL: return "invalid argument";
    case RATTN_EUNSUPPORTED: return "unsupported configuration";
    case RATTN_EHIP: return "HIP error while enqueueing work";
    case RATTN_ESCRATCH: return "larger than the library's fixed scratch";
    default: return "unknown status";
  }
}
