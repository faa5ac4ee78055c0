// launch.h -- host-side entry points of the kernels (HIP path only).
#pragma once
#include <hip/hip_runtime.h>

#include "kcommon.h"

namespace rattn {

// Query rows per tile of each forward kernel; the schedule is built for it.
constexpr int kGenericBr = 64;
constexpr int kMfmaBr = 128;     // fwd_mfma (16-bit, d = 16)
constexpr int kMfma128Br = 256;  // fwd_mfma128 (16-bit, d = 32, 64, 128)
constexpr int kShortBr = 32;     // fwd_short (16-bit, d = 32, 64, 128, few query rows)

hipError_t launch_fwd_generic(int dtype, int d, const void* q, const void* k, const void* v,
                              void* out, float* lse, bool out_f32, const FwdParams& p,
                              const Sched& s, hipStream_t stream);

// Work-item queues of a queued forward launch: one 32-bit counter per XCD.
constexpr int kFwdQueues = 8;

// 16-bit inputs, d = 32, 64 or 128 (direct-to-LDS tiles, transposing V reads).
// queues: nullptr, or kFwdQueues counters in device memory that no other
// launch uses meanwhile; with them, a d = 128 grid larger than twice what the
// chip holds at once runs as a persistent grid fed from per-XCD queues (the
// counters are zeroed on `stream` first).
hipError_t launch_fwd_mfma128(int dtype, int d, const void* q, const void* k, const void* v,
                              void* out, float* lse, bool out_f32, const FwdParams& p,
                              const Sched& s, uint32_t* queues, hipStream_t stream);

// 16-bit inputs, d in {16, 32, 64, 128} (d = 32, 64 and 128 are routed to
// launch_fwd_mfma128, with `queues`; d = 16 ignores them).
hipError_t launch_fwd_mfma(int dtype, int d, const void* q, const void* k, const void* v,
                           void* out, float* lse, bool out_f32, const FwdParams& p,
                           const Sched& s, uint32_t* queues, hipStream_t stream);

// 16-bit inputs, d = 32, 64 or 128, schedule built for kShortBr-row query
// tiles: one workgroup per tile, whose 8 waves split the tile's key tiles and
// merge their partial results in LDS (for launches with few query rows).
hipError_t launch_fwd_short(int dtype, int d, const void* q, const void* k, const void* v,
                            void* out, float* lse, bool out_f32, const FwdParams& p,
                            const Sched& s, hipStream_t stream);

hipError_t launch_merge(float* out, float* lse, const float* blk_out, const float* blk_lse,
                        int B, int H, int64_t Nq, int64_t Nb, int64_t row_off, int d,
                        hipStream_t stream);

// n-way log-sum-exp merge of split-KV partials (rows = B*Nq*H; split s at
// ws_out + s*rows*d, ws_lse + s*rows) into out (input type) and lse.
hipError_t launch_split_reduce(int dtype, int d, void* out, float* lse, const float* ws_out,
                               const float* ws_lse, int n_splits, int64_t rows,
                               hipStream_t stream);

}  // namespace rattn
