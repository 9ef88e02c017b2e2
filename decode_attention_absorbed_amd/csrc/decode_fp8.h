// Internal interface between the C ABI and the FP8 decode kernel.  Not part
// of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan_internal.h"

namespace mla {

constexpr int32_t kFp8TileTokens = 64;  // keys per LDS tile of the FP8 kernel
constexpr int32_t kFp8Waves = 4;        // 128 query rows per workgroup

// Launches the FP8 decode kernel for plan `d` (made for 64-key tiles) on
// `stream`.  `sched` is the device copy of the plan's schedule; the offsets
// locate its parts.  Returns the launch status.
hipError_t launch_decode_fp8(const PlanData& d, const char* sched, size_t off_segs, size_t off_wgs, size_t off_lens,
                             const void* q_nope, const void* q_pe, const void* cache, const void* kv_scale,
                             int64_t num_pages, const int32_t* block_table, int32_t bt_stride,
                             const int32_t* seq_lens, float scale_log2, float* out, float* lse, uint16_t* ws_o,
                             float* ws_lse, float* ws_f, hipStream_t stream);

}  // namespace mla
