// Internal interface between the C ABI and the prolog / epilog kernels.  Not
// part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// One launch: q_abs[m, h, :] (bf16, 512) = W_UK^T q_nope[m, h, :] with
// w_uk_t [H, 512, 128]; RoPE of q_pe; RMSNorm of c_kv, RoPE of k_pe and the new
// rows into the cache (m = b * q_len + j).
hipError_t launch_prolog(int32_t B, int32_t q_len, int32_t H, const uint16_t* q_nope, const uint16_t* w_uk_t,
                         uint16_t* q_abs, const uint16_t* q_pe_raw, const uint16_t* c_kv_raw, const uint16_t* norm_w,
                         float eps, const uint16_t* k_pe_raw, const float* cos_sin, int32_t max_pos,
                         const int32_t* seq_lens, const int32_t* block_table, int32_t bt_stride, int64_t num_pages,
                         int32_t page_log2, bool fp8, void* cache, uint8_t* scales, uint16_t* q_pe_out,
                         hipStream_t stream);
// o[m, h, :] (bf16, 128) = W_UV[h] attn_out[m, h, :] with w_uv [H, 128, 512].
hipError_t launch_up_project(int32_t M, int32_t H, const float* attn_out, const uint16_t* w_uv, uint16_t* o,
                             hipStream_t stream);
}  // namespace mla
