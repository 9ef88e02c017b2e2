// The steps next to the decode attention, for gfx950: the absorbed-query
// projection, RoPE, the new tokens' cache rows (prolog) and the value
// up-projection (epilog).
//
// The Huawei report ("DeepSeek V3/R1 inference deployment best practices on
// Ascend servers", section 6.1, the operators before MLA) absorbs the weights
// and fuses the decode prolog into one operator; the CloudMatrix384 digest
// (its MLA optimization paragraph) names RMSNorm, the projections and RoPE as
// its parts.  Here:
//  * head_gemm_kernel: Y[m, h, :] = W[h] X[m, h, :] per head (W[h] is N x K,
//    rows contiguous in K).  Absorption: X = q_nope (128), W = W_UK^T
//    (512 x 128), Y = q_nope_absorbed (bf16).  Up-projection: X = the
//    attention output (fp32, 512), W = W_UV (128 x 512), Y = o (bf16).
//    Computed as Y^T = W X^T on v_mfma_f32_16x16x32_bf16 so that a lane's
//    four results are four consecutive outputs of one row; the weights stream
//    from HBM once (the operation is bound by their bytes).
//  * rope_append_kernel: one workgroup per new token: RoPE of every head's
//    q_pe, RMSNorm of c_kv, RoPE of k_pe, and the row [c_kv | k_pe] (bf16)
//    written into the paged cache at the token's position, or quantized to
//    E4M3 with the row's E8M0 exponent for the FP8 cache.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "prolog.h"

namespace mla {
namespace {

#include "device_common.h"

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Round to bf16 (nearest even), as bits.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <typename XT>
__device__ __forceinline__ bf16x8 load_row8(const XT* p);

template <>
__device__ __forceinline__ bf16x8 load_row8<uint16_t>(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

template <>
__device__ __forceinline__ bf16x8 load_row8<float>(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  return bf16x8{(__bf16)a[0], (__bf16)a[1], (__bf16)a[2], (__bf16)a[3],
                (__bf16)b[0], (__bf16)b[1], (__bf16)b[2], (__bf16)b[3]};
}

// Workgroup: 4 waves; wave w covers outputs n in [nb + 16 NA w, +16 NA) of
// head blockIdx.y for rows m in [32 blockIdx.z, +32).  Lane l reads weight row
// n = nb + 16a + l%16 and input row m = mb + 16b + l%16, K slice 8(l/16) .. +7
// of each 32-wide K step, and holds outputs n = nb + 16a + 4(l/16) + 0..3 of
// row m = mb + 16b + l%16.
template <typename XT, int K, int N, int NA>
__global__ __launch_bounds__(256) void head_gemm_kernel(int32_t M, int32_t H, const XT* __restrict__ X,
                                                        const uint16_t* __restrict__ W, uint16_t* __restrict__ Y) {
  static_assert(K % 32 == 0 && N % (64 * NA) == 0, "tile sizes");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int h = blockIdx.y;
  const int nb = blockIdx.x * (64 * NA) + wave * (16 * NA);
  const int mb = blockIdx.z * 32;
  const uint16_t* wrow[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) wrow[a] = W + ((size_t)h * N + nb + 16 * a + l16) * K + 8 * grp;
  const XT* xrow[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int m = min(mb + 16 * b + l16, M - 1);  // rows past M load row M-1 and are not stored
    xrow[b] = X + ((size_t)m * H + h) * K + 8 * grp;
  }
  f32x4 acc[NA][2];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 32) {
    bf16x8 wa[NA], xb[2];
#pragma unroll
    for (int a = 0; a < NA; ++a) wa[a] = *reinterpret_cast<const bf16x8*>(wrow[a] + k0);
#pragma unroll
    for (int b = 0; b < 2; ++b) xb[b] = load_row8<XT>(xrow[b] + k0);
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wa[a], xb[b], acc[a][b], 0, 0, 0);
  }
  typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int m = mb + 16 * b + l16;
    if (m >= M) continue;
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      const u16x4 v = {f32_to_bf16(acc[a][b][0]), f32_to_bf16(acc[a][b][1]), f32_to_bf16(acc[a][b][2]),
                       f32_to_bf16(acc[a][b][3])};
      *reinterpret_cast<u16x4*>(Y + ((size_t)m * H + h) * N + nb + 16 * a + 4 * grp) = v;
    }
  }
}

// Sum / max over the 256 threads of the workgroup (every thread gets it).
__device__ __forceinline__ float block_sum(float x, float* red) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
__device__ __forceinline__ float block_max(float x, float* red) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// One workgroup (256 threads) per new token: blockIdx.x = b * q_len + j.
template <bool FP8>
__global__ __launch_bounds__(256) void rope_append_kernel(
    int32_t q_len, int32_t H, const uint16_t* __restrict__ q_pe_raw, const uint16_t* __restrict__ c_kv_raw,
    const uint16_t* __restrict__ norm_w, float eps, const uint16_t* __restrict__ k_pe_raw,
    const float* __restrict__ cos_sin, int32_t max_pos, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ block_table, int32_t bt_stride, int64_t num_pages, int32_t page_log2,
    void* __restrict__ cache, uint8_t* __restrict__ scales, uint16_t* __restrict__ q_pe_out) {
  __shared__ uint16_t row[576];
  __shared__ float red[4];
  const int tok = blockIdx.x;
  const int b = tok / q_len, j = tok - b * q_len;
  const int t = threadIdx.x;
  const int p = seq_lens[b] - q_len + j;  // position of this token
  const bool valid = p >= 0 && p < max_pos;
  const float* cs = cos_sin + (size_t)(valid ? p : 0) * 64;

  // q_pe of every head: pair i of head hh turns by the angle of pair i.
  for (int idx = t; idx < H * 32; idx += 256) {
    const int hh = idx >> 5, i = idx & 31;
    const size_t o = ((size_t)tok * H + hh) * 64 + 2 * i;
    const float x0 = bf16_to_f32(q_pe_raw[o]), x1 = bf16_to_f32(q_pe_raw[o + 1]);
    const float c = cs[i], s = cs[32 + i];
    float y0 = x0 * c - x1 * s, y1 = x0 * s + x1 * c;
    if (!valid) y0 = y1 = NAN;  // a position outside the table is loud
    q_pe_out[o] = f32_to_bf16(y0);
    q_pe_out[o + 1] = f32_to_bf16(y1);
  }

  // c_kv: RMSNorm, then the weight.  The values are first scaled by 2^-e
  // (amax = m 2^e, m in [0.5, 1)) so that the fp32 sum of squares neither
  // overflows nor underflows anywhere in the bf16 range; mean + eps and its
  // reciprocal square root are taken in double, and 2^e r (at most
  // sqrt(2048)) scales the scaled values.
  const float c0 = bf16_to_f32(c_kv_raw[(size_t)tok * 512 + 2 * t]);
  const float c1 = bf16_to_f32(c_kv_raw[(size_t)tok * 512 + 2 * t + 1]);
  const float am = block_max(fmaxf(fabsf(c0), fabsf(c1)), red);
  const int e = am > 0.f ? __builtin_amdgcn_frexp_expf(am) : 0;
  const float a0 = __builtin_ldexpf(c0, -e), a1 = __builtin_ldexpf(c1, -e);
  const float ss = block_sum(a0 * a0 + a1 * a1, red);
  const double r = 1.0 / __builtin_sqrt(__builtin_ldexp((double)ss * (1.0 / 512.0), 2 * e) + (double)eps);
  const float rs = (float)__builtin_ldexp(r, e);
  row[2 * t] = f32_to_bf16(a0 * rs * bf16_to_f32(norm_w[2 * t]));
  row[2 * t + 1] = f32_to_bf16(a1 * rs * bf16_to_f32(norm_w[2 * t + 1]));
  if (t < 32) {
    const float x0 = bf16_to_f32(k_pe_raw[(size_t)tok * 64 + 2 * t]);
    const float x1 = bf16_to_f32(k_pe_raw[(size_t)tok * 64 + 2 * t + 1]);
    const float c = cs[t], s = cs[32 + t];
    row[512 + 2 * t] = f32_to_bf16(x0 * c - x1 * s);
    row[513 + 2 * t] = f32_to_bf16(x0 * s + x1 * c);
  }
  __syncthreads();

  // The slot of the token (an id outside [0, num_pages) or a position outside
  // the table writes nothing).
  const bool in_table = valid && (p >> page_log2) < bt_stride;
  const int page = in_table ? block_table[(int64_t)b * bt_stride + (p >> page_log2)] : -1;
  const bool ok = in_table && (uint64_t)(int64_t)page < (uint64_t)num_pages;
  const int64_t slot = ((int64_t)page << page_log2) + (p & ((1 << page_log2) - 1));
  typedef short i16x2 __attribute__((ext_vector_type(2)));
  if constexpr (!FP8) {
    if (ok)
      for (int i = t; i < 288; i += 256)
        reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(cache) + slot * 576)[i] =
            reinterpret_cast<const uint32_t*>(row)[i];
  } else {
    // amax over the bf16 row (exact), the row's exponent f (smallest with
    // amax * 2^-f <= 448, limited to [-127, 127]), codes of row / 2^f.
    float am = 0.f;
    for (int i = t; i < 576; i += 256) am = fmaxf(am, fabsf(bf16_to_f32(row[i])));
    am = block_max(am, red);
    int f = 0;
    if (am > 0.f) {
      const int x = __builtin_amdgcn_frexp_expf(am);
      const float m = __builtin_amdgcn_frexp_mantf(am);
      f = min(max(x - 9 + (m > 0.875f ? 1 : 0), -127), 127);
    }
    const float sc = __builtin_ldexpf(1.f, f);
    if (ok) {
      uint8_t* dst = static_cast<uint8_t*>(cache) + slot * 576;
      for (int i = t; i < 288; i += 256) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(row)[i];
        i16x2 c = {0, 0};
        c = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(c, __builtin_bit_cast(bf16x2, w), sc, false);
        reinterpret_cast<uint16_t*>(dst)[i] = (uint16_t)__builtin_bit_cast(uint32_t, c);
      }
      if (t == 0) scales[slot] = (uint8_t)(127 + f);
    }
  }
}

}  // namespace

hipError_t launch_absorb(int32_t M, int32_t H, const uint16_t* q_nope, const uint16_t* w_uk_t, uint16_t* q_abs,
                         hipStream_t stream) {
  constexpr int NA = 2;
  hipLaunchKernelGGL((head_gemm_kernel<uint16_t, 128, 512, NA>), dim3(512 / (64 * NA), H, (M + 31) / 32), dim3(256),
                     0, stream, M, H, q_nope, w_uk_t, q_abs);
  return hipGetLastError();
}

hipError_t launch_up_project(int32_t M, int32_t H, const float* attn_out, const uint16_t* w_uv, uint16_t* o,
                             hipStream_t stream) {
  constexpr int NA = 1;
  hipLaunchKernelGGL((head_gemm_kernel<float, 512, 128, NA>), dim3(128 / (64 * NA), H, (M + 31) / 32), dim3(256), 0,
                     stream, M, H, attn_out, w_uv, o);
  return hipGetLastError();
}

hipError_t launch_rope_append(int32_t B, int32_t q_len, int32_t H, const uint16_t* q_pe_raw, const uint16_t* c_kv_raw,
                              const uint16_t* norm_w, float eps, const uint16_t* k_pe_raw, const float* cos_sin,
                              int32_t max_pos, const int32_t* seq_lens, const int32_t* block_table, int32_t bt_stride,
                              int64_t num_pages, int32_t page_log2, bool fp8, void* cache, uint8_t* scales,
                              uint16_t* q_pe_out, hipStream_t stream) {
  if (fp8)
    hipLaunchKernelGGL(rope_append_kernel<true>, dim3(B * q_len), dim3(256), 0, stream, q_len, H, q_pe_raw, c_kv_raw,
                       norm_w, eps, k_pe_raw, cos_sin, max_pos, seq_lens, block_table, bt_stride, num_pages, page_log2,
                       cache, scales, q_pe_out);
  else
    hipLaunchKernelGGL(rope_append_kernel<false>, dim3(B * q_len), dim3(256), 0, stream, q_len, H, q_pe_raw, c_kv_raw,
                       norm_w, eps, k_pe_raw, cos_sin, max_pos, seq_lens, block_table, bt_stride, num_pages, page_log2,
                       cache, scales, q_pe_out);
  return hipGetLastError();
}

}  // namespace mla
