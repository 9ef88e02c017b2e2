// The steps next to the decode attention, for gfx950: the absorbed-query
// projection, RoPE, the new tokens' cache rows (prolog), the value
// up-projection and the output projection (epilog).
//
// The Huawei report ("DeepSeek V3/R1 inference deployment best practices on
// Ascend servers", section 6.1, the operators before MLA) absorbs the weights
// and fuses the decode prolog into one operator; the CloudMatrix384 digest
// (its MLA optimization paragraph) names RMSNorm, the projections and RoPE as
// its parts; the report's decode flow (section 3.2.1) closes MLA with the
// output projection.  Here:
//  * proj_kernel: Y[m, h, :] = W[h] X[m, h, :] per head (W[h] is N x K, rows
//    contiguous in K), bound by the weights' bytes.  Absorption: X = q_nope
//    (128), W = W_UK^T (512 x 128), Y = q_nope_absorbed (bf16).
//    Up-projection: X = the attention output (fp32, 512), W = W_UV
//    (128 x 512), Y = o (bf16).
//  * oproj_kernel + sum_kernel: the output projection Y = X W_O^T (X the
//    up-projected heads concatenated, [M, K]; W_O [N, K]), split over K into
//    S slices whose fp32 partials a second launch sums into bf16.
//  * the prolog is one launch: besides the absorption's workgroups, one more
//    workgroup per head and chunk of query rows does the per-token part --
//    RoPE of that head's q_pe, and for the chunk's tokens h, h + H, ... the
//    RMSNorm of c_kv, RoPE of k_pe and the row [c_kv | k_pe] written into the
//    paged cache at the token's position (bf16, or E4M3 codes with the row's
//    E8M0 exponent for the FP8 cache).  These workgroups load no weights, so
//    their short dependent loads run beside the weight stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "abi_common.h"
#include "mla_decode.h"

namespace mla {
namespace {

#include "device_common.h"

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Round to bf16 (nearest even), as bits.
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Arguments of the prolog's per-token part (RoPE, RMSNorm, cache append).
struct PrologArgs {
  int32_t q_len;
  const uint16_t* q_pe_raw;
  const uint16_t* c_kv_raw;
  const uint16_t* norm_w;
  float eps;
  const uint16_t* k_pe_raw;
  const float* cos_sin;
  int32_t max_pos;
  const int32_t* seq_lens;
  const int32_t* block_table;
  int32_t bt_stride;
  int64_t num_pages;
  int32_t page_log2;
  void* cache;
  uint8_t* scales;
  uint16_t* q_pe_out;
};

// Position of query row m (= b * q_len + j): L_b - q_len + j.
__device__ __forceinline__ int row_position(const PrologArgs& a, int m) {
  const int b = m / a.q_len;
  return a.seq_lens[b] - a.q_len + (m - b * a.q_len);
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

// RoPE of q_pe for head h, query rows [m0, m0 + rows): pair i turns by the
// angle of pair i at the row's position; 4 pairs (16 bytes) per thread step.
__device__ void rope_query(const PrologArgs& a, int H, int h, int m0, int rows) {
  for (int v = threadIdx.x; v < rows * 8; v += 256) {
    const int m = m0 + (v >> 3), c = v & 7;
    const int p = row_position(a, m);
    const bool valid = p >= 0 && p < a.max_pos;
    const size_t o = ((size_t)m * H + h) * 64 + 8 * c;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(a.q_pe_raw + o);
    const float* cs = a.cos_sin + (size_t)(valid ? p : 0) * 64;
    const f32x4 cv = *reinterpret_cast<const f32x4*>(cs + 4 * c);
    const f32x4 sv = *reinterpret_cast<const f32x4*>(cs + 32 + 4 * c);
    bf16x8 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = (float)x[2 * i], x1 = (float)x[2 * i + 1];
      float y0 = x0 * cv[i] - x1 * sv[i], y1 = x0 * sv[i] + x1 * cv[i];
      if (!valid) y0 = y1 = NAN;  // a position outside the table is loud
      y[2 * i] = (__bf16)y0;
      y[2 * i + 1] = (__bf16)y1;
    }
    *reinterpret_cast<bf16x8*>(a.q_pe_out + o) = y;
  }
}

// The cache row of new token m: [RMSNorm(c_kv) * w | RoPE(k_pe)] in bf16,
// written at the token's slot as it is (bf16 cache) or as E4M3 codes of
// row * 2^-f with the E8M0 byte 127 + f (FP8 cache).  Every thread of the
// workgroup takes part (block reductions); `row` holds 576 bf16 in LDS.
template <bool FP8>
__device__ void append_token(const PrologArgs& a, int m, uint16_t* row, float* red) {
  const int t = threadIdx.x;
  const int p = row_position(a, m);
  const bool valid = p >= 0 && p < a.max_pos;
  const float* cs = a.cos_sin + (size_t)(valid ? p : 0) * 64;

  // c_kv: RMSNorm, then the weight.  The values are first scaled by 2^-e
  // (amax = m 2^e, m in [0.5, 1)) so that the fp32 sum of squares neither
  // overflows nor underflows anywhere in the bf16 range; mean + eps and its
  // reciprocal square root are taken in double, and 2^e r (at most
  // sqrt(2048)) scales the scaled values.
  const float c0 = bf16_to_f32(a.c_kv_raw[(size_t)m * 512 + 2 * t]);
  const float c1 = bf16_to_f32(a.c_kv_raw[(size_t)m * 512 + 2 * t + 1]);
  const float am = block_max(fmaxf(fabsf(c0), fabsf(c1)), red);
  const int e = am > 0.f ? __builtin_amdgcn_frexp_expf(am) : 0;
  const float a0 = __builtin_ldexpf(c0, -e), a1 = __builtin_ldexpf(c1, -e);
  const float ss = block_sum(a0 * a0 + a1 * a1, red);
  const double r = 1.0 / __builtin_sqrt(__builtin_ldexp((double)ss * (1.0 / 512.0), 2 * e) + (double)a.eps);
  const float rs = (float)__builtin_ldexp(r, e);
  row[2 * t] = f32_to_bf16(a0 * rs * bf16_to_f32(a.norm_w[2 * t]));
  row[2 * t + 1] = f32_to_bf16(a1 * rs * bf16_to_f32(a.norm_w[2 * t + 1]));
  if (t < 32) {
    const float x0 = bf16_to_f32(a.k_pe_raw[(size_t)m * 64 + 2 * t]);
    const float x1 = bf16_to_f32(a.k_pe_raw[(size_t)m * 64 + 2 * t + 1]);
    const float c = cs[t], s = cs[32 + t];
    row[512 + 2 * t] = f32_to_bf16(x0 * c - x1 * s);
    row[513 + 2 * t] = f32_to_bf16(x0 * s + x1 * c);
  }
  __syncthreads();

  // The slot of the token (an id outside [0, num_pages) or a position outside
  // the table writes nothing).
  const int b = m / a.q_len;
  const bool in_table = valid && (p >> a.page_log2) < a.bt_stride;
  const int page = in_table ? a.block_table[(int64_t)b * a.bt_stride + (p >> a.page_log2)] : -1;
  const bool ok = in_table && (uint64_t)(int64_t)page < (uint64_t)a.num_pages;
  const int64_t slot = ((int64_t)page << a.page_log2) + (p & ((1 << a.page_log2) - 1));
  typedef short i16x2 __attribute__((ext_vector_type(2)));
  if constexpr (!FP8) {
    if (ok)
      for (int i = t; i < 288; i += 256)
        reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.cache) + slot * 576)[i] =
            reinterpret_cast<const uint32_t*>(row)[i];
  } else {
    // amax over the bf16 row (exact), the row's exponent f (smallest with
    // amax * 2^-f <= 448, limited to [-127, 127]), codes of row / 2^f.
    float amx = 0.f;
    for (int i = t; i < 576; i += 256) amx = fmaxf(amx, fabsf(bf16_to_f32(row[i])));
    amx = block_max(amx, red);
    int f = 0;
    if (amx > 0.f) {
      const int x = __builtin_amdgcn_frexp_expf(amx);
      const float mt = __builtin_amdgcn_frexp_mantf(amx);
      f = min(max(x - 9 + (mt > 0.875f ? 1 : 0), -127), 127);
    }
    const float sc = __builtin_ldexpf(1.f, f);
    if (ok) {
      uint8_t* dst = static_cast<uint8_t*>(a.cache) + slot * 576;
      for (int i = t; i < 288; i += 256) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(row)[i];
        i16x2 c = {0, 0};
        c = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(c, __builtin_bit_cast(bf16x2, w), sc, false);
        reinterpret_cast<uint16_t*>(dst)[i] = (uint16_t)__builtin_bit_cast(uint32_t, c);
      }
      if (t == 0) a.scales[slot] = (uint8_t)(127 + f);
    }
  }
  __syncthreads();  // `row` and `red` are reused by the next token
}

// Per-head weight-streaming projection Y[m, h, :] = W[h] X[m, h, :] for the
// query rows m in [MC z, MC z + MC) (z = blockIdx.z), computed as
// Y^T = W X^T on v_mfma_f32_16x16x32_bf16.
//
// The weights are the bytes that matter (M is small): every lane issues the
// loads of all its weight fragments at once -- wave w of workgroup x covers
// rows n in [64 NA x + 16 NA w, +16 NA), lane l row n0 + 16a + l%16 and K
// slice 8(l/16) of each 32-wide step -- and keeps them in registers.  The
// chunk of X (its loads issued before the weights', so waiting for it does
// not wait for them) goes to LDS as bf16, row stride K + 8, which every wave
// then reads as the B operand: lane l reads row l%16 of a 16-row block, K
// slice 8(l/16).  A lane's four results are outputs n0 + 16a + 4(l/16) + 0..3
// of row m = 16-row block + l%16, stored as 8 bytes.
//
// With PROLOG >= 0 the workgroups x = N / (64 NA) do the per-token part of the
// prolog for the chunk instead: RoPE of head h's q_pe, and the cache rows of
// tokens m0 + h, m0 + h + H, ... (PROLOG = 1: FP8 cache).
template <typename XT, int K, int N, int NA, int MC, int PROLOG>
__global__ __launch_bounds__(256) void proj_kernel(int32_t M, int32_t H, const XT* __restrict__ X,
                                                   const uint16_t* __restrict__ W, uint16_t* __restrict__ Y,
                                                   PrologArgs pa) {
  constexpr int LDK = K + 8;
  constexpr int KS = K / 32;
  constexpr int XN = 16 / (int)sizeof(XT);  // elements per 16-byte load
  constexpr int VPR = K / XN;  // 16-byte vectors per row of X
  constexpr int PER = MC * VPR / 256;
  static_assert(K % 32 == 0 && N % (64 * NA) == 0 && MC % 16 == 0 && (MC * VPR) % 256 == 0, "tile sizes");
  static_assert(MC * LDK >= 576, "the per-token part reuses the X buffer for one cache row");
  __shared__ __align__(16) uint16_t xs[MC * LDK];
  __shared__ float red[4];

  const int t = threadIdx.x;
  const int h = blockIdx.y, m0 = blockIdx.z * MC;
  const int rows = min(MC, M - m0);
  if constexpr (PROLOG >= 0) {
    if (blockIdx.x == N / (64 * NA)) {
      rope_query(pa, H, h, m0, rows);
      for (int m = m0 + h; m < m0 + rows; m += H) append_token<PROLOG == 1>(pa, m, xs, red);
      return;
    }
  }
  const int lane = t & 63, wave = t >> 6;
  const int l16 = lane & 15, grp = lane >> 4;

  // Every load of the workgroup is issued up front, as inline asm with
  // explicit waits (the compiler would otherwise sink the weight loads below
  // the staging): the chunk of X first -- rows past the chunk's end load (and
  // stage) its last row again, so no load is conditional -- then all weight
  // fragments.  Loads complete in order, so once at most NA * KS are
  // outstanding X has arrived and can be staged while the weights stream.
  bf16x8 xr[PER];  // 16 raw bytes each: 8 bf16 or 4 fp32
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int v = t + 256 * i, r = min(v / VPR, rows - 1);
    xr[i] = load16(X + ((size_t)(m0 + r) * H + h) * K + (v % VPR) * XN);
  }
  const int nb = blockIdx.x * (64 * NA) + wave * (16 * NA);
  bf16x8 w[NA][KS];
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const uint16_t* wp = W + ((size_t)h * N + nb + 16 * a + l16) * K + 8 * grp;
#pragma unroll
    for (int s = 0; s < KS; ++s) w[a][s] = load16(wp + 32 * s);
  }
  wait_vmem<NA * KS>();
  // The compiler sees the asm loads' results as ready at once: tie each one to
  // a volatile asm placed after the wait, so no use moves above it.
#pragma unroll
  for (int i = 0; i < PER; ++i) asm volatile("" : "+v"(xr[i]));
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int v = t + 256 * i;
    uint16_t* dst = xs + (v / VPR) * LDK + (v % VPR) * XN;
    if constexpr (XN == 8) {
      *reinterpret_cast<bf16x8*>(dst) = xr[i];
    } else {
      typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
      const f32x4 x = __builtin_bit_cast(f32x4, xr[i]);
      *reinterpret_cast<u16x4*>(dst) = u16x4{f32_to_bf16(x[0]), f32_to_bf16(x[1]), f32_to_bf16(x[2]), f32_to_bf16(x[3])};
    }
  }
  __syncthreads();
  wait_vmem<0>();
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" : "+v"(w[a][s]));

  typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
  for (int mb = 0; mb < rows; mb += 16) {
    f32x4 acc[NA];
#pragma unroll
    for (int a = 0; a < NA; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(xs + (mb + l16) * LDK + 32 * s + 8 * grp);
#pragma unroll
      for (int a = 0; a < NA; ++a) acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[a][s], b, acc[a], 0, 0, 0);
    }
    const int m = m0 + mb + l16;
    if (m < M) {
#pragma unroll
      for (int a = 0; a < NA; ++a)
        *reinterpret_cast<u16x4*>(Y + ((size_t)m * H + h) * N + nb + 16 * a + 4 * grp) =
            u16x4{f32_to_bf16(acc[a][0]), f32_to_bf16(acc[a][1]), f32_to_bf16(acc[a][2]), f32_to_bf16(acc[a][3])};
    }
  }
}


// Output projection, split over K: slice s = blockIdx.y covers K columns
// [s * kslice, +kslice); P[s][m][n] (fp32) = sum over the slice of
// X[m, k] W[n, k].  Wave w of workgroup x owns output rows n in
// [64 NA x + 16 NA w, +16 NA) (fragment a: lane l reads row 16a + l%16, K
// slice 8(l/16) of each 32-wide step) and query rows [MC z, +MC).  The slice
// is walked in KC-column chunks: the chunk of X (its loads first) and the
// wave's NA * KC / 32 weight fragments are issued together as asm loads, X is
// staged in LDS as the MFMA's B operand, and the 16-row blocks of X
// accumulate in registers.  Several workgroups per CU keep the weight stream
// going while one of them computes.
template <int MC, int KC, int NA>
__global__ __launch_bounds__(256) void oproj_kernel(int32_t M, int32_t N, int32_t K, int32_t kslice,
                                                    const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                                                    float* __restrict__ P) {
  constexpr int LDK = KC + 8, KS = KC / 32;
  constexpr int VPR = KC / 8;           // 16-byte vectors per row of a chunk
  constexpr int PER = MC * VPR / 256;   // ... per thread
  constexpr int MB = MC / 16;           // 16-row blocks
  __shared__ __align__(16) uint16_t xs[MC * LDK];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l16 = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * (64 * NA) + wave * (16 * NA);
  const int s = blockIdx.y, m0 = blockIdx.z * MC;
  const int rows = min(MC, M - m0);
  f32x4 acc[NA][MB];
#pragma unroll
  for (int a = 0; a < NA; ++a)
#pragma unroll
    for (int b = 0; b < MB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint16_t* wp = W + (size_t)(n0 + l16) * K + 8 * grp;
  // Workgroups of neighbouring row blocks walk their slice's chunks from
  // different starting points: all workgroups run at once, and in lockstep
  // they would read the same column offset of rows 2K bytes apart, which
  // lands on few HBM channels (measured: 4.0 vs 6.1 TB/s for a 256 MB read).
  const int nch = kslice / KC;
  for (int c = 0; c < nch; ++c) {
    const int kc = s * kslice + ((c + (int)blockIdx.x) % nch) * KC;
    bf16x8 xr[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = t + 256 * i, r = min(v / VPR, rows - 1);  // rows past the end repeat the last one
      xr[i] = load16(X + (size_t)(m0 + r) * K + kc + 8 * (v % VPR));
    }
    bf16x8 w[NA][KS];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int j = 0; j < KS; ++j) w[a][j] = load16(wp + (size_t)16 * a * K + kc + 32 * j);
    wait_vmem<NA * KS>();  // X has arrived (loads complete in order); the weights stream on
#pragma unroll
    for (int i = 0; i < PER; ++i) asm volatile("" : "+v"(xr[i]));
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = t + 256 * i;
      *reinterpret_cast<bf16x8*>(xs + (v / VPR) * LDK + 8 * (v % VPR)) = xr[i];
    }
    __syncthreads();
    wait_vmem<0>();
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
      for (int j = 0; j < KS; ++j) asm volatile("" : "+v"(w[a][j]));
#pragma unroll
    for (int b = 0; b < MB; ++b) {
      if (16 * b < rows) {
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(xs + (16 * b + l16) * LDK + 32 * j + 8 * grp);
#pragma unroll
          for (int a = 0; a < NA; ++a)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[a][j], x, acc[a][b], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // the next chunk overwrites xs
  }
  // lane: outputs n0 + 16a + 4(l/16) + 0..3 of row 16b + l%16
#pragma unroll
  for (int b = 0; b < MB; ++b) {
    const int m = m0 + 16 * b + l16;
    if (m < M)
#pragma unroll
      for (int a = 0; a < NA; ++a)
        *reinterpret_cast<f32x4*>(P + ((size_t)s * M + m) * N + n0 + 16 * a + 4 * grp) = acc[a][b];
  }
}

// Y[m, n] (bf16) = sum over the S slices of P[s][m][n]; 4 outputs per thread.
__global__ __launch_bounds__(256) void sum_kernel(int64_t MN4, int32_t S, int64_t MN, const float* __restrict__ P,
                                                  uint16_t* __restrict__ Y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= MN4) return;
  f32x4 a = *reinterpret_cast<const f32x4*>(P + 4 * i);
  for (int s = 1; s < S; ++s) {
    const f32x4 b = *reinterpret_cast<const f32x4*>(P + (size_t)s * MN + 4 * i);
    a[0] += b[0];
    a[1] += b[1];
    a[2] += b[2];
    a[3] += b[3];
  }
  typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<u16x4*>(Y + 4 * i) = u16x4{f32_to_bf16(a[0]), f32_to_bf16(a[1]), f32_to_bf16(a[2]), f32_to_bf16(a[3])};
}

}  // namespace

constexpr int kAbsorbRows = 128;  // query rows per workgroup chunk of the absorption

hipError_t launch_prolog(int32_t B, int32_t q_len, int32_t H, const uint16_t* q_nope, const uint16_t* w_uk_t,
                         uint16_t* q_abs, const uint16_t* q_pe_raw, const uint16_t* c_kv_raw, const uint16_t* norm_w,
                         float eps, const uint16_t* k_pe_raw, const float* cos_sin, int32_t max_pos,
                         const int32_t* seq_lens, const int32_t* block_table, int32_t bt_stride, int64_t num_pages,
                         int32_t page_log2, bool fp8, void* cache, uint8_t* scales, uint16_t* q_pe_out,
                         hipStream_t stream) {
  const int32_t M = B * q_len;
  const PrologArgs pa{q_len,   q_pe_raw,    c_kv_raw,  norm_w,    eps,       k_pe_raw, cos_sin, max_pos,
                      seq_lens, block_table, bt_stride, num_pages, page_log2, cache,    scales,  q_pe_out};
  constexpr int NA = 2;
  // 32-row chunks up to 32 rows: X's staging loads scale with the chunk
  const int mc = M <= 32 ? 32 : kAbsorbRows;
  const dim3 grid(512 / (64 * NA) + 1, H, (M + mc - 1) / mc);
  if (mc == 32 && fp8)
    hipLaunchKernelGGL((proj_kernel<uint16_t, 128, 512, NA, 32, 1>), grid, dim3(256), 0, stream, M, H, q_nope, w_uk_t,
                       q_abs, pa);
  else if (mc == 32)
    hipLaunchKernelGGL((proj_kernel<uint16_t, 128, 512, NA, 32, 0>), grid, dim3(256), 0, stream, M, H, q_nope, w_uk_t,
                       q_abs, pa);
  else if (fp8)
    hipLaunchKernelGGL((proj_kernel<uint16_t, 128, 512, NA, kAbsorbRows, 1>), grid, dim3(256), 0, stream, M, H,
                       q_nope, w_uk_t, q_abs, pa);
  else
    hipLaunchKernelGGL((proj_kernel<uint16_t, 128, 512, NA, kAbsorbRows, 0>), grid, dim3(256), 0, stream, M, H,
                       q_nope, w_uk_t, q_abs, pa);
  return hipGetLastError();
}

hipError_t launch_up_project(int32_t M, int32_t H, const float* attn_out, const uint16_t* w_uv, uint16_t* o,
                             hipStream_t stream) {
  const PrologArgs none{};
  if (M <= 32) {
    // two workgroups per head (64 outputs each), all rows in one 32-row chunk
    hipLaunchKernelGGL((proj_kernel<float, 512, 128, 1, 32, -1>), dim3(2, H, 1), dim3(256), 0, stream, M, H, attn_out,
                       w_uv, o, none);
  } else if (M <= 64) {
    // two workgroups per head (64 outputs each), all rows in one chunk
    hipLaunchKernelGGL((proj_kernel<float, 512, 128, 1, 64, -1>), dim3(2, H, 1), dim3(256), 0, stream, M, H, attn_out,
                       w_uv, o, none);
  } else {
    // one workgroup per head and 32-row chunk: the fp32 input (the larger
    // operand at these sizes) is read once
    hipLaunchKernelGGL((proj_kernel<float, 512, 128, 2, 32, -1>), dim3(1, H, (M + 31) / 32), dim3(256), 0, stream, M,
                       H, attn_out, w_uv, o, none);
  }
  return hipGetLastError();
}

// Shape of the output projection's launch, from interleaved A/B runs at
// 7168 x 16384: query rows per chunk 32, 64 or 128 (the smallest that holds
// every row: X's staging loads scale with it); up to 64 rows, 128 output rows
// per workgroup when N allows (X's chunks, re-read by every workgroup, then
// serve twice the rows) with 8 slices of K, else 64 with 4 slices, and
// 128-column chunks; above 64 rows, 64 output rows, 256-column chunks and 4
// slices.  Narrower chunks spread the concurrently
// read column offsets over more HBM channels.  S is halved until it divides K
// into whole chunks.
void oproj_split(int32_t M, int32_t N, int32_t K, int* mc, int* S, int* kc, int* na) {
  *mc = M > 64 ? 128 : M > 32 ? 64 : 32;
  *kc = *mc <= 64 ? 128 : 256;
  *na = *mc <= 64 && N % 128 == 0 ? 2 : 1;
  int s = *na == 2 ? 8 : 4;
  while (s > 1 && (K / *kc) % s != 0) s >>= 1;
  *S = s;
}

size_t oproj_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  int mc, S, kc, na;
  oproj_split(M, N, K, &mc, &S, &kc, &na);
  return (size_t)S * M * N * sizeof(float);
}

hipError_t launch_o_project(int32_t M, int32_t N, int32_t K, const uint16_t* x, const uint16_t* w, uint16_t* y,
                            float* partials, hipStream_t stream) {
  int mc, S, kc, na;
  oproj_split(M, N, K, &mc, &S, &kc, &na);
  const dim3 grid(N / (64 * na), S, (M + mc - 1) / mc);
  if (mc == 32 && na == 2)
    hipLaunchKernelGGL((oproj_kernel<32, 128, 2>), grid, dim3(256), 0, stream, M, N, K, K / S, x, w, partials);
  else if (mc == 32)
    hipLaunchKernelGGL((oproj_kernel<32, 128, 1>), grid, dim3(256), 0, stream, M, N, K, K / S, x, w, partials);
  else if (mc == 64 && na == 2)
    hipLaunchKernelGGL((oproj_kernel<64, 128, 2>), grid, dim3(256), 0, stream, M, N, K, K / S, x, w, partials);
  else if (mc == 64)
    hipLaunchKernelGGL((oproj_kernel<64, 128, 1>), grid, dim3(256), 0, stream, M, N, K, K / S, x, w, partials);
  else
    hipLaunchKernelGGL((oproj_kernel<128, 256, 1>), grid, dim3(256), 0, stream, M, N, K, K / S, x, w, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t mn4 = (int64_t)M * N / 4;
  hipLaunchKernelGGL(sum_kernel, dim3((unsigned)((mn4 + 255) / 256)), dim3(256), 0, stream, mn4, S, (int64_t)M * N,
                     partials, y);
  return hipGetLastError();
}

}  // namespace mla

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------

mla_status mla_prolog(int32_t batch, int32_t q_len, int32_t num_heads, const void* q_nope128, const void* q_pe_raw,
                      const void* w_uk_t, const void* c_kv_raw, const void* kv_norm_w, float rms_eps,
                      const void* k_pe_raw, const float* rope_cos_sin, int32_t max_pos, const int32_t* seq_lens,
                      const int32_t* block_table, int32_t bt_stride, int64_t num_pages, int32_t page_size,
                      int32_t kv_format, void* kv_cache, void* kv_scales, void* q_nope_absorbed, void* q_pe,
                      void* stream) {
  if (!q_nope128 || !q_pe_raw || !w_uk_t || !c_kv_raw || !kv_norm_w || !k_pe_raw || !rope_cos_sin || !seq_lens ||
      !block_table || !kv_cache || !q_nope_absorbed || !q_pe)
    return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (kv_format != MLA_KV_BF16 && kv_format != MLA_KV_FP8)
    return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT, "kv_format must be MLA_KV_BF16 or MLA_KV_FP8");
  if (kv_format == MLA_KV_FP8 && !kv_scales) return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT, "kv_scales is NULL");
  if (batch < 1 || q_len < 1 || q_len > 8 || num_heads < 1 || num_heads > 128 || (int64_t)batch * q_len > (1 << 21))
    return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT,
                "batch >= 1, q_len in [1, 8], batch * q_len <= 2^21 and num_heads in [1, 128] are required");
  if (page_size < 16 || page_size > 4096 || (page_size & (page_size - 1)) != 0)
    return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT, "page_size must be a power of two in [16, 4096]");
  if (max_pos < 1 || bt_stride < 1 || num_pages <= 0)
    return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT, "max_pos, bt_stride and num_pages must be >= 1");
  if (!std::isfinite(rms_eps) || rms_eps < 0.f) return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT, "rms_eps must be finite and >= 0");
  if (!mla::abi_aligned(q_nope128, 16) || !mla::abi_aligned(w_uk_t, 16) || !mla::abi_aligned(q_nope_absorbed, 16) || !mla::abi_aligned(kv_cache, 16) ||
      !mla::abi_aligned(q_pe_raw, 16) || !mla::abi_aligned(q_pe, 16) || !mla::abi_aligned(rope_cos_sin, 16) || !mla::abi_aligned(c_kv_raw, 4) ||
      !mla::abi_aligned(kv_norm_w, 4) || !mla::abi_aligned(k_pe_raw, 4) || !mla::abi_aligned(seq_lens, 4) || !mla::abi_aligned(block_table, 4))
    return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT,
                "q_nope128, q_pe_raw, w_uk_t, rope_cos_sin, kv_cache, q_nope_absorbed and q_pe must be 16-byte "
                "aligned, the rest 4-byte aligned");
  int page_log2 = 0;
  while ((1 << page_log2) < page_size) ++page_log2;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = mla::launch_prolog(
      batch, q_len, num_heads, static_cast<const uint16_t*>(q_nope128), static_cast<const uint16_t*>(w_uk_t),
      static_cast<uint16_t*>(q_nope_absorbed), static_cast<const uint16_t*>(q_pe_raw),
      static_cast<const uint16_t*>(c_kv_raw), static_cast<const uint16_t*>(kv_norm_w), rms_eps,
      static_cast<const uint16_t*>(k_pe_raw), rope_cos_sin, max_pos, seq_lens, block_table, bt_stride, num_pages,
      page_log2, kv_format == MLA_KV_FP8, kv_cache, static_cast<uint8_t*>(kv_scales), static_cast<uint16_t*>(q_pe), st);
  if (e != hipSuccess) return mla::abi_hip_fail(e, "prolog kernel launch");
  mla::abi_ok();
  return MLA_OK;
}

mla_status mla_up_project(int32_t batch, int32_t q_len, int32_t num_heads, const float* attn_out, const void* w_uv,
                          void* o, void* stream) {
  if (!attn_out || !w_uv || !o) return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (batch < 1 || q_len < 1 || q_len > 8 || num_heads < 1 || num_heads > 128 || (int64_t)batch * q_len > (1 << 21))
    return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT,
                "batch >= 1, q_len in [1, 8], batch * q_len <= 2^21 and num_heads in [1, 128] are required");
  if (!mla::abi_aligned(attn_out, 16) || !mla::abi_aligned(w_uv, 16) || !mla::abi_aligned(o, 8))
    return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT, "attn_out and w_uv must be 16-byte aligned, o 8-byte aligned");
  hipError_t e = mla::launch_up_project(batch * q_len, num_heads, attn_out, static_cast<const uint16_t*>(w_uv),
                                        static_cast<uint16_t*>(o), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return mla::abi_hip_fail(e, "up-projection kernel launch");
  mla::abi_ok();
  return MLA_OK;
}

size_t mla_o_project_workspace_bytes(int32_t batch, int32_t q_len, int32_t k_in, int32_t n_out) {
  if (batch < 1 || q_len < 1 || q_len > 8 || k_in < 256 || k_in % 256 != 0 || k_in > (1 << 20) || n_out < 64 ||
      n_out % 64 != 0 || n_out > (1 << 22) || (int64_t)batch * q_len * n_out > (1 << 28))
    return 0;
  return mla::oproj_workspace_bytes(batch * q_len, n_out, k_in);
}

mla_status mla_o_project(int32_t batch, int32_t q_len, int32_t k_in, int32_t n_out, const void* x, const void* w_o,
                         void* y, void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !w_o || !y || !workspace) return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT, "a pointer is NULL");
  if (batch < 1 || q_len < 1 || q_len > 8 || (int64_t)batch * q_len > (1 << 21))
    return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT, "batch >= 1, q_len in [1, 8] and batch * q_len <= 2^21 are required");
  if (k_in < 256 || k_in % 256 != 0 || k_in > (1 << 20) || n_out < 64 || n_out % 64 != 0 || n_out > (1 << 22) ||
      (int64_t)batch * q_len * n_out > (1 << 28))
    return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT,
                         "k_in must be a multiple of 256 in [256, 2^20], n_out a multiple of 64 in [64, 2^22], and "
                         "batch * q_len * n_out <= 2^28");
  if (!mla::abi_aligned(x, 16) || !mla::abi_aligned(w_o, 16) || !mla::abi_aligned(workspace, 16) ||
      !mla::abi_aligned(y, 8))
    return mla::abi_fail(MLA_ERR_INVALID_ARGUMENT, "x, w_o and workspace must be 16-byte aligned, y 8-byte aligned");
  const size_t need = mla::oproj_workspace_bytes(batch * q_len, n_out, k_in);
  if (workspace_bytes < need) return mla::abi_fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than mla_o_project_workspace_bytes");
  hipError_t e = mla::launch_o_project(batch * q_len, n_out, k_in, static_cast<const uint16_t*>(x),
                                       static_cast<const uint16_t*>(w_o), static_cast<uint16_t*>(y),
                                       static_cast<float*>(workspace), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return mla::abi_hip_fail(e, "output projection kernel launch");
  mla::abi_ok();
  return MLA_OK;
}

