// Weight-absorbed MLA decode over an FP8 latent cache, for gfx950 (MI355X).
//
// The computation is the bf16 kernel's (Huawei, "DeepSeek V3/R1 inference
// deployment best practices on Ascend servers", section 3.2.1 and section
// 6.1): every head of a request attends over the same cached rows
// [c_kv | k_pe]; V is c_kv.  The same report names 8-bit keys and values as
// future work for MLA (section 8 on next steps, the bullet on quantized MLA
// operators); this kernel takes them
// in the OCP FP8 formats that gfx950's matrix cores read natively:
//  * cache: each token is 576 E4M3 codes plus one E8M0 scale byte e_t
//    (value 2^(e_t - 127)), so K_t = 2^(e_t - 127) * codes_t and V_t = K_t[0:512];
//  * queries arrive in bf16 and are quantized here to MXFP8: every block of 32
//    consecutive values of a 576-wide query row gets its own E8M0 exponent f
//    (the smallest with amax * 2^-f <= 448) and the E4M3 codes of q * 2^-f;
//  * QK^T runs on v_mfma_scale_f32_32x32x64_f8f6f4: the key scale (per token)
//    and the query block scale ride along as the instruction's per-lane scale
//    operands, so the fp32 scores come out fully scaled at no extra cost;
//  * PV runs on the same scaled instruction with P rounded to E4M3.  V's
//    per-token scale goes into P: p_t 2^(e_t - E + 6), E the largest scale
//    byte of the tile, and each tile's weights are taken relative to
//    2^x (x = floor of the tile's row maximum above the row's reference), so
//    the tile's largest weight lands in [2^6, 2^7), where E4M3 keeps 3
//    mantissa bits; 2^x and the tile's E go back in exactly through the P^T
//    scale operand.  The output therefore needs no rescale when a row's
//    maximum grows (only a growth beyond 2^32 moves the reference).
//
// Structure (one workgroup = 4 waves = 128 query rows; rows are the flattened
// (query token, head) pairs of one request):
//  * tiles of 64 keys (36 KB of codes, the bf16 kernel's stage size), copied
//    HBM -> LDS with 16-byte direct loads into a ring of 4 stages, plus each
//    tile's 64 scale bytes; one barrier per tile;
//  * wave w owns 32 query rows, one 32x32 MFMA block: S^T = K Q^T gives lane
//    l row l%32 and keys 32kb + 8a + 4(l/32) + b (kb, a < 4, b < 4 its
//    registers), so the row max and sum take one lane swap;
//  * O^T = V^T P^T accumulates 16 blocks of 32 columns x 32 rows in the 256
//    AGPRs; P^T is built in registers from the S^T layout (K slot
//    16kb + 4a + b of lane half l/32 is that key) and V^T comes from the same
//    LDS tile through ds_read_b64_tr_b8 in the same key order;
//  * software pipeline as in the bf16 kernel: QK^T of tile i+1 (with the
//    copies of tile i+3 between its MFMAs), then PV of tile i with the softmax
//    of tile i+1 between its MFMAs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <utility>

#include "decode_fp8.h"
#include "plan_internal.h"

namespace mla {
namespace {

#include "device_common.h"

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRowBytes8 = 576;                           // one cached token (HBM and LDS)
constexpr int kTile8 = kFp8TileTokens;                    // 64 keys per tile
constexpr int kWaves8 = kFp8Waves;                        // 4
constexpr int kRowsPerBlock8 = 32 * kWaves8;              // 128
constexpr int kBlockBytes8 = 32 * kRowBytes8;             // 18432: one 32-key block of a tile
constexpr int kStageBytes8 = kTile8 * kRowBytes8;         // 36864
constexpr int kStages8 = 4;
constexpr int kLoadsPerWave8 = kStageBytes8 / 1024 / kWaves8;  // 9 one-KB copies
constexpr int kCopiesPerWave8 = kLoadsPerWave8 + 1;            // + the scale bytes
constexpr int kScaleArea8 = 256;                          // one wave's copy of a tile's scale bytes
constexpr int kKSteps8 = 576 / 64;                        // 9 K steps of QK^T
#ifndef MLA8_QK_DEPTH
#define MLA8_QK_DEPTH 1
#endif
#ifndef MLA8_PV_DEPTH
#define MLA8_PV_DEPTH 1
#endif
constexpr int kQkDepth8 = MLA8_QK_DEPTH;  // MFMAs of K-operand reads in flight ahead
constexpr int kPvDepth8 = MLA8_PV_DEPTH;  // column blocks of V^T reads in flight ahead
constexpr int kWeightExp8 = 6;                            // P is scaled by 2^6 before rounding
constexpr float kRefStep8 = 32.0f;                        // reference moves past this (log2 units)
constexpr float kLn2_8 = 0.69314718055994530942f;
constexpr float kMuFloor8 = -1e30f;
constexpr int kLdsBytes8 = kStages8 * kStageBytes8 + kStages8 * kWaves8 * kScaleArea8 + kWaves8 * 256;
static_assert(kLdsBytes8 <= 160 * 1024, "LDS budget of one workgroup");

// LDS layout of a tile: two 32-key blocks of 18 KB, each column major as in
// the bf16 kernel: the 16-byte chunk c (0..35) of key row t (0..31) sits at
// slot 32c + (t ^ 16(c & 1)).
//  * copy n (0..17) of a block fills slots 64n .. 64n+63: lane l brings chunk
//    2n + l/32 of key row (l % 32) ^ 16(l / 32);
//  * QK^T: the scaled instruction orders K as (byte / 16, lane half, byte %
//    16) and applies the scale of lane half g to K slots 32g .. 32g+31, i.e.
//    to bytes 16g .. 16g+15 of both lane halves (measured).  So K step s,
//    lane half g reads chunks 4s + g (its bytes 0..15: channels 64s + 16g ..,
//    half of query block 2s) and 4s + 2 + g (bytes 16..31: half of block
//    2s + 1) of key row l%32, and carries the scale of query block 2s + g; a
//    half wave covers 32 rows of one chunk: 512 distinct bytes modulo 512;
//  * PV: ds_read_b64_tr_b8 hands output lane i of each 16-lane group byte i%8
//    of source lanes 2k + i/8 (k = 0..7).  Source lane 2k + h of group G reads
//    8 bytes of chunk 2cb + (G & 1), byte 8h, of the key row that is K slot
//    8r + k of lane half G/2 (read r = 0..3 of the column block), so output
//    lane i gets column 32cb + 16(G & 1) + i of 8 keys.  A read covers 16 key
//    rows of an even and an odd chunk, which the half swap separates.

// v_max over the whole wave of a non-negative integer, result in every lane.
__device__ __forceinline__ int wave_max_u32(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false));  // row_ror:8
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x124, 0xf, 0xf, false));  // row_ror:4
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x122, 0xf, 0xf, false));  // row_ror:2
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x121, 0xf, 0xf, false));  // row_ror:1
  auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  x = max((int)r[0], (int)r[1]);
  auto s = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return max((int)s[0], (int)s[1]);
}

// Sum / max over lanes l and l ^ 32 (the two lanes of a query row).
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}

// 4-byte global -> LDS copy (global_load_lds_dword): lane l writes LDS byte
// M0 + 4l.  Inline asm for the same reason as dma16.
__device__ __forceinline__ void dma4(const void* src, uint32_t lds_dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds_dst) : "memory");
}

// Scaled QK^T MFMA: acc (+)= (2^(sa-127) K) (2^(sb-127) Q)^T, each scale an
// E8M0 byte alone in its register (byte 0; the other bytes zero: measured,
// nonzero upper bytes change the result even with byte 0 selected).
// As for the bf16 kernel's S^T accumulators: pinned to VGPRs, srcC = 0 on
// the first step, results read only after s_mfma8_drain.
__device__ __forceinline__ void s_mfma8(f32x16& acc, const i32x8& a, const i32x8& b, int sa, int sb, bool first) {
  if (first)
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %4"
                 : "=&v"(acc)
                 : "v"(a), "v"(b), "v"(sa), "v"(sb));
  else
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4"
                 : "+v"(acc)
                 : "v"(a), "v"(b), "v"(sa), "v"(sb));
}

// XDL write -> VALU read of a 16-pass MFMA result: 18 wait states needed.
__device__ __forceinline__ void s_mfma8_drain(f32x16 (&acc)[2]) {
  asm volatile("s_nop 15\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]));
}

// The output accumulators: 16 blocks of a 32x32 fp32 MFMA result in the AGPRs
// a[0:255], block cb = a[16cb : 16cb+15] (columns 32cb .. 32cb+31 of the 32
// query rows of the wave).  Register r of block cb in lane l holds row l%32,
// column 32cb + 8(r/4) + 4(l/32) + r%4.  Same discipline as the bf16 kernel:
// only inline asm that names and clobbers them touches them.
template <int N>
struct OBlock;
template <int N>
struct OBlock8;
template <int N>
__device__ __forceinline__ float o_get();
template <int N>
__device__ __forceinline__ void o_set(float x);
#include "agpr_tiles.inc"
#include "agpr_tiles_fp8.inc"

template <int R>
__device__ __forceinline__ void o8_zero_rec() {
  if constexpr (R < 256) {
    o_set<R>(0.f);
    o8_zero_rec<R + 1>();
  }
}

template <int R>
__device__ __forceinline__ void o8_scale_rec(float alpha) {
  if constexpr (R < 256) {
    o_set<R>(o_get<R>() * alpha);
    o8_scale_rec<R + 1>(alpha);
  }
}

// MFMA (16 passes) -> accvgpr_read of the results.
__device__ __forceinline__ void o8_drain() { asm volatile("s_nop 15\n\ts_nop 7" ::: "memory"); }

template <int CB>
__device__ __forceinline__ float o8_absmax_rec(float m) {
  if constexpr (CB < 64) {
    constexpr int r = 4 * CB;
    float a, b;
    asm volatile("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(a) : "v"(m), "v"(o_get<r + 0>()), "v"(o_get<r + 1>()));
    asm volatile("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(b) : "v"(a), "v"(o_get<r + 2>()), "v"(o_get<r + 3>()));
    return o8_absmax_rec<CB + 1>(b);
  }
  return m;
}

// The epilogue stages each wave's 32 rows through LDS (its own 36 KB stage,
// rows kStageRow8 bytes apart: the 16-byte pad puts the 32 rows of one write
// in distinct banks) so that every global store writes 1 KB of one row; stored
// straight from the 32x32 layout, a store would write 32 bytes of 32 rows.
constexpr int kStageRow8 = 1024 + 16;

// fp32 output, half H (columns 256H .. 256H+255): block cb, register quad i
// holds columns 32cb + 8i + 4(l/32) .. +3; `row` is this lane's row base
// in the stage plus 16(l/32).
template <int H, int CB>
__device__ __forceinline__ void o8_stage_f32_rec(uint32_t row, float inv) {
  if constexpr (CB < 8) {
    constexpr int r = 16 * (8 * H + CB);
    *LDS_AS(f32x4, (uintptr_t)(row + 128 * CB + 0)) =
        f32x4{o_get<r + 0>() * inv, o_get<r + 1>() * inv, o_get<r + 2>() * inv, o_get<r + 3>() * inv};
    *LDS_AS(f32x4, (uintptr_t)(row + 128 * CB + 32)) =
        f32x4{o_get<r + 4>() * inv, o_get<r + 5>() * inv, o_get<r + 6>() * inv, o_get<r + 7>() * inv};
    *LDS_AS(f32x4, (uintptr_t)(row + 128 * CB + 64)) =
        f32x4{o_get<r + 8>() * inv, o_get<r + 9>() * inv, o_get<r + 10>() * inv, o_get<r + 11>() * inv};
    *LDS_AS(f32x4, (uintptr_t)(row + 128 * CB + 96)) =
        f32x4{o_get<r + 12>() * inv, o_get<r + 13>() * inv, o_get<r + 14>() * inv, o_get<r + 15>() * inv};
    o8_stage_f32_rec<H, CB + 1>(row, inv);
  }
}

// Half-precision partial in the bf16 kernel's stored order (position
// 32(c/2) + 8grp + 4(c%2) + i holds column 16c + 4grp + i for 16-column
// block c and 16-lane group grp of that kernel): here column
// 32cb + 8i + 4g + j sits at 32cb + 16(i%2) + 8g + 4(i/2) + j, so register
// quads 0 and 2 of a block form 8 consecutive positions, and so do 1 and 3
// (`row` is this lane's row base in the stage plus 16(l/32)).
template <int CB>
__device__ __forceinline__ void o8_stage_half_rec(uint32_t row, float c) {
  if constexpr (CB < 16) {
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    constexpr int r = 16 * CB;
    f16x8 w0 = {(_Float16)(o_get<r + 0>() * c), (_Float16)(o_get<r + 1>() * c), (_Float16)(o_get<r + 2>() * c),
                (_Float16)(o_get<r + 3>() * c), (_Float16)(o_get<r + 8>() * c), (_Float16)(o_get<r + 9>() * c),
                (_Float16)(o_get<r + 10>() * c), (_Float16)(o_get<r + 11>() * c)};
    f16x8 w1 = {(_Float16)(o_get<r + 4>() * c), (_Float16)(o_get<r + 5>() * c), (_Float16)(o_get<r + 6>() * c),
                (_Float16)(o_get<r + 7>() * c), (_Float16)(o_get<r + 12>() * c), (_Float16)(o_get<r + 13>() * c),
                (_Float16)(o_get<r + 14>() * c), (_Float16)(o_get<r + 15>() * c)};
    *LDS_AS(f16x8, (uintptr_t)(row + 64 * CB)) = w0;
    *LDS_AS(f16x8, (uintptr_t)(row + 64 * CB + 32)) = w1;
    o8_stage_half_rec<CB + 1>(row, c);
  }
}

// E4M3 codes of this lane's 32 bf16 values of one K step: values 0..15 are
// half of query block 2s, values 16..31 half of block 2s + 1; the other
// halves sit in the partner lane l ^ 32.  Each block's exponent f is the
// smallest with amax * 2^-f <= 448 (0 for amax = 0), limited to [-127, 127];
// returns the 8 code words and the scale byte 127 + f of block 2s + g.
struct QBlock {
  i32x8 codes;
  int e8m0;
};

// Packed unsigned 16-bit max of two words (v_pk_max_u16).
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_u16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ int block_exponent(float amax) {
  // amax = m 2^x with m in [0.5, 1); 448 = 0.875 * 2^9: f = x - 9 if
  // m <= 0.875, else x - 8
  if (!(amax > 0.f)) return 0;
  const int x = __builtin_amdgcn_frexp_expf(amax);
  const float m = __builtin_amdgcn_frexp_mantf(amax);
  return min(max(x - 9 + (m > 0.875f ? 1 : 0), -127), 127);
}

__device__ __forceinline__ QBlock quantize_block(const bf16x8 (&v)[4], int g) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef short i16x2 __attribute__((ext_vector_type(2)));
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 u = __builtin_bit_cast(u32x4, v[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) w[4 * i + j] = u[j];
  }
  // Largest magnitude of each half: the bf16 bit patterns without their sign
  // order like the magnitudes, so a packed 16-bit max finds it exactly.
  float am[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t m = w[8 * h] & 0x7fff7fffu;
#pragma unroll
    for (int i = 1; i < 8; ++i) m = pk_max_u16(m, w[8 * h + i] & 0x7fff7fffu);
    am[h] = __uint_as_float(max(m & 0xffffu, m >> 16) << 16);
  }
  int f[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) f[h] = block_exponent(pair_max(am[h]));
  // v_cvt_scalef32_pk_fp8_bf16 rounds (x / scale) to E4M3, nearest even:
  // scale = 2^f is exact.
  QBlock q;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float sc = __builtin_ldexpf(1.f, f[i >> 2]);
    i16x2 c = {0, 0};
    c = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(c, __builtin_bit_cast(bf16x2, w[2 * i]), sc, false);
    c = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(c, __builtin_bit_cast(bf16x2, w[2 * i + 1]), sc, true);
    q.codes[i] = __builtin_bit_cast(int, c);
  }
  q.e8m0 = 127 + (g ? f[1] : f[0]);
  return q;
}

// Page ids a 64-key tile touches (NPG = 64 / page size, at most 4).
template <int NPG>
struct TilePages8 {
  int first;
  int pg[NPG];
};

template <int NPG>
__global__ __launch_bounds__(64 * kWaves8, 1) void decode_fp8_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe, const uint8_t* __restrict__ cache,
    const uint8_t* __restrict__ kv_scale, int64_t num_pages, const int32_t* __restrict__ block_table,
    int32_t bt_stride, const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ planned_lens,
    const Segment* __restrict__ segs, const WorkgroupRange* __restrict__ wgs, float scale_log2, int32_t rows,
    int32_t heads, int32_t q_len, int32_t page_log2, int32_t nrb, float* __restrict__ out, float* __restrict__ lse,
    uint16_t* __restrict__ ws_o, float* __restrict__ ws_lse, float* __restrict__ ws_f) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes8];
  uint8_t* const scl_lds = smem + kStages8 * kStageBytes8;                 // [stage][wave][256]
  uint8_t* const sc_lds = scl_lds + kStages8 * kWaves8 * kScaleArea8;      // [wave][64] fp32

  const WorkgroupRange wr = wgs[blockIdx.x];
  if (wr.seg_begin >= wr.seg_end) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;  // K half of operands, key quad of results
  const int l32 = lane & 31;
  const int rb = wr.row_block;
  const int psize = 1 << page_log2;

  // This lane's query row.
  const int row_local = wave * 32 + l32;
  const int row = rb * kRowsPerBlock8 + row_local;
  const bool row_ok = row < rows;
  const int jq = row_ok ? row / heads : 0;
  const int wave_row0 = rb * kRowsPerBlock8 + wave * 32;
  const bool wave_full = wave_row0 + 31 < rows;
  const int wave_jq0 = wave_row0 / heads;

  // Per-lane LDS byte offsets within a stage.
  // QK^T A operand: key l32 of block kb, chunks 4s + g and 4s + 2 + g (both
  // of parity g): + 2048 s + 18432 kb.
  const int qk_off0 = 512 * g + 16 * (l32 ^ (16 * g));
  const int qk_off1 = qk_off0 + 1024;
  // PV tr reads: lane l = 16G + i, i = 2k + h; read r of column block cb at
  // pv_off0 (^ 256 for odd r) + 18432 (r / 2) + 1024 cb.
  const int G = lane >> 4, ik = (lane & 15) >> 1, ih = lane & 1;
  const int t0 = 8 * (ik >> 2) + 4 * (G >> 1) + (ik & 3);
  const int pv_off0 = 768 * (G & 1) + 16 * t0 + 8 * ih;
  // Copies: wave w fills 1 KB pieces 9w .. 9w+8 of the stage (block w/2,
  // copies 9(w%2) .. of it); lane l reads key row dma_row of that block,
  // bytes 288(w%2) + 16(l/32) + 32i of it.
  const int dma_row = (lane & 31) ^ (16 * (lane >> 5));
  const int dma_kb = wave >> 1;
  const int dma_col = 288 * (wave & 1) + 16 * (lane >> 5);

  for (int si = wr.seg_begin; si < wr.seg_end; ++si) {
    const Segment sg = segs[si];
    const int b = sg.b, kv0 = sg.kv_begin, kv1 = sg.kv_end;
    const int32_t* bt_row = block_table + (int64_t)b * bt_stride;

    const int first_pg = kv0 >> page_log2;
    const int last_pg = (kv1 - 1) >> page_log2;
    int pg_lane = load4(bt_row + min(first_pg + lane, last_pg));

    // Query row in bf16: K step s, lane half g holds channels 64s + 16g ..
    // +15 and 64s + 32 + 16g .. +15 (q_nope for s < 8, q_pe for s = 8) as 4
    // loads of 16 bytes, loaded and quantized in three groups of three steps
    // (so that at most two groups of raw values are live).  Rows past the end
    // load row 0 (masked, never stored).
    const int qrow = row_ok ? row : 0;
    const uint16_t* qn = q_nope + ((int64_t)b * rows + qrow) * 512 + 16 * g;
    const uint16_t* qp = q_pe + ((int64_t)b * rows + qrow) * 64 + 16 * g;
    bf16x8 qraw[2][3][4];
    auto load_group = [&](int grp_, bf16x8 (&dst)[3][4]) {
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int s = 3 * grp_ + k;
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[k][i] = load16((s < 8 ? qn + 64 * s : qp) + 8 * (i & 1) + 32 * (i >> 1));
      }
    };
    load_group(0, qraw[0]);
    load_group(1, qraw[1]);

    const int L = seq_lens[b];
    const bool bad_len = (L != planned_lens[b]);
    const int lim = row_ok ? min(kv1, L - q_len + 1 + jq) : kv0;
    // uniform: the per-tile masking test is then a scalar compare and branch
    const int lim_wave = __builtin_amdgcn_readfirstlane(wave_full ? min(kv1, L - q_len + 1 + wave_jq0) : kv0);

    auto page_at = [&](int pidx) {
      const int rel = pidx - first_pg;
      if (rel < 64) return __builtin_amdgcn_readlane(pg_lane, rel);
      // Further pages: a uniform index read through the constant address
      // space, so the compiler issues a scalar load (waited for with lgkmcnt)
      // instead of a vector load whose vmcnt(0) would drain the tile copies.
      const __attribute__((address_space(4))) int32_t* bt_s = (const __attribute__((address_space(4))) int32_t*)bt_row;
      return bt_s[__builtin_amdgcn_readfirstlane(pidx)];
    };
    auto fetch_pages = [&](int tb) {
      TilePages8<NPG> tp;
      tp.first = tb >> page_log2;
      const int last = (min(tb + kTile8, kv1) - 1) >> page_log2;
#pragma unroll
      for (int k = 0; k < NPG; ++k) tp.pg[k] = page_at(min(tp.first + k, last));
      return tp;
    };
    // A page id outside [0, num_pages) is never followed: page 0 is read
    // instead, and the piece's rows end as NaN (bad_pg), like a length mismatch.
    // page ids are int32: a pool of 2^31 pages or more holds every id
    const uint32_t num_pages_u32 = (uint32_t)min(num_pages, (int64_t)0x80000000LL);
    bool bad_pg = false;
    auto checked = [&](TilePages8<NPG> tp) {
#pragma unroll
      for (int k = 0; k < NPG; ++k) {
        const bool ok = (uint32_t)tp.pg[k] < num_pages_u32;  // scalar compare (ids are uniform)
        bad_pg = bad_pg || !ok;
        tp.pg[k] = ok ? tp.pg[k] : 0;
      }
      return tp;
    };
    // Page of token tok (inside the tile of tp).
    auto page_of = [&](const TilePages8<NPG>& tp, int tok) {
      if constexpr (NPG == 1) {
        return tp.pg[0];
      } else {
        const int k = (tok >> page_log2) - tp.first;
        int p = tp.pg[0];
#pragma unroll
        for (int j = 1; j < NPG; ++j) {
          // the empty asm keeps the (uniform) ids out of an indexed stack
          // array, which the compiler otherwise builds from this select chain
          int c = tp.pg[j];
          asm("" : "+s"(c));
          p = (k == j) ? c : p;
        }
        return p;
      }
    };

    // Per-tile sources of this lane's copies.  Key rows past the piece are
    // clamped to its last key (masked; finite values for PV); the scale copy
    // reads the aligned 4 bytes holding keys 4(l%16) .. +3 of the tile,
    // clamped to the 4-byte group of the last key (inside its page).
    struct TileSrc8 {
      const uint8_t* base;  // uniform (one page per tile)
      uint32_t off;         // per lane
      const uint8_t* ptr;   // per lane (several pages per tile)
      const uint8_t* sptr;  // per lane: scale bytes
    };
    auto tile_src = [&](int tb, const TilePages8<NPG>& tp) {
      TileSrc8 ts;
      const int tok = min(tb + 32 * dma_kb + dma_row, kv1 - 1);
      if constexpr (NPG == 1) {
        ts.base = cache + ((int64_t)tp.pg[0] << page_log2) * kRowBytes8;
        ts.off = (uint32_t)((tok & (psize - 1)) * kRowBytes8 + dma_col);
        ts.ptr = nullptr;
      } else {
        ts.base = nullptr;
        ts.off = 0;
        ts.ptr = cache + (((int64_t)page_of(tp, tok) << page_log2) + (tok & (psize - 1))) * kRowBytes8 + dma_col;
      }
      const int stok = min(tb + 4 * (lane & 15), (kv1 - 1) & ~3);
      ts.sptr = kv_scale + ((int64_t)page_of(tp, stok) << page_log2) + (stok & (psize - 1));
      return ts;
    };
    auto dma = [&](auto ic, const TileSrc8& ts, int stage) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i < kLoadsPerWave8) {
        const uint32_t dst = lds_addr(smem + stage * kStageBytes8) + (uint32_t)(9216 * wave + 1024 * i - 32 * i);
        if constexpr (NPG == 1)
          dma16_saddr<32 * i>(ts.base, ts.off, dst);
        else
          dma16_off<32 * i>(ts.ptr, dst);
      } else {
        dma4(ts.sptr, lds_addr(scl_lds + (stage * kWaves8 + wave) * kScaleArea8));
      }
    };
    auto dma_all = [&](const TileSrc8& ts, int stage) {
      static_for<kCopiesPerWave8>([&](auto ic) { dma(ic, ts, stage); });
    };

    const int ntiles = (kv1 - kv0 + kTile8 - 1) / kTile8;
    const int last_tile = ntiles - 1;

    __syncthreads();  // the previous piece is done with every stage
    wait_vmem<2 * 12>();  // page ids (issued before the query loads)
    asm volatile("" : "+v"(pg_lane));

    auto dma_tile = [&](int st) {
      const int ti = min(st, last_tile);
      const int tb_c = kv0 + ti * kTile8;
      dma_all(tile_src(tb_c, checked(fetch_pages(tb_c))), st);
    };
    i32x8 q8[kKSteps8];
    int qsc[kKSteps8];  // block scale byte of K step s (byte 0; upper bytes zero)
    auto quantize_group = [&](int grp_, bf16x8 (&raw)[3][4]) {
#pragma unroll
      for (int k = 0; k < 3; ++k) {
        const int s = 3 * grp_ + k;
        asm volatile("" : "+v"(raw[k][0]), "+v"(raw[k][1]), "+v"(raw[k][2]), "+v"(raw[k][3]));
        const QBlock qb = quantize_block(raw[k], g);
        q8[s] = qb.codes;
        qsc[s] = qb.e8m0;
      }
    };
    // Issue order (the counter retires vector memory operations in issue
    // order): query groups 0 and 1, tile 0, query group 2, tiles 1 and 2.
    dma_tile(0);
    wait_vmem<12 + kCopiesPerWave8>();  // query group 0 (group 1, tile 0 may fly)
    quantize_group(0, qraw[0]);
    load_group(2, qraw[0]);
    wait_vmem<kCopiesPerWave8 + 12>();  // query group 1 (tile 0, group 2 may fly)
    quantize_group(1, qraw[1]);
    dma_tile(1);
    dma_tile(2);
    wait_vmem<2 * kCopiesPerWave8>();  // query group 2 (and tile 0) have landed
    quantize_group(2, qraw[0]);
    TilePages8<NPG> pg_raw = fetch_pages(kv0 + min(3, last_tile) * kTile8);

    // ---- per-tile scale handling (this wave's copy of the tile's bytes) ----
    // ea[kb]: scale byte of key 32kb + l32 (the QK^T A-operand scale).
    // E_tile: the largest scale byte of the tile's keys; sc (LDS, per wave):
    // 2^(e_t - E_tile + 6) for every key t of the tile, read back per lane.
    // e0: E_tile of the piece's first tile; a tile's P carries
    // 2^(E_tile - e0) in its PV scale operand, so the output accumulates
    // p_t 2^(e_t - e0 + 6) codes_t throughout.  Only a tile more than 2^64
    // above e0 moves e0 (and rescales the output).
    int e0 = -1;
    int de = 0;              // E_tile - e0 of the tile just prepared
    bool e_moved = false;    // e0 moved on it
    float e_alpha = 1.f;     // 2^(e0_old - e0_new)
    int ea[2];
    const uint32_t sc_base = lds_addr(sc_lds + wave * 256);
    // Keys past the piece (tb + k >= kv1) take the neutral byte 127 for QK^T
    // and 0 for E_tile: the copied 4-byte groups may hold bytes of slots past
    // the request's end, which must not steer anything.
    auto prep_scales = [&](int stage, int tb_s) {
      const uint8_t* sa = scl_lds + (stage * kWaves8 + wave) * kScaleArea8;
      const int e0b = *LDS_AS(const uint8_t, (uintptr_t)lds_addr(sa + l32));
      const int e1b = *LDS_AS(const uint8_t, (uintptr_t)lds_addr(sa + 32 + l32));
      const bool v0 = tb_s + l32 < kv1, v1 = tb_s + 32 + l32 < kv1;
      ea[0] = v0 ? e0b : 127;
      ea[1] = v1 ? e1b : 127;
      const int ej = g ? (v1 ? e1b : 0) : (v0 ? e0b : 0);  // key `lane` of the tile
      const int et = __builtin_amdgcn_readfirstlane(wave_max_u32(ej));
      e_moved = false;
      e_alpha = 1.f;
      if (e0 < 0) {
        e0 = et;
      } else if (et - e0 > 64) {
        e_moved = true;
        e_alpha = __builtin_ldexpf(1.f, e0 - et);
        e0 = et;
      }
      de = et - e0;
      const int ex = ej - et + 127 + kWeightExp8;
      const float sc = ex > 0 ? __int_as_float(ex << 23) : 0.f;
      *LDS_AS(float, (uintptr_t)(sc_base + 4 * lane)) = sc;
    };

    // QK^T of one tile: acc[kb] = S^T block (keys 32kb.., the wave's 32 rows).
    auto qk_tile = [&](int stage, f32x16(&acc)[2], auto&& extra) {
      const uint32_t base = lds_addr(smem + stage * kStageBytes8);
      // One address register per operand half for the whole tile; every read
      // adds a compile-time offset in the instruction (the empty asm keeps
      // the compiler from splitting the sum into a per-read VALU op).
      uint32_t b0 = base + qk_off0, b1 = base + qk_off1;
      asm volatile("" : "+v"(b0), "+v"(b1));
      // MFMA m = 2s + kb; its operand is read one MFMA ahead.
      constexpr int D = kQkDepth8;
      i32x8 a[D + 1];
      auto read = [&](int m, i32x8& dst) {
        const uint32_t o = 18432 * (m & 1) + 2048 * (m >> 1);
        const f32x4 lo = *LDS_AS(const f32x4, (uintptr_t)(b0 + o));
        const f32x4 hi = *LDS_AS(const f32x4, (uintptr_t)(b1 + o));
        dst = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
#pragma unroll
      for (int d = 0; d < D; ++d) read(d, a[d]);
      static_for<2 * kKSteps8>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        constexpr int s = m >> 1, kb = m & 1;
        if constexpr (m + D < 2 * kKSteps8) read(m + D, a[(m + D) % (D + 1)]);
        extra(m);
        s_mfma8(acc[kb], a[m % (D + 1)], q8[s], ea[kb], qsc[s], s == 0);
        __builtin_amdgcn_sched_barrier(0);
      });
      s_mfma8_drain(acc);
    };

    // O^T += V^T P^T for one tile (16 column blocks, 4 transposed reads each).
    // Addresses of the four reads of column block cb: v0 + 1024 cb, v1 +
    // 1024 cb and both + 18432, with v0 = stage + pv_off0 and v1 = stage +
    // (pv_off0 ^ 256) (stage bases and 1024 cb leave bits 0..9 alone, so the
    // bit-8 flip of the other row half commutes with the sum).
    struct PvBase8 {
      uint32_t v0, v1;
    };
    auto pv_base = [&](int stage) {
      const uint32_t st = lds_addr(smem + stage * kStageBytes8);
      PvBase8 pb{st + pv_off0, st + (pv_off0 ^ 256)};
      asm volatile("" : "+v"(pb.v0), "+v"(pb.v1));  // one register each for the tile
      return pb;
    };
    auto read_v = [&](const PvBase8& pb, int cb, i32x8& dst) {
      const uint32_t o = 1024 * cb;
      i32x2 r0 = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_AS(i32x2, (uintptr_t)(pb.v0 + o))));
      i32x2 r1 = __builtin_bit_cast(i32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_AS(i32x2, (uintptr_t)(pb.v1 + o))));
      i32x2 r2 = __builtin_bit_cast(
          i32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_AS(i32x2, (uintptr_t)(pb.v0 + o + 18432))));
      i32x2 r3 = __builtin_bit_cast(
          i32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDS_AS(i32x2, (uintptr_t)(pb.v1 + o + 18432))));
      dst = i32x8{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
    };
    const int one_e8m0 = 127;  // V^T is not scaled
    auto pv_tile = [&](int stage, const i32x8& pt, int pscale, auto&& extra) {
      constexpr int DV = kPvDepth8;
      const PvBase8 pb = pv_base(stage);
      i32x8 v[DV + 1];
#pragma unroll
      for (int d = 0; d < DV; ++d) read_v(pb, d, v[d]);
      static_for<16>([&](auto cbc) {
        constexpr int cb = decltype(cbc)::value;
        if constexpr (cb + DV < 16) read_v(pb, cb + DV, v[(cb + DV) % (DV + 1)]);
        extra(cb);
        OBlock8<cb>::mfma(v[cb % (DV + 1)], pt, one_e8m0, pscale);
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // ---- online softmax state (base 2, one row per lane) ----
    // mu: the row's reference (log2 units), set by its first finite maximum
    // and moved only when the maximum passes it by more than kRefStep8 (an
    // fp32 range guard; the output is then rescaled).  Each tile's weights
    // are taken relative to mu + x, x = floor(tile max - mu), so that the
    // tile's largest weight times 2^6 lands in [2^6, 2^7) before rounding to
    // E4M3; 2^x goes back in through the PV scale operand (with 2^de).
    float mu = kMuFloor8, l_part = 0.f, alpha_o = 1.f;
    bool any_scale = false;
    float mx = 0.f, mu_t = 0.f, px = 1.f;
    int psc = 127;  // PV scale byte of the tile in flight
    // Softmax of one tile of scores s (s[kb][4a + b] = key tb_s + 32kb + 8a +
    // 4g + b of this lane's row), in kSmSteps8 steps, one per PV MFMA gap:
    //   0: mask the keys past the row's limit (tiles that need it), lane max;
    //   1: row max (lane pair), reference and x; the LDS reads of the first
    //      two key groups' factors sc;
    //   2, 3: element pairs 0-1 and 2-3; 4..15: pair `step` (pair j = elements
    //      2(j%2), 2(j%2)+1 of key group j/2, group q = (kb, a) = (q/4, q%4)):
    //      p = 2^(s*scale - mu - x), running sum p 2^x, P' = p * sc, and half a
    //      word of P^T (K slots 4(4kb + a) ..).  The factors of group q are read
    //      two groups ahead into sc_buf[q % 2].
    constexpr int kSmSteps8 = 16;
    f32x4 sc_buf[2];
    auto sc_read = [&](int q) {
      const int kb = q >> 2, a = q & 3;
      sc_buf[q & 1] = *LDS_AS(const f32x4, (uintptr_t)(sc_base + 4 * (32 * kb + 8 * a + 4 * g)));
    };
    auto sm_pair = [&](int j, f32x16(&s)[2], i32x8& pt) {
      const int q = j >> 1, h = j & 1, kb = q >> 2, a = q & 3;
      const f32x4& sc = sc_buf[q & 1];
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * a + 2 * h], scale_log2, -mu_t));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * a + 2 * h + 1], scale_log2, -mu_t));
      l_part = __builtin_fmaf(p0, px, l_part);
      l_part = __builtin_fmaf(p1, px, l_part);
      if (h)
        pt[4 * kb + a] = __builtin_amdgcn_cvt_pk_fp8_f32(p0 * sc[2], p1 * sc[3], pt[4 * kb + a], true);
      else
        pt[4 * kb + a] = __builtin_amdgcn_cvt_pk_fp8_f32(p0 * sc[0], p1 * sc[1], 0, false);
      if (h == 1 && q + 2 < 8) sc_read(q + 2);
    };
    auto softmax_step = [&](int step, f32x16(&s)[2], int need_mask, int tb_s, i32x8& pt, int& pscale) {
      if (step == 0) {
        if (need_mask) {  // uniform (scalar compare of uniform limits): a scalar branch
          // Keys left of the row's limit, counted from this lane's first key;
          // the empty asm keeps the subtraction inside the branch.
          int room = lim - (tb_s + 4 * g);
          asm volatile("" : "+v"(room));
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int k = 32 * kb + 8 * (r >> 2) + (r & 3);
              s[kb][r] = k < room ? s[kb][r] : -INFINITY;
            }
        }
        float m0 = max3(max3(s[0][0], s[0][1], s[0][2]), max3(s[0][3], s[0][4], s[0][5]), max3(s[0][6], s[0][7], s[0][8]));
        float m1 = max3(max3(s[0][9], s[0][10], s[0][11]), max3(s[0][12], s[0][13], s[0][14]), max3(s[0][15], s[1][0], s[1][1]));
        float m2 = max3(max3(s[1][2], s[1][3], s[1][4]), max3(s[1][5], s[1][6], s[1][7]), max3(s[1][8], s[1][9], s[1][10]));
        float m3 = max3(max3(s[1][11], s[1][12], s[1][13]), s[1][14], s[1][15]);
        mx = max3(m0, m1, max3(m2, m3, m3));
      } else if (step == 1) {
        sc_read(0);
        sc_read(1);
        mx = pair_max(mx);
        const float m = mx * scale_log2;
        const bool fin = m > kMuFloor8;
        const bool had = mu > kMuFloor8;
        float alpha = 1.f;
        if (fin && !had) {
          mu = m;  // first finite maximum: nothing accumulated yet
        } else if (fin && m > mu + kRefStep8) {
          alpha = __builtin_amdgcn_exp2f(mu - m);
          mu = m;
        }
        l_part *= alpha;
        alpha_o = alpha * e_alpha;
        any_scale = any_scale || (had && (alpha != 1.f || e_moved));
        // x = floor(m - mu) (m - mu >= -2^9 before the conversion: a tile far
        // below the reference has weights that round to zero anyway), with
        // x + de kept inside the E8M0 range
        int x = fin ? (int)__builtin_floorf(fmaxf(m - mu, -512.f)) : 0;
        x = min(max(x + de, -127), 127) - de;
        mu_t = mu + (float)x;
        px = __builtin_ldexpf(1.f, x);
        pscale = 127 + x + de;
      } else if (step < 4) {
        sm_pair(2 * (step - 2), s, pt);
        sm_pair(2 * (step - 2) + 1, s, pt);
      } else if (step < kSmSteps8) {
        sm_pair(step, s, pt);
      }
    };

    // ---- prologue: tile 0 ----
    o8_zero_rec<0>();
    i32x8 pt;
    __syncthreads();  // tile 0 (every wave's part, landed above) is visible
    {
      f32x16 s0[2];
      prep_scales(0, kv0);
      qk_tile(0, s0, [](int) {});
      const int nm0 = kv0 + kTile8 > lim_wave ? 1 : 0;  // uniform (scalar)
#pragma unroll
      for (int step = 0; step < kSmSteps8; ++step) softmax_step(step, s0, nm0, kv0, pt, psc);
      any_scale = false;  // nothing accumulated yet
    }

    for (int it = 0; it < ntiles; ++it) {
      const bool has_next = it + 1 < ntiles;
      // Tile it+1 has landed once only tile it+2's copies are in flight; the
      // barrier publishes every wave's part and frees the stage of tile it-1.
      wait_vmem<kCopiesPerWave8>();
      __syncthreads();

      const int tb = kv0 + it * kTile8;
      const int st_cur = it % kStages8, st_next = (it + 1) % kStages8;
      const int nt = it + 3;
      const int st_copy = nt % kStages8;
      const int tb_c = kv0 + min(nt, last_tile) * kTile8;
      const TileSrc8 nsrc = tile_src(tb_c, checked(pg_raw));
      __builtin_amdgcn_sched_barrier(0);

      auto copy_at = [&](int k) {
        static_for<kCopiesPerWave8>([&](auto ic) {
          if (decltype(ic)::value == k) dma(ic, nsrc, st_copy);
        });
      };
      f32x16 s_next[2];
      i32x8 pt_next = pt;
      int psc_next = psc;
      if (has_next) {
        prep_scales(st_next, tb + kTile8);
        qk_tile(st_next, s_next, [&](int k) {
          if ((k & 1) == 0 && (k >> 1) < kCopiesPerWave8) copy_at(k >> 1);
          if (k == 17) copy_at(kCopiesPerWave8 - 1);
        });
      } else {
        dma_all(nsrc, st_copy);
      }
      __builtin_amdgcn_sched_barrier(0);

      if (has_next) {
        const int nm = tb + 2 * kTile8 > lim_wave ? 1 : 0;  // uniform (scalar)
        pv_tile(st_cur, pt, psc, [&](int cb) {
          softmax_step(cb, s_next, nm, tb + kTile8, pt_next, psc_next);
        });
        if (__any(any_scale)) {
          o8_drain();
          o8_scale_rec<0>(alpha_o);
        }
        any_scale = false;
        pt = pt_next;
        psc = psc_next;
      } else {
        pv_tile(st_cur, pt, psc, [](int) {});
      }
      pg_raw = fetch_pages(kv0 + min(nt + 1, last_tile) * kTile8);
    }

    wait_vmem<0>();

    // ---- epilogue ----
    o8_drain();
    const float l_tot = pair_sum(l_part);
    float lse_v = l_tot > 0.f ? (mu + __builtin_amdgcn_logf(l_tot)) * kLn2_8 : -INFINITY;
    if (bad_len || bad_pg) lse_v = NAN;
    // O holds sum_t p_t 2^(e_t - e0 + 6) codes_t = 2^(133 - e0) sum_t p_t V_t.
    const int oexp = e0 - 127 - kWeightExp8;
    // Every wave is past its last LDS read of the piece (and its copies have
    // landed): the stages are free for staging, wave w using stage w.
    __syncthreads();
    const uint32_t stg = lds_addr(smem + wave * kStageBytes8);
    const uint32_t stg_row = stg + l32 * kStageRow8 + 16 * g;
    const int nrow = min(32, rows - wave_row0);  // rows of this wave to store
    if (sg.partial < 0) {
      float inv = l_tot > 0.f ? __builtin_ldexpf(1.f / l_tot, oexp) : 0.f;
      if (bad_len || bad_pg) inv = NAN;
      // The lane index goes through an empty asm so that this address is
      // formed here and not hoisted above the tile loop, where it would hold
      // a register pair for the whole piece.
      int ln = lane;
      asm volatile("" : "+v"(ln));
      float* obase = out + ((int64_t)b * rows + wave_row0) * 512 + 4 * ln;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if (h == 0)
          o8_stage_f32_rec<0, 0>(stg_row, inv);
        else
          o8_stage_f32_rec<1, 0>(stg_row, inv);
        for (int r = 0; r < nrow; ++r) {
          const f32x4 v = *LDS_AS(const f32x4, (uintptr_t)(stg + r * kStageRow8 + 16 * lane));
          store_wt(obase + (int64_t)r * 512 + 256 * h, v);
        }
      }
      if (row_ok && g == 0) {
        int r = row;  // formed here, not hoisted above the tile loop
        asm volatile("" : "+v"(r));
        lse[(int64_t)b * rows + r] = lse_v;
      }
    } else {
      const int64_t slot = (int64_t)sg.partial * nrb + rb;
      float amax = pair_max(o8_absmax_rec<0>(0.f));
      const int e = max(__builtin_amdgcn_frexp_expf(amax), -110);
      const float c = __builtin_ldexpf(1.f, 15 - e);
      float f = l_tot > 0.f ? __builtin_ldexpf(1.f / l_tot, e - 15 + oexp) : 0.f;
      if (bad_len || bad_pg) f = NAN;
      o8_stage_half_rec<0>(stg_row, c);
      typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
      int ln = lane;  // formed here, not hoisted above the tile loop (see above)
      asm volatile("" : "+v"(ln));
      _Float16* hbase = reinterpret_cast<_Float16*>(ws_o) + (slot * kRowsPerBlock8 + wave * 32) * 512 + 8 * ln;
      for (int r = 0; r < nrow; ++r) {
        const f16x8 v = *LDS_AS(const f16x8, (uintptr_t)(stg + r * kStageRow8 + 16 * lane));
        store_wt(hbase + (int64_t)r * 512, v);
      }
      if (row_ok && g == 0) {
        int rl = row_local;  // formed here, not hoisted above the tile loop
        asm volatile("" : "+v"(rl));
        const int64_t ri = slot * kRowsPerBlock8 + rl;
        ws_lse[ri] = lse_v;
        ws_f[ri] = f;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_fp8(const PlanData& d, const char* sched, size_t off_segs, size_t off_wgs, size_t off_lens,
                             const void* q_nope, const void* q_pe, const void* cache, const void* kv_scale,
                             int64_t num_pages, const int32_t* block_table, int32_t bt_stride,
                             const int32_t* seq_lens, float scale_log2, float* out, float* lse, uint16_t* ws_o,
                             float* ws_lse, float* ws_f, hipStream_t stream) {
  int page_log2 = 0;
  while ((1 << page_log2) < d.page) ++page_log2;
  const int npg = d.page >= kTile8 ? 1 : kTile8 / d.page;
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3(d.grid), dim3(64 * kWaves8), 0, stream, static_cast<const uint16_t*>(q_nope),
                       static_cast<const uint16_t*>(q_pe), static_cast<const uint8_t*>(cache),
                       static_cast<const uint8_t*>(kv_scale), num_pages, block_table, bt_stride, seq_lens,
                       reinterpret_cast<const int32_t*>(sched + off_lens),
                       reinterpret_cast<const Segment*>(sched + off_segs),
                       reinterpret_cast<const WorkgroupRange*>(sched + off_wgs), scale_log2, d.rows, d.heads,
                       d.q_len, page_log2, d.nrb, out, lse, ws_o, ws_lse, ws_f);
  };
  if (npg == 1)
    go(decode_fp8_kernel<1>);
  else if (npg == 2)
    go(decode_fp8_kernel<2>);
  else if (npg == 4)
    go(decode_fp8_kernel<4>);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mla
