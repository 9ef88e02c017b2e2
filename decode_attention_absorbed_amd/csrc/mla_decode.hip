// Weight-absorbed MLA decode attention for gfx950 (MI355X): split-KV decode
// kernel, log-sum-exp combine kernel and the C ABI around them.
//
// The computation (Huawei, "DeepSeek V3/R1 inference deployment best practices
// on Ascend servers", section 3.2.1 and section 6.1): every head of a request
// attends over the same cached 576-wide rows [c_kv | k_pe]; V is c_kv.  With
// the heads as one dimension of the product, QK^T and PV are dense
// contractions against a shared key tile, so both run on bf16 MFMA with fp32
// accumulation.
//
// Decode kernel: one workgroup = 4 waves = 128 query rows (rows are the
// flattened (query token, head) pairs of one request), walking one or more
// pieces of key range in tiles of 32 keys:
//  * tiles are copied HBM -> LDS with 16-byte direct loads
//    (global_load_lds_dwordx4) into a ring of 4 buffers; while tile i is
//    computed, tiles i+1 .. i+3 are resident or in flight (about 110 KB per
//    CU, enough to cover HBM latency at full bandwidth).  One barrier per tile;
//  * a cached row is 72 chunks of 16 bytes; LDS holds the tile column major
//    (all 32 rows of a chunk together) with the two row halves of odd chunks
//    swapped, so that both the row reads of QK^T and the transposed reads of
//    PV hit distinct banks (layout below);
//  * all products are v_mfma_f32_16x16x32_bf16: a K of 32 lets one PV
//    product cover a whole tile, and two rows per lane keep the P^T operand
//    in registers.  (A version on v_mfma_f32_32x32x16_bf16, with half the
//    MFMA instructions and one row per lane, took 8% fewer cycles per tile,
//    but the chip's clock under that load dropped by as much: measured, no
//    net gain.)
//  * wave w owns 32 query rows as two blocks of 16 (hb = 0, 1).  Its query
//    rows stay in 144 VGPRs as the B operand for the whole piece.
//    S^T = K Q^T for the tile: 2 key blocks x 2 row blocks; lane l holds rows
//    16hb + l%16 and keys 16kb + 4(l/16) + 0..3, so the row maximum and sum
//    reduce over the four 16-lane groups (two lane swaps);
//  * online softmax in base 2 with a lazy reference: the output is rescaled
//    only when a row's maximum grows by more than 2^8;
//  * O^T = V^T P^T accumulates in 64 MFMA blocks of 16 columns x 16 rows
//    (256 registers, AGPR).  P^T is built in registers from the S^T lane
//    layout (K slot 8g + j of lane group g stands for key 4g + j, j < 4, and
//    key 16 + 4g + j - 4 otherwise); V^T comes straight from the same LDS
//    tile through ds_read_b64_tr_b16 in that key order (no second copy of V);
//  * the piece ends with out = O / l and lse = ln(sum) written either to the
//    final tensors (a request in one piece) or to a workspace partial.
// Combine kernel: per split request and row, lse = logsumexp over its pieces,
// out = sum_s exp(lse_s - lse) o_s (the flash-decoding merge).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <type_traits>
#include <utility>

#include "decode_fp8.h"
#include "mla_decode.h"
#include "plan_internal.h"
#include "abi_common.h"

namespace mla {
namespace {

#include "device_common.h"

constexpr int kRowBytes = 576 * 2;  // one cached token (HBM and LDS)
constexpr int kChunks = 72;         // 16-byte chunks per cached token
constexpr int kTile = 32;           // keys per tile
constexpr int kWaves = 4;
constexpr int kRowsPerBlock = 32 * kWaves;
constexpr int kStageBytes = kTile * kRowBytes;         // 36864
constexpr int kStages = 4;                             // LDS tile ring
constexpr int kSoftmaxSteps = 28;                      // pieces of the per-tile softmax
constexpr int kLoadsPerTile = kTile * kChunks / 64;     // 36 one-KB copies
constexpr int kLoadsPerWave = kLoadsPerTile / kWaves;  // 9
constexpr int kQSteps = 576 / 32;                      // 18 K steps of QK^T
constexpr int kNopeSteps = 512 / 32;                   // the first 16 come from c_kv
#ifndef MLA_QK_DEPTH
#define MLA_QK_DEPTH 1
#endif
#ifndef MLA_PV_DEPTH
#define MLA_PV_DEPTH 2
#endif
constexpr int kQkDepth = MLA_QK_DEPTH;  // K steps of LDS reads in flight ahead of the QK^T MFMAs
constexpr int kPvDepth = MLA_PV_DEPTH;  // column blocks of V^T reads in flight ahead of the PV MFMAs
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr float kMuFloor = -1e30f;         // subtracted reference of a row with no visible key yet
static_assert(kLoadsPerTile % kWaves == 0, "every wave issues the same number of copies");
static_assert(2 * kPvDepth <= 4, "the V^T prefetch reads fit the four slots of the last QK^T step");
static_assert(kLoadsPerWave - 5 + kSoftmaxSteps == 32, "PV gaps: 4 copies, then the softmax steps");

// LDS layout of a 32-key tile (36 KB), column major: the 16-byte chunk c
// (0..71) of key row t (0..31) sits at slot 32c + (t ^ 16(c & 1)).
// gfx950's LDS has 128 four-byte banks (512 bytes) and serves a 128-bit read
// 32 lanes at a time, so a read is conflict-free when each half wave covers
// 512 distinct bytes modulo 512.
//  * a 1 KB copy n fills slots 64n .. 64n+63: lane l brings chunk 2n + l/32 of
//    key row (l % 32) ^ 16(l / 32), so a lane's source row is the same for every
//    copy and the copies of a tile differ only by a constant offset;
//  * QK^T reads 16 consecutive key rows of one chunk per 16 lanes (256
//    contiguous bytes); a half wave reads chunks 2j and 2j + 1, which the
//    half swap puts 256 bytes apart modulo 512;
//  * PV's transposed reads take 8 rows x 2 chunks per half wave (8 bytes per
//    lane, 256 bytes per half wave), again in distinct banks.

// The S^T accumulators are pinned to VGPRs (the softmax reads them with VALU
// right away) while the output accumulators live in AGPRs; the compiler left to
// itself puts both in AGPRs and spills.  So the QK^T MFMA is issued as inline
// asm with a VGPR constraint.  The hazards the compiler cannot see inside the
// asm are handled here: the first step takes srcC = 0 (no VALU write of the
// accumulator right before an MFMA reads it; early clobber so the result does
// not share registers with an operand), and s_mfma_drain waits out the
// XDL-write -> VALU-read latency before anything reads the results.  No MFMA
// operand is written by VALU right before the MFMA (two wait states are
// needed); the operands come from LDS, global loads or much earlier VALU
// work, and the build's assembly is checked for the hazard.
__device__ __forceinline__ void s_mfma(f32x4& acc, const bf16x8& a, const bf16x8& b, bool first) {
  if (first)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ void s_mfma_drain(f32x4 (&acc)[4]) {
  asm volatile("s_nop 15\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
}

// The output accumulators O^T (64 blocks of 16x16 fp32 = 256 registers per
// lane) live in the physical AGPRs a[0:255]: block n = 2 * cb + hb (columns
// 16cb .. 16cb+15, row block hb) is a[4n : 4n+3].  Lane l of block n holds
// row 16hb + l%16, columns 16cb + 4(l/16) + 0..3.  They are only touched by
// inline asm that names them and lists them as clobbered, so the compiler
// never allocates them (left to itself it carries them through VGPRs around
// the rare rescale branch and spills the query rows).  Hazards the compiler
// cannot see are handled where the code runs:
//  * MFMA -> accvgpr_read of the results: o_drain waits 24 wait states;
//  * accvgpr_write (rescale) -> MFMA srcC: the whole softmax runs in between,
//    plus the s_nop in front of every MFMA.
template <int N>
struct OBlock;
template <int N>
__device__ __forceinline__ float o_get();
template <int N>
__device__ __forceinline__ void o_set(float x);
#include "agpr_tiles.inc"

// Zero all 256 accumulators (start of a piece).
template <int R>
__device__ __forceinline__ void o_zero_rec() {
  if constexpr (R < 256) {
    o_set<R>(0.f);
    o_zero_rec<R + 1>();
  }
}

// Multiply the accumulators of row block 0 by alpha0 and of row block 1 by
// alpha1 (register r belongs to block r / 4, row block (r / 4) % 2).
template <int R>
__device__ __forceinline__ void o_scale_rec(float alpha0, float alpha1) {
  if constexpr (R < 256) {
    o_set<R>(o_get<R>() * (((R >> 2) & 1) ? alpha1 : alpha0));
    o_scale_rec<R + 1>(alpha0, alpha1);
  }
}

__device__ __forceinline__ void o_scale_all(float alpha0, float alpha1) { o_scale_rec<0>(alpha0, alpha1); }

// Power-of-two form of the same update: O <- O * 2^e0 (row block 0) and
// O * 2^e1 (row block 1), exact, by v_ldexp_f32 (an add to the exponent that
// also handles zeros, subnormals and underflow).
template <int R>
__device__ __forceinline__ void o_ldexp_rec(int e0, int e1) {
  if constexpr (R < 256) {
    o_set<R>(__builtin_ldexpf(o_get<R>(), ((R >> 2) & 1) ? e1 : e0));
    o_ldexp_rec<R + 1>(e0, e1);
  }
}

// Wait out the MFMA write -> AGPR read latency before reading results.
__device__ __forceinline__ void o_drain() { asm volatile("s_nop 15\n\ts_nop 7" ::: "memory"); }


// Store the 32 blocks of row block HB, scaled: block (cb, HB) goes to
// dst[16cb .. 16cb+3] (dst already points at this lane's 4 columns).
template <int HB, int CB>
__device__ __forceinline__ void o_store_rec(float* dst, float inv) {
  if constexpr (CB < 32) {
    constexpr int r = 4 * (2 * CB + HB);
    f32x4 w = {o_get<r + 0>() * inv, o_get<r + 1>() * inv, o_get<r + 2>() * inv, o_get<r + 3>() * inv};
    store_wt(dst + 16 * CB, w);
    o_store_rec<HB, CB + 1>(dst, inv);
  }
}

// Largest |O| over the 32 blocks of row block HB held by this lane.
template <int HB, int CB>
__device__ __forceinline__ float o_absmax_rec(float m) {
  if constexpr (CB < 32) {
    constexpr int r = 4 * (2 * CB + HB);
    float a, b;
    asm volatile("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(a) : "v"(m), "v"(o_get<r + 0>()), "v"(o_get<r + 1>()));
    asm volatile("v_max3_f32 %0, %1, |%2|, |%3|" : "=v"(b) : "v"(a), "v"(o_get<r + 2>()), "v"(o_get<r + 3>()));
    return o_absmax_rec<HB, CB + 1>(b);
  }
  return m;
}

// Store row block HB as a half-precision partial O * c.  Column block pair
// (cb, cb+1) of a row is 32 consecutive values, lane group g's 8 of them at
// [8g, 8g+8): block (cb, HB) value i at dst[16cb + i], block (cb+1, HB) value
// i at dst[16cb + 4 + i] (dst already points at this lane's group), so the
// four lanes of a row write 64 contiguous bytes per store.
template <int HB, int CB>
__device__ __forceinline__ void o_store_half_rec(_Float16* dst, float c) {
  if constexpr (CB < 32) {
    constexpr int r0 = 4 * (2 * CB + HB), r1 = 4 * (2 * (CB + 1) + HB);
    typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
    f16x8 w = {(_Float16)(o_get<r0 + 0>() * c), (_Float16)(o_get<r0 + 1>() * c), (_Float16)(o_get<r0 + 2>() * c),
               (_Float16)(o_get<r0 + 3>() * c), (_Float16)(o_get<r1 + 0>() * c), (_Float16)(o_get<r1 + 1>() * c),
               (_Float16)(o_get<r1 + 2>() * c), (_Float16)(o_get<r1 + 3>() * c)};
    store_wt(dst + 16 * CB, w);
    o_store_half_rec<HB, CB + 2>(dst, c);
  }
}

// Page ids a tile touches (uniform; at most 2 since pages hold >= 16 keys and
// tiles hold 32).  Out-of-range ids are replaced by page 0 so that a corrupt
// block table can never make the kernel read outside the cache.
struct TilePages {
  int first;
  int pg[2];
};

// POW2 selects the power-of-two form of the online softmax's reference (the
// running maximum rounded up to an integer in log2 units, so that O is
// rescaled by exact powers of two); rescale_events (may be NULL) counts, per
// wave, the tiles after which O was rescaled.
template <bool SINGLE_PAGE, bool POW2>
__global__ __launch_bounds__(64 * kWaves, 1) void decode_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const uint8_t* __restrict__ cache, int64_t num_pages,
    const int32_t* __restrict__ block_table, int32_t bt_stride,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ planned_lens,
    const Segment* __restrict__ segs, const WorkgroupRange* __restrict__ wgs,
    float scale_log2, int32_t rows, int32_t heads, int32_t q_len, int32_t page_log2, int32_t nrb,
    float* __restrict__ out, float* __restrict__ lse, uint16_t* __restrict__ ws_o,
    float* __restrict__ ws_lse, float* __restrict__ ws_f, uint32_t* __restrict__ rescale_events) {
  // 4 tile stages (144 KB); the query rows live in registers.
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages * kStageBytes];

  const WorkgroupRange wr = wgs[blockIdx.x];
  if (wr.seg_begin >= wr.seg_end) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4;  // 16-lane group: K slice of operands, row quad of results
  const int l16 = lane & 15;
  const int rb = wr.row_block;
  const int psize = 1 << page_log2;

  // This lane's two query rows: row block hb of the wave, row l16 in it.
  int row_local[2], row[2], jq[2];
  bool row_ok[2];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    row_local[hb] = wave * 32 + hb * 16 + l16;
    row[hb] = rb * kRowsPerBlock + row_local[hb];
    row_ok[hb] = row[hb] < rows;
    jq[hb] = row_ok[hb] ? row[hb] / heads : 0;  // query token of the row
  }
  // The wave's first row has the fewest visible keys; a wave with rows past
  // the end masks every tile.
  const int wave_row0 = rb * kRowsPerBlock + wave * 32;
  uint32_t n_rescale = 0;  // tiles after which this wave rescaled O (uniform)
  const bool wave_full = wave_row0 + 31 < rows;
  const int wave_jq0 = wave_row0 / heads;

  // Per-lane LDS byte offsets (within a stage) of the operand reads; the
  // remaining terms are compile-time offsets.
  // QK^T, A operand = key rows: key 16kb + l16, chunk 4ks + grp:
  //   qk_off0 + 2048 ks for key block 0; key block 1 sits in the other half
  //   of the chunk (odd chunks hold rows 16.. first): bit 8 flipped.
  const int qk_off0 = 512 * grp + 16 * l16 + 256 * (grp & 1);
  // PV, A operand = V^T via transposed reads.  Within 16-lane group grp, lane
  // l16 addresses key row 16rd + 4grp + l16/4, columns 16cb + 4(l16%4) .. +3
  // (chunk 2cb + (l16%4)/2, byte 8(l16%2)); the read hands it column 16cb + l16
  // of those 4 keys (K slots 4rd .. 4rd+3 of the group):
  //   pv_off0 + 1024 cb for rd = 0, in row half hsel of the chunk; rd = 1
  //   reads the other half (bit 8 flipped).
  const int hsel = (l16 >> 1) & 1;
  const int pv_off0 = 768 * hsel + 16 * (4 * grp + (l16 >> 2)) + 8 * (l16 & 1);
  // Tile copies: wave w issues copies n = 4i + w (i = 0..8) of a tile; lane l
  // reads key row dma_row, bytes dma_col + 128 i of it.
  const int dma_row = (lane & 31) ^ (16 * (lane >> 5));
  const int dma_col = 16 * (lane >> 5) + 32 * wave;

  for (int si = wr.seg_begin; si < wr.seg_end; ++si) {
    const Segment sg = segs[si];
    const int b = sg.b, kv0 = sg.kv_begin, kv1 = sg.kv_end;
    const int32_t* bt_row = block_table + (int64_t)b * bt_stride;

    // The piece's first 64 block-table entries sit in one register, lane i
    // holding page first_pg + i (lanes past the piece repeat its last page),
    // loaded once per piece; the tile loop reads them with readlane, so no
    // memory load (and no wait on one) sits between the LDS reads of the
    // loop.  Pages beyond the first 64 of a piece come from scalar loads.
    // The load is issued before the query loads; it is waited for (vmcnt in
    // order) once only the query loads are still in flight.
    const int first_pg = kv0 >> page_log2;
    const int last_pg = (kv1 - 1) >> page_log2;
    int pg_lane = load4(bt_row + min(first_pg + lane, last_pg));

    // Query rows as the B operand, all in registers: q[16hb + ks] holds
    // dims 32ks + 8grp .. +7 of row hb (the c_kv part, steps 0..15) and
    // qr[e][hb] dims 32e + 8grp .. +7 of its rope part (steps 16 + e).  Rows
    // past the end load row 0: their scores are masked and they are never
    // stored.
    bf16x8 q[2 * kNopeSteps];
    bf16x8 qr[2][2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int qrow = row_ok[hb] ? row[hb] : 0;
      const uint16_t* qn = q_nope + ((int64_t)b * rows + qrow) * 512 + 8 * grp;
      const uint16_t* qp = q_pe + ((int64_t)b * rows + qrow) * 64 + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < kNopeSteps; ++ks) q[kNopeSteps * hb + ks] = load16(qn + 32 * ks);
#pragma unroll
      for (int e = 0; e < 2; ++e) qr[e][hb] = load16(qp + 32 * e);
    }

    const int L = seq_lens[b];
    const bool bad_len = (L != planned_lens[b]);

    // Keys each of this lane's rows may see inside the piece: [kv0, lim).
    int lim[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) lim[hb] = row_ok[hb] ? min(kv1, L - q_len + 1 + jq[hb]) : kv0;
    // A tile starting at key tb needs masking iff tb + kTile > lim_wave.
    // uniform: the per-tile masking test is then a scalar compare and branch
    const int lim_wave = __builtin_amdgcn_readfirstlane(wave_full ? min(kv1, L - q_len + 1 + wave_jq0) : kv0);

    // Block-table entries of a tile (checked when used).
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
      TilePages tp;
      tp.first = tb >> page_log2;
      const int last = (min(tb + kTile, kv1) - 1) >> page_log2;
      tp.pg[0] = page_at(tp.first);
      tp.pg[1] = SINGLE_PAGE ? tp.pg[0] : page_at(min(tp.first + 1, last));
      return tp;
    };
    // A page id outside [0, num_pages) is never followed: page 0 is read
    // instead, and the piece's rows end as NaN (bad_pg), like a length mismatch.
    // page ids are int32: a pool of 2^31 pages or more holds every id
    const uint32_t num_pages_u32 = (uint32_t)min(num_pages, (int64_t)0x80000000LL);
    bool bad_pg = false;
    auto checked = [&](TilePages tp) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const bool ok = (uint32_t)tp.pg[k] < num_pages_u32;  // scalar compare (ids are uniform)
        bad_pg = bad_pg || !ok;
        tp.pg[k] = ok ? tp.pg[k] : 0;
      }
      return tp;
    };

    // Per-tile source of this lane's copies.  Key rows past the piece are
    // clamped to its last key: their scores are masked, and the copy stays
    // inside the request's pages with finite values for PV.
    struct TileSrc {
      const uint8_t* base;  // uniform (one page per tile)
      uint32_t off;         // per lane
      const uint8_t* ptr;   // per lane (two pages per tile)
    };
    auto tile_src = [&](int tb, const TilePages& tp) {
      TileSrc ts;
      const int tok = min(tb + dma_row, kv1 - 1);
      if (SINGLE_PAGE) {
        ts.base = cache + ((int64_t)tp.pg[0] << page_log2) * kRowBytes;
        ts.off = (uint32_t)((tok & (psize - 1)) * kRowBytes + dma_col);
        ts.ptr = nullptr;
      } else {
        const int page = ((tok >> page_log2) == tp.first) ? tp.pg[0] : tp.pg[1];
        ts.base = nullptr;
        ts.off = 0;
        ts.ptr = cache + (((int64_t)page << page_log2) + (tok & (psize - 1))) * kRowBytes + dma_col;
      }
      return ts;
    };
    // Copy i (0..8) of this wave for a tile into `stage`.
    auto dma = [&](auto ic, const TileSrc& ts, uint8_t* stage) {
      constexpr int i = decltype(ic)::value;
      const uint32_t dst = lds_addr(stage) + (uint32_t)((4 * i + wave) * 1024 - 128 * i);
      if (SINGLE_PAGE)
        dma16_saddr<128 * i>(ts.base, ts.off, dst);
      else
        dma16_off<128 * i>(ts.ptr, dst);
    };
    auto dma_all = [&](const TileSrc& ts, uint8_t* stage) {
      static_for<kLoadsPerWave>([&](auto ic) { dma(ic, ts, stage); });
    };

    const int ntiles = (kv1 - kv0 + kTile - 1) / kTile;

    // All waves must be done with the previous piece's tiles before the first
    // tiles of this one land in LDS.
    __syncthreads();

    // Page ids have landed once only the 36 query loads are in flight.
    wait_vmem<2 * kNopeSteps + 4>();  // 32 c_kv + 4 rope
    asm volatile("" : "+v"(pg_lane));

    const int last_tile = ntiles - 1;
    dma_all(tile_src(kv0, checked(fetch_pages(kv0))), smem);

    // Software pipeline over tiles (4 LDS stages).  Iteration `it`:
    //   QK^T of tile it+1, with the copies of tile it+3 issued between its
    //   MFMAs (into the stage tile it-1 used);
    //   PV of tile it, with the softmax of tile it+1 (mask, row max, lazy
    //   reference update, P) issued between its MFMAs;
    //   the rare rescale of O when a row's reference moved.
    // Tiles it and it+1 are resident, it+2 and it+3 in flight.  Every
    // iteration issues exactly one tile of copies (past the end of the piece
    // it repeats the last tile into a stage nobody reads), so every wait below
    // has a fixed count.
#pragma unroll
    for (int st = 1; st < 3; ++st) {
      const int ti = min(st, last_tile);
      const int tb_c = kv0 + ti * kTile;
      dma_all(tile_src(tb_c, checked(fetch_pages(tb_c))), smem + st * kStageBytes);
    }
    TilePages pg_raw = fetch_pages(kv0 + min(3, last_tile) * kTile);

    // QK^T of one tile: acc[2kb + hb] = S^T block (keys 16kb.., rows 16hb..).
    // `extra(k)` (k = 4ks + j) is called between the MFMAs so that
    // independent work issues while the matrix pipe runs; `tail(j)` before
    // MFMA j of the last step (the next phase's first LDS reads).  With
    // `drain`, the results are readable by VALU on return; without, the
    // caller keeps >= 19 instructions between the last MFMA and any VALU
    // access of acc (checked on the assembly).
    // One wave issues at most one LDS read per MFMA slot: a second read
    // right behind the first waits for the LDS issue port and holds back the
    // next MFMA, so the reads of a step are spread over its four slots.
    auto qk_tile = [&](const uint8_t* kb, f32x4(&acc)[4], auto&& extra, auto&& tail, bool drain) {
      constexpr int D = kQkDepth;
      bf16x8 a[D + 1][2];
      // Stage bases are multiples of 512 bytes: bit 8 of the sum is the lane's.
      const uint32_t k0 = lds_addr(kb) + qk_off0, k1 = k0 ^ 256u;
      // Read of step ks issued in slot j: key block 0 (j = 0), key block 1
      // (j = 2); slots 1 and 3 issue none.
      auto read = [&](int ks, int j) {
        if (j == 0) {
          a[ks % (D + 1)][0] = *LDS_AS(const bf16x8, (uintptr_t)(k0 + 2048 * ks));
        } else if (j == 2) {
          a[ks % (D + 1)][1] = *LDS_AS(const bf16x8, (uintptr_t)(k1 + 2048 * ks));
        }
      };
#pragma unroll
      for (int d = 0; d < D; ++d)
#pragma unroll
        for (int j = 0; j < 4; ++j) read(d, j);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < kQSteps; ++ks) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (ks + D < kQSteps) read(ks + D, j);
          if (ks == kQSteps - 1) tail(j);
          extra(4 * ks + j);
          const bf16x8& bq = ks < kNopeSteps ? q[kNopeSteps * (j & 1) + ks] : qr[ks - kNopeSteps][j & 1];
          s_mfma(acc[j], a[ks % (D + 1)][j >> 1], bq, ks == 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (drain) s_mfma_drain(acc);
    };

    // O^T += V^T P^T for one tile, V^T read transposed from its stage (two
    // reads per column block, rd = 0 and 1, one per MFMA slot).
    // pv_prefetch(i) issues read i (column block i/2, rd i%2) of the first
    // kPvDepth column blocks (it runs inside the previous phase); pv_run does
    // the 32 column blocks and calls `extra(cb)` between the two MFMAs of each.
    constexpr int DV = kPvDepth;
    struct PvBase {
      uint32_t r0, r1;  // LDS addresses of the rd = 0 and rd = 1 reads of column block 0
    };
    auto pv_base = [&](const uint8_t* kb) {
      const uint32_t r0 = lds_addr(kb) + pv_off0;
      return PvBase{r0, r0 ^ 256u};
    };
    auto read_v = [&](const PvBase& vb, int cb, int rd) {
      return __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(i16x4, (uintptr_t)((rd ? vb.r1 : vb.r0) + 1024 * cb)));
    };
    auto pv_prefetch = [&](const PvBase& vb, i16x4 (&v)[DV + 1][2], int i) {
      v[i >> 1][i & 1] = read_v(vb, i >> 1, i & 1);
    };
    auto pv_run = [&](const PvBase& vb, const bf16x8 (&pb)[2], i16x4 (&v)[DV + 1][2], auto&& extra) {
      static_for<32>([&](auto cbc) {
        constexpr int cb = decltype(cbc)::value;
        constexpr int nb = (cb + DV) % (DV + 1), b = cb % (DV + 1);
        if constexpr (cb + DV < 32) v[nb][0] = read_v(vb, cb + DV, 0);
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[b][0], v[b][1], 0, 1, 2, 3, 4, 5, 6, 7));
        OBlock<2 * cb + 0>::mfma(va, pb[0]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (cb + DV < 32) v[nb][1] = read_v(vb, cb + DV, 1);
        extra(cb);
        OBlock<2 * cb + 1>::mfma(va, pb[1]);
        __builtin_amdgcn_sched_barrier(0);
      });
    };

    // ---- online softmax state (base 2, lazy reference) ----
    // m_ref: reference max per row block (log2 units), the same in the four
    // lanes of a row; l_part: this lane's share of the running sum.
    float m_ref[2] = {-INFINITY, -INFINITY};
    float l_part[2] = {0.f, 0.f};
    float l_wt[2] = {0.f, 0.f};  // this lane's share of the sum of the bf16 weights
    const bf16x2 kOnes2 = {(__bf16)1.f, (__bf16)1.f};
    float alpha[2] = {1.f, 1.f};
    bool any_scale = false;
    float mx[2], mu[2] = {kMuFloor, kMuFloor};
    bool ref_check = true;  // some row of the wave may move its reference this tile
    bf16x2 pw[2][4];  // P^T operand under construction: K slots 2m, 2m+1
    float p_even = 0.f;
    float xt[2];  // exponent of the element whose exp comes next

    // Softmax of one tile of raw scores s (s[2kb + hb][i] = key tb_s + 16kb +
    // 4grp + i, row block hb), as kSoftmaxSteps short steps so that it can be
    // spread between MFMAs:
    //   0-3: mask block (kb, hb)'s keys past the row's limit (only on tiles
    //        that need it), 4: both row blocks' max over this lane's keys and
    //        whether any lane of the wave passes its row's threshold,
    //   5: only then (after fewer than one tile in a thousand, measured): max
    //      over the 4 lane groups and the reference update (a row moves its
    //      reference only when its maximum grows by more than
    //      kRescaleThreshold; the first finite maximum needs no rescale
    //      because nothing has been accumulated yet); 6-10: nothing,
    //   11-27: p = 2^(s * scale - mu), running sum, bf16 pairs of P^T (K slot
    //      j of row block hb is s[2(j/4) + hb][j%4]); software-pipelined so
    //      that a step's exp never waits on the same step's fma.
    auto softmax_step = [&](int step, f32x4(&s)[4], int need_mask, int tb_s) {
      if (step < 4) {
        const int kbk = step >> 1, hb = step & 1;
        if (need_mask) {  // uniform (scalar compare of uniform limits): a scalar branch
          // Keys left of the row's limit: lim - (this lane's first key), so
          // that the per-key test is one compare against a constant; the
          // empty asm keeps the subtraction inside the branch.
          int room = lim[hb] - (tb_s + 16 * kbk + 4 * grp);
          asm volatile("" : "+v"(room));
#pragma unroll
          for (int i = 0; i < 4; ++i) s[2 * kbk + hb][i] = i < room ? s[2 * kbk + hb][i] : -INFINITY;
        }
      } else if (step == 4) {
        bool exceed = false;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const f32x4& x0 = s[hb];
          const f32x4& x1 = s[2 + hb];
          mx[hb] = max3(max3(x0[0], x0[1], x0[2]), max3(x0[3], x1[0], x1[1]), max3(x1[2], x1[3], x1[3]));
          exceed = exceed || (mx[hb] * scale_log2 > m_ref[hb] + kRescaleThreshold);
        }
        // A row's reference can only move if the maximum of one of its
        // lanes' keys passes it by the threshold (the row maximum is one of
        // them, and rounding the product is monotonic); otherwise steps 5-10
        // would leave every reference and sum as it is (alpha = 2^0), so the
        // wave skips them.
        ref_check = __builtin_amdgcn_ballot_w64(exceed) != 0;
      } else if (step < 11) {
        if (step == 5 && ref_check) {
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) mx[hb] = group_max16(group_max32(mx[hb]));
          // mu = max(m_ref, kMuFloor) is the reference actually subtracted,
          // so alpha = 2^(mu_old - mu_new) needs no case for -inf: it is 1
          // without an update and 0 for a row's first finite maximum (when
          // nothing has been accumulated for that row).
#pragma unroll
          for (int hb = 0; hb < 2; ++hb) {
            const float m = mx[hb] * scale_log2;
            const bool upd = m > m_ref[hb] + kRescaleThreshold;
            const float m_new = upd ? (POW2 ? __builtin_ceilf(m) : m) : m_ref[hb];
            const float mu_new = fmaxf(m_new, kMuFloor);
            if constexpr (POW2) {
              // alpha holds the integer exponent mu - mu_new <= 0 (clamped:
              // a first finite maximum scales a sum that is still 0).
              alpha[hb] = fmaxf(mu[hb] - mu_new, -256.f);
              l_part[hb] = __builtin_ldexpf(l_part[hb], (int)alpha[hb]);
              l_wt[hb] = __builtin_ldexpf(l_wt[hb], (int)alpha[hb]);
            } else {
              alpha[hb] = __builtin_amdgcn_exp2f(mu[hb] - mu_new);
              l_part[hb] *= alpha[hb];
              l_wt[hb] *= alpha[hb];
            }
            any_scale = any_scale || (upd && mu[hb] > kMuFloor);
            m_ref[hb] = m_new;
            mu[hb] = mu_new;
          }
        }
      } else if (step < kSoftmaxSteps) {
        const int j = step - 11;  // 0..16: exp of element j-1, fma of element j
        if (j >= 1) {
          const int k = j - 1, hb = k >> 3, kk = k & 7;
          const float p = __builtin_amdgcn_exp2f(xt[k & 1]);
          l_part[hb] += p;
          if (kk & 1) {
            pw[hb][kk >> 1] = bf16x2{(__bf16)p_even, (__bf16)p};
            asm volatile("" : "+v"(pw[hb][kk >> 1]));  // pack now, not at the end
            // The bf16 weights PV multiplies by, summed (one dot2 per pair):
            // O is divided by this sum, so that a row stays a weighted mean
            // of V rows under one set of weights (a row dominated by one key
            // returns that key's V row, whatever the rounding of its weight);
            // lse uses the exact sum.
            l_wt[hb] = __builtin_amdgcn_fdot2_f32_bf16(pw[hb][kk >> 1], kOnes2, l_wt[hb], false);
          } else {
            p_even = p;
          }
        }
        if (j < 16) {
          const int hb = j >> 3, jj = j & 7;
          xt[j & 1] = __builtin_fmaf(s[2 * (jj >> 2) + hb][jj & 3], scale_log2, -mu[hb]);
        }
      }
    };
    auto pack_half = [&](bf16x8 (&pb)[2], int hb) {
      pb[hb] = __builtin_shufflevector(__builtin_shufflevector(pw[hb][0], pw[hb][1], 0, 1, 2, 3),
                                       __builtin_shufflevector(pw[hb][2], pw[hb][3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5,
                                       6, 7);
    };
    auto pack_p = [&](bf16x8 (&pb)[2]) {
      pack_half(pb, 0);
      pack_half(pb, 1);
    };

    // The query rows and tile 0 (issued before tiles 1 and 2) have landed
    // once two tiles of copies are still in flight.  The empty asm statements tie the
    // query registers to this point: the loads fill them asynchronously, so
    // nothing may read, copy or reuse them before the wait.
    {
      wait_vmem<2 * kLoadsPerWave>();
      asm volatile("" : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]), "+v"(q[4]), "+v"(q[5]), "+v"(q[6]),
                   "+v"(q[7]));
      asm volatile("" : "+v"(q[8]), "+v"(q[9]), "+v"(q[10]), "+v"(q[11]), "+v"(q[12]), "+v"(q[13]),
                   "+v"(q[14]), "+v"(q[15]));
      asm volatile("" : "+v"(q[16]), "+v"(q[17]), "+v"(q[18]), "+v"(q[19]), "+v"(q[20]), "+v"(q[21]),
                   "+v"(q[22]), "+v"(q[23]));
      asm volatile("" : "+v"(q[24]), "+v"(q[25]), "+v"(q[26]), "+v"(q[27]), "+v"(q[28]), "+v"(q[29]),
                   "+v"(q[30]), "+v"(q[31]));
      asm volatile("" : "+v"(qr[0][0]), "+v"(qr[0][1]), "+v"(qr[1][0]), "+v"(qr[1][1]));
      __syncthreads();
    }
    o_zero_rec<0>();
    bf16x8 pb[2];
    {
      f32x4 s0[4];
      qk_tile(smem, s0, [](int) {}, [](int) {}, true);
      const int nm0 = kv0 + kTile > lim_wave ? 1 : 0;  // uniform (scalar)
#pragma unroll
      for (int step = 0; step < kSoftmaxSteps; ++step) softmax_step(step, s0, nm0, kv0);
      pack_p(pb);
      any_scale = false;  // nothing accumulated yet
    }

    for (int it = 0; it < ntiles; ++it) {
      const bool has_next = it + 1 < ntiles;
      // Tile it+1 has landed once only tile it+2's copies of this wave are in
      // flight; the barrier publishes every wave's part and frees the stage of
      // tile it-1 for the next copy.
      wait_vmem<kLoadsPerWave>();
      __syncthreads();

      const int tb = kv0 + it * kTile;
      const PvBase vb = pv_base(smem + (it % kStages) * kStageBytes);     // tile it (PV)
      const uint8_t* kb_next = smem + ((it + 1) % kStages) * kStageBytes;  // tile it+1 (QK^T)
      const int nt = it + 3;                                               // tile to copy now
      const int tb_c = kv0 + min(nt, last_tile) * kTile;
      uint8_t* nbuf = smem + (nt % kStages) * kStageBytes;
      const TileSrc nsrc = tile_src(tb_c, checked(pg_raw));
      __builtin_amdgcn_sched_barrier(0);

      // ---- QK^T of tile it+1, copies of tile it+3 between its MFMAs ----
      // Copies 0..4 of tile it+3 go between QK^T MFMAs, copies 5..8 between
      // the first PV MFMAs (before the softmax steps start).
      auto copy_at = [&](int i) {
        static_for<kLoadsPerWave>([&](auto ic) {
          if (decltype(ic)::value == i) dma(ic, nsrc, nbuf);
        });
      };
      i16x4 v[DV + 1][2];
      f32x4 s_next[4];
      if (has_next) {
        // P of tile it (from the previous iteration's softmax) becomes the PV
        // operand between QK^T MFMAs, where the VALU is otherwise idle.
        qk_tile(
            kb_next, s_next,
            [&](int k) {
              if ((k & 15) == 4) copy_at(k >> 4);
              if (k == 10 || k == 26) pack_half(pb, k == 26);
            },
            [&](int j) {
              if (j < 2 * DV) pv_prefetch(vb, v, j);
            },
            false);
      } else {
        pack_p(pb);
        dma_all(nsrc, nbuf);
#pragma unroll
        for (int i = 0; i < 2 * DV; ++i) pv_prefetch(vb, v, i);
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- PV of tile it, softmax of tile it+1 between its MFMAs (from
      //      column block 4 on: by then the QK^T results are readable) ----
      if (has_next) {
        const int nm = tb + 2 * kTile > lim_wave ? 1 : 0;  // uniform (scalar)
        pv_run(vb, pb, v, [&](int cb) {
          if (cb < kLoadsPerWave - 5) {
            copy_at(5 + cb);
          } else {
            softmax_step(cb - (kLoadsPerWave - 5), s_next, nm, tb + kTile);
          }
        });
        // A row whose reference moved rescales everything accumulated so far
        // (tiles <= it).
        if (__any(any_scale)) {
          o_drain();
          if constexpr (POW2)
            o_ldexp_rec<0>((int)alpha[0], (int)alpha[1]);
          else
            o_scale_all(alpha[0], alpha[1]);
          ++n_rescale;
        }
        any_scale = false;
      } else {
        pv_run(vb, pb, v, [](int) {});
      }
      // Pages of the tile the next iteration copies.  Looked up here, after
      // the last LDS read of the iteration: a scalar load in flight would make
      // every LDS wait until it lands a full wait.
      pg_raw = fetch_pages(kv0 + min(nt + 1, last_tile) * kTile);
    }

    // The repeated copies past the end of the piece must land before the next
    // piece reuses their stages.
    wait_vmem<0>();

    // ---- epilogue: normalize and store (final output or a workspace partial) ----
    o_drain();
    float l_tot[2], lse_v[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      l_tot[hb] = group_sum(l_part[hb]);
      lse_v[hb] = l_tot[hb] > 0.f ? (m_ref[hb] + __builtin_amdgcn_logf(l_tot[hb])) * kLn2 : -INFINITY;
      l_tot[hb] = group_sum(l_wt[hb]);  // O's divisor from here on
      if (bad_len || bad_pg) lse_v[hb] = NAN;
    }
    if (sg.partial < 0) {
      // Whole request: out = O / l in fp32.
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float inv = l_tot[hb] > 0.f ? 1.f / l_tot[hb] : 0.f;
        if (bad_len || bad_pg) inv = NAN;
        if (!row_ok[hb]) continue;
        // Computed here, not hoisted above the tile loop (it would hold two
        // registers through the loop).
        int r = row[hb];
        asm volatile("" : "+v"(r));
        const int64_t oi = (int64_t)b * rows + r;
        float* dst = out + oi * 512 + 4 * grp;
        if (hb == 0)
          o_store_rec<0, 0>(dst, inv);
        else
          o_store_rec<1, 0>(dst, inv);
        if (grp == 0) lse[oi] = lse_v[hb];
      }
    } else {
      // Piece of a split request: the partial o = O / l is stored as O * 2^(15-e)
      // in fp16, e the binary exponent of the row's largest |O| (so every
      // stored value is below 2^15 in magnitude and keeps 11 bits), with
      // f = 2^(e-15) / l and lse beside it: o = stored * f.  Within a row,
      // position 32 (cb / 2) + 8 grp + 4 (cb % 2) + i holds column
      // 16 cb + 4 grp + i.
      const int64_t slot = (int64_t)sg.partial * nrb + rb;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float amax = hb == 0 ? o_absmax_rec<0, 0>(0.f) : o_absmax_rec<1, 0>(0.f);
        amax = group_max16(group_max32(amax));
        const int e = max(__builtin_amdgcn_frexp_expf(amax), -110);
        const float c = __builtin_ldexpf(1.f, 15 - e);
        float f = l_tot[hb] > 0.f ? __builtin_ldexpf(1.f / l_tot[hb], e - 15) : 0.f;
        if (bad_len || bad_pg) f = NAN;
        if (!row_ok[hb]) continue;
        const int64_t ri = slot * kRowsPerBlock + row_local[hb];
        _Float16* dst = reinterpret_cast<_Float16*>(ws_o) + ri * 512 + 8 * grp;
        if (hb == 0)
          o_store_half_rec<0, 0>(dst, c);
        else
          o_store_half_rec<1, 0>(dst, c);
        if (grp == 0) {
          ws_lse[ri] = lse_v[hb];
          ws_f[ri] = f;
        }
      }
    }
  }
  // After the last piece: no tile copy is in flight any more.
  if (rescale_events != nullptr && n_rescale != 0 && lane == 0) atomicAdd(rescale_events, n_rescale);
}

// One workgroup = one row of one split request (the unit's row0).  Stored position 8l + e of a
// row (lane l) holds column 32(l/4) + 4(l%4) + e for e < 4 and
// 32(l/4) + 16 + 4(l%4) + e - 4 otherwise.  All waves derive
// lse = logsumexp_s lse_s for the row; the partial weights
// exp(lse_s - lse) f_s go to LDS in chunks of kCombineChunk; wave j (0..3)
// then sums the partials s = j, j+4, ... of the chunk, kCombineBatch loads at
// a time, and the four waves' sums meet in LDS.
constexpr int kCombineChunk = 256;
constexpr int kCombineBatch = 16;
__global__ __launch_bounds__(256) void combine_kernel(const CombineUnit* __restrict__ units,
                                                       const uint16_t* __restrict__ ws_o,
                                                       const float* __restrict__ ws_lse,
                                                       const float* __restrict__ ws_f, int32_t rows, int32_t rpb,
                                                       int32_t nrb, float* __restrict__ out,
                                                       float* __restrict__ lse) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  __shared__ float wts[kCombineChunk];
  __shared__ f32x4 red[3][64][2];
  const CombineUnit job = units[blockIdx.x];
  if (job.n == 0) return;
  const int row = job.row0;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int rb = row / rpb, rl = row - rb * rpb;
  auto ri_of = [&](int s) { return ((int64_t)(job.p0 + s) * nrb + rb) * rpb + rl; };

  // The partials' lse values, four per lane in flight at once (indices past
  // the end load the last one again and are masked).
  float m = -INFINITY;
  bool any_nan = false;  // fmaxf drops NaN; a NaN partial (length mismatch) must stay loud
  for (int s0 = 0; s0 < job.n; s0 += 256) {
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = ws_lse[ri_of(min(s0 + lane + 64 * i, job.n - 1))];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (s0 + lane + 64 * i < job.n) {
        any_nan |= (x[i] != x[i]);
        m = fmaxf(m, x[i]);
      }
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  any_nan = __any(any_nan);
  float z = 0.f;
  if (m != -INFINITY)
    for (int s0 = 0; s0 < job.n; s0 += 256) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = ws_lse[ri_of(min(s0 + lane + 64 * i, job.n - 1))];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (s0 + lane + 64 * i < job.n) z += __expf(x[i] - m);
    }
  for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
  const float lse_v = any_nan ? NAN : (m == -INFINITY ? -INFINITY : m + __logf(z));
  const bool live = !any_nan && m != -INFINITY;

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  if (live) {
    for (int c0 = 0; c0 < job.n; c0 += kCombineChunk) {
      const int cn = min(kCombineChunk, job.n - c0);
      if (threadIdx.x < cn) {
        const int64_t ri = ri_of(c0 + threadIdx.x);
        wts[threadIdx.x] = __expf(ws_lse[ri] - lse_v) * ws_f[ri];
      }
      __syncthreads();
      // kCombineBatch partials per wave in flight at once (past the chunk's
      // end the last one is loaded again with weight 0), so a wave's share
      // of the chunk costs a few round trips, not one per partial.
      for (int k0 = wv; k0 < cn; k0 += 4 * kCombineBatch) {
        f16x8 v[kCombineBatch];
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
          const int k = min(k0 + 4 * i, cn - 1);
          v[i] = *reinterpret_cast<const f16x8*>(ws_o + ri_of(c0 + k) * 512 + 8 * lane);
        }
#pragma unroll
        for (int i = 0; i < kCombineBatch; ++i) {
          const int k = k0 + 4 * i;
          const float w = k < cn ? wts[k] : 0.f;
          acc0 += w * f32x4{(float)v[i][0], (float)v[i][1], (float)v[i][2], (float)v[i][3]};
          acc1 += w * f32x4{(float)v[i][4], (float)v[i][5], (float)v[i][6], (float)v[i][7]};
        }
      }
      __syncthreads();
    }
  }
  if (wv > 0) {
    red[wv - 1][lane][0] = acc0;
    red[wv - 1][lane][1] = acc1;
  }
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      acc0 += red[j][lane][0];
      acc1 += red[j][lane][1];
    }
    if (any_nan) {
      acc0 = f32x4{NAN, NAN, NAN, NAN};
      acc1 = acc0;
    }
    float* dst = out + ((int64_t)job.b * rows + row) * 512 + 32 * (lane >> 2) + 4 * (lane & 3);
    *reinterpret_cast<f32x4*>(dst) = acc0;
    *reinterpret_cast<f32x4*>(dst + 16) = acc1;
    if (lane == 0) lse[(int64_t)job.b * rows + row] = lse_v;
  }
}

// Combine for requests split into at most kCombineSmallMax pieces: one wave
// per row (kCombineSmallRows rows per workgroup, from the unit's row0).  Lane l owns stored positions 8l .. 8l+7 (as
// in combine_kernel); every partial value of the row and the per-partial lse
// and scale (lane s holds partial s) are loaded at once, so the row costs one
// memory round trip.  Weights exp(lse_s - lse) f_s are broadcast from lane s.
__global__ __launch_bounds__(64 * kCombineSmallRows) void combine_small_kernel(const CombineUnit* __restrict__ units,
                                                             const uint16_t* __restrict__ ws_o,
                                                             const float* __restrict__ ws_lse,
                                                             const float* __restrict__ ws_f, int32_t rows,
                                                             int32_t rpb, int32_t nrb, float* __restrict__ out,
                                                             float* __restrict__ lse) {
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  const CombineUnit job = units[blockIdx.x];
  const int lane = threadIdx.x & 63;
  const int row = job.row0 + (threadIdx.x >> 6);
  if (job.n == 0 || row >= rows) return;
  const int rb = row / rpb, rl = row - rb * rpb;
  auto ri_of = [&](int s) { return ((int64_t)(job.p0 + s) * nrb + rb) * rpb + rl; };
  const int n = job.n;  // <= kCombineSmallMax (checked on the host)

  f16x8 v[kCombineSmallMax];
#pragma unroll
  for (int s = 0; s < kCombineSmallMax; ++s)
    if (s < n) v[s] = *reinterpret_cast<const f16x8*>(ws_o + ri_of(s) * 512 + 8 * lane);
  const float lse_s = lane < n ? ws_lse[ri_of(lane)] : -INFINITY;
  const float f_s = lane < n ? ws_f[ri_of(lane)] : 0.f;

  float m = lse_s;
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const bool any_nan = __any(lse_s != lse_s);  // fmaxf drops NaN; a NaN partial must stay loud
  float z = (m != -INFINITY && lane < n) ? __expf(lse_s - m) : 0.f;
  for (int o = 32; o > 0; o >>= 1) z += __shfl_xor(z, o);
  const float lse_v = any_nan ? NAN : (m == -INFINITY ? -INFINITY : m + __logf(z));
  const bool live = !any_nan && m != -INFINITY;
  const float w_s = (live && lane < n) ? __expf(lse_s - lse_v) * f_s : 0.f;

  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kCombineSmallMax; ++s) {
    if (s < n) {
      const float w = __shfl(w_s, s);
      acc0 += w * f32x4{(float)v[s][0], (float)v[s][1], (float)v[s][2], (float)v[s][3]};
      acc1 += w * f32x4{(float)v[s][4], (float)v[s][5], (float)v[s][6], (float)v[s][7]};
    }
  }
  if (any_nan) {
    acc0 = f32x4{NAN, NAN, NAN, NAN};
    acc1 = acc0;
  }
  float* dst = out + ((int64_t)job.b * rows + row) * 512 + 32 * (lane >> 2) + 4 * (lane & 3);
  *reinterpret_cast<f32x4*>(dst) = acc0;
  *reinterpret_cast<f32x4*>(dst + 16) = acc1;
  if (lane == 0) lse[(int64_t)job.b * rows + row] = lse_v;
}

}  // namespace
}  // namespace mla

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------

// Device memory of mla_decode_noalloc: the partial outputs of split requests
// live in this array instead of a caller-provided workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// the name is only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is ever passed
// to a kernel.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];


struct mla_plan {
  mla::PlanData d;
  int32_t variant = 1;  // planner variant (1: bf16 kernel, 2: FP8 kernel)
  // Device schedule: segs | wgs | combine units | planned lens, each region
  // sized for the largest schedule any lengths can give at this batch, query
  // length, head count and CU count, so that an update never reallocates.
  void* dev = nullptr;
  size_t off_segs = 0, off_wgs = 0, off_units = 0, off_lens = 0, total = 0;
  size_t cap_segs = 0, cap_wgs = 0, cap_units = 0;
  void* stage = nullptr;        // pinned host copy of the schedule (source of the uploads)
  hipEvent_t staged = nullptr;  // recorded after the last upload from `stage`
  int device = -1;
};

namespace {

thread_local std::string g_last_error;

mla_status fail(mla_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

mla_status hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Writes schedule d into the plan's pinned staging copy (the region layout
// is fixed at creation).
void stage_schedule(mla_plan* p, const mla::PlanData& d) {
  char* h = static_cast<char*>(p->stage);
  std::memcpy(h + p->off_segs, d.segs.data(), d.segs.size() * sizeof(mla::Segment));
  std::memcpy(h + p->off_wgs, d.wgs.data(), d.wgs.size() * sizeof(mla::WorkgroupRange));
  if (!d.cunits.empty()) std::memcpy(h + p->off_units, d.cunits.data(), d.cunits.size() * sizeof(mla::CombineUnit));
  std::memcpy(h + p->off_lens, d.lens.data(), d.lens.size() * sizeof(int32_t));
}

void release_plan(mla_plan* p) {
  if (p->staged) (void)hipEventSynchronize(p->staged);
  if (p->dev) (void)hipFree(p->dev);
  if (p->stage) (void)hipHostFree(p->stage);
  if (p->staged) (void)hipEventDestroy(p->staged);
  delete p;
}

mla_status make_plan(const int32_t* seq_lens_host, int32_t batch, int32_t q_len, int32_t num_heads,
                     int32_t page_size, int32_t num_cus, mla_plan** plan_out, bool upload, int32_t variant = 1) {
  if (!plan_out) return fail(MLA_ERR_INVALID_ARGUMENT, "plan_out is NULL");
  *plan_out = nullptr;
  if (!seq_lens_host) return fail(MLA_ERR_INVALID_ARGUMENT, "seq_lens_host is NULL");
  int device = -1;
  if (num_cus == 0 && upload) {
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    num_cus = cus;
  }
  if (num_cus <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "num_cus must be > 0 (or 0 to query the device)");
  mla_plan* p = new (std::nothrow) mla_plan();
  if (!p) return fail(MLA_ERR_OUT_OF_MEMORY, "host allocation failed");
  std::string err;
  int rc;
  try {
    mla::PlanTuning tuning;
    tuning.variant = variant;
    rc = mla::build_plan(seq_lens_host, batch, q_len, num_heads, page_size, num_cus, tuning, &p->d, &err);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(MLA_ERR_OUT_OF_MEMORY, "host allocation failed while planning");
  }
  if (rc != 0) {
    delete p;
    return fail((mla_status)rc, err);
  }
  p->variant = variant;
  if (upload) {
    if (device < 0) {
      hipError_t e = hipGetDevice(&device);
      if (e != hipSuccess) {
        delete p;
        return hip_fail(e, "hipGetDevice");
      }
    }
    p->device = device;
    const mla::PlanData& d = p->d;
    // Largest schedule at this shape: at most max_slots slots of nrb
    // workgroups, one piece per request plus one per slot boundary, the grid
    // rounded up to whole XCD blocks of row blocks, one combine unit per split
    // row (and padding to the XCD count).
    const int64_t max_slots = std::max<int64_t>(1, (int64_t)d.num_cus * d.v.wg_per_cu / d.nrb);
    p->cap_segs = std::max<size_t>(d.segs.size(), (size_t)(d.batch + max_slots));
    p->cap_wgs = std::max<size_t>(d.wgs.size(), (size_t)(max_slots * d.nrb + mla::kNumXcd * (d.nrb + 1)));
    p->cap_units = std::max<size_t>(d.cunits.size(), (size_t)d.batch * d.rows + mla::kNumXcd);
    p->off_segs = 0;
    p->off_wgs = align256(p->cap_segs * sizeof(mla::Segment));
    p->off_units = p->off_wgs + align256(p->cap_wgs * sizeof(mla::WorkgroupRange));
    p->off_lens = p->off_units + align256(p->cap_units * sizeof(mla::CombineUnit));
    p->total = p->off_lens + align256((size_t)d.batch * sizeof(int32_t));
    hipError_t e = hipMalloc(&p->dev, p->total);
    if (e == hipSuccess) e = hipHostMalloc(&p->stage, p->total, hipHostMallocDefault);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&p->staged, hipEventDisableTiming);
    if (e == hipSuccess) {
      stage_schedule(p, p->d);
      e = hipMemcpy(p->dev, p->stage, p->total, hipMemcpyHostToDevice);
    }
    if (e != hipSuccess) {
      release_plan(p);
      return e == hipErrorOutOfMemory ? fail(MLA_ERR_OUT_OF_MEMORY, "allocation of the plan schedule failed")
                                      : hip_fail(e, "upload of the plan schedule");
    }
  }
  *plan_out = p;
  g_last_error.clear();
  return MLA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Workspace checks shared by the entry points; splits it into the partial
// outputs (fp16), the partial lse and the partial scale factors.
struct Workspace {
  uint16_t* o = nullptr;
  float* lse = nullptr;
  float* f = nullptr;
};

mla_status check_workspace(const mla_plan* plan, void* workspace, size_t workspace_bytes, Workspace* ws) {
  const mla::PlanData& d = plan->d;
  const size_t need = mla::workspace_bytes(d);
  *ws = Workspace{};
  if (need == 0) return MLA_OK;
  if (!workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "workspace is NULL but the plan needs " + std::to_string(need) + " bytes");
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                "workspace has " + std::to_string(workspace_bytes) + " bytes, the plan needs " + std::to_string(need));
  if (!aligned(workspace, 256)) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  const mla::WorkspaceLayout lay = mla::workspace_layout(d);
  char* base = static_cast<char*>(workspace);
  ws->o = reinterpret_cast<uint16_t*>(base + lay.off_o);
  ws->lse = reinterpret_cast<float*>(base + lay.off_lse);
  ws->f = reinterpret_cast<float*>(base + lay.off_f);
  return MLA_OK;
}

// The plan's schedule lives on one device; refuse to run it from another.
mla_status check_device(const mla_plan* plan) {
  if (!plan->dev) return fail(MLA_ERR_INVALID_ARGUMENT, "plan was made by mla_decode_plan_host and cannot run");
  int device = -1;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (device != plan->device)
    return fail(MLA_ERR_INVALID_ARGUMENT, "the current device is not the one the plan was made on");
  return MLA_OK;
}

// Device address of `scratch` on `device` (the current device), looked up
// on the first call for that device and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

mla_status scratch_address(int device, void** addr) {
  if (device < 0 || device >= kMaxDevices) return fail(MLA_ERR_UNSUPPORTED, "device id beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[device]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the no-allocation scratch");
    if (!p) return fail(MLA_ERR_HIP, "hipGetSymbolAddress returned NULL for the no-allocation scratch");
    g_scratch_addr[device] = p;
  }
  *addr = g_scratch_addr[device];
  return MLA_OK;
}

template <bool SINGLE_PAGE, bool POW2>
hipError_t launch_decode(const mla_plan* plan, const void* q_nope, const void* q_pe, const void* cache,
                         int64_t num_pages, const int32_t* bt, int32_t bt_stride, const int32_t* seq_lens,
                         float scale_log2, float* out, float* lse, const Workspace& ws, uint32_t* rescale_events,
                         hipStream_t stream) {
  const mla::PlanData& d = plan->d;
  const char* base = static_cast<const char*>(plan->dev);
  int page_log2 = 0;
  while ((1 << page_log2) < d.page) ++page_log2;
  hipLaunchKernelGGL((mla::decode_kernel<SINGLE_PAGE, POW2>), dim3(d.grid), dim3(64 * mla::kWaves), 0, stream,
                     static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_pe),
                     static_cast<const uint8_t*>(cache), num_pages, bt, bt_stride, seq_lens,
                     reinterpret_cast<const int32_t*>(base + plan->off_lens),
                     reinterpret_cast<const mla::Segment*>(base + plan->off_segs),
                     reinterpret_cast<const mla::WorkgroupRange*>(base + plan->off_wgs), scale_log2, d.rows,
                     d.heads, d.q_len, page_log2, d.nrb, out, lse, ws.o, ws.lse, ws.f, rescale_events);
  return hipGetLastError();
}

}  // namespace

namespace mla {
mla_status abi_fail(mla_status s, const char* msg) { return fail(s, msg); }
mla_status abi_hip_fail(hipError_t e, const char* what) { return hip_fail(e, what); }
void abi_ok() { g_last_error.clear(); }
bool abi_aligned(const void* p, uintptr_t a) { return aligned(p, a); }
}  // namespace mla

extern "C" {

mla_status mla_decode_plan(const int32_t* seq_lens_host, int32_t batch, int32_t q_len, int32_t num_heads,
                           int32_t page_size, int32_t num_cus, mla_plan** plan_out) {
  return make_plan(seq_lens_host, batch, q_len, num_heads, page_size, num_cus, plan_out, true);
}

mla_status mla_decode_plan_host(const int32_t* seq_lens_host, int32_t batch, int32_t q_len, int32_t num_heads,
                                int32_t page_size, int32_t num_cus, mla_plan** plan_out) {
  return make_plan(seq_lens_host, batch, q_len, num_heads, page_size, num_cus, plan_out, false);
}

size_t mla_decode_workspace_bytes(const mla_plan* plan) { return plan ? mla::workspace_bytes(plan->d) : 0; }

void mla_decode_plan_destroy(mla_plan* plan) {
  if (plan) release_plan(plan);
}

mla_status mla_decode_plan_update(mla_plan* plan, const int32_t* seq_lens_host, void* stream) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!seq_lens_host) return fail(MLA_ERR_INVALID_ARGUMENT, "seq_lens_host is NULL");
  if (!plan->dev) return fail(MLA_ERR_INVALID_ARGUMENT, "plan was made by a _plan_host call and has no device schedule");
  mla_status st_dev = check_device(plan);
  if (st_dev != MLA_OK) return st_dev;
  const mla::PlanData& old = plan->d;
  mla::PlanData next;
  std::string err;
  int rc;
  try {
    mla::PlanTuning tuning;
    tuning.variant = plan->variant;
    rc = mla::build_plan(seq_lens_host, old.batch, old.q_len, old.heads, old.page, old.num_cus, tuning, &next, &err);
  } catch (const std::bad_alloc&) {
    return fail(MLA_ERR_OUT_OF_MEMORY, "host allocation failed while planning");
  }
  if (rc != 0) return fail((mla_status)rc, err);
  if (next.segs.size() > plan->cap_segs || next.wgs.size() > plan->cap_wgs || next.cunits.size() > plan->cap_units)
    return fail(MLA_ERR_UNSUPPORTED, "the new schedule does not fit the room reserved at creation");
  // The previous upload must have left the staging copy before it is rewritten.
  hipError_t e = hipEventSynchronize(plan->staged);
  if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize on the previous schedule upload");
  stage_schedule(plan, next);
  hipStream_t st = static_cast<hipStream_t>(stream);
  e = hipMemcpyAsync(plan->dev, plan->stage, plan->total, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipEventRecord(plan->staged, st);
  if (e != hipSuccess) return hip_fail(e, "upload of the updated schedule");
  plan->d = std::move(next);
  g_last_error.clear();
  return MLA_OK;
}

const char* mla_status_string(mla_status s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARGUMENT: return "MLA_ERR_INVALID_ARGUMENT";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    case MLA_ERR_OUT_OF_MEMORY: return "MLA_ERR_OUT_OF_MEMORY";
  }
  return "MLA_ERR_UNKNOWN";
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

int64_t mla_plan_query(const mla_plan* plan, int32_t key) {
  if (!plan) return -1;
  const mla::PlanData& d = plan->d;
  switch (key) {
    case MLA_Q_NUM_SEGMENTS: return (int64_t)d.segs.size();
    case MLA_Q_NUM_WORKGROUPS: return d.grid;
    case MLA_Q_NUM_PARTIALS: return d.num_partials;
    case MLA_Q_ROWS_PER_BLOCK: return d.v.rows_per_block();
    case MLA_Q_TILE_TOKENS: return d.v.tile_tokens;
    case MLA_Q_NUM_ROW_BLOCKS: return d.nrb;
    case MLA_Q_NUM_COMBINE_WGS: return d.jobs.empty() ? 0 : (int64_t)d.cunits.size();
  }
  return -1;
}

mla_status mla_plan_copy(const mla_plan* plan, int32_t* seg, int32_t* wg) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  const mla::PlanData& d = plan->d;
  if (seg)
    for (size_t i = 0; i < d.segs.size(); ++i) {
      seg[4 * i + 0] = d.segs[i].b;
      seg[4 * i + 1] = d.segs[i].kv_begin;
      seg[4 * i + 2] = d.segs[i].kv_end;
      seg[4 * i + 3] = d.segs[i].partial;
    }
  if (wg)
    for (size_t i = 0; i < d.wgs.size(); ++i) {
      wg[4 * i + 0] = d.wgs[i].seg_begin;
      wg[4 * i + 1] = d.wgs[i].seg_end;
      wg[4 * i + 2] = d.wgs[i].row_block;
      wg[4 * i + 3] = 0;
    }
  return MLA_OK;
}

mla_status mla_plan_copy_combine(const mla_plan* plan, int32_t* unit) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  const mla::PlanData& d = plan->d;
  if (unit && !d.jobs.empty())
    for (size_t i = 0; i < d.cunits.size(); ++i) {
      unit[4 * i + 0] = d.cunits[i].b;
      unit[4 * i + 1] = d.cunits[i].p0;
      unit[4 * i + 2] = d.cunits[i].n;
      unit[4 * i + 3] = d.cunits[i].row0;
    }
  return MLA_OK;
}

static mla_status decode_partials(const mla_plan* plan, const void* q_nope_absorbed, const void* q_pe,
                                  const void* kv_cache, int64_t num_pages, const int32_t* block_table,
                                  int32_t bt_stride, const int32_t* seq_lens, float softmax_scale, float* out,
                                  float* lse, void* workspace, size_t workspace_bytes, int32_t variant,
                                  uint32_t* rescale_events, void* stream) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (variant != MLA_RESCALE_LAZY && variant != MLA_RESCALE_POW2)
    return fail(MLA_ERR_INVALID_ARGUMENT, "variant must be MLA_RESCALE_LAZY or MLA_RESCALE_POW2");
  if (!aligned(rescale_events, 4)) return fail(MLA_ERR_INVALID_ARGUMENT, "rescale_events must be 4-byte aligned");
  if (!q_nope_absorbed || !q_pe || !kv_cache || !block_table || !seq_lens || !out || !lse)
    return fail(MLA_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (!aligned(q_nope_absorbed, 16) || !aligned(q_pe, 16) || !aligned(kv_cache, 16) || !aligned(out, 16))
    return fail(MLA_ERR_INVALID_ARGUMENT, "q_nope_absorbed, q_pe, kv_cache and out must be 16-byte aligned");
  if (!aligned(lse, 4) || !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return fail(MLA_ERR_INVALID_ARGUMENT, "lse, block_table and seq_lens must be 4-byte aligned");
  if (num_pages <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages must be > 0");
  const mla::PlanData& d = plan->d;
  if (bt_stride < d.max_pages)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bt_stride (" + std::to_string(bt_stride) +
                                              ") is smaller than the longest request's page count (" +
                                              std::to_string(d.max_pages) + ")");
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  Workspace ws;
  mla_status st_ws = check_workspace(plan, workspace, workspace_bytes, &ws);
  if (st_ws != MLA_OK) return st_ws;
  mla_status st_dev = check_device(plan);
  if (st_dev != MLA_OK) return st_dev;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const float scale_log2 = softmax_scale * 1.44269504088896340736f;
  const bool single = d.page >= d.v.tile_tokens;
  if (d.v.waves != mla::kWaves || d.v.tile_tokens != mla::kTile)
    return fail(MLA_ERR_INVALID_ARGUMENT, "plan was not made by mla_decode_plan (an FP8 plan runs with mla_decode_fp8)");
  auto launch = [&](auto single_c, auto pow2_c) {
    return launch_decode<decltype(single_c)::value, decltype(pow2_c)::value>(
        plan, q_nope_absorbed, q_pe, kv_cache, num_pages, block_table, bt_stride, seq_lens, scale_log2, out, lse, ws,
        rescale_events, st);
  };
  using T = std::true_type;
  using F = std::false_type;
  const bool pow2 = variant == MLA_RESCALE_POW2;
  hipError_t e = single ? (pow2 ? launch(T{}, T{}) : launch(T{}, F{})) : (pow2 ? launch(F{}, T{}) : launch(F{}, F{}));
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  g_last_error.clear();
  return MLA_OK;
}

mla_status mla_decode_partials(const mla_plan* plan, const void* q_nope_absorbed, const void* q_pe,
                               const void* kv_cache, int64_t num_pages, const int32_t* block_table, int32_t bt_stride,
                               const int32_t* seq_lens, float softmax_scale, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return decode_partials(plan, q_nope_absorbed, q_pe, kv_cache, num_pages, block_table, bt_stride, seq_lens,
                         softmax_scale, out, lse, workspace, workspace_bytes, MLA_RESCALE_LAZY, nullptr, stream);
}

mla_status mla_decode_variant(const mla_plan* plan, const void* q_nope_absorbed, const void* q_pe,
                              const void* kv_cache, int64_t num_pages, const int32_t* block_table, int32_t bt_stride,
                              const int32_t* seq_lens, float softmax_scale, float* out, float* lse, void* workspace,
                              size_t workspace_bytes, int32_t variant, uint32_t* rescale_events, void* stream) {
  mla_status s = decode_partials(plan, q_nope_absorbed, q_pe, kv_cache, num_pages, block_table, bt_stride, seq_lens,
                                 softmax_scale, out, lse, workspace, workspace_bytes, variant, rescale_events, stream);
  if (s != MLA_OK) return s;
  return mla_decode_combine(plan, out, lse, workspace, workspace_bytes, stream);
}

mla_status mla_decode_combine(const mla_plan* plan, float* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!out || !lse) return fail(MLA_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (!aligned(out, 16) || !aligned(lse, 4)) return fail(MLA_ERR_INVALID_ARGUMENT, "out must be 16-byte aligned");
  Workspace ws;
  mla_status st_ws = check_workspace(plan, workspace, workspace_bytes, &ws);
  if (st_ws != MLA_OK) return st_ws;
  mla_status st_dev = check_device(plan);
  if (st_dev != MLA_OK) return st_dev;
  const mla::PlanData& d = plan->d;
  if (!d.jobs.empty()) {
    const char* base = static_cast<const char*>(plan->dev);
    const mla::CombineUnit* units = reinterpret_cast<const mla::CombineUnit*>(base + plan->off_units);
    if (d.max_pieces <= mla::kCombineSmallMax)
      hipLaunchKernelGGL(mla::combine_small_kernel, dim3((unsigned)d.cunits.size()), dim3(64 * mla::kCombineSmallRows),
                         0, static_cast<hipStream_t>(stream), units, ws.o, ws.lse, ws.f, d.rows, d.v.rows_per_block(),
                         d.nrb, out, lse);
    else
      hipLaunchKernelGGL(mla::combine_kernel, dim3((unsigned)d.cunits.size()), dim3(256), 0,
                         static_cast<hipStream_t>(stream), units, ws.o, ws.lse, ws.f, d.rows, d.v.rows_per_block(),
                         d.nrb, out, lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  }
  g_last_error.clear();
  return MLA_OK;
}

mla_status mla_decode_fp8_plan(const int32_t* seq_lens_host, int32_t batch, int32_t q_len, int32_t num_heads,
                               int32_t page_size, int32_t num_cus, mla_plan** plan_out) {
  return make_plan(seq_lens_host, batch, q_len, num_heads, page_size, num_cus, plan_out, true, 2);
}

mla_status mla_decode_fp8_plan_host(const int32_t* seq_lens_host, int32_t batch, int32_t q_len, int32_t num_heads,
                                    int32_t page_size, int32_t num_cus, mla_plan** plan_out) {
  return make_plan(seq_lens_host, batch, q_len, num_heads, page_size, num_cus, plan_out, false, 2);
}

mla_status mla_decode_fp8_partials(const mla_plan* plan, const void* q_nope_absorbed, const void* q_pe,
                                   const void* kv_codes, const void* kv_scales, int64_t num_pages,
                                   const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                                   float softmax_scale, float* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!q_nope_absorbed || !q_pe || !kv_codes || !kv_scales || !block_table || !seq_lens || !out || !lse)
    return fail(MLA_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (!aligned(q_nope_absorbed, 16) || !aligned(q_pe, 16) || !aligned(kv_codes, 16) || !aligned(out, 16))
    return fail(MLA_ERR_INVALID_ARGUMENT, "q_nope_absorbed, q_pe, kv_codes and out must be 16-byte aligned");
  if (!aligned(kv_scales, 4) || !aligned(lse, 4) || !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return fail(MLA_ERR_INVALID_ARGUMENT, "kv_scales, lse, block_table and seq_lens must be 4-byte aligned");
  if (num_pages <= 0) return fail(MLA_ERR_INVALID_ARGUMENT, "num_pages must be > 0");
  const mla::PlanData& d = plan->d;
  if (d.v.tile_tokens != mla::kFp8TileTokens || d.v.waves != mla::kFp8Waves)
    return fail(MLA_ERR_INVALID_ARGUMENT, "plan was not made by mla_decode_fp8_plan");
  if (bt_stride < d.max_pages)
    return fail(MLA_ERR_INVALID_ARGUMENT, "bt_stride (" + std::to_string(bt_stride) +
                                              ") is smaller than the longest request's page count (" +
                                              std::to_string(d.max_pages) + ")");
  if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
    return fail(MLA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and > 0");
  Workspace ws;
  mla_status st_ws = check_workspace(plan, workspace, workspace_bytes, &ws);
  if (st_ws != MLA_OK) return st_ws;
  mla_status st_dev = check_device(plan);
  if (st_dev != MLA_OK) return st_dev;
  const float scale_log2 = softmax_scale * 1.44269504088896340736f;
  hipError_t e = mla::launch_decode_fp8(d, static_cast<const char*>(plan->dev), plan->off_segs, plan->off_wgs,
                                        plan->off_lens, q_nope_absorbed, q_pe, kv_codes, kv_scales, num_pages,
                                        block_table, bt_stride, seq_lens, scale_log2, out, lse, ws.o, ws.lse, ws.f,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "FP8 decode kernel launch");
  g_last_error.clear();
  return MLA_OK;
}

mla_status mla_decode_fp8(const mla_plan* plan, const void* q_nope_absorbed, const void* q_pe, const void* kv_codes,
                          const void* kv_scales, int64_t num_pages, const int32_t* block_table, int32_t bt_stride,
                          const int32_t* seq_lens, float softmax_scale, float* out, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  mla_status s = mla_decode_fp8_partials(plan, q_nope_absorbed, q_pe, kv_codes, kv_scales, num_pages, block_table,
                                         bt_stride, seq_lens, softmax_scale, out, lse, workspace, workspace_bytes,
                                         stream);
  if (s != MLA_OK) return s;
  return mla_decode_combine(plan, out, lse, workspace, workspace_bytes, stream);
}

mla_status mla_decode(const mla_plan* plan, const void* q_nope_absorbed, const void* q_pe, const void* kv_cache,
                      int64_t num_pages, const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                      float softmax_scale, float* out, float* lse, void* workspace, size_t workspace_bytes,
                      void* stream) {
  mla_status s = mla_decode_partials(plan, q_nope_absorbed, q_pe, kv_cache, num_pages, block_table, bt_stride,
                                     seq_lens, softmax_scale, out, lse, workspace, workspace_bytes, stream);
  if (s != MLA_OK) return s;
  return mla_decode_combine(plan, out, lse, workspace, workspace_bytes, stream);
}

mla_status mla_decode_noalloc(const mla_plan* plan, const void* q_nope_absorbed, const void* q_pe, const void* kv_cache,
                              int64_t num_pages, const int32_t* block_table, int32_t bt_stride, const int32_t* seq_lens,
                              float softmax_scale, float* out, float* lse, void* stream) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  const size_t need = mla::workspace_bytes(plan->d);
  if (need > kNoAllocScratchBytes)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "the plan needs " + std::to_string(need) +
                                                 " bytes of partials, more than the " +
                                                 std::to_string(kNoAllocScratchBytes) +
                                                 "-byte scratch of mla_decode_noalloc (use mla_decode with a workspace)");
  if (!q_nope_absorbed || !q_pe || !kv_cache || !block_table || !seq_lens || !out || !lse)
    return fail(MLA_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
  mla_status st = check_device(plan);
  if (st != MLA_OK) return st;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(plan->device, &ws);
    if (st != MLA_OK) return st;
  }
  return mla_decode(plan, q_nope_absorbed, q_pe, kv_cache, num_pages, block_table, bt_stride, seq_lens, softmax_scale,
                    out, lse, ws, need > 0 ? kNoAllocScratchBytes : 0, stream);
}

}  // extern "C"
