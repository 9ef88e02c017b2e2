// Weight-absorbed MLA decode attention for gfx950 (MI355X): split-KV decode
// kernel, log-sum-exp combine kernel and the C ABI around them.
//
// The computation (Huawei, "DeepSeek V3/R1 inference deployment best practices
// on Ascend servers", section 3.2.1 and section 6.1): every head of a request
// attends over the same cached 576-wide rows [c_kv | k_pe]; V is c_kv.  With
// the heads as the M dimension, QK^T and PV are dense contractions against a
// shared key tile, so both run on bf16 MFMA with fp32 accumulation.
//
// Decode kernel: one workgroup = 4 waves = 128 query rows (rows are the
// flattened (query token, head) pairs of one request), walking one or more
// pieces of key range in tiles of 32 keys:
//  * tiles are copied HBM -> LDS with 16-byte direct loads
//    (global_load_lds_dwordx4) into a ring of NSTAGE buffers; while tile i is
//    computed, tiles i+1 .. i+NSTAGE-1 are in flight (about 110 KB per CU, to
//    cover HBM latency at full bandwidth).  One barrier per tile;
//  * a cached row is 72 chunks of 16 bytes; inside each aligned group of 8
//    chunks, chunk c of key row t is stored at c ^ swz(t).  The swizzle makes
//    both the row reads of QK^T (16 rows, same chunk) and the transposed reads
//    of PV (4 rows x 4 chunks) hit 16 distinct 4-bank groups;
//  * wave w keeps its 32 query rows, as the B operand of
//    v_mfma_f32_32x32x16_bf16, in 144 VGPRs for the whole piece, and computes
//    S^T = K Q^T for the tile's 32 keys (A operand = key rows read from LDS);
//    in that layout each lane holds one head and 16 keys, so the row maximum
//    needs one cross-half swap and the running (max, sum) is lane-local;
//  * online softmax in base 2 with a lazy reference: the output is rescaled
//    only when a row's maximum grows by more than 2^8;
//  * O^T = V^T P^T accumulates in 16 MFMA tiles (256 registers, AGPR); V^T
//    comes straight from the same LDS tile through ds_read_b64_tr_b16 (the
//    c_kv columns of the key rows; no second copy of V);
//  * the piece ends with out = O / l and lse = ln(sum) written either to the
//    final tensors (a request in one piece) or to a workspace partial.
// Combine kernel: per split request and row, lse = logsumexp over its pieces,
// out = sum_s exp(lse_s - lse) o_s (the flash-decoding merge).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "mla_decode.h"
#include "plan_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kRowBytes = 576 * 2;  // one cached token (HBM and LDS)
constexpr int kChunks = 72;         // 16-byte chunks per cached token
constexpr int kTile = 32;           // keys per tile
constexpr int kWaves = 4;
constexpr int kRowsPerBlock = 32 * kWaves;
constexpr int kStageBytes = kTile * kRowBytes;         // 36864
constexpr int kLoadsPerTile = kTile * kChunks / 64;     // 36 one-KB copies
constexpr int kLoadsPerWave = kLoadsPerTile / kWaves;  // 9
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
static_assert(kLoadsPerTile % kWaves == 0, "every wave issues the same number of copies");

// Chunk swizzle of key row t (t = row within the tile).
__device__ __forceinline__ int swz(int t) { return (((t >> 1) & 1) << 2) | ((t >> 2) & 3); }

__device__ __forceinline__ float partner_max(float x) {
  // permlane32_swap(x, x) returns {lanes 0-31: x, 32-63: x of lane-32} and
  // {lanes 0-31: x of lane+32, 32-63: x}; the max/sum of the pair is symmetric.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float partner_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (N is an immediate).  The query loads and LDS copies are inline asm the
// compiler does not count, so every wait on them is explicit.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte global -> LDS copies (global_load_lds_dwordx4).  Each lane names its
// own source; the 64 lanes of the wave fill 1 KB of LDS starting at M0.  They
// are issued as inline asm on purpose: the compiler's wait-count pass treats a
// pending LDS copy as aliasing every later LDS read and would insert
// s_waitcnt vmcnt(0) before them, serializing the copy of later tiles with the
// compute on this one.  (s_nop 0: one wait state between the M0 write and the
// copy that reads it.)
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void dma16(const void* src, uint32_t lds_dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_dst) : "memory");
}

__device__ __forceinline__ void dma16_saddr(const void* base, uint32_t off, uint32_t lds_dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_dst) : "memory");
}

// 16-byte global load into VGPRs, invisible to the compiler's wait counts
// (the explicit wait before the first QK^T covers it).
__device__ __forceinline__ bf16x8 load16(const void* src) {
  bf16x8 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(src) : "memory");
  return v;
}

// The S^T accumulators are pinned to VGPRs (the softmax reads them with VALU
// right away) while the output accumulators live in AGPRs; the compiler left to
// itself puts both in AGPRs and spills.  So the QK^T MFMA is issued as inline
// asm with a VGPR constraint.  The hazards the compiler cannot see inside the
// asm are handled here: the first step takes srcC = 0 (no VALU write of the
// accumulator right before an MFMA reads it), and s_mfma_drain waits out the
// XDL-write -> VALU-read latency before anything reads the results.  Every
// MFMA issued as asm starts with s_nop 1: a VALU write of a source register
// needs two wait states before an MFMA reads it.
__device__ __forceinline__ void s_mfma(f32x16& acc, const bf16x8& a, const bf16x8& b, bool first) {
  if (first)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ void s_mfma_drain(f32x16& acc) { asm volatile("s_nop 15\n\ts_nop 7" : "+v"(acc)); }

// The output accumulators O^T (16 tiles of 32x32 fp32 = 256 registers per
// lane) live in the physical AGPRs a[0:255]: tile cb is a[16cb : 16cb+15].
// They are only touched by inline asm that names them and lists them as
// clobbered, so the compiler never allocates them (left to itself it carries
// them through VGPRs around the rare rescale branch and spills the query rows).
// Hazards the compiler cannot see are handled where the code runs:
//  * MFMA -> accvgpr_read of the results: o_drain waits 24 wait states;
//  * accvgpr_write (rescale) -> MFMA srcC: the whole softmax runs in between,
//    plus the s_nop in front of every MFMA.
template <int CB>
struct OTile;
template <int N>
__device__ __forceinline__ float o_get();
template <int N>
__device__ __forceinline__ void o_set(float x);
#include "agpr_tiles.inc"

// Dispatch on a tile index that is a constant after unrolling.
__device__ __forceinline__ void o_mfma(int cb, const bf16x8& a, const bf16x8& b, bool first) {
#define MLA_CASE(n)               \
  case n:                         \
    if (first)                    \
      OTile<n>::mfma_first(a, b); \
    else                          \
      OTile<n>::mfma(a, b);       \
    break;
  switch (cb) {
    MLA_CASE(0) MLA_CASE(1) MLA_CASE(2) MLA_CASE(3) MLA_CASE(4) MLA_CASE(5) MLA_CASE(6) MLA_CASE(7)
    MLA_CASE(8) MLA_CASE(9) MLA_CASE(10) MLA_CASE(11) MLA_CASE(12) MLA_CASE(13) MLA_CASE(14) MLA_CASE(15)
  }
#undef MLA_CASE
}

template <int N>
__device__ __forceinline__ void o_scale_rec(float alpha) {
  if constexpr (N < 256) {
    o_set<N>(o_get<N>() * alpha);
    o_scale_rec<N + 1>(alpha);
  }
}

// Multiply all 256 accumulators by this lane's alpha.
__device__ __forceinline__ void o_scale_all(float alpha) { o_scale_rec<0>(alpha); }

// Wait out the MFMA write -> AGPR read latency before reading results.
__device__ __forceinline__ void o_drain() { asm volatile("s_nop 15\n\ts_nop 7" ::: "memory"); }

// Store tile register group [4g, 4g+3] of tile cb (lane: 4 consecutive columns), scaled.
template <int CB, int G>
__device__ __forceinline__ void o_store4(float* dst, float inv) {
  constexpr int n = 16 * CB + 4 * G;
  f32x4 w = {o_get<n + 0>() * inv, o_get<n + 1>() * inv, o_get<n + 2>() * inv, o_get<n + 3>() * inv};
  *reinterpret_cast<f32x4*>(dst) = w;
}

template <int CB>
__device__ __forceinline__ void o_store_rec(float* dst, int half, float inv) {
  if constexpr (CB < 16) {
    o_store4<CB, 0>(dst + CB * 32 + 0 * 8 + 4 * half, inv);
    o_store4<CB, 1>(dst + CB * 32 + 1 * 8 + 4 * half, inv);
    o_store4<CB, 2>(dst + CB * 32 + 2 * 8 + 4 * half, inv);
    o_store4<CB, 3>(dst + CB * 32 + 3 * 8 + 4 * half, inv);
    o_store_rec<CB + 1>(dst, half, inv);
  }
}

// Page ids a tile touches (uniform; at most 2 since pages hold >= 16 keys and
// tiles hold 32).  Out-of-range ids are replaced by page 0 so that a corrupt
// block table can never make the kernel read outside the cache.
struct TilePages {
  int first;
  int pg[2];
};

template <int NSTAGE, bool SINGLE_PAGE>
__global__ __launch_bounds__(64 * kWaves, 1) void decode_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const uint8_t* __restrict__ cache, int64_t num_pages,
    const int32_t* __restrict__ block_table, int32_t bt_stride,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ planned_lens,
    const Segment* __restrict__ segs, const WorkgroupRange* __restrict__ wgs,
    float scale_log2, int32_t rows, int32_t heads, int32_t q_len, int32_t page_log2, int32_t nrb,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o,
    float* __restrict__ ws_lse) {
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "2..4 LDS stages");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NSTAGE * kStageBytes];

  const WorkgroupRange wr = wgs[blockIdx.x];
  if (wr.seg_begin >= wr.seg_end) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;  // which 8-wide k slice of an MFMA operand this lane holds
  const int rb = wr.row_block;
  const int row_local = wave * 32 + (lane & 31);
  const int row = rb * kRowsPerBlock + row_local;
  const bool row_ok = row < rows;
  const int jq = row_ok ? row / heads : 0;  // query token of this row
  const int psize = 1 << page_log2;

  // Per-lane LDS byte offsets (within a stage) of the operand reads.
  // QK^T, A operand = key rows: key t = lane & 31, logical chunk 2*kk + half,
  // stored at chunk (2*kk + half) ^ swz(t) of its 8-group.  For kk = 4*g + m
  // the offset is qk_base[m] + 128*g.
  int qk_base[4];
  {
    const int t = lane & 31;
#pragma unroll
    for (int m = 0; m < 4; ++m) qk_base[m] = t * kRowBytes + 16 * ((2 * m + half) ^ swz(t));
  }
  // PV, A operand = V^T via transposed reads: within each 16-lane group g, lane k
  // addresses key row (k / 4) of a 4-key strip, columns 4 * (k % 4) .. + 3 of a
  // 16-column strip; the read hands lane k column k of the 4 x 16 block.  Key
  // row r = 16*ks + 8*qq + 4*half + k/4, column 32*cb + 16*(g&1) + 4*(k&3); its
  // chunk (column / 8) is swizzled by the row.  The offset is
  // pv_base[qq][cb&1] + 18432*ks + 128*(cb>>1).
  int pv_base[2][2];
  {
    const int grp = lane >> 4, k16 = lane & 15;
    const int clow = 2 * (grp & 1) + ((k16 & 3) >> 1);  // chunk within a 4-chunk (32-column) group
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int r = 8 * qq + 4 * half + (k16 >> 2);
#pragma unroll
      for (int odd = 0; odd < 2; ++odd)
        pv_base[qq][odd] = r * kRowBytes + 16 * ((4 * odd + clow) ^ swz(r)) + 8 * (k16 & 1);
    }
  }

  for (int si = wr.seg_begin; si < wr.seg_end; ++si) {
    const Segment sg = segs[si];
    const int b = sg.b, kv0 = sg.kv_begin, kv1 = sg.kv_end;
    const int L = seq_lens[b];
    const bool bad_len = (L != planned_lens[b]);
    const int32_t* bt_row = block_table + (int64_t)b * bt_stride;

    // Keys this row may see inside the piece: [kv0, lim).
    const int lim = row_ok ? min(kv1, L - q_len + 1 + jq) : kv0;

    // Block-table entries of a tile (scalar loads, checked when used).
    auto fetch_pages = [&](int tb) {
      TilePages tp;
      tp.first = tb >> page_log2;
      const int last = (min(tb + kTile, kv1) - 1) >> page_log2;
      tp.pg[0] = bt_row[tp.first];
      tp.pg[1] = SINGLE_PAGE ? tp.pg[0] : bt_row[min(tp.first + 1, last)];
      return tp;
    };
    auto checked = [&](TilePages tp) {
#pragma unroll
      for (int k = 0; k < 2; ++k) tp.pg[k] = ((uint64_t)(int64_t)tp.pg[k] < (uint64_t)num_pages) ? tp.pg[k] : 0;
      return tp;
    };

    // Copy i of this wave for the tile at key tb: LDS slots [64 n, 64 n + 64)
    // of the stage, n = i * 4 + wave; slot p holds chunk (p % 72) ^ swz of key
    // p / 72.  Keys past the piece are clamped to its last key (their scores
    // are masked; the copy stays inside the request's pages).
    auto dma = [&](int i, int tb, const TilePages& tp, uint8_t* stage) {
      const int n = i * kWaves + wave;
      int lane_v = lane;
      asm volatile("" : "+v"(lane_v));  // keep the address math next to its use
      const int pos = n * 64 + lane_v;
      const int t = pos / kChunks;
      const int pc = pos - t * kChunks;
      const int c = pc ^ swz(t);
      const int tok = min(tb + t, kv1 - 1);
      const uint32_t lds_dst = lds_addr(stage + n * 1024);
      if (SINGLE_PAGE) {
        const uint8_t* pbase = cache + ((int64_t)tp.pg[0] << page_log2) * kRowBytes;
        dma16_saddr(pbase, (uint32_t)((tok & (psize - 1)) * kRowBytes + c * 16), lds_dst);
      } else {
        const int page = ((tok >> page_log2) == tp.first) ? tp.pg[0] : tp.pg[1];
        dma16(cache + (((int64_t)page << page_log2) + (tok & (psize - 1))) * kRowBytes + c * 16, lds_dst);
      }
    };

    const int ntiles = (kv1 - kv0 + kTile - 1) / kTile;

    // All waves must be done with the previous piece's tiles before the first
    // tiles of this one land in LDS.
    __syncthreads();

    // Query rows as the MFMA B operand: lane holds dims 16*kk + 8*half .. +7.
    // Issued first so that the wait for tile 0 also covers them.
    bf16x8 q[36];
    {
      const int qrow = row_ok ? row : 0;  // rows past the end load row 0 and are zeroed below
      const uint16_t* qn = q_nope + ((int64_t)b * rows + qrow) * 512 + 8 * half;
      const uint16_t* qp = q_pe + ((int64_t)b * rows + qrow) * 64 + 8 * half;
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) q[kk] = load16(qn + 16 * kk);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) q[32 + kk] = load16(qp + 16 * kk);
    }

    // Software pipeline over tiles (4 LDS stages): iteration `it` runs the
    // QK^T MFMAs of tile it+1 interleaved with the softmax VALU work of tile
    // it, then the PV MFMAs of tile it.  Tiles it and it+1 are resident, it+2
    // and it+3 are in flight; the copy of tile it+3 goes into the stage tile
    // it-1 used.  Every iteration issues exactly one tile of copies (past the
    // end of the piece it repeats the last tile into a stage nobody reads), so
    // every wait below has a fixed count.
    static_assert(NSTAGE == 4, "the pipeline keeps two tiles resident and two in flight");
    const int last_tile = ntiles - 1;
#pragma unroll
    for (int st = 0; st < 3; ++st) {
      const int ti = min(st, last_tile);
      const TilePages tp = checked(fetch_pages(kv0 + ti * kTile));
#pragma unroll
      for (int i = 0; i < kLoadsPerWave; ++i) dma(i, kv0 + ti * kTile, tp, smem + st * kStageBytes);
    }
    TilePages pg_raw = fetch_pages(kv0 + min(3, last_tile) * kTile);

    // QK^T of one tile into acc (lane: head lane&31, 16 keys).  `extra(kk)`
    // is called between the MFMAs so that independent VALU/VMEM work issues
    // while the matrix pipe runs.
    auto qk_tile = [&](const uint8_t* kb, f32x16& acc, auto&& extra) {
      bf16x8 a[3];
      auto read_k = [&](int kk) {
        return *reinterpret_cast<const bf16x8*>(kb + qk_base[kk & 3] + 128 * (kk >> 2));
      };
      a[0] = read_k(0);
      a[1] = read_k(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < 36; ++kk) {
        if (kk + 2 < 36) a[(kk + 2) % 3] = read_k(kk + 2);
        extra(kk);
        s_mfma(acc, a[kk % 3], q[kk], kk == 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      s_mfma_drain(acc);
    };

    // Tile 0 (and the query rows, loaded before it) have landed once two
    // tiles of copies are still in flight.  The empty asm statements tie the
    // query registers to this point: the loads fill them asynchronously, so
    // nothing may read, copy or reuse them before the wait.
    {
      wait_vmem<2 * kLoadsPerWave>();
      asm volatile("" : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]), "+v"(q[4]), "+v"(q[5]), "+v"(q[6]),
                   "+v"(q[7]), "+v"(q[8]));
      asm volatile("" : "+v"(q[9]), "+v"(q[10]), "+v"(q[11]), "+v"(q[12]), "+v"(q[13]), "+v"(q[14]),
                   "+v"(q[15]), "+v"(q[16]), "+v"(q[17]));
      asm volatile("" : "+v"(q[18]), "+v"(q[19]), "+v"(q[20]), "+v"(q[21]), "+v"(q[22]), "+v"(q[23]),
                   "+v"(q[24]), "+v"(q[25]), "+v"(q[26]));
      asm volatile("" : "+v"(q[27]), "+v"(q[28]), "+v"(q[29]), "+v"(q[30]), "+v"(q[31]), "+v"(q[32]),
                   "+v"(q[33]), "+v"(q[34]), "+v"(q[35]));
      if (!row_ok) {
#pragma unroll
        for (int kk = 0; kk < 36; ++kk) q[kk] = bf16x8{};
      }
      __syncthreads();
    }
    f32x16 s_cur;
    qk_tile(smem, s_cur, [](int) {});

    float m_ref = -INFINITY;  // running reference max (log2 units), same in lanes l and l^32
    float l_part = 0.f;       // this lane's share of the running sum

    for (int it = 0; it < ntiles; ++it) {
      const bool has_next = it + 1 < ntiles;
      // Tile it+1 has landed once only tile it+2's copies of this wave are in
      // flight; the barrier publishes every wave's part and frees the stage of
      // tile it-1 for the next copy.
      wait_vmem<kLoadsPerWave>();
      __syncthreads();

      const int tb = kv0 + it * kTile;
      const uint8_t* kb = smem + (it % NSTAGE) * kStageBytes;             // tile it (PV)
      const uint8_t* kb_next = smem + ((it + 1) % NSTAGE) * kStageBytes;  // tile it+1 (QK^T)
      const int nt = it + 3;                                              // tile to copy now
      const int nti = min(nt, last_tile);
      uint8_t* nbuf = smem + (nt % NSTAGE) * kStageBytes;
      const TilePages npg = checked(pg_raw);
      pg_raw = fetch_pages(kv0 + min(nt + 1, last_tile) * kTile);
      __builtin_amdgcn_sched_barrier(0);

      // ---- tile it: mask, scale to log2 units, tile max ----
      const bool need_mask = tb + kTile > lim;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s_cur[i] * scale_log2;
        if (need_mask) {
          const int tok = tb + (i >> 2) * 8 + half * 4 + (i & 3);
          x = tok < lim ? x : -INFINITY;
        }
        s_cur[i] = x;
      }
      float mx = fmaxf(fmaxf(fmaxf(s_cur[0], s_cur[1]), fmaxf(s_cur[2], s_cur[3])),
                       fmaxf(fmaxf(s_cur[4], s_cur[5]), fmaxf(s_cur[6], s_cur[7])));
      mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s_cur[8], s_cur[9]), fmaxf(s_cur[10], s_cur[11])),
                           fmaxf(fmaxf(s_cur[12], s_cur[13]), fmaxf(s_cur[14], s_cur[15]))));
      mx = partner_max(mx);

      // ---- lazy rescale of the running output ----
      // A row moves its reference only when its maximum grows by more than
      // kRescaleThreshold; the first finite maximum needs no rescale because
      // nothing has been accumulated yet.
      const bool need_update = mx > m_ref + kRescaleThreshold;
      if (__any(need_update)) {
        const bool need_scale = need_update && m_ref != -INFINITY;
        const float m_new = need_update ? mx : m_ref;
        const float alpha = need_scale ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
        l_part *= alpha;
        if (__any(need_scale)) o_scale_all(alpha);
        m_ref = m_new;
      }
      const float mu = (m_ref == -INFINITY) ? 0.f : m_ref;
      __builtin_amdgcn_sched_barrier(0);

      // ---- QK^T of tile it+1, with P = 2^(x - mu) of tile it (bf16 MFMA B
      //      operands, 8 keys per 16-key step) and the copies of tile it+3
      //      issued between its MFMAs ----
      bf16x8 pb[2];
      auto softmax_step = [&](int kk) {
        if (kk < 16) {
          const float p = __builtin_amdgcn_exp2f(s_cur[kk] - mu);
          l_part += p;
          pb[kk >> 3][kk & 7] = (__bf16)p;
        }
        if (kk >= 16 && kk < 16 + kLoadsPerWave) dma(kk - 16, kv0 + nti * kTile, npg, nbuf);
      };
      f32x16 s_next;
      if (has_next) {
        qk_tile(kb_next, s_next, softmax_step);
      } else {
#pragma unroll
        for (int kk = 0; kk < 36; ++kk) softmax_step(kk);
      }
      // Materialize the bf16 operands here, not next to the MFMAs.
      asm volatile("" : "+v"(pb[0]), "+v"(pb[1]));
      __builtin_amdgcn_sched_barrier(0);

      // ---- O^T += V^T P^T for tile it, V^T read transposed from its stage ----
      i16x8 v[3];
      auto read_v = [&](int idx) {
        const int ks = idx >> 4, cb = idx & 15;
        const uint8_t* v0p = kb + pv_base[0][cb & 1] + 18432 * ks + 128 * (cb >> 1);
        const uint8_t* v1p = kb + pv_base[1][cb & 1] + 18432 * ks + 128 * (cb >> 1);
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(i16x4, v0p));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(i16x4, v1p));
        return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      v[0] = read_v(0);
      v[1] = read_v(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int idx = 0; idx < 32; ++idx) {
        if (idx + 2 < 32) v[(idx + 2) % 3] = read_v(idx + 2);
        const int ks = idx >> 4, cb = idx & 15;
        o_mfma(cb, __builtin_bit_cast(bf16x8, v[idx % 3]), pb[ks], it == 0 && ks == 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      s_cur = s_next;
    }

    // The repeated copies past the end of the piece must land before the next
    // piece reuses their stages.
    wait_vmem<0>();

    // ---- epilogue: normalize and store (final output or a workspace partial) ----
    o_drain();
    const float l_tot = partner_sum(l_part);
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float lse_v = l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    if (bad_len) {
      inv = NAN;
      lse_v = NAN;
    }
    if (row_ok) {
      float* dst;
      float* dl;
      if (sg.partial < 0) {
        dst = out + ((int64_t)b * rows + row) * 512;
        dl = lse + (int64_t)b * rows + row;
      } else {
        const int64_t slot = (int64_t)sg.partial * nrb + rb;
        dst = ws_o + (slot * kRowsPerBlock + row_local) * 512;
        dl = ws_lse + slot * kRowsPerBlock + row_local;
      }
      o_store_rec<0>(dst, half, inv);
      if (half == 0) *dl = lse_v;
    }
  }
}

// One workgroup = 2 rows x 512 columns of one split request; each thread owns
// 4 columns of one row and walks that request's partials.
__global__ __launch_bounds__(256) void combine_kernel(const CombineJob* __restrict__ jobs,
                                                       const float* __restrict__ ws_o,
                                                       const float* __restrict__ ws_lse, int32_t rows,
                                                       int32_t rpb, int32_t nrb, float* __restrict__ out,
                                                       float* __restrict__ lse) {
  const CombineJob job = jobs[blockIdx.x];
  const int row = blockIdx.y * 2 + (threadIdx.x >> 7);
  if (row >= rows) return;
  const int c = (threadIdx.x & 127) * 4;
  const int rb = row / rpb, rl = row - rb * rpb;
  auto slot_of = [&](int s) { return ((int64_t)(job.p0 + s) * nrb + rb) * rpb + rl; };

  float m = -INFINITY;
  bool any_nan = false;  // fmaxf drops NaN; a NaN partial (length mismatch) must stay loud
  for (int s = 0; s < job.n; ++s) {
    const float v = ws_lse[slot_of(s)];
    any_nan |= (v != v);
    m = fmaxf(m, v);
  }
  float lse_v = -INFINITY;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (any_nan) {
    lse_v = NAN;
    acc = f32x4{NAN, NAN, NAN, NAN};
  } else if (m != -INFINITY) {
    float z = 0.f;
    for (int s = 0; s < job.n; ++s) z += __expf(ws_lse[slot_of(s)] - m);
    lse_v = m + __logf(z);
#pragma unroll 4
    for (int s = 0; s < job.n; ++s) {
      const int64_t sl = slot_of(s);
      const float w = __expf(ws_lse[sl] - lse_v);
      const f32x4 v = *reinterpret_cast<const f32x4*>(ws_o + sl * 512 + c);
      acc += w * v;
    }
  }
  *reinterpret_cast<f32x4*>(out + ((int64_t)job.b * rows + row) * 512 + c) = acc;
  if (c == 0) lse[(int64_t)job.b * rows + row] = lse_v;
}

}  // namespace
}  // namespace mla

// ----------------------------------------------------------------------------
// C ABI
// ----------------------------------------------------------------------------

struct mla_plan {
  mla::PlanData d;
  void* dev = nullptr;  // device schedule: segs | wgs | jobs | planned lens
  size_t off_segs = 0, off_wgs = 0, off_jobs = 0, off_lens = 0;
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

mla_status make_plan(const int32_t* seq_lens_host, int32_t batch, int32_t q_len, int32_t num_heads,
                     int32_t page_size, int32_t num_cus, mla_plan** plan_out, bool upload) {
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
    rc = mla::build_plan(seq_lens_host, batch, q_len, num_heads, page_size, num_cus, mla::PlanTuning{}, &p->d,
                         &err);
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(MLA_ERR_OUT_OF_MEMORY, "host allocation failed while planning");
  }
  if (rc != 0) {
    delete p;
    return fail((mla_status)rc, err);
  }
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
    p->off_segs = 0;
    p->off_wgs = align256(d.segs.size() * sizeof(mla::Segment));
    p->off_jobs = p->off_wgs + align256(d.wgs.size() * sizeof(mla::WorkgroupRange));
    p->off_lens = p->off_jobs + align256(d.jobs.size() * sizeof(mla::CombineJob));
    const size_t total = p->off_lens + align256(d.lens.size() * sizeof(int32_t));
    std::string host(total, '\0');
    std::memcpy(&host[p->off_segs], d.segs.data(), d.segs.size() * sizeof(mla::Segment));
    std::memcpy(&host[p->off_wgs], d.wgs.data(), d.wgs.size() * sizeof(mla::WorkgroupRange));
    if (!d.jobs.empty()) std::memcpy(&host[p->off_jobs], d.jobs.data(), d.jobs.size() * sizeof(mla::CombineJob));
    std::memcpy(&host[p->off_lens], d.lens.data(), d.lens.size() * sizeof(int32_t));
    hipError_t e = hipMalloc(&p->dev, total);
    if (e != hipSuccess) {
      delete p;
      return e == hipErrorOutOfMemory ? fail(MLA_ERR_OUT_OF_MEMORY, "hipMalloc of the plan schedule failed")
                                      : hip_fail(e, "hipMalloc");
    }
    e = hipMemcpy(p->dev, host.data(), total, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(p->dev);
      delete p;
      return hip_fail(e, "hipMemcpy of the plan schedule");
    }
  }
  *plan_out = p;
  g_last_error.clear();
  return MLA_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Workspace checks shared by the entry points; splits it into the partial
// outputs and the partial lse arrays.
mla_status check_workspace(const mla_plan* plan, void* workspace, size_t workspace_bytes, float** ws_o,
                           float** ws_lse) {
  const mla::PlanData& d = plan->d;
  const size_t need = mla::workspace_bytes(d);
  *ws_o = nullptr;
  *ws_lse = nullptr;
  if (need == 0) return MLA_OK;
  if (!workspace)
    return fail(MLA_ERR_INVALID_ARGUMENT, "workspace is NULL but the plan needs " + std::to_string(need) + " bytes");
  if (workspace_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                "workspace has " + std::to_string(workspace_bytes) + " bytes, the plan needs " + std::to_string(need));
  if (!aligned(workspace, 256)) return fail(MLA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  const size_t slots = (size_t)d.num_partials * d.nrb;
  const size_t o_bytes = align256(slots * d.v.rows_per_block() * 512 * sizeof(float));
  *ws_o = static_cast<float*>(workspace);
  *ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + o_bytes);
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

template <int NSTAGE, bool SINGLE_PAGE>
hipError_t launch_decode(const mla_plan* plan, const void* q_nope, const void* q_pe, const void* cache,
                         int64_t num_pages, const int32_t* bt, int32_t bt_stride, const int32_t* seq_lens,
                         float scale_log2, float* out, float* lse, float* ws_o, float* ws_lse,
                         hipStream_t stream) {
  const mla::PlanData& d = plan->d;
  const char* base = static_cast<const char*>(plan->dev);
  int page_log2 = 0;
  while ((1 << page_log2) < d.page) ++page_log2;
  hipLaunchKernelGGL((mla::decode_kernel<NSTAGE, SINGLE_PAGE>), dim3(d.grid), dim3(64 * mla::kWaves), 0, stream,
                     static_cast<const uint16_t*>(q_nope), static_cast<const uint16_t*>(q_pe),
                     static_cast<const uint8_t*>(cache), num_pages, bt, bt_stride, seq_lens,
                     reinterpret_cast<const int32_t*>(base + plan->off_lens),
                     reinterpret_cast<const mla::Segment*>(base + plan->off_segs),
                     reinterpret_cast<const mla::WorkgroupRange*>(base + plan->off_wgs), scale_log2, d.rows,
                     d.heads, d.q_len, page_log2, d.nrb, out, lse, ws_o, ws_lse);
  return hipGetLastError();
}

}  // namespace

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
  if (!plan) return;
  if (plan->dev) (void)hipFree(plan->dev);
  delete plan;
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

mla_status mla_decode_partials(const mla_plan* plan, const void* q_nope_absorbed, const void* q_pe,
                               const void* kv_cache, int64_t num_pages, const int32_t* block_table, int32_t bt_stride,
                               const int32_t* seq_lens, float softmax_scale, float* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
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
  float* ws_o = nullptr;
  float* ws_lse = nullptr;
  mla_status st_ws = check_workspace(plan, workspace, workspace_bytes, &ws_o, &ws_lse);
  if (st_ws != MLA_OK) return st_ws;
  mla_status st_dev = check_device(plan);
  if (st_dev != MLA_OK) return st_dev;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const float scale_log2 = softmax_scale * 1.44269504088896340736f;
  const bool single = d.page >= d.v.tile_tokens;
  if (d.v.waves != mla::kWaves || d.v.tile_tokens != mla::kTile) return fail(MLA_ERR_UNSUPPORTED, "plan variant has no kernel");
  hipError_t e = single ? launch_decode<4, true>(plan, q_nope_absorbed, q_pe, kv_cache, num_pages, block_table, bt_stride,
                                                 seq_lens, scale_log2, out, lse, ws_o, ws_lse, st)
                        : launch_decode<4, false>(plan, q_nope_absorbed, q_pe, kv_cache, num_pages, block_table,
                                                  bt_stride, seq_lens, scale_log2, out, lse, ws_o, ws_lse, st);
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  g_last_error.clear();
  return MLA_OK;
}

mla_status mla_decode_combine(const mla_plan* plan, float* out, float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!plan) return fail(MLA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!out || !lse) return fail(MLA_ERR_INVALID_ARGUMENT, "a tensor pointer is NULL");
  if (!aligned(out, 16) || !aligned(lse, 4)) return fail(MLA_ERR_INVALID_ARGUMENT, "out must be 16-byte aligned");
  float* ws_o = nullptr;
  float* ws_lse = nullptr;
  mla_status st_ws = check_workspace(plan, workspace, workspace_bytes, &ws_o, &ws_lse);
  if (st_ws != MLA_OK) return st_ws;
  mla_status st_dev = check_device(plan);
  if (st_dev != MLA_OK) return st_dev;
  const mla::PlanData& d = plan->d;
  if (!d.jobs.empty()) {
    const char* base = static_cast<const char*>(plan->dev);
    hipLaunchKernelGGL(mla::combine_kernel, dim3((unsigned)d.jobs.size(), (unsigned)((d.rows + 1) / 2)), dim3(256),
                       0, static_cast<hipStream_t>(stream),
                       reinterpret_cast<const mla::CombineJob*>(base + plan->off_jobs), ws_o, ws_lse, d.rows,
                       d.v.rows_per_block(), d.nrb, out, lse);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  }
  g_last_error.clear();
  return MLA_OK;
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

}  // extern "C"
