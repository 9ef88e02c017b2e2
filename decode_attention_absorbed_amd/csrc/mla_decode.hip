// Weight-absorbed MLA decode attention for gfx950 (MI355X): split-KV decode
// kernel, log-sum-exp combine kernel and the C ABI around them.
//
// The computation (Huawei, "DeepSeek V3/R1 inference deployment best practices
// on Ascend servers", section 3.2.1 and section 6.1): every head of a request
// attends over the same cached 576-wide rows [c_kv | k_pe]; V is c_kv.  With
// the heads as the M dimension, QK^T and PV are dense contractions against a
// shared key tile, so both run on bf16 MFMA with fp32 accumulation.
//
// Decode kernel, one workgroup = NW waves = 32*NW query rows (rows are the
// flattened (query token, head) pairs of one request), walking one or more
// pieces of key range:
//  * a tile of TILE keys x 576 bf16 is copied HBM -> LDS with 16-byte direct
//    loads (global_load_lds_dwordx4), double buffered, one barrier per tile.
//    Rows are stored with a 16-byte pad (1168 B stride) so that both the
//    row-wise reads of QK^T and the transposed reads of PV hit distinct banks;
//  * wave w keeps its 32 query rows, as the B operand of
//    v_mfma_f32_32x32x16_bf16, in 144 VGPRs for the whole piece, and computes
//    S^T = K Q^T for 32 keys at a time (A operand = key rows read from LDS);
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

constexpr int kRowBytesHbm = 576 * 2;  // one cached token
constexpr int kChunksHbm = 72;         // 16-byte chunks per cached token
constexpr int kChunksLds = 73;         // plus one pad chunk in LDS
constexpr int kRowBytesLds = kChunksLds * 16;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units

template <int NW, int TILE>
struct Shape {
  static constexpr int kThreads = 64 * NW;
  static constexpr int kRowsPerBlock = 32 * NW;
  static constexpr int kBlocks = TILE / 32;            // 32-key MFMA blocks per tile
  static constexpr int kKSteps = TILE / 16;            // 16-key PV steps per tile
  static constexpr int kPositions = TILE * kChunksLds; // 16-byte LDS slots per tile
  static constexpr int kLoads = (kPositions + 63) / 64;
  static constexpr int kLoadsPerWave = (kLoads + NW - 1) / NW;
  static constexpr int kBufBytes = kLoads * 1024;
  static_assert(TILE == 32 || TILE == 64, "tile is 32 or 64 keys");
};

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

__device__ __forceinline__ void wait_vmem_all() {
  // s_waitcnt vmcnt(0) (expcnt, lgkmcnt at their maxima).  It also covers the
  // LDS copies issued as inline asm; issued as the builtin so that the
  // compiler's own wait-count bookkeeping sees that every load has landed.
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

// The S^T accumulators are pinned to VGPRs (the softmax reads them with VALU
// right away) while the output accumulators live in AGPRs; the compiler left to
// itself puts both in AGPRs and spills.  So the QK^T MFMA is issued as inline
// asm with a VGPR constraint.  The hazards the compiler cannot see inside the
// asm are handled here: the first step takes srcC = 0 (no VALU write of the
// accumulator right before an MFMA reads it), and s_mfma_drain waits out the
// XDL-write -> VALU-read latency (at most 18 wait states for a 16-pass MFMA)
// before anything reads the results.
// Like every MFMA issued as asm here it starts with s_nop 1: a VALU write of a
// source register (e.g. a zeroed query row) needs two wait states before an
// MFMA reads it, and the compiler adds none around inline asm.
__device__ __forceinline__ void s_mfma(f32x16& acc, const bf16x8& a, const bf16x8& b, bool first) {
  if (first)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// The output accumulators O^T (16 tiles of 32x32 fp32 = 256 registers per
// lane) live in the physical AGPRs a[0:255]: tile cb is a[16cb : 16cb+15].
// They are only touched by inline asm that names them and lists them as
// clobbered, so the compiler never allocates them (left to itself it carries
// them through VGPRs around the rare rescale branch and spills the query rows).
// Hazards the compiler cannot see are handled where the code runs:
//  * MFMA -> accvgpr_read of the results: o_drain waits 24 wait states;
//  * accvgpr_write (rescale) -> MFMA srcC: the whole softmax runs in between,
//    plus an s_nop at the head of the PV loop;
//  * VALU-written P operand -> MFMA srcA/B: same s_nop.
template <int CB>
struct OTile;
template <int N>
__device__ __forceinline__ float o_get();
template <int N>
__device__ __forceinline__ void o_set(float x);
#include "agpr_tiles.inc"

// Dispatch on a tile index that is a constant after unrolling.
__device__ __forceinline__ void o_mfma(int cb, const bf16x8& a, const bf16x8& b, bool first) {
#define MLA_CASE(n)                 \
  case n:                           \
    if (first)                      \
      OTile<n>::mfma_first(a, b);   \
    else                            \
      OTile<n>::mfma(a, b);         \
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

__device__ __forceinline__ void s_mfma_drain(f32x16& acc) { asm volatile("s_nop 15\n\ts_nop 7" : "+v"(acc)); }

// 16-byte global -> LDS copies (global_load_lds_dwordx4).  Each lane names its
// own source; the 64 lanes of the wave fill 1 KB of LDS starting at M0.  They
// are issued as inline asm on purpose: the compiler's wait-count pass treats a
// pending LDS-DMA as aliasing every later LDS read and would insert
// s_waitcnt vmcnt(0) before them, serializing the copy of tile i+1 with the
// compute on tile i.  Completion is awaited explicitly (wait_vmem_all) before
// the barrier that publishes a tile.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// (s_nop 0: one wait state between the M0 write and the LDS-DMA that reads it.)
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_dst));
}

__device__ __forceinline__ void dma16_saddr(const void* base, uint32_t off, uint32_t lds_dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds_dst));
}

// Page ids a tile touches (uniform; at most 4 since pages hold >= 16 keys and
// tiles <= 64).  Out-of-range ids are replaced by page 0 so that a corrupt
// block table can never make the kernel read outside the cache.
struct TilePages {
  int first;
  int pg[4];
};

template <int NW, int TILE, bool SINGLE_PAGE>
__global__ __launch_bounds__(64 * NW, 1) void decode_kernel(
    const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
    const uint8_t* __restrict__ cache, int64_t num_pages,
    const int32_t* __restrict__ block_table, int32_t bt_stride,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ planned_lens,
    const Segment* __restrict__ segs, const WorkgroupRange* __restrict__ wgs,
    float scale_log2, int32_t rows, int32_t heads, int32_t q_len, int32_t page_log2, int32_t nrb,
    float* __restrict__ out, float* __restrict__ lse, float* __restrict__ ws_o,
    float* __restrict__ ws_lse) {
  using S = Shape<NW, TILE>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * S::kBufBytes];

  const WorkgroupRange wr = wgs[blockIdx.x];
  if (wr.seg_begin >= wr.seg_end) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;  // which 8-wide k slice of an MFMA operand this lane holds
  const int rb = wr.row_block;
  const int row_local = wave * 32 + (lane & 31);
  const int row = rb * S::kRowsPerBlock + row_local;
  const bool row_ok = row < rows;
  const int jq = row_ok ? row / heads : 0;  // query token of this row
  const int psize = 1 << page_log2;

  // Per-lane LDS byte offsets (within a buffer) of the operand reads.
  // QK^T, A operand = key rows: key (lane & 31) of the 32-key block, k slice `half`.
  const int qk_off = (lane & 31) * kRowBytesLds + half * 16;
  // PV, A operand = V^T via transposed reads: within each 16-lane group g, lane k
  // addresses key row (k / 4) of a 4-key strip, columns 4 * (k % 4) .. + 3 of a
  // 16-column strip; the read hands lane k column k of the 4 x 16 block.
  const int grp = lane >> 4, k16 = lane & 15;
  const int pv_off = (4 * half + (k16 >> 2)) * kRowBytesLds + (16 * (grp & 1) + 4 * (k16 & 3)) * 2;

  for (int si = wr.seg_begin; si < wr.seg_end; ++si) {
    const Segment sg = segs[si];
    const int b = sg.b, kv0 = sg.kv_begin, kv1 = sg.kv_end;
    const int L = seq_lens[b];
    const bool bad_len = (L != planned_lens[b]);
    const int32_t* bt_row = block_table + (int64_t)b * bt_stride;

    // Keys this row may see inside the piece: [kv0, lim).
    const int lim = row_ok ? min(kv1, L - q_len + 1 + jq) : kv0;

    // Block-table entries of a tile: loaded one tile ahead of use (scalar
    // loads), checked against num_pages when used.
    auto fetch_pages = [&](int tb) {
      TilePages tp;
      tp.first = tb >> page_log2;
      const int last = (min(tb + TILE, kv1) - 1) >> page_log2;
#pragma unroll
      for (int k = 0; k < (SINGLE_PAGE ? 1 : 4); ++k) tp.pg[k] = bt_row[min(tp.first + k, last)];
      if (SINGLE_PAGE) tp.pg[1] = tp.pg[2] = tp.pg[3] = tp.pg[0];
      return tp;
    };
    auto checked = [&](TilePages tp) {
#pragma unroll
      for (int k = 0; k < 4; ++k) tp.pg[k] = ((uint64_t)(int64_t)tp.pg[k] < (uint64_t)num_pages) ? tp.pg[k] : 0;
      return tp;
    };

    // One 1 KB direct-to-LDS copy: LDS slots [64 n, 64 n + 64) of the tile,
    // slot = 73 * key + chunk (chunk 72 is the row pad and is not loaded).
    auto dma = [&](int i, int tb, const TilePages& tp, uint8_t* lbase) {
      const int n = i * NW + wave;
      if (n < S::kLoads) {
        int lane_v = lane;
        asm volatile("" : "+v"(lane_v));  // keep the address math next to its use
        const int pos = n * 64 + lane_v;
        const int t = pos / kChunksLds;
        const int c = pos - t * kChunksLds;
        if (c < kChunksHbm && t < TILE) {
          const int tok = min(tb + t, kv1 - 1);
          const uint32_t lds_dst = lds_addr(lbase + n * 1024);
          if (SINGLE_PAGE) {
            const uint8_t* pbase = cache + ((int64_t)tp.pg[0] << page_log2) * kRowBytesHbm;
            const uint32_t off = (uint32_t)((tok & (psize - 1)) * kRowBytesHbm + c * 16);
            dma16_saddr(pbase, off, lds_dst);
          } else {
            const int k = (tok >> page_log2) - tp.first;
            const int page = k == 0 ? tp.pg[0] : (k == 1 ? tp.pg[1] : (k == 2 ? tp.pg[2] : tp.pg[3]));
            dma16(cache + (((int64_t)page << page_log2) + (tok & (psize - 1))) * kRowBytesHbm + c * 16, lds_dst);
          }
        }
      }
    };

    // All waves must be done with the previous piece's last tile before the
    // first tile of this one lands in LDS.
    __syncthreads();

    const int ntiles = (kv1 - kv0 + TILE - 1) / TILE;
    TilePages pg_next = checked(fetch_pages(kv0));
#pragma unroll
    for (int i = 0; i < S::kLoadsPerWave; ++i) dma(i, kv0, pg_next, smem);
    TilePages pg_raw = pg_next;
    if (ntiles > 1) pg_raw = fetch_pages(kv0 + TILE);

    // Query rows as the MFMA B operand: lane holds dims 16*kk + 8*half .. +7.
    bf16x8 q[36];
    if (row_ok) {
      const bf16x8* qn = reinterpret_cast<const bf16x8*>(q_nope + ((int64_t)b * rows + row) * 512);
      const bf16x8* qp = reinterpret_cast<const bf16x8*>(q_pe + ((int64_t)b * rows + row) * 64);
#pragma unroll
      for (int kk = 0; kk < 32; ++kk) q[kk] = qn[2 * kk + half];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) q[32 + kk] = qp[2 * kk + half];
    } else {
#pragma unroll
      for (int kk = 0; kk < 36; ++kk) q[kk] = bf16x8{};
    }

    float m_ref = -INFINITY;  // running reference max (log2 units), same in lanes l and l^32
    float l_part = 0.f;       // this lane's share of the running sum

    for (int it = 0; it < ntiles; ++it) {
      wait_vmem_all();
      __syncthreads();
      const bool has_next = it + 1 < ntiles;
      const int tb = kv0 + it * TILE;
      // Pages of tile it+1 (loaded during tile it-1); fetch those of tile it+2.
      if (has_next) pg_next = checked(pg_raw);
      if (it + 2 < ntiles) pg_raw = fetch_pages(tb + 2 * TILE);
      __builtin_amdgcn_sched_barrier(0);
      const uint8_t* kb = smem + (it & 1) * S::kBufBytes;
      uint8_t* nb = smem + ((it + 1) & 1) * S::kBufBytes;

      // The tile is processed in 32-key blocks: QK^T, softmax and PV per block
      // (one block's scores and probabilities in registers at a time).
#pragma unroll
      for (int blk = 0; blk < S::kBlocks; ++blk) {
        const uint8_t* kblk = kb + blk * 32 * kRowBytesLds;
        const int t0 = tb + blk * 32;

        // ---- S^T = K Q^T for 32 keys (lane: head lane&31, 16 keys); during the
        //      first block the next tile's copies are issued between the MFMAs ----
        f32x16 s;
        bf16x8 a[3];
        a[0] = *reinterpret_cast<const bf16x8*>(kblk + qk_off);
        a[1] = *reinterpret_cast<const bf16x8*>(kblk + qk_off + 32);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < 36; ++kk) {
          if (kk + 2 < 36) a[(kk + 2) % 3] = *reinterpret_cast<const bf16x8*>(kblk + qk_off + (kk + 2) * 32);
          if (blk == 0 && kk < S::kLoadsPerWave && has_next) dma(kk, tb + TILE, pg_next, nb);
          s_mfma(s, a[kk % 3], q[kk], kk == 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        s_mfma_drain(s);

        // ---- mask, scale to log2 units, block max ----
        const bool need_mask = t0 + 32 > lim;
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = s[i] * scale_log2;
          if (need_mask) {
            const int tok = t0 + (i >> 2) * 8 + half * 4 + (i & 3);
            x = tok < lim ? x : -INFINITY;
          }
          s[i] = x;
          mx = fmaxf(mx, x);
        }
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

        // ---- P = 2^(x - mu), as bf16 MFMA B operands, 8 keys per 16-key step ----
        bf16x8 pb[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(s[i] - mu);
          l_part += p;
          pb[i >> 3][i & 7] = (__bf16)p;
        }
        // Materialize the bf16 operands here, not next to the MFMAs.
        asm volatile("" : "+v"(pb[0]), "+v"(pb[1]));
        __builtin_amdgcn_sched_barrier(0);

        // ---- O^T += V^T P^T, V^T read transposed from the same block ----
        i16x8 v[3];
        auto read_v = [&](int idx) {
          const int ks = idx >> 4, cb = idx & 15;
          const uint8_t* vb = kblk + pv_off + ks * 16 * kRowBytesLds + cb * 64;
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(i16x4, vb));
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_AS(i16x4, vb + 8 * kRowBytesLds));
          return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        v[0] = read_v(0);
        v[1] = read_v(1);
        asm volatile("s_nop 4" ::: );
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int idx = 0; idx < 32; ++idx) {
          if (idx + 2 < 32) v[(idx + 2) % 3] = read_v(idx + 2);
          const int ks = idx >> 4, cb = idx & 15;
          o_mfma(cb, __builtin_bit_cast(bf16x8, v[idx % 3]), pb[ks], it == 0 && blk == 0 && ks == 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

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
        dst = ws_o + (slot * S::kRowsPerBlock + row_local) * 512;
        dl = ws_lse + slot * S::kRowsPerBlock + row_local;
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

template <int NW, int TILE, bool SINGLE_PAGE>
hipError_t launch_decode(const mla_plan* plan, const void* q_nope, const void* q_pe, const void* cache,
                         int64_t num_pages, const int32_t* bt, int32_t bt_stride, const int32_t* seq_lens,
                         float scale_log2, float* out, float* lse, float* ws_o, float* ws_lse,
                         hipStream_t stream) {
  const mla::PlanData& d = plan->d;
  const char* base = static_cast<const char*>(plan->dev);
  int page_log2 = 0;
  while ((1 << page_log2) < d.page) ++page_log2;
  hipLaunchKernelGGL((mla::decode_kernel<NW, TILE, SINGLE_PAGE>), dim3(d.grid), dim3(64 * NW), 0, stream,
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
  hipError_t e;
#define MLA_LAUNCH(NW, TILE, SP)                                                                                 \
  launch_decode<NW, TILE, SP>(plan, q_nope_absorbed, q_pe, kv_cache, num_pages, block_table, bt_stride, seq_lens, \
                              scale_log2, out, lse, ws_o, ws_lse, st)
  if (d.v.waves == 4 && d.v.tile_tokens == 64)
    e = single ? MLA_LAUNCH(4, 64, true) : MLA_LAUNCH(4, 64, false);
  else if (d.v.waves == 2 && d.v.tile_tokens == 32)
    e = single ? MLA_LAUNCH(2, 32, true) : MLA_LAUNCH(2, 32, false);
  else
    return fail(MLA_ERR_UNSUPPORTED, "plan variant has no kernel");
#undef MLA_LAUNCH
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
