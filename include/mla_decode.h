/*
 * mla_decode.h -- C ABI of libmla_decode.so: weight-absorbed MLA decode
 * attention (DeepSeek-V3/R1 Multi-head Latent Attention) over a paged latent
 * cache, flash-decoding style, for AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  Decode-time MLA in its weight-absorbed form, as
 * the Huawei report "DeepSeek V3/R1 inference deployment best practices on
 * Ascend servers" runs it (section 3.2.1: decode MLA with data parallelism and
 * weight absorption; every head shares the compressed KV cache; section 6.1:
 * a FlashAttention-style tiled attention operator; section 7.2: the
 * (576 + 512) x 128-head work per key).  For request b, query token j and
 * head h, with q = [q_nope_absorbed[b,j,h,0:512] | q_pe[b,j,h,0:64]] and the
 * 576-wide cached row K_t of token t (V_t = its first 512 values):
 *     n   = seq_lens[b] - q_len + 1 + j            (keys visible to query j)
 *     s_t = softmax_scale * (q . K_t),  t < n
 *     lse[b,j,h]    = ln sum_t exp(s_t)
 *     out[b,j,h,:]  = sum_t exp(s_t - lse) * V_t
 * The key range of each request is cut into pieces that run on different
 * workgroups; the pieces are merged with a log-sum-exp combine (the
 * flash-decoding split named in the Ascend troubleshooting note on decode TPOT
 * jitter, section 4.2(3)).  How the range is cut is chosen by a planner that
 * looks at all sequence lengths at once, so that a batch mixing long and short
 * requests, or a single very long request, still fills every compute unit
 * (the same note, section 5.1, names sequence-length-aware scheduling as the
 * cure for the imbalance it diagnosed).
 *
 * Conventions
 *  - bf16 = IEEE bfloat16 bits, fp32 = IEEE binary32.  All tensors are dense,
 *    row-major (C order), with the shapes given below.
 *  - "device" pointers point to memory of the current HIP device; "host"
 *    pointers to ordinary host memory.  The caller owns every buffer it
 *    passes; the library never frees or retains them beyond the call.
 *  - Functions return an mla_status; none aborts, exits or throws.  On failure
 *    mla_last_error() gives a human-readable detail (thread-local).
 *  - Nothing here synchronizes the device.  Faults inside a kernel surface at
 *    the caller's next synchronization.
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1,   /* a null pointer, a bad size, a plan/argument mismatch  */
  MLA_ERR_UNSUPPORTED = 2,        /* a shape this build does not implement                  */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,/* workspace_bytes < mla_decode_workspace_bytes(plan)     */
  MLA_ERR_HIP = 4,                /* a HIP runtime call failed; detail in mla_last_error()  */
  MLA_ERR_OUT_OF_MEMORY = 5       /* host or device allocation failed while planning        */
} mla_status;

/* Opaque split plan.  Changed only by mla_decode_plan_update; otherwise it may
 * be shared by any number of mla_decode calls (e.g. by every layer of one
 * decode step), concurrently too, as long as concurrent calls use separate
 * workspaces. */
typedef struct mla_plan mla_plan;

/*
 * mla_decode_plan -- choose how the key ranges are split across workgroups.
 *
 *  seq_lens_host  host int32 [batch]: cached tokens of each request, counting
 *                 the q_len new tokens (already written to the cache).  Each
 *                 must satisfy q_len <= seq_lens_host[b] <= 2^24.
 *  batch          >= 1.
 *  q_len          query tokens per request, 1 <= q_len <= 8 (2 = one MTP draft
 *                 token; query j sees one key more than query j-1).
 *  num_heads      1 <= num_heads <= 128, and q_len * num_heads <= 1024.
 *  page_size      tokens per cache page: a power of two, 16 <= page_size <= 4096.
 *  num_cus        compute units to plan for, at most 65536; 0 = ask the
 *                 current device.
 *  plan_out       receives the new plan (set to NULL on failure).
 *
 * Allocates host memory, pinned host memory and a small device buffer holding
 * the schedule (hipMalloc, hipHostMalloc and a synchronous hipMemcpy on the
 * current device); per-step re-planning without any of these is
 * mla_decode_plan_update.  Release with mla_decode_plan_destroy.  Errors:
 * MLA_ERR_INVALID_ARGUMENT, MLA_ERR_UNSUPPORTED, MLA_ERR_OUT_OF_MEMORY,
 * MLA_ERR_HIP.
 */
mla_status mla_decode_plan(const int32_t* seq_lens_host, int32_t batch, int32_t q_len,
                           int32_t num_heads, int32_t page_size, int32_t num_cus,
                           mla_plan** plan_out);

/*
 * mla_decode_plan_update -- re-plan in place for new sequence lengths, for a
 * serving loop that re-plans every decode step: same batch, q_len, num_heads,
 * page_size and CU count as at creation, new seq_lens_host (host int32
 * [batch], checked as in mla_decode_plan).  Allocates nothing and never
 * synchronizes the device: the new schedule is copied to the plan's device
 * memory with hipMemcpyAsync on `stream` (hipStream_t; NULL = the default
 * stream) from pinned host memory the plan owns (reserved at creation, sized
 * for the largest schedule of its shape).  Stream order decides which
 * schedule a call sees: decode calls enqueued on `stream` before the update
 * run the old schedule, later ones the new.  Only the host waits, and only
 * for the previous update's copy to have left the pinned memory.  Callers
 * must not update a plan while another thread uses it, nor while calls on
 * other streams may still read it.  mla_decode_workspace_bytes may change:
 * query it again.  Errors: MLA_ERR_INVALID_ARGUMENT (NULL arguments, lengths
 * out of range, a plan from a _plan_host call, another current device; the
 * plan is unchanged), MLA_ERR_UNSUPPORTED (the schedule exceeds the reserved
 * room -- not expected, the room is the bound; the plan is unchanged),
 * MLA_ERR_HIP (the copy could not be enqueued; destroy the plan).
 */
mla_status mla_decode_plan_update(mla_plan* plan, const int32_t* seq_lens_host, void* stream);

/* Same as mla_decode_plan but makes no HIP call at all (num_cus must be > 0):
 * the plan can be inspected with mla_plan_query but not run (mla_decode then
 * returns MLA_ERR_INVALID_ARGUMENT).  For host-side tools and tests. */
mla_status mla_decode_plan_host(const int32_t* seq_lens_host, int32_t batch, int32_t q_len,
                                int32_t num_heads, int32_t page_size, int32_t num_cus,
                                mla_plan** plan_out);

/* Bytes of device workspace mla_decode needs with this plan (0 if no request
 * is split).  The workspace holds one partial per piece of every split
 * request: rows x 512 values in fp16 (scaled per row so that no value
 * overflows), plus a log-sum-exp and a scale factor per row in fp32. */
size_t mla_decode_workspace_bytes(const mla_plan* plan);

/*
 * mla_decode -- enqueue the decode attention for one layer on `stream`.
 *
 *  plan             from mla_decode_plan with the same seq_lens, q_len,
 *                   num_heads and page_size.
 *  q_nope_absorbed  device bf16 [B, q_len, H, 512]; 16-byte aligned.
 *                   The query's no-rope part already multiplied by W_UK^T.
 *  q_pe             device bf16 [B, q_len, H, 64]; 16-byte aligned; post-RoPE.
 *  kv_cache         device bf16 [num_pages, page_size, 576]; 16-byte aligned.
 *                   Row = [c_kv (512) | k_pe (64)]; V is the c_kv part.
 *  num_pages        pages in kv_cache (> 0).  A page id outside [0, num_pages)
 *                   is never followed: the request whose block-table entry it
 *                   is gets NaN in all of its out and lse (loud, no fault);
 *                   other requests are unaffected.
 *  block_table      device int32 [B, bt_stride]: token t of request b lives in
 *                   slot t % page_size of page block_table[b, t / page_size].
 *                   Entries past ceil(seq_lens[b] / page_size) are never read;
 *                   pages may be shared between requests (read only).
 *  bt_stride        row stride of block_table, >= max_b ceil(seq_lens[b] / page_size).
 *  seq_lens         device int32 [B]; must equal the lengths the plan was made
 *                   with.  A request whose device length differs gets NaN in
 *                   out and lse (loud, never an out-of-bounds access).
 *  softmax_scale    finite, > 0 (1/sqrt(192) for DeepSeek-V3's 128 + 64 head dims).
 *  out              device fp32 [B, q_len, H, 512], 16-byte aligned (normalized output).
 *  lse              device fp32 [B, q_len, H]: natural log of the sum of exp of
 *                   the scaled scores.
 *  workspace        device buffer of >= mla_decode_workspace_bytes(plan) bytes,
 *                   256-byte aligned (may be NULL when that size is 0).
 *                   Contents on entry are ignored; it is scratch for this call.
 *  stream           hipStream_t to enqueue on; NULL = the default stream.
 *
 * Enqueues at most two kernels and nothing else (no memset, no copy), allocates
 * nothing, never synchronizes, so a call may be captured in a HIP graph and
 * replayed (the graph then holds the plan's and buffers' addresses).  The
 * result is deterministic for a given plan.  Argument checks run on the host
 * before any HIP call.  Errors: MLA_ERR_INVALID_ARGUMENT,
 * MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_HIP (launch failure).
 */
mla_status mla_decode(const mla_plan* plan,
                      const void* q_nope_absorbed, const void* q_pe,
                      const void* kv_cache, int64_t num_pages,
                      const int32_t* block_table, int32_t bt_stride,
                      const int32_t* seq_lens, float softmax_scale,
                      float* out, float* lse,
                      void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * mla_decode_noalloc -- mla_decode for callers that cannot allocate device
 * memory at call time (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation and arguments
 * without the workspace.  The partials of split requests go to a scratch
 * array the library holds in device memory, 64 MiB per GPU (one copy per
 * device the library runs on, kept until the process ends; its address is
 * looked up on the first call on each device).  Allocates nothing and never
 * synchronizes.
 *  - A plan whose mla_decode_workspace_bytes exceeds 64 MiB is refused with
 *    MLA_ERR_WORKSPACE_TOO_SMALL before any HIP call.
 *  - Every call on one GPU shares that GPU's scratch and leaves its contents
 *    behind: calls that overlap in time on the same GPU (different streams
 *    without ordering between them) race and give wrong results.  Calls on one
 *    stream, or otherwise ordered, are safe.  No part of the scratch needs to
 *    start at zero.
 * Errors: as for mla_decode (MLA_ERR_INVALID_ARGUMENT, MLA_ERR_WORKSPACE_TOO_SMALL,
 * MLA_ERR_UNSUPPORTED for device ids beyond 63, MLA_ERR_HIP).
 */
mla_status mla_decode_noalloc(const mla_plan* plan,
                              const void* q_nope_absorbed, const void* q_pe,
                              const void* kv_cache, int64_t num_pages,
                              const int32_t* block_table, int32_t bt_stride,
                              const int32_t* seq_lens, float softmax_scale,
                              float* out, float* lse, void* stream);

/*
 * The two halves of mla_decode, for callers that want to time, reorder or
 * overlap them.  mla_decode == mla_decode_partials followed by
 * mla_decode_combine on the same stream, with the same plan and workspace.
 *
 * mla_decode_partials -- the split decode kernel alone.  Same arguments and
 *   checks as mla_decode.  Requests the plan keeps in one piece get their final
 *   out/lse; pieces of split requests leave normalized partials in the workspace.
 * mla_decode_combine -- merges the partials of split requests into out/lse
 *   (the log-sum-exp combine).  A no-op kernel-wise when nothing is split.
 *   out/lse as for mla_decode; the workspace must hold what the partials call
 *   left there.  Errors: MLA_ERR_INVALID_ARGUMENT, MLA_ERR_WORKSPACE_TOO_SMALL,
 *   MLA_ERR_HIP.
 */
mla_status mla_decode_partials(const mla_plan* plan,
                               const void* q_nope_absorbed, const void* q_pe,
                               const void* kv_cache, int64_t num_pages,
                               const int32_t* block_table, int32_t bt_stride,
                               const int32_t* seq_lens, float softmax_scale,
                               float* out, float* lse,
                               void* workspace, size_t workspace_bytes,
                               void* stream);
mla_status mla_decode_combine(const mla_plan* plan, float* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_decode_variant -- mla_decode with a choice of how the online softmax
 * rescales O, and an optional count of the rescales.
 *
 * The Huawei report ("DeepSeek V3/R1 inference deployment best practices on
 * Ascend servers", section 6.1 on the MLA operator, the AMLA bullet) turns the
 * multiplicative update of O into an additive one by working on the float's
 * binary encoding.  Here both forms keep a lazy reference (a row moves it only
 * when its maximum grows by more than 2^8):
 *  variant MLA_RESCALE_LAZY (0): the reference is the row maximum itself and
 *    O, l are multiplied by 2^(mu_old - mu_new) (what mla_decode runs);
 *  variant MLA_RESCALE_POW2 (1): the reference is the row maximum rounded up
 *    to an integer (log2 units), so the factor is an exact power of two and O,
 *    l are updated by adding to their exponents (v_ldexp_f32, which also keeps
 *    zeros and underflow right); l sums the bf16-rounded weights that multiply
 *    V (with an integer reference even a row's largest weight is rounded, and
 *    one set of weights keeps O / l a weighted mean).
 * Both give the same result up to rounding (each within the bar of mla_decode).
 *  rescale_events   NULL, or a device uint32 that the call adds to: one per
 *                   wave (32 query rows) and tile after which that wave
 *                   rescaled its O; 4-byte aligned; the caller zeroes it.
 * Other arguments, checks and errors as for mla_decode; an unknown variant is
 * MLA_ERR_INVALID_ARGUMENT.
 */
#define MLA_RESCALE_LAZY 0
#define MLA_RESCALE_POW2 1
mla_status mla_decode_variant(const mla_plan* plan,
                              const void* q_nope_absorbed, const void* q_pe,
                              const void* kv_cache, int64_t num_pages,
                              const int32_t* block_table, int32_t bt_stride,
                              const int32_t* seq_lens, float softmax_scale,
                              float* out, float* lse,
                              void* workspace, size_t workspace_bytes,
                              int32_t variant, uint32_t* rescale_events,
                              void* stream);

/*
 * FP8 latent cache.
 *
 * The Huawei report ("DeepSeek V3/R1 inference deployment best practices on
 * Ascend servers", section 8 on next steps, the bullet on quantized MLA
 * operators) names 8-bit keys and values as future work for MLA decode; these
 * entry points take the cache in the OCP FP8 formats
 * that gfx950's matrix cores read.  Same computation and output as
 * mla_decode, except:
 *
 *  kv_codes   device uint8 [num_pages, page_size, 576]; 16-byte aligned.
 *             E4M3 ("fn": bias 7, max 448, S.1111.111 = NaN) codes of the
 *             row [c_kv (512) | k_pe (64)].
 *  kv_scales  device uint8 [num_pages, page_size]; 4-byte aligned.  E8M0
 *             scale of each token: row value = 2^(e - 127) * decode(code).
 *             e must be <= 254 (255 is NaN in E8M0).
 *  q_nope_absorbed, q_pe stay bf16; each block of 32 consecutive values of a
 *             576-wide query row is quantized in the kernel to E4M3 codes
 *             with its own E8M0 exponent (OCP MXFP8): f = the smallest
 *             integer with max|q| * 2^-f <= 448, limited to [-127, 127],
 *             codes = round-to-nearest-even of q * 2^-f (saturated at 448).
 *
 * The softmax weights are rounded to E4M3 for the PV product (each tile's
 * largest weight scaled into [64, 128)); the output therefore carries a
 * relative error of a few percent of the weights' rounding, averaged over
 * the keys; lse is unaffected.  Scores (softmax_scale * q . k) must stay
 * below ~2^19 in magnitude, where fp32 still resolves their differences
 * (per-token scales allow far larger values; results are then not defined).
 *
 * mla_decode_fp8_plan / _plan_host: as mla_decode_plan / _plan_host, for the
 *   FP8 kernel (64-key tiles).  A plan of one kind is refused by the other
 *   kind's decode calls (MLA_ERR_INVALID_ARGUMENT); mla_decode_combine,
 *   mla_decode_workspace_bytes and the inspection calls take either.
 * mla_decode_fp8 == mla_decode_fp8_partials + mla_decode_combine.
 * Errors as for mla_decode.
 */
mla_status mla_decode_fp8_plan(const int32_t* seq_lens_host, int32_t batch, int32_t q_len,
                               int32_t num_heads, int32_t page_size, int32_t num_cus,
                               mla_plan** plan_out);
mla_status mla_decode_fp8_plan_host(const int32_t* seq_lens_host, int32_t batch, int32_t q_len,
                                    int32_t num_heads, int32_t page_size, int32_t num_cus,
                                    mla_plan** plan_out);
mla_status mla_decode_fp8(const mla_plan* plan,
                          const void* q_nope_absorbed, const void* q_pe,
                          const void* kv_codes, const void* kv_scales, int64_t num_pages,
                          const int32_t* block_table, int32_t bt_stride,
                          const int32_t* seq_lens, float softmax_scale,
                          float* out, float* lse,
                          void* workspace, size_t workspace_bytes,
                          void* stream);
mla_status mla_decode_fp8_partials(const mla_plan* plan,
                                   const void* q_nope_absorbed, const void* q_pe,
                                   const void* kv_codes, const void* kv_scales, int64_t num_pages,
                                   const int32_t* block_table, int32_t bt_stride,
                                   const int32_t* seq_lens, float softmax_scale,
                                   float* out, float* lse,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * The steps next to the decode attention.
 *
 * The Huawei report (section 6.1, the operators before MLA) absorbs the
 * weights and fuses the decode prolog into one operator; the CloudMatrix384
 * digest (its MLA optimization paragraph) names RMSNorm, the projections and
 * RoPE as its parts; the report's decode flow (section 3.2.1) ends MLA with
 * the output projection, whose input is the up-projected attention output.
 *
 * mla_prolog -- for the q_len new tokens of each request (positions
 *   seq_lens[b] - q_len + j, j < q_len), enqueue on `stream`:
 *     q_nope_absorbed[b, j, h] = W_UK[h]^T q_nope128[b, j, h]        (bf16, 512)
 *     q_pe[b, j, h]            = RoPE(q_pe_raw[b, j, h])              (bf16, 64)
 *     cache row of the token   = [RMSNorm(c_kv_raw[b, j]) * kv_norm_w | RoPE(k_pe_raw[b, j])]
 *   rounded to bf16 (kv_format MLA_KV_BF16: kv_cache bf16 [num_pages,
 *   page_size, 576]) or quantized per token (MLA_KV_FP8: kv_cache uint8
 *   codes, kv_scales uint8 [num_pages, page_size]; exponent f = smallest with
 *   max|row| * 2^-f <= 448, codes = nearest-even E4M3 of row * 2^-f).
 *  q_nope128     device bf16 [B, q_len, H, 128] (16-byte aligned)
 *  q_pe_raw      device bf16 [B, q_len, H, 64], before RoPE (16-byte aligned)
 *  w_uk_t        device bf16 [H, 512, 128]: element [h, c, d] = W_UK[h][d][c]
 *                (the key up-projection, stored transposed for the absorption)
 *  c_kv_raw      device bf16 [B, q_len, 512], before the RMSNorm
 *  kv_norm_w     device bf16 [512]; rms_eps >= 0: RMSNorm(x) = x / sqrt(mean(x^2) + eps)
 *  k_pe_raw      device bf16 [B, q_len, 64], before RoPE
 *  rope_cos_sin  device fp32 [max_pos, 64] (16-byte aligned): row p holds cos of the 32 pair
 *                angles at position p, then their sin; RoPE turns the pair
 *                (x[2i], x[2i+1]) by angle i (the table carries any frequency
 *                scaling).  A position >= max_pos gives NaN in q_pe and no
 *                cache write.
 *  seq_lens, block_table, bt_stride, num_pages, page_size: as for
 *                mla_decode (lengths include the new tokens); a token whose
 *                page id is outside [0, num_pages) is not written.
 *  q_nope_absorbed, q_pe: device bf16 outputs [B, q_len, H, 512] / [.., 64],
 *                16-byte aligned.  batch * q_len <= 2^21; the other
 *                pointers 4-byte aligned.
 * One kernel, no allocation, no synchronization.  Errors:
 * MLA_ERR_INVALID_ARGUMENT, MLA_ERR_HIP.
 *
 * mla_up_project -- o[b, j, h] = W_UV[h] attn_out[b, j, h] (bf16, 128 per
 *   head; the output projection's input; the fp32 input is rounded to bf16
 *   for the bf16 MFMA).  attn_out: device fp32
 *   [B, q_len, H, 512] (mla_decode's out), 16-byte aligned; w_uv: device bf16
 *   [H, 128, 512], 16-byte aligned; o: device bf16 [B, q_len, H, 128],
 *   8-byte aligned; batch * q_len <= 2^21.  One kernel.
 *
 * mla_o_project -- the output projection that closes the attention block
 *   (the Huawei report's decode flow, section 3.2.1, ends MLA with it):
 *     y[b, j, :] = W_O x[b, j, :],  x = the up-projected heads concatenated
 *   in head order (mla_up_project's o viewed as [B * q_len, H * 128]).
 *  x          device bf16 [B * q_len, k_in], 16-byte aligned (k_in = H * 128:
 *             a multiple of 256 up to 2^20)
 *  w_o        device bf16 [n_out, k_in] (row n = output n, as a linear layer
 *             stores it), 16-byte aligned; n_out a multiple of 64 up to 2^22
 *  y          device bf16 [B * q_len, n_out], 8-byte aligned
 *  workspace  device, 16-byte aligned, at least
 *             mla_o_project_workspace_bytes(batch, q_len, k_in, n_out) bytes
 *             (fp32 partial sums over slices of k_in; contents not kept)
 *  batch * q_len * n_out <= 2^28.  Two kernels (fp32 accumulation, the sum
 *  rounded to bf16), no allocation, no synchronization.  Errors:
 *  MLA_ERR_INVALID_ARGUMENT, MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_HIP.
 *  mla_o_project_workspace_bytes returns 0 for sizes mla_o_project refuses.
 */
enum { MLA_KV_BF16 = 0, MLA_KV_FP8 = 1 };
mla_status mla_prolog(int32_t batch, int32_t q_len, int32_t num_heads,
                      const void* q_nope128, const void* q_pe_raw, const void* w_uk_t,
                      const void* c_kv_raw, const void* kv_norm_w, float rms_eps,
                      const void* k_pe_raw, const float* rope_cos_sin, int32_t max_pos,
                      const int32_t* seq_lens, const int32_t* block_table, int32_t bt_stride,
                      int64_t num_pages, int32_t page_size, int32_t kv_format,
                      void* kv_cache, void* kv_scales,
                      void* q_nope_absorbed, void* q_pe, void* stream);
mla_status mla_up_project(int32_t batch, int32_t q_len, int32_t num_heads,
                          const float* attn_out, const void* w_uv, void* o, void* stream);
size_t mla_o_project_workspace_bytes(int32_t batch, int32_t q_len, int32_t k_in, int32_t n_out);
mla_status mla_o_project(int32_t batch, int32_t q_len, int32_t k_in, int32_t n_out,
                         const void* x, const void* w_o, void* y,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Free a plan (its host memory, pinned staging memory and device schedule;
 * waits for its last schedule upload).  NULL is a no-op.  The plan must not be
 * in use by a kernel still running. */
void mla_decode_plan_destroy(mla_plan* plan);

/* Static description of a status code. */
const char* mla_status_string(mla_status s);

/* Detail of the last failure on this thread ("" if none). */
const char* mla_last_error(void);

/*
 * Plan inspection (host only; for tests and tools).
 *  MLA_Q_NUM_SEGMENTS     number of (request, key range) pieces
 *  MLA_Q_NUM_WORKGROUPS   grid size of the decode kernel
 *  MLA_Q_NUM_PARTIALS     pieces that write a partial (0 when nothing is split)
 *  MLA_Q_ROWS_PER_BLOCK   query rows (q_len*H flattened) one workgroup holds
 *  MLA_Q_TILE_TOKENS      keys per tile
 *  MLA_Q_NUM_ROW_BLOCKS   row blocks per request
 *  MLA_Q_NUM_COMBINE_WGS  grid size of the combine kernel (0 when nothing is split)
 * mla_plan_query returns the value (or -1 for an unknown key / NULL plan).
 */
enum { MLA_Q_NUM_SEGMENTS = 0, MLA_Q_NUM_WORKGROUPS = 1, MLA_Q_NUM_PARTIALS = 2,
       MLA_Q_ROWS_PER_BLOCK = 3, MLA_Q_TILE_TOKENS = 4, MLA_Q_NUM_ROW_BLOCKS = 5,
       MLA_Q_NUM_COMBINE_WGS = 6 };
int64_t mla_plan_query(const mla_plan* plan, int32_t key);

/* Copy the pieces out: for segment i, seg[4*i + 0..3] = {request, first key,
 * end key (exclusive), partial id or -1 when the piece is the whole request}.
 * wg[4*w + 0..3] = {first segment, end segment, row block, 0} for workgroup w.
 * Either pointer may be NULL.  Returns MLA_ERR_INVALID_ARGUMENT for a NULL plan. */
mla_status mla_plan_copy(const mla_plan* plan, int32_t* seg, int32_t* wg);

/* Copy the combine kernel's workgroups out (host only; for tests and tools):
 * unit[4*i + 0..3] = {request, first partial id, pieces (0 = empty slot),
 * first query row} for combine workgroup i, which the hardware places on XCD
 * i % 8.  A workgroup merges 4 rows when no request has more than 16 pieces,
 * else one.  `unit` holds MLA_Q_NUM_COMBINE_WGS entries of 4 int32 (caller
 * owned); NULL is allowed.  Returns MLA_ERR_INVALID_ARGUMENT for a NULL plan. */
mla_status mla_plan_copy_combine(const mla_plan* plan, int32_t* unit);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H_ */
