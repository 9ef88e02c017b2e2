// Internal layout of a split plan, shared by the host planner and the kernel
// launcher.  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

namespace mla {

// One piece of work: key range [kv_begin, kv_end) of request b.  partial < 0
// means the piece is the whole request and writes the final output; otherwise
// it writes partial slot (partial * nrb + row_block) of the workspace.
struct Segment {
  int32_t b, kv_begin, kv_end, partial;
};

// The pieces workgroup w runs, in order, for one row block.
struct WorkgroupRange {
  int32_t seg_begin, seg_end, row_block, pad;
};

// One split request for the combine kernel: partial ids p0 .. p0 + n - 1.
struct CombineJob {
  int32_t b, p0, n, pad;
};

// One combine workgroup: rows row0 .. row0 + kCombineSmallRows - 1 (short
// kernel) or row row0 (long kernel) of request b, whose pieces are partials
// p0 .. p0 + n - 1.  n = 0 marks an empty launch slot.
struct CombineUnit {
  int32_t b, p0, n, row0;
};

// Kernel shape a plan is made for.
struct Variant {
  int32_t waves;           // waves per workgroup (32 query rows each)
  int32_t tile_tokens;     // keys per LDS tile
  int32_t wg_per_cu;       // workgroups resident per compute unit
  int32_t rows_per_block() const { return 32 * waves; }
};

constexpr int32_t kNumXcd = 8;       // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr int32_t kMaxQLen = 8;
constexpr int32_t kMaxHeads = 128;
constexpr int32_t kMaxRows = 1024;
constexpr int32_t kMaxSeqLen = 1 << 24;
// Requests split into at most this many pieces are merged by the short
// combine kernel, one wave per row and kCombineSmallRows rows per workgroup.
constexpr int32_t kCombineSmallMax = 16;
constexpr int32_t kCombineSmallRows = 4;

struct PlanData {
  int32_t batch = 0, q_len = 0, heads = 0, page = 0, num_cus = 0;
  int32_t rows = 0, nrb = 0;
  Variant v{};
  int32_t max_pages = 0;  // max_b ceil(L_b / page)
  int32_t num_partials = 0;
  int32_t max_pieces = 0;   // most pieces of one split request (combine kernel choice)
  int32_t grid = 0;       // decode-kernel workgroups (>= wgs actually used)
  std::vector<int32_t> lens;
  std::vector<Segment> segs;
  std::vector<WorkgroupRange> wgs;  // size grid
  std::vector<CombineJob> jobs;
  // combine workgroups in launch order (workgroup i runs on XCD i % kNumXcd)
  std::vector<CombineUnit> cunits;
};

// Tunables of the planner (exposed for tests; defaults used by the ABI).
struct PlanTuning {
  double seg_overhead_tiles = 8.0;  // cost of one extra piece, in 32-key tiles
  double min_fragment_tiles = 4.0;  // do not start a piece smaller than this when splitting
  int32_t variant = 0;              // 0 = automatic (1); 1 = 4 waves x 32-key tiles (bf16 kernel);
                                    // 2 = 4 waves x 64-key tiles (FP8 kernel)
};

// Validate and build the host schedule.  Returns 0 on success, otherwise an
// mla_status value with `err` filled in.
int build_plan(const int32_t* lens, int32_t batch, int32_t q_len, int32_t heads, int32_t page,
               int32_t num_cus, const PlanTuning& tuning, PlanData* out, std::string* err);

// Byte offsets of the workspace parts (all zero when no request is split).
struct WorkspaceLayout {
  size_t off_o = 0, off_lse = 0, off_f = 0, total = 0;
};
WorkspaceLayout workspace_layout(const PlanData& p);
size_t workspace_bytes(const PlanData& p);

}  // namespace mla
