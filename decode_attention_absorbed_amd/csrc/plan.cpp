// Host-side split planner for absorbed-MLA decode.
//
// Problem: B requests of very different lengths (a 20K/400 mix, or one 128K
// request) must keep every compute unit busy for about the same time.  The
// Ascend troubleshooting note on decode TPOT jitter (section 4.2(3)) traces a
// latency spike to a flash-decoding split that did not trigger for such a mix,
// and names length-aware scheduling as the fix (section 5.1).  Here the plan
// looks at all lengths at once:
//
//  * work is counted in tiles of `tile_tokens` keys; each extra piece of a
//    request costs `seg_overhead_tiles` more (query load, partial write and
//    its re-read by the combine);
//  * a binary search finds the smallest per-slot capacity C for which a greedy
//    pass over the requests, in order, cutting a request whenever the current
//    slot is full, needs no more slots than the device holds at once;
//  * the pieces of one request therefore sit in consecutive slots, and those
//    slots are mapped to workgroup ids on the same XCD (ids are dealt to the 8
//    XCDs round robin), so a request's query rows and partials stay in one L2;
//  * every slot runs once per row block (128 or 64 query rows); the row blocks
//    of one slot get workgroup ids on the same XCD too, so they stream the same
//    pages through that L2 at about the same time.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "plan_internal.h"

namespace mla {
namespace {

constexpr int kOk = 0, kInvalid = 1, kUnsupported = 2;
// Largest CU count a plan is made for (bounds the schedule's size; MI355X has 256).
constexpr int32_t kMaxCus = 65536;

struct Piece {
  int32_t b, t0, t1;  // tile range
};

// Greedy pass: returns the number of slots used with capacity C (in tiles),
// or a huge number if a single piece does not fit.  Fills `slots` if given.
int64_t greedy(const std::vector<int32_t>& tiles, double C, double c0, double min_frag,
               std::vector<std::vector<Piece>>* slots) {
  if (slots) slots->assign(1, {});
  int64_t used = 1;
  double cost = 0.0;
  bool empty = true;
  for (int32_t b = 0; b < (int32_t)tiles.size(); ++b) {
    int32_t lo = 0;
    const int32_t n = tiles[b];
    while (lo < n) {
      const double room = std::floor(C - cost - c0 + 1e-9);
      const int32_t rem = n - lo;
      const bool fits_whole = room >= rem;
      // Start a new slot if nothing fits, or if only a small fragment would.
      if (room < 1.0 || (!fits_whole && room < min_frag && !empty)) {
        if (empty) return INT64_MAX;  // C smaller than one tile plus overhead
        ++used;
        if (slots) slots->push_back({});
        cost = 0.0;
        empty = true;
        continue;
      }
      const int32_t take = fits_whole ? rem : (int32_t)room;
      if (slots) slots->back().push_back({b, lo, lo + take});
      cost += c0 + take;
      empty = false;
      lo += take;
      if (lo < n) {
        ++used;
        if (slots) slots->push_back({});
        cost = 0.0;
        empty = true;
      }
    }
  }
  if (empty && used > 1) {
    --used;
    if (slots) slots->pop_back();
  }
  return used;
}

}  // namespace

int build_plan(const int32_t* lens, int32_t batch, int32_t q_len, int32_t heads, int32_t page,
               int32_t num_cus, const PlanTuning& tuning, PlanData* out, std::string* err) {
  if (!lens || !out) {
    *err = "null pointer argument";
    return kInvalid;
  }
  if (batch <= 0) {
    *err = "batch must be >= 1";
    return kInvalid;
  }
  if (q_len < 1 || q_len > kMaxQLen) {
    *err = "q_len must be in [1, 8]";
    return q_len < 1 ? kInvalid : kUnsupported;
  }
  if (heads < 1 || heads > kMaxHeads || q_len * heads > kMaxRows) {
    *err = "num_heads must be in [1, 128] with q_len * num_heads <= 1024";
    return heads < 1 ? kInvalid : kUnsupported;
  }
  if (page < 16 || page > 4096 || (page & (page - 1)) != 0) {
    *err = "page_size must be a power of two in [16, 4096]";
    return kUnsupported;
  }
  if (num_cus <= 0 || num_cus > kMaxCus) {
    *err = "num_cus must be in [1, 65536]";
    return kInvalid;
  }
  for (int32_t b = 0; b < batch; ++b) {
    if (lens[b] < q_len) {
      *err = "seq_lens[" + std::to_string(b) + "] = " + std::to_string(lens[b]) + " is smaller than q_len";
      return kInvalid;
    }
    if (lens[b] > kMaxSeqLen) {
      *err = "seq_lens[" + std::to_string(b) + "] exceeds 2^24";
      return kUnsupported;
    }
  }

  PlanData& p = *out;
  p = PlanData{};
  p.batch = batch;
  p.q_len = q_len;
  p.heads = heads;
  p.page = page;
  p.num_cus = num_cus;
  p.rows = q_len * heads;
  // Two kernel shapes, both 4 waves (128 query rows) per workgroup and one
  // workgroup per compute unit (LDS rings of 144 KB): the bf16 kernel's
  // 32-key tiles (variant 1, the default) and the FP8 kernel's 64-key tiles
  // (variant 2).
  if (tuning.variant < 0 || tuning.variant > 2) {
    *err = "unknown kernel variant";
    return kInvalid;
  }
  p.v = tuning.variant == 2 ? Variant{4, 64, 1} : Variant{4, 32, 1};
  p.nrb = (p.rows + p.v.rows_per_block() - 1) / p.v.rows_per_block();
  p.lens.assign(lens, lens + batch);
  for (int32_t b = 0; b < batch; ++b) p.max_pages = std::max(p.max_pages, (lens[b] + page - 1) / page);

  const int32_t T = p.v.tile_tokens;
  std::vector<int32_t> tiles(batch);
  int64_t total_tiles = 0;
  for (int32_t b = 0; b < batch; ++b) {
    tiles[b] = (lens[b] + T - 1) / T;
    total_tiles += tiles[b];
  }
  // Slots: each slot is executed by nrb workgroups (one per row block).
  int64_t max_slots = (int64_t)num_cus * p.v.wg_per_cu / p.nrb;
  if (max_slots < 1) max_slots = 1;
  // the tunables count 32-key tiles
  const double c0 = tuning.seg_overhead_tiles * 32.0 / T;
  const double min_frag = tuning.min_fragment_tiles * 32.0 / T;

  // Smallest capacity (in whole tiles) whose greedy pass fits in max_slots.
  int64_t lo_c = std::max<int64_t>((int64_t)std::ceil(c0) + 1, (total_tiles + max_slots - 1) / max_slots);
  // with C = hi_c every request fits whole in one slot
  int64_t hi_c = ((int64_t)std::ceil(c0) + 1) * batch + total_tiles;
  while (lo_c < hi_c) {
    const int64_t mid = (lo_c + hi_c) / 2;
    if (greedy(tiles, (double)mid, c0, min_frag, nullptr) <= max_slots)
      hi_c = mid;
    else
      lo_c = mid + 1;
  }
  std::vector<std::vector<Piece>> slots;
  greedy(tiles, (double)lo_c, c0, min_frag, &slots);
  const int32_t S = (int32_t)slots.size();

  // Segments in slot order; partial ids for requests with more than one piece.
  std::vector<int32_t> pieces_of(batch, 0);
  for (auto& s : slots)
    for (auto& pc : s) pieces_of[pc.b]++;
  std::vector<int32_t> first_partial(batch, -1);
  std::vector<int32_t> next_partial(batch, 0);
  int32_t np = 0;
  for (auto& s : slots)
    for (auto& pc : s)
      if (pieces_of[pc.b] > 1 && first_partial[pc.b] < 0) {
        first_partial[pc.b] = np;
        np += pieces_of[pc.b];
      }
  p.num_partials = np;

  std::vector<int32_t> slot_of_partial(np, 0);
  std::vector<std::pair<int32_t, int32_t>> slot_range(S);  // [begin, end) in segs
  for (int32_t s = 0; s < S; ++s) {
    slot_range[s].first = (int32_t)p.segs.size();
    for (auto& pc : slots[s]) {
      Segment g;
      g.b = pc.b;
      g.kv_begin = pc.t0 * T;
      g.kv_end = std::min(pc.t1 * T, lens[pc.b]);
      g.partial = pieces_of[pc.b] > 1 ? first_partial[pc.b] + next_partial[pc.b]++ : -1;
      if (g.partial >= 0) slot_of_partial[g.partial] = s;
      p.segs.push_back(g);
    }
    slot_range[s].second = (int32_t)p.segs.size();
  }

  // Units (slot, row block), slot-major.  Deal consecutive units to the same
  // XCD in blocks of K; workgroup id = i * kNumXcd + xcd.
  const int64_t G = (int64_t)S * p.nrb;
  int64_t K = (G + kNumXcd - 1) / kNumXcd;
  K = (K + p.nrb - 1) / p.nrb * p.nrb;
  p.grid = (int32_t)(K * kNumXcd);
  if (G <= 1) p.grid = (int32_t)G;
  p.wgs.assign(p.grid, WorkgroupRange{0, 0, 0, 0});
  for (int64_t u = 0; u < G; ++u) {
    const int32_t s = (int32_t)(u / p.nrb), rb = (int32_t)(u % p.nrb);
    const int64_t w = (G <= 1) ? u : (u % K) * kNumXcd + u / K;
    p.wgs[w] = WorkgroupRange{slot_range[s].first, slot_range[s].second, rb, 0};
  }
  // Drop trailing empty workgroups (they would exit at once anyway).
  while (p.grid > 1 && p.wgs[p.grid - 1].seg_begin == p.wgs[p.grid - 1].seg_end) {
    p.wgs.pop_back();
    --p.grid;
  }

  for (int32_t b = 0; b < batch; ++b)
    if (pieces_of[b] > 1) {
      p.jobs.push_back(CombineJob{b, first_partial[b], pieces_of[b], 0});
      p.max_pieces = std::max(p.max_pieces, pieces_of[b]);
    }

  // Combine workgroups.  The partials of one (request, row block) were
  // written by the workgroups of its pieces, on the XCDs chosen above; the
  // combine workgroup that reads them goes to the XCD that wrote most of them,
  // so that its reads can hit that XCD's L2.  Each XCD takes at most an even
  // share; the rest go to the XCDs with the fewest.
  if (!p.jobs.empty()) {
    const int32_t per_unit = p.max_pieces <= kCombineSmallMax ? kCombineSmallRows : 1;
    const int32_t rpb = p.v.rows_per_block();
    const size_t units = p.jobs.size() * (size_t)((p.rows + per_unit - 1) / per_unit);
    const size_t cap = (units + kNumXcd - 1) / kNumXcd;
    std::vector<std::vector<CombineUnit>> lists(kNumXcd);
    std::vector<CombineUnit> spill;
    for (const CombineJob& j : p.jobs)
      for (int32_t r0 = 0; r0 < p.rows; r0 += per_unit) {
        const int64_t rb = r0 / rpb;
        int32_t votes[kNumXcd] = {};
        for (int32_t k = 0; k < j.n; ++k) votes[((slot_of_partial[j.p0 + k] * p.nrb + rb) / K) % kNumXcd]++;
        const int32_t x = (int32_t)(std::max_element(votes, votes + kNumXcd) - votes);
        const CombineUnit cu{j.b, j.p0, j.n, r0};
        if (lists[x].size() < cap)
          lists[x].push_back(cu);
        else
          spill.push_back(cu);
      }
    for (const CombineUnit& cu : spill) {
      auto it = std::min_element(lists.begin(), lists.end(),
                                 [](const std::vector<CombineUnit>& a, const std::vector<CombineUnit>& b) {
                                   return a.size() < b.size();
                                 });
      it->push_back(cu);
    }
    p.cunits.assign(cap * kNumXcd, CombineUnit{0, 0, 0, 0});
    for (int32_t x = 0; x < kNumXcd; ++x)
      for (size_t i = 0; i < lists[x].size(); ++i) p.cunits[i * kNumXcd + x] = lists[x][i];
    while (!p.cunits.empty() && p.cunits.back().n == 0) p.cunits.pop_back();
  }
  return kOk;
}

WorkspaceLayout workspace_layout(const PlanData& p) {
  // fp16 partial outputs [slots][rows_per_block][512], then lse and scale
  // factors [slots][rows_per_block] in fp32, each part 256-byte aligned.
  const size_t slots = (size_t)p.num_partials * p.nrb;
  const size_t rpb = (size_t)p.v.rows_per_block();
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  WorkspaceLayout w;
  if (slots == 0) return w;
  w.off_o = 0;
  w.off_lse = al(slots * rpb * 512 * 2);
  w.off_f = w.off_lse + al(slots * rpb * 4);
  w.total = w.off_f + al(slots * rpb * 4);
  return w;
}

size_t workspace_bytes(const PlanData& p) { return workspace_layout(p).total; }

}  // namespace mla
