// Randomized check of the host split planner (built with the host compiler and
// its address and undefined-behaviour checks by tests/test_plan_fuzz.py).
//
// For random batches, lengths, query shapes, page sizes and CU counts it
// checks what every schedule must satisfy: each key of each request covered
// exactly once by tile-aligned pieces, every piece run once per row block,
// partial ids distinct and dense, combine units covering every row of every
// split request once, and the schedule no larger than the room a plan
// reserves for in-place updates (at most batch + S pieces, S * nrb + 8 (nrb + 1)
// workgroups and batch * rows + 8 combine units, S = max(1, num_cus / nrb)
// slots).  Invalid arguments must be refused, never crash.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "plan_internal.h"

namespace {

int fails = 0;
#define CHECK(c, ...)                             \
  do {                                            \
    if (!(c)) {                                   \
      std::fprintf(stderr, "FAIL %s: ", #c);      \
      std::fprintf(stderr, __VA_ARGS__);          \
      std::fprintf(stderr, "\n");                 \
      ++fails;                                    \
      return;                                     \
    }                                             \
  } while (0)

void check_case(const std::vector<int32_t>& lens, int32_t q_len, int32_t heads, int32_t page, int32_t num_cus,
                int32_t variant) {
  mla::PlanTuning tune;
  tune.variant = variant;
  mla::PlanData p;
  std::string err;
  const int rc = mla::build_plan(lens.data(), (int32_t)lens.size(), q_len, heads, page, num_cus, tune, &p, &err);
  CHECK(rc == 0, "rc %d (%s) batch %zu q %d h %d page %d cus %d", rc, err.c_str(), lens.size(), q_len, heads, page,
        num_cus);
  const int32_t B = (int32_t)lens.size(), T = p.v.tile_tokens, rows = q_len * heads;
  CHECK(p.nrb == (rows + p.v.rows_per_block() - 1) / p.v.rows_per_block(), "nrb");
  // coverage, tile alignment, piece order
  std::vector<std::vector<int32_t>> cover(B);
  for (int32_t b = 0; b < B; ++b) cover[b].assign(lens[b], 0);
  std::vector<int32_t> pieces(B, 0);
  for (const auto& s : p.segs) {
    CHECK(s.b >= 0 && s.b < B, "segment request %d", s.b);
    CHECK(0 <= s.kv_begin && s.kv_begin < s.kv_end && s.kv_end <= lens[s.b] && s.kv_begin % T == 0,
          "segment range [%d, %d) of %d", s.kv_begin, s.kv_end, lens[s.b]);
    for (int32_t k = s.kv_begin; k < s.kv_end; ++k) cover[s.b][k]++;
    pieces[s.b]++;
  }
  for (int32_t b = 0; b < B; ++b)
    for (int32_t k = 0; k < lens[b]; ++k) CHECK(cover[b][k] == 1, "request %d key %d covered %d times", b, k, cover[b][k]);
  // partial ids: -1 for whole requests; 0 .. num_partials-1 once each otherwise
  std::vector<int32_t> seen(p.num_partials, 0);
  for (const auto& s : p.segs) {
    CHECK((s.partial < 0) == (pieces[s.b] == 1), "partial id of request %d", s.b);
    if (s.partial >= 0) {
      CHECK(s.partial < p.num_partials, "partial id %d of %d", s.partial, p.num_partials);
      seen[s.partial]++;
    }
  }
  for (int32_t i = 0; i < p.num_partials; ++i) CHECK(seen[i] == 1, "partial %d used %d times", i, seen[i]);
  // every segment once per row block
  std::vector<std::vector<int32_t>> runs(p.segs.size());
  CHECK((int32_t)p.wgs.size() == p.grid, "grid %d vs %zu", p.grid, p.wgs.size());
  for (const auto& w : p.wgs) {
    CHECK(0 <= w.seg_begin && w.seg_begin <= w.seg_end && w.seg_end <= (int32_t)p.segs.size(), "workgroup range");
    CHECK(w.seg_begin == w.seg_end || (0 <= w.row_block && w.row_block < p.nrb), "row block %d", w.row_block);
    for (int32_t s = w.seg_begin; s < w.seg_end; ++s) runs[s].push_back(w.row_block);
  }
  for (size_t s = 0; s < runs.size(); ++s) {
    CHECK((int32_t)runs[s].size() == p.nrb, "segment %zu run %zu times", s, runs[s].size());
    std::vector<int32_t> rb(p.nrb, 0);
    for (int32_t r : runs[s]) rb[r]++;
    for (int32_t r = 0; r < p.nrb; ++r) CHECK(rb[r] == 1, "segment %zu row block %d", s, r);
  }
  // combine units: every row of every split request exactly once
  const int32_t per = p.max_pieces <= mla::kCombineSmallMax ? mla::kCombineSmallRows : 1;
  std::vector<std::vector<int32_t>> rowseen(B);
  for (int32_t b = 0; b < B; ++b) rowseen[b].assign(rows, 0);
  for (const auto& u : p.cunits) {
    if (u.n == 0) continue;
    CHECK(u.b >= 0 && u.b < B && u.n == pieces[u.b] && u.n > 1, "combine unit of request %d", u.b);
    CHECK(u.p0 >= 0 && u.p0 + u.n <= p.num_partials, "combine unit partials");
    for (int32_t r = u.row0; r < std::min(u.row0 + per, rows); ++r) rowseen[u.b][r]++;
  }
  for (int32_t b = 0; b < B; ++b)
    for (int32_t r = 0; r < rows; ++r)
      CHECK(rowseen[b][r] == (pieces[b] > 1 ? 1 : 0), "request %d row %d combined %d times", b, r, rowseen[b][r]);
  // the room reserved for in-place updates
  const int64_t slots = std::max<int64_t>(1, (int64_t)num_cus * p.v.wg_per_cu / p.nrb);
  CHECK((int64_t)p.segs.size() <= B + slots, "segments %zu > %lld", p.segs.size(), (long long)(B + slots));
  CHECK((int64_t)p.wgs.size() <= slots * p.nrb + mla::kNumXcd * (p.nrb + 1), "workgroups %zu", p.wgs.size());
  CHECK((int64_t)p.cunits.size() <= (int64_t)B * rows + mla::kNumXcd, "combine units %zu", p.cunits.size());
  // workspace offsets are ordered and 256-byte aligned
  const mla::WorkspaceLayout w = mla::workspace_layout(p);
  CHECK(w.off_o % 256 == 0 && w.off_lse % 256 == 0 && w.off_f % 256 == 0 && w.total % 256 == 0, "alignment");
  CHECK(p.num_partials == 0 ? w.total == 0 : (w.off_o < w.off_lse && w.off_lse < w.off_f && w.off_f < w.total),
        "layout order");
}

void check_refused(const std::vector<int32_t>& lens, int32_t q_len, int32_t heads, int32_t page, int32_t num_cus,
                   int32_t variant) {
  mla::PlanTuning tune;
  tune.variant = variant;
  mla::PlanData p;
  std::string err;
  const int rc = mla::build_plan(lens.data(), (int32_t)lens.size(), q_len, heads, page, num_cus, tune, &p, &err);
  CHECK(rc != 0 && !err.empty(), "accepted: batch %zu q %d h %d page %d cus %d", lens.size(), q_len, heads, page,
        num_cus);
}

}  // namespace

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 300;
  std::mt19937_64 rng(argc > 2 ? std::strtoull(argv[2], nullptr, 10) : 12345);
  auto uni = [&](int64_t lo, int64_t hi) { return (int64_t)(lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1))); };
  const int32_t pages[] = {16, 32, 64, 128, 256, 512, 1024, 4096};
  const int32_t cu_choices[] = {1, 2, 3, 7, 8, 64, 255, 256, 304, 1024};
  for (int c = 0; c < cases; ++c) {
    const int32_t q_len = (int32_t)uni(1, 8);
    const int32_t heads = (int32_t)uni(1, 1024 / q_len < 128 ? 1024 / q_len : 128);
    const int32_t page = pages[uni(0, 7)];
    const int32_t num_cus = cu_choices[uni(0, 9)];
    const int32_t batch = (int32_t)(c % 5 == 0 ? uni(1, 3) : uni(1, 96));
    std::vector<int32_t> lens(batch);
    const int kind = (int)uni(0, 3);
    for (auto& L : lens) {
      int64_t v = kind == 0 ? uni(q_len, 64) : kind == 1 ? uni(q_len, 5000) : kind == 2 ? (uni(0, 4) ? uni(q_len, 600) : uni(10000, 40000)) : uni(q_len, 20000);
      L = (int32_t)v;
    }
    check_case(lens, q_len, heads, page, num_cus, (int32_t)uni(1, 2));
  }
  // one request at the maximum length, on one CU and on many
  check_case({1 << 24}, 1, 128, 4096, 256, 1);
  check_case({1 << 24, 2}, 2, 64, 64, 1, 2);
  // refused arguments
  check_refused({0}, 1, 128, 64, 256, 1);
  check_refused({(1 << 24) + 1}, 1, 128, 64, 256, 1);
  check_refused({100}, 9, 64, 64, 256, 1);
  check_refused({100}, 8, 129, 64, 256, 1);
  check_refused({100}, 1, 128, 48, 256, 1);
  check_refused({100}, 1, 128, 8192, 256, 1);
  check_refused({100}, 1, 128, 64, 0, 1);
  check_refused({100}, 1, 128, 64, 65537, 1);
  check_refused({100}, 1, 128, 64, 256, 3);
  std::printf("%s: %d random cases, %d failures\n", fails ? "FAIL" : "ok", cases, fails);
  return fails ? 1 : 0;
}
