// Host-only invariants of the launch plans (compiled with g++ by
// tests/test_plan_cpu.py; no GPU involved).
//
// Flat split, for every (R, V, element size, grid) on a grid of sizes:
//   * the active groups' ranges are non-empty, contiguous and cover the
//     stream [0, R*V) exactly once;
//   * split_group(e) names the group whose range holds e;
//   * the partial slot r + g of every (row, group) piece is unique and below
//     R + G, and split_row_slots(r) lists exactly the pieces of row r, in
//     order, as consecutive slots;
//   * a launch never has more active groups than kMaxGrid, so every slot fits
//     the workspace sized by partial_bytes(max_rows).
// Plans: the draw tiles of the largest vocabulary fit the LDS tile array and
// 32-bit offsets; workspace sections are 256-byte aligned and do not overlap.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "dbv_plan.h"

using namespace dbv;

static int failures = 0;

#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) {                                \
      if (failures < 20) {                        \
        std::printf("FAIL %s: ", #cond);          \
        std::printf(__VA_ARGS__);                 \
        std::printf("\n");                        \
      }                                           \
      ++failures;                                 \
    }                                             \
  } while (0)

static void check_split(int64_t R, int64_t V, int64_t eb, int64_t grid) {
  const FlatSplit f = make_split(R, V, eb, grid);
  const int64_t E = R * V;
  CHECK(f.G >= 1 && f.G <= grid && f.G <= f.NQ, "R=%lld V=%lld grid=%lld G=%lld", (long long)R,
        (long long)V, (long long)grid, (long long)f.G);
  // Pieces in stream order, as the kernels visit them.
  std::vector<int64_t> slot_row(static_cast<size_t>(R + f.G), -1);
  std::vector<std::vector<int64_t>> row_groups(static_cast<size_t>(R));
  int64_t expect = 0;
  for (int64_t g = 0; g < f.G; ++g) {
    int64_t e0, e1;
    split_range(f, g, e0, e1);
    CHECK(e0 == expect && e1 > e0 && e1 <= E, "R=%lld V=%lld g=%lld [%lld,%lld) expect %lld", (long long)R,
          (long long)V, (long long)g, (long long)e0, (long long)e1, (long long)expect);
    if (e1 <= e0) return;
    expect = e1;
    CHECK(split_group(f, e0) == g && split_group(f, e1 - 1) == g, "split_group g=%lld", (long long)g);
    for (int64_t r = e0 / V; r * V < e1; ++r) {
      const int64_t s = r + g;
      CHECK(s >= 0 && s < R + f.G, "slot %lld", (long long)s);
      if (s < 0 || s >= R + f.G) return;
      CHECK(slot_row[s] == -1, "slot %lld reused (rows %lld, %lld)", (long long)s, (long long)slot_row[s],
            (long long)r);
      slot_row[s] = r;
      row_groups[r].push_back(g);
    }
  }
  CHECK(expect == E, "coverage R=%lld V=%lld ends at %lld", (long long)R, (long long)V, (long long)expect);
  for (int64_t r = 0; r < R; ++r) {
    int64_t first, n;
    split_row_slots(f, r, first, n);
    const auto& gs = row_groups[r];
    CHECK(n == static_cast<int64_t>(gs.size()) && n >= 1, "row %lld groups %lld vs %zu", (long long)r,
          (long long)n, gs.size());
    for (int64_t k = 0; k < n && k < static_cast<int64_t>(gs.size()); ++k)
      CHECK(gs[k] == first - r + k, "row %lld piece %lld group %lld", (long long)r, (long long)k,
            (long long)gs[k]);
  }
}

int main() {
  // Flat split over small and benchmark-like shapes.
  const int64_t Rs[] = {1, 2, 3, 5, 9, 17, 64, 136, 1000, 1056, 3124};
  const int64_t Vs[] = {1, 2, 7, 255, 1000, 1024, 2047, 2048, 2049, 32000, 128256, 151936};
  const int64_t grids[] = {1, 7, 256, 2048};
  for (int64_t R : Rs)
    for (int64_t V : Vs)
      for (int64_t eb : {2, 4})
        for (int64_t grid : grids) check_split(R, V, eb, grid);
  // A tree-sized stream.
  check_split(21000, 151936, 2, 2048);

  // Launch grids stay within kMaxGrid for any device.
  CHECK(stream_grid(1000000, 151936, 2, 1 << 20) == kMaxGrid, "stream_grid cap");
  CHECK(stream_grid(9, 1024, 4, 2048) == 9, "stream_grid small");

  const int64_t PVs[] = {1, 2, 7, 255, 256, 257, 1000, 1024, 2047, 2048, 2049, 8191, 8192, 8193,
                         32000, 32768, 50257, 65536, 128256, 131072, 151936, 152064, 262144,
                         1 << 20, kMaxSampleV};
  const int Bs[] = {1, 2, 3, 8, 16, 32, 64, 128, 1000};
  const int Ks[] = {0, 1, 4, 8, 16, 31, 64};
  for (int64_t V : PVs) {
    // The draw's tiles fit the LDS array of tile masses for either element
    // size, and byte offsets within a row fit 32 bits.
    for (int64_t eb : {2, 4}) {
      if (V <= kMaxSampleV)
        CHECK(cdiv(V, draw_tile(eb)) <= kMaxDrawTiles, "V=%lld eb=%lld tiles", (long long)V, (long long)eb);
    }
    CHECK(kMaxSampleV * 4 < (int64_t(1) << 32), "draw offsets");
    for (int B : Bs) {
      for (int K : Ks) {
        for (int64_t eb : {2, 4}) {
          const SamplePlan s = plan_sample(B, K, static_cast<int>(V), eb);
          CHECK(s.max_rows == static_cast<int64_t>(B) * (2 * K + 1), "sample rows");
          CHECK(s.tiles == cdiv(V, draw_tile(eb)) && s.tpc >= 1 && s.chunks * s.tpc >= s.tiles &&
                    (s.chunks - 1) * s.tpc < s.tiles,
                "V=%lld B=%d tiles %lld tpc %lld chunks %lld", (long long)V, B, (long long)s.tiles,
                (long long)s.tpc, (long long)s.chunks);
          CHECK(s.off_pre % 256 == 0 && s.off_rec % 256 == 0 && s.off_tmass % 256 == 0, "sample offsets");
          CHECK(s.off_pre >= static_cast<size_t>(s.max_rows + kMaxGrid) * kWavesPlan * 8, "pre overlaps stats");
          CHECK(s.off_rec >= s.off_pre + static_cast<size_t>(B + 1) * 4, "rec overlaps pre");
          CHECK(s.off_tmass >= s.off_rec + static_cast<size_t>(B) * sizeof(DrawRecord), "tmass overlaps rec");
          CHECK(s.bytes >= s.off_tmass + static_cast<size_t>(B) * s.tiles * 4, "sample bytes");
        }

        const GreedyPlan g = plan_greedy(B, K, K + 1, static_cast<int>(V));
        CHECK(g.max_rows == static_cast<int64_t>(B) * (2 * K + 2), "greedy rows");
        CHECK(g.off_pre % 256 == 0, "greedy offsets");
        CHECK(g.off_pre >= static_cast<size_t>(g.max_rows + kMaxGrid) * kWavesPlan * 8, "greedy pre overlaps");
        CHECK(g.bytes >= g.off_pre + static_cast<size_t>(B + 1) * 4, "greedy bytes");
      }
      const int Ss[] = {1, 2, 9, 64, 200};
      const int Ls[] = {1, 8, 32, 100};
      for (int S : Ss) {
        for (int L : Ls) {
          const TreePlan t = plan_tree(B, S, L, static_cast<int>(V));
          const size_t rows = static_cast<size_t>(B) * S * L;
          CHECK(t.max_rows == static_cast<int64_t>(rows), "tree rows");
          CHECK(t.split2 >= 1 && t.split2 <= kMaxSplit, "tree split2=%d", t.split2);
          CHECK(static_cast<int64_t>(t.split2) * t.chunk2 >= V, "tree V=%lld B=%d S=%d split2=%d chunk2=%lld",
                (long long)V, B, S, t.split2, (long long)t.chunk2);
          CHECK(static_cast<int64_t>(t.split2 - 1) * t.chunk2 < V, "tree empty split V=%lld split2=%d chunk2=%lld",
                (long long)V, t.split2, (long long)t.chunk2);
          CHECK(t.off_list % 256 == 0 && t.off_map % 256 == 0 && t.off_conf % 256 == 0 &&
                    t.off_pick % 256 == 0 && t.off_sel % 256 == 0, "tree offsets");
          CHECK(t.off_list >= t.off_count + 4, "list overlaps count");
          CHECK(t.off_map >= t.off_list + rows * 4, "map overlaps list");
          CHECK(t.off_conf >= t.off_map + rows * 4, "conf overlaps map");
          CHECK(t.off_pick >= t.off_conf + (rows + kMaxGrid) * kWavesPlan * 8, "pick overlaps conf");
          CHECK(t.off_sel >= t.off_pick + static_cast<size_t>(t.states) * t.split2 * 8, "sel overlaps pick");
          CHECK(t.bytes >= t.off_sel + static_cast<size_t>(t.states) * 4, "tree bytes");
        }
      }
    }
  }
  if (failures) {
    std::printf("%d failures\n", failures);
    return 1;
  }
  std::printf("plan invariants ok\n");
  return 0;
}
