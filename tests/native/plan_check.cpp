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
//   * a launch never has more active groups than kMaxGrid (kMaxGridShort
//     for short fp32 sampling rows), so every slot fits the workspace sized
//     by partial_bytes(max_rows, ..., that cap).
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

// Merged partials of multi-part rows: a logical row is P consecutive stream
// rows (a target row read with its Gumbel row) or one; each group writes one
// partial per logical row it touches, at slot (first stream row) + group.
// The slots are unique and below R + G, and the span the decision step
// computes for a P-part row (groups of its first through last element)
// lists exactly the groups that wrote it.
static void check_merged(const std::vector<int>& parts, int64_t V, int64_t eb, int64_t grid) {
  std::vector<int64_t> start;   // first stream row of each logical row
  int64_t R = 0;
  for (int p : parts) {
    start.push_back(R);
    R += p;
  }
  const FlatSplit f = make_split(R, V, eb, grid);
  std::vector<int64_t> owner(static_cast<size_t>(R), -1);   // logical row of each stream row
  for (size_t l = 0; l < parts.size(); ++l)
    for (int k = 0; k < parts[l]; ++k) owner[start[l] + k] = static_cast<int64_t>(l);
  std::vector<int> used(static_cast<size_t>(R + f.G), 0);
  std::vector<std::vector<int64_t>> writers(parts.size());
  for (int64_t g = 0; g < f.G; ++g) {
    int64_t e0, e1;
    split_range(f, g, e0, e1);
    int64_t last = -1;
    for (int64_t r = e0 / V; r * V < e1; ++r) {
      const int64_t l = owner[r];
      if (l == last) continue;   // accumulated into the same partial
      last = l;
      const int64_t s = start[l] + g;
      CHECK(s < R + f.G && used[s] == 0, "merged slot %lld (V=%lld)", (long long)s, (long long)V);
      if (s < R + f.G) used[s] = 1;
      writers[l].push_back(g);
    }
  }
  for (size_t l = 0; l < parts.size(); ++l) {
    const int64_t v = start[l], P = parts[l];
    const int64_t glo = split_group(f, v * V), ghi = split_group(f, (v + P) * V - 1);
    const auto& w = writers[l];
    CHECK(static_cast<int64_t>(w.size()) == ghi - glo + 1, "row %zu writers %zu vs %lld", l, w.size(),
          (long long)(ghi - glo + 1));
    for (size_t k = 0; k < w.size(); ++k) CHECK(w[k] == glo + static_cast<int64_t>(k), "row %zu writer", l);
  }
}

// FastDiv32 against plain division: every divisor up to 4096 and around
// powers of two, over small values, values near multiples and the top of
// the range.
static void check_fastdiv() {
  std::vector<uint32_t> ds;
  for (uint32_t d = 1; d <= 4096; ++d) ds.push_back(d);
  for (int k = 12; k < 32; ++k)
    for (int64_t o = -3; o <= 3; ++o) ds.push_back(static_cast<uint32_t>((int64_t(1) << k) + o));
  ds.push_back(2147483647u);
  ds.push_back(2147483648u);
  for (uint32_t d : ds) {
    const dbv::FastDiv32 f(d);
    auto chk = [&](uint64_t n) {
      if (n > 0xffffffffull) return;
      const uint32_t v = static_cast<uint32_t>(n);
      if (f.div(v) != v / d) {
        std::printf("FastDiv32 %u / %u: %u != %u\n", v, d, f.div(v), v / d);
        std::exit(1);
      }
    };
    for (uint64_t n = 0; n < 3000; ++n) chk(n);
    for (uint64_t q : {1ull, 2ull, 3ull, 1000ull, 65535ull, 1000003ull})
      for (int64_t o = -2; o <= 2; ++o) chk(q * d + o);
    for (uint64_t n = 0xffffffffull - 3000; n <= 0xffffffffull; ++n) chk(n);
    uint64_t x = 88172645463325252ull ^ d;
    for (int i = 0; i < 2000; ++i) {
      x ^= x << 13; x ^= x >> 7; x ^= x << 17;
      chk(x & 0xffffffffull);
    }
  }
}

int main() {
  check_fastdiv();
  // Sequences of P-part target rows followed by one-part drafter rows.
  for (int P : {2, 3})
    for (int64_t V : {1, 7, 1000, 2048, 32000, 151936})
      for (int64_t grid : {1, 5, 256, 1024}) {
        std::vector<int> parts;
        for (int n : {0, 3, 1, 8, 0, 5}) {
          for (int i = 0; i <= n; ++i) parts.push_back(P);
          for (int i = 0; i < n; ++i) parts.push_back(1);
        }
        check_merged(parts, V, P == 3 ? 2 : 4, grid);
      }

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

  // Parts of a target row read with its Gumbel row: contiguous, in order,
  // covering [0, V), 16-byte aligned starts, each within 16 + (V mod 8P) of
  // V / P elements.
  for (int64_t V : {1, 7, 8, 23, 24, 25, 48, 1000, 1024, 2049, 32000, 151936, 152064}) {
    for (int P : {2, 3}) {
      int64_t prev = 0;
      for (int k = 0; k < P; ++k) {
        const int64_t lo = part_offset(V, P, k, 0), hi = part_offset(V, P, k, V);
        CHECK(lo == prev && hi >= lo && lo % 8 == 0, "part V=%lld P=%d k=%d [%lld, %lld)", (long long)V, P, k,
              (long long)lo, (long long)hi);
        const int64_t want = V / P;
        CHECK(hi - lo <= want + 16 + V % (8 * P) && hi - lo + 16 + V % (8 * P) >= want, "part balance V=%lld",
              (long long)V);
        int64_t last = lo;
        for (int64_t v = 0; v <= V; v += (V > 4096 ? 2048 : 1)) {   // monotone inside the part
          const int64_t o = part_offset(V, P, k, v);
          CHECK(o >= last && o >= lo && o <= hi, "part monotone V=%lld P=%d v=%lld", (long long)V, P, (long long)v);
          last = o;
        }
        prev = hi;
      }
      CHECK(prev == V, "parts cover V=%lld P=%d", (long long)V, P);
    }
  }

  // Launch grids stay within kMaxGrid for any device.
  CHECK(stream_grid(1000000, 151936, 2, 1 << 20) == kMaxGrid, "stream_grid cap");
  CHECK(stream_grid(9, 1024, 4, 2048) == 3, "stream_grid small: four units a group up to 1 MiB");
  CHECK(stream_grid(300, 1024, 4, 2048) == 300, "stream_grid: one unit a group past 1 MiB");
  CHECK(stream_grid(1000000, 1024, 4, 1 << 20, sample_max_grid(1024, 4, false)) == kMaxGridShort,
        "short-row grid cap");
  CHECK(sample_max_grid(1024, 2, false) == kMaxGrid && sample_max_grid(1024, 4, true) == kMaxGrid &&
            sample_max_grid(8192, 4, false) == kMaxGrid && kMaxGridShort >= kMaxGrid,
        "short-row grid only for fp32 rows of at most kSmallRowBytes without Gumbel rows");

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
          CHECK(s.off_pre % 256 == 0 && s.off_rec % 256 == 0 && s.off_tmass % 256 == 0 && s.off_gpart % 256 == 0,
                "sample offsets");
          // Gumbel-row streams: P parts per target row, at most 3.
          const int64_t P = gumbel_parts(eb);
          CHECK(P >= 2 && P <= 3 && s.max_vrows >= static_cast<int64_t>(B) * (P * (K + 1) + K), "vrows");
          CHECK(s.off_gpart >= static_cast<size_t>(s.max_vrows + kMaxGridShort) * kWavesPlan * 16,
                "gpart overlaps stats");
          CHECK(s.off_pre >= s.off_gpart + static_cast<size_t>(s.max_vrows + kMaxGridShort) * kWavesPlan * 8,
                "pre overlaps gpart");
          CHECK(s.off_rec >= s.off_pre + static_cast<size_t>(B + 1) * 4, "rec overlaps pre");
          CHECK(s.off_tmass >= s.off_rec + static_cast<size_t>(B) * sizeof(DrawRecord), "tmass overlaps rec");
          CHECK(s.off_sq >= s.off_tmass + static_cast<size_t>(B) * s.tiles * 4, "sq overlaps tmass");
          CHECK(s.off_blk % 256 == 0 && s.off_blk >= s.off_sq + static_cast<size_t>(B) * sizeof(SparseRow),
                "blk overlaps sq");
          CHECK(s.bytes >= s.off_blk + static_cast<size_t>(kSeqBlocks) * 4, "sample bytes");
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
          CHECK(t.off_map >= t.off_list + (rows + kTreePlanThreads) * 4, "map overlaps list padding");
          CHECK(t.off_conf >= t.off_map + (rows + kTreePlanPass) * 4, "conf overlaps map padding");
          CHECK(t.off_pick >= t.off_conf + (rows + kMaxGrid) * kWavesPlan * 8, "pick overlaps conf");
          CHECK(t.off_sel >= t.off_pick + static_cast<size_t>(t.states) * t.split2 * 8, "sel overlaps pick");
          CHECK(t.off_selconf >= t.off_sel + static_cast<size_t>(t.states) * 4, "selconf overlaps sel");
          CHECK(t.off_selstat >= t.off_selconf + static_cast<size_t>(t.states) * 4, "selstat overlaps selconf");
          CHECK(t.off_selgap >= t.off_selstat + static_cast<size_t>(t.states) * 4, "selgap overlaps selstat");
          CHECK(t.off_batch % 256 == 0 && t.off_nbat % 256 == 0, "batch offsets");
          CHECK(t.off_batch >= t.off_selgap + static_cast<size_t>(t.states) * 4, "batch overlaps selgap");
          CHECK(t.off_nbat >= t.off_batch + static_cast<size_t>(t.states) * 32, "nbat overlaps batch");
          CHECK(t.bytes >= t.off_nbat + static_cast<size_t>(B) * 4, "tree bytes");
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
