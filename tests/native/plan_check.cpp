// Host-only invariants of the launch plans (compiled with g++ by
// tests/test_plan_cpu.py; no GPU involved).  For every size on a grid:
//   * the vocabulary chunks of every plan cover the whole row and no chunk
//     starts past it (except the sampling draw, whose empty trailing chunks
//     contribute zero mass),
//   * the draw chunk fits the select kernel's register scan,
//   * workspace sections are 256-byte aligned and do not overlap.
#include <cstdio>
#include <cstdlib>

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

static void check_rows(const RowPlan& r, int64_t rows, int64_t V, const char* what) {
  CHECK(r.chunk > 0 && r.chunk % 256 == 0, "%s rows=%lld V=%lld chunk=%lld", what, (long long)rows,
        (long long)V, (long long)r.chunk);
  CHECK(r.nchunk * r.chunk >= V, "%s V=%lld chunk=%lld nchunk=%lld", what, (long long)V,
        (long long)r.chunk, (long long)r.nchunk);
  CHECK((r.nchunk - 1) * r.chunk < V, "%s V=%lld chunk=%lld nchunk=%lld", what, (long long)V,
        (long long)r.chunk, (long long)r.nchunk);
  CHECK(r.items == rows * r.nchunk, "%s items", what);
  CHECK(r.part_bytes >= static_cast<size_t>(r.items) * kWavesPlan * 8, "%s part bytes", what);
}

int main() {
  const int64_t Vs[] = {1, 2, 7, 255, 256, 257, 1000, 1024, 2047, 2048, 2049, 8191, 8192, 8193,
                        32000, 32768, 50257, 65536, 128256, 131072, 151936, 152064, 262144,
                        1 << 20, kMaxSampleV};
  const int Bs[] = {1, 2, 3, 8, 16, 32, 64, 128, 1000};
  const int Ks[] = {0, 1, 4, 8, 16, 31, 64};
  for (int64_t V : Vs) {
    for (int B : Bs) {
      for (int K : Ks) {
        const SamplePlan s = plan_sample(B, K, static_cast<int>(V));
        check_rows(s.r, static_cast<int64_t>(B) * (2 * K + 1), V, "sample");
        CHECK(s.draw_chunks >= 1 && s.draw_chunks <= kMaxDrawChunks, "V=%lld B=%d draw_chunks=%d",
              (long long)V, B, s.draw_chunks);
        CHECK(s.draw_chunk <= kDrawChunkMax && s.draw_chunk % 256 == 0, "V=%lld draw_chunk=%lld",
              (long long)V, (long long)s.draw_chunk);
        CHECK(s.draw_chunks * s.draw_chunk >= V, "V=%lld B=%d draw %d x %lld", (long long)V, B,
              s.draw_chunks, (long long)s.draw_chunk);
        CHECK(s.off_rec % 256 == 0 && s.off_dsum % 256 == 0, "sample offsets");
        CHECK(s.off_rec >= s.r.part_bytes, "rec overlaps stats");
        CHECK(s.off_dsum >= s.off_rec + static_cast<size_t>(B) * sizeof(DrawRecord), "dsum overlaps rec");
        CHECK(s.bytes >= s.off_dsum + static_cast<size_t>(B) * s.draw_chunks * 4, "sample bytes");

        const GreedyPlan g = plan_greedy(B, K, K + 1, static_cast<int>(V));
        check_rows(g.r, static_cast<int64_t>(B) * (2 * K + 2), V, "greedy");
      }
      const int Ss[] = {1, 2, 9, 64, 200};
      const int Ls[] = {1, 8, 32, 100};
      for (int S : Ss) {
        for (int L : Ls) {
          const TreePlan t = plan_tree(B, S, L, static_cast<int>(V));
          check_rows(t.r, static_cast<int64_t>(B) * S * L, V, "tree");
          CHECK(t.split2 >= 1 && t.split2 <= kMaxSplit, "tree split2=%d", t.split2);
          CHECK(static_cast<int64_t>(t.split2) * t.chunk2 >= V, "tree V=%lld B=%d S=%d split2=%d chunk2=%lld",
                (long long)V, B, S, t.split2, (long long)t.chunk2);
          CHECK(static_cast<int64_t>(t.split2 - 1) * t.chunk2 < V, "tree empty split V=%lld split2=%d chunk2=%lld",
                (long long)V, t.split2, (long long)t.chunk2);
          CHECK(t.off_pick % 256 == 0 && t.off_sel % 256 == 0, "tree offsets");
          CHECK(t.off_pick >= t.r.part_bytes, "pick overlaps conf");
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
