// Launch plan and workspace layout: a pure function of the call's sizes, so
// verify_workspace_size() and the launchers always agree.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace dbv {

constexpr float kLog2eHost = 1.4426950408889634f;

// Enough workgroups to keep every CU of an MI355X (256 CUs) busy with a few
// resident groups each; a row is split over its vocabulary (split-V) only when
// there are too few rows, and never into pieces below kMinChunk elements.
constexpr int64_t kTargetGroups = 2048;
constexpr int64_t kMinChunk = 4096;
constexpr int kMaxSplit = 64;
constexpr int kMaxDraft = 1024;       // K and W limit of the chain modes
constexpr int kMaxStates = 1024;      // S limit of the tree mode
constexpr int kMaxBlockLen = 1024;    // L limit of the tree mode

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Number of vocabulary chunks per row for `rows` rows of length V.
inline int choose_split(int64_t rows, int64_t V) {
  if (rows <= 0) return 1;
  int64_t s = cdiv(kTargetGroups, rows);
  const int64_t cap = V / kMinChunk > 0 ? V / kMinChunk : 1;
  if (s > cap) s = cap;
  if (s > kMaxSplit) s = kMaxSplit;
  return s < 1 ? 1 : static_cast<int>(s);
}

// Chunk length (elements) for `split` chunks of a length-V row, rounded up to
// a multiple of 256 elements so chunk starts keep the row's alignment.
inline int64_t chunk_len(int64_t V, int split) {
  int64_t c = cdiv(V, split);
  return cdiv(c, 256) * 256;
}

// Number of chunks of the correction / bonus draw (one row per sequence).
inline int choose_draw_chunks(int64_t B, int64_t V) {
  int64_t s = cdiv(1024, B > 0 ? B : 1);
  const int64_t cap = V / 2048 > 0 ? V / 2048 : 1;
  if (s > cap) s = cap;
  if (s > kMaxSplit) s = kMaxSplit;
  return s < 1 ? 1 : static_cast<int>(s);
}

// ---------------------------------------------------------------- greedy ---
struct GreedyPlan {
  int64_t rows;        // B*(K+1) target rows followed by B*W draft rows
  int split;
  int64_t chunk;
  size_t off_part;     // float2 {value, index-as-bits} per (row, split)
  size_t bytes;
};

inline GreedyPlan plan_greedy(int B, int K, int W, int V) {
  GreedyPlan p{};
  p.rows = static_cast<int64_t>(B) * (K + 1) + static_cast<int64_t>(B) * W;
  p.split = choose_split(p.rows, V);
  p.chunk = chunk_len(V, p.split);
  p.off_part = 0;
  p.bytes = align256(static_cast<size_t>(p.rows) * p.split * 8);
  return p;
}

// -------------------------------------------------------------- sampling ---
// Per-sequence record written by the decide step and read by the draw steps.
struct DrawRecord {
  int kind;     // 0 residual at row `row`, 1 bonus at row `row`, -1 done/error
  int row;
  float Mp, kp, Sp;   // target row statistics
  float Mq, kq, Sq;   // draft row statistics (residual only)
  float u;            // resample uniform
  int pad[7];
};
static_assert(sizeof(DrawRecord) == 64, "DrawRecord is one 64-byte line");

struct SamplePlan {
  int64_t rows;        // B*(K+1) target rows followed by B*K draft rows
  int split;
  int64_t chunk;
  int draw_chunks;
  int64_t draw_chunk;
  size_t off_stats;    // float2 {M, S} per (row, split)
  size_t off_rec;      // DrawRecord per sequence
  size_t off_dsum;     // float per (sequence, draw chunk)
  size_t bytes;
};

inline SamplePlan plan_sample(int B, int K, int V) {
  SamplePlan p{};
  p.rows = static_cast<int64_t>(B) * (K + 1) + static_cast<int64_t>(B) * K;
  p.split = choose_split(p.rows, V);
  p.chunk = chunk_len(V, p.split);
  p.draw_chunks = choose_draw_chunks(B, V);
  p.draw_chunk = chunk_len(V, p.draw_chunks);
  p.off_stats = 0;
  p.off_rec = align256(static_cast<size_t>(p.rows) * p.split * 8);
  p.off_dsum = p.off_rec + align256(static_cast<size_t>(B) * sizeof(DrawRecord));
  p.bytes = p.off_dsum + align256(static_cast<size_t>(B) * p.draw_chunks * 4);
  return p;
}

// ------------------------------------------------------------------ tree ---
struct TreePlan {
  int64_t conf_rows;   // B*S*L (masked rows only do work)
  int split1;
  int64_t chunk1;
  int64_t states;      // B*S
  int split2;
  int64_t chunk2;
  size_t off_conf;     // float2 {M, S} per (b, y, s, split1)
  size_t off_pick;     // float2 {score, index-as-bits} per (b, y, split2)
  size_t off_sel;      // int per (b, y): selected position
  size_t bytes;
};

inline TreePlan plan_tree(int B, int S, int L, int V) {
  TreePlan p{};
  p.conf_rows = static_cast<int64_t>(B) * S * L;
  // About 64% of a block's rows are masked in practice; plan for all.
  p.split1 = choose_split(p.conf_rows, V);
  p.chunk1 = chunk_len(V, p.split1);
  p.states = static_cast<int64_t>(B) * S;
  p.split2 = choose_split(p.states, V);
  p.chunk2 = chunk_len(V, p.split2);
  p.off_conf = 0;
  p.off_pick = align256(static_cast<size_t>(p.conf_rows) * p.split1 * 8);
  p.off_sel = p.off_pick + align256(static_cast<size_t>(p.states) * p.split2 * 8);
  p.bytes = p.off_sel + align256(static_cast<size_t>(p.states) * 4);
  return p;
}

}  // namespace dbv
