// Launch plan and workspace layout: a pure function of the call's sizes, so
// verify_workspace_size() and the launchers always agree.  (The grid size of
// the persistent kernels depends on the device and is chosen at launch; it
// does not change the workspace.)
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace dbv {

constexpr float kLog2eHost = 1.4426950408889634f;

// Row-streaming kernels are persistent: about kResidentPerCU groups per CU
// walk a list of (row, vocabulary chunk) items in grid-stride order, so the
// tail of a launch is one small chunk, not one long row.  Each of a group's
// kWavesPlan waves reduces its share of an item and writes its own partial.
constexpr int kResidentPerCU = 8;
constexpr int kWavesPlan = 4;             // waves per 256-thread group
constexpr int64_t kPlanGroups = 2048;     // 256 CUs x 8 resident groups
constexpr int64_t kChunkMin = 2048;
constexpr int64_t kChunkMax = 32768;
constexpr int64_t kItemsPerGroup = 4;
constexpr int kMaxSplit = 64;
constexpr int kMaxDraft = 1024;       // K and W limit of the chain modes
constexpr int kMaxStates = 1024;      // S limit of the tree mode
constexpr int kMaxBlockLen = 1024;    // L limit of the tree mode

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Chunk length (elements, multiple of 256) for `rows` rows of length V: about
// kItemsPerGroup items per resident group, within [kChunkMin, max_chunk],
// never longer than the row.
inline int64_t choose_chunk(int64_t rows, int64_t V, int64_t max_chunk = kChunkMax) {
  int64_t c = cdiv(rows * V, kItemsPerGroup * kPlanGroups);
  if (c < kChunkMin) c = kChunkMin;
  if (c > max_chunk) c = max_chunk;
  c = cdiv(c, 256) * 256;
  const int64_t whole = cdiv(V, 256) * 256;
  return c < whole ? c : whole;
}

struct RowPlan {
  int64_t rows;
  int64_t chunk;     // elements per item
  int64_t nchunk;    // items per row
  int64_t items;     // rows * nchunk
  size_t part_bytes; // float2 partial per (item, wave)
};

inline RowPlan plan_rows(int64_t rows, int64_t V, int64_t max_chunk = kChunkMax) {
  RowPlan r{};
  r.rows = rows;
  r.chunk = choose_chunk(rows, V, max_chunk);
  r.nchunk = cdiv(V, r.chunk);
  r.items = rows * r.nchunk;
  r.part_bytes = align256(static_cast<size_t>(r.items) * kWavesPlan * 8);
  return r;
}

// Chunks of the correction / bonus draw (one row per sequence): enough
// groups in total, at least 2048 elements each, and never more than
// kDrawChunkMax elements so that the final in-order scan holds a chunk in
// registers (kBlock threads x kDrawVecs vectors of 8).
constexpr int kDrawVecs = 4;
constexpr int kDrawPerThread = 8 * kDrawVecs;          // elements per thread
constexpr int64_t kDrawChunkMax = 256 * kDrawPerThread;
constexpr int kMaxDrawChunks = 256;                    // V <= 2^21 in sampling
constexpr int64_t kMaxSampleV = kDrawChunkMax * kMaxDrawChunks;
inline int choose_draw_chunks(int64_t B, int64_t V) {
  int64_t s = cdiv(1024, B > 0 ? B : 1);
  const int64_t cap = V / 2048 > 0 ? V / 2048 : 1;
  if (s > cap) s = cap;
  if (s > kMaxDrawChunks) s = kMaxDrawChunks;
  const int64_t need = cdiv(V, kDrawChunkMax);   // <= kMaxDrawChunks for V <= kMaxSampleV
  if (s < need) s = need;
  return s < 1 ? 1 : static_cast<int>(s);
}

inline int64_t chunk_len(int64_t V, int split) {
  int64_t c = cdiv(V, split);
  c = cdiv(c, 256) * 256;
  return c < kDrawChunkMax ? c : kDrawChunkMax;
}

// ---------------------------------------------------------------- greedy ---
struct GreedyPlan {
  RowPlan r;          // B*(K+1) target rows followed by B*W draft rows
  size_t off_part;    // float2 {value, index-as-bits} per (item, wave)
  size_t bytes;
};

inline GreedyPlan plan_greedy(int B, int K, int W, int V) {
  GreedyPlan p{};
  p.r = plan_rows(static_cast<int64_t>(B) * (K + 1) + static_cast<int64_t>(B) * W, V);
  p.off_part = 0;
  p.bytes = p.r.part_bytes;
  return p;
}

// -------------------------------------------------------------- sampling ---
// Per-sequence decision handed from the draw-mass kernel to the select
// kernel (written by the sequence's chunk-0 group).
struct DrawRecord {
  int status;        // sequence status bits; error bits mean "done"
  int h;             // accepted drafts; the draw uses row h
  int resid;         // 1: residual [p - q]_+ at row h, 0: bonus from p
  float cp, isp;     // exp2 offset and 1/S of target row h
  float cq, isq;     // same for drafter row h (residual only)
  float u;           // resample uniform of row h
};

struct SamplePlan {
  RowPlan r;           // B*(K+1) target rows followed by B*K draft rows
  int draw_chunks;
  int64_t draw_chunk;
  size_t off_stats;    // float2 {M, S} per (item, wave)
  size_t off_rec;      // DrawRecord per sequence
  size_t off_dsum;     // float per (sequence, draw chunk)
  size_t bytes;
};

inline SamplePlan plan_sample(int B, int K, int V) {
  SamplePlan p{};
  p.r = plan_rows(static_cast<int64_t>(B) * (K + 1) + static_cast<int64_t>(B) * K, V);
  p.draw_chunks = choose_draw_chunks(B, V);
  p.draw_chunk = chunk_len(V, p.draw_chunks);
  p.off_stats = 0;
  p.off_rec = p.r.part_bytes;
  p.off_dsum = p.off_rec + align256(static_cast<size_t>(B) * sizeof(DrawRecord));
  p.bytes = p.off_dsum + align256(static_cast<size_t>(B) * p.draw_chunks * 4);
  return p;
}

// ------------------------------------------------------------------ tree ---
struct TreePlan {
  RowPlan r;           // B*S*L rows (masked rows only do work)
  int64_t states;      // B*S
  int split2;
  int64_t chunk2;
  size_t off_conf;     // float2 {M, S} per (item, wave)
  size_t off_pick;     // float2 {score, index-as-bits} per (state, split2)
  size_t off_sel;      // int per state: selected position
  size_t bytes;
};

// Vocabulary chunks per state for the Gumbel argmax (one row per state).
inline int choose_split(int64_t rows, int64_t V) {
  if (rows <= 0) return 1;
  int64_t s = cdiv(kPlanGroups, rows);
  const int64_t cap = V / 4096 > 0 ? V / 4096 : 1;
  if (s > cap) s = cap;
  if (s > kMaxSplit) s = kMaxSplit;
  return s < 1 ? 1 : static_cast<int>(s);
}

inline TreePlan plan_tree(int B, int S, int L, int V) {
  TreePlan p{};
  // Many rows: a whole row per item keeps the per-position combine short.
  p.r = plan_rows(static_cast<int64_t>(B) * S * L, V, V > kChunkMax ? V : kChunkMax);
  p.states = static_cast<int64_t>(B) * S;
  // The Gumbel argmax keeps no chunk in registers, so its chunks only need to
  // cover the row: ceil(V / split2) rounded up to 256 elements.
  p.split2 = choose_split(p.states, V);
  p.chunk2 = cdiv(cdiv(V, p.split2), 256) * 256;
  p.split2 = static_cast<int>(cdiv(V, p.chunk2));
  p.off_conf = 0;
  p.off_pick = p.r.part_bytes;
  p.off_sel = p.off_pick + align256(static_cast<size_t>(p.states) * p.split2 * 8);
  p.bytes = p.off_sel + align256(static_cast<size_t>(p.states) * 4);
  return p;
}

}  // namespace dbv
