// Launch plan and workspace layout: a pure function of the call's sizes, so
// verify_workspace_size() and the launchers always agree.  The split of the
// streamed rows over the groups of a launch (FlatSplit) is computed on the
// device from the rows a call actually needs, with the same inline functions
// the host uses to size the workspace for the largest possible row count.
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define DBV_HD __host__ __device__
#else
#define DBV_HD
#endif

namespace dbv {

constexpr float kLog2eHost = 1.4426950408889634f;

// Row-streaming kernels are persistent: at most kMaxGrid groups of 256
// threads share the needed rows.  On 256 CUs that is 4 groups (16 waves,
// 64 KiB of 16-byte loads in flight) per CU, which measured faster than 2, 3,
// 6 or 8 groups per CU on every workload; kResidentPerCU bounds the grid on
// smaller devices.
constexpr int kResidentPerCU = 8;
constexpr int kWavesPlan = 4;             // waves per 256-thread group
constexpr int64_t kMaxGrid = 1024;
constexpr int64_t kUnitBytes = 4096;      // granularity of a group's range
constexpr int kMaxSplit = 64;
constexpr int kXcds = 8;              // XCDs of an MI355X; workgroups go to them in turn
constexpr int kMaxDraft = 1024;       // K and W limit of the chain modes
constexpr int kMaxStates = 1024;      // S limit of the tree mode
constexpr int kMaxBlockLen = 1024;    // L limit of the tree mode
constexpr int kSeqBlocks = 1024;      // LDS prefix entries over sequences

// Division of non-negative values; on the device it takes the 32-bit
// instruction sequence when both operands fit (64-bit division is a long
// software routine on this GPU).
DBV_HD inline int64_t udiv(int64_t a, int64_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
  if (((static_cast<uint64_t>(a) | static_cast<uint64_t>(b)) >> 32) == 0)
    return static_cast<int64_t>(static_cast<uint32_t>(a) / static_cast<uint32_t>(b));
#endif
  return a / b;
}

DBV_HD inline int64_t cdiv(int64_t a, int64_t b) { return udiv(a + b - 1, b); }

// Division of 32-bit unsigned values by a fixed divisor d >= 1 through one
// multiply-high and a shift (the round-up method): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(m, n) + n) >> l for
// every n < 2^32 (the sum formed in 64 bits).
struct FastDiv32 {
  uint32_t m = 1, l = 0;
  FastDiv32() = default;
  explicit FastDiv32(uint32_t d) {
    while ((uint64_t(1) << l) < d) ++l;
    m = static_cast<uint32_t>(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  }
  DBV_HD uint32_t div(uint32_t n) const {
    const uint64_t t = (static_cast<uint64_t>(m) * n) >> 32;
    return static_cast<uint32_t>((t + n) >> l);
  }
};
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// ---------------------------------------------------------------------------
// Flat split.  The R needed rows of a call, in a fixed order, form one
// stream of E = R*V elements.  It is cut into NQ units of Q elements (Q*eb =
// kUnitBytes) and group g of the G active groups owns the units
// [g*NQ/G, (g+1)*NQ/G): a contiguous element range, equal to within one
// unit for every group, which may start and end inside rows.  G = min(grid,
// NQ), so no active group is empty.
//
// The piece of row r inside group g's range is reduced to one partial per
// wave, stored at slot (r + g) * waves + wave.  Along the stream each next
// piece advances r, g or both, so r + g is unique per piece and below R + G;
// the partials of one row are the contiguous slots of its groups
// g_lo(r)..g_hi(r).
// ---------------------------------------------------------------------------
struct FlatSplit {
  int64_t V;    // row length (elements)
  int64_t R;    // rows in the stream
  int64_t Q;    // elements per unit
  int64_t NQ;   // units, ceil(R * V / Q)
  int64_t G;    // active groups
};

DBV_HD inline FlatSplit make_split(int64_t R, int64_t V, int64_t elem_bytes, int64_t grid) {
  FlatSplit f;
  f.V = V;
  f.R = R;
  f.Q = kUnitBytes / elem_bytes;
  f.NQ = cdiv(R * V, f.Q);
  f.G = f.NQ < grid ? f.NQ : grid;
  return f;
}

// Element range [e0, e1) of active group g; never empty.
DBV_HD inline void split_range(const FlatSplit& f, int64_t g, int64_t& e0, int64_t& e1) {
  const int64_t E = f.R * f.V;
  e0 = udiv(g * f.NQ, f.G) * f.Q;
  e1 = udiv((g + 1) * f.NQ, f.G) * f.Q;
  if (e1 > E) e1 = E;
}

// The active group whose range holds element e (0 <= e < R*V): the largest g
// with floor(g*NQ/G) <= e / Q.
DBV_HD inline int64_t split_group(const FlatSplit& f, int64_t e) {
  return udiv((udiv(e, f.Q) + 1) * f.G - 1, f.NQ);
}

// First partial slot (in units of waves) and number of groups of row r.
DBV_HD inline void split_row_slots(const FlatSplit& f, int64_t r, int64_t& first, int64_t& ngroups) {
  const int64_t glo = split_group(f, r * f.V);
  const int64_t ghi = split_group(f, r * f.V + f.V - 1);
  first = r + glo;
  ngroups = ghi - glo + 1;
}

// Launch grid of a streaming kernel: enough groups for the largest stream
// the call can need, at most max_grid and the resident groups of the device.
// Streams of at most 1 MiB take four units per group: each CU a group runs
// on fetches the kernel's code (about 25 KB), which on the tiny rejection
// call (36 KB of rows) was over six times the rows' bytes with a group per
// unit, and three groups take the same time as nine.  (Giving larger
// streams fewer, fuller groups measured no faster.)
inline int64_t stream_grid(int64_t max_rows, int64_t V, int64_t elem_bytes, int64_t resident,
                           int64_t max_grid = kMaxGrid) {
  const int64_t bytes = max_rows * V * elem_bytes;
  const int64_t units = cdiv(max_rows * V, (bytes <= (int64_t(1) << 20) ? 4 * kUnitBytes : kUnitBytes) / elem_bytes);
  int64_t g = resident < max_grid ? resident : max_grid;
  return units < g ? units : g;
}

// Bytes of the per-(slot, wave) partials (float2: 8 bytes; the sampling
// statistics with a float64 sum: 16) for up to max_rows rows and max_grid
// groups.
inline size_t partial_bytes(int64_t max_rows, size_t bytes_per = 8, int64_t max_grid = kMaxGrid) {
  return align256(static_cast<size_t>(max_rows + max_grid) * kWavesPlan * bytes_per);
}

// Sampling rows of at most kSmallRowBytes are streamed a piece per wave.
// The fp32 instance of that kernel holds few enough registers for seven
// groups per CU, so its grid may take up to kMaxGridShort groups (more
// pieces in flight per CU); partial buffers of sampling calls are sized for
// it.
constexpr int64_t kSmallRowBytes = 16384;
constexpr int64_t kMaxGridShort = 7 * 256;
DBV_HD inline bool short_rows(int64_t V, int64_t elem_bytes) { return V * elem_bytes <= kSmallRowBytes; }
inline int64_t sample_max_grid(int64_t V, int64_t elem_bytes, bool gumbel) {
  return !gumbel && elem_bytes == 4 && short_rows(V, elem_bytes) ? kMaxGridShort : kMaxGrid;
}

// The correction / bonus draw.  Its row is cut into tiles of 64 16-byte
// vectors (one coalesced wave load per row: 512 bf16 or 256 fp32 elements).
// The mass kernel gives each sequence draw_chunks groups of whole tiles and
// stores every tile's mass; the select kernel (one group per sequence: 256
// threads for rows of at most 1024 tiles, else kDrawThreads) scans the tile
// masses for the tile where the running mass crosses u*Z, and one wave
// rescans that tile in vocabulary order.  kMaxDrawTiles bounds the tiles per
// row (at most kDrawTilesPerThread per thread of a kDrawThreads group), and
// so the vocabulary of the sampling entry points.
// Rows of at most kFusedDrawTiles tiles skip the split: one group per
// sequence makes the decision, computes every tile mass into LDS and draws,
// which saves a kernel boundary and the round trip of the masses.
constexpr int kDrawThreads = 1024;
constexpr int kFusedDrawTiles = 16;
// Stored sparse drafter distributions: at most kMaxNnz entries per row.
constexpr int kMaxNnz = 256;
constexpr int kMaxDrawTiles = 8192;
constexpr int kDrawTilesPerThread = kMaxDrawTiles / kDrawThreads;
constexpr int64_t kMaxSampleV = int64_t(1) << 21;   // <= kMaxDrawTiles tiles of 256 fp32
constexpr int64_t kDrawGroups = 1024;               // mass-kernel groups to aim for

DBV_HD inline int64_t draw_tile(int64_t elem_bytes) { return 64 * 16 / elem_bytes; }
inline int64_t draw_tiles(int64_t V, int64_t elem_bytes) { return cdiv(V, draw_tile(elem_bytes)); }

// Tiles per mass-kernel group: about kDrawGroups groups in all, at least one
// tile each.
inline int64_t draw_tiles_per_chunk(int64_t B, int64_t V, int64_t elem_bytes) {
  const int64_t nt = draw_tiles(V, elem_bytes);
  const int64_t chunks = cdiv(kDrawGroups, B > 0 ? B : 1);
  const int64_t tpc = cdiv(nt, chunks);
  return tpc > 0 ? tpc : 1;
}

// ---------------------------------------------------------------- greedy ---
// Stream order: for each sequence b, target rows 0..n_b, then its W drafter
// rows (a sequence with an invalid draft length contributes no rows).
struct GreedyPlan {
  int64_t max_rows;   // B * (K + 1 + W)
  size_t off_part;    // float2 {value, index-as-bits} per (slot, wave)
  size_t off_pre;     // int32 [B + 1]: first stream row of each sequence
  size_t bytes;
};

inline GreedyPlan plan_greedy(int B, int K, int W, int V) {
  GreedyPlan p{};
  p.max_rows = static_cast<int64_t>(B) * (K + 1 + W);
  p.off_part = 0;
  p.off_pre = partial_bytes(p.max_rows);
  p.bytes = p.off_pre + align256(static_cast<size_t>(B + 1) * 4);
  (void)V;
  return p;
}

// ------------------------------------------------------------- any-order ---
// Stream order: for each sequence b, its verifier rows by rank 0..nver_b-1
// (nver_b = min(kappa_b + 1, u_b)), then its drafter rows by slot 0..u_b-1.
struct AnyOrderPlan {
  int64_t max_rows;   // B * 2U
  size_t off_part;    // float2 {value, index-as-bits} per (slot, wave)
  size_t off_pre;     // int32 [B + 1]: first stream row of each sequence
  size_t off_seq;     // int32 [4][B]: rows, nver, kappa, status per sequence
  size_t bytes;
};

inline AnyOrderPlan plan_any_order(int B, int U) {
  AnyOrderPlan p{};
  p.max_rows = static_cast<int64_t>(B) * 2 * U;
  p.off_part = 0;
  p.off_pre = partial_bytes(p.max_rows);
  p.off_seq = p.off_pre + align256(static_cast<size_t>(B + 1) * 4);
  p.bytes = p.off_seq + align256(static_cast<size_t>(B) * 4 * 4);
  return p;
}

// -------------------------------------------------------------- sampling ---
// Per-sequence decision handed from the mass kernel to the select kernel
// (written by the sequence's chunk-0 group).
struct DrawRecord {
  int status;        // sequence status bits; error bits mean "done"
  int h;             // accepted drafts; the draw uses row h
  int resid;         // 1: residual [p~ - q]_+ at row h, 2: against stored
                     // sparse Q, 0: bonus from p
  float ep, isp;     // target row h: p(v) = exp2(x_v kp - ep) * isp, ep the
                     // integer reference of the row maximum and isp = 1/S
                     // (times the Cactus rescaling of the other tokens; 0
                     // where the residual is known to vanish)
  float chi, clo;    // residual: log2(q(v) / p~(v)) = (y_v kq - x_v kp) +
                     // chi + clo (the row constant in two parts)
  float u;           // resample uniform of row h
  int excl;          // Cactus: the drafted token of row h, whose weight is
  float wexcl;       // wexcl = [gamma - q(d)]_+; -1 for the linear rule
  int fixed;         // >= 0: the committed token is known (a coupled-noise
                     // commit) and nothing is drawn; -1 otherwise
  int pad;
  double isp64;      // 1/S in float64 (stored sparse Q: p(v) - Q(v) of the
                     // listed tokens is formed in float64)
};

// Softmax statistics partial of one piece of a sampling row: the running
// maximum M and the rest R, the sum of exp2(x k - floor(M k)) over all
// elements but one copy of M, in float64.
struct Stat64 {
  float M;
  float pad;
  double R;
};

// The stored sparse Q of the draw row h, handed from the mass kernel to the
// select kernel (which then reads it together with the record).
struct SparseRow {
  int nnz;
  int pad[3];
  int idx[kMaxNnz];
  float prob[kMaxNnz];
};

// Stream order: for each sequence b, target rows 0..n_b, then drafter rows
// 0..n_b-1.  With Gumbel rows each target row is cut into gumbel_parts(eb)
// stream rows ("parts"), so that every stream row carries about the same
// bytes: a target element then costs eb + 4 bytes against eb for a drafter
// element.
DBV_HD inline int gumbel_parts(int64_t elem_bytes) { return static_cast<int>((elem_bytes + 4) / elem_bytes); }

// Element offset in target row of stream offset v (a multiple of 8 below V,
// or V) in part k of P: parts are V_P = floor(V / 8P) * 8 elements wide, the
// last takes the rest.  Monotone in v, so pieces stay contiguous.
DBV_HD inline int64_t part_offset(int64_t V, int P, int k, int64_t v) {
  const int64_t vp = V / (8 * P) * 8;
  if (v >= V) return k + 1 < P ? (k + 1) * vp : V;
  return k * vp + v / (8 * P) * 8;
}

struct SamplePlan {
  int64_t max_rows;    // B * (2K + 1)
  int64_t max_vrows;   // B * (4K + 3): stream rows with Gumbel rows (<= 3 parts)
  int64_t tiles;       // draw tiles per row
  int64_t tpc;         // draw tiles per mass-kernel group
  int64_t chunks;      // mass-kernel groups per sequence
  size_t off_stats;    // {M, float64 S} (16 bytes) per (slot, wave)
  size_t off_gpart;    // float2 {score, index-as-bits} per (slot, wave):
                       // Gumbel argmax partials of target rows
  size_t off_pre;      // int32 [B + 1]: first stream row of each sequence
  size_t off_rec;      // DrawRecord per sequence
  size_t off_tmass;    // float per (sequence, draw tile)
  size_t off_sq;       // SparseRow per sequence (stored sparse Q of row h)
  size_t off_blk;      // int32 [kSeqBlocks]: stream rows per directory block
                       // (B > kSeqBlocks: summed once by k_seq_blocks)
  size_t bytes;
};

inline SamplePlan plan_sample(int B, int K, int V, int64_t elem_bytes) {
  SamplePlan p{};
  p.max_rows = static_cast<int64_t>(B) * (2 * K + 1);
  p.max_vrows = static_cast<int64_t>(B) * (4 * K + 3);
  p.tiles = draw_tiles(V, elem_bytes);
  p.tpc = draw_tiles_per_chunk(B, V, elem_bytes);
  p.chunks = cdiv(p.tiles, p.tpc);
  p.off_stats = 0;
  // partials for the short-row grid, whichever path a call takes
  p.off_gpart = partial_bytes(p.max_vrows, 16, kMaxGridShort);
  p.off_pre = p.off_gpart + partial_bytes(p.max_vrows, 8, kMaxGridShort);
  p.off_rec = p.off_pre + align256(static_cast<size_t>(B + 1) * 4);
  p.off_tmass = p.off_rec + align256(static_cast<size_t>(B) * sizeof(DrawRecord));
  p.off_sq = p.off_tmass + align256(static_cast<size_t>(B) * p.tiles * 4);
  p.off_blk = p.off_sq + align256(static_cast<size_t>(B) * sizeof(SparseRow));
  p.bytes = p.off_blk + align256(static_cast<size_t>(kSeqBlocks) * 4);
  return p;
}

// ------------------------------------------------------------------ tree ---
// Stream order: the needed (state, position) rows in (b, y, s) order, listed
// by the planning kernel: one group of kTreePlanThreads threads, kTreePlanPer
// row ids per thread and pass.  Its list has room for one slot per planning
// thread past B*S*L, its map for the ids of a partial last pass, so that
// every store of a pass is made without a branch.
constexpr int kTreePlanThreads = 1024;
constexpr int kTreePlanPer = 16;
constexpr int64_t kTreePlanPass = static_cast<int64_t>(kTreePlanThreads) * kTreePlanPer;
struct TreePlan {
  int64_t max_rows;    // B*S*L
  int64_t states;      // B*S
  int split2;
  int64_t chunk2;
  size_t off_count;    // int32: rows in the stream
  size_t off_list;     // int32 [max_rows]: flat (b*S + y)*L + s of stream row r
  size_t off_map;      // int32 [max_rows]: stream row of flat row id, or -1
  size_t off_conf;     // float2 {M, S} per (slot, wave)
  size_t off_pick;     // float2 {score, index-as-bits} per (state, split2)
  size_t off_pick2;    // float per (state, split2): the chunk's second-best score
  size_t off_sel;      // int per state: selected position
  size_t off_selconf;  // float per state: confidence at the selected position
  size_t off_selstat;  // int per state: status bits of the state's rows
  size_t off_selgap;   // float per state: relative gap of the two best confidences
  size_t off_batch;    // two int4 per (sequence, batch slot): {s*, n, 0, 0}, the batch's states
  size_t off_nbat;     // int per sequence: batches of the Gumbel argmax
  size_t bytes;
};

// Vocabulary chunks per state for the Gumbel argmax (one row per state):
// about kGumbelGroups one-wave items in all, chunks of at least 4096
// elements.
constexpr int64_t kGumbelGroups = 16384;
inline int choose_split(int64_t rows, int64_t V) {
  if (rows <= 0) return 1;
  int64_t s = cdiv(kGumbelGroups, rows);
  const int64_t cap = V / 4096 > 0 ? V / 4096 : 1;
  if (s > cap) s = cap;
  if (s > kMaxSplit) s = kMaxSplit;
  return s < 1 ? 1 : static_cast<int>(s);
}

inline TreePlan plan_tree(int B, int S, int L, int V) {
  TreePlan p{};
  p.max_rows = static_cast<int64_t>(B) * S * L;
  p.states = static_cast<int64_t>(B) * S;
  // The Gumbel argmax keeps no chunk in registers, so its chunks only need to
  // cover the row: ceil(V / split2) rounded up to 256 elements.
  p.split2 = choose_split(p.states, V);
  p.chunk2 = cdiv(cdiv(V, p.split2), 256) * 256;
  p.split2 = static_cast<int>(cdiv(V, p.chunk2));
  p.off_count = 0;
  p.off_list = 256;
  p.off_map = p.off_list + align256(static_cast<size_t>(p.max_rows + kTreePlanThreads) * 4);
  p.off_conf = p.off_map + align256(static_cast<size_t>(p.max_rows + kTreePlanPass) * 4);
  p.off_pick = p.off_conf + partial_bytes(p.max_rows);
  p.off_pick2 = p.off_pick + align256(static_cast<size_t>(p.states) * p.split2 * 8);
  p.off_sel = p.off_pick2 + align256(static_cast<size_t>(p.states) * p.split2 * 4);
  p.off_selconf = p.off_sel + align256(static_cast<size_t>(p.states) * 4);
  p.off_selstat = p.off_selconf + align256(static_cast<size_t>(p.states) * 4);
  p.off_selgap = p.off_selstat + align256(static_cast<size_t>(p.states) * 4);
  p.off_batch = p.off_selgap + align256(static_cast<size_t>(p.states) * 4);
  p.off_nbat = p.off_batch + align256(static_cast<size_t>(p.states) * 32);
  p.bytes = p.off_nbat + align256(static_cast<size_t>(B) * 4);
  return p;
}

// DDTree: hypotheses over the masked stale rows, then the search.  Blocks of
// at most kDDMaxBlock positions (one bit each in a 64-bit mask) and budgets
// of at most kDDMaxBudget states; the search keeps the tree, the frontier and
// up to kDDMaxCand candidates of one level in LDS.
constexpr int kDDMaxBlock = 64;
constexpr int kDDMaxBudget = 64;
constexpr int kDDMaxCand = kDDMaxBudget * kDDMaxBlock * 2;
constexpr int kDDPartBytes = 32;

struct DDHypPlan {
  int64_t max_rows;    // B*L
  size_t off_count;    // int32
  size_t off_list;     // int32 [max_rows]
  size_t off_map;      // int32 [max_rows]
  size_t off_part;     // DDPart per (slot, wave)
  size_t bytes;
};

inline DDHypPlan plan_dd_hypotheses(int B, int L) {
  DDHypPlan p{};
  p.max_rows = static_cast<int64_t>(B) * L;
  p.off_count = 0;
  p.off_list = 256;
  p.off_map = p.off_list + align256(static_cast<size_t>(p.max_rows) * 4);
  p.off_part = p.off_map + align256(static_cast<size_t>(p.max_rows) * 4);
  p.bytes = p.off_part + align256(static_cast<size_t>(p.max_rows + kMaxGrid) * kWavesPlan * kDDPartBytes);
  return p;
}

// Search state between levels: a 64-bit sort key and a 64-bit masked-set per
// tree node.
inline size_t dd_tree_bytes(int B, int D) {
  return align256(static_cast<size_t>(B) * (D + 1) * 16);
}

}  // namespace dbv
