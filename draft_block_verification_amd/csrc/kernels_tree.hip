// Draft-tree verification by shared-Gumbel state equality (SPOT, Sec. 4.1,
// Sec. 4.3 and App. A.1).
//
//   k_tree_plan    lists the needed rows -- every masked row of every valid
//                  state, or in the fixed-position mode only the given
//                  position's row -- in (sequence, state, position) order,
//                  and maps each (state, position) to its list index: one
//                  group per 1024 row ids, each counting the needed ids
//                  before its range itself (trees of at most 2^18 row ids),
//                  else one group in passes
//   k_tree_conf    persistent: softmax statistics (M, S) partials of every
//                  listed row (the position's confidence is 1/S = max_v p);
//                  the listed rows form one stream split evenly over the
//                  groups (FlatSplit)
//   k_tree_select  per state: s*(y) from the confidences (lowest position on
//                  ties), the status of the state's rows and its margins
//   k_tree_batch   per sequence: its states with a selection, ordered by
//                  (s*, index) and cut into batches of states sharing s*
//   k_tree_gumbel  per (batch, vocabulary chunk): the argmax over v of
//                  z_v / T + G[s*, v] (z_v at T = 0) for each state of the
//                  batch -- the token of Phi(y); one load of a Gumbel chunk
//                  serves the batch, and batches of one s* run on one XCD
//   k_tree_walk    per sequence: validates the tree, gathers Phi(y) for every
//                  state, walks from the root along the child equal to Phi(y)
//                  and commits Phi of the last accepted state.
// The kernel boundaries are the only cross-group synchronisation.
#include "dbv_device.h"
#include "dbv_launch.h"

#include <climits>
#include <type_traits>

namespace dbv {

__device__ __forceinline__ int state_count(const int32_t* num_states, int b, int S) {
  const int ns = num_states ? num_states[b] : S;
  return (ns < 1 || ns > S) ? -1 : ns;
}

// Flat row id (b*S + y)*L + s -> (sequence, state, position); ids are below
// 2^31 (checked by the host), so 32-bit arithmetic suffices.
__device__ __forceinline__ void split_flat(const TreeArgs& a, uint32_t flat, int& b, int& y, int& s) {
  const uint32_t sy = a.divL.div(flat);
  s = static_cast<int>(flat - sy * static_cast<uint32_t>(a.L));
  const uint32_t bb = a.divS.div(sy);
  y = static_cast<int>(sy - bb * static_cast<uint32_t>(a.S));
  b = static_cast<int>(bb);
}

// Is row (b, y, s) needed: a masked position (or the given position in the
// fixed mode) of a state below num_states[b]?
__device__ __forceinline__ bool tree_row_needed(const TreeArgs& a, uint32_t flat) {
  int b, y, s;
  split_flat(a, flat, b, y, s);
  const int ns = state_count(a.num_states, b, a.S);
  if (ns < 0 || y >= ns) return false;
  const int64_t sy = static_cast<int64_t>(b) * a.S + y;
  return a.fixed ? a.next_pos[sy] == s : a.masked[flat] != 0;
}

constexpr int kPlanThreads = kTreePlanThreads;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanPer = kTreePlanPer;    // row ids per thread per pass
constexpr int kScanPer = kPlanPer * kPlanWaves / 64;   // wave counts per lane of the scan
static_assert(kPlanPer * kPlanWaves % 64 == 0, "the scan takes whole lanes");

// Row id t0 + k * kPlanThreads + threadIdx.x is element k of a thread, so
// that every wave reads and writes 64 consecutive ids (coalesced).  List
// order is id order: the listing position of an id is the count of needed
// ids before it, from per-wave ballots and one scan of the kPlanPer x
// kPlanWaves wave counts in id order.  The next pass's loads are issued
// before this pass's stores, and every store is unconditional (ids past F
// and rows not needed write to the padding past the list and the map), so
// the compiler can count the stores and a wait for the loads is not a wait
// for the stores as well (the counter retires them in issue order).
struct PlanLoads {
  int ns[kPlanPer], aux[kPlanPer];
};

// The state count of each id's sequence (NS: from num_states, else S) and
// its mask byte (FIXED: the given position); ids past F are clamped to F - 1
// and ignored.  The modes are template arguments so that the loads form one
// straight run.
template <bool FIXED, bool NS>
__device__ __forceinline__ void plan_load(const TreeArgs& a, uint32_t t0, uint32_t F, PlanLoads& l) {
#pragma unroll
  for (int k = 0; k < kPlanPer; ++k) {
    const uint32_t id = t0 + k * kPlanThreads + threadIdx.x;
    const uint32_t flat = id < F ? id : F - 1;
    int b, y, sp;
    split_flat(a, flat, b, y, sp);
    l.ns[k] = NS ? a.num_states[b] : a.S;
    l.aux[k] = FIXED ? a.next_pos[static_cast<int64_t>(b) * a.S + y] : a.masked[flat];
  }
}

// One pass over ids t0 .. t0 + kPass - 1, whose loads are in l: lists the
// needed ids after the `base` rows of earlier passes, issues the next pass's
// loads into l, and returns base plus the rows listed.
template <bool FIXED, bool NS>
__device__ __forceinline__ int plan_pass(const TreeArgs& a, uint32_t t0, uint32_t F, int base, PlanLoads& l,
                                         int* s_cnt, int* s_total) {
  constexpr uint32_t kPass = kPlanThreads * kPlanPer;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  uint32_t bits = 0;
#pragma unroll
  for (int k = 0; k < kPlanPer; ++k) {
    const uint32_t id = t0 + k * kPlanThreads + threadIdx.x;
    int b, y, sp;
    split_flat(a, id < F ? id : F - 1, b, y, sp);
    // a state count outside [1, S] lists nothing (state_count); & rather
    // than && keeps the test free of branches
    const bool need = (id < F) & (l.ns[k] >= 1) & (l.ns[k] <= a.S) & (y < l.ns[k]) &
                      (FIXED ? l.aux[k] == sp : l.aux[k] != 0);
    bits |= static_cast<uint32_t>(need) << k;
    const uint64_t m = __ballot(need);
    if (lane == 0) s_cnt[k * kPlanWaves + wv] = __popcll(m);
  }
  if (t0 + kPass < F) plan_load<FIXED, NS>(a, t0 + kPass, F, l);
  __syncthreads();
  // Exclusive scan of the kPlanPer * kPlanWaves counts in id order by wave 0,
  // kScanPer consecutive counts per lane; the pass total to s_total.
  if (wv == 0) {
    int c[kScanPer], sum = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      c[j] = s_cnt[lane * kScanPer + j];
      sum += c[j];
    }
    int inc = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(inc, d, 64);
      if (lane >= d) inc += o;
    }
    int run = inc - sum;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      s_cnt[lane * kScanPer + j] = run;
      run += c[j];
    }
    if (lane == 63) *s_total = inc;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPlanPer; ++k) {
    const uint32_t id = t0 + k * kPlanThreads + threadIdx.x;
    const bool need = (bits >> k) & 1u;
    const uint64_t m = __ballot(need);
    const int off = base + s_cnt[k * kPlanWaves + wv] + __popcll(m & below);
    a.list[need ? static_cast<int64_t>(off) : static_cast<int64_t>(F) + threadIdx.x] = static_cast<int32_t>(id);
    a.map[id] = need ? off : -1;   // id < F + kPass: within the padded map
  }
  const int n = *s_total;
  __syncthreads();
  return base + n;
}

// Is flat row id u (< F) needed: a valid state's masked position, or its
// given position in the fixed mode?  Reads the state count and the mask
// byte (the given position) of u.
template <bool FIXED, bool NS>
__device__ __forceinline__ bool plan_need(const TreeArgs& a, uint32_t u) {
  int b, y, sp;
  split_flat(a, u, b, y, sp);
  const int ns = NS ? a.num_states[b] : a.S;
  const int aux = FIXED ? a.next_pos[static_cast<int64_t>(b) * a.S + y] : a.masked[u];
  return (ns >= 1) & (ns <= a.S) & (y < ns) & (FIXED ? aux == sp : aux != 0);
}

// Trees of at most kPlanWideMax row ids: one group of kPlanThreads threads
// per kPlanThreads consecutive ids, one id per thread.  Group g counts the
// needed ids before its range itself (about g ids per thread, spread over
// the group), so the groups need nothing from each other; the list position
// of an id is that count plus the needed ids before it in the group (wave
// ballots and the wave counts).  The last group writes the stream length.
constexpr uint32_t kPlanWideMax = 1u << 18;

template <bool FIXED, bool NS>
__global__ __launch_bounds__(kPlanThreads) void k_tree_plan_wide(TreeArgs a) {
  __shared__ int s_w[kPlanWaves], s_c[kPlanWaves];
  const uint32_t F = static_cast<uint32_t>(a.B) * a.S * a.L;
  const uint32_t g0 = blockIdx.x * kPlanThreads;
  const uint32_t id = g0 + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const bool need = id < F && plan_need<FIXED, NS>(a, id);
  int before = 0;
#pragma unroll 8
  for (uint32_t u = threadIdx.x; u < g0; u += kPlanThreads) before += plan_need<FIXED, NS>(a, u) ? 1 : 0;
  for (int m = 32; m >= 1; m >>= 1) before += __shfl_xor(before, m, 64);
  const uint64_t bal = __ballot(need);
  if (lane == 0) {
    s_c[wv] = before;
    s_w[wv] = __popcll(bal);
  }
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) {
    base += s_c[w];
    if (w < wv) total += s_w[w];
  }
  const int off = base + total + __popcll(bal & ((uint64_t(1) << lane) - 1));
  a.list[need ? static_cast<int64_t>(off) : static_cast<int64_t>(F) + threadIdx.x] = static_cast<int32_t>(id);
  a.map[id] = need ? off : -1;   // id < F + kPlanThreads: within the padded map
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == kPlanThreads - 1) *a.count = off + (need ? 1 : 0);
}

// The first pass is peeled from the loop, so that the loop is entered only
// where a pass's stores follow the next pass's loads, and its waits for
// those loads count the stores.
template <bool FIXED, bool NS>
__global__ __launch_bounds__(kPlanThreads) void k_tree_plan(TreeArgs a) {
  __shared__ int s_cnt[kPlanPer * kPlanWaves];
  __shared__ int s_total;
  const uint32_t F = static_cast<uint32_t>(a.B) * a.S * a.L;
  constexpr uint32_t kPass = kPlanThreads * kPlanPer;
  int base = 0;  // stream rows listed by earlier passes
  if (F > 0) {
    PlanLoads l;
    plan_load<FIXED, NS>(a, 0, F, l);
    base = plan_pass<FIXED, NS>(a, 0, F, base, l, s_cnt, &s_total);
    for (uint32_t t0 = kPass; t0 < F; t0 += kPass) base = plan_pass<FIXED, NS>(a, t0, F, base, l, s_cnt, &s_total);
  }
  if (threadIdx.x == 0) *a.count = base;
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_tree_conf(TreeArgs a) {
  const FlatSplit f = make_split(*a.count, a.V, Elem<DT>::kBytes, a.grid);
  const int64_t g = blockIdx.x;
  if (g >= f.G) return;
  for_pieces(f, g, [&](int64_t r, int64_t v0, int64_t v1, const Progress& pg) {
    int b, y, s;
    split_flat(a, static_cast<uint32_t>(a.list[r]), b, y, s);
    const char* rowp = static_cast<const char*>(a.logits) +
                       (b * a.ss + y * a.sy + s * a.sp) * Elem<DT>::kBytes;
    SoftmaxStats st(kLog2e);
    stream_row<DT, 4>(rowp, v0, v1, st, pg);
    float M = st.M, S = st.S;
    wave_stats(M, S, kLog2e);
    if ((threadIdx.x & 63) == 0) a.conf[(r + g) * kWaves + (threadIdx.x >> 6)] = make_float2(M, S);
  });
}

// Combined statistics of the listed row with flat id `flat`.
__device__ __forceinline__ void combine_conf(const TreeArgs& a, const FlatSplit& f, int64_t flat, float& M,
                                             float& S) {
  int64_t first, n;
  split_row_slots(f, a.map[flat], first, n);
  merge_span_stats(a.conf, first * kWaves, n * kWaves, kLog2e, M, S);
}

// s*(y): the masked position of largest confidence 1/S (lowest on ties), or
// the given position in the fixed mode; -1 when there is none.  Also the
// status bits of every row the state reads, the confidence at s*, and (with
// `gap`) the relative gap 1 - S(s*)/S(second) of the two best confidences
// (1 with a single masked position, 0 in the fixed mode).  Every thread of
// the group calls it; the results are uniform.
struct Selection {
  int pos;
  int status;
  float conf;
  float gap;
};

__device__ Selection select_position(const TreeArgs& a, const FlatSplit& f, int b, int y, bool gap, float* s_v,
                                     int* s_i, int* s_n, int* s_out, float* s_f) {
  const int64_t sy = static_cast<int64_t>(b) * a.S + y;
  Selection r{-1, 0, __builtin_nanf(""), 0.f};
  if (a.fixed) {
    const int np = a.next_pos[sy];
    if (np >= 0 && np < a.L) {
      float M, S;
      combine_conf(a, f, sy * a.L + np, M, S);
      r.pos = np;
      r.status = stats_status(M, S);
      r.conf = 1.f / S;
    }
    return r;
  }
  constexpr int kPer = (kMaxBlockLen + kBlock - 1) / kBlock;   // positions of one thread
  float negs[kPer];
  float v = -kInf;
  int idx = -1, nan = 0, st = 0;
  if (threadIdx.x == 0) s_out[1] = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int s = static_cast<int>(threadIdx.x) + k * kBlock;
    negs[k] = -kInf;
    if (s < a.L && a.masked[sy * a.L + s]) {
      float M, S;
      combine_conf(a, f, sy * a.L + s, M, S);
      st |= stats_status(M, S);
      negs[k] = -S;
      if (pick_better(-S, s, v, idx)) { v = -S; idx = s; }   // max of -S = min of S
    }
  }
  __syncthreads();
  if (st) atomicOr(&s_out[1], st);
  block_argmax(v, idx, nan, s_v, s_i, s_n);
  if (threadIdx.x == 0) {
    s_out[0] = idx;
    s_f[0] = v;
  }
  __syncthreads();
  r.pos = s_out[0];
  r.status = s_out[1];
  const float best = s_f[0];
  r.conf = r.pos >= 0 ? -1.f / best : __builtin_nanf("");
  __syncthreads();
  if (gap && r.pos >= 0) {
    // the largest -S over the other masked positions
    float v2 = -kInf;
    int i2 = -1, n2 = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int s = static_cast<int>(threadIdx.x) + k * kBlock;
      if (s < a.L && s != r.pos && negs[k] > -kInf && pick_better(negs[k], s, v2, i2)) { v2 = negs[k]; i2 = s; }
    }
    block_argmax(v2, i2, n2, s_v, s_i, s_n);
    if (threadIdx.x == 0) s_f[1] = i2 >= 0 ? 1.f - best / v2 : 1.f;   // 1 - S(s*) / S(second)
    __syncthreads();
    r.gap = s_f[1];
    __syncthreads();
  }
  return r;
}

// Lowest-index argmax that also keeps the second-largest score: per element
// second = med3(best, second, x) before best = max(best, x), so two equal
// largest scores leave second = best.
struct ArgmaxPick2 : ArgmaxPick {
  float second = -kInf;
  template <int N>
  __device__ __forceinline__ void group(const float* x, int64_t idx0) {
    float b1 = best;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      second = __builtin_amdgcn_fmed3f(b1, second, x[j]);
      b1 = fmaxf(b1, x[j]);
    }
    ArgmaxPick::group<N>(x, idx0);
  }
  template <int U, int W>
  __device__ __forceinline__ void block(const float* x, int64_t idx0, int64_t ustride) {
#pragma unroll
    for (int u = 0; u < U; ++u) group<W>(x + u * W, idx0 + u * ustride);
  }
};

// Argmax of z/T + g over a logit row and its Gumbel row read together.
template <int DT, int NT, class Pick>
__device__ void gumbel_argmax(const char* xr, const float* gr, int64_t v0, int64_t v1, float inv_t,
                              Pick& pk) {
  using E = Elem<DT>;
  constexpr int W = E::kVec;
  const int t = threadIdx.x;
  const uintptr_t ax = reinterpret_cast<uintptr_t>(xr + v0 * E::kBytes);
  int64_t head = static_cast<int64_t>(((16u - (ax & 15u)) & 15u) / E::kBytes);
  if (head > v1 - v0) head = v1 - v0;
  const int64_t a0 = v0 + head;
  const bool gal = ((reinterpret_cast<uintptr_t>(gr + a0)) & 15u) == 0;
  if (!gal) {  // Gumbel row not aligned with the logits: scalar path
    for (int64_t j = v0 + t; j < v1; j += NT) {
      float x[1] = {__builtin_fmaf(E::load1(xr, j), inv_t, gr[j])};
      pk.template group<1>(x, j);
    }
    return;
  }
  const int64_t nvec = (v1 - a0) / W;
  const int64_t a1 = a0 + nvec * W;
  if (t < head) {
    float x[1] = {__builtin_fmaf(E::load1(xr, v0 + t), inv_t, gr[v0 + t])};
    pk.template group<1>(x, v0 + t);
  }
  const char* xb = xr + a0 * E::kBytes;
  const char* gb = reinterpret_cast<const char*>(gr + a0);
  constexpr int GV = W / 4;  // 16-byte Gumbel loads per logit vector
  constexpr int U = 4;       // logit vectors in flight per lane
  int64_t i = t;
  for (; i + (U - 1) * NT < nvec; i += U * NT) {
    u32x4 xv[U], g[U][GV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      xv[u] = load16(xb + (i + u * NT) * 16);
#pragma unroll
      for (int q = 0; q < GV; ++q) g[u][q] = load16(gb + ((i + u * NT) * W + q * 4) * 4);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[W];
      E::unpack(xv[u], x);
#pragma unroll
      for (int j = 0; j < W; ++j) x[j] = __builtin_fmaf(x[j], inv_t, __uint_as_float(g[u][j / 4][j % 4]));
      pk.template group<W>(x, a0 + (i + u * NT) * W);
    }
  }
  for (; i < nvec; i += NT) {
    u32x4 xv = load16(xb + i * 16);
    u32x4 g[GV];
#pragma unroll
    for (int q = 0; q < GV; ++q) g[q] = load16(gb + (i * W + q * 4) * 4);
    float x[W];
    E::unpack(xv, x);
#pragma unroll
    for (int j = 0; j < W; ++j) x[j] = __builtin_fmaf(x[j], inv_t, __uint_as_float(g[j / 4][j % 4]));
    pk.template group<W>(x, a0 + i * W);
  }
  if (a1 + t < v1) {
    float x[1] = {__builtin_fmaf(E::load1(xr, a1 + t), inv_t, gr[a1 + t])};
    pk.template group<1>(x, a1 + t);
  }
}

// Argmax of z/T + g for up to NB logit rows that share one Gumbel row (the
// states of one batch have the same s*): each Gumbel vector is loaded once
// and used for every row.  Rows and the Gumbel row must be 16-byte aligned
// at v0 (the caller checks); n rows are live (uniform across the group).
template <int DT, int NB, int NT, class Pick>
__device__ void gumbel_argmax_batch(const char* const (&xr)[NB], int n, const float* gr, int64_t v0, int64_t v1,
                                    float inv_t, Pick (&pk)[NB]) {
  using E = Elem<DT>;
  constexpr int W = E::kVec;
  constexpr int GV = W / 4;
  constexpr int U = 2;   // vectors in flight per row and lane
  const int t = threadIdx.x;
  const int64_t nvec = (v1 - v0) / W;
  const char* gb = reinterpret_cast<const char*>(gr + v0);
  int64_t i = t;
  for (; i + (U - 1) * NT < nvec; i += U * NT) {
    u32x4 g[U][GV], xv[NB][U];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < GV; ++q) g[u][q] = load16(gb + ((i + u * NT) * W + q * 4) * 4);
#pragma unroll
    for (int r = 0; r < NB; ++r)
      if (r < n)
#pragma unroll
        for (int u = 0; u < U; ++u) xv[r][u] = load16(xr[r] + (v0 + (i + u * NT) * W) * E::kBytes);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      if (r < n) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float x[W];
          E::unpack(xv[r][u], x);
#pragma unroll
          for (int j = 0; j < W; ++j) x[j] = __builtin_fmaf(x[j], inv_t, __uint_as_float(g[u][j / 4][j % 4]));
          pk[r].template group<W>(x, v0 + (i + u * NT) * W);
        }
      }
    }
  }
  for (; i < nvec; i += NT) {
    u32x4 g[GV];
#pragma unroll
    for (int q = 0; q < GV; ++q) g[q] = load16(gb + (i * W + q * 4) * 4);
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      if (r < n) {
        float x[W];
        E::unpack(load16(xr[r] + (v0 + i * W) * E::kBytes), x);
#pragma unroll
        for (int j = 0; j < W; ++j) x[j] = __builtin_fmaf(x[j], inv_t, __uint_as_float(g[j / 4][j % 4]));
        pk[r].template group<W>(x, v0 + i * W);
      }
    }
  }
  for (int64_t e = v0 + nvec * W + t; e < v1; e += NT) {
    const float ge = gr[e];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      if (r < n) {
        float x[1] = {__builtin_fmaf(E::load1(xr[r], e), inv_t, ge)};
        pk[r].template group<1>(x, e);
      }
    }
  }
}

// The walk of one sequence, from the per-state selections of k_tree_gumbel.
__device__ void tree_walk(const TreeArgs& a, int b, int* s_pos, int* s_tok) {
  __shared__ int s_st, s_child, s_y, s_len, s_ncommit;
  const int t = threadIdx.x;
  const int S = a.S;
  const int ns = state_count(a.num_states, b, S);
  const int64_t base = static_cast<int64_t>(b) * S;
  const int32_t* par = a.parent + base;
  const int32_t* ep = a.edge_pos + base;
  const int32_t* et = a.edge_tok + base;
  if (t == 0) s_st = ns < 0 ? SEQ_BAD_INPUT : 0;
  __syncthreads();
  int st = 0;
  if (ns > 0) {
    if (t == 0 && par[0] != -1) st |= SEQ_BAD_INPUT;
    for (int z = t + 1; z < ns; z += kBlock) {
      const int pz = par[z];
      if (pz < 0 || pz >= z) st |= SEQ_BAD_INPUT;
      if (ep[z] < 0 || ep[z] >= a.L || et[z] < 0 || et[z] >= a.V) st |= SEQ_BAD_INPUT;
    }
    if (a.fixed) {
      for (int z = t; z < ns; z += kBlock) {
        const int np = a.next_pos[base + z];
        if (np < -1 || np >= a.L) st |= SEQ_BAD_INPUT;
      }
    }
  }
  if (st) atomicOr(&s_st, st);
  __syncthreads();
  st = 0;
  const bool valid = !(s_st & SEQ_BAD_INPUT);
  // Phi(y) per state: s* with the status of the state's rows, the token
  // from the chunks' picks (largest score, lowest index).
  for (int y = t; y < S; y += kBlock) {
    int pos = -1, tok = -1;
    float conf = __builtin_nanf(""), pgap = 0.f, tgap = 0.f;
    if (valid && y < ns) {
      const int64_t sy = base + y;
      pos = a.sel[sy];
      st |= a.selstat[sy];
      if (pos >= 0) {
        conf = a.selconf[sy];
        pgap = a.selgap[sy];
        float v = -kInf;
        int idx = -1, nan = 0;
        const float2* pk = a.pick + sy * a.split2;
        // the chunks in order, eight requested at a time
        for (int k0 = 0; k0 < a.split2; k0 += 8) {
          float2 q[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) q[u] = pk[k0 + u < a.split2 ? k0 + u : a.split2 - 1];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            if (k0 + u < a.split2) {
              const int i2 = __float_as_int(q[u].y);
              if (q[u].x != q[u].x) nan = 1;
              else if (pick_better(q[u].x, i2, v, idx)) { v = q[u].x; idx = i2; }
            }
          }
        }
        st |= nan ? SEQ_NONFINITE : max_status(v);
        tok = idx;
        if (a.tok_margin) {
          float v2 = -kInf;
          for (int k = 0; k < a.split2; ++k) {
            const bool win = pk[k].x == v && __float_as_int(pk[k].y) == idx;
            v2 = fmaxf(v2, win ? a.pick2[sy * a.split2 + k] : pk[k].x);
          }
          tgap = v - v2;
        }
      }
    }
    s_pos[y] = pos;
    s_tok[y] = tok;
    if (a.sel_pos) a.sel_pos[base + y] = pos;
    if (a.sel_tok) a.sel_tok[base + y] = tok;
    if (a.sel_conf) a.sel_conf[base + y] = conf;
    if (a.pos_margin) a.pos_margin[base + y] = pgap;
    if (a.tok_margin) a.tok_margin[base + y] = tgap;
  }
  if (st) atomicOr(&s_st, st);
  __syncthreads();
  const int status = s_st;
  int32_t* pn = a.path_nodes + base;
  int32_t* cp = a.commit_pos + base;
  int32_t* ct = a.commit_tok + base;
  for (int z = t; z < S; z += kBlock) { pn[z] = -1; cp[z] = -1; ct[z] = -1; }
  __syncthreads();
  if (status & SEQ_ERROR_MASK) {
    if (t == 0) {
      a.path_len[b] = -1;
      a.num_commits[b] = 0;
      if (a.status) a.status[b] = status;
    }
    return;
  }
  if (t == 0) { s_y = 0; s_len = 0; s_ncommit = 0; }
  __syncthreads();
  // Accept the child equal to Phi(y) (lowest node index), else commit Phi(y)
  // and stop; a state without transition ends the walk.
  for (int step = 0; step < ns; ++step) {
    const int y = s_y;
    const int pos = s_pos[y], tok = s_tok[y];
    if (pos < 0) break;
    if (t == 0) s_child = INT_MAX;
    __syncthreads();
    for (int z = y + 1 + t; z < ns; z += kBlock)
      if (par[z] == y && ep[z] == pos && et[z] == tok) atomicMin(&s_child, z);
    __syncthreads();
    const int child = s_child;
    __syncthreads();
    if (t == 0) {
      if (child == INT_MAX) {
        cp[s_ncommit] = pos;
        ct[s_ncommit] = tok;
        s_ncommit += 1;
      } else {
        s_len += 1;
        pn[s_len] = child;
        cp[s_ncommit] = ep[child];
        ct[s_ncommit] = et[child];
        s_ncommit += 1;
        s_y = child;
      }
    }
    __syncthreads();
    if (child == INT_MAX) break;
  }
  if (t == 0) {
    pn[0] = 0;
    a.path_len[b] = s_len;
    a.num_commits[b] = s_ncommit;
    if (a.status) a.status[b] = status;
  }
}

// Per state: s*(y) with the status of the state's rows, the confidence at
// s* and (pos_margin) the gap of the two best confidences.
template <int DT>
__global__ __launch_bounds__(kBlock) void k_tree_select(TreeArgs a) {
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves], s_n[kWaves], s_sel[2];
  __shared__ float s_f[2];
  const int64_t sy = blockIdx.x;
  const int b = static_cast<int>(sy / a.S);
  const int y = static_cast<int>(sy - static_cast<int64_t>(b) * a.S);
  const int ns = state_count(a.num_states, b, a.S);
  if (ns > 0 && y < ns) {
    const FlatSplit f = make_split(*a.count, a.V, Elem<DT>::kBytes, a.grid);
    const Selection sel = select_position(a, f, b, y, a.pos_margin != nullptr, s_v, s_i, s_n, s_sel, s_f);
    if (threadIdx.x == 0) {
      a.sel[sy] = sel.pos;
      a.selstat[sy] = sel.status;
      a.selconf[sy] = sel.conf;
      a.selgap[sy] = sel.gap;
    }
  }
}

// States of at most this many per sequence are taken in batches of states
// sharing s* (below); larger trees one state per batch in index order.
constexpr int kGroupStates = 128;
constexpr int kBatch = 4;   // states per batch (at most 4: one int4 holds them)
static_assert(kBatch >= 1 && kBatch <= 4, "batch size");

// Batching of one sequence's states in LDS.
struct BatchLds {
  __align__(16) int key[kGroupStates];
  int rank[kGroupStates], q[kGroupStates], flag[kGroupStates], bid[kGroupStates];
  int bs[kGroupStates], bn[kGroupStates], by[kGroupStates][kBatch];
  int wave[kPlanWaves], nb;
};

// The states y < num_states of sequence b with a selection, ordered by
// (s*, index) and cut into batches of at most kBatch consecutive states with
// the same s*.  Batch j of sequence b is batch[2 (b S + j)] = {s*, n, 0, 0}
// and batch[2 (b S + j) + 1] = its n states (-1 past n); nbat[b] = the
// number of batches.  On entry (before a barrier) s.key[t], t <
// kGroupStates, holds state t's s*, L (after every position) for a state
// past ns or without a selection -- such states join no batch -- and
// INT_MAX past S.  S <= kGroupStates; NT threads, NT >= kGroupStates.
template <int NT>
__device__ __forceinline__ void batch_states(const TreeArgs& a, int b, BatchLds& s) {
  static_assert(kGroupStates % 4 == 0 && kGroupStates <= NT && NT / 64 <= kPlanWaves, "batching layout");
  const int t = threadIdx.x;
  int4* out = a.batch + 2 * static_cast<int64_t>(b) * a.S;
  if (t < kGroupStates) {
    s.bn[t] = 0;
#pragma unroll
    for (int r = 0; r < kBatch; ++r) s.by[t][r] = -1;
  }
  __syncthreads();
  // rank r of state t by (key, index) and its place q among the states with
  // its key; a batch starts at every q divisible by kBatch
  int kt = INT_MAX, r = 0;
  if (t < a.S) {
    kt = s.key[t];
    int less = 0;
#pragma unroll
    for (int u = 0; u < kGroupStates; u += 4) {
      const int4 k4 = *reinterpret_cast<const int4*>(&s.key[u]);
      const int ku[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        less += ku[e] < kt ? 1 : 0;
        r += (ku[e] < kt || (ku[e] == kt && u + e < t)) ? 1 : 0;
      }
    }
    s.rank[t] = r;
    s.q[t] = r - less;
    s.flag[r] = ((r - less) % kBatch == 0 && kt < a.L) ? 1 : 0;
  }
  __syncthreads();
  // batch id of rank r: the batch starts at ranks up to r, minus one (an
  // inclusive count by wave ballots, then the counts of earlier waves)
  const int lane = t & 63, wv = t >> 6;
  const int f = t < a.S ? s.flag[t] : 0;
  const uint64_t m = __ballot(f != 0);
  if (lane == 0) s.wave[wv] = __popcll(m);
  __syncthreads();
  if (t < a.S) {
    int c = __popcll(m & ((uint64_t(2) << lane) - 1));   // lanes 0..lane
    for (int w = 0; w < wv; ++w) c += s.wave[w];
    s.bid[t] = c - 1;
  }
  if (t == 0) {
    int nb = 0;
    for (int w = 0; w < NT / 64; ++w) nb += s.wave[w];
    s.nb = nb;
  }
  __syncthreads();
  if (t < a.S && kt < a.L) {
    const int bid = s.bid[r];
    const int slot = s.q[t] % kBatch;
    s.by[bid][slot] = t;
    atomicMax(&s.bn[bid], slot + 1);
    if (slot == 0) s.bs[bid] = kt;
  }
  __syncthreads();
  const int nb = s.nb;
  for (int j = t; j < nb; j += NT) {
    out[2 * j] = make_int4(s.bs[j], s.bn[j], 0, 0);
    int ys[4] = {-1, -1, -1, -1};
#pragma unroll
    for (int q = 0; q < kBatch; ++q) ys[q] = s.by[j][q];
    out[2 * j + 1] = make_int4(ys[0], ys[1], ys[2], ys[3]);
  }
  if (t == 0) a.nbat[b] = nb;
}

// The batches of sequence b from the selections k_tree_select wrote (see
// batch_states); nbat[b] = 0 for an invalid state count.  In a tree of more
// than kGroupStates states batch j is state j alone (n = 0 without a
// selection).
__global__ __launch_bounds__(kBlock) void k_tree_batch(TreeArgs a) {
  __shared__ BatchLds s;
  const int b = blockIdx.x;
  const int ns = state_count(a.num_states, b, a.S);
  const int64_t base = static_cast<int64_t>(b) * a.S;
  if (ns <= 0) {
    if (threadIdx.x == 0) a.nbat[b] = 0;
    return;
  }
  if (a.S > kGroupStates) {
    int4* out = a.batch + 2 * base;
    for (int t = threadIdx.x; t < ns; t += kBlock) {
      const int p = a.sel[base + t];
      out[2 * t] = make_int4(p, p >= 0 ? 1 : 0, 0, 0);
      out[2 * t + 1] = make_int4(t, -1, -1, -1);
    }
    if (threadIdx.x == 0) a.nbat[b] = ns;
    return;
  }
  const int t = threadIdx.x;
  if (t < kGroupStates) {
    const int p = t < ns ? a.sel[base + t] : -1;
    s.key[t] = t >= a.S ? INT_MAX : p >= 0 ? p : a.L;
  }
  batch_states<kBlock>(a, b, s);
}

// Items of the Gumbel argmax, one group each: (batch slot j, sequence,
// chunk) in that order, j-major, the (sequence, chunk) count padded to a
// multiple of the XCD count, so that the items of one (sequence, chunk) for
// consecutive j -- batches that mostly share s*, so read the same Gumbel
// chunk -- land on one XCD (workgroups go to the XCDs in turn), and the live
// batches of every sequence are dispatched first.
__host__ __device__ inline int64_t gumbel_stride(int B, int split2) {
  return (static_cast<int64_t>(B) * split2 + kXcds - 1) / kXcds * kXcds;
}

// One wave per Gumbel item: with many small groups instead of fewer large
// ones the hardware places about the same work on every CU (with 256-thread
// items the CUs held 13 to 20 states and the kernel waited for the fullest).
constexpr int kGumbelThreads = 64;

// Item w, one wave: each state's argmax over the chunk of z/T + G[s*] (z at
// T = 0).  TWO: also the chunk's second-largest score (tok_margin).  One
// load of a Gumbel chunk serves every state of the batch.
template <int DT, bool TWO>
__device__ __forceinline__ void gumbel_item(const TreeArgs& a, int64_t w) {
  constexpr int NT = kGumbelThreads;
  using E = Elem<DT>;
  using Pick = typename std::conditional<TWO, ArgmaxPick2, ArgmaxPick>::type;
  const int64_t P = gumbel_stride(a.B, a.split2);
  const int j = static_cast<int>(w / P);
  const int64_t rem = w - j * P;
  if (rem >= static_cast<int64_t>(a.B) * a.split2) return;
  const int b = static_cast<int>(rem / a.split2);
  const int sp = static_cast<int>(rem - static_cast<int64_t>(b) * a.split2);
  if (j >= a.nbat[b]) return;
  const int64_t base = static_cast<int64_t>(b) * a.S;
  const int4 hd = a.batch[2 * (base + j)];
  const int4 yv = a.batch[2 * (base + j) + 1];
  const int n = hd.y < kBatch ? hd.y : kBatch;
  const int s = hd.x;
  if (n <= 0 || s < 0 || s >= a.L) return;
  const int ya[4] = {yv.x, yv.y, yv.z, yv.w};
  int sy[kBatch];
#pragma unroll
  for (int r = 0; r < kBatch; ++r) sy[r] = ya[r];
  const int64_t v0 = static_cast<int64_t>(sp) * a.chunk2;
  const int64_t v1 = v0 + a.chunk2 < a.V ? v0 + a.chunk2 : a.V;
  const char* xr[kBatch];
  uintptr_t al = 0;
#pragma unroll
  for (int r = 0; r < kBatch; ++r) {
    const int y = sy[r < n ? r : 0];
    xr[r] = static_cast<const char*>(a.logits) + (b * a.ss + y * a.sy + s * a.sp) * E::kBytes;
    al |= reinterpret_cast<uintptr_t>(xr[r] + v0 * E::kBytes);
  }
  Pick pk[kBatch];
  if (a.inv_t > 0.f) {
    const float* gr = a.gumbel + b * a.gs + s * a.gp;
    if (((al | reinterpret_cast<uintptr_t>(gr + v0)) & 15u) == 0) {
      gumbel_argmax_batch<DT, kBatch, NT>(xr, n, gr, v0, v1, a.inv_t, pk);
    } else {
#pragma unroll
      for (int r = 0; r < kBatch; ++r)
        if (r < n) gumbel_argmax<DT, NT>(xr[r], gr, v0, v1, a.inv_t, pk[r]);
    }
  } else {
#pragma unroll
    for (int r = 0; r < kBatch; ++r)
      if (r < n) stream_row<DT, 4, Pick, NT>(xr[r], v0, v1, pk[r]);
  }
#pragma unroll
  for (int r = 0; r < kBatch; ++r) {
    if (r < n) {
      const int64_t gid = (base + sy[r]) * a.split2 + sp;
      float v = pk[r].best;
      int ii = static_cast<int>(pk[r].bidx);
      int nan = pk[r].nan ? 1 : 0;
      const float tb = v;
      const int ti = ii;
      wave_argmax(v, ii, nan);
      if (threadIdx.x == 0) a.pick[gid] = make_float2(nan ? __builtin_nanf("") : v, __int_as_float(ii));
      if constexpr (TWO) {
        // the largest of every other lane's best and the winning lane's
        // second
        float c = (tb == v && ti == ii) ? pk[r].second : tb;
        int ci = 0, cn = 0;
        wave_argmax(c, ci, cn);
        if (threadIdx.x == 0) a.pick2[gid] = c;
      }
    }
  }
}

template <int DT, bool TWO>
__global__ __launch_bounds__(kGumbelThreads) void k_tree_gumbel(TreeArgs a) {
  gumbel_item<DT, TWO>(a, blockIdx.x);
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_tree_walk(TreeArgs a) {
  __shared__ int s_pos[kMaxStates], s_tok[kMaxStates];
  tree_walk(a, blockIdx.x, s_pos, s_tok);
}

template <typename K>
static const void* fn(K* k) {
  return reinterpret_cast<const void*>(k);
}

bool launch_tree(const TreeArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev) {
  const bool bf = dtype == DT_BF16;
  const bool two = a.tok_margin != nullptr;
  const void* gum = bf ? (two ? fn(k_tree_gumbel<DT_BF16, true>) : fn(k_tree_gumbel<DT_BF16, false>))
                       : (two ? fn(k_tree_gumbel<DT_F32, true>) : fn(k_tree_gumbel<DT_F32, false>));
  const int64_t items = static_cast<int64_t>(a.S) * gumbel_stride(a.B, a.split2);
  const bool ns = a.num_states != nullptr;
  const uint32_t F = static_cast<uint32_t>(a.B) * a.S * a.L;
  const bool wide = F <= kPlanWideMax;
  const void* plan =
      wide ? (a.fixed ? (ns ? fn(k_tree_plan_wide<true, true>) : fn(k_tree_plan_wide<true, false>))
                      : (ns ? fn(k_tree_plan_wide<false, true>) : fn(k_tree_plan_wide<false, false>)))
           : (a.fixed ? (ns ? fn(k_tree_plan<true, true>) : fn(k_tree_plan<true, false>))
                      : (ns ? fn(k_tree_plan<false, true>) : fn(k_tree_plan<false, false>)));
  const int64_t plan_groups = wide ? (static_cast<int64_t>(F) + kPlanThreads - 1) / kPlanThreads : 1;
  return launch_threads(plan, plan_groups, kPlanThreads, stream, a) &&
         launch(bf ? fn(k_tree_conf<DT_BF16>) : fn(k_tree_conf<DT_F32>), a.grid, stream, a, ev) &&
         launch(bf ? fn(k_tree_select<DT_BF16>) : fn(k_tree_select<DT_F32>), static_cast<int64_t>(a.B) * a.S, stream,
                a) &&
         launch(fn(k_tree_batch), a.B, stream, a) &&
         launch_threads(gum, items, kGumbelThreads, stream, a) &&
         launch(bf ? fn(k_tree_walk<DT_BF16>) : fn(k_tree_walk<DT_F32>), a.B, stream, a);
}

}  // namespace dbv
