// Prefix-conditional draft-tree construction (SPOT, Sec. 4.2 Eq. 3, Sec. 4.3
// Eq. 4 and App. C.2 Algorithm 2).
//
//   k_dd_plan   one group: lists the stale rows to read -- the masked
//               positions of every sequence -- and maps (b, s) to the list
//               (only for large B*L; otherwise every group of k_dd_rows lists
//               them itself in LDS and group 0 writes the map).
//   k_dd_rows   persistent: per listed row, partial reductions of its pieces
//               (FlatSplit, as the verification streams): the softmax
//               statistics at temperature 1 with the two largest logits
//               (T = 0), or with the argmax of z/T + G and the logit there
//               (T > 0, logit and Gumbel rows read together).
//   k_dd_hyp    per (sequence, position), one wave: merges the row's
//               partials into the token hypotheses H(s) and their stale
//               probabilities p^_s(v).
//   k_dd_tree   per sequence, in LDS: the level-batched top-D search.  A
//               level expands the states admitted by the previous one: q(s|y)
//               = softmax over M(y) of the order logits / tau, children
//               m(z) = m(y) q(s|y) p^_s(v), and the D best of the tree and the
//               new candidates are kept (radix selection on 64-bit keys).
//               One level per call with order rows supplied per frontier
//               state, or every level in one launch with the first-order
//               order table (row = last committed position, L for the root).
// The kernel boundaries are the only cross-group synchronisation.
#include "dbv_device.h"
#include "dbv_launch.h"

namespace dbv {

// Reduction of a wave's partial values with a commutative, associative
// merge: after the six DPP steps (partners always cover disjoint lanes) lane
// 63 holds the merge of all 64 lanes.  P provides
//   template <int C, int R> P moved() const   (the partner's value, or the
//                                             identity where a row is masked)
//   void merge(const P&)
template <class P>
__device__ __forceinline__ P wave_merge_dpp(P p) {
  p.merge(p.template moved<0xB1, 0xf>());
  p.merge(p.template moved<0x4E, 0xf>());
  p.merge(p.template moved<0x141, 0xf>());
  p.merge(p.template moved<0x140, 0xf>());
  p.merge(p.template moved<0x142, 0xa>());
  p.merge(p.template moved<0x143, 0xc>());
  return p;
}

// Wave maximum (NaN-propagating) and sum of one float by the same DPP steps;
// the result is read from lane 63 and returned to every lane.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxp(v, dpp_move<0xB1, 0xf>(-kInf, v));    // quad_perm 1,0,3,2
  v = fmaxp(v, dpp_move<0x4E, 0xf>(-kInf, v));    // quad_perm 2,3,0,1
  v = fmaxp(v, dpp_move<0x141, 0xf>(-kInf, v));   // row_half_mirror
  v = fmaxp(v, dpp_move<0x140, 0xf>(-kInf, v));   // row_mirror
  v = fmaxp(v, dpp_move<0x142, 0xa>(-kInf, v));   // row_bcast15 into rows 1, 3
  v = fmaxp(v, dpp_move<0x143, 0xc>(-kInf, v));   // row_bcast31 into rows 2, 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_move<0xB1, 0xf>(0.f, v);
  v += dpp_move<0x4E, 0xf>(0.f, v);
  v += dpp_move<0x141, 0xf>(0.f, v);
  v += dpp_move<0x140, 0xf>(0.f, v);
  v += dpp_move<0x142, 0xa>(0.f, v);
  v += dpp_move<0x143, 0xc>(0.f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// ------------------------------------------------------------ hypotheses ---

constexpr int kDDPlanThreads = 1024;
// Up to this many (sequence, position) flags, every group of the row stream
// lists the rows itself and no plan kernel runs.
constexpr int kDDFusedPlan = 8192;

__global__ __launch_bounds__(kDDPlanThreads) void k_dd_plan(DDHypArgs a) {
  __shared__ int s_w[kDDPlanThreads / 64];
  const int F = a.B * a.L;
  int base = 0;
  for (int f0 = 0; f0 < F; f0 += kDDPlanThreads) {
    const int f = f0 + static_cast<int>(threadIdx.x);
    const int need = (f < F && a.masked[f]) ? 1 : 0;
    int total;
    const int off = base + group_exclusive_scan<kDDPlanThreads / 64>(need, total, s_w);
    if (f < F) {
      a.map[f] = need ? off : -1;
      if (need) a.list[off] = f;
    }
    base += total;
  }
  if (threadIdx.x == 0) *a.count = base;
  if (a.status)
    for (int b = threadIdx.x; b < a.B; b += kDDPlanThreads) a.status[b] = 0;
}

// Two largest values with the softmax statistics at temperature 1, tracked
// per group of contiguous elements: per element one median-of-three (the new
// second value) and one max; per group only the start index of the group
// that holds each of the two values (the earlier group on equal values).
// The exact indices are found afterwards inside those groups (find_first).
// Each lane sees its groups in increasing index order.
struct Top2Stats {
  SoftmaxStats st{kLog2e};
  float v1 = -kInf, v2 = -kInf;
  int g1 = -1, g2 = -1;                 // start index of the group holding v1 / v2

  template <int N>
  __device__ __forceinline__ void track(const float* x, int idx0) {
    float n1 = v1, n2 = v2;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      n2 = __builtin_amdgcn_fmed3f(x[j], n1, n2);
      n1 = fmaxf(n1, x[j]);
    }
    if (n1 > v1) {
      g2 = (n2 == v1) ? g1 : idx0;      // the old first value, demoted, is earlier
      g1 = idx0;
    } else if (n2 > v2) {
      g2 = idx0;
    }
    v1 = n1;
    v2 = n2;
  }
  template <int N>
  __device__ __forceinline__ void group(const float* x, int64_t idx0) {
    st.absorb<N>(x);
    track<N>(x, static_cast<int>(idx0));
  }
  template <int U, int W>
  __device__ __forceinline__ void block(const float* x, int64_t idx0, int64_t ustride) {
    st.absorb<U * W>(x);
#pragma unroll
    for (int u = 0; u < U; ++u) track<W>(x + u * W, static_cast<int>(idx0 + u * ustride));
  }
};

// Top-2 of two top-2 lists (each ordered); index -1 = empty.
__device__ __forceinline__ void top2_merge(float& a1, int& b1, float& a2, int& b2, float c1, int d1, float c2,
                                           int d2) {
  if (pick_better(c1, d1, a1, b1)) {
    if (pick_better(c2, d2, a1, b1)) { a2 = c2; b2 = d2; } else { a2 = a1; b2 = b1; }
    a1 = c1; b1 = d1;
  } else if (pick_better(c1, d1, a2, b2)) {
    a2 = c1; b2 = d1;
  }
}

// Argmax of the scores z/T + g, tracked per group of four contiguous
// elements (the start index of the first group holding the best score), and
// the softmax statistics of z at temperature 1.  The exact index and the
// logit there are found afterwards inside that group (find_first).
struct GumbelHyp {
  SoftmaxStats st{kLog2e};
  float best = -kInf;
  int gbest = -1;
  bool nan = false;

  template <int UG>
  __device__ __forceinline__ void steps(const float (&x)[UG][4], const float (&sc)[UG][4], const int (&idx0)[UG]) {
    st.absorb<UG * 4>(&x[0][0]);
#pragma unroll
    for (int u = 0; u < UG; ++u) {
      const float m = fmaxp(fmaxp(sc[u][0], sc[u][1]), fmaxp(sc[u][2], sc[u][3]));
      nan |= (m != m);
      if (m > best) { best = m; gbest = idx0[u]; }
    }
  }
  __device__ __forceinline__ void one(float x, float sc, int idx) {
    st.absorb<1>(&x);
    nan |= (sc != sc);
    if (sc > best) { best = sc; gbest = idx; }
  }
};

// Row partials during the wave merge.  T = 0: statistics and the two largest
// values with the start index of the group holding each; T > 0: statistics
// and the best score with its group.  Exact indices are resolved per row by
// k_dd_hyp inside those groups.
struct Top2Part {
  float M, S, v1, v2;
  int g1, g2;
  template <int C, int R>
  __device__ __forceinline__ Top2Part moved() const {
    return Top2Part{dpp_move<C, R>(-kInf, M), dpp_move<C, R>(0.f, S), dpp_move<C, R>(-kInf, v1),
                    dpp_move<C, R>(-kInf, v2), dpp_move<C, R>(-1, g1), dpp_move<C, R>(-1, g2)};
  }
  __device__ __forceinline__ void merge(const Top2Part& o) {
    stats_merge(M, S, o.M, o.S, kLog2e);
    top2_merge(v1, g1, v2, g2, o.v1, o.g1, o.v2, o.g2);
  }
};

struct PickPart {
  float M, S, v;
  int g, nan;
  template <int C, int R>
  __device__ __forceinline__ PickPart moved() const {
    return PickPart{dpp_move<C, R>(-kInf, M), dpp_move<C, R>(0.f, S), dpp_move<C, R>(-kInf, v),
                    dpp_move<C, R>(-1, g), dpp_move<C, R>(0, nan)};
  }
  __device__ __forceinline__ void merge(const PickPart& o) {
    stats_merge(M, S, o.M, o.S, kLog2e);
    nan |= o.nan;
    if (pick_better(o.v, o.g, v, g)) { v = o.v; g = o.g; }
  }
};

// Four consecutive logits as floats from one 8-byte (bf16) or 16-byte
// (fp32) load.
template <int DT>
__device__ __forceinline__ void load_x4(const char* p, float (&x)[4]) {
  if (DT == DT_BF16) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xffff0000u);
  } else {
    const u32x4 w = load16(p);
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
}

// Streams a logit row and its Gumbel row over [v0, v1) into `op`.  A lane
// takes four consecutive elements per step: one 16-byte Gumbel load and one
// 8- or 16-byte logit load, so each wave instruction reads one contiguous
// span of either row.
template <int DT>
__device__ void stream_gumbel(const char* xr, const float* gr, int64_t v0, int64_t v1, float inv_t,
                              GumbelHyp& op) {
  using E = Elem<DT>;
  constexpr int XB = 4 * E::kBytes;   // logit bytes per step
  const int t = threadIdx.x;
  if (v1 <= v0) return;
  const uintptr_t ag = reinterpret_cast<uintptr_t>(gr + v0);
  int64_t head = static_cast<int64_t>(((16u - (ag & 15u)) & 15u) / 4);
  if (head > v1 - v0) head = v1 - v0;
  const int64_t a0 = v0 + head;
  const bool xal = (reinterpret_cast<uintptr_t>(xr + a0 * E::kBytes) & (XB - 1)) == 0;
  if (!xal) {  // logits not aligned with the Gumbel row: scalar path
    for (int64_t j = v0 + t; j < v1; j += kBlock) {
      const float x = E::load1(xr, j);
      op.one(x, __builtin_fmaf(x, inv_t, gr[j]), static_cast<int>(j));
    }
    return;
  }
  const int64_t nvec = (v1 - a0) / 4;
  const int64_t a1 = a0 + nvec * 4;
  if (t < head) {
    const float x = E::load1(xr, v0 + t);
    op.one(x, __builtin_fmaf(x, inv_t, gr[v0 + t]), static_cast<int>(v0 + t));
  }
  const char* xb = xr + a0 * E::kBytes;
  const char* gb = reinterpret_cast<const char*>(gr + a0);
  constexpr int UG = 4;      // steps per lane in flight
  int64_t i = t;
  for (; i + (UG - 1) * kBlock < nvec; i += UG * kBlock) {
    float x[UG][4];
    u32x4 g[UG];
#pragma unroll
    for (int u = 0; u < UG; ++u) {
      load_x4<DT>(xb + (i + u * kBlock) * XB, x[u]);
      g[u] = load16(gb + (i + u * kBlock) * 16);
    }
    float sc[UG][4];
    int id[UG];
#pragma unroll
    for (int u = 0; u < UG; ++u) {
      sc[u][0] = __builtin_fmaf(x[u][0], inv_t, __uint_as_float(g[u].x));
      sc[u][1] = __builtin_fmaf(x[u][1], inv_t, __uint_as_float(g[u].y));
      sc[u][2] = __builtin_fmaf(x[u][2], inv_t, __uint_as_float(g[u].z));
      sc[u][3] = __builtin_fmaf(x[u][3], inv_t, __uint_as_float(g[u].w));
      id[u] = static_cast<int>(a0 + (i + u * kBlock) * 4);
    }
    op.steps<UG>(x, sc, id);
  }
  for (; i < nvec; i += kBlock) {
    float x[1][4];
    load_x4<DT>(xb + i * XB, x[0]);
    const u32x4 g = load16(gb + i * 16);
    const float sc[1][4] = {{__builtin_fmaf(x[0][0], inv_t, __uint_as_float(g.x)),
                             __builtin_fmaf(x[0][1], inv_t, __uint_as_float(g.y)),
                             __builtin_fmaf(x[0][2], inv_t, __uint_as_float(g.z)),
                             __builtin_fmaf(x[0][3], inv_t, __uint_as_float(g.w))}};
    const int id[1] = {static_cast<int>(a0 + i * 4)};
    op.steps<1>(x, sc, id);
  }
  if (a1 + t < v1) {
    const float x = E::load1(xr, a1 + t);
    op.one(x, __builtin_fmaf(x, inv_t, gr[a1 + t]), static_cast<int>(a1 + t));
  }
}

// The first element of [g0, g0 + W) inside [lo, hi), other than `skip`,
// whose value (the logit, or its score z/T + G with a Gumbel row) equals
// `val`; -1 if none.  Every lane of the wave calls it.
template <int DT, bool GUM>
__device__ __forceinline__ int find_first(const char* row, const float* gr, float inv_t, int g0, int W, int64_t lo,
                                          int64_t hi, float val, int skip) {
  const int lane = threadIdx.x & 63;
  const int64_t j = static_cast<int64_t>(g0) + lane;
  bool hit = false;
  if (g0 >= 0 && lane < W && j >= lo && j < hi && j != skip) {
    const float x = Elem<DT>::load1(row, j);
    hit = (GUM ? __builtin_fmaf(x, inv_t, gr[j]) : x) == val;
  }
  const uint64_t bal = __ballot(hit);
  return bal ? g0 + static_cast<int>(__ffsll(static_cast<unsigned long long>(bal))) - 1 : -1;
}

// Rows of the stream listed by every group itself when B*L is small (no plan
// kernel): the masked flags in LDS with the count before each thread's chunk.
struct RowDir {
  uint8_t m[kDDFusedPlan];
  int pre[kBlock + 1];
  int w[kWaves];
};

// Builds the directory and returns the number of stream rows.  Group 0 also
// writes what the plan kernel would: map, count, and the cleared status.
__device__ int row_dir(const DDHypArgs& a, RowDir& d, bool writer) {
  const int t = threadIdx.x;
  const int F = a.B * a.L;
  const int C = (F + kBlock - 1) / kBlock;
  const int lo = t * C, hi = min(F, lo + C);
  int cnt = 0;
  for (int i = lo; i < hi; ++i) {
    const uint8_t v = a.masked[i] != 0;
    d.m[i] = v;
    cnt += v;
  }
  int total;
  const int off = group_exclusive_scan<kWaves>(cnt, total, d.w);
  d.pre[t] = off;
  if (t == 0) d.pre[kBlock] = total;
  if (writer) {
    int k = off;
    for (int i = lo; i < hi; ++i) {
      a.map[i] = d.m[i] ? k : -1;
      k += d.m[i];
    }
    if (t == 0) *a.count = total;
    if (a.status)
      for (int b = t; b < a.B; b += kBlock) a.status[b] = 0;
  }
  __syncthreads();
  return total;
}

// The flat id b*L + s of stream row r (the r-th masked flag).
__device__ __forceinline__ int row_flat(const DDHypArgs& a, const RowDir& d, int r) {
  const int F = a.B * a.L;
  const int C = (F + kBlock - 1) / kBlock;
  int lo = 0, hi = kBlock;                 // largest j with pre[j] <= r
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (d.pre[mid] <= r) lo = mid; else hi = mid;
  }
  int left = r - d.pre[lo];
  int i = lo * C;
  for (; i < F; ++i) {                     // the chunk holds row r
    if (d.m[i]) {
      if (left == 0) break;
      --left;
    }
  }
  return i;
}

template <int DT, bool GUM>
__global__ __launch_bounds__(kBlock) void k_dd_rows(DDHypArgs a) {
  __shared__ RowDir d;
  const int64_t g = blockIdx.x;
  const int R = a.fused_plan ? row_dir(a, d, g == 0) : *a.count;
  const FlatSplit f = make_split(R, a.V, a.split_bytes, a.grid);
  if (g >= f.G) return;
  for_pieces(f, g, [&](int64_t r, int64_t v0, int64_t v1, const Progress& pg) {
    const int flat = a.fused_plan ? row_flat(a, d, static_cast<int>(r)) : a.list[r];
    const int b = flat / a.L;
    const int s = flat - b * a.L;
    const char* rowp = static_cast<const char*>(a.stale) +
                       (b * a.ss + s * a.sp) * Elem<DT>::kBytes;
    DDPart out;
    if (GUM) {
      GumbelHyp op;
      stream_gumbel<DT>(rowp, a.gumbel + b * a.gs + s * a.gp, v0, v1, a.inv_t, op);
      const PickPart q = wave_merge_dpp(PickPart{op.st.M, op.st.S, op.best, op.gbest, op.nan ? 1 : 0});
      out = DDPart{q.M, q.S, q.v, q.g, -kInf, -1, 0.f, q.nan};
    } else {
      Top2Stats op;
      stream_row<DT, 4>(rowp, v0, v1, op, pg);
      const Top2Part q = wave_merge_dpp(Top2Part{op.st.M, op.st.S, op.v1, op.v2, op.g1, op.g2});
      out = DDPart{q.M, q.S, q.v1, q.g1, q.v2, q.g2, 0.f, 0};
    }
    if ((threadIdx.x & 63) == 63) a.part[(r + g) * kWaves + (threadIdx.x >> 6)] = out;
  });
}

// One wave per (sequence, position): merges the row's partials (statistics
// and the groups of the picks), finds the exact tokens inside those groups
// (find_first) and writes H(s) with p^_s of its tokens; the row's status bits
// go to status[b] (cleared by the plan kernel).
template <int DT, bool GUM>
__global__ __launch_bounds__(kBlock) void k_dd_hyp(DDHypArgs a) {
  const int lane = threadIdx.x & 63;
  const int flat = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (flat >= a.B * a.L) return;
  const int b = flat / a.L;
  const int s = flat - b * a.L;
  int32_t* ht = a.hyp_tok + static_cast<int64_t>(flat) * 2;
  float* hp = a.hyp_prob + static_cast<int64_t>(flat) * 2;
  const int r = a.map[flat];
  if (r < 0) {
    if (lane == 0) { ht[0] = -1; ht[1] = -1; hp[0] = 0.f; hp[1] = 0.f; }
    return;
  }
  const FlatSplit f = make_split(*a.count, a.V, a.split_bytes, a.grid);
  int64_t first, n;
  split_row_slots(f, r, first, n);
  const DDPart* p = a.part + first * kWaves;
  const int cnt = static_cast<int>(n * kWaves);
  const char* rowp = static_cast<const char*>(a.stale) + (b * a.ss + s * a.sp) * Elem<DT>::kBytes;
  const float* gr = GUM ? a.gumbel + b * a.gs + s * a.gp : nullptr;
  int rs = 0, t0 = -1, t1 = -1;
  float M, S, x0 = 0.f, x1 = 0.f;
  if (GUM) {
    PickPart q{-kInf, 0.f, -kInf, -1, 0};
    for (int j = lane; j < cnt; j += 64) {
      const DDPart d = p[j];
      q.merge(PickPart{d.M, d.S, d.v1, d.i1, d.nan});
    }
    q = wave_merge_dpp(q);
    M = __shfl(q.M, 63, 64); S = __shfl(q.S, 63, 64);
    const float v = __shfl(q.v, 63, 64);
    const int g = __shfl(q.g, 63, 64), nan = __shfl(q.nan, 63, 64);
    rs = stats_status(M, S);
    if (!rs) rs = nan ? SEQ_NONFINITE : max_status(v);
    t0 = find_first<DT, true>(rowp, gr, a.inv_t, g, 4, 0, a.V, v, -1);
    if (t0 >= 0) x0 = Elem<DT>::load1(rowp, t0);
  } else {
    Top2Part q{-kInf, 0.f, -kInf, -kInf, -1, -1};
    for (int j = lane; j < cnt; j += 64) {
      const DDPart d = p[j];
      q.merge(Top2Part{d.M, d.S, d.v1, d.v2, d.i1, d.i2});
    }
    q = wave_merge_dpp(q);
    M = __shfl(q.M, 63, 64); S = __shfl(q.S, 63, 64);
    const float v1 = __shfl(q.v1, 63, 64), v2 = __shfl(q.v2, 63, 64);
    const int g1 = __shfl(q.g1, 63, 64), g2 = __shfl(q.g2, 63, 64);
    rs = stats_status(M, S);
    constexpr int W = Elem<DT>::kVec;
    t0 = find_first<DT, false>(rowp, nullptr, 0.f, g1, W, 0, a.V, v1, -1);
    t1 = find_first<DT, false>(rowp, nullptr, 0.f, g2, W, 0, a.V, v2, t0);
    x0 = v1;
    x1 = v2;
  }
  if (lane == 0) {
    float p0 = 0.f, p1 = 0.f;
    if (!rs) {
      const float inv_s = 1.f / S;
      // p^(v) = exp(z_v - M) / S at temperature 1
      p0 = fast_exp2((x0 - M) * kLog2e) * inv_s;
      if (!GUM && p0 < a.below && t1 >= 0) {
        p1 = fast_exp2((x1 - M) * kLog2e) * inv_s;
      } else {
        t1 = -1;
      }
    } else {
      t0 = t1 = -1;
      if (a.status) atomicOr(a.status + b, rs);
    }
    ht[0] = t0; ht[1] = t1; hp[0] = fminf(p0, 1.f); hp[1] = fminf(p1, 1.f);
  }
}

// ---------------------------------------------------------------- search ---

constexpr int kDDNodes = kDDMaxBudget + 1;
constexpr int kDDThreads = 1024;
// Up to kRankMax contenders are ranked directly (threads count the larger
// keys); more are first cut to the D best by the radix selection.
constexpr int kRankMax = 1024;
static_assert(kRankMax >= kDDMaxBudget && kRankMax <= kDDThreads, "one contender per thread");
constexpr int kSeqBits = 25;

// Sort key of a state: mass (a non-negative float's bits order as integers),
// then the smaller depth, then the smaller creation number (frontier slot,
// position, hypothesis) within its level.  Keys are unique.
__device__ __forceinline__ uint64_t dd_key(float mass, int depth, int seq) {
  return (static_cast<uint64_t>(__float_as_uint(mass)) << 32) |
         (static_cast<uint64_t>(127 - depth) << kSeqBits) |
         static_cast<uint64_t>((1 << kSeqBits) - 1 - seq);
}
__device__ __forceinline__ float key_mass(uint64_t k) { return __uint_as_float(static_cast<uint32_t>(k >> 32)); }
__device__ __forceinline__ int key_depth(uint64_t k) { return 127 - static_cast<int>((k >> kSeqBits) & 127); }
__device__ __forceinline__ int key_seq(uint64_t k) {
  return (1 << kSeqBits) - 1 - static_cast<int>(k & ((1u << kSeqBits) - 1));
}

struct DDTreeLds {
  uint64_t key[kDDNodes], msk[kDDNodes];     // current tree in rank order (0 = root)
  float mass[kDDNodes];
  int par[kDDNodes], pos[kDDNodes], tok[kDDNodes];
  uint64_t nkey[kDDNodes], nmsk[kDDNodes];   // next tree
  float nmass[kDDNodes];
  int npar[kDDNodes], npos[kDDNodes], ntok[kDDNodes];
  int remap[kDDNodes];                       // old node -> new node or -1
  int fr[kDDMaxBudget];                      // frontier: nodes admitted last
  int htok[kDDMaxBlock][2];
  float hp[kDDMaxBlock][2];
  float otab[kDDMaxBlock + 1][kDDMaxBlock];  // the order table of the sequence (table mode)
  uint64_t ul[kDDMaxBudget];                 // the D best after a radix cut: keys
  int us[kDDMaxBudget];                      //   and their tree node (-1: a new candidate)
  uint64_t ck[kDDMaxCand];                   // candidates above the cut of the tree
  int hist[256];
  int n, nf, nc, nu, st, digit, above;
};

// The bin of the want-th largest key among the histogram (bins scanned from
// 255 down); sets s.digit and s.above (keys in higher bins).  One wave.
__device__ __forceinline__ void dd_pick_digit(DDTreeLds& s, int want) {
  const int t = threadIdx.x;
  if (t < 64) {
    int c[4];
    int loc = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = s.hist[255 - (t * 4 + q)];
      loc += c[q];
    }
    int inc = loc;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int o = __shfl_up(inc, m, 64);
      if (t >= m) inc += o;
    }
    int run = inc - loc;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (run < want && run + c[q] >= want) {
        s.digit = 255 - (t * 4 + q);
        s.above = run;
      }
      run += c[q];
    }
  }
  __syncthreads();
}

// Cut of the want-th largest key among tree nodes 1..n-1 and the candidates:
// exactly `want` keys are >= the returned value.
__device__ uint64_t dd_select(DDTreeLds& s, int want) {
  uint64_t prefix = 0, hmask = 0;
  const int t = threadIdx.x;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int j = t; j < 256; j += kDDThreads) s.hist[j] = 0;
    __syncthreads();
    for (int i = 1 + t; i < s.n; i += kDDThreads) {
      const uint64_t k = s.key[i];
      if ((k & hmask) == prefix) atomicAdd(&s.hist[(k >> shift) & 255], 1);
    }
    for (int i = t; i < s.nc; i += kDDThreads) {
      const uint64_t k = s.ck[i];
      if ((k & hmask) == prefix) atomicAdd(&s.hist[(k >> shift) & 255], 1);
    }
    __syncthreads();
    dd_pick_digit(s, want);
    const int d = s.digit;
    want -= s.above;
    const int inbin = s.hist[d];
    prefix |= static_cast<uint64_t>(d) << shift;
    hmask |= static_cast<uint64_t>(255) << shift;
    __syncthreads();
    if (inbin == want) break;   // the whole bin is kept
  }
  return prefix;
}

// Loads the root (first call) or the stored state of sequence b.
__device__ bool dd_load(const DDTreeArgs& a, DDTreeLds& s, int b, bool init) {
  const int t = threadIdx.x;
  const int NN = a.D + 1;
  const int64_t nb = static_cast<int64_t>(b) * NN;
  int bad = 0;                          // this thread's input errors
  if (t == 0) {
    s.st = a.status ? a.status[b] : 0;
    s.nc = 0;
    s.nu = 0;
  }
  if (init) {
    if (t < 64) {
      const bool m = t < a.L && a.masked[static_cast<int64_t>(b) * a.L + t] != 0;
      const uint64_t bits = __ballot(m);
      if (t == 0) {
        s.key[0] = dd_key(1.f, 0, 0);
        s.msk[0] = bits;
        s.mass[0] = 1.f;
        s.par[0] = -1; s.pos[0] = -1; s.tok[0] = -1;
        s.n = 1;
        s.fr[0] = 0;
        s.nf = a.D > 0 ? 1 : 0;
      }
    }
  } else {
    if (t == 0) {
      s.n = a.num_nodes[b];
      s.nf = a.num_frontier[b];
    }
    __syncthreads();
    const int n = s.n, nf = s.nf;
    if (n < 1 || n > NN || nf < 0 || nf > a.D) {
      if (t == 0) s.st |= SEQ_BAD_INPUT;
      __syncthreads();
      return false;
    }
    for (int z = t; z < n; z += kDDThreads) {
      s.key[z] = a.keys[nb + z];
      s.msk[z] = a.masks[nb + z];
      s.mass[z] = a.mass[nb + z];
      s.par[z] = a.parent[nb + z];
      s.pos[z] = a.edge_pos[nb + z];
      s.tok[z] = a.edge_tok[nb + z];
    }
    for (int j = t; j < nf; j += kDDThreads) {
      const int z = a.frontier[static_cast<int64_t>(b) * a.D + j];
      const bool ok = z >= 1 && z < n;
      s.fr[j] = ok ? z : 0;
      if (!ok) bad = SEQ_BAD_INPUT;
    }
  }
  if (a.table) {                        // the order table, once per search
    const float* tb = a.order + static_cast<int64_t>(b) * a.os;
    for (int i = t; i < (a.L + 1) * a.L; i += kDDThreads) {
      const int c = i / a.L, p = i - c * a.L;
      s.otab[c][p] = tb[static_cast<int64_t>(c) * a.orow + p];
    }
  }
  // hypotheses of the root's masked positions
  for (int i = t; i < a.L * 2; i += kDDThreads) {
    const int p = i >> 1, k = i & 1;
    const int64_t o = (static_cast<int64_t>(b) * a.L + p) * 2 + k;
    int tk = a.hyp_tok[o];
    const float pr = a.hyp_prob[o];
    const bool m = a.masked[static_cast<int64_t>(b) * a.L + p] != 0;
    if (!m) tk = -1;
    if (m && ((k == 0 && tk < 0) || (tk >= 0 && !(pr >= 0.f && pr <= 1.f)))) bad = SEQ_BAD_INPUT;
    s.htok[p][k] = tk;
    s.hp[p][k] = tk >= 0 ? pr : 0.f;
  }
  __syncthreads();                      // s.st holds the entry status
  // A sequence that enters in error keeps its status (its hypotheses are
  // absent); the only bit or-ed here is SEQ_BAD_INPUT, so the order of the
  // reads and the atomics does not matter.
  if (bad && !(s.st & SEQ_ERROR_MASK)) atomicOr(&s.st, bad);
  __syncthreads();
  return !(s.st & SEQ_ERROR_MASK);      // an error on entry or in the inputs
}

// Places contender i (key k, tree node src or -1 for a new candidate) at
// rank r of the next tree.
__device__ __forceinline__ void dd_place(DDTreeLds& s, uint64_t k, int src, int r) {
  const int z = r + 1;
  s.nkey[z] = k;
  if (src >= 0) {
    s.remap[src] = z;
    s.nmsk[z] = s.msk[src]; s.nmass[z] = s.mass[src];
    s.npos[z] = s.pos[src]; s.ntok[z] = s.tok[src]; s.npar[z] = s.par[src];
  } else {
    const int sq = key_seq(k);
    const int j = sq >> 7, p = (sq >> 1) & 63, hk = sq & 1;
    const int y = s.fr[j];
    s.nmsk[z] = s.msk[y] & ~(1ull << p);
    s.nmass[z] = key_mass(k);
    s.npos[z] = p;
    s.ntok[z] = s.htok[p][hk];
    s.npar[z] = y;                           // old index; remapped below
  }
}

// Ranks the contenders A[0..na) then B[0..nb) (keys are unique: rank =
// number of larger keys) and places the D best; P adjacent threads share a
// contender and count over every P-th key.  src(i) gives the tree node of
// contender i, or -1.
template <class Src>
__device__ __forceinline__ void dd_rank(const DDTreeArgs& a, DDTreeLds& s, const uint64_t* A, int na,
                                        const uint64_t* B, int nb, Src src) {
  const int t = threadIdx.x;
  const int nu = na + nb;
  int P = 1;
  while (P < 16 && P * 2 * nu <= kDDThreads) P *= 2;
  const int item = t / P, part = t - item * P;
  int r = 0;
  uint64_t k = 0;
  if (item < nu) {
    k = item < na ? A[item] : B[item - na];
    for (int pass = 0; pass < 2; ++pass) {
      const uint64_t* X = pass ? B : A;
      const int nx = pass ? nb : na;
      int j = part;
      for (; j + 7 * P < nx; j += 8 * P) {   // eight LDS reads in flight
        uint64_t c[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) c[e] = X[j + e * P];
#pragma unroll
        for (int e = 0; e < 8; ++e) r += c[e] > k;
      }
      for (; j < nx; j += P) r += X[j] > k;
    }
  }
  // sum over the P lanes of a contender (P <= 16: within one DPP row)
  if (P >= 2) r += dpp_move<0xB1, 0xf>(0, r);     // quad_perm 1,0,3,2
  if (P >= 4) r += dpp_move<0x4E, 0xf>(0, r);     // quad_perm 2,3,0,1
  if (P >= 8) r += dpp_move<0x141, 0xf>(0, r);    // row_half_mirror
  if (P >= 16) r += dpp_move<0x140, 0xf>(0, r);   // row_mirror
  if (item < nu && part == 0 && r < a.D) dd_place(s, k, src(item), r);
}

// One level: expands the frontier, keeps the D best, sets the new frontier.
// Entry: s.nc == s.nu == 0.  Three barriers when at most kRankMax states
// contend.
__device__ void dd_level(const DDTreeArgs& a, DDTreeLds& s, int b) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int L = a.L;
  const int n = s.n;
  const int nf = s.nf;
  const uint64_t theta = (n - 1 == a.D) ? s.key[a.D] : 0;
  const int depth = key_depth(s.key[s.fr[0]]) + 1;
  for (int i = t; i < n; i += kDDThreads) s.remap[i] = i == 0 ? 0 : -1;
  for (int j = w; j < nf; j += kDDThreads / 64) {
    const int y = s.fr[j];
    const uint64_t my = s.msk[y];
    const bool in = lane < L && ((my >> lane) & 1);
    float zr = 0.f;
    if (in) {
      if (a.table) {
        zr = s.otab[y == 0 ? L : s.pos[y]][lane];
      } else {
        zr = a.order[static_cast<int64_t>(b) * a.os + static_cast<int64_t>(j) * a.orow + lane];
      }
    }
    const float z = in ? zr * a.inv_tau : -kInf;
    if (my == 0) continue;                   // a terminal state: no children
    const float mx = wave_max_dpp(z);
    if (mx != mx || mx == kInf || mx == -kInf) {
      if (lane == 0) atomicOr(&s.st, mx == -kInf ? SEQ_EMPTY_ROW : SEQ_NONFINITE);
      continue;
    }
    const float e = in ? fast_exp2((z - mx) * kLog2e) : 0.f;
    const float q = e / wave_sum_dpp(e);
    const float my_mass = s.mass[y];
    uint64_t key[2];
    bool keep[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int tk = in ? s.htok[lane][k] : -1;
      const float m = fminf(my_mass * q * s.hp[in ? lane : 0][k], my_mass);
      key[k] = dd_key(m, depth, j * 128 + lane * 2 + k);
      keep[k] = tk >= 0 && m >= a.gamma && key[k] > theta;
    }
    const uint64_t b0 = __ballot(keep[0]), b1 = __ballot(keep[1]);
    const int c0 = __popcll(b0);
    if (c0 + __popcll(b1) == 0) continue;
    int base = 0;
    if (lane == 0) base = atomicAdd(&s.nc, c0 + __popcll(b1));   // one LDS atomic per row
    base = __builtin_amdgcn_readfirstlane(base);
    const uint64_t below = (1ull << lane) - 1;
    if (keep[0]) s.ck[base + __popcll(b0 & below)] = key[0];
    if (keep[1]) s.ck[base + c0 + __popcll(b1 & below)] = key[1];
  }
  __syncthreads();
  if (s.st & SEQ_ERROR_MASK) return;
  const int nc = s.nc;
  const int U = (n - 1) + nc;
  if (U <= kRankMax) {
    // every contender: tree nodes 1..n-1, then the candidates
    dd_rank(a, s, s.key + 1, n - 1, s.ck, nc, [&](int i) { return i < n - 1 ? i + 1 : -1; });
  } else {
    // more contenders than ranked directly: cut to the D best first
    const uint64_t cut = dd_select(s, a.D);
    for (int i0 = w * 64; i0 < U; i0 += kDDThreads) {
      const int i = i0 + lane;
      uint64_t k = 0;
      int src = -1;
      if (i < n - 1) {
        k = s.key[i + 1];
        src = i + 1;
      } else if (i < U) {
        k = s.ck[i - (n - 1)];
      }
      const bool keep = i < U && k >= cut;
      const uint64_t bal = __ballot(keep);
      if (bal == 0) continue;
      int base = 0;
      if (lane == 0) base = atomicAdd(&s.nu, __popcll(bal));
      base = __builtin_amdgcn_readfirstlane(base);
      const int slot = base + __popcll(bal & ((1ull << lane) - 1));
      if (keep && slot < kDDMaxBudget) {     // exactly D keys reach the cut
        s.ul[slot] = k;
        s.us[slot] = src;
      }
    }
    __syncthreads();
    dd_rank(a, s, s.ul, min(s.nu, a.D), nullptr, 0, [&](int i) { return s.us[i]; });
  }
  __syncthreads();
  // the next tree: parents remapped, copied back, the new frontier (the
  // admitted candidates in rank order), counters reset for the next level
  const int n2 = 1 + min(U, a.D);
  for (int z = 1 + t; z < n2; z += kDDThreads) {
    s.par[z] = s.remap[s.npar[z]];
    s.key[z] = s.nkey[z]; s.msk[z] = s.nmsk[z]; s.mass[z] = s.nmass[z];
    s.pos[z] = s.npos[z]; s.tok[z] = s.ntok[z];
  }
  if (t < 64) {
    const int z = t + 1;
    const bool nw = z < n2 && key_depth(s.nkey[z]) == depth;
    const uint64_t bal = __ballot(nw);
    if (nw) s.fr[__popcll(bal & ((1ull << t) - 1))] = z;
    if (t == 0) {
      s.nf = __popcll(bal);
      s.n = n2;
      s.nc = 0;
      s.nu = 0;
    }
  }
  __syncthreads();
}

__device__ void dd_store(const DDTreeArgs& a, DDTreeLds& s, int b) {
  const int t = threadIdx.x;
  const int NN = a.D + 1;
  const int64_t nb = static_cast<int64_t>(b) * NN;
  const int n = s.n, nf = s.nf;
  for (int z = t; z < NN; z += kDDThreads) {
    const bool in = z < n;
    a.parent[nb + z] = in ? s.par[z] : -1;
    a.edge_pos[nb + z] = in ? s.pos[z] : -1;
    a.edge_tok[nb + z] = in ? s.tok[z] : -1;
    a.mass[nb + z] = in ? s.mass[z] : 0.f;
    if (in) {
      a.keys[nb + z] = s.key[z];
      a.masks[nb + z] = s.msk[z];
    }
  }
  if (a.node_masked) {
    for (int i = t; i < NN * a.L; i += kDDThreads) {
      const int z = i / a.L, p = i - z * a.L;
      a.node_masked[nb * a.L + i] = (z < n && ((s.msk[z] >> p) & 1)) ? 1 : 0;
    }
  }
  for (int j = t; j < a.D; j += kDDThreads)
    a.frontier[static_cast<int64_t>(b) * a.D + j] = j < nf ? s.fr[j] : -1;
  if (t == 0) {
    a.num_nodes[b] = n;
    a.num_frontier[b] = nf;
    if (a.status) a.status[b] = s.st;
  }
}

__global__ __launch_bounds__(kDDThreads) void k_dd_tree(DDTreeArgs a) {
  __shared__ DDTreeLds s;
  const int b = blockIdx.x;
  const bool init = a.table || a.first;
  if (!dd_load(a, s, b, init)) {
    // an error found before the search: a fresh tree is the root alone
    if (init) {
      if (threadIdx.x == 0) {
        s.n = 1; s.nf = 0;
        s.key[0] = dd_key(1.f, 0, 0); s.msk[0] = 0; s.mass[0] = 1.f;
        s.par[0] = -1; s.pos[0] = -1; s.tok[0] = -1;
      }
      __syncthreads();
      dd_store(a, s, b);
    } else if (threadIdx.x == 0 && a.status) {
      a.status[b] = s.st;
    }
    return;
  }
  if (a.table) {
    for (int level = 0; level <= kDDMaxBudget && s.nf > 0 && !(s.st & SEQ_ERROR_MASK); ++level) dd_level(a, s, b);
  } else if (s.nf > 0) {
    dd_level(a, s, b);
  }
  if (threadIdx.x == 0 && (s.st & SEQ_ERROR_MASK)) s.nf = 0;
  __syncthreads();
  dd_store(a, s, b);
}

template <typename K>
static const void* fn(K* k) {
  return reinterpret_cast<const void*>(k);
}

bool launch_dd_hypotheses(const DDHypArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev) {
  const bool bf = dtype == DT_BF16;
  const bool gum = a.inv_t > 0.f;
  const void* rows = gum ? (bf ? fn(k_dd_rows<DT_BF16, true>) : fn(k_dd_rows<DT_F32, true>))
                         : (bf ? fn(k_dd_rows<DT_BF16, false>) : fn(k_dd_rows<DT_F32, false>));
  DDHypArgs b = a;
  b.fused_plan = static_cast<int64_t>(a.B) * a.L <= kDDFusedPlan ? 1 : 0;
  return (b.fused_plan || launch_threads(fn(k_dd_plan), 1, kDDPlanThreads, stream, b)) &&
         launch(rows, b.grid, stream, b, ev) &&
         launch(gum ? (bf ? fn(k_dd_hyp<DT_BF16, true>) : fn(k_dd_hyp<DT_F32, true>))
                    : (bf ? fn(k_dd_hyp<DT_BF16, false>) : fn(k_dd_hyp<DT_F32, false>)),
                cdiv(static_cast<int64_t>(a.B) * a.L, kWaves), stream, b);
}

bool launch_dd_tree(const DDTreeArgs& a, hipStream_t stream, const TimingEvents& ev) {
  return launch_threads(fn(k_dd_tree), a.B, kDDThreads, stream, a, ev);
}

}  // namespace dbv
