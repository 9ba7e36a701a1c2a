// Prefix-conditional draft-tree construction (SPOT, Sec. 4.2 Eq. 3, Sec. 4.3
// Eq. 4 and App. C.2 Algorithm 2).
//
//   k_dd_plan   one group: lists the stale rows to read -- the masked
//               positions of every sequence -- and maps (b, s) to the list.
//   k_dd_rows   persistent: per listed row, partial reductions of its pieces
//               (FlatSplit, as the verification streams): the softmax
//               statistics at temperature 1 with the two largest logits
//               (T = 0), or with the argmax of z/T + G and the logit there
//               (T > 0, logit and Gumbel rows read together).
//   k_dd_hyp    per sequence: merges each row's partials into the token
//               hypotheses H(s) and their stale probabilities p^_s(v).
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

// ------------------------------------------------------------ hypotheses ---

constexpr int kDDPlanThreads = 1024;

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
}

// Two largest values (value descending, index ascending) with the softmax
// statistics at temperature 1.  Each lane sees its indices in increasing
// order, so a later equal value never displaces an earlier one.
struct Top2Stats {
  SoftmaxStats st{kLog2e};
  float v1 = -kInf, v2 = -kInf;
  int64_t i1 = -1, i2 = -1;

  __device__ __forceinline__ void take(float y, int64_t i) {
    if (y > v1) {
      v2 = v1; i2 = i1;
      v1 = y; i1 = i;
    } else if (y > v2) {
      v2 = y; i2 = i;
    }
  }
  template <int N>
  __device__ __forceinline__ void group(const float* x, int64_t idx0) {
    st.absorb<N>(x);
    float m = x[0];
#pragma unroll
    for (int j = 1; j < N; ++j) m = fmaxp(m, x[j]);
    if (m > v2) {
#pragma unroll
      for (int j = 0; j < N; ++j) take(x[j], idx0 + j);
    }
  }
  template <int U, int W>
  __device__ __forceinline__ void block(const float* x, int64_t idx0, int64_t ustride) {
    st.absorb<U * W>(x);
    float m = x[0];
#pragma unroll
    for (int j = 1; j < U * W; ++j) m = fmaxp(m, x[j]);
    if (m > v2) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < W; ++j) take(x[u * W + j], idx0 + u * ustride + j);
    }
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

// Argmax of z/T + g (lowest index), the logit z there, and the softmax
// statistics of z at temperature 1.
struct GumbelHyp {
  SoftmaxStats st{kLog2e};
  float best = -kInf, bx = 0.f;
  int64_t bidx = -1;
  bool nan = false;

  template <int N>
  __device__ __forceinline__ void pair(const float* x, const float* sc, int64_t idx0) {
    st.absorb<N>(x);
    float m = sc[0];
#pragma unroll
    for (int j = 1; j < N; ++j) m = fmaxp(m, sc[j]);
    nan |= (m != m);
    if (m > best || (bidx < 0 && m == best)) {
      int j0 = 0;
#pragma unroll
      for (int j = N - 1; j >= 0; --j)
        if (sc[j] == m) j0 = j;
      best = m;
      bidx = idx0 + j0;
      bx = x[j0];
    }
  }
};

// Streams a logit row and its Gumbel row over [v0, v1) into `op`.
template <int DT>
__device__ void stream_gumbel(const char* xr, const float* gr, int64_t v0, int64_t v1, float inv_t,
                              GumbelHyp& op) {
  using E = Elem<DT>;
  constexpr int W = E::kVec;
  const int t = threadIdx.x;
  if (v1 <= v0) return;
  const uintptr_t ax = reinterpret_cast<uintptr_t>(xr + v0 * E::kBytes);
  int64_t head = static_cast<int64_t>(((16u - (ax & 15u)) & 15u) / E::kBytes);
  if (head > v1 - v0) head = v1 - v0;
  const int64_t a0 = v0 + head;
  const bool gal = ((reinterpret_cast<uintptr_t>(gr + a0)) & 15u) == 0;
  if (!gal) {  // Gumbel row not aligned with the logits: scalar path
    for (int64_t j = v0 + t; j < v1; j += kBlock) {
      float x[1] = {E::load1(xr, j)};
      float s[1] = {__builtin_fmaf(x[0], inv_t, gr[j])};
      op.pair<1>(x, s, j);
    }
    return;
  }
  const int64_t nvec = (v1 - a0) / W;
  const int64_t a1 = a0 + nvec * W;
  if (t < head) {
    float x[1] = {E::load1(xr, v0 + t)};
    float s[1] = {__builtin_fmaf(x[0], inv_t, gr[v0 + t])};
    op.pair<1>(x, s, v0 + t);
  }
  const char* xb = xr + a0 * E::kBytes;
  const char* gb = reinterpret_cast<const char*>(gr + a0);
  constexpr int GV = W / 4;  // 16-byte Gumbel loads per logit vector
  int64_t i = t;
  for (; i + kBlock < nvec; i += 2 * kBlock) {
    u32x4 xr0 = load16(xb + i * 16), xr1 = load16(xb + (i + kBlock) * 16);
    u32x4 g0[GV], g1[GV];
#pragma unroll
    for (int q = 0; q < GV; ++q) {
      g0[q] = load16(gb + (i * W + q * 4) * 4);
      g1[q] = load16(gb + ((i + kBlock) * W + q * 4) * 4);
    }
    float x0[W], x1[W], s0[W], s1[W];
    E::unpack(xr0, x0);
    E::unpack(xr1, x1);
#pragma unroll
    for (int j = 0; j < W; ++j) {
      s0[j] = __builtin_fmaf(x0[j], inv_t, __uint_as_float(g0[j / 4][j % 4]));
      s1[j] = __builtin_fmaf(x1[j], inv_t, __uint_as_float(g1[j / 4][j % 4]));
    }
    op.pair<W>(x0, s0, a0 + i * W);
    op.pair<W>(x1, s1, a0 + (i + kBlock) * W);
  }
  for (; i < nvec; i += kBlock) {
    u32x4 xv = load16(xb + i * 16);
    u32x4 g[GV];
#pragma unroll
    for (int q = 0; q < GV; ++q) g[q] = load16(gb + (i * W + q * 4) * 4);
    float x[W], s[W];
    E::unpack(xv, x);
#pragma unroll
    for (int j = 0; j < W; ++j) s[j] = __builtin_fmaf(x[j], inv_t, __uint_as_float(g[j / 4][j % 4]));
    op.pair<W>(x, s, a0 + i * W);
  }
  if (a1 + t < v1) {
    float x[1] = {E::load1(xr, a1 + t)};
    float s[1] = {__builtin_fmaf(x[0], inv_t, gr[a1 + t])};
    op.pair<1>(x, s, a1 + t);
  }
}

template <int DT, bool GUM>
__global__ __launch_bounds__(kBlock) void k_dd_rows(DDHypArgs a) {
  const FlatSplit f = make_split(*a.count, a.V, a.split_bytes, a.grid);
  const int64_t g = blockIdx.x;
  if (g >= f.G) return;
  for_pieces(f, g, [&](int64_t r, int64_t v0, int64_t v1) {
    const int flat = a.list[r];
    const int b = flat / a.L;
    const int s = flat - b * a.L;
    const char* rowp = static_cast<const char*>(a.stale) +
                       (b * a.ss + s * a.sp) * Elem<DT>::kBytes;
    DDPart out;
    if (GUM) {
      GumbelHyp op;
      stream_gumbel<DT>(rowp, a.gumbel + b * a.gs + s * a.gp, v0, v1, a.inv_t, op);
      float M = op.st.M, S = op.st.S, v = op.best, x = op.bx;
      int idx = static_cast<int>(op.bidx), nan = op.nan ? 1 : 0;
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        stats_merge(M, S, wave_shfl_xor(M, m), wave_shfl_xor(S, m), kLog2e);
        const float v2 = wave_shfl_xor(v, m), x2 = wave_shfl_xor(x, m);
        const int i2 = wave_shfl_xor(idx, m);
        nan |= wave_shfl_xor(nan, m);
        if (pick_better(v2, i2, v, idx)) { v = v2; idx = i2; x = x2; }
      }
      out = DDPart{M, S, v, idx, -kInf, -1, x, nan};
    } else {
      Top2Stats op;
      stream_row<DT, 4>(rowp, v0, v1, op);
      float M = op.st.M, S = op.st.S, a1 = op.v1, a2 = op.v2;
      int b1 = static_cast<int>(op.i1), b2 = static_cast<int>(op.i2);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        stats_merge(M, S, wave_shfl_xor(M, m), wave_shfl_xor(S, m), kLog2e);
        const float c1 = wave_shfl_xor(a1, m), c2 = wave_shfl_xor(a2, m);
        const int d1 = wave_shfl_xor(b1, m), d2 = wave_shfl_xor(b2, m);
        top2_merge(a1, b1, a2, b2, c1, d1, c2, d2);
      }
      out = DDPart{M, S, a1, b1, a2, b2, 0.f, 0};
    }
    if ((threadIdx.x & 63) == 0) a.part[(r + g) * kWaves + (threadIdx.x >> 6)] = out;
  });
}

// One group per sequence; wave w merges rows s = w, w + 4, ...
template <bool GUM>
__global__ __launch_bounds__(kBlock) void k_dd_hyp(DDHypArgs a) {
  __shared__ int s_st;
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  if (threadIdx.x == 0) s_st = 0;
  __syncthreads();
  const FlatSplit f = make_split(*a.count, a.V, a.split_bytes, a.grid);
  int st = 0;
  for (int s = w; s < a.L; s += kWaves) {
    const int flat = b * a.L + s;
    int32_t* ht = a.hyp_tok + static_cast<int64_t>(flat) * 2;
    float* hp = a.hyp_prob + static_cast<int64_t>(flat) * 2;
    const int r = a.map[flat];
    if (r < 0) {
      if (lane == 0) { ht[0] = -1; ht[1] = -1; hp[0] = 0.f; hp[1] = 0.f; }
      continue;
    }
    int64_t first, n;
    split_row_slots(f, r, first, n);
    const DDPart* p = a.part + first * kWaves;
    const int64_t cnt = n * kWaves;
    float M = -kInf, S = 0.f, v1 = -kInf, v2 = -kInf, x = 0.f;
    int i1 = -1, i2 = -1, nan = 0;
    for (int64_t j = lane; j < cnt; j += 64) {
      const DDPart q = p[j];
      stats_merge(M, S, q.M, q.S, kLog2e);
      if (GUM) {
        nan |= q.nan;
        if (pick_better(q.v1, q.i1, v1, i1)) { v1 = q.v1; i1 = q.i1; x = q.x; }
      } else {
        top2_merge(v1, i1, v2, i2, q.v1, q.i1, q.v2, q.i2);
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      stats_merge(M, S, wave_shfl_xor(M, m), wave_shfl_xor(S, m), kLog2e);
      const float c1 = wave_shfl_xor(v1, m), c2 = wave_shfl_xor(v2, m), x2 = wave_shfl_xor(x, m);
      const int d1 = wave_shfl_xor(i1, m), d2 = wave_shfl_xor(i2, m);
      nan |= wave_shfl_xor(nan, m);
      if (GUM) {
        if (pick_better(c1, d1, v1, i1)) { v1 = c1; i1 = d1; x = x2; }
      } else {
        top2_merge(v1, i1, v2, i2, c1, d1, c2, d2);
      }
    }
    if (lane == 0) {
      int rs = stats_status(M, S);
      if (GUM && !rs) rs = nan ? SEQ_NONFINITE : max_status(v1);
      st |= rs;
      int t0 = -1, t1 = -1;
      float p0 = 0.f, p1 = 0.f;
      if (!rs) {
        const float inv_s = 1.f / S;
        t0 = i1;
        // p^(v) = exp(z_v - M) / S at temperature 1
        p0 = (GUM ? fast_exp2((x - M) * kLog2e) : 1.f) * inv_s;
        if (!GUM && p0 < a.below && i2 >= 0) {
          t1 = i2;
          p1 = fast_exp2((v2 - M) * kLog2e) * inv_s;
        }
      }
      ht[0] = t0; ht[1] = t1; hp[0] = fminf(p0, 1.f); hp[1] = fminf(p1, 1.f);
    }
  }
  if (st) atomicOr(&s_st, st);
  __syncthreads();
  if (threadIdx.x == 0 && a.status) a.status[b] = s_st;
}

// ---------------------------------------------------------------- search ---

constexpr int kDDNodes = kDDMaxBudget + 1;
constexpr int kDDThreads = 256;
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
  uint64_t kc[kDDMaxBudget];                 // kept candidates
  uint64_t ck[kDDMaxCand];                   // candidates above the cut of the tree
  int hist[256];
  int n, nf, nc, nkc, st, digit, above, nkt;
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
  if (t == 0) s.st = a.status ? a.status[b] : 0;
  __syncthreads();
  if (s.st & SEQ_ERROR_MASK) return false;
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
      s.fr[j] = (z >= 1 && z < n) ? z : 0;
      if (!(z >= 1 && z < n)) atomicOr(&s.st, SEQ_BAD_INPUT);
    }
  }
  // hypotheses of the root's masked positions
  for (int i = t; i < a.L * 2; i += kDDThreads) {
    const int p = i >> 1, k = i & 1;
    const int64_t o = (static_cast<int64_t>(b) * a.L + p) * 2 + k;
    int tk = a.hyp_tok[o];
    float pr = a.hyp_prob[o];
    const bool m = a.masked[static_cast<int64_t>(b) * a.L + p] != 0;
    if (!m) tk = -1;
    if (m && ((k == 0 && tk < 0) || (tk >= 0 && !(pr >= 0.f && pr <= 1.f)))) atomicOr(&s.st, SEQ_BAD_INPUT);
    s.htok[p][k] = tk;
    s.hp[p][k] = tk >= 0 ? pr : 0.f;
  }
  __syncthreads();
  return !(s.st & SEQ_ERROR_MASK);
}

// One level: expands the frontier, keeps the D best, sets the new frontier.
__device__ void dd_level(const DDTreeArgs& a, DDTreeLds& s, int b) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int L = a.L;
  if (t == 0) s.nc = 0;
  __syncthreads();
  const int n = s.n;
  const int nf = s.nf;
  const uint64_t theta = (n - 1 == a.D) ? s.key[a.D] : 0;
  const int depth = key_depth(s.key[s.fr[0]]) + 1;
  for (int j = w; j < nf; j += kDDThreads / 64) {
    const int y = s.fr[j];
    const uint64_t my = s.msk[y];
    const bool in = lane < L && ((my >> lane) & 1);
    const float* row = a.order + static_cast<int64_t>(b) * a.os +
                       static_cast<int64_t>(a.table ? (y == 0 ? L : s.pos[y]) : j) * a.orow;
    const float z = in ? row[lane] * a.inv_tau : -kInf;
    float mx = z;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxp(mx, wave_shfl_xor(mx, m));
    if (my == 0) continue;                   // a terminal state: no children
    if (mx != mx || mx == kInf || mx == -kInf) {
      if (lane == 0) atomicOr(&s.st, mx == -kInf ? SEQ_EMPTY_ROW : SEQ_NONFINITE);
      continue;
    }
    const float e = in ? fast_exp2((z - mx) * kLog2e) : 0.f;
    float sum = e;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sum += wave_shfl_xor(sum, m);
    const float q = e / sum;
    const float my_mass = s.mass[y];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int tk = in ? s.htok[lane][k] : -1;
      const float m = fminf(my_mass * q * s.hp[in ? lane : 0][k], my_mass);
      const bool ok = tk >= 0 && m >= a.gamma;
      const uint64_t key = dd_key(m, depth, j * 128 + lane * 2 + k);
      const bool keep = ok && key > theta;
      const uint64_t bal = __ballot(keep);
      if (bal == 0) continue;
      int base = 0;
      if (lane == 0) base = atomicAdd(&s.nc, __popcll(bal));
      base = __shfl(base, 0, 64);
      if (keep) s.ck[base + __popcll(bal & ((1ull << lane) - 1))] = key;
    }
  }
  __syncthreads();
  if (s.st & SEQ_ERROR_MASK) return;
  const int nc = s.nc;
  const int U = (n - 1) + nc;
  const uint64_t cut = U <= a.D ? 0 : dd_select(s, a.D);
  // kept tree prefix and kept candidates
  if (t == 0) { s.nkc = 0; s.nkt = 0; }
  __syncthreads();
  for (int i = 1 + t; i < n; i += kDDThreads)
    if (s.key[i] >= cut) atomicAdd(&s.nkt, 1);
  for (int i = t; i < nc; i += kDDThreads) {
    const uint64_t k = s.ck[i];
    if (k >= cut) {
      const int slot = atomicAdd(&s.nkc, 1);
      if (slot < kDDMaxBudget) s.kc[slot] = k;   // at most D keys reach the cut
    }
  }
  __syncthreads();
  // (keys are unique, so exactly min(U, D) keys are kept; the bounds below
  // only guard the LDS arrays)
  const int nkt = s.nkt;
  const int nkc = min(s.nkc, a.D - nkt);
  // ranks: the tree prefix keeps its order; candidates interleave by key
  for (int i = t; i < n; i += kDDThreads) {
    int r = -1;
    if (i == 0) {
      r = 0;
    } else if (i <= nkt) {
      const uint64_t k = s.key[i];
      int above = 0;
      for (int c = 0; c < nkc; ++c) above += s.kc[c] > k;
      r = i + above;
    }
    s.remap[i] = r;
    if (r >= 0) {
      s.nkey[r] = s.key[i]; s.nmsk[r] = s.msk[i]; s.nmass[r] = s.mass[i];
      s.npos[r] = s.pos[i]; s.ntok[r] = s.tok[i]; s.npar[r] = s.par[i];
    }
  }
  for (int c = t; c < nkc; c += kDDThreads) {
    const uint64_t k = s.kc[c];
    int above = 0;
    for (int i = 1; i <= nkt; ++i) above += s.key[i] > k;
    for (int e = 0; e < nkc; ++e) above += s.kc[e] > k;
    const int r = 1 + above;
    const int sq = key_seq(k);
    const int j = sq >> 7, p = (sq >> 1) & 63, hk = sq & 1;
    const int y = s.fr[j];
    s.nkey[r] = k;
    s.nmsk[r] = s.msk[y] & ~(1ull << p);
    s.nmass[r] = key_mass(k);
    s.npos[r] = p;
    s.ntok[r] = s.htok[p][hk];
    s.npar[r] = y;                         // old index; remapped below
  }
  __syncthreads();
  const int n2 = 1 + nkt + nkc;
  for (int z = 1 + t; z < n2; z += kDDThreads) s.npar[z] = s.remap[s.npar[z]];
  if (t == 0) s.npar[0] = -1;
  __syncthreads();
  // new frontier: the admitted candidates in rank order (depth = this level)
  if (t < 64) {
    const int z = t + 1;
    const bool nw = z < n2 && key_depth(s.nkey[z]) == depth;
    const uint64_t bal = __ballot(nw);
    if (nw) s.fr[__popcll(bal & ((1ull << t) - 1))] = z;
    if (t == 0) s.nf = __popcll(bal);
  }
  for (int z = t; z < n2; z += kDDThreads) {
    s.key[z] = s.nkey[z]; s.msk[z] = s.nmsk[z]; s.mass[z] = s.nmass[z];
    s.pos[z] = s.npos[z]; s.tok[z] = s.ntok[z]; s.par[z] = s.npar[z];
  }
  if (t == 0) s.n = n2;
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
  return launch_threads(fn(k_dd_plan), 1, kDDPlanThreads, stream, a) &&
         launch(rows, a.grid, stream, a, ev) &&
         launch(gum ? fn(k_dd_hyp<true>) : fn(k_dd_hyp<false>), a.B, stream, a);
}

bool launch_dd_tree(const DDTreeArgs& a, hipStream_t stream) {
  return launch_threads(fn(k_dd_tree), a.B, kDDThreads, stream, a);
}

}  // namespace dbv
