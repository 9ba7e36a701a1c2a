// Chain verification kernels: greedy match with next-draft retention, and the
// rejection / linear-lenient sampler with its correction or bonus draw.
//
// Greedy  (Packed-SS, Sec. 3.1, Eq. 1-4, Algorithm 1):
//   k_greedy_rows      persistent: argmax partials of every needed target /
//                      drafter row; the needed rows form one stream split
//                      evenly over the groups (FlatSplit)
//   k_greedy_finalize  per sequence: combine, leading matches h, C, ending
//                      condition a, next draft z_{a+1..W}
// Sampling (Packed-SS, Algorithm 2; Two Tradeoffs, Theorem 1, Algorithm 1):
//   k_sample_rows      persistent: online softmax statistics (M, S) partials
//                      of every needed row, split like k_greedy_rows
//   k_draw_mass        per (sequence, chunk of draw tiles): the sequence's
//                      decision (p(d), q(d), the acceptance tests, h) and the
//                      masses of [p - q]_+ (or of p for the bonus) over the
//                      chunk's tiles of row h
//   k_draw_select      per sequence (256 or 1024 threads): the tile, then the token,
//                      where the running mass first exceeds u*Z (vocabulary
//                      order), and output assembly.
//   k_draw_fused       per sequence (256 threads), rows of a few tiles: the
//                      decision, the tile masses and the select in one group
// The kernel boundaries are the only cross-group synchronisation.
#include "dbv_device.h"
#include "dbv_launch.h"

#include <climits>

namespace dbv {

constexpr int kUnroll = 4;

__device__ __forceinline__ int draft_count(const int32_t* draft_len, int b, int K, bool& bad) {
  int n = draft_len ? draft_len[b] : K;
  bad = n < 0 || n > K;
  return bad ? 0 : n;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// ================================================================ greedy ===

// Stream rows of sequence b: target rows 0..n_b (none for an invalid draft
// length), then its W drafter rows.
__device__ __forceinline__ int greedy_targets(const GreedyArgs& a, int b) {
  bool bad;
  const int n = draft_count(a.draft_len, b, a.K, bad);
  return bad ? 0 : n + 1;
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_greedy_rows(GreedyArgs a) {
  __shared__ int s_pre[kSeqBlocks + 1];
  __shared__ int s_w[kWaves];
  auto count = [&](int b) { return greedy_targets(a, b) + a.W; };
  const SeqDir dir = build_seq_dir(a.B, count, s_pre, s_w);
  write_seq_starts(dir, s_pre, a.B, count, a.pre, blockIdx.x, gridDim.x);
  const FlatSplit f = make_split(s_pre[dir.nblk], a.V, Elem<DT>::kBytes, a.grid);
  const int64_t g = blockIdx.x;
  if (g >= f.G) return;
  SeqCursor cur;
  for_pieces(f, g, [&](int64_t r, int64_t v0, int64_t v1, const Progress& pg) {
    const int b = find_seq(dir, s_pre, static_cast<int>(r), count, cur);
    const int first = cur.first, cnt = cur.cnt;
    const int j = static_cast<int>(r) - first;
    const int nt = cnt - a.W;
    const char* rowp =
        j < nt ? static_cast<const char*>(a.tgt) + (static_cast<int64_t>(b) * a.ts + j * a.tr) * Elem<DT>::kBytes
               : static_cast<const char*>(a.dr) +
                     (static_cast<int64_t>(b) * a.ds + static_cast<int64_t>(j - nt) * a.drr) * Elem<DT>::kBytes;
    ArgmaxPick pk;
    stream_row<DT, kUnroll>(rowp, v0, v1, pk, pg);
    float v = pk.best;
    int ii = static_cast<int>(pk.bidx);
    int nan = pk.nan ? 1 : 0;
    wave_argmax(v, ii, nan);
    if (lane_id() == 0)
      a.part[(r + g) * kWaves + wave_id()] = make_float2(nan ? __builtin_nanf("") : v, __int_as_float(ii));
  });
}

__global__ __launch_bounds__(kBlock) void k_greedy_finalize(GreedyArgs a) {
  __shared__ int s_v[kMaxDraft + 1];
  __shared__ int s_z[kMaxDraft];
  __shared__ int s_st, s_h, s_a;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  bool nbad;
  const int n = draft_count(a.draft_len, b, a.K, nbad);
  const int budget = a.budget ? a.budget[b] : INT_MAX;
  const int p0 = a.pre[b];
  const FlatSplit f = make_split(a.pre[a.B], a.V, a.elem_bytes, a.grid);
  if (t == 0) {
    s_st = (nbad || budget < 0) ? SEQ_BAD_INPUT : 0;
    s_h = n;
  }
  __syncthreads();
  const int32_t* d = a.draft_tokens + static_cast<int64_t>(b) * a.K;
  int st = 0;
  for (int i = t; i < n; i += kBlock) {
    const int di = d[i];
    if (di < 0 || di >= a.V) st |= SEQ_BAD_INPUT;
  }
  // Stream rows p0.. of the sequence: target rows 0..n, then the W drafter rows.
  const int nt = nbad ? 0 : n + 1;
  combine_rows_pick(
      nt + a.W, a.part,
      [&](int r, int64_t& first, int64_t& cnt) {
        split_row_slots(f, p0 + r, first, cnt);
        first *= kWaves;
        cnt *= kWaves;
      },
      [&](int r, float v, int idx, int nan) {
        st |= nan ? SEQ_NONFINITE : max_status(v);
        if (r < nt) s_v[r] = idx;
        else s_z[r - nt] = idx;
      });
  if (st) atomicOr(&s_st, st);
  __syncthreads();
  const int status = s_st;
  int32_t* out = a.out_tokens + static_cast<int64_t>(b) * (a.K + 1);
  int32_t* nd = a.next_draft ? a.next_draft + static_cast<int64_t>(b) * a.W : nullptr;
  if (status & SEQ_ERROR_MASK) {
    for (int i = t; i <= a.K; i += kBlock) out[i] = -1;
    if (nd) for (int j = t; j < a.W; j += kBlock) nd[j] = -1;
    if (t == 0) {
      a.accept_len[b] = -1;
      a.num_out[b] = 0;
      if (a.next_len) a.next_len[b] = 0;
      if (a.status) a.status[b] = status;
    }
    return;
  }
  // h = number of leading matches d_i == v_i (Eq. 2)
  for (int i = t; i < n; i += kBlock)
    if (d[i] != s_v[i]) atomicMin(&s_h, i);
  __syncthreads();
  const int h = s_h;
  const int A = h + 1;
  if (t == 0) s_a = A < budget ? A : budget;
  __syncthreads();
  // ending condition: first EOS among C_1..C_A (1-based)
  if (a.eos >= 0) {
    for (int i = t; i < A; i += kBlock) {
      const int ci = i < h ? d[i] : s_v[h];
      if (ci == a.eos) atomicMin(&s_a, i + 1);
    }
  }
  __syncthreads();
  const int an = s_a;
  for (int i = t; i <= a.K; i += kBlock) out[i] = i < an ? (i < h ? d[i] : s_v[h]) : -1;
  const int keep = a.W - an > 0 ? a.W - an : 0;
  if (nd) for (int j = t; j < a.W; j += kBlock) nd[j] = j < keep ? s_z[an + j] : -1;
  if (t == 0) {
    a.accept_len[b] = h;
    a.num_out[b] = an;
    if (a.next_len) a.next_len[b] = keep;
    if (a.status) a.status[b] = status;
  }
}

// ============================================================== sampling ===

// Stream rows of sequence b: target rows 0..n_b (P stream rows each), then
// drafter rows 0..n_b-1 when they are streamed; none for an invalid draft
// length.
__device__ __forceinline__ int sample_count(const SampleArgs& a, int b, int P) {
  bool bad;
  const int n = draft_count(a.draft_len, b, a.K, bad);
  return bad ? 0 : P * (n + 1) + (a.drows ? n : 0);
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Four consecutive logits as float32, from one 8-byte (bf16) or 16-byte
// (fp32) nontemporal load.
template <int DT>
struct Quad;

template <>
struct Quad<DT_BF16> {
  typedef u32x2 raw;
  __device__ static __forceinline__ raw load(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  }
  __device__ static __forceinline__ void unpack(raw w, float (&x)[4]) {
    x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xffff0000u);
  }
};

template <>
struct Quad<DT_F32> {
  typedef u32x4 raw;
  __device__ static __forceinline__ raw load(const char* p) { return load16(p); }
  __device__ static __forceinline__ void unpack(raw w, float (&x)[4]) {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
};

// One pass over elements [v0, v1) of a target row and its Gumbel row: the
// softmax statistics of x and the lowest-index argmax of x/T + g.  Lane l
// takes four consecutive elements per step, so both the logit loads (8 or
// 16 bytes) and the Gumbel loads (16 bytes) are contiguous across the wave;
// every lane keeps U steps in flight.  Rows whose logits and Gumbel values
// cannot both be aligned are read element by element.
template <int DT, int U, class Stats>
__device__ void stats_and_gumbel(const char* xr, const float* gr, int64_t v0, int64_t v1, float inv_t,
                                 Stats& st, ArgmaxPick& pk, const Progress& pg, int64_t done0, int quad_units) {
  using E = Elem<DT>;
  using Q = Quad<DT>;
  constexpr int XB = 4 * E::kBytes;
  const int t = threadIdx.x;
  auto one = [&](int64_t j) {
    float x[1] = {E::load1(xr, j)};
    float sc[1] = {__builtin_fmaf(x[0], inv_t, gr[j])};
    st.template absorb<1>(x);
    pk.group<1>(sc, j);
  };
  // The Gumbel scores of four elements go to the argmax; their logits stay
  // in x for one absorb per U steps.
  auto scores = [&](const float (&x)[4], u32x4 g, int64_t idx) {
    float sc[4];
    sc[0] = __builtin_fmaf(x[0], inv_t, __uint_as_float(g.x));
    sc[1] = __builtin_fmaf(x[1], inv_t, __uint_as_float(g.y));
    sc[2] = __builtin_fmaf(x[2], inv_t, __uint_as_float(g.z));
    sc[3] = __builtin_fmaf(x[3], inv_t, __uint_as_float(g.w));
    pk.group<4>(sc, idx);
  };
  auto use = [&](typename Q::raw xv, u32x4 g, int64_t idx) {
    float x[4];
    Q::unpack(xv, x);
    scores(x, g, idx);
    st.template absorb<4>(x);
  };
  if (v1 <= v0) return;
  const uintptr_t ag = reinterpret_cast<uintptr_t>(gr + v0);
  int64_t head = static_cast<int64_t>(((16u - (ag & 15u)) & 15u) / 4u);
  if (head > v1 - v0) head = v1 - v0;
  const int64_t a0 = v0 + head;
  if ((ag & 3u) != 0 || (reinterpret_cast<uintptr_t>(xr + a0 * E::kBytes) % XB) != 0) {
    for (int64_t j = v0 + t; j < v1; j += kBlock) one(j);
    return;
  }
  const int64_t nq = (v1 - a0) / 4;
  const int64_t a1 = a0 + nq * 4;
  if (t < head) one(v0 + t);
  const char* xb = xr + a0 * E::kBytes;
  const char* gb = reinterpret_cast<const char*>(gr + a0);
  int64_t i = t;
  // ib: i - t, the same in every lane; a step of quads moves the stream
  // position by quad_units each
  for (int64_t ib = 0; i + (U - 1) * kBlock < nq; i += U * kBlock, ib += U * kBlock) {
    steer_priority(pg, done0 + ib * quad_units);
    typename Q::raw xv[U];
    u32x4 g[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = i + u * kBlock;
      xv[u] = Q::load(xb + k * XB);
      g[u] = load16(gb + k * 16);
    }
    __builtin_amdgcn_sched_barrier(0);
    float xs[U * 4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x[4];
      Q::unpack(xv[u], x);
      scores(x, g[u], a0 + (i + u * kBlock) * 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) xs[u * 4 + j] = x[j];
    }
    st.template absorb<U * 4>(xs);
  }
  for (; i < nq; i += kBlock) use(Q::load(xb + i * XB), load16(gb + i * 16), a0 + i * 4);
  if (a1 + t < v1) one(a1 + t);
}


// Rows per directory block for calls of more than kSeqBlocks sequences
// (SeqDir): one wave per block sums its sequences' row counts, 64 at a
// time, so that the row kernel's groups load the block sums instead of
// counting every sequence each.
template <int DT, bool GUM>
__global__ __launch_bounds__(kBlock) void k_seq_blocks(SampleArgs a) {
  constexpr int P = GUM ? (Elem<DT>::kBytes + 4) / Elem<DT>::kBytes : 1;
  const SeqDir d = seq_dir_shape(a.B);
  const int j = static_cast<int>(blockIdx.x) * kWaves + wave_id();
  if (j >= d.nblk) return;
  const int lane = lane_id();
  const int b1 = (j + 1) * d.q < a.B ? (j + 1) * d.q : a.B;
  int sum = 0;
  for (int b = j * d.q + lane; b < b1; b += 64) sum += sample_count(a, b, P);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
  if (lane == 0) a.blk[j] = sum;
}

// GUM: target rows are read with their Gumbel rows (joint-space chain with
// coupled-noise links).
// SMALL: rows of at most kSmallRowBytes, streamed a piece per wave.
template <int DT, bool GUM, bool SMALL = false>
__global__ __launch_bounds__(kBlock) void k_sample_rows(SampleArgs a) {
  __shared__ int s_pre[kSeqBlocks + 1];
  __shared__ int s_w[kWaves];
  constexpr int P = GUM ? (Elem<DT>::kBytes + 4) / Elem<DT>::kBytes : 1;
  auto count = [&](int b) { return sample_count(a, b, P); };
  const SeqDir dir = a.blk ? load_seq_dir(a.B, a.blk, s_pre, s_w) : build_seq_dir(a.B, count, s_pre, s_w);
  write_seq_starts(dir, s_pre, a.B, count, a.pre, blockIdx.x, gridDim.x);
  const FlatSplit f = make_split(s_pre[dir.nblk], a.V, Elem<DT>::kBytes, a.grid);
  const int64_t g = blockIdx.x;
  if (g >= f.G) return;
  // With Gumbel rows, the parts of one target row that this group reads are
  // accumulated together and written once, at slot (first stream row of the
  // target row) + group.
  SoftmaxStats64 acc(a.kp);
  ArgmaxPick accp;
  int64_t pend = -1;
  auto put = [&](int64_t slot, float M, double R) {
    Stat64 st;
    st.M = M;
    st.pad = 0.f;
    st.R = R;
    a.stats[slot] = st;
  };
  auto flush = [&]() {
    float M = acc.M;
    double R = static_cast<double>(acc.R);
    wave_stats64(M, R, a.kp);
    float v = accp.best;
    int ii = static_cast<int>(accp.bidx);
    int nan = accp.nan ? 1 : 0;
    wave_argmax(v, ii, nan);
    if (lane_id() == 0) {
      put((pend + g) * kWaves + wave_id(), M, R);
      a.gpart[(pend + g) * kWaves + wave_id()] = make_float2(nan ? __builtin_nanf("") : v, __int_as_float(ii));
    }
    acc = SoftmaxStats64(a.kp);
    accp = ArgmaxPick();
    pend = -1;
  };
  // Short rows (a few loads per lane) are taken a whole piece per wave, so
  // that each piece costs one wave reduction instead of four.
  static_assert(!(GUM && SMALL), "Gumbel rows take the group path");
  int piece = 0;
  SeqCursor cur;
  for_pieces(f, g, [&](int64_t r, int64_t v0, int64_t v1, const Progress& pg) {
    if (SMALL && (piece++ % kWaves) != wave_id()) return;
    const int b = SMALL ? find_seq_wave(dir, s_pre, static_cast<int>(r), a.B, count, cur)
                        : find_seq(dir, s_pre, static_cast<int>(r), count, cur);
    const int first = cur.first, cnt = cur.cnt;
    const int j = static_cast<int>(r) - first;
    const int n = a.drows ? (cnt - P) / (P + 1) : cnt / P - 1;
    const bool target = j < P * (n + 1);
    const int jt = j / P;   // target row of a target part
    const float k = target ? a.kp : a.kq;
    const char* rowp =
        target ? static_cast<const char*>(a.tgt) + (static_cast<int64_t>(b) * a.ts + jt * a.tr) * Elem<DT>::kBytes
               : static_cast<const char*>(a.drf) +
                     (static_cast<int64_t>(b) * a.ds + static_cast<int64_t>(j - P * (n + 1)) * a.dr) *
                         Elem<DT>::kBytes;
    if (GUM && target) {
      const int part = j - jt * P;
      const int64_t base = r - part;
      if (pend != base) {
        if (pend >= 0) flush();
        pend = base;
      }
      stats_and_gumbel<DT, 2 * kUnroll>(rowp, a.gumbel + b * a.gs + static_cast<int64_t>(jt) * a.grs,
                                    part_offset(a.V, P, part, v0), part_offset(a.V, P, part, v1), a.inv_t, acc,
                                    accp, pg, pg.off + v0, 4 * P);
      return;
    }
    if (GUM && pend >= 0) flush();
    SoftmaxStats64 st(k);
    if constexpr (SMALL) {
      // One wave per piece: its statistics, and the identity in the other
      // waves' slots of the piece.
      stream_row<DT, kUnroll, SoftmaxStats64, 64>(rowp, v0, v1, st);
      float M = st.M;
      double R = static_cast<double>(st.R);
      wave_stats64(M, R, k);
      const int lane = lane_id();
      if (lane < kWaves) put((r + g) * kWaves + lane, lane == wave_id() ? M : -kInf, lane == wave_id() ? R : 0.0);
      return;
    }
    stream_row<DT, kUnroll>(rowp, v0, v1, st, pg);
    float M = st.M;
    double R = static_cast<double>(st.R);
    wave_stats64(M, R, k);
    if (lane_id() == 0) put((r + g) * kWaves + wave_id(), M, R);
  });
  if (GUM && pend >= 0) flush();
}

// 1 - 2^d for d < 0 to float32 relative precision also where 2^d is close
// to 1: for d > -0.5 a Taylor polynomial of -expm1(d ln 2) (the first
// omitted term is below 2e-8 relative there), else 1 - exp2(d).  (Where one
// token carries nearly all of both rows' mass, 1 - exp2(d) alone would leave
// an error of an ulp of 1 on the whole residual.)
__device__ __forceinline__ float one_minus_exp2(float d) {
  const float z = d * 0.6931471805599453f;
  float t = __builtin_fmaf(z, 1.f / 5040.f, 1.f / 720.f);
  t = __builtin_fmaf(z, t, 1.f / 120.f);
  t = __builtin_fmaf(z, t, 1.f / 24.f);
  t = __builtin_fmaf(z, t, 1.f / 6.f);
  t = __builtin_fmaf(z, t, 0.5f);
  t = __builtin_fmaf(z, t, 1.f);
  return d > -0.5f ? -z * t : 1.f - fast_exp2(d);
}

// Per-element weight of the draw: residual [p~ - q]_+ or the bonus weight.
// The bonus weight is exp2(x kp - ep), p up to the row normaliser.  The
// residual is p (1 - 2^d) with d = log2(q/p) = (y kq - x kp) + C formed from
// the logits directly (x kp split into an exact sum hx + lx), so the
// normalisers never enter as two rounded scales whose difference would
// dominate where p and q nearly cancel, and each weight keeps float32
// relative precision.  For the linear rule p~ = p up to the
// (1 - lambda) factor, which the normalisation removes; for the Cactus rule
// isp also carries the rescaling (1 - gamma) / (1 - p(d)) of every token but
// the drafted one, element `excl`, whose weight is wexcl = [gamma - q(d)]_+.
// The row constant of the log-ratio, C - (mq kq - mp kp) for the rows'
// largest logits mp, mq, in float64 (the products of float32 values are
// exact there), split into float32 hi + lo.
__device__ __forceinline__ void split_row_constant(float C, float mp, float mq, float kp, float kq, float& hi,
                                                   float& lo) {
  const double A = kp == kq ? (static_cast<double>(mq) - static_cast<double>(mp)) * static_cast<double>(kp)
                            : static_cast<double>(mq) * kq - static_cast<double>(mp) * kp;
  const double c = static_cast<double>(C) - A;
  hi = static_cast<float>(c);
  const double r = c - static_cast<double>(hi);
  lo = r == r ? static_cast<float>(r) : 0.f;   // an infinite C leaves no low part
}

struct DrawWeight {
  float kp, ep, isp, kq;
  float chi, clo;  // the row constant of the log-ratio, hi + lo
  int resid;
  int same_t;      // kp == kq
  int excl;
  float wexcl;
  double isp64;
  // d = log2(q(v) / p~(v)) = (y kq - x kp) + chi + clo.  The logit term is
  // formed without rounding where it is small: y - x is exact for bf16
  // logits and, for float32 ones, carries its rounding error (TwoSum), and
  // with two temperatures x kp is split into an exact sum.  The row constant
  // holds the two rows' log-partition difference in float64 precision, so d
  // keeps float32 relative precision wherever p and q nearly cancel.
  template <int DT>
  __device__ __forceinline__ float log_ratio(float x, float y) const {
    if (same_t) {
      const float s = y - x;
      float d = __builtin_fmaf(s, kp, chi);
      if constexpr (DT == DT_F32) {
        const float bp = s - y;
        const float err = (y - (s - bp)) + (-x - bp);
        // NaN only where s is infinite, where d already is too
        d += fminf(fmaxf(__builtin_fmaf(err, kp, clo), -1e30f), 1e30f);
      } else {
        d += clo;
      }
      return d;
    }
    const float hx = x * kp;
    const float lx = __builtin_fmaf(x, kp, -hx);
    return ((__builtin_fmaf(y, kq, -hx) - lx) + chi) + clo;
  }
  template <int DT>
  __device__ __forceinline__ float weight(float x, float y) const {
    const float e = fast_exp2(__builtin_fmaf(x, kp, -ep));
    if (!resid) return e;
    const float d = log_ratio<DT>(x, y);
    // d >= 0: q >= p; d NaN only where p = 0 (x = -inf)
    return d < 0.f ? e * isp * one_minus_exp2(d) : 0.f;
  }
  // The weight of element e.
  template <int DT>
  __device__ __forceinline__ float at(uint32_t e, float x, float y) const {
    const float v = weight<DT>(x, y);
    return static_cast<int>(e) == excl ? wexcl : v;
  }
  // [p - Q]_+ against a stored sparse Q: p itself off the list (Q = 0); on
  // it the difference is formed in float64, where p and Q may nearly cancel.
  __device__ __forceinline__ float sparse(float x, float q) const {
    const float p = fast_exp2(__builtin_fmaf(x, kp, -ep)) * isp;
    if (q == 0.f) return p;
    const double pd = exp2(static_cast<double>(x) * static_cast<double>(kp) - static_cast<double>(ep)) * isp64;
    return static_cast<float>(fmax(pd - static_cast<double>(q), 0.0));
  }
};

// The modified Cactus target mass on a drafted token ("Speculative Diffusion
// is a Tale of Two Tradeoffs", App. E): the largest gamma in [p, 1] with
//   Phi(gamma) = gamma log(gamma/p) + (1-gamma) log((1-gamma)/(1-p)) <= delta,
// the Bernoulli KL of Eq. 17 (the KL of the modified target from p).  Solved
// as the page does, by Newton's method, from the Taylor value of Eq. 18.
// With x = gamma - p both logarithms are log1p terms, L1 = log1p(x/p) and
// L2 = log1p(-x/(1-p)), shared by Phi = gamma L1 + (1-gamma) L2 and
// Phi' = L1 - L2; float32 then loses accuracy in Phi only where Phi is of
// order x^2, and the error that leaves in gamma is of order x times that
// loss.  The iteration stops once the Newton step is below float32
// resolution of gamma (it converges in at most 8 steps over p in
// [1e-12, 1), delta in [1e-8, 40]); a step that would leave the bracket
// [lo, hi] known around the root bisects instead.
__device__ float cactus_gamma(float p, float delta) {
  if (!(p > 0.f)) return 0.f;            // Phi = +inf for any gamma > 0
  if (p >= 1.f) return 1.f;
  if (!(delta > 0.f)) return p;          // delta = 0: the lossless target
  if (-logf(p) <= delta) return 1.f;     // Phi(1) = -log p
  const float xmax = 1.f - p;            // x lives in (0, 1 - p)
  float lo = 0.f, hi = xmax;
  float x = sqrtf(2.f * delta * p * xmax);
  if (!(x < hi)) x = 0.5f * hi;
  for (int it = 0; it < 40; ++it) {
    const float g = p + x;
    const float L1 = log1pf(x / p);
    const float L2 = log1pf(-x / xmax);
    const float f = g * L1 + (1.f - g) * L2 - delta;
    if (f > 0.f) hi = x;
    else lo = x;
    const float step = f / (L1 - L2);
    if (fabsf(step) <= 2e-7f * g) break;
    float xn = x - step;
    if (!(xn > lo && xn < hi)) xn = 0.5f * (lo + hi);
    x = xn;
  }
  return fminf(p + x, 1.f);
}

constexpr int kTileBatch = 4;   // tiles a wave reads together (8 loads per lane)

// Masses of the draw row's tiles [t_lo, t_hi) (64 16-byte vectors each, of
// the row and, for the residual, of drafter row yr), by the NW waves of the
// group: wave w takes tiles t_lo + w, t_lo + w + NW, ..., TB of them
// at a time with all their loads in flight; lane l sums the weights of the
// tile's l-th vector and the wave reduces them into out[tile].  `vec` says
// both rows are 16-byte aligned; otherwise (and for the row's last, partial
// vector) elements are loaded one by one.  Byte offsets stay below 2^32
// (V <= kMaxSampleV), so the loads take a uniform 64-bit base and 32-bit lane
// offsets.
// Stored entries of a sparse Q that fall in some element range, in LDS:
// Q(v) is the sum of the entries naming v (zero off the list).
struct QList {
  const int* idx;
  const float* prob;
  int n;
  // Q of the N consecutive elements from e0.
  template <int N>
  __device__ __forceinline__ void lookup(uint32_t e0, float (&q)[N]) const {
#pragma unroll
    for (int j = 0; j < N; ++j) q[j] = 0.f;
#pragma unroll 4
    for (int k = 0; k < n; ++k) {
      const uint32_t d = static_cast<uint32_t>(idx[k]) - e0;
      const float pr = prob[k];
#pragma unroll
      for (int j = 0; j < N; ++j) q[j] += d == static_cast<uint32_t>(j) ? pr : 0.f;
    }
  }
};

// SP: the residual against a stored sparse Q, weight [p - Q]_+ with p =
// exp2(x kp + cp) isp and Q from `ql`; no drafter row is read.
// ws (not with SP): also every element's weight, at ws[element].
template <int DT, int NW, int TB = kTileBatch, bool SP = false>
__device__ __forceinline__ void tile_masses(const char* xr, const char* yr, int64_t V, int t_lo, int t_hi, bool vec,
                            const DrawWeight& w, float* out, const QList* ql = nullptr, float* ws = nullptr) {
  using E = Elem<DT>;
  constexpr int W = E::kVec;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const uint32_t Vn = static_cast<uint32_t>(V);
  for (int t0 = t_lo + wv; t0 < t_hi; t0 += NW * TB) {
    u32x4 rx[TB], ry[TB];
    bool full[TB];
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      const int tile = t0 + k * NW;
      const uint32_t e = static_cast<uint32_t>(tile) * (64 * W) + lane * W;   // the lane's first element
      full[k] = vec && tile < t_hi && e + W <= Vn;
      if (full[k]) {
        rx[k] = load16(xr + e * E::kBytes);
        ry[k] = (!SP && w.resid) ? load16(yr + e * E::kBytes) : rx[k];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      const int tile = t0 + k * NW;
      if (tile < t_hi) {   // uniform across the wave
        const uint32_t e = static_cast<uint32_t>(tile) * (64 * W) + lane * W;
        float m = 0.f;
        if constexpr (SP) {
          float x[W], q[W];
          if (full[k]) {
            E::unpack(rx[k], x);
          } else {
#pragma unroll
            for (int j = 0; j < W; ++j) x[j] = e + j < Vn ? E::load1(xr, e + j) : 0.f;
          }
          ql->lookup<W>(e, q);
#pragma unroll
          for (int j = 0; j < W; ++j) m += e + j < Vn ? w.sparse(x[j], q[j]) : 0.f;
        } else if (full[k]) {
          float x[W], y[W];
          E::unpack(rx[k], x);
          E::unpack(ry[k], y);
#pragma unroll
          for (int j = 0; j < W; ++j) {
            const float wt = w.template at<DT>(e + j, x[j], y[j]);
            m += wt;
            if (ws) ws[e + j] = wt;
          }
        } else {
          for (int j = 0; j < W; ++j) {
            if (e + j < Vn) {
              const float wt = w.template at<DT>(e + j, E::load1(xr, e + j), w.resid ? E::load1(yr, e + j) : 0.f);
              m += wt;
              if (ws) ws[e + j] = wt;
            }
          }
        }
#pragma unroll
        for (int sh = 32; sh >= 1; sh >>= 1) m += wave_shfl_xor(m, sh);
        if (lane == 0) out[tile] = m;
      }
      // One tile's weights at a time: interleaving the tiles' arithmetic
      // only raises register pressure (the loads are already in flight).
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Exclusive scan of one float per thread over NW waves, in thread order;
// also returns the total.  Two barriers.
template <int NW>
__device__ __forceinline__ float group_exclusive_scan_f(float v, float& total, float* s_w) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  float inc = v;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float o = __shfl_up(inc, m, 64);
    if (lane >= m) inc += o;
  }
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  float base = 0.f;
  total = 0.f;
  for (int j = 0; j < NW; ++j) {
    if (j < w) base += s_w[j];
    total += s_w[j];
  }
  __syncthreads();
  return base + inc - v;
}

// Rule families, one set of draw kernels each, so that no family carries
// another's code: the token chain (linear and Cactus rules), the joint-space
// chain, and the token chain against stored sparse Q.
enum : int { FAM_TOKEN = 0, FAM_SPOT = 1, FAM_SPARSE = 2 };

// The probability of a logit x in a row with statistics (M, R) (float64 rest
// relative to the reference floor(M k)).
__device__ __forceinline__ float prob64(float x, float k, float M, double R) {
  return fast_exp2(__builtin_fmaf(x, k, -ref_exp(M, k))) * static_cast<float>(1.0 / stats64_total(M, R, k));
}

// LDS of the decision step (per sequence): the status, h, and d, p(d),
// p~(d), q(d) of the rejected draft ...
struct DecideScalars {
  int st, h;
  int dh, modeh;
  float ph, pth, qh, ch;
};

// ... and, in the launch's dynamic LDS sized for the call's K
// (decide_lds_bytes), the row statistics of the target rows 0..n and the
// drafter rows 0..n-1 -- or (stored sparse Q) each draft's token and Q(d)
// summed from its row's entries -- and (joint-space chain) the Gumbel argmax
// of the target rows.  Every thread holds the same view.
struct DecideLds {
  double* Rp;
  double* Rq;
  float* Mp;
  float* Mq;
  int* g;
  float* qd;     // aliases Mq
  int* dtok;     // aliases Rq
  DecideScalars* sc;
};

__host__ __device__ constexpr size_t decide_lds_bytes(int K) {
  return static_cast<size_t>(K + 1) * 8 + static_cast<size_t>(K) * 8 + static_cast<size_t>(K + 1) * 4 +
         static_cast<size_t>(K) * 4 + static_cast<size_t>(K + 1) * 4;
}

// The fused draw also keeps every weight of row h in dynamic LDS, after the
// decision's arrays, where both fit in 32 KB: the select step's rescan then
// reads the chosen tile's weights instead of loading and weighing it again.
__host__ __device__ constexpr size_t fused_weights_offset(int K) { return (decide_lds_bytes(K) + 15) / 16 * 16; }
__host__ __device__ constexpr bool fused_weights_fit(int K, int64_t V) {
  return fused_weights_offset(K) + static_cast<size_t>(V) * 4 <= 32768;
}

__device__ __forceinline__ DecideLds decide_view(char* dyn, int K, DecideScalars* sc) {
  DecideLds v;
  v.Rp = reinterpret_cast<double*>(dyn);
  v.Rq = v.Rp + (K + 1);
  v.Mp = reinterpret_cast<float*>(v.Rq + K);
  v.Mq = v.Mp + (K + 1);
  v.g = reinterpret_cast<int*>(v.Mq + K);
  v.qd = v.Mq;
  v.dtok = reinterpret_cast<int*>(v.Rq);
  v.sc = sc;
  return v;
}

// The decision of sequence b by a group of NT threads:
//  1. Every input is requested at once: the length, budget, draft tokens,
//     accept uniforms and stream position; then the row statistics partials
//     and the logits at the draft tokens.
//  2. p(d), q(d), the acceptance tests (u * q(d) < p~(d)) and h.  With
//     `first`, the group writes the diagnostics (and, for a sequence with a
//     data error, every output).
// Returns the draw record: row h, its weight parameters and the uniform; its
// status carries the error bits when there is nothing to draw.
template <int DT, int NT, int FAM>
__device__ __forceinline__ DrawRecord draw_decide(const SampleArgs& a, int b, bool first, DecideLds& s) {
  constexpr int DPT = (kMaxDraft + NT - 1) / NT;   // drafts of one thread
  using E = Elem<DT>;
  const int t = threadIdx.x;
  bool nbad;
  const int n = draft_count(a.draft_len, b, a.K, nbad);
  const int budget = a.budget ? a.budget[b] : INT_MAX;
  const int p0 = a.pre[b];
  const int R = a.pre[a.B];
  const int32_t* d = a.draft_tokens + static_cast<int64_t>(b) * a.K;
  constexpr bool spot = FAM == FAM_SPOT;
  constexpr bool sparse = FAM == FAM_SPARSE;
  int di[DPT], psk[DPT], ppk[DPT];
  float ui[DPT], xi[DPT], yi[DPT], ck[DPT];
#pragma unroll
  for (int k = 0; k < DPT; ++k) {
    const int i = t + k * NT;
    const int64_t o = static_cast<int64_t>(b) * a.K + i;
    di[k] = i < a.K ? d[i] : 0;
    ui[k] = i < a.K ? a.u_accept[o] : 0.f;
    psk[k] = ppk[k] = 0;
    ck[k] = 0.f;
    if (spot) {
      // pos_star covers links 0..K (the bonus row's position included).
      psk[k] = i <= a.K ? a.pos_star[static_cast<int64_t>(b) * (a.K + 1) + i] : 0;
      ppk[k] = i < a.K ? a.prop_pos[o] : 0;
      ck[k] = i < a.K ? a.qpos[o] : 0.f;
    }
  }
  int st = 0;
#pragma unroll
  for (int k = 0; k < DPT; ++k) {
    const int i = t + k * NT;
    xi[k] = yi[k] = 0.f;
    if (spot && i < n && psk[k] < 0) st |= SEQ_BAD_INPUT;
    if (spot && i < n && !(ck[k] >= 0.f && ck[k] <= 1.f)) st |= SEQ_BAD_INPUT;
    if (i < n) {
      if (di[k] < 0 || di[k] >= a.V) {
        st |= SEQ_BAD_INPUT;
      } else {
        xi[k] = E::load1(static_cast<const char*>(a.tgt) + (b * a.ts + i * a.tr) * E::kBytes, di[k]);
        if (!sparse)
          yi[k] = E::load1(static_cast<const char*>(a.drf) + (b * a.ds + i * a.dr) * E::kBytes, di[k]);
      }
    }
  }
  if (t == 0) {
    // pos_star of the bonus row n (rows 0..n-1 are checked with their links)
    const bool bad_star = spot && !nbad && a.pos_star[static_cast<int64_t>(b) * (a.K + 1) + n] < 0;
    s.sc->st = (nbad || budget < 0 || bad_star) ? SEQ_BAD_INPUT : 0;
    s.sc->h = n;
  }
  __syncthreads();
  if (!nbad) {
    // Stream rows from p0: target rows 0..n (k = kp), each in P parts when
    // read with Gumbel rows (their partials are merged part by part: the
    // thread that finishes row r is the same in every pass); then drafter
    // rows 0..n-1 (k = kq).
    const FlatSplit f = make_split(R, a.V, E::kBytes, a.grid);
    // With Gumbel rows a target row is P consecutive stream rows; each group
    // that reads any of them wrote one partial at slot (first stream row of
    // the target row) + group.
    const int P = (spot && a.gumbel) ? gumbel_parts(E::kBytes) : 1;
    auto tspan = [&](int r, int64_t& first_slot, int64_t& cnt) {
      const int64_t v = p0 + static_cast<int64_t>(r) * P;
      const int64_t glo = split_group(f, v * f.V);
      const int64_t ghi = split_group(f, (v + P) * f.V - 1);
      first_slot = (v + glo) * kWaves;
      cnt = (ghi - glo + 1) * kWaves;
    };
    // The target rows 0..n and the drafter rows 0..n-1 in one pass, so all
    // their partials are requested together.
    const int nd = a.drows ? n : 0;
    const int nr = n + 1 + nd;
    auto kfn = [&](int r) { return r <= n ? a.kp : a.kq; };
    auto span = [&](int r, int64_t& first_slot, int64_t& cnt) {
      if (r <= n) {
        tspan(r, first_slot, cnt);
      } else {
        split_row_slots(f, p0 + static_cast<int64_t>(P) * (n + 1) + (r - n - 1), first_slot, cnt);
        first_slot *= kWaves;
        cnt *= kWaves;
      }
    };
    auto done = [&](int r, float M, double R) {
      if (r <= n) {
        s.Mp[r] = M; s.Rp[r] = R;
      } else {
        s.Mq[r - n - 1] = M; s.Rq[r - n - 1] = R;
      }
      st |= stats64_status(M, R);
    };
    // Half the lanes per row where that takes every row in one pass.
    if (nr > NT / kRowLanes && nr <= 2 * NT / kRowLanes)
      combine_rows_stats64<NT, kRowLanes / 2>(nr, a.stats, kfn, span, done);
    else
      combine_rows_stats64<NT>(nr, a.stats, kfn, span, done);
    if (P > 1)
      combine_rows_pick<NT>(n + 1, a.gpart, tspan, [&](int r, float v, int idx, int nan) {
        s.g[r] = idx;
        st |= nan ? SEQ_NONFINITE : max_status(v);
      });
  }
  if (sparse && !nbad) {
    // Q(d_i) from row i's stored entries, every (draft, entry) pair one work
    // item of the group; each draft's thread checks its entry count.
#pragma unroll
    for (int k = 0; k < DPT; ++k) {
      const int i = t + k * NT;
      if (i < n) {
        const int nz = a.qnnz[static_cast<int64_t>(b) * a.K + i];
        if (nz < 0 || nz > a.kmax) st |= SEQ_BAD_INPUT;
        s.dtok[i] = di[k];
        s.qd[i] = 0.f;
      }
    }
    __syncthreads();
    const int64_t items = static_cast<int64_t>(n) * a.kmax;
    for (int64_t it = t; it < items; it += NT) {
      const int i = static_cast<int>(it / a.kmax);
      const int e = static_cast<int>(it - static_cast<int64_t>(i) * a.kmax);
      const int64_t row = static_cast<int64_t>(b) * a.K + i;
      const int nz = a.qnnz[row];
      if (e >= nz) continue;
      const int v = a.qidx[row * a.kmax + e];
      const float pr = a.qprob[row * a.kmax + e];
      if (v < 0 || v >= a.V || !(pr >= 0.f && pr <= 3.402823466e38f)) {
        st |= SEQ_BAD_INPUT;
        continue;
      }
      if (v == s.dtok[i]) atomicAdd(&s.qd[i], pr);
    }
  }
  if (st) atomicOr(&s.sc->st, st);
  __syncthreads();
  DrawRecord rec{};
  if (s.sc->st & SEQ_ERROR_MASK) {
    rec.status = s.sc->st;
    if (first) {
      int32_t* out = a.out_tokens + static_cast<int64_t>(b) * (a.K + 1);
      for (int i = t; i <= a.K; i += NT) out[i] = -1;
      for (int i = t; i < a.K; i += NT) {
        const int64_t o = static_cast<int64_t>(b) * a.K + i;
        if (a.p_draft) a.p_draft[o] = 0.f;
        if (a.q_draft) a.q_draft[o] = 0.f;
        if (a.alpha) a.alpha[o] = 0.f;
        if (a.accept_margin) a.accept_margin[o] = 0.f;
      }
      if (t == 0) {
        a.accept_len[b] = -1;
        a.num_out[b] = 0;
        if (a.residual_mass) a.residual_mass[b] = 0.f;
        if (a.draw_margin) a.draw_margin[b] = 1.f;
        if (a.status) a.status[b] = s.sc->st;
      }
    }
    return rec;
  }

  // Acceptance tests: accept d_i iff u_i * q_i(d_i) < p~_i(d_i).  Linear
  // rule: p~(d) = (1 - lambda) p(d) + lambda q(d).  Cactus rule:
  // p~(d) = gamma(p(d), delta).
  // Joint-space chain: q(z~) = c qhat(v~) on s*; a proposal elsewhere is
  // rejected (alpha = 0).  A link whose drafter confidence max qhat = 1/S
  // reaches tau (with Gumbel rows) is verified by coupled-noise match.
  float pk[DPT], ptk[DPT], qk[DPT];
  int mk[DPT];
#pragma unroll
  for (int k = 0; k < DPT; ++k) {
    const int i = t + k * NT;
    float p = 0.f, q = 0.f, pt = 0.f, al = 0.f;
    mk[k] = 0;
    if (i < n) {
      p = prob64(xi[k], a.kp, s.Mp[i], s.Rp[i]);
      q = sparse ? s.qd[i] : prob64(yi[k], a.kq, s.Mq[i], s.Rq[i]);
      bool acc;
      if (spot) {
        const bool on = ppk[k] == psk[k];
        // the drafter's confidence at s*: its largest token probability
        mk[k] = (a.gumbel && prob64(s.Mq[i], a.kq, s.Mq[i], s.Rq[i]) >= a.tau) ? 1 : 0;
        q *= ck[k];
        pt = p;
        if (mk[k]) {
          acc = on && di[k] == s.g[i];
          al = acc ? 1.f : 0.f;
        } else {
          if (on && q == 0.f && p > 0.f) atomicOr(&s.sc->st, SEQ_Q_ZERO);
          al = on ? (q > 0.f ? fminf(1.f, p / q) : (p > 0.f ? 1.f : 0.f)) : 0.f;
          acc = on && ui[k] * q < p;
        }
      } else {
        pt = a.rule == RULE_CACTUS ? cactus_gamma(p, a.delta) : (1.f - a.lam) * p + a.lam * q;
        if (q == 0.f && pt > 0.f) atomicOr(&s.sc->st, SEQ_Q_ZERO);
        al = q > 0.f ? fminf(1.f, pt / q) : (pt > 0.f ? 1.f : 0.f);
        acc = ui[k] * q < pt;
      }
      if (!acc) atomicMin(&s.sc->h, i);
    }
    pk[k] = p;
    ptk[k] = pt;
    qk[k] = q;
    if (first && i < a.K) {
      const int64_t o = static_cast<int64_t>(b) * a.K + i;
      if (a.p_draft) a.p_draft[o] = p;
      if (a.q_draft) a.q_draft[o] = q;
      if (a.alpha) a.alpha[o] = al;
      if (a.accept_margin) a.accept_margin[o] = i < n ? (mk[k] ? 1.f : fabsf(ui[k] - al)) : 0.f;
    }
  }
  __syncthreads();
  // Uniform across the group: keeps the row addresses in scalar registers.
  const int h = __builtin_amdgcn_readfirstlane(s.sc->h);
  const bool resid = h < n;
  if (resid && a.rule != RULE_LINEAR) {
    // The owner of draft h shares its token, probabilities and verifier.
#pragma unroll
    for (int k = 0; k < DPT; ++k)
      if (t + k * NT == h) {
        s.sc->dh = di[k];
        s.sc->ph = pk[k];
        s.sc->pth = ptk[k];
        s.sc->qh = qk[k];
        s.sc->modeh = mk[k];
        s.sc->ch = ck[k];
      }
    __syncthreads();
  }
  rec.status = s.sc->st;
  rec.h = h;
  rec.resid = resid ? (sparse ? 2 : 1) : 0;
  rec.ep = ref_exp(s.Mp[h], a.kp);
  rec.isp64 = 1.0 / stats64_total(s.Mp[h], s.Rp[h], a.kp);
  rec.isp = static_cast<float>(rec.isp64);
  // log2(q(v) / p(v)) = ((y_v - mq) kq - (x_v - mp) kp) + C with
  // C = log2(Sp' / Sq'), Sp' = 1 + Rp' the target row's sum relative to its
  // maximum's term (Rp' its rest relative to it, likewise for q).  In that
  // form C is exact to the rests' relative precision: where one token holds
  // nearly all of both rows' mass, C is the small difference of the two
  // rests, which the residual weight at that token needs.  The weights take
  // (y_v kq - x_v kp) + (C - (mq kq - mp kp)), the row constant in float64.
  float Cf = 0.f;
  if (resid && !sparse) {
    Cf = log2_sum_ratio(stats64_rest_rel(s.Mp[h], s.Rp[h], a.kp), stats64_rest_rel(s.Mq[h], s.Rq[h], a.kq));
  }
  rec.u = a.u_resample[static_cast<int64_t>(b) * (a.K + 1) + h];
  if (resid && a.rule == RULE_LINEAR && !(a.lam < 1.f)) {
    // lambda = 1: p~ = q, so [p~ - q]_+ = (1 - lambda) [p - q]_+ vanishes
    // (a draft is rejected only where q(d) = 0); the draw then falls back to
    // p like any residual of zero mass.
    rec.isp = 0.f;
    rec.isp64 = 0.0;
  }
  rec.excl = -1;
  rec.wexcl = 0.f;
  rec.fixed = -1;
  if (spot) {
    if (resid ? s.sc->modeh != 0 : a.gumbel != nullptr) {
      // A match link's rejection, or the bonus with Gumbel rows: the commit
      // is the target's coupled-noise token; nothing is drawn.
      rec.fixed = s.g[h];
      rec.resid = 0;
    } else if (resid) {
      Cf += log2f(s.sc->ch);   // residual [p - c qhat]_+
    }
  }
  if (resid && a.rule == RULE_CACTUS) {
    // p~(v) = (1 - gamma) / (1 - p(d)) p(v) for v != d, p~(d) = gamma.
    // c_rest = 1 - (gamma - p(d)) / (1 - p(d)) is often within an ulp of 1:
    // its logarithm comes from the excess gamma - p(d) (exact in float64)
    // through log1p.
    const double ph = s.sc->ph;
    const double c_rest = ph < 1.0 ? (1.0 - static_cast<double>(s.sc->pth)) / (1.0 - ph) : 0.0;
    rec.isp = static_cast<float>(rec.isp * c_rest);
    rec.isp64 *= c_rest;
    // residual [c_rest p - q]_+
    Cf -= ph < 1.0 ? static_cast<float>(log1p(-(static_cast<double>(s.sc->pth) - ph) / (1.0 - ph)) * 1.4426950408889634)
                   : -kInf;
    rec.excl = s.sc->dh;
    rec.wexcl = fmaxf(s.sc->pth - s.sc->qh, 0.f);
  }
  if (resid && !sparse) split_row_constant(Cf, s.Mp[h], s.Mq[h], a.kp, a.kq, rec.chi, rec.clo);
  return rec;
}

__device__ __forceinline__ DrawWeight draw_weight(const SampleArgs& a, const DrawRecord& r) {
  DrawWeight w;
  w.kp = a.kp; w.ep = r.ep; w.isp = r.isp;
  w.kq = a.kq;
  w.chi = r.chi; w.clo = r.clo;
  w.isp64 = r.isp64;
  w.resid = r.resid;
  w.same_t = a.kp == a.kq;
  w.excl = r.excl;
  w.wexcl = r.wexcl;
  return w;
}

// Row h of sequence b: the target row, and the drafter row for a residual.
template <int DT>
__device__ __forceinline__ void draw_rows(const SampleArgs& a, int b, int h, bool resid, const char*& xr,
                                          const char*& yr) {
  using E = Elem<DT>;
  xr = static_cast<const char*>(a.tgt) + (b * a.ts + static_cast<int64_t>(h) * a.tr) * E::kBytes;
  yr = resid && a.drows ? static_cast<const char*>(a.drf) + (b * a.ds + static_cast<int64_t>(h) * a.dr) * E::kBytes
                        : xr;
}

// Per (sequence, chunk of draw tiles), kBlock threads: the decision (chunk 0
// writes the diagnostics and the record), then the masses of the chunk's
// tiles of row h: [p~ - q]_+ against drafter row h if a draft was rejected,
// else the bonus weight p.  Against a stored sparse Q the masses are those of
// p; the select step redoes the tiles that hold stored entries.
template <int DT, int FAM>
__global__ __launch_bounds__(kBlock) void k_draw_mass(SampleArgs a) {
  extern __shared__ __align__(16) char s_dyn[];
  __shared__ DecideScalars s_sc;
  DecideLds s = decide_view(s_dyn, a.K, &s_sc);
  const int b = blockIdx.x / a.chunks;
  const int c = blockIdx.x - b * a.chunks;
  const DrawRecord rec = draw_decide<DT, kBlock, FAM>(a, b, c == 0, s);
  if (c == 0 && threadIdx.x == 0) a.rec[b] = rec;
  if ((rec.status & SEQ_ERROR_MASK) || rec.fixed >= 0) return;
  const char *xr, *yr;
  draw_rows<DT>(a, b, rec.h, rec.resid != 0, xr, yr);
  const bool vec = ((reinterpret_cast<uintptr_t>(xr) | reinterpret_cast<uintptr_t>(yr)) & 15u) == 0;
  const int t_lo = c * a.tpc;
  const int t_hi = t_lo + a.tpc < a.tiles ? t_lo + a.tpc : a.tiles;
  const DrawWeight w = draw_weight(a, rec);
  float* out = a.tmass + static_cast<int64_t>(b) * a.tiles;
  if constexpr (FAM == FAM_SPARSE) {
    if (w.resid == 2) {
      // Residual against the stored Q of row h: the entries that fall in this
      // group's tiles go to LDS; chunk 0 hands the whole row to the select
      // kernel.
      __shared__ int c_idx[kMaxNnz];
      __shared__ float c_prob[kMaxNnz];
      __shared__ int c_n;
      constexpr int TE = 64 * Elem<DT>::kVec;
      const int64_t row = static_cast<int64_t>(b) * a.K + rec.h;
      const int nnz = a.qnnz[row];
      const int t = threadIdx.x;
      if (t == 0) c_n = 0;
      __syncthreads();
      SparseRow* sr = a.sq + b;
      for (int e = t; e < nnz; e += kBlock) {
        const int v = a.qidx[row * a.kmax + e];
        const float pr = a.qprob[row * a.kmax + e];
        if (c == 0) {
          sr->idx[e] = v;
          sr->prob[e] = pr;
        }
        if (v >= t_lo * TE && v < t_hi * TE) {
          const int k = atomicAdd(&c_n, 1);
          c_idx[k] = v;
          c_prob[k] = pr;
        }
      }
      if (c == 0 && t == 0) sr->nnz = nnz;
      __syncthreads();
      const QList ql{c_idx, c_prob, c_n};
      tile_masses<DT, kWaves, 4, true>(xr, yr, a.V, t_lo, t_hi, vec, w, out, &ql);
      return;
    }
  }
  tile_masses<DT, kWaves, 4>(xr, yr, a.V, t_lo, t_hi, vec, w, out);
}

// Combined float64 statistics (maximum, rest) of one stream row's partials
// (one thread).
__device__ __forceinline__ void merge_span_stats64(const Stat64* part, int64_t first, int64_t n, float k, float& M,
                                                   double& R) {
  M = -kInf;
  R = 0.0;
  for (int64_t j = 0; j < n; ++j) stats64_merge(M, R, part[first + j].M, part[first + j].R, k);
}

// Diagnostic mode: TV(p_i, q_i) = 1/2 sum_v |p_i(v) - q_i(v)| of draft row i
// (Two Tradeoffs Sec. 2: the lossless acceptance rate of the row is 1 - TV),
// one group per (sequence, draft row).  Dense rows: both rows are streamed
// and |p - q| is p (1 - 2^d) where q < p, q (1 - 2^-d) elsewhere, with
// d = log2(q/p) from the logits as in the draw.  Stored sparse Q: the sum
// needs only the stored tokens, 1 - sum_list p + sum_list |p - Q|.
template <int DT, int FAM>
__global__ __launch_bounds__(kBlock) void k_row_tv(SampleArgs a) {
  using E = Elem<DT>;
  __shared__ float s_red[kWaves];
  __shared__ float s_row[8];   // ep, isp, eq, isq, C, status, mp, mq
  const int b = blockIdx.x / a.K;
  const int i = blockIdx.x - b * a.K;
  const int t = threadIdx.x;
  bool nbad;
  const int n = draft_count(a.draft_len, b, a.K, nbad);
  float* out = a.row_tv + static_cast<int64_t>(b) * a.K + i;
  if (nbad || i >= n) {
    if (t == 0) *out = 0.f;
    return;
  }
  const int p0 = a.pre[b];
  const FlatSplit f = make_split(a.pre[a.B], a.V, E::kBytes, a.grid);
  const int P = (FAM == FAM_SPOT && a.gumbel) ? gumbel_parts(E::kBytes) : 1;
  if (t == 0) {
    // target row i: P stream rows, one partial per group that read any part
    const int64_t v = p0 + static_cast<int64_t>(i) * P;
    const int64_t glo = split_group(f, v * f.V);
    const int64_t ghi = split_group(f, (v + P) * f.V - 1);
    float Mp, Mq = 0.f;
    double Rp, Rq = 0.0;
    merge_span_stats64(a.stats, (v + glo) * kWaves, (ghi - glo + 1) * kWaves, a.kp, Mp, Rp);
    int st = stats64_status(Mp, Rp);
    if (a.drows) {
      int64_t first, cnt;
      split_row_slots(f, p0 + static_cast<int64_t>(P) * (n + 1) + i, first, cnt);
      merge_span_stats64(a.stats, first * kWaves, cnt * kWaves, a.kq, Mq, Rq);
      st |= stats64_status(Mq, Rq);
    }
    s_row[0] = ref_exp(Mp, a.kp);
    s_row[5] = __int_as_float(st);
    s_row[6] = Mp;
    s_row[7] = Mq;
    if (!(st & SEQ_ERROR_MASK)) {
      s_row[1] = static_cast<float>(1.0 / stats64_total(Mp, Rp, a.kp));
      if (a.drows) {
        s_row[2] = ref_exp(Mq, a.kq);
        s_row[3] = static_cast<float>(1.0 / stats64_total(Mq, Rq, a.kq));
        s_row[4] = log2_sum_ratio(stats64_rest_rel(Mp, Rp, a.kp), stats64_rest_rel(Mq, Rq, a.kq));
      }
    }
  }
  __syncthreads();
  if (__float_as_int(s_row[5]) & SEQ_ERROR_MASK) {
    if (t == 0) *out = __builtin_nanf("");
    return;
  }
  const float ep = s_row[0], isp = s_row[1];
  const char* xr = static_cast<const char*>(a.tgt) + (b * a.ts + static_cast<int64_t>(i) * a.tr) * E::kBytes;
  float acc = 0.f;
  if constexpr (FAM == FAM_SPARSE) {
    // (S - sum_list e_v) / S + sum_list |e_v / S - Q_v| with e_v = exp2(x_v kp
    // - ep) and S = sum_v e_v summed here in float64 over the whole row: the
    // mass off the list is then a difference of two float64 sums of the same
    // rounded terms (no cancellation error where the list holds nearly all
    // of p), and the rounding of a dominant e_v cancels in e_v / S.
    __shared__ double s_d[kWaves];
    const int64_t row = static_cast<int64_t>(b) * a.K + i;
    const int nz = min(a.qnnz[row], a.kmax);
    double sa = 0.0;
    const bool vec = (reinterpret_cast<uintptr_t>(xr) & 15u) == 0;
    constexpr int W = E::kVec;
    const int64_t nvec = vec ? a.V / W : 0;
    for (int64_t j = t; j < nvec; j += kBlock) {
      float x[W];
      E::unpack(load16(xr + j * 16), x);
#pragma unroll
      for (int q = 0; q < W; ++q) sa += fast_exp2(__builtin_fmaf(x[q], a.kp, -ep));
    }
    for (int64_t e = nvec * W + t; e < a.V; e += kBlock) sa += fast_exp2(__builtin_fmaf(E::load1(xr, e), a.kp, -ep));
    auto bsum = [&](double v) {
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      __syncthreads();
      if ((t & 63) == 0) s_d[t >> 6] = v;
      __syncthreads();
      v = 0.0;
      for (int w = 0; w < kWaves; ++w) v += s_d[w];
      return v;
    };
    const double S = bsum(sa);
    double se = 0.0, sd = 0.0;
    for (int e = t; e < nz; e += kBlock) {
      const int v = a.qidx[row * a.kmax + e];
      if (v < 0 || v >= a.V) continue;
      const double ev = fast_exp2(__builtin_fmaf(E::load1(xr, v), a.kp, -ep));
      se += ev;
      sd += fabs(ev / S - static_cast<double>(a.qprob[row * a.kmax + e]));
    }
    se = bsum(se);
    sd = bsum(sd);
    if (t == 0) *out = static_cast<float>(0.5 * ((S - se) / S + sd));
    (void)isp;
    return;
  } else {
    const float eq = s_row[2], isq = s_row[3];
    const char* yr = static_cast<const char*>(a.drf) + (b * a.ds + static_cast<int64_t>(i) * a.dr) * E::kBytes;
    DrawWeight w{};
    w.kp = a.kp; w.kq = a.kq;
    split_row_constant(s_row[4], s_row[6], s_row[7], a.kp, a.kq, w.chi, w.clo);
    w.same_t = a.kp == a.kq;
    auto absdiff = [&](float x, float y) {
      const float d = w.template log_ratio<DT>(x, y);
      if (!(d == d)) return 0.f;   // both logits -inf: p = q = 0
      return d < 0.f ? fast_exp2(__builtin_fmaf(x, a.kp, -ep)) * isp * one_minus_exp2(d)
                     : fast_exp2(__builtin_fmaf(y, a.kq, -eq)) * isq * one_minus_exp2(-d);
    };
    const bool vec = ((reinterpret_cast<uintptr_t>(xr) | reinterpret_cast<uintptr_t>(yr)) & 15u) == 0;
    constexpr int W = E::kVec;
    const int64_t nvec = vec ? a.V / W : 0;
    for (int64_t j = t; j < nvec; j += kBlock) {
      float x[W], y[W];
      E::unpack(load16(xr + j * 16), x);
      E::unpack(load16(yr + j * 16), y);
#pragma unroll
      for (int q = 0; q < W; ++q) acc += absdiff(x[q], y[q]);
    }
    for (int64_t e = nvec * W + t; e < a.V; e += kBlock) acc += absdiff(E::load1(xr, e), E::load1(yr, e));
    acc = block_sum(acc, s_red);
    if (t == 0) *out = 0.5f * acc;
  }
}


// LDS of the select step for NT threads holding TPT tile masses each (the
// tile array serves the zero-mass fallback, which recomputes every tile).
template <int NT, int TPT>
struct SelectLdsT {
  static constexpr int kThreads = NT;
  static constexpr int kTiles = TPT;
  float tile[NT * TPT];
  float w[NT / 64];
  int whit[NT / 64], wlast[NT / 64];   // per wave: first hit, last positive tile
  float Z, base, margin;
  int cs, pick, a;
};
using SelectLds = SelectLdsT<kDrawThreads, kDrawTilesPerThread>;
// Rows of at most kSmallSelect * kSmallSelectTiles tiles are selected by
// kSmallSelect threads: four waves scan and synchronise faster than sixteen.
constexpr int kSmallSelect = kBlock;
constexpr int kSmallSelectTiles = 4;
using SmallSelectLds = SelectLdsT<kSmallSelect, kSmallSelectTiles>;

// Draft tokens d_{t + k NT + 1} of this thread (-1 past K).
template <int NT>
__device__ __forceinline__ void load_draft_tokens(const SampleArgs& a, int b, int (&dt)[(kMaxDraft + NT - 1) / NT]) {
  constexpr int DPT = (kMaxDraft + NT - 1) / NT;
#pragma unroll
  for (int k = 0; k < DPT; ++k) {
    const int i = static_cast<int>(threadIdx.x) + k * NT;
    dt[k] = i < a.K ? a.draft_tokens[static_cast<int64_t>(b) * a.K + i] : -1;
  }
}

// The stored sparse Q of row h, as the mass kernel handed it over.
struct SparseLds {
  int idx[kMaxNnz];
  float prob[kMaxNnz];
  int nnz;
};


// The draw of sequence b by the NT = LDS::kThreads threads of the group,
// given its record and this thread's TPT = LDS::kTiles tile masses m0 (tiles
// [t*q, (t+1)*q), q = ceil(tiles / NT) <= TPT):
// the tile where the running mass first exceeds u*Z (the last positive tile
// if rounding leaves u*Z at or past the total), the token inside it in
// vocabulary order, and the output assembly C = (d_1..d_h, c) with the
// ending condition.
// dt[k] is draft token d_{t + k NT + 1}, requested with the first loads;
// output position i = t + k NT, and k = DPT reaches i <= K only where i >= h.
// SPARSE: the call verifies against a stored sparse Q, whose LDS is sp.
template <int DT, bool SPARSE, class LDS>
__device__ __forceinline__ void draw_select(const SampleArgs& a, int b, const DrawRecord& rec, int budget,
                            const int (&dt)[(kMaxDraft + LDS::kThreads - 1) / LDS::kThreads],
                            const float (&m0)[LDS::kTiles], LDS& s, SparseLds* sp, const float* wl = nullptr) {
  constexpr int NT = LDS::kThreads;
  constexpr int TPT = LDS::kTiles;
  constexpr int DPT = (kMaxDraft + NT - 1) / NT;
  using E = Elem<DT>;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = t >> 6;
  const int ntiles = a.tiles;
  const int q = static_cast<int>(cdiv(ntiles, NT));   // tiles per thread, <= TPT
  const int h = __builtin_amdgcn_readfirstlane(rec.h);
  int status = rec.status;
  const bool resid0 = rec.resid != 0;
  const char *xr, *yr;
  draw_rows<DT>(a, b, h, resid0, xr, yr);
  DrawWeight w = draw_weight(a, rec);
  constexpr int TE = 64 * E::kVec;                              // elements per tile
  const bool draw = rec.fixed < 0;   // uniform across the group
  float mt[TPT];
#pragma unroll
  for (int k = 0; k < TPT; ++k) mt[k] = m0[k];

  // Thread t holds the masses of tiles [t*q, (t+1)*q); an exclusive scan
  // gives it the mass before them, and the group's total Z.
  auto locate = [&](const float (&m)[TPT]) {
    float loc = 0.f;
#pragma unroll
    for (int k = 0; k < TPT; ++k) loc += m[k];
    float Z;
    const float start = group_exclusive_scan_f<NT / 64>(loc, Z, s.w);
    const float target = rec.u * Z;
    int hit = INT_MAX, last = -1;
    float run = start;
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      if (m[k] > 0.f) {
        if (hit == INT_MAX && run + m[k] > target) hit = t * q + k;
        last = t * q + k;
      }
      run += m[k];
    }
    // Tiles increase with the thread index: the first hit is the first lane
    // with one in the first wave with one, the last positive tile the last
    // such lane of the last such wave (ballots, no LDS atomics).
    const uint64_t hb = __ballot(hit != INT_MAX);
    const uint64_t lb = __ballot(last >= 0);
    const int whit = __shfl(hit, hb ? __builtin_ctzll(hb) : 0, 64);
    const int wlast = __shfl(last, lb ? 63 - __builtin_clzll(lb) : 0, 64);
    if (lane == 0) {
      s.whit[wv] = hb ? whit : INT_MAX;
      s.wlast[wv] = lb ? wlast : -1;
    }
    __syncthreads();
    int fh = INT_MAX, fl = -1;
#pragma unroll
    for (int j = 0; j < NT / 64; ++j) {
      if (fh == INT_MAX) fh = s.whit[j];
      fl = s.wlast[j] >= 0 ? s.wlast[j] : fl;
    }
    const int ct = fh != INT_MAX ? fh : (fl >= 0 ? fl : 0);
    if (t == ct / q) {   // the owner of the chosen tile writes the mass before it
      float before = start;
#pragma unroll
      for (int k = 0; k < TPT; ++k)
        if (t * q + k < ct) before += m[k];
      s.base = before;
      s.Z = Z;
      s.cs = ct;
    }
    __syncthreads();
  };
  if (draw) locate(mt);
  const float Zres = resid0 ? s.Z : 0.f;
  if (draw && resid0 && !(s.Z > 0.f)) {
    // Residual mass vanished in float32 (p == q up to rounding): draw from p
    // with the same uniform instead, and flag it.  (This group recomputes
    // the tile masses of p alone; the case has probability zero in exact
    // arithmetic.)
    status |= SEQ_Z_ZERO;
    w.resid = 0;
    w.excl = -1;
    yr = xr;
    wl = nullptr;   // the stored weights were the residual's
    const bool vec = (reinterpret_cast<uintptr_t>(xr) & 15u) == 0;
    tile_masses<DT, NT / 64, 2>(xr, yr, a.V, 0, ntiles, vec, w, s.tile);
    __syncthreads();
    float m1[TPT];
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int tile = t * q + k;
      m1[k] = (k < q && tile < ntiles) ? s.tile[tile] : 0.f;
    }
    locate(m1);
  }
  const float target = rec.u * s.Z;

  // Wave 0 rescans the chosen tile in vocabulary order: lane l holds the
  // weights of the tile's l-th vector; a wave scan gives each lane the mass
  // before its vector.
  if (!draw) {
    if (t == 0) s.pick = rec.fixed;
  } else if (wv == 0) {
    const int ct = __builtin_amdgcn_readfirstlane(s.cs);
    const int64_t e0 = static_cast<int64_t>(ct) * TE + lane * E::kVec;
    float wt[E::kVec];
    float loc = 0.f;
    if (SPARSE && w.resid == 2) {
      // [p - Q]_+ against the stored Q of row h (as in the mass kernel)
      float q[E::kVec];
      const QList ql{sp->idx, sp->prob, sp->nnz};
      ql.lookup<E::kVec>(static_cast<uint32_t>(e0), q);
#pragma unroll
      for (int j = 0; j < E::kVec; ++j)
        wt[j] = e0 + j < a.V ? w.sparse(E::load1(xr, e0 + j), q[j]) : 0.f;
    } else if (wl) {
      // the weights the mass step stored in LDS (the same values)
#pragma unroll
      for (int j = 0; j < E::kVec; ++j) wt[j] = e0 + j < a.V ? wl[e0 + j] : 0.f;
    } else if (e0 + E::kVec <= a.V &&
               ((reinterpret_cast<uintptr_t>(xr) | reinterpret_cast<uintptr_t>(yr)) & 15u) == 0) {
      // the lane's vector of the row (and of the drafter row) in one load each
      float x[E::kVec], y[E::kVec];
      E::unpack(load16(xr + e0 * E::kBytes), x);
      if (w.resid) E::unpack(load16(yr + e0 * E::kBytes), y);
#pragma unroll
      for (int j = 0; j < E::kVec; ++j)
        wt[j] = w.template at<DT>(static_cast<uint32_t>(e0 + j), x[j], w.resid ? y[j] : 0.f);
    } else {
#pragma unroll
      for (int j = 0; j < E::kVec; ++j) {
        const int64_t e = e0 + j;
        wt[j] = e < a.V ? w.template at<DT>(static_cast<uint32_t>(e), E::load1(xr, e), w.resid ? E::load1(yr, e) : 0.f)
                        : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < E::kVec; ++j) loc += wt[j];
    float inc = loc;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) {
      const float o = __shfl_up(inc, k, 64);
      if (lane >= k) inc += o;
    }
    const float start = s.base + inc - loc;
    int found = -1, lastpos = -1;
    float r = start;
    float gap = 0.f;   // distance of u*Z from the nearer end of the found token's interval
#pragma unroll
    for (int j = 0; j < E::kVec; ++j) {
      const float before = r;
      r += wt[j];
      if (wt[j] > 0.f) {
        if (found < 0 && r > target) {
          found = static_cast<int>(e0 + j);
          gap = fminf(target - before, r - target);
        }
        lastpos = static_cast<int>(e0 + j);
      }
    }
    const uint64_t hits = __ballot(found >= 0);
    const uint64_t poss = __ballot(lastpos >= 0);
    int tok = -1;
    float mg = 0.f;
    if (hits) {
      const int src = __builtin_ctzll(hits);
      tok = __shfl(found, src, 64);
      mg = __shfl(gap, src, 64);
    } else if (poss) {
      tok = __shfl(lastpos, 63 - __builtin_clzll(poss), 64);
    }
    if (lane == 0) {
      s.pick = tok;
      s.margin = s.Z > 0.f ? fmaxf(mg, 0.f) / s.Z : 0.f;
    }
  }
  // ---- output assembly: C = (d_1..d_h, c), then the ending condition ----
  const int A = h + 1;
  if (t == 0) s.a = A < budget ? A : budget;
  __syncthreads();
  const int tok = s.pick;
  if (a.eos >= 0) {
#pragma unroll
    for (int k = 0; k <= DPT; ++k) {
      const int i = t + k * NT;
      const int ci = i < h ? dt[k < DPT ? k : DPT - 1] : tok;
      if (i < A && ci == a.eos) atomicMin(&s.a, i + 1);
    }
  }
  __syncthreads();
  const int an = s.a;
  int32_t* out = a.out_tokens + static_cast<int64_t>(b) * (a.K + 1);
#pragma unroll
  for (int k = 0; k <= DPT; ++k) {
    const int i = t + k * NT;
    if (i <= a.K) out[i] = i < an ? (i < h ? dt[k < DPT ? k : DPT - 1] : tok) : -1;
  }
  if (t == 0) {
    a.accept_len[b] = h;
    a.num_out[b] = an;
    // Mass of [p~ - q]_+ = (1 - lambda) [p - q]_+: the rejection probability.
    if (a.residual_mass) a.residual_mass[b] = Zres * (1.f - a.lam);
    if (a.draw_margin) a.draw_margin[b] = draw ? s.margin : 1.f;
    if (a.status) a.status[b] = status;
  }
}

// Second kernel of the split draw: one group of LDS::kThreads threads per
// sequence reads the record and the tile masses that k_draw_mass wrote.
template <int DT, int FAM, class LDS>
__global__ __launch_bounds__(LDS::kThreads) void k_draw_select(SampleArgs a) {
  constexpr int NT = LDS::kThreads;
  constexpr int TPT = LDS::kTiles;
  __shared__ LDS s;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int ntiles = a.tiles;
  const int q = static_cast<int>(cdiv(ntiles, NT));
  // Everything this group reads first is requested together: the decision
  // record, the budget, the draft tokens and this thread's tile masses.
  const DrawRecord rec = a.rec[b];
  const int budget = a.budget ? a.budget[b] : INT_MAX;
  int dt[(kMaxDraft + NT - 1) / NT];
  load_draft_tokens<NT>(a, b, dt);
  const float* tmass = a.tmass + static_cast<int64_t>(b) * ntiles;
  float m0[TPT];
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int tile = t * q + k;
    m0[k] = (k < q && tile < ntiles) ? tmass[tile] : 0.f;
  }
  if constexpr (FAM == FAM_SPARSE) {
    // The stored Q of row h, requested with the record (entries past nnz
    // are never used).
    __shared__ SparseLds sp;
    const SparseRow* sr = a.sq + b;
    for (int e = t; e < kMaxNnz; e += NT) {
      sp.idx[e] = sr->idx[e];
      sp.prob[e] = sr->prob[e];
    }
    if (t == 0) sp.nnz = sr->nnz;
    __syncthreads();
    if (rec.status & SEQ_ERROR_MASK) return;        // outputs already written
    draw_select<DT, true>(a, b, rec, budget, dt, m0, s, &sp);
  } else {
    if (rec.status & SEQ_ERROR_MASK) return;        // outputs already written
    draw_select<DT, false>(a, b, rec, budget, dt, m0, s, nullptr);
  }
}

// The whole draw of one sequence in one group of kSmallSelect threads (for
// rows of at most kFusedDrawTiles tiles): the decision, every tile mass of
// row h into LDS, then the draw.  Four waves keep a row of a few tiles as
// close to its loads as sixteen would, and let four times as many
// sequences share a CU.
template <int DT, int FAM>
__global__ __launch_bounds__(kSmallSelect) void k_draw_fused(SampleArgs a) {
  static_assert(FAM != FAM_SPARSE, "stored sparse Q takes the split draw");
  static_assert(kFusedDrawTiles <= SmallSelectLds::kThreads * SmallSelectLds::kTiles, "fused rows fit the LDS");
  constexpr int NT = SmallSelectLds::kThreads;
  constexpr int TPT = SmallSelectLds::kTiles;
  extern __shared__ __align__(16) char s_dyn[];
  __shared__ DecideScalars s_sc;
  DecideLds sd = decide_view(s_dyn, a.K, &s_sc);
  __shared__ SmallSelectLds s;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const DrawRecord rec = draw_decide<DT, NT, FAM>(a, b, true, sd);
  if (rec.status & SEQ_ERROR_MASK) return;
  const int budget = a.budget ? a.budget[b] : INT_MAX;
  int dt[(kMaxDraft + NT - 1) / NT];
  load_draft_tokens<NT>(a, b, dt);
  const char *xr, *yr;
  draw_rows<DT>(a, b, rec.h, rec.resid != 0, xr, yr);
  const bool vec = ((reinterpret_cast<uintptr_t>(xr) | reinterpret_cast<uintptr_t>(yr)) & 15u) == 0;
  const int ntiles = a.tiles;
  float* wl = fused_weights_fit(a.K, a.V) ? reinterpret_cast<float*>(s_dyn + fused_weights_offset(a.K)) : nullptr;
  if (rec.fixed < 0)
    tile_masses<DT, NT / 64, 4>(xr, yr, a.V, 0, ntiles, vec, draw_weight(a, rec), s.tile, nullptr, wl);
  __syncthreads();
  const int q = static_cast<int>(cdiv(ntiles, NT));
  float m0[TPT];
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const int tile = t * q + k;
    m0[k] = (k < q && tile < ntiles) ? s.tile[tile] : 0.f;
  }
  __syncthreads();   // the fallback in draw_select may overwrite s.tile
  draw_select<DT, false>(a, b, rec, budget, dt, m0, s, nullptr, wl);
}

// ============================================================== launches ===

template <typename K>
static const void* fn(K* k) {
  return reinterpret_cast<const void*>(k);
}

bool launch_greedy(const GreedyArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev) {
  const bool bf = dtype == DT_BF16;
  return launch(bf ? fn(k_greedy_rows<DT_BF16>) : fn(k_greedy_rows<DT_F32>), a.grid, stream, a, ev) &&
         launch(fn(k_greedy_finalize), a.B, stream, a);
}

bool launch_sample(const SampleArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev) {
  const bool bf = dtype == DT_BF16;
  const bool short_v = short_rows(a.V, bf ? 2 : 4);
  const void* rows = a.gumbel ? (bf ? fn(k_sample_rows<DT_BF16, true>) : fn(k_sample_rows<DT_F32, true>))
                     : short_v ? (bf ? fn(k_sample_rows<DT_BF16, false, true>) : fn(k_sample_rows<DT_F32, false, true>))
                              : (bf ? fn(k_sample_rows<DT_BF16, false>) : fn(k_sample_rows<DT_F32, false>));
  if (a.blk) {
    const void* blocks = a.gumbel ? (bf ? fn(k_seq_blocks<DT_BF16, true>) : fn(k_seq_blocks<DT_F32, true>))
                                  : (bf ? fn(k_seq_blocks<DT_BF16, false>) : fn(k_seq_blocks<DT_F32, false>));
    if (!launch(blocks, (seq_dir_shape(a.B).nblk + kWaves - 1) / kWaves, stream, a)) return false;
  }
  if (!launch(rows, a.grid, stream, a, ev)) return false;
  const int fam = a.rule == RULE_SPOT ? FAM_SPOT : (a.rule == RULE_SPARSE ? FAM_SPARSE : FAM_TOKEN);
  // [family][dtype == bf16]
  static const void* const fused[2][2] = {{fn(k_draw_fused<DT_F32, FAM_TOKEN>), fn(k_draw_fused<DT_BF16, FAM_TOKEN>)},
                                          {fn(k_draw_fused<DT_F32, FAM_SPOT>), fn(k_draw_fused<DT_BF16, FAM_SPOT>)}};
  static const void* const mass[3][2] = {{fn(k_draw_mass<DT_F32, FAM_TOKEN>), fn(k_draw_mass<DT_BF16, FAM_TOKEN>)},
                                         {fn(k_draw_mass<DT_F32, FAM_SPOT>), fn(k_draw_mass<DT_BF16, FAM_SPOT>)},
                                         {fn(k_draw_mass<DT_F32, FAM_SPARSE>), fn(k_draw_mass<DT_BF16, FAM_SPARSE>)}};
  // [small][family][dtype == bf16]
  static const void* const select[2][3][2] = {
      {{fn(k_draw_select<DT_F32, FAM_TOKEN, SelectLds>), fn(k_draw_select<DT_BF16, FAM_TOKEN, SelectLds>)},
       {fn(k_draw_select<DT_F32, FAM_SPOT, SelectLds>), fn(k_draw_select<DT_BF16, FAM_SPOT, SelectLds>)},
       {fn(k_draw_select<DT_F32, FAM_SPARSE, SelectLds>), fn(k_draw_select<DT_BF16, FAM_SPARSE, SelectLds>)}},
      {{fn(k_draw_select<DT_F32, FAM_TOKEN, SmallSelectLds>), fn(k_draw_select<DT_BF16, FAM_TOKEN, SmallSelectLds>)},
       {fn(k_draw_select<DT_F32, FAM_SPOT, SmallSelectLds>), fn(k_draw_select<DT_BF16, FAM_SPOT, SmallSelectLds>)},
       {fn(k_draw_select<DT_F32, FAM_SPARSE, SmallSelectLds>),
        fn(k_draw_select<DT_BF16, FAM_SPARSE, SmallSelectLds>)}}};
  // [family][dtype == bf16]
  static const void* const tv[3][2] = {{fn(k_row_tv<DT_F32, FAM_TOKEN>), fn(k_row_tv<DT_BF16, FAM_TOKEN>)},
                                       {fn(k_row_tv<DT_F32, FAM_SPOT>), fn(k_row_tv<DT_BF16, FAM_SPOT>)},
                                       {fn(k_row_tv<DT_F32, FAM_SPARSE>), fn(k_row_tv<DT_BF16, FAM_SPARSE>)}};
  if (a.row_tv && !launch(tv[fam][bf], static_cast<int64_t>(a.B) * a.K, stream, a)) return false;
  // the decision's row statistics in dynamic LDS, sized for this K
  const size_t dl = decide_lds_bytes(a.K);
  if (a.tiles <= kFusedDrawTiles && fam != FAM_SPARSE)
    return launch_threads(fused[fam][bf], a.B, kSmallSelect, stream, a, TimingEvents(),
                          fused_weights_fit(a.K, a.V) ? fused_weights_offset(a.K) + static_cast<size_t>(a.V) * 4 : dl);
  const bool small = a.tiles <= kSmallSelect * kSmallSelectTiles;
  return launch_threads(mass[fam][bf], static_cast<int64_t>(a.B) * a.chunks, kBlock, stream, a, TimingEvents(), dl) &&
         launch_threads(select[small][fam][bf], a.B, small ? kSmallSelect : kDrawThreads, stream, a);
}

}  // namespace dbv
