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
//   k_draw_mass        per (sequence, vocabulary chunk): the sequence's
//                      decision (p(d), q(d), the acceptance tests, h) and the
//                      chunk's mass of [p - q]_+ (or of p for the bonus)
//   k_draw_select      per sequence: the token where the running mass first
//                      exceeds u*Z (vocabulary order), output assembly.
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
  if (blockIdx.x == 0) write_seq_starts(dir, s_pre, a.B, count, a.pre);
  const FlatSplit f = make_split(s_pre[dir.nblk], a.V, Elem<DT>::kBytes, a.grid);
  const int64_t g = blockIdx.x;
  if (g >= f.G) return;
  for_pieces(f, g, [&](int64_t r, int64_t v0, int64_t v1) {
    int first, cnt;
    const int b = find_seq(dir, s_pre, static_cast<int>(r), count, first, cnt);
    const int j = static_cast<int>(r) - first;
    const int nt = cnt - a.W;
    const char* rowp =
        j < nt ? static_cast<const char*>(a.tgt) + (static_cast<int64_t>(b) * a.ts + j * a.tr) * Elem<DT>::kBytes
               : static_cast<const char*>(a.dr) +
                     (static_cast<int64_t>(b) * a.ds + static_cast<int64_t>(j - nt) * a.drr) * Elem<DT>::kBytes;
    ArgmaxPick pk;
    stream_row<DT, kUnroll>(rowp, v0, v1, pk);
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

// Stream rows of sequence b: target rows 0..n_b, then drafter rows
// 0..n_b-1; none for an invalid draft length.
__device__ __forceinline__ int sample_count(const SampleArgs& a, int b) {
  bool bad;
  const int n = draft_count(a.draft_len, b, a.K, bad);
  return bad ? 0 : 2 * n + 1;
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_sample_rows(SampleArgs a) {
  __shared__ int s_pre[kSeqBlocks + 1];
  __shared__ int s_w[kWaves];
  auto count = [&](int b) { return sample_count(a, b); };
  const SeqDir dir = build_seq_dir(a.B, count, s_pre, s_w);
  if (blockIdx.x == 0) write_seq_starts(dir, s_pre, a.B, count, a.pre);
  const FlatSplit f = make_split(s_pre[dir.nblk], a.V, Elem<DT>::kBytes, a.grid);
  const int64_t g = blockIdx.x;
  if (g >= f.G) return;
  for_pieces(f, g, [&](int64_t r, int64_t v0, int64_t v1) {
    int first, cnt;
    const int b = find_seq(dir, s_pre, static_cast<int>(r), count, first, cnt);
    const int j = static_cast<int>(r) - first;
    const int n = (cnt - 1) / 2;
    const bool target = j <= n;
    const float k = target ? a.kp : a.kq;
    const char* rowp =
        target ? static_cast<const char*>(a.tgt) + (static_cast<int64_t>(b) * a.ts + j * a.tr) * Elem<DT>::kBytes
               : static_cast<const char*>(a.drf) +
                     (static_cast<int64_t>(b) * a.ds + static_cast<int64_t>(j - n - 1) * a.dr) * Elem<DT>::kBytes;
    SoftmaxStats st(k);
    stream_row<DT, kUnroll>(rowp, v0, v1, st);
    float M = st.M, S = st.S;
    wave_stats(M, S, k);
    if (lane_id() == 0) a.stats[(r + g) * kWaves + wave_id()] = make_float2(M, S);
  });
}

// Per-element weight of the draw: residual [p - q]_+ or bonus exp2 weight.
struct DrawWeight {
  float kp, cp, isp, kq, cq, isq;
  int resid;
  __device__ __forceinline__ float operator()(float x, float y) const {
    const float ep = fast_exp2(__builtin_fmaf(x, kp, cp));
    if (!resid) return ep;
    const float eq = fast_exp2(__builtin_fmaf(y, kq, cq));
    return fmaxf(ep * isp - eq * isq, 0.f);
  }
};

struct SumOne {
  DrawWeight w;
  float s = 0.f;
  template <int N>
  __device__ __forceinline__ void group(const float* x, int64_t) {
#pragma unroll
    for (int j = 0; j < N; ++j) s += w(x[j], 0.f);
  }
  template <int U, int W>
  __device__ __forceinline__ void block(const float* x, int64_t, int64_t) { group<U * W>(x, 0); }
};

// Sum of the residual weights over [v0, v1) of two rows read together.
template <int DT>
__device__ float sum_resid(const char* xr, const char* yr, int64_t v0, int64_t v1, const DrawWeight& w) {
  using E = Elem<DT>;
  constexpr int W = E::kVec;
  float s = 0.f;
  const uintptr_t ax = reinterpret_cast<uintptr_t>(xr + v0 * E::kBytes);
  const uintptr_t ay = reinterpret_cast<uintptr_t>(yr + v0 * E::kBytes);
  const int t = threadIdx.x;
  if (((ax ^ ay) & 15u) != 0) {  // rows disagree on alignment: scalar path
    for (int64_t j = v0 + t; j < v1; j += kBlock) s += w(E::load1(xr, j), E::load1(yr, j));
    return s;
  }
  int64_t head = static_cast<int64_t>(((16u - (ax & 15u)) & 15u) / E::kBytes);
  if (head > v1 - v0) head = v1 - v0;
  const int64_t a0 = v0 + head;
  const int64_t nvec = (v1 - a0) / W;
  const int64_t a1 = a0 + nvec * W;
  if (t < head) s += w(E::load1(xr, v0 + t), E::load1(yr, v0 + t));
  const char* xb = xr + a0 * E::kBytes;
  const char* yb = yr + a0 * E::kBytes;
  for (int64_t i = t; i < nvec; i += kBlock) {
    float x[W], y[W];
    E::unpack(load16(xb + i * 16), x);
    E::unpack(load16(yb + i * 16), y);
#pragma unroll
    for (int j = 0; j < W; ++j) s += w(x[j], y[j]);
  }
  if (a1 + t < v1) s += w(E::load1(xr, a1 + t), E::load1(yr, a1 + t));
  return s;
}

// WG-wide exclusive scan of one float per thread in thread order; also
// returns the total.  Contains two barriers.
__device__ __forceinline__ float block_exclusive_scan(float v, float& total, float* s_w) {
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
  for (int j = 0; j < kWaves; ++j) {
    if (j < w) base += s_w[j];
    total += s_w[j];
  }
  __syncthreads();
  return base + inc - v;
}

// Weights of elements [e0, e0 + kDrawPerThread) (0 at or past `end`): the
// thread's loads are all issued before any weight is computed.
template <int DT>
__device__ __forceinline__ void load_weights(const char* xr, const char* yr, int64_t e0, int64_t end,
                                             const DrawWeight& w, float (&wv)[kDrawPerThread]) {
  using E = Elem<DT>;
  constexpr int W = E::kVec;
  constexpr int NV = kDrawPerThread / W;
  const bool vec = (((reinterpret_cast<uintptr_t>(xr + e0 * E::kBytes) |
                      reinterpret_cast<uintptr_t>(yr + e0 * E::kBytes)) & 15u) == 0) &&
                   e0 + kDrawPerThread <= end;
  if (vec) {
    u32x4 rx[NV], ry[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      rx[k] = load16(xr + (e0 + k * W) * E::kBytes);
      if (w.resid) ry[k] = load16(yr + (e0 + k * W) * E::kBytes);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      float x[W], y[W];
      E::unpack(rx[k], x);
      if (w.resid) E::unpack(ry[k], y);
#pragma unroll
      for (int j = 0; j < W; ++j) wv[k * W + j] = w(x[j], w.resid ? y[j] : 0.f);
    }
  } else {
    float x[kDrawPerThread], y[kDrawPerThread];
#pragma unroll
    for (int j = 0; j < kDrawPerThread; ++j) {
      const bool in = e0 + j < end;
      x[j] = in ? E::load1(xr, e0 + j) : 0.f;
      y[j] = in && w.resid ? E::load1(yr, e0 + j) : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kDrawPerThread; ++j) wv[j] = e0 + j < end ? w(x[j], y[j]) : 0.f;
  }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_draw_mass(SampleArgs a) {
  __shared__ float s_Mp[kMaxDraft + 1], s_Sp[kMaxDraft + 1];
  __shared__ float s_Mq[kMaxDraft], s_Sq[kMaxDraft];
  __shared__ float s_red[kWaves];
  __shared__ int s_st, s_h;
  const int NC = a.draw_chunks;
  const int b = blockIdx.x / NC;
  const int c = blockIdx.x % NC;
  const int t = threadIdx.x;

  // ---- the sequence's decision (every group of the sequence) ------------
  bool nbad;
  const int n = draft_count(a.draft_len, b, a.K, nbad);
  const int budget = a.budget ? a.budget[b] : INT_MAX;
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
  if (!nbad) {
    // Stream rows p0..p0+n: target rows 0..n (k = kp); p0+n+1..: drafter
    // rows 0..n-1 (k = kq).
    const int p0 = a.pre[b];
    const FlatSplit f = make_split(a.pre[a.B], a.V, Elem<DT>::kBytes, a.grid);
    combine_rows_stats(
        n + 1, a.stats, a.kp,
        [&](int r, int64_t& first, int64_t& cnt) {
          split_row_slots(f, p0 + r, first, cnt);
          first *= kWaves;
          cnt *= kWaves;
        },
        [&](int r, float M, float S) {
          s_Mp[r] = M; s_Sp[r] = S;
          st |= stats_status(M, S);
        });
    combine_rows_stats(
        n, a.stats, a.kq,
        [&](int r, int64_t& first, int64_t& cnt) {
          split_row_slots(f, p0 + n + 1 + r, first, cnt);
          first *= kWaves;
          cnt *= kWaves;
        },
        [&](int r, float M, float S) {
          s_Mq[r] = M; s_Sq[r] = S;
          st |= stats_status(M, S);
        });
  }
  if (st) atomicOr(&s_st, st);
  __syncthreads();
  if (s_st & SEQ_ERROR_MASK) {
    if (c == 0) {
      int32_t* out = a.out_tokens + static_cast<int64_t>(b) * (a.K + 1);
      for (int i = t; i <= a.K; i += kBlock) out[i] = -1;
      for (int i = t; i < a.K; i += kBlock) {
        const int64_t o = static_cast<int64_t>(b) * a.K + i;
        if (a.p_draft) a.p_draft[o] = 0.f;
        if (a.q_draft) a.q_draft[o] = 0.f;
        if (a.alpha) a.alpha[o] = 0.f;
      }
      if (t == 0) {
        a.accept_len[b] = -1;
        a.num_out[b] = 0;
        if (a.residual_mass) a.residual_mass[b] = 0.f;
        if (a.status) a.status[b] = s_st;
        a.rec[b].status = s_st;
      }
    }
    return;
  }
  // Acceptance tests: accept d_i iff u_i * q_i(d_i) < p~_i(d_i).
  const float lam = a.lam, oml = 1.f - a.lam;
  int qz = 0;
  for (int i = t; i < a.K; i += kBlock) {
    float p = 0.f, q = 0.f, al = 0.f;
    if (i < n) {
      const int di = d[i];
      const char* xr = static_cast<const char*>(a.tgt) + (b * a.ts + i * a.tr) * Elem<DT>::kBytes;
      const char* yr = static_cast<const char*>(a.drf) + (b * a.ds + i * a.dr) * Elem<DT>::kBytes;
      const float x = Elem<DT>::load1(xr, di);
      const float y = Elem<DT>::load1(yr, di);
      p = fast_exp2(__builtin_fmaf(x, a.kp, -s_Mp[i] * a.kp)) / s_Sp[i];
      q = fast_exp2(__builtin_fmaf(y, a.kq, -s_Mq[i] * a.kq)) / s_Sq[i];
      const float pt = oml * p + lam * q;
      const float u = a.u_accept[static_cast<int64_t>(b) * a.K + i];
      if (q == 0.f && pt > 0.f) qz = 1;
      al = q > 0.f ? fminf(1.f, pt / q) : (pt > 0.f ? 1.f : 0.f);
      if (!(u * q < pt)) atomicMin(&s_h, i);
    }
    if (c == 0) {
      const int64_t o = static_cast<int64_t>(b) * a.K + i;
      if (a.p_draft) a.p_draft[o] = p;
      if (a.q_draft) a.q_draft[o] = q;
      if (a.alpha) a.alpha[o] = al;
    }
  }
  if (qz) atomicOr(&s_st, SEQ_Q_ZERO);
  __syncthreads();
  const int h = s_h;
  const bool resid = h < n;
  const char* xr = static_cast<const char*>(a.tgt) + (b * a.ts + static_cast<int64_t>(h) * a.tr) * Elem<DT>::kBytes;
  const char* yr = resid
      ? static_cast<const char*>(a.drf) + (b * a.ds + static_cast<int64_t>(h) * a.dr) * Elem<DT>::kBytes
      : xr;
  DrawWeight w;
  w.kp = a.kp; w.cp = -s_Mp[h] * a.kp; w.isp = 1.f / s_Sp[h];
  w.kq = a.kq; w.cq = resid ? -s_Mq[h] * a.kq : 0.f; w.isq = resid ? 1.f / s_Sq[h] : 1.f;
  w.resid = resid ? 1 : 0;

  // ---- this group's chunk of the draw mass ------------------------------
  {
    const int64_t v0 = static_cast<int64_t>(c) * a.draw_chunk;
    const int64_t v1 = v0 + a.draw_chunk < a.V ? v0 + a.draw_chunk : a.V;
    float s;
    if (resid) {
      s = sum_resid<DT>(xr, yr, v0, v1, w);
    } else {
      SumOne op{w};
      stream_row<DT, kUnroll>(xr, v0, v1, op);
      s = op.s;
    }
    s = block_sum(s, s_red);
    if (t == 0) a.dsum[static_cast<int64_t>(b) * NC + c] = s;
  }
  if (c == 0 && t == 0) {
    DrawRecord r;
    r.status = s_st;
    r.h = h;
    r.resid = resid ? 1 : 0;
    r.cp = w.cp; r.isp = w.isp;
    r.cq = w.cq; r.isq = w.isq;
    r.u = a.u_resample[static_cast<int64_t>(b) * (a.K + 1) + h];
    a.rec[b] = r;
  }
}


// One group per sequence: find the token whose running mass first exceeds
// u * Z (vocabulary order), then assemble the outputs.
template <int DT>
__global__ __launch_bounds__(kBlock) void k_draw_select(SampleArgs a) {
  __shared__ float s_dsum[kMaxDrawChunks];
  __shared__ float s_red[kWaves], s_w[kWaves];
  __shared__ int s_pick, s_lastpos, s_a;
  const int NC = a.draw_chunks;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const DrawRecord rec = a.rec[b];
  if (rec.status & SEQ_ERROR_MASK) return;          // outputs already written
  int status = rec.status;
  const int h = rec.h;
  bool resid = rec.resid != 0;
  const int32_t* d = a.draft_tokens + static_cast<int64_t>(b) * a.K;
  const int budget = a.budget ? a.budget[b] : INT_MAX;
  const char* xr = static_cast<const char*>(a.tgt) + (b * a.ts + static_cast<int64_t>(h) * a.tr) * Elem<DT>::kBytes;
  const char* yr = resid
      ? static_cast<const char*>(a.drf) + (b * a.ds + static_cast<int64_t>(h) * a.dr) * Elem<DT>::kBytes
      : xr;
  DrawWeight w;
  w.kp = a.kp; w.cp = rec.cp; w.isp = rec.isp;
  w.kq = a.kq; w.cq = rec.cq; w.isq = rec.isq;
  w.resid = rec.resid;

  // ---- locate u * Z in vocabulary order ----------------------------------
  for (int k = t; k < NC; k += kBlock) s_dsum[k] = a.dsum[static_cast<int64_t>(b) * NC + k];
  __syncthreads();
  float Z = 0.f;
  for (int k = 0; k < NC; ++k) Z += s_dsum[k];
  const float Zres = resid ? Z : 0.f;
  if (resid && !(Z > 0.f)) {
    // Residual mass vanished in float32 (p == q up to rounding): draw from p
    // with the same uniform instead, and flag it.
    status |= SEQ_Z_ZERO;
    resid = false;
    w.resid = 0;
    for (int k = 0; k < NC; ++k) {
      const int64_t v0 = static_cast<int64_t>(k) * a.draw_chunk;
      const int64_t v1 = v0 + a.draw_chunk < a.V ? v0 + a.draw_chunk : a.V;
      float s = 0.f;
      for (int64_t j = v0 + t; j < v1; j += kBlock) s += w(Elem<DT>::load1(xr, j), 0.f);
      s = block_sum(s, s_red);
      __syncthreads();
      if (t == 0) s_dsum[k] = s;
      __syncthreads();
    }
    Z = 0.f;
    for (int k = 0; k < NC; ++k) Z += s_dsum[k];
  }
  const float target = rec.u * Z;
  // Chunk whose running mass first exceeds u*Z (positive chunks only).
  int cs = -1, clast = -1;
  float base = 0.f, run = 0.f;
  for (int k = 0; k < NC; ++k) {
    if (!(s_dsum[k] > 0.f)) continue;
    clast = k;
    if (run + s_dsum[k] > target) { cs = k; base = run; break; }
    run += s_dsum[k];
  }
  if (cs < 0) {  // rounding: u*Z at or past the total -> last positive chunk
    cs = clast >= 0 ? clast : 0;
    base = run - (clast >= 0 ? s_dsum[clast] : 0.f);
  }
  if (t == 0) { s_pick = INT_MAX; s_lastpos = -1; }
  __syncthreads();
  // Thread t holds elements [c0 + t*P, c0 + (t+1)*P) of the chunk (P =
  // kDrawPerThread): their weights stay in registers for the scan.
  const int64_t c0 = static_cast<int64_t>(cs) * a.draw_chunk;
  const int64_t c1 = c0 + a.draw_chunk < a.V ? c0 + a.draw_chunk : a.V;
  const int64_t e0 = c0 + static_cast<int64_t>(t) * kDrawPerThread;
  float wv[kDrawPerThread];
  load_weights<DT>(xr, yr, e0, c1, w, wv);
  float loc = 0.f;
  int lastpos = -1;
#pragma unroll
  for (int j = 0; j < kDrawPerThread; ++j) {
    loc += wv[j];
    if (wv[j] > 0.f) lastpos = static_cast<int>(e0 + j);
  }
  float tot;
  const float start = base + block_exclusive_scan(loc, tot, s_w);
  if (lastpos >= 0) atomicMax(&s_lastpos, lastpos);
  if (loc > 0.f && start + loc > target) {
    float r = start;
    int found = INT_MAX;
#pragma unroll
    for (int j = 0; j < kDrawPerThread; ++j) {
      r += wv[j];
      if (found == INT_MAX && wv[j] > 0.f && r > target) found = static_cast<int>(e0 + j);
    }
    if (found != INT_MAX) atomicMin(&s_pick, found);
  }
  __syncthreads();
  const int tok = s_pick != INT_MAX ? s_pick : s_lastpos;

  // ---- output assembly: C = (d_1..d_h, c), then the ending condition ----
  const int A = h + 1;
  if (t == 0) s_a = A < budget ? A : budget;
  __syncthreads();
  if (a.eos >= 0) {
    for (int i = t; i < A; i += kBlock) {
      const int ci = i < h ? d[i] : tok;
      if (ci == a.eos) atomicMin(&s_a, i + 1);
    }
  }
  __syncthreads();
  const int an = s_a;
  int32_t* out = a.out_tokens + static_cast<int64_t>(b) * (a.K + 1);
  for (int i = t; i <= a.K; i += kBlock) out[i] = i < an ? (i < h ? d[i] : tok) : -1;
  if (t == 0) {
    a.accept_len[b] = h;
    a.num_out[b] = an;
    // Mass of [p~ - q]_+ = (1 - lambda) [p - q]_+: the rejection probability.
    if (a.residual_mass) a.residual_mass[b] = Zres * (1.f - a.lam);
    if (a.status) a.status[b] = status;
  }
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
  return launch(bf ? fn(k_sample_rows<DT_BF16>) : fn(k_sample_rows<DT_F32>), a.grid, stream, a, ev) &&
         launch(bf ? fn(k_draw_mass<DT_BF16>) : fn(k_draw_mass<DT_F32>),
                static_cast<int64_t>(a.B) * a.draw_chunks, stream, a) &&
         launch(bf ? fn(k_draw_select<DT_BF16>) : fn(k_draw_select<DT_F32>), a.B, stream, a);
}

}  // namespace dbv
