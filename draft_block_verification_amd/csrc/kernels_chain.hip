// Chain verification kernels: greedy match with next-draft retention, and the
// rejection / linear-lenient sampler with its correction or bonus draw.
//
// Greedy  (Packed-SS, Sec. 3.1, Eq. 1-4, Algorithm 1):
//   k_greedy_rows      split-V argmax of every needed target / draft row
//   k_greedy_finalize  per sequence: combine, leading matches h, C, ending
//                      condition a, next draft z_{a+1..W}
// Sampling (Packed-SS, Algorithm 2; Two Tradeoffs, Theorem 1, Algorithm 1):
//   k_sample_rows      split-V online softmax statistics (M, S) per row
//   k_sample_decide    per sequence: p(d), q(d), the acceptance tests, h,
//                      which row the draw uses
//   k_draw_partial     split-V mass of [p - q]_+ (or of p for the bonus)
//   k_draw_select      per sequence: chunk holding u*Z, in-chunk scan in
//                      vocabulary order, output assembly
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

__device__ __forceinline__ float2 pack_pick(float v, int idx, int nan) {
  return make_float2(nan ? __builtin_nanf("") : v, __int_as_float(idx));
}

// Combine the split partials of one argmax row.  Returns the index and ORs
// the row's status into st.
__device__ __forceinline__ int combine_pick(const float2* part, int split, int& st) {
  float v = -kInf;
  int idx = -1;
  int nan = 0;
  for (int s = 0; s < split; ++s) {
    const float2 p = part[s];
    const int i2 = __float_as_int(p.y);
    if (p.x != p.x) { nan = 1; continue; }
    if (pick_better(p.x, i2, v, idx)) { v = p.x; idx = i2; }
  }
  if (nan) st |= SEQ_NONFINITE;
  else st |= max_status(v);
  return idx;
}

// ================================================================ greedy ===

template <int DT>
__global__ __launch_bounds__(kBlock) void k_greedy_rows(GreedyArgs a) {
  __shared__ float s_v[kWaves];
  __shared__ int s_i[kWaves], s_n[kWaves];
  const int64_t gid = blockIdx.x;
  const int64_t row = gid / a.split;
  const int sp = static_cast<int>(gid % a.split);
  const int64_t ntr = static_cast<int64_t>(a.B) * (a.K + 1);
  const char* rowp;
  if (row < ntr) {
    const int b = static_cast<int>(row / (a.K + 1));
    const int i = static_cast<int>(row % (a.K + 1));
    bool bad;
    const int n = draft_count(a.draft_len, b, a.K, bad);
    if (bad || i > n) return;  // row is not read
    rowp = static_cast<const char*>(a.tgt) + (b * a.ts + i * a.tr) * Elem<DT>::kBytes;
  } else {
    const int64_t r = row - ntr;
    const int b = static_cast<int>(r / a.W);
    const int j = static_cast<int>(r % a.W);
    rowp = static_cast<const char*>(a.dr) + (b * a.ds + j * a.drr) * Elem<DT>::kBytes;
  }
  const int64_t v0 = static_cast<int64_t>(sp) * a.chunk;
  const int64_t v1 = v0 + a.chunk < a.V ? v0 + a.chunk : a.V;
  ArgmaxPick pk;
  stream_row<DT, kUnroll>(rowp, v0, v1, pk);
  const int64_t idx = resolve_argmax<DT>(pk, v1, [&](int64_t j) { return Elem<DT>::load1(rowp, j); });
  float v = pk.best;
  int ii = static_cast<int>(idx);
  int nan = pk.nan ? 1 : 0;
  block_argmax(v, ii, nan, s_v, s_i, s_n);
  if (threadIdx.x == 0) a.part[gid] = pack_pick(v, ii, nan);
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
  const int64_t ntr = static_cast<int64_t>(a.B) * (a.K + 1);
  if (!nbad) {
    for (int i = t; i <= n; i += kBlock)
      s_v[i] = combine_pick(a.part + (static_cast<int64_t>(b) * (a.K + 1) + i) * a.split, a.split, st);
  }
  for (int j = t; j < a.W; j += kBlock)
    s_z[j] = combine_pick(a.part + (ntr + static_cast<int64_t>(b) * a.W + j) * a.split, a.split, st);
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

template <int DT>
__global__ __launch_bounds__(kBlock) void k_sample_rows(SampleArgs a) {
  __shared__ float s_m[kWaves], s_s[kWaves];
  const int64_t gid = blockIdx.x;
  const int64_t row = gid / a.split;
  const int sp = static_cast<int>(gid % a.split);
  const int64_t ntr = static_cast<int64_t>(a.B) * (a.K + 1);
  const char* rowp;
  float k;
  bool bad;
  if (row < ntr) {
    const int b = static_cast<int>(row / (a.K + 1));
    const int i = static_cast<int>(row % (a.K + 1));
    const int n = draft_count(a.draft_len, b, a.K, bad);
    if (bad || i > n) return;
    rowp = static_cast<const char*>(a.tgt) + (b * a.ts + i * a.tr) * Elem<DT>::kBytes;
    k = a.kp;
  } else {
    const int64_t r = row - ntr;
    const int b = static_cast<int>(r / a.K);
    const int i = static_cast<int>(r % a.K);
    const int n = draft_count(a.draft_len, b, a.K, bad);
    if (bad || i >= n) return;
    rowp = static_cast<const char*>(a.drf) + (b * a.ds + i * a.dr) * Elem<DT>::kBytes;
    k = a.kq;
  }
  const int64_t v0 = static_cast<int64_t>(sp) * a.chunk;
  const int64_t v1 = v0 + a.chunk < a.V ? v0 + a.chunk : a.V;
  SoftmaxStats st(k);
  stream_row<DT, kUnroll>(rowp, v0, v1, st);
  float M = st.M, S = st.S;
  block_stats(M, S, k, s_m, s_s);
  if (threadIdx.x == 0) a.stats[gid] = make_float2(M, S);
}

__device__ __forceinline__ void combine_stats(const float2* part, int split, float k, float& M, float& S) {
  M = -kInf;
  S = 0.f;
  for (int s = 0; s < split; ++s) stats_merge(M, S, part[s].x, part[s].y, k);
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_sample_decide(SampleArgs a) {
  __shared__ float s_Mp[kMaxDraft + 1], s_Sp[kMaxDraft + 1];
  __shared__ float s_Mq[kMaxDraft], s_Sq[kMaxDraft];
  __shared__ int s_st, s_h;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  bool nbad;
  const int n = draft_count(a.draft_len, b, a.K, nbad);
  const int budget = a.budget ? a.budget[b] : INT_MAX;
  if (t == 0) {
    s_st = (nbad || budget < 0) ? SEQ_BAD_INPUT : 0;
    s_h = n;
  }
  __syncthreads();
  const int32_t* d = a.draft_tokens + static_cast<int64_t>(b) * a.K;
  const int64_t ntr = static_cast<int64_t>(a.B) * (a.K + 1);
  int st = 0;
  for (int i = t; i < n; i += kBlock) {
    const int di = d[i];
    if (di < 0 || di >= a.V) st |= SEQ_BAD_INPUT;
  }
  if (!nbad) {
    for (int i = t; i <= n; i += kBlock) {
      float M, S;
      combine_stats(a.stats + (static_cast<int64_t>(b) * (a.K + 1) + i) * a.split, a.split, a.kp, M, S);
      s_Mp[i] = M; s_Sp[i] = S;
      st |= stats_status(M, S);
    }
    for (int i = t; i < n; i += kBlock) {
      float M, S;
      combine_stats(a.stats + (ntr + static_cast<int64_t>(b) * a.K + i) * a.split, a.split, a.kq, M, S);
      s_Mq[i] = M; s_Sq[i] = S;
      st |= stats_status(M, S);
    }
  }
  if (st) atomicOr(&s_st, st);
  __syncthreads();
  int status = s_st;
  DrawRecord* rec = a.rec + b;
  if (status & SEQ_ERROR_MASK) {
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
      if (a.status) a.status[b] = status;
      rec->kind = -1;
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
      const bool acc = u * q < pt;
      if (q == 0.f && pt > 0.f) qz = 1;
      al = q > 0.f ? fminf(1.f, pt / q) : (pt > 0.f ? 1.f : 0.f);
      if (!acc) atomicMin(&s_h, i);
    }
    const int64_t o = static_cast<int64_t>(b) * a.K + i;
    if (a.p_draft) a.p_draft[o] = p;
    if (a.q_draft) a.q_draft[o] = q;
    if (a.alpha) a.alpha[o] = al;
  }
  if (qz) atomicOr(&s_st, SEQ_Q_ZERO);
  __syncthreads();
  if (t == 0) {
    const int h = s_h;
    status = s_st;
    rec->kind = h < n ? 0 : 1;
    rec->row = h;
    rec->Mp = s_Mp[h]; rec->kp = a.kp; rec->Sp = s_Sp[h];
    rec->Mq = h < n ? s_Mq[h] : 0.f; rec->kq = a.kq; rec->Sq = h < n ? s_Sq[h] : 1.f;
    rec->u = a.u_resample[static_cast<int64_t>(b) * (a.K + 1) + h];
    rec->pad[0] = status;
    a.accept_len[b] = h;
  }
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

__device__ __forceinline__ DrawWeight make_weight(const DrawRecord& r, bool resid) {
  DrawWeight w;
  w.kp = r.kp; w.cp = -r.Mp * r.kp; w.isp = 1.f / r.Sp;
  w.kq = r.kq; w.cq = -r.Mq * r.kq; w.isq = 1.f / r.Sq;
  w.resid = resid ? 1 : 0;
  return w;
}

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

template <int DT>
__global__ __launch_bounds__(kBlock) void k_draw_partial(SampleArgs a) {
  __shared__ float s_sum[kWaves];
  const int b = blockIdx.x / a.draw_chunks;
  const int c = blockIdx.x % a.draw_chunks;
  const DrawRecord r = a.rec[b];
  if (r.kind < 0) return;
  const int64_t v0 = static_cast<int64_t>(c) * a.draw_chunk;
  const int64_t v1 = v0 + a.draw_chunk < a.V ? v0 + a.draw_chunk : a.V;
  const char* xr = static_cast<const char*>(a.tgt) + (b * a.ts + static_cast<int64_t>(r.row) * a.tr) * Elem<DT>::kBytes;
  float s;
  if (r.kind == 0) {
    const char* yr = static_cast<const char*>(a.drf) + (b * a.ds + static_cast<int64_t>(r.row) * a.dr) * Elem<DT>::kBytes;
    s = sum_resid<DT>(xr, yr, v0, v1, make_weight(r, true));
  } else {
    SumOne op{make_weight(r, false)};
    stream_row<DT, kUnroll>(xr, v0, v1, op);
    s = op.s;
  }
  s = block_sum(s, s_sum);
  if (threadIdx.x == 0) a.dsum[static_cast<int64_t>(b) * a.draw_chunks + c] = s;
}

// WG-wide exclusive scan of one float per thread (fixed order); also returns
// the total.  Thread order is element order.
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

template <int DT>
__global__ __launch_bounds__(kBlock) void k_draw_select(SampleArgs a) {
  __shared__ float s_dsum[kMaxSplit];
  __shared__ float s_w[kWaves];
  __shared__ int s_pick, s_last, s_a;
  __shared__ float s_red[kWaves];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  DrawRecord r = a.rec[b];
  if (r.kind < 0) return;
  int status = r.pad[0];
  const char* xr = static_cast<const char*>(a.tgt) + (b * a.ts + static_cast<int64_t>(r.row) * a.tr) * Elem<DT>::kBytes;
  const char* yr = r.kind == 0
      ? static_cast<const char*>(a.drf) + (b * a.ds + static_cast<int64_t>(r.row) * a.dr) * Elem<DT>::kBytes
      : xr;
  const int NC = a.draw_chunks;
  for (int c = t; c < NC; c += kBlock) s_dsum[c] = a.dsum[static_cast<int64_t>(b) * NC + c];
  __syncthreads();
  float Z = 0.f;
  for (int c = 0; c < NC; ++c) Z += s_dsum[c];
  bool resid = r.kind == 0;
  const float Zres = resid ? Z : 0.f;
  if (resid && !(Z > 0.f)) {
    // Residual mass vanished in float32 (p == q up to rounding): draw from p
    // with the same uniform instead, and flag it.
    status |= SEQ_Z_ZERO;
    resid = false;
    const DrawWeight w = make_weight(r, false);
    for (int c = 0; c < NC; ++c) {
      const int64_t v0 = static_cast<int64_t>(c) * a.draw_chunk;
      const int64_t v1 = v0 + a.draw_chunk < a.V ? v0 + a.draw_chunk : a.V;
      float s = 0.f;
      for (int64_t j = v0 + t; j < v1; j += kBlock) s += w(Elem<DT>::load1(xr, j), 0.f);
      s = block_sum(s, s_red);
      __syncthreads();
      if (t == 0) s_dsum[c] = s;
      __syncthreads();
    }
    Z = 0.f;
    for (int c = 0; c < NC; ++c) Z += s_dsum[c];
  }
  const DrawWeight w = make_weight(r, resid);
  const float target = r.u * Z;
  // Chunk whose running mass first exceeds u*Z (positive chunks only).
  int cs = -1, clast = -1;
  float base = 0.f, run = 0.f;
  for (int c = 0; c < NC; ++c) {
    if (!(s_dsum[c] > 0.f)) continue;
    clast = c;
    if (run + s_dsum[c] > target) { cs = c; base = run; break; }
    run += s_dsum[c];
  }
  if (cs < 0) {  // rounding: u*Z at or past the total -> last positive chunk
    cs = clast >= 0 ? clast : 0;
    base = run - (clast >= 0 ? s_dsum[clast] : 0.f);
  }
  // Scan chunk cs in vocabulary order, 8 elements per thread per tile.
  if (t == 0) { s_pick = INT_MAX; s_last = -1; }
  __syncthreads();
  const int64_t c0 = static_cast<int64_t>(cs) * a.draw_chunk;
  const int64_t c1 = c0 + a.draw_chunk < a.V ? c0 + a.draw_chunk : a.V;
  constexpr int P = 8;
  for (int64_t tile = c0; tile < c1; tile += static_cast<int64_t>(kBlock) * P) {
    float wv[P];
    float tot = 0.f;
    int lastpos = -1;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int64_t e = tile + static_cast<int64_t>(t) * P + j;
      wv[j] = e < c1 ? w(Elem<DT>::load1(xr, e), Elem<DT>::load1(yr, e)) : 0.f;
      tot += wv[j];
      if (wv[j] > 0.f) lastpos = static_cast<int>(e);
    }
    float tile_total;
    float runv = base + block_exclusive_scan(tot, tile_total, s_w);
    int found = INT_MAX;
#pragma unroll
    for (int j = 0; j < P; ++j) {
      runv += wv[j];
      if (found == INT_MAX && wv[j] > 0.f && runv > target)
        found = static_cast<int>(tile + static_cast<int64_t>(t) * P + j);
    }
    if (found != INT_MAX) atomicMin(&s_pick, found);
    if (lastpos >= 0) atomicMax(&s_last, lastpos);
    __syncthreads();
    if (s_pick != INT_MAX) break;
    base += tile_total;
    __syncthreads();
  }
  __syncthreads();
  const int c = s_pick != INT_MAX ? s_pick : s_last;

  // Output assembly: C = (d_1..d_h, c), then the ending condition.
  const int h = r.row;
  const int32_t* d = a.draft_tokens + static_cast<int64_t>(b) * a.K;
  const int budget = a.budget ? a.budget[b] : INT_MAX;
  const int A = h + 1;
  if (t == 0) s_a = A < budget ? A : budget;
  __syncthreads();
  if (a.eos >= 0) {
    for (int i = t; i < A; i += kBlock) {
      const int ci = i < h ? d[i] : c;
      if (ci == a.eos) atomicMin(&s_a, i + 1);
    }
  }
  __syncthreads();
  const int an = s_a;
  int32_t* out = a.out_tokens + static_cast<int64_t>(b) * (a.K + 1);
  for (int i = t; i <= a.K; i += kBlock) out[i] = i < an ? (i < h ? d[i] : c) : -1;
  if (t == 0) {
    a.num_out[b] = an;
    // Mass of [p~ - q]_+ = (1 - lambda) [p - q]_+: the rejection probability.
    if (a.residual_mass) a.residual_mass[b] = Zres * (1.f - a.lam);
    if (a.status) a.status[b] = status;
  }
}

// ============================================================== launches ===

#define DBV_LAUNCH(kern, grid, stream, arg)                                         \
  do {                                                                               \
    if ((grid) > 0) hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)),      \
                                       dim3(kBlock), 0, (stream), (arg));            \
    if (hipGetLastError() != hipSuccess) return false;                               \
  } while (0)

static void mark(hipEvent_t e, hipStream_t s) {
  if (e) (void)hipEventRecord(e, s);
}

bool launch_greedy(const GreedyArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev) {
  const int64_t grid = static_cast<int64_t>(a.B) * ((a.K + 1) + a.W) * a.split;
  mark(ev.begin, stream);
  if (dtype == DT_BF16) DBV_LAUNCH(k_greedy_rows<DT_BF16>, grid, stream, a);
  else DBV_LAUNCH(k_greedy_rows<DT_F32>, grid, stream, a);
  mark(ev.end, stream);
  DBV_LAUNCH(k_greedy_finalize, a.B, stream, a);
  return true;
}

bool launch_sample(const SampleArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev) {
  const int64_t grid = static_cast<int64_t>(a.B) * ((a.K + 1) + a.K) * a.split;
  const int64_t dgrid = static_cast<int64_t>(a.B) * a.draw_chunks;
  mark(ev.begin, stream);
  if (dtype == DT_BF16) DBV_LAUNCH(k_sample_rows<DT_BF16>, grid, stream, a);
  else DBV_LAUNCH(k_sample_rows<DT_F32>, grid, stream, a);
  mark(ev.end, stream);
  if (dtype == DT_BF16) {
    DBV_LAUNCH(k_sample_decide<DT_BF16>, a.B, stream, a);
    DBV_LAUNCH(k_draw_partial<DT_BF16>, dgrid, stream, a);
    DBV_LAUNCH(k_draw_select<DT_BF16>, a.B, stream, a);
  } else {
    DBV_LAUNCH(k_sample_decide<DT_F32>, a.B, stream, a);
    DBV_LAUNCH(k_draw_partial<DT_F32>, dgrid, stream, a);
    DBV_LAUNCH(k_draw_select<DT_F32>, a.B, stream, a);
  }
  return true;
}

}  // namespace dbv
