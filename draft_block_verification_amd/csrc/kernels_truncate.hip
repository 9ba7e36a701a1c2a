// Top-k / top-p truncation of drafter rows into stored sparse form
// ("One Call Ahead: Packed Self-Speculative Decoding with Diffusion
// Drafting", Sec. 3.2: only the nonzero entries of a truncated drafter
// distribution need storing).
//
//   k_truncate  one group of kTB threads per row (b, i), i < n_b:
//     1. one streaming pass: each thread keeps its three largest logits (a
//        median-of-three cascade per element), the start of the contiguous
//        group of each (its occurrence among the equal logits of that group
//        follows from the entries above it), and the largest logit it
//        dropped; the row's NaN / +inf check comes from the thread maxima;
//     2. tau = the smallest, over the waves, of each wave's ceil(k/16)-th
//        largest thread maximum: at least k logits are >= tau;
//     3. the kept entries >= tau are the candidates, each with its place
//        (group start, occurrence), which orders equal logits as their
//        token ids do; with at most kRankCand candidates each counts its rank by
//        (logit descending, place ascending) against the others, else a
//        radix select in LDS gives the k-th largest key and the place
//        cut-off (ties go to the lower ids); the k kept find their token
//        ids inside their groups;
//     4. if some thread dropped a logit >= that k-th key, the candidates may
//        miss a kept token: the row is read again and every logit >= tau
//        collected (and if those overflow LDS, a radix select over the
//        whole row, one pass per 8-bit digit, takes their place);
//     5. the k kept sorted by (logit descending, id ascending) (already in
//        rank order on the counting path); weights exp((x - x_max) / T);
//        the shortest prefix whose mass reaches p of the total (all k for
//        p = 1), renormalised and written in order (by one wave for k <=
//        64).
#include "dbv_device.h"
#include "dbv_launch.h"

namespace dbv {

// Order-preserving key of a logit: larger logits get larger keys (equal
// logits equal keys).  bf16
// logits have zero low halves, so their keys are the upper 16 bits.
template <int DT>
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;   // -0 ranks with +0
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return DT == DT_BF16 ? (k >> 16) : k;
}

template <int DT>
constexpr int key_bits() {
  return DT == DT_BF16 ? 16 : 32;
}

constexpr int kTB = 1024;          // threads per row
constexpr int kTW = kTB / 64;      // waves per row
constexpr int kTruncCand = 4096;   // LDS candidates (>= 3 per thread)
constexpr int kRankCand = 256;     // candidates ranked by counting (else radix select)
static_assert(kTruncCand >= 3 * kTB, "every thread's three kept logits fit");

struct TruncLds {
  int hist[256];
  int bad, digit, above, n, keep, nc, chunk;
  uint32_t tau_key, drop_key;
  uint32_t wtau[kTW];
  __align__(16) uint64_t rk[kRankCand + 2];   // ranked candidates: key, ~place
  float cx[kTruncCand];            // candidates: logit and token id
  int cid[kTruncCand];
  uint32_t ckey[kMaxNnz];          // the kept k
  int cidx[kMaxNnz];
  float kx[kMaxNnz];
  int sidx[kMaxNnz];
  float sx[kMaxNnz];
  float fw[kTW];
  float sum;
};

// The three largest logits of a thread in order (equal logits: the earlier
// first), each with the start index of its contiguous group, and the
// largest logit that fell out.  The maximum propagates NaN (the row check);
// a row with NaN never reads the others.  The occurrence of an entry among
// the equal logits of its group is not tracked while streaming: the earlier
// equal logits of that group rank above it, so they are the entries before
// it with the same logit and group (occurrence1, occurrence2).
struct Top3Op {
  float v0 = -kInf, v1 = -kInf, v2 = -kInf;
  int g0 = -1, g1 = -1, g2 = -1;
  float drop = -kInf;

  template <int N>
  __device__ __forceinline__ void group(const float* x, int64_t idx0) {
    // Work on copies: every select below is between values, never between
    // fields (a select between fields would become a select of addresses
    // and keep the tracker out of registers).
    const float o0 = v0, o1 = v1, o2 = v2;
    const int h0 = g0, h1 = g1, h2 = g2;
    // A fourth slot under the three: the largest logit that fell out is
    // the thread's fourth largest.
    float n0 = o0, n1 = o1, n2 = o2, n3 = drop;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      n3 = __builtin_amdgcn_fmed3f(x[j], n2, n3);
      n2 = __builtin_amdgcn_fmed3f(x[j], n1, n2);
      n1 = __builtin_amdgcn_fmed3f(x[j], n0, n1);
      n0 = fmaxp(n0, x[j]);
    }
    drop = n3;
    // The new list is the stable merge of the old list with the group's
    // logits (old entries first on equal logits): walk it, matching old
    // entries in order; the rest come from this group.
    const int gi = static_cast<int>(idx0);
    const bool m0 = n0 == o0;                    // slot 0: old entry 0?
    const float p1 = m0 ? o1 : o0;               // next old entry
    const bool m1 = n1 == p1;
    const int io = (m0 ? 1 : 0) + (m1 ? 1 : 0);  // old entries used so far
    const float p2 = io == 2 ? o2 : io == 1 ? o1 : o0;
    const bool m2 = n2 == p2;
    v0 = n0; v1 = n1; v2 = n2;
    g0 = m0 ? h0 : gi;
    g1 = m1 ? (m0 ? h1 : h0) : gi;
    g2 = m2 ? (io == 2 ? h2 : io == 1 ? h1 : h0) : gi;
  }
  template <int U, int W>
  __device__ __forceinline__ void block(const float* x, int64_t idx0, int64_t ustride) {
#pragma unroll
    for (int u = 0; u < U; ++u) group<W>(x + u * W, idx0 + u * ustride);
  }
  // Occurrences of entries 1 and 2 among the equal logits of their groups
  // (entry 0's is 0).
  __device__ __forceinline__ int occurrence1() const { return (v1 == v0 && g1 == g0) ? 1 : 0; }
  __device__ __forceinline__ int occurrence2() const {
    return (v2 == v1 && g2 == g1) ? occurrence1() + 1 : 0;
  }
};

// Candidates: every logit >= tau goes to LDS while there is room; the count
// goes on regardless.
template <int DT>
struct CandOp {
  TruncLds& s;
  uint32_t tkey;
  template <int N>
  __device__ __forceinline__ void group(const float* x, int64_t idx0) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      if (order_key<DT>(x[j]) >= tkey) {
        const int slot = atomicAdd(&s.nc, 1);
        if (slot < kTruncCand) {
          s.cx[slot] = x[j];
          s.cid[slot] = static_cast<int>(idx0 + j);
        }
      }
    }
  }
  template <int U, int W>
  __device__ __forceinline__ void block(const float* x, int64_t idx0, int64_t ustride) {
#pragma unroll
    for (int u = 0; u < U; ++u) group<W>(x + u * W, idx0 + u * ustride);
  }
};

// Histogram of 8-bit digits of the keys (or of the token ids) that match a
// prefix, over one pass of the row (the fallback when tau lets too many
// logits through).
template <int DT>
struct HistOp {
  TruncLds& s;
  uint32_t prefix, mask;
  int shift;
  bool by_index;       // digits of the token id among keys equal to `prefix_key`
  uint32_t prefix_key;
  template <int N>
  __device__ __forceinline__ void group(const float* x, int64_t idx0) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const uint32_t key = order_key<DT>(x[j]);
      if (by_index) {
        const uint32_t id = static_cast<uint32_t>(idx0 + j);
        if (key == prefix_key && (id & mask) == prefix) atomicAdd(&s.hist[(id >> shift) & 255u], 1);
      } else if ((key & mask) == prefix) {
        atomicAdd(&s.hist[(key >> shift) & 255u], 1);
      }
    }
  }
  template <int U, int W>
  __device__ __forceinline__ void block(const float* x, int64_t idx0, int64_t ustride) {
#pragma unroll
    for (int u = 0; u < U; ++u) group<W>(x + u * W, idx0 + u * ustride);
  }
};

// Collects the kept tokens: keys above the cut, and keys equal to it at ids
// up to `id_cut`.
__device__ __forceinline__ void keep_token(TruncLds& s, uint32_t key, float x, int id, uint32_t kth,
                                           uint32_t id_cut) {
  if (key > kth || (key == kth && static_cast<uint32_t>(id) <= id_cut)) {
    const int slot = atomicAdd(&s.n, 1);
    if (slot < kMaxNnz) {
      s.ckey[slot] = key;
      s.cidx[slot] = id;
      s.kx[slot] = x;
    }
  }
}

template <int DT>
struct CollectOp {
  TruncLds& s;
  uint32_t kth;
  uint32_t id_cut;
  template <int N>
  __device__ __forceinline__ void group(const float* x, int64_t idx0) {
#pragma unroll
    for (int j = 0; j < N; ++j) keep_token(s, order_key<DT>(x[j]), x[j], static_cast<int>(idx0 + j), kth, id_cut);
  }
  template <int U, int W>
  __device__ __forceinline__ void block(const float* x, int64_t idx0, int64_t ustride) {
#pragma unroll
    for (int u = 0; u < U; ++u) group<W>(x + u * W, idx0 + u * ustride);
  }
};

// One radix digit: after a histogram pass, the digit (from the top, or from
// the bottom with `ascending`) at which the running count reaches `want`,
// and the count before it.  Wave 0 scans the 256 bins.
__device__ __forceinline__ void pick_digit(TruncLds& s, int want, bool ascending) {
  const int t = threadIdx.x;
  if (t < 64) {
    int c[4];
    int loc = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int bin = t * 4 + q;
      c[q] = s.hist[ascending ? bin : 255 - bin];
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
        const int bin = t * 4 + q;
        s.digit = ascending ? bin : 255 - bin;
        s.above = run;
      }
      run += c[q];
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void clear_hist(TruncLds& s) {
  for (int j = threadIdx.x; j < 256; j += kTB) s.hist[j] = 0;
  if (threadIdx.x == 0) {
    s.digit = 0;
    s.above = 0;
  }
  __syncthreads();
}

// Radix select over a source of (key, id): `hist(prefix, mask, shift,
// by_index, key)` fills s.hist for one digit.  Returns the k-th largest key
// and the id cut-off among the keys equal to it (ties to the lower ids).
template <int KB, class Hist>
__device__ __forceinline__ void radix_select(TruncLds& s, int k, Hist hist, uint32_t& kth, uint32_t& id_cut) {
  uint32_t prefix = 0, mask = 0;
  int want = k;
  for (int shift = KB - 8; shift >= 0; shift -= 8) {
    clear_hist(s);
    hist(prefix, mask, shift, false, 0u);
    __syncthreads();
    pick_digit(s, want, false);
    prefix |= static_cast<uint32_t>(s.digit) << shift;
    mask |= 255u << shift;
    want -= s.above;
    __syncthreads();
  }
  kth = prefix;
  const int ties = want;
  const int eq_count = s.hist[s.digit];
  __syncthreads();
  id_cut = 0xFFFFFFFFu;
  if (ties < eq_count) {
    uint32_t ip = 0, im = 0;
    int iw = ties;
    for (int shift = 24; shift >= 0; shift -= 8) {
      clear_hist(s);
      hist(ip, im, shift, true, kth);
      __syncthreads();
      pick_digit(s, iw, true);
      ip |= static_cast<uint32_t>(s.digit) << shift;
      im |= 255u << shift;
      iw -= s.above;
      __syncthreads();
    }
    id_cut = ip;
  }
}

static_assert(kMaxNnz <= kTB, "one kept entry per thread");

// The token id of a kept logit x at occurrence c of group g: the c-th
// element equal to x in [g, g + W) (a group holds at most W elements; a
// one-element group's logit is its first element).  load_group issues the
// loads of the group's elements, scan_group finds the id in them, so other
// work can run while the loads are in flight.
template <int DT>
__device__ __forceinline__ void load_group(const char* row, int64_t V, int g, float (&y)[Elem<DT>::kVec]) {
#pragma unroll
  for (int j = 0; j < Elem<DT>::kVec; ++j) {
    const int64_t id = static_cast<int64_t>(g) + j;
    y[j] = Elem<DT>::load1(row, id < V ? id : V - 1);
  }
}
template <int DT>
__device__ __forceinline__ int scan_group(int64_t V, int g, int c, float x, const float (&y)[Elem<DT>::kVec]) {
  int seen = 0, hit = -1;
#pragma unroll
  for (int j = 0; j < Elem<DT>::kVec; ++j) {
    const bool eq = static_cast<int64_t>(g) + j < V && y[j] == x;
    if (eq && seen == c && hit < 0) hit = g + j;
    seen += eq ? 1 : 0;
  }
  return hit;
}
template <int DT>
__device__ __forceinline__ int find_in_group(const char* row, int64_t V, int g, int c, float x) {
  float y[Elem<DT>::kVec];
  load_group<DT>(row, V, g, y);
  return scan_group<DT>(V, g, c, x, y);
}

// Wave-wide unsigned maximum by DPP lane moves (identity 0); every lane of
// the wave must be active.  The result is read from lane 63.
template <int C, int R>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), C, R, 0xf, false));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1, 0xf>(v));    // quad_perm 1,0,3,2
  v = max(v, dpp_u32<0x4E, 0xf>(v));    // quad_perm 2,3,0,1
  v = max(v, dpp_u32<0x141, 0xf>(v));   // row_half_mirror
  v = max(v, dpp_u32<0x140, 0xf>(v));   // row_mirror
  v = max(v, dpp_u32<0x142, 0xa>(v));   // row_bcast15 into rows 1, 3
  v = max(v, dpp_u32<0x143, 0xc>(v));   // row_bcast31 into rows 2, 3
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// The kw-th largest of the wave's keys (with multiplicity): kw times the
// wave maximum, each time removing one lane that holds it.
__device__ __forceinline__ uint32_t wave_kth_key(uint32_t key, int kw) {
  const int lane = threadIdx.x & 63;
  uint32_t res = 0;
  for (int it = 0; it < kw; ++it) {
    res = wave_max_u32(key);
    const uint64_t hit = __ballot(key == res);
    if (lane == __ffsll(static_cast<unsigned long long>(hit)) - 1) key = 0;
  }
  return res;
}

// stream_row over [0, V) for a whole group whose waves share the SIMDs
// (several waves each): the waves claim chunks of U vectors per lane from
// s.chunk in turn, instead of fixed strides, so that a wave the SIMD
// arbiter favours takes more chunks and the waves finish together.  Each
// lane's vectors still come in increasing order.  s.chunk must be 0.
template <int DT, int U, class Op>
__device__ __forceinline__ void stream_row_claimed(const char* row, int64_t V, Op& op, int* chunk) {
  using E = Elem<DT>;
  constexpr int W = E::kVec;
  constexpr int CV = 64 * U;   // vectors of one chunk
  const int t = threadIdx.x;
  const int lane = t & 63;
  const uintptr_t a = reinterpret_cast<uintptr_t>(row);
  int64_t head = static_cast<int64_t>(((16u - (a & 15u)) & 15u) / E::kBytes);
  if (head > V) head = V;
  const int64_t nvec = (V - head) / W;
  const int64_t a1 = head + nvec * W;
  if (t < head) {
    float x[1] = {E::load1(row, t)};
    op.template group<1>(x, t);
  }
  const char* vb = row + head * E::kBytes;
  const int64_t nchunk = (nvec + CV - 1) / CV;
  for (;;) {
    int c = 0;
    if (lane == 0) c = atomicAdd(chunk, 1);
    c = __builtin_amdgcn_readfirstlane(c);
    if (c >= nchunk) break;
    const int64_t i0 = static_cast<int64_t>(c) * CV + lane;
    if (static_cast<int64_t>(c + 1) * CV <= nvec) {
      u32x4 r[U];
#pragma unroll
      for (int u = 0; u < U; ++u) r[u] = load16(vb + (i0 + u * 64) * 16);
      __builtin_amdgcn_sched_barrier(0);
      float x[U * W];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float y[W];
        E::unpack(r[u], y);
#pragma unroll
        for (int j = 0; j < W; ++j) x[u * W + j] = y[j];
      }
      op.template block<U, W>(x, head + i0 * W, static_cast<int64_t>(64) * W);
    } else {   // the last chunk, partly past the row
      u32x4 r[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u * 64 < nvec) r[u] = load16(vb + (i0 + u * 64) * 16);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (i0 + u * 64 < nvec) {
          float y[W];
          E::unpack(r[u], y);
          op.template group<W>(y, head + (i0 + u * 64) * W);
        }
      }
    }
  }
  if (a1 + t < V) {
    float x[1] = {E::load1(row, a1 + t)};
    op.template group<1>(x, a1 + t);
  }
}

// Two groups per CU: at most 64 VGPRs (8 waves per SIMD).
template <int DT>
__global__ __launch_bounds__(kTB, 8) void k_truncate(TruncArgs a) {
  __shared__ TruncLds s;
  const int r = blockIdx.x;
  const int b = r / a.K;
  const int i = r - b * a.K;
  const int t = threadIdx.x;
  const int64_t out = static_cast<int64_t>(r) * a.kmax;
  const int n = a.lengths ? a.lengths[b] : a.K;
  if (i >= n) {                         // a row no draft uses
    if (t == 0) a.q_nnz[r] = 0;
    return;
  }
  const char* row = static_cast<const char*>(a.rows) +
                    (static_cast<int64_t>(b) * a.ss + static_cast<int64_t>(i) * a.rs) * Elem<DT>::kBytes;
  const int64_t V = a.V;
  const int k = a.top_k < V ? a.top_k : static_cast<int>(V);
  constexpr int KB = key_bits<DT>();
  static_assert(Elem<DT>::kVec <= 8, "a place packs the occurrence in three bits");

  // 1. one pass: each thread's top three, the largest dropped logit
  if (t == 0) {
    s.bad = 0;
    s.nc = 0;
    s.n = 0;
    s.chunk = 0;
    s.tau_key = 0xFFFFFFFFu;
    s.drop_key = 0;
  }
  __syncthreads();
  Top3Op op;
  stream_row_claimed<DT, 2>(row, V, op, &s.chunk);
  // one LDS atomic per wave for the row check and the largest dropped key
  // (a thread that dropped nothing reports -inf: a k-th key of -inf, from a
  // row with fewer than k finite logits, always takes the exact path)
  {
    const bool bad = __ballot(op.v0 != op.v0 || op.v0 == kInf) != 0;
    const uint32_t dk = wave_max_u32(order_key<DT>(op.drop));
    if ((t & 63) == 0) {
      if (bad) atomicOr(&s.bad, 1);
      atomicMax(&s.drop_key, dk);
    }
  }
  // 2. tau: the smallest over waves of each wave's ceil(k/waves)-th largest
  //    thread maximum (each wave has that many logits >= it)
  {
    const int kw = (k + kTW - 1) / kTW;
    const uint32_t wk = wave_kth_key(order_key<DT>(op.v0), kw);
    if ((t & 63) == 0) atomicMin(&s.tau_key, wk);
  }
  __syncthreads();
  if (s.bad) {                          // not a distribution
    if (t == 0) a.q_nnz[r] = -1;
    return;
  }
  const uint32_t tkey = s.tau_key;

  // 3. candidates: the kept logits >= tau, with their places g * 8 + c
  //    (group start g, occurrence c < W <= 8 among its equal logits)
  {
    auto cand = [&](float v, int g, int c) {
      if (g >= 0 && order_key<DT>(v) >= tkey) {
        const int slot = atomicAdd(&s.nc, 1);   // at most 3 per thread: always fits
        s.cx[slot] = v;
        s.cid[slot] = g * 8 + c;
      }
    };
    cand(op.v0, op.g0, 0);
    cand(op.v1, op.g1, op.occurrence1());
    cand(op.v2, op.g2, op.occurrence2());
  }
  __syncthreads();
  int nc = s.nc;
  auto lds_hist = [&](uint32_t prefix, uint32_t mask, int shift, bool by_index, uint32_t pkey) {
    for (int c = t; c < nc; c += kTB) {
      const uint32_t key = order_key<DT>(s.cx[c]);
      if (by_index) {
        const uint32_t id = static_cast<uint32_t>(s.cid[c]);
        if (key == pkey && (id & mask) == prefix) atomicAdd(&s.hist[(id >> shift) & 255u], 1);
      } else if ((key & mask) == prefix) {
        atomicAdd(&s.hist[(key >> shift) & 255u], 1);
      }
    }
  };
  uint32_t kth = 0, id_cut = 0;
  bool exact = nc >= k;
  // kept entries in s.ckey / s.cidx / s.kx hold places, not token ids,
  // after the radix select over the candidates (the rank path stores token
  // ids); `ranked`: already in rank order
  bool ranked = false;
  if (exact && nc <= kRankCand) {
    // One 64-bit number per candidate, key above the complemented place:
    // a larger number ranks first (larger logit, then lower place).  Two
    // per 16-byte read; the pad 0 after the last ranks below every one.
    if (t <= nc) s.rk[t] = t < nc ? (static_cast<uint64_t>(order_key<DT>(s.cx[t])) << 32) |
                                        static_cast<uint32_t>(~s.cid[t])
                                  : uint64_t(0);
    __syncthreads();
    if (t < nc) {
      const uint64_t mine = s.rk[t];
      const uint32_t kc = static_cast<uint32_t>(mine >> 32);
      const int pc = s.cid[t];
      // every candidate's group is loaded while the ranks are counted; the
      // kept ones then store token ids, not places
      float y[Elem<DT>::kVec];
      load_group<DT>(row, V, pc >> 3, y);
      int rank = 0;
#pragma unroll 8
      for (int d = 0; d < nc; d += 2) {
        const ulonglong2 q = *reinterpret_cast<const ulonglong2*>(&s.rk[d]);
        rank += q.x > mine ? 1 : 0;
        rank += q.y > mine ? 1 : 0;
      }
      if (rank < k) {
        const float x = s.cx[t];
        s.ckey[rank] = kc;
        s.cidx[rank] = scan_group<DT>(V, pc >> 3, pc & 7, x, y);
        s.kx[rank] = x;
      }
    }
    __syncthreads();
    kth = s.ckey[k - 1];
    ranked = true;
    // a dropped logit at or above the k-th key may belong to the top k
    exact = s.drop_key < kth;
    if (exact && t == 0) s.n = k;
  } else if (exact) {
    radix_select<KB>(s, k, lds_hist, kth, id_cut);
    exact = s.drop_key < kth;
  }
  __syncthreads();
  if (exact) {
    if (!ranked) {
      for (int c = t; c < nc; c += kTB) keep_token(s, order_key<DT>(s.cx[c]), s.cx[c], s.cid[c], kth, id_cut);
      __syncthreads();
      // the kept places to token ids
      const int mk = s.n < kMaxNnz ? s.n : kMaxNnz;
      if (t < mk) {
        const int pc = s.cidx[t];
        s.cidx[t] = find_in_group<DT>(row, V, pc >> 3, pc & 7, s.kx[t]);
      }
    }
  } else {
    ranked = false;
    // 4. read the row again: every logit >= tau
    if (t == 0) s.nc = 0;
    __syncthreads();
    {
      CandOp<DT> cop{s, tkey};
      stream_row<DT, 4, CandOp<DT>, kTB>(row, 0, V, cop);
    }
    __syncthreads();
    nc = s.nc;
    if (nc <= kTruncCand) {
      radix_select<KB>(s, k, lds_hist, kth, id_cut);
      for (int c = t; c < nc; c += kTB) keep_token(s, order_key<DT>(s.cx[c]), s.cx[c], s.cid[c], kth, id_cut);
    } else {
      // too many logits at or above tau: select over the whole row
      radix_select<KB>(s, k, [&](uint32_t prefix, uint32_t mask, int shift, bool by_index, uint32_t pkey) {
        HistOp<DT> hop{s, prefix, mask, shift, by_index, pkey};
        stream_row<DT, 4, HistOp<DT>, kTB>(row, 0, V, hop);
      }, kth, id_cut);
      CollectOp<DT> cop{s, kth, id_cut};
      stream_row<DT, 4, CollectOp<DT>, kTB>(row, 0, V, cop);
    }
  }
  __syncthreads();

  // 5. sort, weights, top-p prefix
  const int m = s.n < kMaxNnz ? s.n : kMaxNnz;   // == k
  if (ranked) {
    if (t < m) {
      s.sidx[t] = s.cidx[t];
      s.sx[t] = s.kx[t];
    }
  } else {
    for (int c = t; c < m; c += kTB) {
      const uint32_t kc = s.ckey[c];
      const int ic = s.cidx[c];
      int rank = 0;
      for (int d = 0; d < m; ++d) {
        const uint32_t kd = s.ckey[d];
        rank += (kd > kc || (kd == kc && s.cidx[d] < ic)) ? 1 : 0;
      }
      s.sidx[rank] = ic;
      s.sx[rank] = s.kx[c];
    }
  }
  __syncthreads();
  const float xmax = s.sx[0];
  const bool bad = !(xmax > -kInf) || m != k;
  // One entry per thread: m <= kMaxNnz <= kTB.
  const float wt = (t < m && !bad) ? fast_exp2((s.sx[t] - xmax) * a.kq) : 0.f;
  const int lane = t & 63;
  const int w = t >> 6;
  if (m <= 64) {
    // one wave: the same sums as below, where waves past the first add 0
    if (w == 0) {
      float inc = wt;
#pragma unroll
      for (int q = 1; q < 64; q <<= 1) {
        const float o = __shfl_up(inc, q, 64);
        if (lane >= q) inc += o;
      }
      const float total = __shfl(inc, 63, 64);
      const uint64_t hit = __ballot(a.top_p < 1.f && t < m && inc >= a.top_p * total);
      const int keep = hit ? __ffsll(static_cast<unsigned long long>(hit)) : m;
      const float sum = __shfl(inc, keep - 1, 64);
      if (!bad && t < keep) {
        a.q_idx[out + t] = s.sidx[t];
        a.q_prob[out + t] = wt / sum;
      }
      if (t == 0) a.q_nnz[r] = bad ? -1 : keep;
    }
    return;
  }
  float inc = wt;
#pragma unroll
  for (int q = 1; q < 64; q <<= 1) {
    const float o = __shfl_up(inc, q, 64);
    if (lane >= q) inc += o;
  }
  if (lane == 63) s.fw[w] = inc;
  if (t == 0) s.keep = m;
  __syncthreads();
  float base = 0.f, total = 0.f;
#pragma unroll
  for (int j = 0; j < kTW; ++j) {
    if (j < w) base += s.fw[j];
    total += s.fw[j];
  }
  const float run = base + inc;   // mass of entries 0..t
  if (a.top_p < 1.f && t < m && run >= a.top_p * total) atomicMin(&s.keep, t + 1);
  __syncthreads();
  const int keep = s.keep;
  if (t == keep - 1) s.sum = run;
  __syncthreads();
  if (!bad && t < keep) {
    a.q_idx[out + t] = s.sidx[t];
    a.q_prob[out + t] = wt / s.sum;
  }
  if (t == 0) a.q_nnz[r] = bad ? -1 : keep;
}

template <typename K>
static const void* fn(K* k) {
  return reinterpret_cast<const void*>(k);
}

bool launch_truncate(const TruncArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev) {
  const bool bf = dtype == DT_BF16;
  return launch_threads(bf ? fn(k_truncate<DT_BF16>) : fn(k_truncate<DT_F32>), static_cast<int64_t>(a.B) * a.K, kTB,
                        stream, a, ev);
}

}  // namespace dbv
