// Top-k / top-p truncation of drafter rows into stored sparse form
// ("One Call Ahead: Packed Self-Speculative Decoding with Diffusion
// Drafting", Sec. 3.2: only the nonzero entries of a truncated drafter
// distribution need storing).
//
//   k_truncate  one group of kBlock threads per row (b, i), i < n_b, every
//   pass streaming the row with 16-byte loads:
//     1. each thread's largest logit (and the row's NaN / +inf check); the
//        k-th largest of these 256 maxima, tau, has at least k logits at or
//        above it, and for a spread-out row only a few times k;
//     2. one pass collects every logit >= tau into LDS (at most
//        kTruncCand); if there are more, a radix select over the whole row
//        (8-bit digits of an order-preserving key, one pass each) takes
//        their place;
//     3. among the candidates, a radix select in LDS of the k-th largest
//        key and, where more logits equal it than the top-k needs, of the
//        cut-off token id (ties go to the lower ids);
//     4. the k kept sorted by (logit descending, id ascending) by counting
//        ranks; weights exp((x - x_max) / T); the shortest prefix whose
//        mass reaches p of the total (all k for p = 1), renormalised and
//        written in order.
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

constexpr int kTruncCand = 4096;   // LDS candidates of the common path

struct TruncLds {
  int hist[256];
  int bad, digit, above, n, keep, nc;
  float tmax[kBlock];
  float cx[kTruncCand];            // candidates: logit and token id
  int cid[kTruncCand];
  uint32_t ckey[kMaxNnz];          // the kept k
  int cidx[kMaxNnz];
  float kx[kMaxNnz];
  int sidx[kMaxNnz];
  float sx[kMaxNnz];
  float fw[kWaves];
  float sum;
};

// Each thread's largest logit and the NaN / +inf check.
struct MaxOp {
  float m = -kInf;
  int bad = 0;
  template <int N>
  __device__ __forceinline__ void group(const float* x, int64_t) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      if (x[j] != x[j] || x[j] == kInf) bad = 1;
      m = fmaxf(m, x[j]);
    }
  }
  template <int U, int W>
  __device__ __forceinline__ void block(const float* x, int64_t idx0, int64_t ustride) {
#pragma unroll
    for (int u = 0; u < U; ++u) group<W>(x + u * W, idx0 + u * ustride);
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
  for (int j = threadIdx.x; j < 256; j += kBlock) s.hist[j] = 0;
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
__device__ void radix_select(TruncLds& s, int k, Hist hist, uint32_t& kth, uint32_t& id_cut) {
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

static_assert(kMaxNnz <= kBlock, "one kept entry per thread");

template <int DT>
__global__ __launch_bounds__(kBlock) void k_truncate(TruncArgs a) {
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

  // 1. per-thread maxima; tau = the k-th largest of them
  if (t == 0) {
    s.bad = 0;
    s.nc = 0;
    s.n = 0;
  }
  {
    MaxOp op;
    stream_row<DT, 4>(row, 0, V, op);
    s.tmax[t] = op.m;
    if (op.bad) atomicOr(&s.bad, 1);
  }
  __syncthreads();
  if (s.bad) {                          // not a distribution
    if (t == 0) a.q_nnz[r] = -1;
    return;
  }
  {
    const float mt = s.tmax[t];
    int rank = 0;
    for (int u = 0; u < kBlock; ++u) {
      const float mu = s.tmax[u];
      rank += (mu > mt || (mu == mt && u < t)) ? 1 : 0;
    }
    // k <= kMaxNnz <= kBlock: some thread has rank k - 1
    if (rank == k - 1) s.digit = static_cast<int>(order_key<DT>(mt));
  }
  __syncthreads();
  const uint32_t tkey = static_cast<uint32_t>(s.digit);
  __syncthreads();

  // 2. candidates >= tau
  {
    CandOp<DT> op{s, tkey};
    stream_row<DT, 4>(row, 0, V, op);
  }
  __syncthreads();
  const int nc = s.nc;
  uint32_t kth, id_cut;
  if (nc <= kTruncCand) {
    // 3. select among the candidates in LDS
    radix_select<KB>(s, k, [&](uint32_t prefix, uint32_t mask, int shift, bool by_index, uint32_t pkey) {
      for (int c = t; c < nc; c += kBlock) {
        const uint32_t key = order_key<DT>(s.cx[c]);
        if (by_index) {
          const uint32_t id = static_cast<uint32_t>(s.cid[c]);
          if (key == pkey && (id & mask) == prefix) atomicAdd(&s.hist[(id >> shift) & 255u], 1);
        } else if ((key & mask) == prefix) {
          atomicAdd(&s.hist[(key >> shift) & 255u], 1);
        }
      }
    }, kth, id_cut);
    for (int c = t; c < nc; c += kBlock) keep_token(s, order_key<DT>(s.cx[c]), s.cx[c], s.cid[c], kth, id_cut);
  } else {
    // too many logits at or above tau: select over the whole row
    radix_select<KB>(s, k, [&](uint32_t prefix, uint32_t mask, int shift, bool by_index, uint32_t pkey) {
      HistOp<DT> op{s, prefix, mask, shift, by_index, pkey};
      stream_row<DT, 4>(row, 0, V, op);
    }, kth, id_cut);
    CollectOp<DT> op{s, kth, id_cut};
    stream_row<DT, 4>(row, 0, V, op);
  }
  __syncthreads();

  // 4. sort, weights, top-p prefix
  const int m = s.n < kMaxNnz ? s.n : kMaxNnz;   // == k
  for (int c = t; c < m; c += kBlock) {
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
  __syncthreads();
  const float xmax = s.sx[0];
  const bool bad = !(xmax > -kInf) || m != k;
  // One entry per thread: m <= kMaxNnz <= kBlock.
  const float wt = (t < m && !bad) ? fast_exp2((s.sx[t] - xmax) * a.kq) : 0.f;
  const int lane = t & 63;
  const int w = t >> 6;
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
  for (int j = 0; j < kWaves; ++j) {
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
  return launch(bf ? fn(k_truncate<DT_BF16>) : fn(k_truncate<DT_F32>), static_cast<int64_t>(a.B) * a.K, stream, a,
                ev);
}

}  // namespace dbv
