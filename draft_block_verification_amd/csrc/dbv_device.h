// Device-side building blocks shared by the verification kernels (gfx950).
//
// A logit row is streamed once from HBM with 16-byte nontemporal loads
// (8 bf16 or 4 fp32 per lane per load, a wave covering 1 KiB contiguous),
// U loads in flight per lane.  Two per-lane reducers consume the stream:
//   * SoftmaxStats: online (max, sum of exp2) in fp32 -- the row's softmax
//     normaliser at temperature T, with exp folded into exp2 by k = log2(e)/T;
//   * ArgmaxPick:   exact (value, lowest index) argmax of a per-element score.
// Lane results are combined by wave shuffles and an LDS cross-wave step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dbv_plan.h"

namespace dbv {

constexpr int kBlock = 256;            // threads per workgroup: 4 wave64
constexpr int kWaves = kBlock / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInf = __builtin_inff();

enum : int { DT_F32 = 0, DT_BF16 = 1 };

// Per-sequence status bits (same values as the public header).
enum : int {
  SEQ_BAD_INPUT = 1, SEQ_NONFINITE = 2, SEQ_EMPTY_ROW = 4,
  SEQ_Q_ZERO = 8, SEQ_Z_ZERO = 16, SEQ_ERROR_MASK = 7
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// NaN-propagating max (v_maximum3_f32 on gfx950): a NaN anywhere in a row
// survives into its maximum, which is how rows with NaN are detected.
__device__ __forceinline__ float fmaxp(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}
// Its minimum counterpart (v_minimum3_f32).
__device__ __forceinline__ float fminp(float a, float b) {
  return __builtin_elementwise_minimum(a, b);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DT> struct Elem;

template <> struct Elem<DT_BF16> {
  static constexpr int kVec = 8;
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float load1(const void* row, int64_t i) {
    const uint16_t h = static_cast<const uint16_t*>(row)[i];
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
  }
  __device__ static __forceinline__ void unpack(u32x4 w, float (&x)[kVec]) {
    x[0] = __uint_as_float(w.x << 16); x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16); x[3] = __uint_as_float(w.y & 0xffff0000u);
    x[4] = __uint_as_float(w.z << 16); x[5] = __uint_as_float(w.z & 0xffff0000u);
    x[6] = __uint_as_float(w.w << 16); x[7] = __uint_as_float(w.w & 0xffff0000u);
  }
};

template <> struct Elem<DT_F32> {
  static constexpr int kVec = 4;
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ float load1(const void* row, int64_t i) {
    return static_cast<const float*>(row)[i];
  }
  __device__ static __forceinline__ void unpack(u32x4 w, float (&x)[kVec]) {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y);
    x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
  }
};

__device__ __forceinline__ u32x4 load16(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ---------------------------------------------------------------------------
// Wave priority steered by progress through a group's share of a flat
// stream.  The SIMD arbiter issues the oldest ready wave first, so among the
// groups that share a CU the first dispatched streams fastest and the last
// runs alone at the end, with too few loads in flight to keep the CU's share
// of HBM busy.  A wave raises its issue priority (s_setprio) while it is
// behind: level 3 before half of its share, 2 before 80%, 1 before 95%, 0
// for the rest, so the groups of a CU finish close together.  (Measured with
// kernel-internal timestamps: the groups of a CU are dispatched in blockIdx
// quarters, and without steering the last of them ended up to 40% later
// than the first on large sampling calls.)
// ---------------------------------------------------------------------------
struct Progress {
  int64_t off = 0;   // flat position of the current row's element 0, minus the group's start
  int64_t th1 = 0, th2 = 0, th3 = 0;   // 50%, 80% and 95% of the group's share
  bool on = false;
};

// done: elements of the group's share before the current step (wave-uniform).
__device__ __forceinline__ void steer_priority(const Progress& pg, int64_t done) {
  if (!pg.on) return;
  if (done < pg.th1) __builtin_amdgcn_s_setprio(3);
  else if (done < pg.th2) __builtin_amdgcn_s_setprio(2);
  else if (done < pg.th3) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// ---------------------------------------------------------------------------
// Row streaming by NT threads (default: one 256-thread group; NT = 64: the
// calling wave alone).  Visits
// elements [v0, v1) of `row`; every thread sees its own elements in
// increasing index order.  The op receives groups:
//   op.template group<N>(x, idx0)  -- N contiguous values starting at idx0
// Groups are the scalar head (to 16-byte alignment), U vectors at a time in
// the body, and the scalar tail.
// ---------------------------------------------------------------------------
template <int DT, int U, class Op, int NT = kBlock>
__device__ __forceinline__ void stream_row(const void* row, int64_t v0, int64_t v1, Op& op,
                                           const Progress& pg = Progress{}) {
  using E = Elem<DT>;
  constexpr int W = E::kVec;
  if (v1 <= v0) return;
  const char* base = static_cast<const char*>(row);
  const uintptr_t a = reinterpret_cast<uintptr_t>(base + v0 * E::kBytes);
  int64_t head = static_cast<int64_t>(((16u - (a & 15u)) & 15u) / E::kBytes);
  if (head > v1 - v0) head = v1 - v0;
  const int64_t a0 = v0 + head;
  const int64_t nvec = (v1 - a0) / W;
  const int64_t a1 = a0 + nvec * W;
  const int t = static_cast<int>(threadIdx.x) % NT;

  if (t < head) {
    float x[1] = {E::load1(row, v0 + t)};
    op.template group<1>(x, v0 + t);
  }
  const char* vb = base + a0 * E::kBytes;
  int64_t i = t;
  // ib: i - t, the same in every lane
  for (int64_t ib = 0; i + (U - 1) * NT < nvec; i += U * NT, ib += U * NT) {
    steer_priority(pg, pg.off + a0 + ib * W);
    u32x4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) r[u] = load16(vb + (i + u * NT) * 16);
    // Keep all U loads in flight before any of them is consumed: without this
    // barrier the scheduler hoists the first unpack above the later loads and
    // waits on the first load alone.
    __builtin_amdgcn_sched_barrier(0);
    float x[U * W];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float y[W];
      E::unpack(r[u], y);
#pragma unroll
      for (int j = 0; j < W; ++j) x[u * W + j] = y[j];
    }
    op.template block<U, W>(x, a0 + i * W, static_cast<int64_t>(NT) * W);
  }
  if (i < nvec) {  // the last (< U) vectors of this lane, loads issued together
    u32x4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + u * NT < nvec) r[u] = load16(vb + (i + u * NT) * 16);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i + u * NT < nvec) {
        float y[W];
        E::unpack(r[u], y);
        op.template group<W>(y, a0 + (i + u * NT) * W);
      }
    }
  }
  if (a1 + t < v1) {
    float x[1] = {E::load1(row, a1 + t)};
    op.template group<1>(x, a1 + t);
  }
}

// ---------------------------------------------------------------------------
// Online softmax statistics: M = max x, S = sum exp2((x - M) k).
// ---------------------------------------------------------------------------
struct SoftmaxStats {
  float M = -kInf;
  float S = 0.f;
  float k;  // log2(e) / T
  __device__ explicit SoftmaxStats(float k_) : k(k_) {}

  template <int N>
  __device__ __forceinline__ void absorb(const float* x) {
    float cm = x[0];
#pragma unroll
    for (int j = 1; j < N; ++j) cm = fmaxp(cm, x[j]);
    const float Mn = fmaxp(M, cm);
    if (Mn == -kInf) return;                 // nothing but -inf so far
    // Exactly 1 when the maximum did not move; 0 when M was -inf.
    const float scale = fast_exp2((M - Mn) * k);
    const float c = -Mn * k;
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j) s += fast_exp2(__builtin_fmaf(x[j], k, c));
    S = S * scale + s;
    M = Mn;
  }
  template <int N>
  __device__ __forceinline__ void group(const float* x, int64_t) { absorb<N>(x); }
  template <int U, int W>
  __device__ __forceinline__ void block(const float* x, int64_t, int64_t) { absorb<U * W>(x); }
};

// Merge two (M, S) pairs; -inf / NaN maxima propagate.
__device__ __forceinline__ void stats_merge(float& M, float& S, float M2, float S2, float k) {
  const float Mn = fmaxp(M, M2);
  if (Mn == -kInf) { M = Mn; S = 0.f; return; }
  const float s1 = (M == -kInf) ? 0.f : S * fast_exp2((M - Mn) * k);
  const float s2 = (M2 == -kInf) ? 0.f : S2 * fast_exp2((M2 - Mn) * k);
  M = Mn;
  S = s1 + s2;
}

// ---------------------------------------------------------------------------
// Softmax statistics for the sampling verifiers, accurate enough that
// differences of two rows' probabilities keep their relative precision.
// The reference of a running maximum M is the integer E = floor(M k): every
// element contributes exp2(x k - E) <= 2, summed in float32 over a block and
// added to a float64 sum.  Moving the reference rescales by an exact power of
// two, so the sum holds exactly the terms a later exp2(x k - E) reproduces
// (no rounded rescale factors), and its float64 accumulation leaves only the
// per-element rounding, which averages out.
// What is accumulated is the rest R: the sum over every element but one copy
// of the maximum.  The maximum's own term t = 2^(M k - E) joins only when the
// row is complete (stats64_total), so where one token carries nearly all of
// a row's mass no float32 addition happens at its magnitude, and the rest
// relative to it, R / t, keeps the relative precision of R
// (stats64_rest_rel): the mass off that token is R / (t + R).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float ref_exp(float M, float k) { return floorf(M * k); }

// A sum relative to the reference of M, rescaled to the reference E; 0 when
// M is -inf.
__device__ __forceinline__ double rescale_to(double S, float M, float k, float E) {
  if (M == -kInf) return 0.0;
  // Shifts below -1100 leave 0 in float64 anyway; the clamp keeps huge
  // logit ranges inside int.
  return __builtin_ldexp(S, static_cast<int>(fmaxf(ref_exp(M, k) - E, -1100.f)));
}

// The maximum's term 2^(M k - E) for E = floor(M k), in [1, 2): one exp2 of
// an argument formed with a single rounding (fma).
__device__ __forceinline__ float max_term(float M, float k) {
  return fast_exp2(__builtin_fmaf(M, k, -ref_exp(M, k)));
}

// The row sum S relative to E = floor(M k): the rest R plus the maximum's
// term.
__device__ __forceinline__ double stats64_total(float M, double R, float k) {
  return R + static_cast<double>(max_term(M, k));
}

// The rest relative to the maximum's term, R / 2^(M k - E) = S / 2^(M k - E)
// - 1 without that cancellation: the mass off one copy of the maximum over
// the mass of that copy.
__device__ __forceinline__ double stats64_rest_rel(float M, double R, float k) {
  return R / static_cast<double>(max_term(M, k));
}

// log2 of the ratio of two rows' sums, each relative to its maximum's term:
// log2((1 + r1) / (1 + r2)) for the rests r = stats64_rest_rel, through
// log1p of (r1 - r2) / (1 + r2), so that it keeps the rests' relative
// precision where both are small.
__device__ __forceinline__ float log2_sum_ratio(double r1, double r2) {
  return log1pf(static_cast<float>((r1 - r2) / (1.0 + r2))) * 1.4426950408889634f;
}

// Per-lane statistics for this scheme: R in float32 relative to E = floor(M
// k), rescaled by exact powers of two (ldexp) when E moves.  A lane's float32
// rounding is independent of the other lanes', so it averages out over the
// float64 merge of the lanes (wave_stats64).
struct SoftmaxStats64 {
  float M = -kInf;
  float E = 0.f;
  float R = 0.f;
  float k;  // log2(e) / T
  __device__ explicit SoftmaxStats64(float k_) : k(k_) {}

  template <int N>
  __device__ __forceinline__ void absorb(const float* x) {
    float cm = x[0];
#pragma unroll
    for (int j = 1; j < N; ++j) cm = fmaxp(cm, x[j]);
    const float Mn = fmaxp(M, cm);
    if (Mn == -kInf) return;                 // nothing but -inf so far
    if (!(Mn < kInf)) { M = Mn; return; }    // NaN / +inf: the row is in error
    const float En = ref_exp(Mn, k);
    // E <= En; R is 0 until the second finite element, and shifts below
    // -200 leave 0 in float32 anyway.
    R = __builtin_ldexpf(R, static_cast<int>(fmaxf(E - En, -200.f)));
    // Elements are taken in pairs with the running maximum r before them:
    // the two smaller of (r, x[j], x[j+1]) add their terms and the largest
    // becomes r.  Each step only orders three values, so the terms added are
    // those of the old M and the x[j] but one copy of the final r = Mn.
    float run = M, s = 0.f;
#pragma unroll
    for (int j = 0; j + 1 < N; j += 2) {
      const float a = x[j], b = x[j + 1];
      const float lo = fminp(fminp(a, b), run);
      const float mid = __builtin_amdgcn_fmed3f(a, b, run);
      run = fmaxp(fmaxp(a, b), run);
      s += fast_exp2(__builtin_fmaf(lo, k, -En));
      s += fast_exp2(__builtin_fmaf(mid, k, -En));
    }
    if constexpr ((N & 1) != 0) s += fast_exp2(__builtin_fmaf(fminp(x[N - 1], run), k, -En));
    R += s;
    M = Mn;
    E = En;
  }
  template <int N>
  __device__ __forceinline__ void group(const float* x, int64_t) { absorb<N>(x); }
  template <int U, int W>
  __device__ __forceinline__ void block(const float* x, int64_t, int64_t) { absorb<U * W>(x); }
};

// Merge two (M, R) pairs with float64 rests: the smaller maximum's own term
// joins the rest.  -inf / NaN maxima propagate.
__device__ __forceinline__ void stats64_merge(float& M, double& R, float M2, double R2, float k) {
  const float Mn = fmaxp(M, M2);
  if (Mn == -kInf) { M = Mn; R = 0.0; return; }
  if (!(Mn < kInf)) { M = Mn; return; }
  const float E = ref_exp(Mn, k);
  // The partial with the smaller maximum lo brings its rest and lo's own
  // term, rescaled by an exact power of two; the other keeps its reference.
  const bool first_hi = M >= M2;
  const float lo = first_hi ? M2 : M;
  const double Rhi = first_hi ? R : R2;
  const double Rlo = first_hi ? R2 : R;
  R = lo == -kInf ? Rhi : Rhi + rescale_to(Rlo + static_cast<double>(max_term(lo, k)), lo, k, E);
  M = Mn;
}

// ---------------------------------------------------------------------------
// Lowest-index argmax of a score.  Per lane, a group whose maximum beats the
// lane's best (rare after the first few groups) also records the exact
// position of its first maximal element, so no element is ever re-read.
// ---------------------------------------------------------------------------
struct ArgmaxPick {
  float best = -kInf;
  int64_t bidx = -1;
  bool nan = false;

  template <int N>
  __device__ __forceinline__ void group(const float* x, int64_t idx0) {
    float m = x[0];
#pragma unroll
    for (int j = 1; j < N; ++j) m = fmaxp(m, x[j]);
    nan |= (m != m);
    if (m > best || (bidx < 0 && m == best)) {
      int j0 = 0;
#pragma unroll
      for (int j = N - 1; j >= 0; --j)
        if (x[j] == m) j0 = j;
      best = m;
      bidx = idx0 + j0;
    }
  }
  template <int U, int W>
  __device__ __forceinline__ void block(const float* x, int64_t idx0, int64_t ustride) {
#pragma unroll
    for (int u = 0; u < U; ++u) group<W>(x + u * W, idx0 + u * ustride);
  }
};

// ------------------------------------------------------------ reductions ---

__device__ __forceinline__ float wave_shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int wave_shfl_xor(int v, int m) { return __shfl_xor(v, m, 64); }

// Is (v2, i2) a better (larger value, then lower index) pick than (v1, i1)?
// Index -1 means "no pick".  NaN never wins here; it is tracked separately.
__device__ __forceinline__ bool pick_better(float v2, int i2, float v1, int i1) {
  if (i2 < 0) return false;
  if (i1 < 0) return true;
  return v2 > v1 || (v2 == v1 && i2 < i1);
}

// Workgroup argmax reduction; results valid in thread 0.
__device__ __forceinline__ void block_argmax(float& v, int& idx, int& nan, float* s_v, int* s_i, int* s_n) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float v2 = wave_shfl_xor(v, m);
    const int i2 = wave_shfl_xor(idx, m);
    const int n2 = wave_shfl_xor(nan, m);
    if (pick_better(v2, i2, v, idx)) { v = v2; idx = i2; }
    nan |= n2;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { s_v[w] = v; s_i[w] = idx; s_n[w] = nan; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kWaves; ++k) {
      if (pick_better(s_v[k], s_i[k], v, idx)) { v = s_v[k]; idx = s_i[k]; }
      nan |= s_n[k];
    }
  }
}

// Workgroup (M, S) reduction; results valid in thread 0.
__device__ __forceinline__ void block_stats(float& M, float& S, float k, float* s_m, float* s_s) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float M2 = wave_shfl_xor(M, m);
    const float S2 = wave_shfl_xor(S, m);
    stats_merge(M, S, M2, S2, k);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { s_m[w] = M; s_s[w] = S; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int j = 1; j < kWaves; ++j) stats_merge(M, S, s_m[j], s_s[j], k);
  }
}

// Workgroup float sum (fixed order); result valid in thread 0.
__device__ __forceinline__ float block_sum(float v, float* s) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += wave_shfl_xor(v, m);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s[w] = v;
  __syncthreads();
  float r = 0.f;
  if (threadIdx.x == 0) {
    for (int j = 0; j < kWaves; ++j) r += s[j];
  }
  return r;
}

// Wave-wide reductions through DPP lane moves (no LDS round trips): the
// quad butterflies, the half-row and row mirrors, then row broadcasts 15 and
// 31 leave the result in lane 63.  Every lane of the wave must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_move(float identity, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v), CTRL, ROWS, 0xf,
                                                    false));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_move(int identity, int v) {
  return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROWS, 0xf, false);
}

// Wave-level (M, S) reduction through DPP lane moves; every lane ends with
// the wave's result (read from lane 63).  Every lane must be active.
__device__ __forceinline__ void wave_stats(float& M, float& S, float k) {
#define DBV_STATS_STEP(C, R)                                                  \
  stats_merge(M, S, dpp_move<C, R>(-kInf, M), dpp_move<C, R>(0.f, S), k);
  DBV_STATS_STEP(0xB1, 0xf)
  DBV_STATS_STEP(0x4E, 0xf)
  DBV_STATS_STEP(0x141, 0xf)
  DBV_STATS_STEP(0x140, 0xf)
  DBV_STATS_STEP(0x142, 0xa)
  DBV_STATS_STEP(0x143, 0xc)
#undef DBV_STATS_STEP
  M = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M), 63));
  S = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(S), 63));
}

template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_move(double identity, double v) {
  const uint64_t iv = __builtin_bit_cast(uint64_t, identity);
  const uint64_t vv = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_update_dpp(static_cast<int>(iv), static_cast<int>(vv), CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(static_cast<int>(iv >> 32), static_cast<int>(vv >> 32), CTRL, ROWS,
                                             0xf, false);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                        static_cast<uint32_t>(lo));
}

__device__ __forceinline__ double readlane63(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(b), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), 63);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// Wave-level (M, R) reduction with float64 rests (SoftmaxStats64), same lane
// moves as wave_stats; R enters as each lane's rest relative to floor(M k).
__device__ __forceinline__ void wave_stats64(float& M, double& S, float k) {
#define DBV_STATS64_STEP(C, R)                                                \
  stats64_merge(M, S, dpp_move<C, R>(-kInf, M), dpp_move<C, R>(0.0, S), k);
  DBV_STATS64_STEP(0xB1, 0xf)
  DBV_STATS64_STEP(0x4E, 0xf)
  DBV_STATS64_STEP(0x141, 0xf)
  DBV_STATS64_STEP(0x140, 0xf)
  DBV_STATS64_STEP(0x142, 0xa)
  DBV_STATS64_STEP(0x143, 0xc)
#undef DBV_STATS64_STEP
  M = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(M), 63));
  S = readlane63(S);
}

// Wave-level argmax (value, lowest index, NaN flag) through DPP lane moves;
// every lane ends with the wave's result.  Every lane must be active.
__device__ __forceinline__ void wave_argmax(float& v, int& idx, int& nan) {
#define DBV_PICK_STEP(C, R)                                                   \
  {                                                                           \
    const float v2 = dpp_move<C, R>(-kInf, v);                                \
    const int i2 = dpp_move<C, R>(-1, idx);                                   \
    nan |= dpp_move<C, R>(0, nan);                                            \
    if (pick_better(v2, i2, v, idx)) { v = v2; idx = i2; }                    \
  }
  DBV_PICK_STEP(0xB1, 0xf)
  DBV_PICK_STEP(0x4E, 0xf)
  DBV_PICK_STEP(0x141, 0xf)
  DBV_PICK_STEP(0x140, 0xf)
  DBV_PICK_STEP(0x142, 0xa)
  DBV_PICK_STEP(0x143, 0xc)
#undef DBV_PICK_STEP
  v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  idx = __builtin_amdgcn_readlane(idx, 63);
  nan = __builtin_amdgcn_readlane(nan, 63);
}

// ---------------------------------------------------------------------------
// Flat split helpers (the split itself is defined in dbv_plan.h).
// ---------------------------------------------------------------------------

// Visits the pieces of active group g in stream order: fn(r, v0, v1, pg) for
// each stream row r that meets the group's range, [v0, v1) being the part of
// the row inside it, and pg the progress of element 0 of row r through the
// group's range (for stream_row's priority steering; the priority is back
// at 0 on return).
template <class Fn>
__device__ __forceinline__ void for_pieces(const FlatSplit& f, int64_t g, Fn fn) {
  int64_t e0, e1;
  split_range(f, g, e0, e1);
  Progress pg;
  const int64_t len = e1 - e0;
  // shares of a few units end before the waves drift apart
  pg.on = len >= 16 * f.Q;
  pg.th1 = len / 2;
  pg.th2 = len - len / 5;
  pg.th3 = len - len / 20;
  int64_t r = udiv(e0, f.V);
  for (int64_t base = r * f.V; base < e1; ++r, base += f.V) {
    const int64_t v0 = e0 > base ? e0 - base : 0;
    const int64_t v1 = e1 < base + f.V ? e1 - base : f.V;
    pg.off = base - e0;
    fn(r, v0, v1, pg);
  }
  __builtin_amdgcn_s_setprio(0);
}

// Exclusive scan of one int per thread over a group of NW waves, in thread
// order; returns the thread's offset and sets `total`.  Two barriers.
template <int NW>
__device__ __forceinline__ int group_exclusive_scan(int v, int& total, int* s_w) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(inc, m, 64);
    if (lane >= m) inc += o;
  }
  if (lane == 63) s_w[w] = inc;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const int x = s_w[j];
    if (j < w) base += x;
    total += x;
  }
  __syncthreads();
  return base + inc - v;
}

// ---------------------------------------------------------------------------
// Sequence directory of a chain call's stream, rebuilt in LDS by every group:
// sequence b contributes count(b) consecutive stream rows.  Sequences are
// taken in blocks of q, a power of two (at most kSeqBlocks blocks); pre[j]
// is the first stream row of block j and pre[nblk] the number of rows R.
// ---------------------------------------------------------------------------
struct SeqDir {
  int q;
  int nblk;
};

// q: a power of two, so that a wave's 64 consecutive sequences cover whole
// blocks (q <= 64) or lie in one block (q >= 64); at most kSeqBlocks blocks.
__host__ __device__ inline SeqDir seq_dir_shape(int B) {
  SeqDir d;
  d.q = 1;
  while (static_cast<int64_t>(d.q) * kSeqBlocks < B) d.q <<= 1;
  d.nblk = static_cast<int>((B + d.q - 1) / d.q);
  return d;
}

// The LDS prefix pre[] from each thread's kSeqBlocks / kBlock block sums
// (blocks threadIdx.x * kPer + k) and their total `mine`.
template <int kPer>
__device__ __forceinline__ void finish_seq_dir(const SeqDir& d, const int (&sums)[kPer], int mine, int* pre,
                                               int* s_w) {
  int total;
  int off = group_exclusive_scan<kWaves>(mine, total, s_w);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = threadIdx.x * kPer + k;
    if (j < d.nblk) pre[j] = off;
    off += sums[k];
  }
  if (threadIdx.x == 0) pre[d.nblk] = total;
  __syncthreads();
}

template <class CountFn>
__device__ __forceinline__ SeqDir build_seq_dir(int B, CountFn count, int* pre, int* s_w) {
  const SeqDir d = seq_dir_shape(B);
  constexpr int kPer = kSeqBlocks / kBlock;     // blocks per thread
  int sums[kPer];
  int mine = 0;
  if (d.q > 1) {
    // Block sums: each wave reads the counts of 64 consecutive sequences at
    // a time (four such loads in flight), sums them over segments of
    // min(q, 64) lanes, and the first lane of each segment adds the sum to
    // its block.
    for (int j = threadIdx.x; j < d.nblk; j += kBlock) pre[j] = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int seg = d.q < 64 ? d.q : 64;
    constexpr int kChunks = 4;
    for (int c0 = wv * 64; c0 < B; c0 += kChunks * kBlock) {
      int c[kChunks];
#pragma unroll
      for (int k = 0; k < kChunks; ++k) {
        const int b = c0 + k * kBlock + lane;
        c[k] = b < B ? count(b) : 0;
      }
#pragma unroll
      for (int k = 0; k < kChunks; ++k) {
        int v = c[k];
        for (int m = 1; m < seg; m <<= 1) v += __shfl_xor(v, m, 64);
        const int b = c0 + k * kBlock + lane;
        if ((lane & (seg - 1)) == 0 && b < B && v != 0) atomicAdd(&pre[b / d.q], v);
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = threadIdx.x * kPer + k;
      sums[k] = j < d.nblk ? pre[j] : 0;
      mine += sums[k];
    }
    __syncthreads();
  } else {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = threadIdx.x * kPer + k;
      const int s = j < d.nblk ? count(j) : 0;
      sums[k] = s;
      mine += s;
    }
  }
  finish_seq_dir(d, sums, mine, pre, s_w);
  return d;
}

// The directory from block sums that a preceding kernel wrote (blk[j] = the
// rows of block j, k_seq_blocks), for calls of more than kSeqBlocks
// sequences: one load per block instead of every sequence's count in every
// group.
__device__ __forceinline__ SeqDir load_seq_dir(int B, const int32_t* blk, int* pre, int* s_w) {
  SeqDir d = seq_dir_shape(B);
  constexpr int kPer = kSeqBlocks / kBlock;
  int sums[kPer];
  int mine = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = threadIdx.x * kPer + k;
    sums[k] = j < d.nblk ? blk[j] : 0;
    mine += sums[k];
  }
  finish_seq_dir(d, sums, mine, pre, s_w);
  return d;
}

// The sequence holding stream row r (0 <= r < R), its first stream row and
// its row count.  With one sequence per block (B <= kSeqBlocks) everything
// comes from the LDS prefix; otherwise the block is walked with count().
template <class CountFn>
__device__ __forceinline__ int find_seq(const SeqDir& d, const int* pre, int r, CountFn count, int& first,
                                        int& cnt) {
  int lo = 0, hi = d.nblk - 1;
  while (lo < hi) {  // largest block j with pre[j] <= r
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  if (d.q == 1) {
    first = pre[lo];
    cnt = pre[lo + 1] - first;
    return lo;
  }
  int b = lo * d.q;
  int acc = pre[lo];
  for (;;) {
    const int c = count(b);
    if (acc + c > r) {
      cnt = c;
      break;
    }
    acc += c;
    ++b;
  }
  first = acc;
  return b;
}

// A group's position in the sequence directory: the sequence of the last
// row looked up, its first stream row and its row count.
struct SeqCursor {
  int b = -1;
  int first = 0;
  int cnt = 0;
  // find_seq_wave's window of 64 sequences from wb0 (wb0 < 0: none): the
  // rows before it, its total rows, and per lane the count and inclusive
  // prefix of sequence wb0 + lane
  int wb0 = -1;
  int wacc = 0;
  int wtot = 0;
  int wcl = 0;
  int wps = 0;
};

// find_seq continued from the cursor when row r lies at or past the
// cursor's sequence: a group visits its rows in increasing order, so each
// sequence it crosses is counted once instead of walking its directory block
// again for every row.
template <class CountFn>
__device__ __forceinline__ int find_seq(const SeqDir& d, const int* pre, int r, CountFn count, SeqCursor& c) {
  if (c.b < 0 || r < c.first) {
    c.b = find_seq(d, pre, r, count, c.first, c.cnt);
  } else {
    while (r >= c.first + c.cnt) {
      c.first += c.cnt;
      ++c.b;
      c.cnt = count(c.b);
    }
  }
  return c.b;
}

// find_seq for one wave (every lane with the same r), continuing from the
// wave's cursor: the counts of 64 sequences are read at once and kept, one
// per lane, with their prefix sum, and the sequence holding r is found by a
// ballot over that window, so a wave visiting increasing rows reads one
// round of counts per 64 sequences it passes.  B bounds the sequences
// counted.
template <class CountFn>
__device__ __forceinline__ int find_seq_wave(const SeqDir& d, const int* pre, int r, int B, CountFn count,
                                             SeqCursor& c) {
  if (c.b >= 0 && r >= c.first && r < c.first + c.cnt) return c.b;
  for (;;) {
    if (c.wb0 >= 0 && r >= c.wacc && r < c.wacc + c.wtot) {
      const uint64_t hit = __ballot(c.wacc + c.wps > r);
      const int L = __builtin_ctzll(hit);
      c.b = c.wb0 + L;
      c.cnt = __shfl(c.wcl, L, 64);
      c.first = c.wacc + __shfl(c.wps, L, 64) - c.cnt;
      return c.b;
    }
    int b0, acc;
    if (c.wb0 >= 0 && r >= c.wacc) {   // past the window: the next 64
      b0 = c.wb0 + 64;
      acc = c.wacc + c.wtot;
    } else {
      int lo = 0, hi = d.nblk - 1;
      while (lo < hi) {  // largest block j with pre[j] <= r
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= r) lo = mid;
        else hi = mid - 1;
      }
      b0 = lo * d.q;
      acc = pre[lo];
    }
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int bl = b0 + lane;
    const int cl = bl < B ? count(bl) : 0;
    int ps = cl;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int o = __shfl_up(ps, m, 64);
      if (lane >= m) ps += o;
    }
    c.wb0 = b0;
    c.wacc = acc;
    c.wtot = __shfl(ps, 63, 64);
    c.wcl = cl;
    c.wps = ps;
  }
}

// The first stream row of every sequence, pre_out[b], and pre_out[B] = R,
// for the kernels that follow, written by all G groups of the launch: group
// g takes directory blocks g, g + G, ...; wave 0 of the group reads the
// counts of 64 of a block's sequences at a time and turns them into starts
// by a prefix sum over its lanes.
template <class CountFn>
__device__ __forceinline__ void write_seq_starts(const SeqDir& d, const int* pre, int B, CountFn count,
                                                 int32_t* pre_out, int g, int G) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  for (int j = g; j < d.nblk; j += G) {
    int acc = pre[j];
    const int b1 = (j + 1) * d.q < B ? (j + 1) * d.q : B;
    for (int b0 = j * d.q; b0 < b1; b0 += 64) {
      const int b = b0 + lane;
      const int c = b < b1 ? count(b) : 0;
      int ps = c;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const int o = __shfl_up(ps, m, 64);
        if (lane >= m) ps += o;
      }
      if (b < b1) pre_out[b] = acc + ps - c;
      acc += __shfl(ps, 63, 64);
    }
  }
  if (g == 0 && lane == 0) pre_out[B] = pre[d.nblk];
}

// ---------------------------------------------------------------------------
// Combining the per-(slot, wave) partials of many rows inside one group:
// kRowLanes lanes share a row, each loading up to kRowLoads of its partials
// before merging (the loads are issued together), then a shuffle tree over
// the row's lanes.  span(r, first, n) gives row r's partials as the n
// consecutive float2 at part + first.  Calls done(r, lane-0 result) once per
// row.
// ---------------------------------------------------------------------------
constexpr int kRowLanes = 8;
constexpr int kRowLoads = 8;

template <int NT = kBlock, class SpanFn, class DoneFn>
__device__ __forceinline__ void combine_rows_stats(int nrows, const float2* part, float k, SpanFn span,
                                                   DoneFn done) {
  const int sub = threadIdx.x % kRowLanes;
  for (int r0 = 0; r0 < nrows; r0 += NT / kRowLanes) {
    const int r = r0 + static_cast<int>(threadIdx.x) / kRowLanes;
    float M = -kInf, S = 0.f;
    if (r < nrows) {
      int64_t first, n;
      span(r, first, n);
      const float2* p = part + first;
      for (int64_t j0 = 0; j0 < n; j0 += kRowLanes * kRowLoads) {
        float2 buf[kRowLoads];
#pragma unroll
        for (int q = 0; q < kRowLoads; ++q) {
          const int64_t j = j0 + sub + static_cast<int64_t>(q) * kRowLanes;
          buf[q] = j < n ? p[j] : make_float2(-kInf, 0.f);
        }
#pragma unroll
        for (int q = 0; q < kRowLoads; ++q) stats_merge(M, S, buf[q].x, buf[q].y, k);
      }
    }
#pragma unroll
    for (int m = kRowLanes / 2; m >= 1; m >>= 1) {
      const float M2 = __shfl_xor(M, m, 64);
      const float S2 = __shfl_xor(S, m, 64);
      stats_merge(M, S, M2, S2, k);
    }
    if (r < nrows && sub == 0) done(r, M, S);
  }
}

// kf(r) is the log2(e)/T of row r; done(r, M, R) receives the row's
// maximum and float64 rest.
// LANES lanes per row (a power of two up to kRowLanes): fewer lanes take
// more rows per pass, so that a sequence's rows are all requested at once.
template <int NT = kBlock, int LANES = kRowLanes, class KFn, class SpanFn, class DoneFn>
__device__ __forceinline__ void combine_rows_stats64(int nrows, const Stat64* part, KFn kf, SpanFn span,
                                                     DoneFn done) {
  static_assert(LANES >= 1 && LANES <= kRowLanes && (LANES & (LANES - 1)) == 0, "lanes per row");
  const int sub = threadIdx.x % LANES;
  for (int r0 = 0; r0 < nrows; r0 += NT / LANES) {
    const int r = r0 + static_cast<int>(threadIdx.x) / LANES;
    const float k = kf(r < nrows ? r : nrows - 1);
    float M = -kInf;
    double S = 0.0;
    if (r < nrows) {
      int64_t first, n;
      span(r, first, n);
      const Stat64* p = part + first;
      for (int64_t j0 = 0; j0 < n; j0 += LANES * kRowLoads) {
        Stat64 buf[kRowLoads];
#pragma unroll
        for (int q = 0; q < kRowLoads; ++q) {
          const int64_t j = j0 + sub + static_cast<int64_t>(q) * LANES;
          if (j < n) buf[q] = p[j];
          else { buf[q].M = -kInf; buf[q].R = 0.0; }
        }
#pragma unroll
        for (int q = 0; q < kRowLoads; ++q) stats64_merge(M, S, buf[q].M, buf[q].R, k);
      }
    }
#pragma unroll
    for (int m = LANES / 2; m >= 1; m >>= 1) {
      const float M2 = __shfl_xor(M, m, 64);
      const double S2 = __shfl_xor(S, m, 64);
      stats64_merge(M, S, M2, S2, k);
    }
    if (r < nrows && sub == 0) done(r, M, S);
  }
}

template <int NT = kBlock, class SpanFn, class DoneFn>
__device__ __forceinline__ void combine_rows_pick(int nrows, const float2* part, SpanFn span, DoneFn done) {
  const int sub = threadIdx.x % kRowLanes;
  for (int r0 = 0; r0 < nrows; r0 += NT / kRowLanes) {
    const int r = r0 + static_cast<int>(threadIdx.x) / kRowLanes;
    float v = -kInf;
    int idx = -1, nan = 0;
    if (r < nrows) {
      int64_t first, n;
      span(r, first, n);
      const float2* p = part + first;
      for (int64_t j0 = 0; j0 < n; j0 += kRowLanes * kRowLoads) {
        float2 buf[kRowLoads];
#pragma unroll
        for (int q = 0; q < kRowLoads; ++q) {
          const int64_t j = j0 + sub + static_cast<int64_t>(q) * kRowLanes;
          buf[q] = j < n ? p[j] : make_float2(-kInf, __int_as_float(-1));
        }
#pragma unroll
        for (int q = 0; q < kRowLoads; ++q) {
          const int i2 = __float_as_int(buf[q].y);
          if (buf[q].x != buf[q].x) nan = 1;
          else if (pick_better(buf[q].x, i2, v, idx)) { v = buf[q].x; idx = i2; }
        }
      }
    }
#pragma unroll
    for (int m = kRowLanes / 2; m >= 1; m >>= 1) {
      const float v2 = __shfl_xor(v, m, 64);
      const int i2 = __shfl_xor(idx, m, 64);
      const int n2 = __shfl_xor(nan, m, 64);
      if (pick_better(v2, i2, v, idx)) { v = v2; idx = i2; }
      nan |= n2;
    }
    if (r < nrows && sub == 0) done(r, v, idx, nan);
  }
}

// Serial merge of one row's n >= 1 partials in order (one thread).  The
// first eight are requested together (a row's partials are mostly the four
// wave partials of one or two groups), the rest one by one.
__device__ __forceinline__ void merge_span_stats(const float2* part, int64_t first, int64_t n, float k,
                                                 float& M, float& S) {
  constexpr int U = 8;
  M = -kInf;
  S = 0.f;
  const float2* p = part + first;
  float2 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = p[u < n ? u : n - 1];
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (u < n) stats_merge(M, S, v[u].x, v[u].y, k);
  for (int64_t j = U; j < n; ++j) stats_merge(M, S, p[j].x, p[j].y, k);
}

// Row status from a reduced maximum: NaN / +inf -> nonfinite, -inf -> empty.
__device__ __forceinline__ int max_status(float M) {
  if (M != M || M == kInf) return SEQ_NONFINITE;
  if (M == -kInf) return SEQ_EMPTY_ROW;
  return 0;
}

// Status of a softmax row from its float64 statistics (M, S).
__device__ __forceinline__ int stats64_status(float M, double R) {
  int st = max_status(M);
  if (!st && !(R >= 0.0 && R < 1e300)) st = SEQ_NONFINITE;
  return st;
}

// Status of a softmax row from its combined statistics (M, S).
__device__ __forceinline__ int stats_status(float M, float S) {
  int st = max_status(M);
  if (!st && !(S > 0.f && S < kInf)) st = SEQ_NONFINITE;
  return st;
}

}  // namespace dbv
