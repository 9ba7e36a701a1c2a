// Any-order greedy verification of one packed call (Packed-SS, App. C,
// Algorithm 3, the verification steps of one iteration):
//
//   k_ao_plan      per sequence: checks the order (a permutation of the u
//                  active slots), the slot positions (increasing) and the
//                  draft tokens (-1 = missing); kappa = leading ranks whose
//                  slot has a draft; the verifier rows to read,
//                  nver = min(kappa + 1, u), and the sequence's stream rows
//   k_ao_rows      persistent: argmax partials of the verifier rows (by
//                  rank) and the drafter rows (by slot), one flat stream
//                  split evenly over the groups (FlatSplit)
//   k_ao_finalize  per sequence: v_r and z_j, h = leading ranks r < kappa
//                  whose draft equals v_r, A = min(h + 1, u), the accepted
//                  pairs C = (pos(pi(r)), v_r)_{r<A}, the ending position E'
//                  from an accepted EOS, C restricted to positions <= E'
//                  (kept in rank order), and the next draft z_j at the slots
//                  neither accepted nor beyond E'.
// The kernel boundaries are the only cross-group synchronisation.
#include "dbv_device.h"
#include "dbv_launch.h"

#include <climits>

namespace dbv {

__device__ __forceinline__ int active_count(const AnyOrderArgs& a, int b, bool& bad) {
  const int u = a.num_active ? a.num_active[b] : a.U;
  bad = u < 0 || u > a.U;
  return bad ? 0 : u;
}

__global__ __launch_bounds__(kBlock) void k_ao_plan(AnyOrderArgs a) {
  __shared__ int s_seen[kMaxDraft];
  __shared__ int s_st, s_kappa;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  bool ubad;
  const int u = active_count(a, b, ubad);
  const int64_t base = static_cast<int64_t>(b) * a.U;
  for (int j = t; j < u; j += kBlock) s_seen[j] = 0;
  if (t == 0) {
    s_st = ubad ? SEQ_BAD_INPUT : 0;
    s_kappa = u;
  }
  __syncthreads();
  int st = 0;
  for (int r = t; r < u; r += kBlock) {
    const int o = a.order[base + r];
    if (o < 0 || o >= u) st |= SEQ_BAD_INPUT;
    else atomicAdd(&s_seen[o], 1);
  }
  for (int j = t; j < u; j += kBlock) {
    const int dj = a.draft_tokens[base + j];
    if (dj < -1 || dj >= a.V) st |= SEQ_BAD_INPUT;
    if (a.positions && j + 1 < u && a.positions[base + j] >= a.positions[base + j + 1]) st |= SEQ_BAD_INPUT;
  }
  __syncthreads();
  for (int j = t; j < u; j += kBlock)
    if (s_seen[j] != 1) st |= SEQ_BAD_INPUT;
  if (st) atomicOr(&s_st, st);
  __syncthreads();
  const bool bad = s_st != 0;
  if (!bad) {
    for (int r = t; r < u; r += kBlock)
      if (a.draft_tokens[base + a.order[base + r]] < 0) atomicMin(&s_kappa, r);
  }
  __syncthreads();
  if (t == 0) {
    const int kappa = bad ? 0 : s_kappa;
    const int nv = bad ? 0 : (kappa + 1 < u ? kappa + 1 : u);
    a.kappa[b] = kappa;
    a.nver[b] = nv;
    a.rows[b] = bad ? 0 : nv + (a.dr ? u : 0);
    a.pstat[b] = s_st;
  }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_ao_rows(AnyOrderArgs a) {
  __shared__ int s_pre[kSeqBlocks + 1];
  __shared__ int s_w[kWaves];
  auto count = [&](int b) { return a.rows[b]; };
  const SeqDir dir = build_seq_dir(a.B, count, s_pre, s_w);
  write_seq_starts(dir, s_pre, a.B, count, a.pre, blockIdx.x, gridDim.x);
  const FlatSplit f = make_split(s_pre[dir.nblk], a.V, Elem<DT>::kBytes, a.grid);
  const int64_t g = blockIdx.x;
  if (g >= f.G) return;
  SeqCursor cur;
  for_pieces(f, g, [&](int64_t r, int64_t v0, int64_t v1, const Progress& pg) {
    const int b = find_seq(dir, s_pre, static_cast<int>(r), count, cur);
    const int first = cur.first;
    const int j = static_cast<int>(r) - first;
    const int nv = a.nver[b];
    const char* rowp =
        j < nv ? static_cast<const char*>(a.tgt) + (static_cast<int64_t>(b) * a.ts + j * a.tr) * Elem<DT>::kBytes
               : static_cast<const char*>(a.dr) +
                     (static_cast<int64_t>(b) * a.ds + static_cast<int64_t>(j - nv) * a.drr) * Elem<DT>::kBytes;
    ArgmaxPick pk;
    stream_row<DT, 4>(rowp, v0, v1, pk, pg);
    float v = pk.best;
    int ii = static_cast<int>(pk.bidx);
    int nan = pk.nan ? 1 : 0;
    wave_argmax(v, ii, nan);
    if ((threadIdx.x & 63) == 0)
      a.part[(r + g) * kWaves + (threadIdx.x >> 6)] = make_float2(nan ? __builtin_nanf("") : v, __int_as_float(ii));
  });
}

template <int DT>
__global__ __launch_bounds__(kBlock) void k_ao_finalize(AnyOrderArgs a) {
  __shared__ int s_v[kMaxDraft], s_z[kMaxDraft], s_acc[kMaxDraft];
  __shared__ int s_st, s_h, s_end, s_w[kWaves];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  bool ubad;
  const int u = active_count(a, b, ubad);
  const int64_t base = static_cast<int64_t>(b) * a.U;
  const int end0 = a.end_pos ? a.end_pos[b] : INT_MAX;
  const int kappa = a.kappa[b];
  const int nv = a.nver[b];
  const int nrows = a.rows[b];
  const int p0 = a.pre[b];
  if (t == 0) {
    s_st = a.pstat[b];
    s_h = kappa;
    s_end = end0;
  }
  for (int j = t; j < u; j += kBlock) s_acc[j] = 0;
  __syncthreads();
  int st = 0;
  if (nrows > 0) {
    const FlatSplit f = make_split(a.pre[a.B], a.V, Elem<DT>::kBytes, a.grid);
    combine_rows_pick(
        nrows, a.part,
        [&](int r, int64_t& first, int64_t& cnt) {
          split_row_slots(f, p0 + r, first, cnt);
          first *= kWaves;
          cnt *= kWaves;
        },
        [&](int r, float v, int idx, int nan) {
          st |= nan ? SEQ_NONFINITE : max_status(v);
          if (r < nv) s_v[r] = idx;
          else s_z[r - nv] = idx;
        });
  }
  if (st) atomicOr(&s_st, st);
  __syncthreads();
  const int status = s_st;
  int32_t* ap = a.acc_pos + base;
  int32_t* at = a.acc_tok + base;
  int32_t* nd = a.next_draft ? a.next_draft + base : nullptr;
  if (status & SEQ_ERROR_MASK) {
    for (int i = t; i < a.U; i += kBlock) {
      ap[i] = -1;
      at[i] = -1;
      if (nd) nd[i] = -1;
    }
    if (t == 0) {
      a.accept_len[b] = -1;
      a.num_accepted[b] = 0;
      a.new_end[b] = end0;
      if (a.status) a.status[b] = status;
    }
    return;
  }
  // h: leading ranks r < kappa whose draft equals the verifier's argmax.
  for (int r = t; r < kappa; r += kBlock)
    if (a.draft_tokens[base + a.order[base + r]] != s_v[r]) atomicMin(&s_h, r);
  __syncthreads();
  const int h = s_h;
  const int A = h + 1 < u ? h + 1 : u;
  // The ending position: the smallest accepted position holding EOS.
  for (int r = t; r < A; r += kBlock) {
    const int slot = a.order[base + r];
    s_acc[slot] = 1;
    if (a.eos >= 0 && s_v[r] == a.eos) {
      const int pos = a.positions ? a.positions[base + slot] : slot;
      atomicMin(&s_end, pos);
    }
  }
  __syncthreads();
  const int E = s_end;
  // C restricted to positions <= E, kept in rank order (a scan per pass of
  // kBlock ranks).
  int kept = 0;
  for (int r0 = 0; r0 < A; r0 += kBlock) {
    const int r = r0 + t;
    int pos = 0, keep = 0;
    if (r < A) {
      const int slot = a.order[base + r];
      pos = a.positions ? a.positions[base + slot] : slot;
      keep = pos <= E ? 1 : 0;
    }
    int total;
    const int off = kept + group_exclusive_scan<kWaves>(keep, total, s_w);
    if (keep) {
      ap[off] = pos;
      at[off] = s_v[r];
    }
    kept += total;
  }
  for (int i = kept + t; i < a.U; i += kBlock) {
    ap[i] = -1;
    at[i] = -1;
  }
  if (nd) {
    for (int j = t; j < a.U; j += kBlock) {
      int z = -1;
      if (a.dr && j < u && !s_acc[j]) {
        const int pos = a.positions ? a.positions[base + j] : j;
        if (pos <= E) z = s_z[j];
      }
      nd[j] = z;
    }
  }
  if (t == 0) {
    a.accept_len[b] = h;
    a.num_accepted[b] = kept;
    a.new_end[b] = E;
    if (a.status) a.status[b] = status;
  }
}

template <typename K>
static const void* fn(K* k) {
  return reinterpret_cast<const void*>(k);
}

bool launch_any_order(const AnyOrderArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev) {
  const bool bf = dtype == DT_BF16;
  return launch(fn(k_ao_plan), a.B, stream, a) &&
         launch(bf ? fn(k_ao_rows<DT_BF16>) : fn(k_ao_rows<DT_F32>), a.grid, stream, a, ev) &&
         launch(bf ? fn(k_ao_finalize<DT_BF16>) : fn(k_ao_finalize<DT_F32>), a.B, stream, a);
}

}  // namespace dbv
