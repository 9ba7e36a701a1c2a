// Kernel argument blocks and launchers (internal to libdbv).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dbv_plan.h"

namespace dbv {

struct GreedyArgs {
  int B, K, V, W;
  const void* tgt; int64_t ts, tr;     // target rows: element strides
  const void* dr; int64_t ds, drr;     // drafter rows
  const int32_t* draft_tokens;
  const int32_t* draft_len;
  int32_t eos;
  const int32_t* budget;
  int32_t* accept_len; int32_t* out_tokens; int32_t* num_out;
  int32_t* next_draft; int32_t* next_len; int32_t* status;
  float2* part;                        // per (slot, wave)
  int32_t* pre;                        // [B + 1] first stream row per sequence
  int64_t grid;                        // groups of the row-streaming launch
  int elem_bytes;                      // 2 (bf16) or 4 (fp32)
};

enum : int { RULE_LINEAR = 0, RULE_CACTUS = 1, RULE_SPOT = 2, RULE_SPARSE = 3 };

struct SampleArgs {
  int B, K, V;
  const void* tgt; int64_t ts, tr;
  const void* drf; int64_t ds, dr;
  const int32_t* draft_tokens;
  const int32_t* draft_len;
  float kp, kq;                        // log2(e) / temperature
  int rule;                            // RULE_LINEAR, RULE_CACTUS, RULE_SPOT or RULE_SPARSE
  float lam;                           // linear rule: 0 = lossless
  float delta;                         // Cactus rule: KL budget
  // Joint-space chain (RULE_SPOT): per link the target's position s*, the
  // proposal's position, the drafter's probability of s*, and optionally
  // the Gumbel rows of the target rows with the gate threshold.
  const int32_t* pos_star;             // [B, K+1]
  const int32_t* prop_pos;             // [B, K]
  const float* qpos;                   // [B, K]
  const float* gumbel; int64_t gs, grs;
  float inv_t;                         // 1 / temperature of the target
  float tau;
  // Stored sparse drafter distributions (RULE_SPARSE): [B, K, kmax] entries,
  // the first qnnz[b, i] of each row in use; no drafter rows are streamed.
  const int32_t* qidx; const float* qprob; const int32_t* qnnz;
  int kmax;
  int drows;                           // drafter rows are streamed (1) or not (0)
  const float* u_accept; const float* u_resample;
  int32_t eos;
  const int32_t* budget;
  int32_t* accept_len; int32_t* out_tokens; int32_t* num_out;
  float* p_draft; float* q_draft; float* alpha; float* residual_mass;
  int32_t* status;
  float* accept_margin;                // [B, K] |u - alpha| (NULL: not written)
  float* draw_margin;                  // [B] the draw's distance from a CDF step over Z (NULL: not written)
  float* row_tv;                       // [B, K] TV(p_i, q_i) of draft rows (NULL: not computed)
  Stat64* stats;                       // per (slot, wave): M and the float64 sum
  float2* gpart;                       // per (slot, wave), with Gumbel rows
  int32_t* pre;                        // [B + 1] first stream row per sequence
  int32_t* blk;                        // [kSeqBlocks] rows per directory block, or NULL (B <= kSeqBlocks)
  DrawRecord* rec;                     // per sequence
  float* tmass;                        // per (sequence, draw tile)
  SparseRow* sq;                       // per sequence: stored sparse Q of row h
  int64_t grid;                        // groups of the row-streaming launch
  int tiles;                           // draw tiles per row
  int tpc;                             // draw tiles per mass-kernel group
  int chunks;                          // mass-kernel groups per sequence
};

struct AnyOrderArgs {
  int B, U, V;
  const void* tgt; int64_t ts, tr;     // verifier rows by rank
  const void* dr; int64_t ds, drr;     // drafter rows by slot (NULL: none)
  const int32_t* order;                // [B, U] slot checked at rank r
  const int32_t* num_active;           // [B] u_b (NULL: U)
  const int32_t* positions;            // [B, U] output position of slot j (NULL: j)
  const int32_t* draft_tokens;         // [B, U] by slot, -1 = missing
  int32_t eos;
  const int32_t* end_pos;              // [B] E (NULL: no limit)
  int32_t* accept_len; int32_t* num_accepted; int32_t* acc_pos; int32_t* acc_tok;
  int32_t* new_end; int32_t* next_draft; int32_t* status;
  float2* part;                        // per (slot, wave)
  int32_t* pre;                        // [B + 1] first stream row per sequence
  int32_t* rows;                       // [B] stream rows of the sequence
  int32_t* nver;                       // [B] verifier rows read
  int32_t* kappa;                      // [B]
  int32_t* pstat;                      // [B] status bits found by the plan
  int64_t grid;                        // groups of the row-streaming launch
};

struct TreeArgs {
  int B, S, L, V;
  const void* logits; int64_t ss, sy, sp;   // sequence, state, position strides
  const uint8_t* masked;
  const int32_t* parent; const int32_t* edge_pos; const int32_t* edge_tok;
  const int32_t* num_states; const int32_t* next_pos;
  const float* gumbel; int64_t gs, gp;
  float inv_t;                               // 1/T, 0 for T = 0 (greedy)
  int fixed;                                 // 1 = fixed-position mode
  int32_t* sel_pos; int32_t* sel_tok; float* sel_conf;
  int32_t* path_len; int32_t* path_nodes;
  int32_t* commit_pos; int32_t* commit_tok; int32_t* num_commits;
  int32_t* status;
  int32_t* count;                            // rows in the stream
  int32_t* list;                             // stream row -> flat row id
  int32_t* map;                              // flat row id -> stream row or -1
  float* pos_margin; float* tok_margin;      // [B, S] diagnostics (NULL: not written)
  float2* conf;                              // per (slot, wave)
  float2* pick;                              // per (state, split2)
  float* pick2;                              // per (state, split2): second-best score (tok_margin only)
  int32_t* sel;                              // per state: s*
  float* selconf;                            // per state: confidence at s*
  int32_t* selstat;                          // per state: status of its rows
  float* selgap;                             // per state: relative gap of the two best confidences
  int4* batch;                               // per (sequence, batch slot): {s*, n}, then the n states
  int32_t* nbat;                             // per sequence: batches of the Gumbel argmax
  int64_t grid;                              // groups of the row-streaming launch
  int split2; int64_t chunk2;
  FastDiv32 divL, divS;                      // division by L and by S
};

// Top-k / top-p truncation of rows [B, K, V] (row i of sequence b read
// only for i < lengths[b]) into stored sparse form [B, K, kmax].
struct TruncArgs {
  int B, K, V;
  const void* rows; int64_t ss, rs;
  const int32_t* lengths;              // [B] or NULL (= K)
  float kq;                            // log2(e) / temperature
  int top_k;
  float top_p;
  int kmax;
  int32_t* q_idx; float* q_prob; int32_t* q_nnz;
};

// DDTree token hypotheses: partial reductions of one piece of a stale row,
// per (slot, wave).  T = 0: softmax statistics (M, S) at temperature 1 and
// the two largest logits v1 >= v2, each with the start index (i1, i2) of the
// group of contiguous elements that holds it.  T > 0: (M, S), the best score
// v1 of z/T + G with its group i1, and a NaN flag of the scores.  (x is
// unused.)
struct DDPart {
  float M, S, v1;
  int i1;
  float v2;
  int i2;
  float x;
  int nan;
};

struct DDHypArgs {
  int B, L, V;
  const void* stale; int64_t ss, sp;   // [B, L, V] stale logits: element strides
  const uint8_t* masked;               // [B, L] masked positions of the current state
  const float* gumbel; int64_t gs, gp; // [B, L, V] Gumbel rows (T > 0)
  float inv_t;                         // 1 / T, 0 for T = 0
  float below;                         // runner-up kept when p^(argmax) < below (T = 0)
  int32_t* hyp_tok; float* hyp_prob;   // [B, L, 2]
  int32_t* status;                     // [B]
  int32_t* count;                      // rows in the stream
  int32_t* list;                       // stream row -> b*L + s
  int32_t* map;                        // b*L + s -> stream row or -1
  DDPart* part;                        // per (slot, wave)
  int64_t grid;                        // groups of the row-streaming launch
  int split_bytes;                     // bytes per element for the split (Gumbel rows included)
  int fused_plan;                      // the row stream lists its rows itself (set by the launcher)
};

struct DDTreeArgs {
  int B, L, D;
  const uint8_t* masked;               // [B, L] masked positions of the root
  const int32_t* hyp_tok; const float* hyp_prob;   // [B, L, 2]
  const float* order; int64_t os, orow;  // order logit rows (per frontier slot, or the table)
  int table;                           // 1: every level from the first-order table
  int first;                           // one-level mode: start from the root
  float inv_tau, gamma;
  int32_t* parent; int32_t* edge_pos; int32_t* edge_tok; float* mass;   // [B, D+1]
  uint8_t* node_masked;                // [B, D+1, L] or NULL
  int32_t* num_nodes; int32_t* frontier; int32_t* num_frontier;        // [B], [B, D], [B]
  int32_t* status;                     // [B] in / out
  uint64_t* keys; uint64_t* masks;     // [B, D+1] search state kept between levels
};

// Optional events recorded around the row-streaming kernel of a call.
struct TimingEvents {
  hipEvent_t begin = nullptr;
  hipEvent_t end = nullptr;
};

// Launch `kern(arg)` on `grid` groups of `threads` threads.  With timing
// events the launch goes through hipExtLaunchKernel, which stamps the events
// at the kernel's own start and end (no launch gap in the interval); an empty
// grid still records both events so that the caller can read them.
template <typename Arg>
bool launch_threads(const void* kern, int64_t grid, int threads, hipStream_t stream, const Arg& arg,
                    const TimingEvents& ev = TimingEvents(), size_t lds_bytes = 0) {
  if (grid <= 0) {
    if (ev.begin) (void)hipEventRecord(ev.begin, stream);
    if (ev.end) (void)hipEventRecord(ev.end, stream);
    return true;
  }
  void* args[] = {const_cast<Arg*>(&arg)};
  return hipExtLaunchKernel(kern, dim3(static_cast<unsigned>(grid)), dim3(threads), args, lds_bytes, stream,
                            ev.begin, ev.end, 0) == hipSuccess;
}

template <typename Arg>
bool launch(const void* kern, int64_t grid, hipStream_t stream, const Arg& arg,
            const TimingEvents& ev = TimingEvents()) {
  return launch_threads(kern, grid, 256, stream, arg, ev);
}

// Resident groups of the current device (kResidentPerCU per CU).
int64_t resident_groups();

bool launch_greedy(const GreedyArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev);
bool launch_sample(const SampleArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev);
bool launch_tree(const TreeArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev);
bool launch_any_order(const AnyOrderArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev);
bool launch_truncate(const TruncArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev);
bool launch_dd_hypotheses(const DDHypArgs& a, int dtype, hipStream_t stream, const TimingEvents& ev);
bool launch_dd_tree(const DDTreeArgs& a, hipStream_t stream, const TimingEvents& ev);

}  // namespace dbv
