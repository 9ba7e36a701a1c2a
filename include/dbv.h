/*
 * dbv.h -- C ABI of libdbv, parallel verification of a drafted token block on
 * AMD Instinct MI355X (gfx950).
 *
 * One call verifies a batch of B independent sequences against target-model
 * logits that are already resident in device memory: per (sequence, position)
 * row it takes a temperature softmax over the vocabulary, applies one
 * acceptance test (greedy argmax match, lossless rejection min(1, p/q), the
 * linear lenient rule, or shared-Gumbel state equality over a draft tree),
 * finds the longest accepted prefix (or tree path) and draws the correction
 * or bonus token from supplied uniforms.  verify_cactus adds the modified
 * Cactus acceptance rule, verify_sparse verification against stored sparse
 * drafter distributions (truncate_top_k_top_p writes them from drafter
 * rows), verify_spot_chain chain verification on the joint
 * (position, token) space and verify_greedy_any_order any-order greedy
 * verification.  ddtree_hypotheses, ddtree_level and ddtree_build construct
 * the draft tree that verify_gumbel_tree checks.
 *
 * Sources (pages by title):
 *   [PSS]  "One Call Ahead: Packed Self-Speculative Decoding with Diffusion
 *          Drafting" -- Sec. 2.2, Sec. 3.1 (Eq. 1-4, Algorithm 1), Sec. 3.2
 *          (stored sparse Q),
 *          App. B.2 (Algorithm 2, Lemma B.3), App. C (Algorithm 3, any-order
 *          verification), App. D.1 (packed row layout).
 *   [SPOT] "On the SPOT: Enhancing Speculative Decoding for Diffusion Language
 *          Models via Commit-Order Prediction" -- Sec. 4.1, Sec. 4.2 (Eq. 3,
 *          prefix mass; adaptive budget), Sec. 4.3 (Eq. 4), App. A.1 (formal
 *          decoding model), App. A.3 (Eq. 5-7), App. B (Eq. 10-14,
 *          Proposition 3), App. C.2 (Algorithm 2, DDTree), Table 22 (regime
 *          law).
 *   [TT]   "Speculative Diffusion is a Tale of Two Tradeoffs" -- Sec. 2
 *          (Eq. 1-5, Theorem 1), Sec. 3.2 (Algorithm 1), App. E (modified
 *          Cactus, Eq. 17-18).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array argument is a DEVICE pointer, allocated and owned by the
 *   caller; the library keeps no pointer after the call returns.  Optional
 *   arrays may be NULL where stated.
 * - Logit tensors are row-major with the vocabulary contiguous; the other
 *   axes are given as element strides (not bytes), so packed layouts need no
 *   copy.  `dtype` applies to every logit tensor of a call; Gumbel tables and
 *   uniforms are float32; tokens, lengths and tree indices are int32.
 * - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *   stream): they return after enqueueing and outputs are valid once the
 *   stream reaches that point.  No host<->device synchronisation and no
 *   device allocation happen inside a call.
 * - Scratch memory: the caller passes `ws` of at least
 *   verify_workspace_size(...) bytes (device memory, any contents, 256-byte
 *   aligned).  Calls that share a workspace must be ordered on one stream.
 * - Errors: invalid host arguments return a dbv_status and launch nothing.
 *   Data errors found on the device are reported per sequence in `status`
 *   (dbv_seq_status bits; NULL = not reported); a sequence with an error bit
 *   gets accept_len = -1 (path_len = -1), num_out = 0 and -1 in its token
 *   slots.  -inf logits are legal and mean zero probability ([PSS] Lemma B.3:
 *   neither distribution needs full support).
 * - Ties: every argmax takes the largest value and, among equal values, the
 *   lowest index, on the raw (untempered) inputs ([PSS] App. B.2 "fixed
 *   tie-breaking rule"; [SPOT] App. A.1 "fixed deterministic tie-breaking").
 */
#ifndef DBV_H
#define DBV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DBV_ABI_VERSION 2

typedef enum {
  DBV_OK = 0,
  DBV_ERR_INVALID_ARG = 1, /* a host argument is out of range / NULL      */
  DBV_ERR_UNSUPPORTED = 2, /* a valid request beyond the library limits  */
  DBV_ERR_NO_DEVICE = 3,   /* no usable gfx950 device                     */
  DBV_ERR_LAUNCH = 4,      /* a kernel launch failed (hipGetLastError)    */
  DBV_ERR_WORKSPACE = 5    /* ws is NULL / too small / misaligned         */
} dbv_status;

typedef enum { DBV_F32 = 0, DBV_BF16 = 1 } dbv_dtype;

typedef enum {
  DBV_TREE_STATE_EQUALITY = 0, /* s*(y) chosen by max confidence ([SPOT] 4.1) */
  DBV_TREE_FIXED_POSITION = 1  /* s*(y) given per state in next_pos           */
} dbv_tree_mode;

/* Per-sequence status bits written to `status[b]`. */
enum {
  DBV_SEQ_BAD_INPUT = 1,  /* token / length / tree index out of range (error) */
  DBV_SEQ_NONFINITE = 2,  /* a row that is read holds NaN or +inf (error)     */
  DBV_SEQ_EMPTY_ROW = 4,  /* a row that is read is all -inf (error)           */
  DBV_SEQ_Q_ZERO = 8,     /* q(d) == 0 < p~(d): accepted by the rule, flagged */
  DBV_SEQ_Z_ZERO = 16     /* residual mass 0 in float32: drew from p, flagged */
};
#define DBV_SEQ_ERROR_MASK 7

/* Workspace kinds for verify_workspace_size. */
typedef enum {
  DBV_KIND_GREEDY = 0,
  DBV_KIND_REJECTION = 1, /* also verify_lenient, verify_cactus, verify_sparse, verify_spot_chain */
  DBV_KIND_TREE = 2,
  DBV_KIND_ANY_ORDER = 3, /* K_or_S = U (window), L ignored */
  DBV_KIND_DDTREE_HYPOTHESES = 4, /* K_or_S = L (block length) */
  DBV_KIND_DDTREE = 5     /* K_or_S = D (budget), L, V and dtype ignored */
} dbv_kind;

/*
 * dbv_options -- optional per-call settings and diagnostic outputs.  Every
 * entry point that launches kernels takes `const dbv_options* opts` as its
 * last argument; NULL means no options.  The library reads the struct during
 * the call and keeps nothing from it (nor any pointer in it) afterwards, so
 * calls on different streams or threads stay independent.  Set `size` to
 * sizeof(dbv_options) and every field the call does not use to 0 / NULL; a
 * diagnostic output that the entry point does not produce is
 * DBV_ERR_INVALID_ARG.
 *
 *   max_groups  an upper bound on the workgroups of the row-streaming kernel
 *       (0: the library's choice, 4 per compute unit), e.g. to leave compute
 *       units to concurrent work.  Every output is the same for any value, up
 *       to decisions whose float64 margin is below 1e-5 (the float32
 *       reductions are grouped differently).
 *   row_begin, row_end  hipEvent_t handles created with timing enabled (both
 *       or neither).  The call launches its row-streaming kernel (the launch
 *       that reads the logit rows: row statistics / argmax, the tree's
 *       confidences, the truncation pass, the hypotheses' row pass, or the
 *       DDTree search kernel) through hipExtLaunchKernel with these events,
 *       which the runtime stamps at that kernel's own start and end, so
 *       hipEventElapsedTime gives its duration without launch gaps.  A call
 *       with no rows to read records both events back to back.
 *   Chain sampling calls (verify_rejection, verify_lenient, verify_cactus,
 *   verify_sparse, verify_spot_chain), the per-decision margins of
 *   [SPOT] App. B.4's implementation check and [TT] Sec. 2:
 *   accept_margin [B, K] float32: |u_accept - alpha| of each draft i < n_b
 *       (the distance of the accept test from flipping), 0 past n_b; a
 *       coupled-noise match link reports 1.
 *   draw_margin [B] float32: for a drawn correction or bonus token c, the
 *       distance of u * Z from the nearer end of c's interval
 *       [F(c-1), F(c)) of the running mass, over Z; 1 where the committed
 *       token was not drawn (a Gumbel argmax) and for sequences in error.
 *   row_tv [B, K] float32: TV(p_i, q_i) = 1/2 sum_v |p_i(v) - q_i(v)| of
 *       each draft row i < n_b (target and drafter at their temperatures;
 *       [TT] Sec. 2 Eq. 1-2: the lossless acceptance rate of row i is
 *       1 - TV), 0 past n_b and for sequences whose draft length is
 *       invalid, NaN for a row pair that holds NaN / +inf or no finite
 *       logit.  Diagnostic mode: one more kernel, one group per draft row,
 *       reading the draft block's target and drafter rows once more.
 *       verify_sparse: TV against the stored Q, from the stored entries
 *       alone; verify_spot_chain: TV of the token rows, p against qhat.
 *   verify_gumbel_tree:
 *   pos_margin [B, S] float32: relative gap (c1 - c2) / c1 of the two largest
 *       confidences over the masked positions of each state (1 with one
 *       masked position; 0 for terminal and unused states and in
 *       FIXED_POSITION mode).
 *   tok_margin [B, S] float32: the gap between the two largest scores
 *       z_v / T + G[s*, v] (T > 0) or logits (T = 0) at s*: the margin of the
 *       coupled transition's token (0 for terminal and unused states).
 *       Tracking the runner-up score costs one more compare per element of
 *       the selected rows.
 */
typedef struct dbv_options {
  uint32_t size;
  uint32_t max_groups;
  void* row_begin;
  void* row_end;
  float* accept_margin;
  float* draw_margin;
  float* row_tv;
  float* pos_margin;
  float* tok_margin;
} dbv_options;

/*
 * verify_greedy -- temperature-0 verification plus next-draft retention.
 * [PSS] Sec. 3.1 Eq. 1-4 and Algorithm 1:
 *   v_i = argmax of target row i-1 for i = 1..n_b+1            (Eq. 1)
 *   h   = leading matches d_i == v_i, h <= n_b                 (Eq. 2)
 *   C   = (d_1..d_h, v_{h+1}),  A = h + 1
 *   a   = min({A, len_budget[b]} U {i <= A : C_i == eos_id})  (ending condition)
 *   z_j = argmax of draft row j-1, j = 1..W                     (Eq. 3)
 *   next draft = (z_{a+1}, ..., z_W), next_len = max(0, W - a)  (Eq. 4)
 *
 * tgt         [B, K+1, V] at tgt + b*tgt_seq_stride + i*tgt_row_stride:
 *             row i is the verifier conditional at draft position i+1; row
 *             n_b is the bonus row; rows after n_b are not read.
 * draft_tokens[B, K] int32 row-major; draft_len [B] (NULL = K everywhere;
 *             a value outside [0, K] is DBV_SEQ_BAD_INPUT).
 * draft_rows  [B, W, V] drafter rows of the same call (NULL with W = 0 to
 *             skip retention); e.g. the packed layout of [PSS] App. D.1 is
 *             tgt = T, draft_rows = T + (K+1)*V with shared strides.
 * eos_id      -1 disables the EOS term; len_budget [B] (NULL disables; a
 *             negative entry is DBV_SEQ_BAD_INPUT).
 * Outputs: accept_len [B] (= h), out_tokens [B, K+1] (C pruned to a, -1
 * after), num_out [B] (= a), next_draft [B, W] (-1 after next_len; NULL
 * allowed when W = 0), next_len [B] (NULL allowed), status [B] (NULL allowed).
 */
dbv_status verify_greedy(int B, int K, int V, dbv_dtype dtype,
                         const void* tgt, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                         const int32_t* draft_tokens, const int32_t* draft_len,
                         const void* draft_rows, int64_t dr_seq_stride, int64_t dr_row_stride,
                         int W, int32_t eos_id, const int32_t* len_budget,
                         int32_t* accept_len, int32_t* out_tokens, int32_t* num_out,
                         int32_t* next_draft, int32_t* next_len, int32_t* status,
                         void* ws, size_t ws_bytes, void* stream,
                         const dbv_options* opts);

/*
 * verify_rejection -- lossless speculative-sampling verification.
 * [PSS] Sec. 3.2 and Algorithm 2; [TT] Sec. 2 "Lossless Speculative Decoding":
 *   p_i = softmax(tgt row i / T_target), i = 0..n_b
 *   q_i = softmax(drf row i / T_draft),  i = 0..n_b-1  (the distribution d_i
 *         was sampled from -- the stored proposal Q of [PSS] Sec. 3.2)
 *   accept d_i iff u_accept[b,i] < min(1, p_i(d_i) / q_i(d_i))
 *         (evaluated as u*q < p; q(d) = 0 < p(d) accepts and is flagged)
 *   h = leading accepts; if h < n_b the token at position h+1 is drawn from
 *   normalize([p_h - q_h]_+) with u_resample[b,h], else the bonus from p_{n_b}
 *   with u_resample[b,n_b]; draws use the inverse CDF in vocabulary order
 *   (smallest c whose running sum exceeds u * total).  Then the ending
 *   condition as in verify_greedy.
 * drf [B, K, V] (same dtype as tgt); temperatures > 0 and finite;
 * u_accept [B, K], u_resample [B, K+1] float32 in [0, 1).
 * Optional diagnostics (NULL to skip): p_draft, q_draft, alpha [B, K]
 * (0 beyond n_b); residual_mass [B] (sum of [p~-q]_+ at the rejected row,
 * i.e. its rejection probability, 0 when the bonus was drawn; p~ = p here).
 */
dbv_status verify_rejection(int B, int K, int V, dbv_dtype dtype,
                            const void* tgt, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                            const void* drf, int64_t drf_seq_stride, int64_t drf_row_stride,
                            const int32_t* draft_tokens, const int32_t* draft_len,
                            float temperature_target, float temperature_draft,
                            const float* u_accept, const float* u_resample,
                            int32_t eos_id, const int32_t* len_budget,
                            int32_t* accept_len, int32_t* out_tokens, int32_t* num_out,
                            float* p_draft, float* q_draft, float* alpha, float* residual_mass,
                            int32_t* status, void* ws, size_t ws_bytes, void* stream,
                            const dbv_options* opts);

/*
 * verify_rejection_noalloc -- verify_rejection for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same arguments without `ws` and
 * `ws_bytes`, the same kernels and outputs.  Its scratch is a 4 MiB device
 * array inside the library, one per GPU, held until the process ends; no
 * call allocates or frees anything.  A call whose workspace
 * (verify_workspace_size(DBV_KIND_REJECTION, ...)) exceeds 4 MiB returns
 * DBV_ERR_UNSUPPORTED and launches nothing (B = 32, K = 16 at V = 151936
 * needs about 0.4 MiB).  All calls on one GPU share its array, which keeps
 * the last call's contents: calls that overlap on one GPU (on different
 * streams, or from several threads without ordering) race; order them on
 * one stream.  The kernels need no zeroed scratch.
 */
dbv_status verify_rejection_noalloc(int B, int K, int V, dbv_dtype dtype,
                                    const void* tgt, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                                    const void* drf, int64_t drf_seq_stride, int64_t drf_row_stride,
                                    const int32_t* draft_tokens, const int32_t* draft_len,
                                    float temperature_target, float temperature_draft,
                                    const float* u_accept, const float* u_resample,
                                    int32_t eos_id, const int32_t* len_budget,
                                    int32_t* accept_len, int32_t* out_tokens, int32_t* num_out,
                                    float* p_draft, float* q_draft, float* alpha, float* residual_mass,
                                    int32_t* status, void* stream,
                                    const dbv_options* opts);

/*
 * verify_lenient -- the linear lenient rule of [TT] Theorem 1 (Eq. 5) used in
 * [TT] Algorithm 1: the target is relaxed to p~ = (1 - lambda) p + lambda q
 * before the draft is tested; accept iff u < min(1, p~(d)/q(d)); a rejected
 * position draws from normalize([p~ - q]_+) (equal to normalize([p - q]_+)
 * for lambda < 1); the bonus after full acceptance is drawn from p, not p~.
 * lambda in [0, 1]: 0 reproduces verify_rejection bit for bit, 1 accepts
 * every draft with q(d) > 0; a draft with q(d) = 0 is still rejected, and
 * since [p~ - q]_+ is then zero everywhere its position draws from p with
 * the Z = 0 status bit, like any residual of zero mass.  All other
 * arguments as verify_rejection.
 */
dbv_status verify_lenient(int B, int K, int V, dbv_dtype dtype,
                          const void* tgt, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                          const void* drf, int64_t drf_seq_stride, int64_t drf_row_stride,
                          const int32_t* draft_tokens, const int32_t* draft_len,
                          float temperature_target, float temperature_draft, float lambda,
                          const float* u_accept, const float* u_resample,
                          int32_t eos_id, const int32_t* len_budget,
                          int32_t* accept_len, int32_t* out_tokens, int32_t* num_out,
                          float* p_draft, float* q_draft, float* alpha, float* residual_mass,
                          int32_t* status, void* ws, size_t ws_bytes, void* stream,
                          const dbv_options* opts);

/*
 * verify_cactus -- the modified Cactus rule of [TT] App. E: the target is
 * modified after the drafted token d is seen, to the p~ with the largest
 * p~(d) = gamma whose KL divergence from p stays within the budget `delta`,
 * every other token rescaled by (1 - gamma) / (1 - p(d)).  gamma solves
 *   gamma log(gamma / p(d)) + (1 - gamma) log((1 - gamma) / (1 - p(d))) = delta
 * ([TT] App. E, Eq. 17) exactly (Newton's method, as the page does), or is 1
 * when -log p(d) <= delta, or 0 when p(d) = 0.  Accept d iff
 * u_accept < min(1, gamma / q(d)); a rejected position draws from
 * normalize([p~ - q]_+); the bonus after full acceptance is drawn from p.
 * delta >= 0 and finite (DBV_ERR_INVALID_ARG otherwise); delta = 0 is the
 * lossless rule.  alpha reports min(1, gamma / q(d)); residual_mass the sum of
 * [p~ - q]_+ at the rejected row.  All other arguments as verify_rejection.
 */
dbv_status verify_cactus(int B, int K, int V, dbv_dtype dtype,
                         const void* tgt, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                         const void* drf, int64_t drf_seq_stride, int64_t drf_row_stride,
                         const int32_t* draft_tokens, const int32_t* draft_len,
                         float temperature_target, float temperature_draft, float delta,
                         const float* u_accept, const float* u_resample,
                         int32_t eos_id, const int32_t* len_budget,
                         int32_t* accept_len, int32_t* out_tokens, int32_t* num_out,
                         float* p_draft, float* q_draft, float* alpha, float* residual_mass,
                         int32_t* status, void* ws, size_t ws_bytes, void* stream,
                         const dbv_options* opts);

/*
 * verify_sparse -- lossless verification against stored sparse drafter
 * distributions ([PSS] Sec. 3.2: with top-k / top-p truncation only the
 * nonzero entries of each draft's Q need storing; the test is the lossless
 * rule of [PSS] App. B.2, Algorithm 2).  Row i of sequence b stores Q as
 * q_nnz[b, i] entries (token q_idx[b, i, e], probability q_prob[b, i, e]),
 * dense [B, K, kmax] arrays of which the first q_nnz entries are used;
 * tokens off the list have Q = 0.  Accept d_i iff u_accept <
 * min(1, p(d_i) / Q(d_i)); a rejection draws from normalize([p - Q]_+)
 * (= p off the stored support); the bonus after full acceptance is drawn
 * from p.  Q is used as stored (not renormalised); the entries of one row
 * must name distinct tokens (not checked).  Only the target rows are read
 * from HBM.  0 <= kmax <= 256 (DBV_ERR_UNSUPPORTED above).  Bad input
 * (DBV_SEQ_BAD_INPUT) in a row the call reads (i < n_b): q_nnz outside
 * [0, kmax], a token outside [0, V), a probability that is negative or not
 * finite.  Outputs as verify_rejection (q_draft = Q(d_i)).  Workspace kind:
 * DBV_KIND_REJECTION.
 */
dbv_status verify_sparse(int B, int K, int V, dbv_dtype dtype,
                         const void* tgt, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                         const int32_t* q_idx, const float* q_prob, const int32_t* q_nnz, int kmax,
                         const int32_t* draft_tokens, const int32_t* draft_len, float temperature_target,
                         const float* u_accept, const float* u_resample,
                         int32_t eos_id, const int32_t* len_budget,
                         int32_t* accept_len, int32_t* out_tokens, int32_t* num_out,
                         float* p_draft, float* q_draft, float* alpha, float* residual_mass,
                         int32_t* status, void* ws, size_t ws_bytes, void* stream,
                         const dbv_options* opts);

/*
 * truncate_top_k_top_p -- stores drafter distributions in the sparse form
 * verify_sparse reads ([PSS] Sec. 3.2: under top-k or top-p truncation only
 * the nonzero entries of Q need storing).  For row i of sequence b (logits
 * at element offset b*seq_stride + i*row_stride, read only for i <
 * lengths[b]; lengths NULL = K): q = softmax(x / temperature); keep the
 * top_k tokens of largest logit (equal logits: the lower token id first);
 * within them, sorted by probability, keep the shortest prefix whose mass
 * reaches top_p of theirs (all of them for top_p = 1); renormalise.  Writes
 * q_idx[b, i, 0..nnz), q_prob[b, i, 0..nnz) in that order ([B, K, kmax]
 * int32 / float32) and q_nnz[b, i] = nnz; rows not read get nnz = 0; a row
 * holding NaN or +inf, or no finite logit, gets nnz = -1 (verify_sparse
 * then reports DBV_SEQ_BAD_INPUT for a draft that uses it).  Entries past
 * nnz are left as they were.  1 <= top_k <= kmax <= 256, 0 < top_p <= 1,
 * temperature > 0 (DBV_ERR_INVALID_ARG; kmax > 256 or V > 2^21:
 * DBV_ERR_UNSUPPORTED).  No workspace.
 */
dbv_status truncate_top_k_top_p(int B, int K, int V, dbv_dtype dtype,
                                const void* rows, int64_t seq_stride, int64_t row_stride,
                                const int32_t* lengths, float temperature, int top_k, float top_p,
                                int kmax, int32_t* q_idx, float* q_prob, int32_t* q_nnz, void* stream,
                                const dbv_options* opts);

/*
 * verify_spot_chain -- chain verification on the joint (position, token)
 * space ([SPOT] App. B, Eq. 10-14 and Proposition 3), optionally gated
 * per link between rejection sampling and coupled-noise match.  Link k
 * (k = 0..n_b-1) sits at verified state y_k; the target commits at position
 * s*_k = pos_star[b, k] with token law p_k = softmax(tgt row k /
 * temperature_target) (Eq. 10); the drafter proposed (prop_pos[b, k],
 * prop_tok[b, k]) from q_k(s, v) = q_pos_k(s) qhat_{k,s}(v) (Eq. 12), where
 * drf row k holds the drafter's logits at position s*_k (qhat =
 * softmax(drf row / temperature_draft)) and q_pos_star[b, k] = q_pos_k(s*_k)
 * (float32 in [0, 1]).  Row n_b of tgt (position pos_star[b, n_b]) is the
 * bonus row.
 *   Rejection sampling (Eq. 13-14): a proposal off s*_k is rejected; on
 *   s*_k accept iff u_accept < min(1, p_k(v) / (c_k qhat(v))), c_k =
 *   q_pos_star; a rejected link commits at s*_k a draw from
 *   normalize([p_k - c_k qhat]_+) with u_resample[b, k].
 *   Coupled-noise match ([SPOT] Sec. 4.1): with Gumbel rows (gumbel[b, k, :]
 *   float32 at element offset b*g_seq_stride + k*g_row_stride, the shared
 *   noise of position s*_k) a link whose drafter confidence max_v qhat(v)
 *   is >= tau accepts iff the proposal is (s*_k, argmax_v(x_v/T + g_v)); a
 *   rejected match link commits that argmax.  tau > 1 disables match;
 *   gumbel = NULL means rejection sampling on every link.
 *   The bonus after n_b accepted links is the Gumbel argmax of row n_b when
 *   Gumbel rows are given, else a draw from p_{n_b} with u_resample[b, n_b].
 * The committed position of output i is pos_star[b, i].  out_tokens, the
 * ending condition, accept_len, num_out and status as verify_rejection;
 * p_draft = p_k(v), q_draft = c_k qhat(v), alpha = the link's acceptance
 * probability (0 off s*_k; 1 or 0 for a match link), residual_mass = the
 * sum of [p - c qhat]_+ at a rejected rejection-sampling link (0 otherwise).
 * Bad input (DBV_SEQ_BAD_INPUT): q_pos_star outside [0, 1], pos_star < 0 at
 * a link or the bonus row, a proposal token outside [0, V).  With Gumbel
 * rows, every row 0..n_b is read with its Gumbel row and their score rows
 * obey the logit-row rule.  tau must not be NaN.  Workspace kind:
 * DBV_KIND_REJECTION.
 */
dbv_status verify_spot_chain(int B, int K, int V, dbv_dtype dtype,
                             const void* tgt, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                             const void* drf, int64_t drf_seq_stride, int64_t drf_row_stride,
                             const int32_t* pos_star, const int32_t* prop_pos, const int32_t* prop_tok,
                             const float* q_pos_star, const int32_t* draft_len,
                             float temperature_target, float temperature_draft,
                             const float* gumbel, int64_t g_seq_stride, int64_t g_row_stride, float tau,
                             const float* u_accept, const float* u_resample,
                             int32_t eos_id, const int32_t* len_budget,
                             int32_t* accept_len, int32_t* out_tokens, int32_t* num_out,
                             float* p_draft, float* q_draft, float* alpha, float* residual_mass,
                             int32_t* status, void* ws, size_t ws_bytes, void* stream,
                             const dbv_options* opts);

/*
 * verify_greedy_any_order -- one any-order greedy verification call
 * ([PSS] App. C, Algorithm 3, its verification steps).  Per sequence b the call covers
 * the u_b unresolved output positions of its active window, in textual order
 * ("slots" j = 0..u_b-1 at output positions pos[j]), checked in the order
 * pi chosen before the call (order[b, r] = the slot checked at rank r):
 *   kappa = leading ranks whose slot has a draft (draft_tokens >= 0)
 *   v_r   = argmax of verifier row r, r < min(kappa + 1, u)       (Eq. 8)
 *   z_j   = argmax of drafter row j, j < u
 *   h     = leading ranks r < kappa with draft(pi(r)) == v_r
 *   A     = min(h + 1, u),  C = ((pos[pi(r)], v_r))_{r < A}
 *   E'    = min({end_pos[b]} U {pos of an accepted EOS})
 *   C'    = the pairs of C at positions <= E' (in rank order)
 *   next draft: z_j at the slots not in C with pos[j] <= E'.
 *
 * tgt         [B, U, V] verifier rows in rank order (row r is the verifier at
 *             pi(r) given the drafts at earlier ranks); rows at ranks >=
 *             min(kappa + 1, u) are not read.
 * order       [B, U] int32, a permutation of 0..u_b-1 in its first u_b entries.
 * num_active  [B] u_b in [0, U] (NULL = U).
 * positions   [B, U] strictly increasing over the first u_b slots (NULL:
 *             slot j is at position j).
 * draft_tokens[B, U] by slot, -1 = no draft yet, else in [0, V).
 * draft_rows  [B, U, V] drafter rows by slot (NULL: no next draft; then
 *             next_draft, if given, is filled with -1).
 * eos_id      -1 disables the EOS term; end_pos [B] E before the call (NULL:
 *             no limit, reported as INT32_MAX).
 * Outputs: accept_len [B] (= h), num_accepted [B] (= |C'|), acc_pos, acc_tok
 * [B, U] (C' in rank order, -1 after), new_end [B] (= E'), next_draft [B, U]
 * (by slot, -1 where no draft is kept; NULL allowed), status [B] (NULL
 * allowed).  An order that is not a permutation, positions that do not
 * increase, a draft token outside [-1, V) or u_b outside [0, U] is
 * DBV_SEQ_BAD_INPUT; no row of that sequence is read.
 */
dbv_status verify_greedy_any_order(int B, int U, int V, dbv_dtype dtype,
                                   const void* tgt, int64_t tgt_seq_stride, int64_t tgt_row_stride,
                                   const int32_t* order, const int32_t* num_active,
                                   const int32_t* positions, const int32_t* draft_tokens,
                                   const void* draft_rows, int64_t dr_seq_stride, int64_t dr_row_stride,
                                   int32_t eos_id, const int32_t* end_pos,
                                   int32_t* accept_len, int32_t* num_accepted,
                                   int32_t* acc_pos, int32_t* acc_tok, int32_t* new_end,
                                   int32_t* next_draft, int32_t* status,
                                   void* ws, size_t ws_bytes, void* stream,
                                   const dbv_options* opts);

/*
 * verify_gumbel_tree -- state-equality verification of one draft tree per
 * sequence with shared Gumbel noise.  [SPOT] Sec. 4.1, Sec. 4.3, App. A.1:
 *   s*(y)  = argmax over masked positions s of max_v p_s(v | y) (untempered;
 *            ties to the lowest position)                   [STATE_EQUALITY]
 *          = next_pos[b, y] (-1: no transition)              [FIXED_POSITION]
 *   v*(y)  = argmax_v ( z_v / T + G[b, s*, v] )  for T > 0  -- equal to
 *            argmax[(1/T) log p + G] since the row constant drops out;
 *          = argmax_v z_v                         for T = 0 (G may be NULL)
 *   An edge y -> z is accepted iff edge_pos[z] == s*(y) and
 *   edge_tok[z] == v*(y) (z equals Phi(y)); the walk starts at node 0,
 *   follows the accepted child (lowest node index if several), and ends by
 *   committing Phi(y) at the first state with no accepted child; a state
 *   with no masked position (or next_pos = -1) makes no transition.
 *
 * logits  [B, S, L, V] at logits + b*seq_stride + y*state_stride + s*pos_stride:
 *         the target conditional at block position s of state y; only the
 *         masked rows of states y < num_states[b] are read.
 * masked  [B, S, L] uint8 (nonzero = masked); may be NULL in FIXED_POSITION.
 * parent  [B, S]: parent[b,0] = -1, 0 <= parent[b,z] < z; edge_pos [B, S] in
 *         [0, L), edge_tok [B, S] in [0, V) for z >= 1 (entry 0 unused).
 * num_states [B] in [1, S] (NULL = S); next_pos [B, S] in [-1, L)
 *         (FIXED_POSITION only, else NULL).
 * gumbel  [B, L, V] float32 at gumbel + b*g_seq_stride + s*g_pos_stride: the
 *         shared table row of block position s (absolute-position indexing is
 *         the caller's job).  temperature >= 0 and finite.
 * Outputs: sel_pos, sel_tok [B, S] (-1 for terminal / unused states; NULL
 * allowed), sel_conf [B, S] (max_v p at s*, NULL allowed), path_len [B]
 * (accepted edges), path_nodes [B, S] (root first, -1 after), commit_pos,
 * commit_tok [B, S] (accepted edges then the final Phi, -1 after),
 * num_commits [B], status [B] (NULL allowed).
 */
dbv_status verify_gumbel_tree(int B, int S, int L, int V, dbv_dtype dtype,
                              const void* logits, int64_t seq_stride, int64_t state_stride,
                              int64_t pos_stride,
                              const uint8_t* masked, const int32_t* parent,
                              const int32_t* edge_pos, const int32_t* edge_tok,
                              const int32_t* num_states, const int32_t* next_pos,
                              const float* gumbel, int64_t g_seq_stride, int64_t g_pos_stride,
                              float temperature, dbv_tree_mode mode,
                              int32_t* sel_pos, int32_t* sel_tok, float* sel_conf,
                              int32_t* path_len, int32_t* path_nodes,
                              int32_t* commit_pos, int32_t* commit_tok, int32_t* num_commits,
                              int32_t* status, void* ws, size_t ws_bytes, void* stream,
                              const dbv_options* opts);

/*
 * ddtree_hypotheses -- token hypotheses of the masked positions for draft-
 * tree construction ([SPOT] Sec. 4.2 "Inference", App. C.2).  For each
 * position s with masked[b, s] != 0 the stale target row (logits at element
 * offset b*seq_stride + s*pos_stride) gives p^_s = softmax(row) at
 * temperature 1 and H(s):
 *   temperature == 0: the argmax v0 of the logits, and the runner-up v1
 *     (largest logit other than v0) when p^_s(v0) < runner_up_below (0.6 in
 *     [SPOT]);
 *   temperature > 0: the coupled stale draw of Eq. 4, argmax_v (z_v /
 *     temperature + g_v) with the Gumbel row of the position (float32 at
 *     element offset b*g_seq_stride + s*g_pos_stride).
 * Writes hyp_tok[b, s, 0..1] (int32, -1 = none) and hyp_prob[b, s, 0..1]
 * (p^_s of the token, float32, 0 for none), both [B, L, 2]; unmasked
 * positions get (-1, 0) and are not read.  status[b] (NULL allowed) is
 * overwritten: a read row holding NaN or +inf, or no finite logit
 * (DBV_SEQ_NONFINITE / DBV_SEQ_EMPTY_ROW), or a Gumbel score row that is not
 * a distribution.  Ties: lowest index.  1 <= L <= 64.  Workspace kind:
 * DBV_KIND_DDTREE_HYPOTHESES.
 */
dbv_status ddtree_hypotheses(int B, int L, int V, dbv_dtype dtype,
                             const void* stale, int64_t seq_stride, int64_t pos_stride,
                             const uint8_t* masked, const float* gumbel,
                             int64_t g_seq_stride, int64_t g_pos_stride,
                             float temperature, float runner_up_below,
                             int32_t* hyp_tok, float* hyp_prob, int32_t* status,
                             void* ws, size_t ws_bytes, void* stream,
                             const dbv_options* opts);

/*
 * ddtree_level -- one level of the DDTree search ([SPOT] Sec. 4.2 Eq. 3 and
 * App. C.2 Algorithm 2), with the order model run by the caller between
 * levels.  State: node 0 is the current state x_t (mass 1, masked positions
 * masked[b, :]); every other node z is a hypothetical state y (+) (s, v)
 * with parent[b, z] < z, edge_pos = s, edge_tok = v and prefix mass
 *   m(z) = m(y) q(s | y) p^_s(v)                                  (Eq. 3)
 * where p^_s(v) = hyp_prob of token v at s (from ddtree_hypotheses) and
 * q(s | y) = softmax over the masked positions M(y) of the order logits /
 * tau (the calibration temperature).  A level takes each state of the
 * frontier (the states admitted by the previous level; the root on the
 * first level, first != 0, which also resets the tree), reads its order
 * logits from row j of order_logits (float32 at element offset
 * b*o_seq_stride + j*o_row_stride for frontier slot j; only entries at M(y)
 * are read), forms every child y (+) (s, v), s in M(y), v in H(s), with
 * m >= gamma (the prefix-mass floor; 0 keeps all), and keeps the D states
 * of largest mass among the tree and the new children; the frontier becomes
 * the children so admitted.  Repeat until num_frontier is 0: the tree then
 * holds the D states of largest mass (sequential best-first order).
 * Outputs (caller-owned, carried between levels; rewritten by each call):
 * nodes in rank order (mass descending, then depth ascending, then the
 * order of creation), parent / edge_pos / edge_tok [B, D+1] int32 (-1 past
 * num_nodes), mass [B, D+1] float32, node_masked [B, D+1, L] uint8 (the
 * masked positions of each state; NULL allowed), num_nodes [B] (incl. the
 * root), frontier [B, D] (node indices, -1 past num_frontier),
 * num_frontier [B].  The layout is the one verify_gumbel_tree reads (S =
 * D+1).  status [B] (NULL allowed) is read and or-ed: a sequence that
 * enters with an error bit is left as it is (on the first level its tree
 * becomes the root alone); an order row with NaN or +inf on M(y) or no
 * finite entry there, a missing argmax hypothesis or a probability outside
 * [0, 1] at a masked position is an error that stops the sequence.  The
 * workspace (kind DBV_KIND_DDTREE) holds the search state from one level
 * to the next: use the same one for every level of a search.  1 <= L <= 64,
 * 0 <= D <= 64, tau > 0, gamma >= 0.
 */
dbv_status ddtree_level(int B, int L, int D, const uint8_t* masked,
                        const int32_t* hyp_tok, const float* hyp_prob,
                        const float* order_logits, int64_t o_seq_stride, int64_t o_row_stride,
                        float tau, float gamma, int first,
                        int32_t* parent, int32_t* edge_pos, int32_t* edge_tok, float* mass,
                        uint8_t* node_masked, int32_t* num_nodes, int32_t* frontier,
                        int32_t* num_frontier, int32_t* status, void* ws, size_t ws_bytes, void* stream,
                        const dbv_options* opts);

/*
 * ddtree_build -- the whole DDTree search in one call with a first-order
 * order model: the order logits of state y are row c of order_table
 * (float32 at element offset b*t_seq_stride + c*t_row_stride), c = the
 * position committed by y's last edge, or c = L for the root; the table
 * has L + 1 rows of L entries per sequence.  Runs the levels of
 * ddtree_level until no state is admitted (num_frontier = 0 on return) and
 * writes the same outputs.  Workspace kind DBV_KIND_DDTREE.
 */
dbv_status ddtree_build(int B, int L, int D, const uint8_t* masked,
                        const int32_t* hyp_tok, const float* hyp_prob,
                        const float* order_table, int64_t t_seq_stride, int64_t t_row_stride,
                        float tau, float gamma,
                        int32_t* parent, int32_t* edge_pos, int32_t* edge_tok, float* mass,
                        uint8_t* node_masked, int32_t* num_nodes, int32_t* frontier,
                        int32_t* num_frontier, int32_t* status, void* ws, size_t ws_bytes, void* stream,
                        const dbv_options* opts);

/*
 * verify_workspace_size -- bytes of scratch one call of `kind` needs.
 *   DBV_KIND_GREEDY:    K_or_S = K, L = W (draft rows)
 *   DBV_KIND_REJECTION: K_or_S = K, L ignored
 *   DBV_KIND_TREE:      K_or_S = S, L = block length
 *   DBV_KIND_ANY_ORDER: K_or_S = U, L ignored
 *   DBV_KIND_DDTREE_HYPOTHESES: K_or_S = L (block length), V, dtype
 *   DBV_KIND_DDTREE:    K_or_S = D (budget); L, V and dtype ignored
 * Returns 0 for invalid sizes.  Depends only on its arguments.
 */
size_t verify_workspace_size(dbv_kind kind, int B, int K_or_S, int L, int V, dbv_dtype dtype);

/* Static text for a dbv_status (never NULL). */
const char* verify_status_string(dbv_status s);

/* DBV_ABI_VERSION of the loaded library. */
int verify_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DBV_H */
