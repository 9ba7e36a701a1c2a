// libdbv C ABI: argument validation, workspace layout and kernel enqueueing.
// The operations are defined in include/dbv.h; this file only checks what the
// host can check and hands the call to the kernels on the caller's stream.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstddef>
#include <cstring>

#include <hip/hip_runtime.h>

#include "../../include/dbv.h"
#include "dbv_launch.h"
#include "dbv_plan.h"

// Scratch of verify_rejection_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never uses its name as
// an address: scratch_address() keeps, per GPU, the device address that
// hipGetSymbolAddress returns for it (looked up on the entry point's first
// call there, with that device current).
constexpr size_t kNoAllocBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {

using dbv::kMaxBlockLen;
using dbv::kMaxDraft;
using dbv::kMaxStates;

constexpr int kMaxDevices = 64;
// Compute units per device, filled with the architecture check.
std::atomic<int> g_cus[kMaxDevices];
// 0 = not yet queried, 1 = gfx950, 2 = some other device.
std::atomic<int> g_arch[kMaxDevices];

// A usable gfx950 device must be current.
dbv_status device_ready() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    return DBV_ERR_NO_DEVICE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DBV_ERR_NO_DEVICE;
  if (dev < kMaxDevices) {
    int s = g_arch[dev].load(std::memory_order_relaxed);
    if (s == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DBV_ERR_NO_DEVICE;
      s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
      g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
      g_arch[dev].store(s, std::memory_order_relaxed);
    }
    if (s != 1) return DBV_ERR_NO_DEVICE;
  }
  return DBV_OK;
}

// The options of one call (include/dbv.h, dbv_options), read once: fields
// past the caller's `size` count as unset.
struct CallOpts {
  dbv::TimingEvents ev;
  int64_t max_groups = 0;             // 0: no bound beyond the device's
  float* accept_margin = nullptr;
  float* draw_margin = nullptr;
  float* row_tv = nullptr;
  float* pos_margin = nullptr;
  float* tok_margin = nullptr;
};

template <typename T>
T opt_field(const dbv_options* o, T dbv_options::*f, size_t off) {
  return (o && o->size >= off + sizeof(T)) ? o->*f : T();
}

// false: a malformed struct (a size too small to hold the timing events, or
// only one of the two events).
bool read_opts(const dbv_options* o, CallOpts& c) {
  if (o == nullptr) return true;
  if (o->size < offsetof(dbv_options, row_end) + sizeof(void*)) return false;
  void* b = o->row_begin;
  void* e = o->row_end;
  if ((b == nullptr) != (e == nullptr)) return false;
  c.max_groups = o->max_groups;
  c.ev.begin = static_cast<hipEvent_t>(b);
  c.ev.end = static_cast<hipEvent_t>(e);
  c.accept_margin = opt_field(o, &dbv_options::accept_margin, offsetof(dbv_options, accept_margin));
  c.draw_margin = opt_field(o, &dbv_options::draw_margin, offsetof(dbv_options, draw_margin));
  c.row_tv = opt_field(o, &dbv_options::row_tv, offsetof(dbv_options, row_tv));
  c.pos_margin = opt_field(o, &dbv_options::pos_margin, offsetof(dbv_options, pos_margin));
  c.tok_margin = opt_field(o, &dbv_options::tok_margin, offsetof(dbv_options, tok_margin));
  return true;
}

// Groups of a row-streaming launch: the device's resident groups, bounded
// by the caller's max_groups.
int64_t group_cap(const CallOpts& c) {
  const int64_t r = dbv::resident_groups();
  return c.max_groups > 0 && c.max_groups < r ? c.max_groups : r;
}

// Options of an entry point without chain or tree diagnostics.
bool read_plain_opts(const dbv_options* o, CallOpts& c) {
  return read_opts(o, c) && !c.accept_margin && !c.draw_margin && !c.row_tv && !c.pos_margin && !c.tok_margin;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

std::atomic<void*> g_scratch[kMaxDevices];

// The current device's address of `scratch`, or NULL.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

size_t elem_bytes(dbv_dtype dt) { return dt == DBV_BF16 ? 2 : 4; }

bool dtype_ok(dbv_dtype dt) { return dt == DBV_F32 || dt == DBV_BF16; }

dbv_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return DBV_OK;
  if (ws == nullptr || ws_bytes < need || !aligned(ws, 256)) return DBV_ERR_WORKSPACE;
  return DBV_OK;
}

bool temp_ok(float t) { return std::isfinite(t) && t > 0.f; }

// Stream rows are indexed in 32 bits on the device; element offsets in 64.
bool stream_fits(int64_t max_rows, int64_t V) {
  return max_rows < (int64_t(1) << 31) && max_rows * V < (int64_t(1) << 52);
}

// The acceptance rule of a sampling call and its parameters.
struct Rule {
  int rule = dbv::RULE_LINEAR;
  float lam = 0.f;                      // linear rule
  float delta = 0.f;                    // Cactus rule
  const int32_t* pos_star = nullptr;    // joint-space chain
  const int32_t* prop_pos = nullptr;
  const float* qpos = nullptr;
  const float* gumbel = nullptr;
  int64_t gs = 0, grs = 0;
  float tau = 0.f;
  const int32_t* qidx = nullptr;        // stored sparse Q
  const float* qprob = nullptr;
  const int32_t* qnnz = nullptr;
  int kmax = 0;
};

dbv_status sample_common(int B, int K, int V, dbv_dtype dtype, const void* tgt, int64_t ts, int64_t tr,
                         const void* drf, int64_t ds, int64_t dr, const int32_t* draft_tokens,
                         const int32_t* draft_len, float tt, float td, const Rule& rl,
                         const float* u_accept,
                         const float* u_resample, int32_t eos_id, const int32_t* len_budget,
                         int32_t* accept_len, int32_t* out_tokens, int32_t* num_out, float* p_draft,
                         float* q_draft, float* alpha, float* residual_mass, int32_t* status, void* ws,
                         size_t ws_bytes, void* stream, const dbv_options* opts, bool noalloc = false) {
  if (B < 0 || K < 0 || K > kMaxDraft || V < 1 || !dtype_ok(dtype)) return DBV_ERR_INVALID_ARG;
  CallOpts co;
  if (!read_opts(opts, co) || co.pos_margin || co.tok_margin) return DBV_ERR_INVALID_ARG;
  if (V > dbv::kMaxSampleV) return DBV_ERR_UNSUPPORTED;
  if (!temp_ok(tt) || !temp_ok(td) || !(rl.lam >= 0.f && rl.lam <= 1.f)) return DBV_ERR_INVALID_ARG;
  if (!(std::isfinite(rl.delta) && rl.delta >= 0.f)) return DBV_ERR_INVALID_ARG;
  if (rl.rule == dbv::RULE_SPOT) {
    if (rl.pos_star == nullptr || (K > 0 && (rl.prop_pos == nullptr || rl.qpos == nullptr)))
      return DBV_ERR_INVALID_ARG;
    if (std::isnan(rl.tau) || rl.gs < 0 || rl.grs < 0) return DBV_ERR_INVALID_ARG;
    if (rl.gumbel && !aligned(rl.gumbel, 4)) return DBV_ERR_INVALID_ARG;
  }
  if (ts < 0 || tr < 0 || ds < 0 || dr < 0) return DBV_ERR_INVALID_ARG;
  const bool sparse = rl.rule == dbv::RULE_SPARSE;
  if (tgt == nullptr || u_resample == nullptr) return DBV_ERR_INVALID_ARG;
  if (K > 0 && ((!sparse && drf == nullptr) || draft_tokens == nullptr || u_accept == nullptr))
    return DBV_ERR_INVALID_ARG;
  if (sparse) {
    if (rl.kmax < 0) return DBV_ERR_INVALID_ARG;
    if (rl.kmax > dbv::kMaxNnz) return DBV_ERR_UNSUPPORTED;
    if (K > 0 && (rl.qnnz == nullptr || (rl.kmax > 0 && (rl.qidx == nullptr || rl.qprob == nullptr))))
      return DBV_ERR_INVALID_ARG;
  }
  if (accept_len == nullptr || out_tokens == nullptr || num_out == nullptr) return DBV_ERR_INVALID_ARG;
  const size_t eb = elem_bytes(dtype);
  if (!aligned(tgt, eb) || (drf && !aligned(drf, eb))) return DBV_ERR_INVALID_ARG;
  const dbv::SamplePlan plan = dbv::plan_sample(B, K, V, static_cast<int64_t>(elem_bytes(dtype)));
  if (!stream_fits(plan.max_vrows, V)) return DBV_ERR_UNSUPPORTED;
  dbv_status s = DBV_OK;
  if (noalloc) {
    if (plan.bytes > kNoAllocBytes) return DBV_ERR_UNSUPPORTED;
  } else if ((s = check_ws(ws, ws_bytes, plan.bytes)) != DBV_OK) {
    return s;
  }
  if ((s = device_ready()) != DBV_OK) return s;
  if (noalloc && (ws = scratch_address()) == nullptr) return DBV_ERR_NO_DEVICE;
  if (B == 0) return DBV_OK;

  dbv::SampleArgs a{};
  a.B = B; a.K = K; a.V = V;
  a.tgt = tgt; a.ts = ts; a.tr = tr;
  a.drf = drf; a.ds = ds; a.dr = dr;
  a.draft_tokens = draft_tokens; a.draft_len = draft_len;
  a.kp = dbv::kLog2eHost / tt; a.kq = dbv::kLog2eHost / td;
  a.rule = rl.rule;
  a.lam = rl.lam;
  a.delta = rl.delta;
  a.pos_star = rl.pos_star; a.prop_pos = rl.prop_pos; a.qpos = rl.qpos;
  a.gumbel = rl.gumbel; a.gs = rl.gs; a.grs = rl.grs;
  a.inv_t = 1.f / tt;
  a.tau = rl.tau;
  a.qidx = rl.qidx; a.qprob = rl.qprob; a.qnnz = rl.qnnz; a.kmax = rl.kmax;
  a.drows = sparse ? 0 : 1;
  a.u_accept = u_accept; a.u_resample = u_resample;
  a.eos = eos_id; a.budget = len_budget;
  a.accept_len = accept_len; a.out_tokens = out_tokens; a.num_out = num_out;
  a.p_draft = p_draft; a.q_draft = q_draft; a.alpha = alpha; a.residual_mass = residual_mass;
  a.status = status;
  a.accept_margin = co.accept_margin;
  a.draw_margin = co.draw_margin;
  a.row_tv = co.row_tv;
  char* w = static_cast<char*>(ws);
  a.stats = reinterpret_cast<dbv::Stat64*>(w + plan.off_stats);
  a.gpart = reinterpret_cast<float2*>(w + plan.off_gpart);
  a.pre = reinterpret_cast<int32_t*>(w + plan.off_pre);
  a.rec = reinterpret_cast<dbv::DrawRecord*>(w + plan.off_rec);
  a.tmass = reinterpret_cast<float*>(w + plan.off_tmass);
  a.sq = reinterpret_cast<dbv::SparseRow*>(w + plan.off_sq);
  a.blk = B > dbv::kSeqBlocks ? reinterpret_cast<int32_t*>(w + plan.off_blk) : nullptr;
  const int64_t P = rl.gumbel ? dbv::gumbel_parts(static_cast<int64_t>(eb)) : 1;
  a.grid = dbv::stream_grid(static_cast<int64_t>(B) * (P * (K + 1) + K), V, static_cast<int64_t>(eb),
                            group_cap(co), dbv::sample_max_grid(V, static_cast<int64_t>(eb), rl.gumbel));
  a.tiles = static_cast<int>(plan.tiles);
  a.tpc = static_cast<int>(plan.tpc);
  a.chunks = static_cast<int>(plan.chunks);
  return dbv::launch_sample(a, dtype, static_cast<hipStream_t>(stream), co.ev) ? DBV_OK : DBV_ERR_LAUNCH;
}

Rule lenient_rule(float lam) {
  Rule r;
  r.lam = lam;
  return r;
}

Rule cactus_rule(float delta) {
  Rule r;
  r.rule = dbv::RULE_CACTUS;
  r.delta = delta;
  return r;
}

dbv_status dd_tree_common(int B, int L, int D, const uint8_t* masked, const int32_t* hyp_tok,
                          const float* hyp_prob, const float* order, int64_t os, int64_t orow, int table,
                          float tau, float gamma, int first, int32_t* parent, int32_t* edge_pos,
                          int32_t* edge_tok, float* mass, uint8_t* node_masked, int32_t* num_nodes,
                          int32_t* frontier, int32_t* num_frontier, int32_t* status, void* ws,
                          size_t ws_bytes, void* stream, const dbv_options* opts) {
  if (B < 0 || L < 1 || L > dbv::kDDMaxBlock || D < 0 || D > dbv::kDDMaxBudget) return DBV_ERR_INVALID_ARG;
  CallOpts co;
  if (!read_plain_opts(opts, co)) return DBV_ERR_INVALID_ARG;
  if (os < 0 || orow < 0 || !(std::isfinite(tau) && tau > 0.f) || !(std::isfinite(gamma) && gamma >= 0.f))
    return DBV_ERR_INVALID_ARG;
  if (B > 0 && (masked == nullptr || hyp_tok == nullptr || hyp_prob == nullptr || order == nullptr ||
                parent == nullptr || edge_pos == nullptr || edge_tok == nullptr || mass == nullptr ||
                num_nodes == nullptr || num_frontier == nullptr || (D > 0 && frontier == nullptr)))
    return DBV_ERR_INVALID_ARG;
  if (order && !aligned(order, 4)) return DBV_ERR_INVALID_ARG;
  dbv_status s = check_ws(ws, ws_bytes, dbv::dd_tree_bytes(B, D));
  if (s != DBV_OK) return s;
  if ((s = device_ready()) != DBV_OK) return s;
  if (B == 0) return DBV_OK;
  dbv::DDTreeArgs a{};
  a.B = B; a.L = L; a.D = D;
  a.masked = masked; a.hyp_tok = hyp_tok; a.hyp_prob = hyp_prob;
  a.order = order; a.os = os; a.orow = orow;
  a.table = table; a.first = first ? 1 : 0;
  a.inv_tau = 1.f / tau; a.gamma = gamma;
  a.parent = parent; a.edge_pos = edge_pos; a.edge_tok = edge_tok; a.mass = mass;
  a.node_masked = node_masked;
  a.num_nodes = num_nodes; a.frontier = frontier; a.num_frontier = num_frontier;
  a.status = status;
  a.keys = static_cast<uint64_t*>(ws);
  a.masks = a.keys + static_cast<size_t>(B) * (D + 1);
  return dbv::launch_dd_tree(a, static_cast<hipStream_t>(stream), co.ev) ? DBV_OK : DBV_ERR_LAUNCH;
}

}  // namespace

namespace dbv {

// Resident groups of the current device (kResidentPerCU per CU).
int64_t resident_groups() {
  int dev = 0;
  int cus = 256;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) cus = c;
  }
  return static_cast<int64_t>(cus) * kResidentPerCU;
}

}  // namespace dbv

extern "C" {

dbv_status verify_greedy(int B, int K, int V, dbv_dtype dtype, const void* tgt, int64_t tgt_seq_stride,
                         int64_t tgt_row_stride, const int32_t* draft_tokens, const int32_t* draft_len,
                         const void* draft_rows, int64_t dr_seq_stride, int64_t dr_row_stride, int W,
                         int32_t eos_id, const int32_t* len_budget, int32_t* accept_len, int32_t* out_tokens,
                         int32_t* num_out, int32_t* next_draft, int32_t* next_len, int32_t* status, void* ws,
                         size_t ws_bytes, void* stream, const dbv_options* opts) {
  if (B < 0 || K < 0 || K > kMaxDraft || W < 0 || W > kMaxDraft || V < 1 || !dtype_ok(dtype))
    return DBV_ERR_INVALID_ARG;
  CallOpts co;
  if (!read_plain_opts(opts, co)) return DBV_ERR_INVALID_ARG;
  if (tgt_seq_stride < 0 || tgt_row_stride < 0 || dr_seq_stride < 0 || dr_row_stride < 0)
    return DBV_ERR_INVALID_ARG;
  if (tgt == nullptr || (K > 0 && draft_tokens == nullptr) || (W > 0 && draft_rows == nullptr))
    return DBV_ERR_INVALID_ARG;
  if (accept_len == nullptr || out_tokens == nullptr || num_out == nullptr) return DBV_ERR_INVALID_ARG;
  const size_t eb = elem_bytes(dtype);
  if (!aligned(tgt, eb) || (draft_rows && !aligned(draft_rows, eb))) return DBV_ERR_INVALID_ARG;
  const dbv::GreedyPlan plan = dbv::plan_greedy(B, K, W, V);
  if (!stream_fits(plan.max_rows, V)) return DBV_ERR_UNSUPPORTED;
  dbv_status s = check_ws(ws, ws_bytes, plan.bytes);
  if (s != DBV_OK) return s;
  if ((s = device_ready()) != DBV_OK) return s;
  if (B == 0) return DBV_OK;

  dbv::GreedyArgs a{};
  a.B = B; a.K = K; a.V = V; a.W = W;
  a.tgt = tgt; a.ts = tgt_seq_stride; a.tr = tgt_row_stride;
  a.dr = draft_rows; a.ds = dr_seq_stride; a.drr = dr_row_stride;
  a.draft_tokens = draft_tokens; a.draft_len = draft_len;
  a.eos = eos_id; a.budget = len_budget;
  a.accept_len = accept_len; a.out_tokens = out_tokens; a.num_out = num_out;
  a.next_draft = next_draft; a.next_len = next_len; a.status = status;
  a.part = reinterpret_cast<float2*>(static_cast<char*>(ws) + plan.off_part);
  a.pre = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + plan.off_pre);
  a.elem_bytes = static_cast<int>(eb);
  a.grid = dbv::stream_grid(plan.max_rows, V, static_cast<int64_t>(eb), group_cap(co));
  return dbv::launch_greedy(a, dtype, static_cast<hipStream_t>(stream), co.ev) ? DBV_OK : DBV_ERR_LAUNCH;
}

dbv_status verify_rejection(int B, int K, int V, dbv_dtype dtype, const void* tgt, int64_t tgt_seq_stride,
                            int64_t tgt_row_stride, const void* drf, int64_t drf_seq_stride,
                            int64_t drf_row_stride, const int32_t* draft_tokens, const int32_t* draft_len,
                            float temperature_target, float temperature_draft, const float* u_accept,
                            const float* u_resample, int32_t eos_id, const int32_t* len_budget,
                            int32_t* accept_len, int32_t* out_tokens, int32_t* num_out, float* p_draft,
                            float* q_draft, float* alpha, float* residual_mass, int32_t* status, void* ws,
                            size_t ws_bytes, void* stream, const dbv_options* opts) {
  return sample_common(B, K, V, dtype, tgt, tgt_seq_stride, tgt_row_stride, drf, drf_seq_stride,
                       drf_row_stride, draft_tokens, draft_len, temperature_target, temperature_draft,
                       Rule{}, u_accept, u_resample, eos_id, len_budget, accept_len, out_tokens, num_out, p_draft,
                       q_draft, alpha, residual_mass, status, ws, ws_bytes, stream, opts);
}

dbv_status verify_rejection_noalloc(int B, int K, int V, dbv_dtype dtype, const void* tgt, int64_t tgt_seq_stride,
                                    int64_t tgt_row_stride, const void* drf, int64_t drf_seq_stride,
                                    int64_t drf_row_stride, const int32_t* draft_tokens, const int32_t* draft_len,
                                    float temperature_target, float temperature_draft, const float* u_accept,
                                    const float* u_resample, int32_t eos_id, const int32_t* len_budget,
                                    int32_t* accept_len, int32_t* out_tokens, int32_t* num_out, float* p_draft,
                                    float* q_draft, float* alpha, float* residual_mass, int32_t* status,
                                    void* stream, const dbv_options* opts) {
  // Validated as verify_rejection; the workspace is the library's scratch.
  return sample_common(B, K, V, dtype, tgt, tgt_seq_stride, tgt_row_stride, drf, drf_seq_stride,
                       drf_row_stride, draft_tokens, draft_len, temperature_target, temperature_draft,
                       Rule{}, u_accept, u_resample, eos_id, len_budget, accept_len, out_tokens, num_out, p_draft,
                       q_draft, alpha, residual_mass, status, nullptr, kNoAllocBytes, stream, opts, true);
}

dbv_status verify_lenient(int B, int K, int V, dbv_dtype dtype, const void* tgt, int64_t tgt_seq_stride,
                          int64_t tgt_row_stride, const void* drf, int64_t drf_seq_stride, int64_t drf_row_stride,
                          const int32_t* draft_tokens, const int32_t* draft_len, float temperature_target,
                          float temperature_draft, float lambda, const float* u_accept, const float* u_resample,
                          int32_t eos_id, const int32_t* len_budget, int32_t* accept_len, int32_t* out_tokens,
                          int32_t* num_out, float* p_draft, float* q_draft, float* alpha, float* residual_mass,
                          int32_t* status, void* ws, size_t ws_bytes, void* stream, const dbv_options* opts) {
  return sample_common(B, K, V, dtype, tgt, tgt_seq_stride, tgt_row_stride, drf, drf_seq_stride,
                       drf_row_stride, draft_tokens, draft_len, temperature_target, temperature_draft,
                       lenient_rule(lambda), u_accept, u_resample, eos_id, len_budget, accept_len, out_tokens,
                       num_out, p_draft,
                       q_draft, alpha, residual_mass, status, ws, ws_bytes, stream, opts);
}

dbv_status verify_cactus(int B, int K, int V, dbv_dtype dtype, const void* tgt, int64_t tgt_seq_stride,
                         int64_t tgt_row_stride, const void* drf, int64_t drf_seq_stride, int64_t drf_row_stride,
                         const int32_t* draft_tokens, const int32_t* draft_len, float temperature_target,
                         float temperature_draft, float delta, const float* u_accept, const float* u_resample,
                         int32_t eos_id, const int32_t* len_budget, int32_t* accept_len, int32_t* out_tokens,
                         int32_t* num_out, float* p_draft, float* q_draft, float* alpha, float* residual_mass,
                         int32_t* status, void* ws, size_t ws_bytes, void* stream, const dbv_options* opts) {
  return sample_common(B, K, V, dtype, tgt, tgt_seq_stride, tgt_row_stride, drf, drf_seq_stride,
                       drf_row_stride, draft_tokens, draft_len, temperature_target, temperature_draft,
                       cactus_rule(delta), u_accept, u_resample, eos_id, len_budget, accept_len,
                       out_tokens, num_out, p_draft, q_draft, alpha, residual_mass, status, ws, ws_bytes, stream, opts);
}

dbv_status verify_spot_chain(int B, int K, int V, dbv_dtype dtype, const void* tgt, int64_t tgt_seq_stride,
                             int64_t tgt_row_stride, const void* drf, int64_t drf_seq_stride,
                             int64_t drf_row_stride, const int32_t* pos_star, const int32_t* prop_pos,
                             const int32_t* prop_tok, const float* q_pos_star, const int32_t* draft_len,
                             float temperature_target, float temperature_draft, const float* gumbel,
                             int64_t g_seq_stride, int64_t g_row_stride, float tau, const float* u_accept,
                             const float* u_resample, int32_t eos_id, const int32_t* len_budget,
                             int32_t* accept_len, int32_t* out_tokens, int32_t* num_out, float* p_draft,
                             float* q_draft, float* alpha, float* residual_mass, int32_t* status, void* ws,
                             size_t ws_bytes, void* stream, const dbv_options* opts) {
  Rule r;
  r.rule = dbv::RULE_SPOT;
  r.pos_star = pos_star;
  r.prop_pos = prop_pos;
  r.qpos = q_pos_star;
  r.gumbel = gumbel;
  r.gs = g_seq_stride;
  r.grs = g_row_stride;
  r.tau = tau;
  return sample_common(B, K, V, dtype, tgt, tgt_seq_stride, tgt_row_stride, drf, drf_seq_stride,
                       drf_row_stride, prop_tok, draft_len, temperature_target, temperature_draft, r, u_accept,
                       u_resample, eos_id, len_budget, accept_len, out_tokens, num_out, p_draft, q_draft, alpha,
                       residual_mass, status, ws, ws_bytes, stream, opts);
}

dbv_status verify_sparse(int B, int K, int V, dbv_dtype dtype, const void* tgt, int64_t tgt_seq_stride,
                         int64_t tgt_row_stride, const int32_t* q_idx, const float* q_prob, const int32_t* q_nnz,
                         int kmax, const int32_t* draft_tokens, const int32_t* draft_len, float temperature_target,
                         const float* u_accept, const float* u_resample, int32_t eos_id, const int32_t* len_budget,
                         int32_t* accept_len, int32_t* out_tokens, int32_t* num_out, float* p_draft,
                         float* q_draft, float* alpha, float* residual_mass, int32_t* status, void* ws,
                         size_t ws_bytes, void* stream, const dbv_options* opts) {
  Rule r;
  r.rule = dbv::RULE_SPARSE;
  r.qidx = q_idx;
  r.qprob = q_prob;
  r.qnnz = q_nnz;
  r.kmax = kmax;
  return sample_common(B, K, V, dtype, tgt, tgt_seq_stride, tgt_row_stride, nullptr, 0, 0, draft_tokens,
                       draft_len, temperature_target, 1.f, r, u_accept, u_resample, eos_id, len_budget, accept_len,
                       out_tokens, num_out, p_draft, q_draft, alpha, residual_mass, status, ws, ws_bytes, stream, opts);
}

dbv_status truncate_top_k_top_p(int B, int K, int V, dbv_dtype dtype, const void* rows, int64_t seq_stride,
                                int64_t row_stride, const int32_t* lengths, float temperature, int top_k,
                                float top_p, int kmax, int32_t* q_idx, float* q_prob, int32_t* q_nnz,
                                void* stream, const dbv_options* opts) {
  if (B < 0 || K < 0 || V < 1 || !dtype_ok(dtype) || seq_stride < 0 || row_stride < 0) return DBV_ERR_INVALID_ARG;
  CallOpts co;
  if (!read_plain_opts(opts, co)) return DBV_ERR_INVALID_ARG;
  if (V > dbv::kMaxSampleV || kmax > dbv::kMaxNnz) return DBV_ERR_UNSUPPORTED;
  if (!temp_ok(temperature) || kmax < 1 || top_k < 1 || top_k > kmax || !(top_p > 0.f && top_p <= 1.f))
    return DBV_ERR_INVALID_ARG;
  if (static_cast<int64_t>(B) * K > 0 && (rows == nullptr || q_idx == nullptr || q_prob == nullptr ||
                                           q_nnz == nullptr))
    return DBV_ERR_INVALID_ARG;
  if (rows && !aligned(rows, elem_bytes(dtype))) return DBV_ERR_INVALID_ARG;
  dbv_status s = device_ready();
  if (s != DBV_OK) return s;
  if (static_cast<int64_t>(B) * K == 0) return DBV_OK;
  dbv::TruncArgs a{};
  a.B = B; a.K = K; a.V = V;
  a.rows = rows; a.ss = seq_stride; a.rs = row_stride;
  a.lengths = lengths;
  a.kq = dbv::kLog2eHost / temperature;
  a.top_k = top_k; a.top_p = top_p; a.kmax = kmax;
  a.q_idx = q_idx; a.q_prob = q_prob; a.q_nnz = q_nnz;
  return dbv::launch_truncate(a, dtype, static_cast<hipStream_t>(stream), co.ev) ? DBV_OK
                                                                                         : DBV_ERR_LAUNCH;
}

dbv_status verify_greedy_any_order(int B, int U, int V, dbv_dtype dtype, const void* tgt, int64_t tgt_seq_stride,
                                   int64_t tgt_row_stride, const int32_t* order, const int32_t* num_active,
                                   const int32_t* positions, const int32_t* draft_tokens, const void* draft_rows,
                                   int64_t dr_seq_stride, int64_t dr_row_stride, int32_t eos_id,
                                   const int32_t* end_pos, int32_t* accept_len, int32_t* num_accepted,
                                   int32_t* acc_pos, int32_t* acc_tok, int32_t* new_end, int32_t* next_draft,
                                   int32_t* status, void* ws, size_t ws_bytes, void* stream, const dbv_options* opts) {
  if (B < 0 || U < 0 || U > kMaxDraft || V < 1 || !dtype_ok(dtype)) return DBV_ERR_INVALID_ARG;
  CallOpts co;
  if (!read_plain_opts(opts, co)) return DBV_ERR_INVALID_ARG;
  if (tgt_seq_stride < 0 || tgt_row_stride < 0 || dr_seq_stride < 0 || dr_row_stride < 0)
    return DBV_ERR_INVALID_ARG;
  if (tgt == nullptr || (U > 0 && (order == nullptr || draft_tokens == nullptr))) return DBV_ERR_INVALID_ARG;
  if (accept_len == nullptr || num_accepted == nullptr || acc_pos == nullptr || acc_tok == nullptr ||
      new_end == nullptr)
    return DBV_ERR_INVALID_ARG;
  const size_t eb = elem_bytes(dtype);
  if (!aligned(tgt, eb) || (draft_rows && !aligned(draft_rows, eb))) return DBV_ERR_INVALID_ARG;
  const dbv::AnyOrderPlan plan = dbv::plan_any_order(B, U);
  if (!stream_fits(plan.max_rows, V)) return DBV_ERR_UNSUPPORTED;
  dbv_status s = check_ws(ws, ws_bytes, plan.bytes);
  if (s != DBV_OK) return s;
  if ((s = device_ready()) != DBV_OK) return s;
  if (B == 0) return DBV_OK;

  dbv::AnyOrderArgs a{};
  a.B = B; a.U = U; a.V = V;
  a.tgt = tgt; a.ts = tgt_seq_stride; a.tr = tgt_row_stride;
  a.dr = draft_rows; a.ds = dr_seq_stride; a.drr = dr_row_stride;
  a.order = order; a.num_active = num_active; a.positions = positions; a.draft_tokens = draft_tokens;
  a.eos = eos_id; a.end_pos = end_pos;
  a.accept_len = accept_len; a.num_accepted = num_accepted; a.acc_pos = acc_pos; a.acc_tok = acc_tok;
  a.new_end = new_end; a.next_draft = next_draft; a.status = status;
  char* w = static_cast<char*>(ws);
  a.part = reinterpret_cast<float2*>(w + plan.off_part);
  a.pre = reinterpret_cast<int32_t*>(w + plan.off_pre);
  int32_t* seq = reinterpret_cast<int32_t*>(w + plan.off_seq);
  a.rows = seq;
  a.nver = seq + B;
  a.kappa = seq + 2 * static_cast<int64_t>(B);
  a.pstat = seq + 3 * static_cast<int64_t>(B);
  a.grid = dbv::stream_grid(plan.max_rows, V, static_cast<int64_t>(eb), group_cap(co));
  return dbv::launch_any_order(a, dtype, static_cast<hipStream_t>(stream), co.ev) ? DBV_OK
                                                                                           : DBV_ERR_LAUNCH;
}

dbv_status verify_gumbel_tree(int B, int S, int L, int V, dbv_dtype dtype, const void* logits, int64_t seq_stride,
                              int64_t state_stride, int64_t pos_stride, const uint8_t* masked,
                              const int32_t* parent, const int32_t* edge_pos, const int32_t* edge_tok,
                              const int32_t* num_states, const int32_t* next_pos, const float* gumbel,
                              int64_t g_seq_stride, int64_t g_pos_stride, float temperature, dbv_tree_mode mode,
                              int32_t* sel_pos, int32_t* sel_tok, float* sel_conf, int32_t* path_len,
                              int32_t* path_nodes, int32_t* commit_pos, int32_t* commit_tok,
                              int32_t* num_commits, int32_t* status, void* ws, size_t ws_bytes, void* stream, const dbv_options* opts) {
  if (B < 0 || S < 1 || S > kMaxStates || L < 1 || L > kMaxBlockLen || V < 1 || !dtype_ok(dtype))
    return DBV_ERR_INVALID_ARG;
  if (mode != DBV_TREE_STATE_EQUALITY && mode != DBV_TREE_FIXED_POSITION) return DBV_ERR_INVALID_ARG;
  CallOpts co;
  if (!read_opts(opts, co) || co.accept_margin || co.draw_margin || co.row_tv) return DBV_ERR_INVALID_ARG;
  if (!(std::isfinite(temperature) && temperature >= 0.f)) return DBV_ERR_INVALID_ARG;
  if (seq_stride < 0 || state_stride < 0 || pos_stride < 0 || g_seq_stride < 0 || g_pos_stride < 0)
    return DBV_ERR_INVALID_ARG;
  if (logits == nullptr || parent == nullptr || edge_pos == nullptr || edge_tok == nullptr)
    return DBV_ERR_INVALID_ARG;
  if (mode == DBV_TREE_STATE_EQUALITY && masked == nullptr) return DBV_ERR_INVALID_ARG;
  if (mode == DBV_TREE_FIXED_POSITION && next_pos == nullptr) return DBV_ERR_INVALID_ARG;
  if (temperature > 0.f && gumbel == nullptr) return DBV_ERR_INVALID_ARG;
  if (path_len == nullptr || path_nodes == nullptr || commit_pos == nullptr || commit_tok == nullptr ||
      num_commits == nullptr)
    return DBV_ERR_INVALID_ARG;
  if (!aligned(logits, elem_bytes(dtype)) || (gumbel && !aligned(gumbel, 4))) return DBV_ERR_INVALID_ARG;
  const dbv::TreePlan plan = dbv::plan_tree(B, S, L, V);
  if (!stream_fits(plan.max_rows, V)) return DBV_ERR_UNSUPPORTED;
  dbv_status s = check_ws(ws, ws_bytes, plan.bytes);
  if (s != DBV_OK) return s;
  if ((s = device_ready()) != DBV_OK) return s;
  if (B == 0) return DBV_OK;

  dbv::TreeArgs a{};
  a.B = B; a.S = S; a.L = L; a.V = V;
  a.divL = dbv::FastDiv32(static_cast<uint32_t>(L));
  a.divS = dbv::FastDiv32(static_cast<uint32_t>(S));
  a.logits = logits; a.ss = seq_stride; a.sy = state_stride; a.sp = pos_stride;
  a.masked = masked; a.parent = parent; a.edge_pos = edge_pos; a.edge_tok = edge_tok;
  a.num_states = num_states; a.next_pos = mode == DBV_TREE_FIXED_POSITION ? next_pos : nullptr;
  a.gumbel = gumbel; a.gs = g_seq_stride; a.gp = g_pos_stride;
  a.inv_t = temperature > 0.f ? 1.f / temperature : 0.f;
  a.fixed = mode == DBV_TREE_FIXED_POSITION ? 1 : 0;
  a.sel_pos = sel_pos; a.sel_tok = sel_tok; a.sel_conf = sel_conf;
  a.path_len = path_len; a.path_nodes = path_nodes;
  a.commit_pos = commit_pos; a.commit_tok = commit_tok; a.num_commits = num_commits;
  a.status = status;
  char* w = static_cast<char*>(ws);
  a.count = reinterpret_cast<int32_t*>(w + plan.off_count);
  a.list = reinterpret_cast<int32_t*>(w + plan.off_list);
  a.map = reinterpret_cast<int32_t*>(w + plan.off_map);
  a.conf = reinterpret_cast<float2*>(w + plan.off_conf);
  a.pick = reinterpret_cast<float2*>(w + plan.off_pick);
  a.pick2 = reinterpret_cast<float*>(w + plan.off_pick2);
  a.sel = reinterpret_cast<int32_t*>(w + plan.off_sel);
  a.selconf = reinterpret_cast<float*>(w + plan.off_selconf);
  a.selstat = reinterpret_cast<int32_t*>(w + plan.off_selstat);
  a.selgap = reinterpret_cast<float*>(w + plan.off_selgap);
  a.batch = reinterpret_cast<int4*>(w + plan.off_batch);
  a.nbat = reinterpret_cast<int32_t*>(w + plan.off_nbat);
  a.pos_margin = co.pos_margin;
  a.tok_margin = co.tok_margin;
  a.grid = dbv::stream_grid(plan.max_rows, V, static_cast<int64_t>(elem_bytes(dtype)), group_cap(co));
  a.split2 = plan.split2; a.chunk2 = plan.chunk2;
  return dbv::launch_tree(a, dtype, static_cast<hipStream_t>(stream), co.ev) ? DBV_OK : DBV_ERR_LAUNCH;
}

dbv_status ddtree_hypotheses(int B, int L, int V, dbv_dtype dtype, const void* stale, int64_t seq_stride,
                             int64_t pos_stride, const uint8_t* masked, const float* gumbel, int64_t g_seq_stride,
                             int64_t g_pos_stride, float temperature, float runner_up_below, int32_t* hyp_tok,
                             float* hyp_prob, int32_t* status, void* ws, size_t ws_bytes, void* stream, const dbv_options* opts) {
  if (B < 0 || L < 1 || L > dbv::kDDMaxBlock || V < 1 || !dtype_ok(dtype)) return DBV_ERR_INVALID_ARG;
  CallOpts co;
  if (!read_plain_opts(opts, co)) return DBV_ERR_INVALID_ARG;
  if (seq_stride < 0 || pos_stride < 0 || g_seq_stride < 0 || g_pos_stride < 0) return DBV_ERR_INVALID_ARG;
  if (!(std::isfinite(temperature) && temperature >= 0.f) || std::isnan(runner_up_below))
    return DBV_ERR_INVALID_ARG;
  if (B > 0 && (stale == nullptr || masked == nullptr || hyp_tok == nullptr || hyp_prob == nullptr))
    return DBV_ERR_INVALID_ARG;
  if (temperature > 0.f && B > 0 && gumbel == nullptr) return DBV_ERR_INVALID_ARG;
  if ((stale && !aligned(stale, elem_bytes(dtype))) || (gumbel && !aligned(gumbel, 4))) return DBV_ERR_INVALID_ARG;
  const dbv::DDHypPlan plan = dbv::plan_dd_hypotheses(B, L);
  if (!stream_fits(plan.max_rows, V)) return DBV_ERR_UNSUPPORTED;
  dbv_status s = check_ws(ws, ws_bytes, plan.bytes);
  if (s != DBV_OK) return s;
  if ((s = device_ready()) != DBV_OK) return s;
  if (B == 0) return DBV_OK;
  dbv::DDHypArgs a{};
  a.B = B; a.L = L; a.V = V;
  a.stale = stale; a.ss = seq_stride; a.sp = pos_stride;
  a.masked = masked;
  a.gumbel = temperature > 0.f ? gumbel : nullptr; a.gs = g_seq_stride; a.gp = g_pos_stride;
  a.inv_t = temperature > 0.f ? 1.f / temperature : 0.f;
  a.below = runner_up_below;
  a.hyp_tok = hyp_tok; a.hyp_prob = hyp_prob; a.status = status;
  char* w = static_cast<char*>(ws);
  a.count = reinterpret_cast<int32_t*>(w + plan.off_count);
  a.list = reinterpret_cast<int32_t*>(w + plan.off_list);
  a.map = reinterpret_cast<int32_t*>(w + plan.off_map);
  a.part = reinterpret_cast<dbv::DDPart*>(w + plan.off_part);
  // Gumbel rows double the bytes per element; units of 512 elements then.
  a.split_bytes = temperature > 0.f ? 8 : static_cast<int>(elem_bytes(dtype));
  a.grid = dbv::stream_grid(plan.max_rows, V, a.split_bytes, group_cap(co));
  return dbv::launch_dd_hypotheses(a, dtype, static_cast<hipStream_t>(stream), co.ev) ? DBV_OK
                                                                                             : DBV_ERR_LAUNCH;
}

dbv_status ddtree_level(int B, int L, int D, const uint8_t* masked, const int32_t* hyp_tok, const float* hyp_prob,
                        const float* order_logits, int64_t o_seq_stride, int64_t o_row_stride, float tau,
                        float gamma, int first, int32_t* parent, int32_t* edge_pos, int32_t* edge_tok,
                        float* mass, uint8_t* node_masked, int32_t* num_nodes, int32_t* frontier,
                        int32_t* num_frontier, int32_t* status, void* ws, size_t ws_bytes, void* stream, const dbv_options* opts) {
  return dd_tree_common(B, L, D, masked, hyp_tok, hyp_prob, order_logits, o_seq_stride, o_row_stride, 0, tau,
                        gamma, first, parent, edge_pos, edge_tok, mass, node_masked, num_nodes, frontier,
                        num_frontier, status, ws, ws_bytes, stream, opts);
}

dbv_status ddtree_build(int B, int L, int D, const uint8_t* masked, const int32_t* hyp_tok, const float* hyp_prob,
                        const float* order_table, int64_t t_seq_stride, int64_t t_row_stride, float tau,
                        float gamma, int32_t* parent, int32_t* edge_pos, int32_t* edge_tok, float* mass,
                        uint8_t* node_masked, int32_t* num_nodes, int32_t* frontier, int32_t* num_frontier,
                        int32_t* status, void* ws, size_t ws_bytes, void* stream, const dbv_options* opts) {
  return dd_tree_common(B, L, D, masked, hyp_tok, hyp_prob, order_table, t_seq_stride, t_row_stride, 1, tau,
                        gamma, 1, parent, edge_pos, edge_tok, mass, node_masked, num_nodes, frontier,
                        num_frontier, status, ws, ws_bytes, stream, opts);
}

size_t verify_workspace_size(dbv_kind kind, int B, int K_or_S, int L, int V, dbv_dtype dtype) {
  if (kind == DBV_KIND_DDTREE) {  // the search state depends on B and D only
    if (B < 0 || K_or_S < 0 || K_or_S > dbv::kDDMaxBudget) return 0;
    return dbv::dd_tree_bytes(B, K_or_S);
  }
  if (B < 0 || V < 1 || !dtype_ok(dtype)) return 0;
  switch (kind) {
    case DBV_KIND_GREEDY:
      if (K_or_S < 0 || K_or_S > kMaxDraft || L < 0 || L > kMaxDraft) return 0;
      return dbv::plan_greedy(B, K_or_S, L, V).bytes;
    case DBV_KIND_REJECTION:
      if (K_or_S < 0 || K_or_S > kMaxDraft) return 0;
      return dbv::plan_sample(B, K_or_S, V, static_cast<int64_t>(elem_bytes(dtype))).bytes;
    case DBV_KIND_TREE:
      if (K_or_S < 1 || K_or_S > kMaxStates || L < 1 || L > kMaxBlockLen) return 0;
      return dbv::plan_tree(B, K_or_S, L, V).bytes;
    case DBV_KIND_ANY_ORDER:
      if (K_or_S < 0 || K_or_S > kMaxDraft) return 0;
      return dbv::plan_any_order(B, K_or_S).bytes;
    case DBV_KIND_DDTREE_HYPOTHESES:
      if (K_or_S < 1 || K_or_S > dbv::kDDMaxBlock) return 0;
      return dbv::plan_dd_hypotheses(B, K_or_S).bytes;
    case DBV_KIND_DDTREE:
      return 0;
  }
  return 0;
}

const char* verify_status_string(dbv_status s) {
  switch (s) {
    case DBV_OK: return "ok";
    case DBV_ERR_INVALID_ARG: return "invalid argument";
    case DBV_ERR_UNSUPPORTED: return "unsupported (device or request)";
    case DBV_ERR_NO_DEVICE: return "no usable GPU device";
    case DBV_ERR_LAUNCH: return "kernel launch failed";
    case DBV_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
  }
  return "unknown status";
}

int verify_abi_version(void) { return DBV_ABI_VERSION; }


}  // extern "C"
