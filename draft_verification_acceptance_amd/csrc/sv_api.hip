// C ABI entry points of libspecverify: host-side argument checks, workspace carve-up, kernel launches.
// Nothing here allocates, synchronises or reads device memory.
#include <math.h>

#include <mutex>

#include "sv_internal.h"

using namespace sv;

// The workspace of spec_verify_chain_noalloc: one copy per GPU, held until the process ends. Host code never
// passes this name to a kernel (on the host it is only a stand-in for the symbol); it looks up the array's
// device address once per GPU and uses that address.
static __device__ __align__(256) char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr double kLog2e = 1.4426950408889634;

// The logits stream launches B x L x P x S workgroups and the draw B x S2: both within one grid dimension.
bool grid_fits(const Layout& lo, int32_t batch) {
  const int64_t stream_wgs = int64_t(batch) * lo.L * lo.P * lo.S;
  const int64_t draw_wgs = int64_t(batch) * (lo.S2 + 1);   // + the scan-only workgroup of a fused commit
  return stream_wgs <= INT32_MAX && draw_wgs <= INT32_MAX;
}

// Profiling events: none, or a start / stop pair per kernel, taken from the kernel's own timestamps.
bool bad_events(hipEvent_t* ev, int32_t n, int32_t kernels) {
  if (n == 0) return false;
  return ev == nullptr || n != 2 * kernels;
}

hipEvent_t ev_at(hipEvent_t* ev, int32_t n, int32_t i) { return n ? ev[i] : nullptr; }

// Nothing to launch: every event is still recorded on the stream, so that it completes.
spec_status record_all(hipEvent_t* ev, int32_t n, hipStream_t stream) {
  for (int32_t i = 0; i < n; ++i)
    if (hipEventRecord(ev[i], stream) != hipSuccess) return SPEC_ELAUNCH;
  return SPEC_OK;
}

template <typename A>
void fill_outputs(VerifyParams& p, const A* a) {
  p.accept_len = a->accept_len;
  p.bonus = a->bonus;
  p.out_tokens = a->out_tokens;
  p.accept_index = a->accept_index;
  p.status = a->status;
  p.accept_prob = a->accept_prob;
  p.residual_mass = a->residual_mass;
}

void carve(VerifyParams& p, const Layout& lo, void* ws) {
  char* w = static_cast<char*>(ws);
  p.cnt2 = reinterpret_cast<unsigned long long*>(w + lo.off_cnt2);
  p.part = reinterpret_cast<Part*>(w + lo.off_part);
  p.seg = reinterpret_cast<float2*>(w + lo.off_seg);
  p.mrow = reinterpret_cast<uint4*>(w + lo.off_mrow);
  p.chunk = lo.chunk;
  p.L = lo.L;
  p.P = lo.P;
  p.S = lo.S;
  p.S2 = lo.S2;
  p.bseg = lo.bseg;
  p.n_seg = lo.n_seg;
}

// The fused commit's arguments (NULL: none), checked as spec_commit_indices checks its own; its counter and
// published accept results live in the workspace. Call after carve() and once p.B is set.
spec_status fill_commit(VerifyParams& p, const spec_commit_args* c, int64_t total_rows, const Layout& lo, void* ws) {
  p.cm_on = 0;
  if (!c) return SPEC_OK;
  if (!c->verify_slots || !c->seq_lens || !c->commit_offsets || !c->src_slots || !c->dst_pos || !c->new_seq_lens ||
      !c->status)
    return SPEC_EINVAL;
  if ((c->evict_slots == nullptr) != (c->evict_offsets == nullptr)) return SPEC_EINVAL;
  if (c->capacity < total_rows) return SPEC_EINVAL;
  char* w = static_cast<char*>(ws) + lo.off_cm;
  p.cm_on = 1;
  p.ccnt = reinterpret_cast<unsigned long long*>(w);
  p.pub_r = reinterpret_cast<int32_t*>(w + kCounterStride);
  p.pub_path = p.tree ? p.pub_r + p.B : nullptr;
  p.verify_slots = c->verify_slots;
  p.seq_lens = c->seq_lens;
  p.commit_offsets = c->commit_offsets;
  p.src_slots = c->src_slots;
  p.dst_pos = c->dst_pos;
  p.new_seq_lens = c->new_seq_lens;
  p.cstatus = c->status;
  p.evict_slots = c->evict_slots;
  p.evict_offsets = c->evict_offsets;
  return SPEC_OK;
}

// The two kernels of a verify call: the logits stream, then the greedy scans, the sample-then-match
// draws or the sampling draw.
spec_status launch_pair(int dtype, int mode, VerifyParams& p, hipEvent_t* ev, int32_t nev, hipStream_t stream) {
  if (launch_stats(dtype, mode, p, stream, ev_at(ev, nev, 0), ev_at(ev, nev, 1)) != hipSuccess)
    return SPEC_ELAUNCH;
  hipEvent_t e0 = ev_at(ev, nev, 2), e1 = ev_at(ev, nev, 3);
  const hipError_t e = mode == SPEC_MODE_GREEDY         ? launch_scan(dtype, p, stream, e0, e1)
                       : mode == SPEC_MODE_SAMPLE_MATCH ? launch_match(dtype, p, stream, e0, e1)
                                                        : launch_draw(dtype, mode, p, stream, e0, e1);
  return e == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each GPU, once looked up

// Device address of `scratch` on the GPU that runs `stream`, looked up (with that GPU current) on the
// first call for that GPU.
spec_status scratch_for(hipStream_t stream, void** out) {
  int dev = -1, cur = -1;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || hipGetDevice(&cur) != hipSuccess) return SPEC_ELAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return SPEC_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return SPEC_ELAUNCH;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return SPEC_ELAUNCH;
    if (e != hipSuccess || p == nullptr) return SPEC_ELAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SPEC_OK;
}

// spec_verify_chain with the workspace given explicitly; `noalloc`: it is the static scratch (a call too large
// for it is SPEC_ESCRATCH, looked up only once the arguments have passed their checks).
spec_status verify_chain_impl(const spec_chain_args* a, void* ws, size_t ws_bytes, bool noalloc,
                              hipStream_t stream);

}  // namespace

extern "C" {

int32_t spec_abi_version(void) { return SPEC_ABI_VERSION; }

size_t spec_args_size(int32_t kind) {
  switch (kind) {
    case SPEC_KIND_CHAIN: return sizeof(spec_chain_args);
    case SPEC_KIND_TREE: return sizeof(spec_tree_args);
    case SPEC_KIND_COMMIT: return sizeof(spec_commit_args);
    case SPEC_KIND_PLAN: return sizeof(spec_plan_args);
    case SPEC_KIND_CAP_TRIM: return sizeof(spec_cap_trim_args);
    case SPEC_KIND_KV_MOVE: return sizeof(spec_kv_move_args);
    case SPEC_KIND_TREE_BUILD: return sizeof(spec_tree_build_args);
    default: return 0;
  }
}

const char* spec_status_string(int32_t code) {
  switch (code) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_EINVAL: return "SPEC_EINVAL: invalid argument (null pointer or size out of range)";
    case SPEC_EDTYPE: return "SPEC_EDTYPE: unsupported logits dtype";
    case SPEC_EUNSUPPORTED: return "SPEC_EUNSUPPORTED: mode / kind / threshold combination not implemented";
    case SPEC_EWORKSPACE: return "SPEC_EWORKSPACE: workspace missing or too small";
    case SPEC_ELAUNCH: return "SPEC_ELAUNCH: kernel launch or event record failed";
    case SPEC_ESCRATCH:
      return "SPEC_ESCRATCH: the call needs a larger workspace than the static scratch of "
             "spec_verify_chain_noalloc (SPEC_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown spec_status";
  }
}

int32_t spec_kernel_count(int32_t kind, int32_t mode) {
  (void)mode;
  if (kind == SPEC_KIND_COMMIT || kind == SPEC_KIND_PLAN || kind == SPEC_KIND_CAP_TRIM || kind == SPEC_KIND_KV_MOVE ||
      kind == SPEC_KIND_TREE_BUILD)
    return 1;
  if (kind != SPEC_KIND_CHAIN && kind != SPEC_KIND_TREE) return 0;
  return 2;
}

size_t spec_workspace_bytes(int32_t kind, int32_t mode, int64_t total_rows, int64_t vocab, int32_t batch,
                            int32_t max_verify_len) {
  if (kind == SPEC_KIND_COMMIT) return 0;
  if (batch < 0 || vocab < 1 || vocab > kMaxVocab || total_rows < batch) return 0;
  if (mode != SPEC_MODE_GREEDY && mode != SPEC_MODE_REJECTION && mode != SPEC_MODE_TARGET_ONLY &&
      mode != SPEC_MODE_REJECTION_SPARSE && mode != SPEC_MODE_SAMPLE_MATCH)
    return 0;
  int32_t L;
  if (kind == SPEC_KIND_CHAIN) {
    L = max_verify_len;
  } else if (kind == SPEC_KIND_TREE) {
    if (batch == 0) return 256;
    if (total_rows % batch) return 0;
    L = int32_t(total_rows / batch);
  } else {
    return 0;
  }
  if (L < 1 || L > kMaxLen) return 0;
  return make_layout(kind, mode, total_rows, vocab, batch, L).bytes;
}

spec_status spec_workspace_init(void* workspace, size_t bytes, hipStream_t stream) {
  if (!workspace && bytes) return SPEC_EINVAL;
  return launch_fill_zero(workspace, bytes, stream) == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

spec_status spec_read_probe(const void* src, size_t bytes, uint32_t* sink, hipEvent_t* events, hipStream_t stream) {
  if (bytes == 0) return SPEC_OK;
  if (!src || !sink || (reinterpret_cast<uintptr_t>(src) & 15) || (bytes & 15)) return SPEC_EINVAL;
  const hipError_t e = launch_read_fold(src, bytes, sink, stream, events ? events[0] : nullptr,
                                        events ? events[1] : nullptr);
  return e == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

spec_status spec_verify_chain(const spec_chain_args* a, hipStream_t stream) {
  if (!a) return SPEC_EINVAL;
  return verify_chain_impl(a, a->workspace, a->workspace_bytes, false, stream);
}

spec_status spec_verify_chain_noalloc(const spec_chain_args* a, hipStream_t stream) {
  if (!a) return SPEC_EINVAL;
  return verify_chain_impl(a, nullptr, SPEC_NOALLOC_SCRATCH_BYTES, true, stream);
}

}  // extern "C"

namespace {

spec_status verify_chain_impl(const spec_chain_args* a, void* ws, size_t ws_bytes, bool noalloc,
                              hipStream_t stream) {
  if (a->dtype != SPEC_DTYPE_F32 && a->dtype != SPEC_DTYPE_BF16) return SPEC_EDTYPE;
  if (a->mode == SPEC_MODE_TARGET_ONLY) return SPEC_EUNSUPPORTED;
  if (a->mode != SPEC_MODE_GREEDY && a->mode != SPEC_MODE_REJECTION && a->mode != SPEC_MODE_REJECTION_SPARSE &&
      a->mode != SPEC_MODE_SAMPLE_MATCH)
    return SPEC_EINVAL;
  if (a->batch < 0 || a->vocab < 1 || a->vocab > kMaxVocab || a->total_rows < a->batch ||
      a->total_rows > INT32_MAX || a->max_verify_len < 1 || a->max_verify_len > kMaxLen)
    return SPEC_EINVAL;
  const bool dense = a->mode == SPEC_MODE_REJECTION;
  const bool sparse = a->mode == SPEC_MODE_REJECTION_SPARSE;
  const bool sampling = a->mode != SPEC_MODE_GREEDY;
  if (sparse && (a->n_cand < 1 || a->n_cand > kMaxCand)) return SPEC_EINVAL;
  if (bad_events(a->profile_events, a->n_profile_events, spec_kernel_count(SPEC_KIND_CHAIN, a->mode)))
    return SPEC_EINVAL;
  if (a->batch == 0) return record_all(a->profile_events, a->n_profile_events, stream);
  const int64_t D = a->total_rows - a->batch;
  if (!a->target_logits || !a->target_offsets || !a->accept_len || !a->bonus || !a->out_tokens ||
      !a->accept_index || !a->status)
    return SPEC_EINVAL;
  if (D > 0 && !a->draft_tokens) return SPEC_EINVAL;
  if (sampling) {
    if (!a->u_final || (D > 0 && !a->u_accept)) return SPEC_EINVAL;
    if (!(a->temperature > 0.f) || !isfinite(a->temperature)) return SPEC_EINVAL;
  }
  if (dense && D > 0 && !a->draft_logits) return SPEC_EINVAL;
  if (sparse && D > 0 && (!a->cand_ids || !a->cand_q)) return SPEC_EINVAL;
  const Layout lo = make_layout(SPEC_KIND_CHAIN, a->mode, a->total_rows, a->vocab, a->batch, a->max_verify_len);
  if (!grid_fits(lo, a->batch)) return SPEC_EINVAL;
  if (noalloc) {
    if (lo.bytes > ws_bytes) return SPEC_ESCRATCH;
    const spec_status st = scratch_for(stream, &ws);
    if (st != SPEC_OK) return st;
  }
  if (!ws || ws_bytes < lo.bytes) return SPEC_EWORKSPACE;

  VerifyParams p{};
  p.target = a->target_logits;
  p.draft = dense ? a->draft_logits : nullptr;
  p.cand_ids = sparse ? a->cand_ids : nullptr;
  p.cand_q = sparse ? a->cand_q : nullptr;
  p.K = sparse ? a->n_cand : 0;
  p.offsets = a->target_offsets;
  p.draft_tokens = a->draft_tokens;
  p.u_accept = a->u_accept;
  p.u_final = a->u_final;
  fill_outputs(p, a);
  carve(p, lo, ws);
  p.V = a->vocab;
  p.total_rows = a->total_rows;
  p.B = a->batch;
  p.tree = 0;
  p.coef = sampling ? float(kLog2e / double(a->temperature)) : 0.f;
  p.mask = a->vocab_mask;
  p.mask_words = (a->vocab + 31) / 32;
  // Piece partials need 16-byte aligned rows: the layout asks for them when vocab % 8 == 0, the base
  // pointer must be aligned too (else the draw narrows whole chunks).
  const bool aligned = (reinterpret_cast<uintptr_t>(a->target_logits) & 15) == 0;
  p.piece = lo.n_piece > 0 && aligned ? reinterpret_cast<float2*>(static_cast<char*>(ws) + lo.off_piece) : nullptr;
  p.n_piece = lo.n_piece;
  const spec_status cs = fill_commit(p, a->commit, a->total_rows, lo, ws);
  if (cs != SPEC_OK) return cs;
  return launch_pair(a->dtype, a->mode, p, a->profile_events, a->n_profile_events, stream);
}

}  // namespace

extern "C" {

spec_status spec_verify_tree(const spec_tree_args* a, hipStream_t stream) {
  if (!a) return SPEC_EINVAL;
  if (a->dtype != SPEC_DTYPE_F32 && a->dtype != SPEC_DTYPE_BF16) return SPEC_EDTYPE;
  // classic p/q rejection needs topk = 1 (a chain); sample-then-match is a chain rule
  if (a->mode == SPEC_MODE_REJECTION || a->mode == SPEC_MODE_REJECTION_SPARSE || a->mode == SPEC_MODE_SAMPLE_MATCH)
    return SPEC_EUNSUPPORTED;
  if (a->mode != SPEC_MODE_GREEDY && a->mode != SPEC_MODE_TARGET_ONLY) return SPEC_EINVAL;
  const bool tgt = a->mode == SPEC_MODE_TARGET_ONLY;
  if (tgt && (a->threshold_single != 1.f || a->threshold_acc != 1.f)) return SPEC_EUNSUPPORTED;
  if (a->batch < 0 || a->vocab < 1 || a->vocab > kMaxVocab || a->n_nodes < 1 || a->n_nodes > kMaxLen ||
      int64_t(a->batch) * a->n_nodes > INT32_MAX)
    return SPEC_EINVAL;
  if (bad_events(a->profile_events, a->n_profile_events, spec_kernel_count(SPEC_KIND_TREE, a->mode)))
    return SPEC_EINVAL;
  if (a->batch == 0) return record_all(a->profile_events, a->n_profile_events, stream);
  if (!a->target_logits || !a->parents || !a->tokens || !a->accept_len || !a->bonus || !a->out_tokens ||
      !a->accept_index || !a->status)
    return SPEC_EINVAL;
  if (tgt) {
    if (!a->u_accept || !a->u_final) return SPEC_EINVAL;
    if (!(a->temperature > 0.f) || !isfinite(a->temperature)) return SPEC_EINVAL;
  }
  const int64_t rows = int64_t(a->batch) * a->n_nodes;
  const Layout lo = make_layout(SPEC_KIND_TREE, a->mode, rows, a->vocab, a->batch, a->n_nodes);
  if (!grid_fits(lo, a->batch)) return SPEC_EINVAL;
  if (!a->workspace || a->workspace_bytes < lo.bytes) return SPEC_EWORKSPACE;

  VerifyParams p{};
  p.target = a->target_logits;
  p.draft = nullptr;
  p.parents = a->parents;
  p.tokens = a->tokens;
  p.u_accept = a->u_accept;
  p.u_final = a->u_final;
  fill_outputs(p, a);
  carve(p, lo, a->workspace);
  p.V = a->vocab;
  p.total_rows = rows;
  p.B = a->batch;
  p.tree = 1;
  p.coef = tgt ? float(kLog2e / double(a->temperature)) : 0.f;
  p.mask = a->vocab_mask;
  p.mask_words = (a->vocab + 31) / 32;
  const spec_status cs = fill_commit(p, a->commit, rows, lo, a->workspace);
  if (cs != SPEC_OK) return cs;
  return launch_pair(a->dtype, a->mode, p, a->profile_events, a->n_profile_events, stream);
}

spec_status spec_commit_indices(const spec_commit_args* a, hipStream_t stream) {
  if (!a) return SPEC_EINVAL;
  if (a->batch < 0 || a->total_rows < a->batch || a->total_rows > INT32_MAX || a->capacity < a->total_rows ||
      a->max_verify_len < 1 || a->max_verify_len > kMaxLen)
    return SPEC_EINVAL;
  if (bad_events(a->profile_events, a->n_profile_events, 1)) return SPEC_EINVAL;
  if (!a->row_offsets || !a->commit_offsets) return SPEC_EINVAL;
  if (a->batch > 0 && (!a->accept_len || !a->accept_index || !a->verify_slots || !a->seq_lens || !a->src_slots ||
                       !a->dst_pos || !a->new_seq_lens || !a->status))
    return SPEC_EINVAL;
  if ((a->evict_slots == nullptr) != (a->evict_offsets == nullptr)) return SPEC_EINVAL;
  const int32_t n = a->n_profile_events;
  if (launch_commit(*a, stream, ev_at(a->profile_events, n, 0), ev_at(a->profile_events, n, 1)) != hipSuccess)
    return SPEC_ELAUNCH;
  return SPEC_OK;
}

spec_status spec_plan_layout(const spec_plan_args* a, hipStream_t stream) {
  if (!a) return SPEC_EINVAL;
  if (a->mode != SPEC_PLAN_TOPK && a->mode != SPEC_PLAN_THRESHOLD) return SPEC_EINVAL;
  if (a->batch < 0 || a->batch >= (1 << 20) || a->width < 0 || a->width > 4095) return SPEC_EINVAL;
  if (int64_t(a->batch) * (int64_t(a->width) + 1) > INT32_MAX) return SPEC_EINVAL;
  if (a->min_verify_len < 1 || a->max_verify_len < a->min_verify_len || a->max_verify_len > a->width + 1)
    return SPEC_EINVAL;   // at most the anchor and every draft: row_index holds batch*(width+1) rows
  if (!(a->survival_eps >= 0.f) || a->threshold != a->threshold) return SPEC_EINVAL;
  if (bad_events(a->profile_events, a->n_profile_events, 1)) return SPEC_EINVAL;
  if (!a->offsets) return SPEC_EINVAL;
  if (a->batch > 0 && (!a->selected || !a->verify_lens || (a->width > 0 && !a->confidence))) return SPEC_EINVAL;
  const int32_t n = a->n_profile_events;
  if (launch_plan(*a, stream, ev_at(a->profile_events, n, 0), ev_at(a->profile_events, n, 1)) != hipSuccess)
    return SPEC_ELAUNCH;
  return SPEC_OK;
}

spec_status spec_plan_budget(const float* conf, int32_t batch, int32_t width, const double* sps_rows,
                             const double* sps, int32_t n_sps, float survival_eps, int32_t* budget, double* theta,
                             int32_t* n_entries) {
  if (batch < 0 || width < 0 || n_sps < 1 || !sps_rows || !sps || !budget) return SPEC_EINVAL;
  if (int64_t(batch) * width > INT32_MAX - 1) return SPEC_EINVAL;
  if (int64_t(batch) * width > 0 && !conf) return SPEC_EINVAL;
  if (!(survival_eps >= 0.f)) return SPEC_EINVAL;
  for (int32_t i = 0; i < n_sps; ++i) {
    if (!isfinite(sps_rows[i]) || !isfinite(sps[i])) return SPEC_EINVAL;
    if (i > 0 && !(sps_rows[i] > sps_rows[i - 1])) return SPEC_EINVAL;
  }
  return plan_budget_host(conf, batch, width, sps_rows, sps, n_sps, survival_eps, budget, theta, n_entries);
}

spec_status spec_plan_budget_cost(const float* conf, int32_t batch, int32_t width, const double* req_rows,
                                  const double* req_cost, int32_t n_req, const double* tok_rows,
                                  const double* tok_cost, int32_t n_tok, float survival_eps, int32_t* budget,
                                  double* theta, int32_t* n_entries) {
  if (batch < 0 || width < 0 || n_req < 1 || n_tok < 1 || !req_rows || !req_cost || !tok_rows || !tok_cost ||
      !budget)
    return SPEC_EINVAL;
  if (int64_t(batch) * width > INT32_MAX - 1) return SPEC_EINVAL;
  if (int64_t(batch) * width > 0 && !conf) return SPEC_EINVAL;
  if (!(survival_eps >= 0.f)) return SPEC_EINVAL;
  // rows strictly increasing; per-batch costs >= 0 and per-row costs > 0, so every predicted step time is > 0
  for (int32_t i = 0; i < n_req; ++i) {
    if (!isfinite(req_rows[i]) || !isfinite(req_cost[i]) || !(req_cost[i] >= 0.0)) return SPEC_EINVAL;
    if (i > 0 && !(req_rows[i] > req_rows[i - 1])) return SPEC_EINVAL;
  }
  for (int32_t i = 0; i < n_tok; ++i) {
    if (!isfinite(tok_rows[i]) || !isfinite(tok_cost[i]) || !(tok_cost[i] > 0.0)) return SPEC_EINVAL;
    if (i > 0 && !(tok_rows[i] > tok_rows[i - 1])) return SPEC_EINVAL;
  }
  return plan_budget_cost_host(conf, batch, width, req_rows, req_cost, n_req, tok_rows, tok_cost, n_tok,
                               survival_eps, budget, theta, n_entries);
}

spec_status spec_cap_trim(const spec_cap_trim_args* a, hipStream_t stream) {
  if (!a) return SPEC_EINVAL;
  if (a->batch < 0 || a->total_rows < 0 || a->total_rows > INT32_MAX) return SPEC_EINVAL;
  if (bad_events(a->profile_events, a->n_profile_events, 1)) return SPEC_EINVAL;
  if (a->batch == 0) return record_all(a->profile_events, a->n_profile_events, stream);
  if (!a->row_offsets || !a->verify_lens || !a->raw_accept_len || !a->raw_bonus || !a->out_tokens ||
      !a->correct_len || !a->cap_trim_lens || !a->commit_lens || !a->block_accept_lens || !a->bonus || !a->status)
    return SPEC_EINVAL;
  const int32_t n = a->n_profile_events;
  if (launch_cap_trim(*a, stream, ev_at(a->profile_events, n, 0), ev_at(a->profile_events, n, 1)) != hipSuccess)
    return SPEC_ELAUNCH;
  return SPEC_OK;
}

spec_status spec_kv_move(const spec_kv_move_args* a, hipStream_t stream) {
  if (!a) return SPEC_EINVAL;
  if (a->batch < 0 || a->n_buffers < 1 || a->n_buffers > 65535 || a->row_bytes < 16 || a->row_bytes % 16 ||
      a->row_bytes > (1 << 20) || a->n_slots < 0 || a->max_context < 0 || a->n_req_rows < 0 || a->capacity < 0)
    return SPEC_EINVAL;
  if (int64_t(a->batch) * a->n_buffers * ((a->row_bytes / 16 + 255) / 256) > INT32_MAX) return SPEC_EINVAL;
  if (bad_events(a->profile_events, a->n_profile_events, 1)) return SPEC_EINVAL;
  if (a->batch == 0) return record_all(a->profile_events, a->n_profile_events, stream);
  if (!a->buffers || !a->commit_offsets || !a->req_pool_indices || (a->n_req_rows > 0 && !a->req_to_token) ||
      (a->capacity > 0 && (!a->src_slots || !a->dst_pos)))
    return SPEC_EINVAL;
  const int32_t n = a->n_profile_events;
  if (launch_kv_move(*a, stream, ev_at(a->profile_events, n, 0), ev_at(a->profile_events, n, 1)) != hipSuccess)
    return SPEC_ELAUNCH;
  return SPEC_OK;
}

spec_status spec_tree_build(const spec_tree_build_args* a, hipStream_t stream) {
  if (!a) return SPEC_EINVAL;
  if (a->batch < 0 || a->n_steps < 1 || a->topk < 1 || a->topk > 64) return SPEC_EINVAL;
  const int64_t n_cand = int64_t(a->topk) + int64_t(a->n_steps - 1) * a->topk * a->topk;
  if (n_cand > 4096 || a->n_nodes < 1 || a->n_nodes > 1024 || a->n_nodes > n_cand + 1) return SPEC_EINVAL;
  if (bad_events(a->profile_events, a->n_profile_events, 1)) return SPEC_EINVAL;
  if (a->batch == 0) return record_all(a->profile_events, a->n_profile_events, stream);
  if (!a->anchors || !a->draft_tokens || !a->draft_probs || !a->seq_lens || !a->tokens || !a->parents ||
      !a->positions || !a->status)
    return SPEC_EINVAL;
  const int32_t n = a->n_profile_events;
  if (launch_tree_build(*a, stream, ev_at(a->profile_events, n, 0), ev_at(a->profile_events, n, 1)) != hipSuccess)
    return SPEC_ELAUNCH;
  return SPEC_OK;
}

}  // extern "C"

