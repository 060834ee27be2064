// Internal definitions shared by the HIP translation units of libspecverify (not part of the ABI).
//
// Workspace state across calls: every call gets a fresh nonzero 32-bit epoch from the host. Per-request
// completion counters are 64-bit words (epoch << 32 | count): k_stats restarts a counter that carries an
// older epoch by compare-and-swap, and each request's scan arms its k_draw counter with the epoch and a
// zero count. A draw descriptor is pending only while its state equals the epoch, so whatever a previous
// call (of any shape) left in the workspace is never mistaken for this call's progress.
//
// Data flow of one verify call (all on the caller's stream, no host synchronisation):
//   k_stats   one workgroup per (request, row slot, target|draft, vocab chunk): streams its slice of a
//             logits row once from HBM and writes a 16-byte partial (greedy: max + lowest argmax;
//             sampling: online max + sum of exp2). The workgroup that completes a request's last slice
//             (device-scope counter) merges the partials and runs the request's accept scan / tree walk,
//             writes every output it can, and for sampling modes leaves a draw descriptor.
//   k_draw    sampling modes only: one workgroup per (request, vocab chunk) re-reads the single row (or
//             target/draft row pair) the final token is drawn from, with the per-token adjustments of a
//             short list (tried tree tokens, sparse q candidates), and writes per-512-token segment sums;
//             the last workgroup of the request locates the inverse-CDF step (fp64 prefix over segments,
//             then inside one segment) and writes the token.
//   k_commit  one workgroup: exclusive scan of accept_len + 1 and the slot gathers of the KV commit.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

constexpr int kThreads = 256;        // threads per workgroup of k_stats / k_draw (4 wave64)
constexpr int kWave = 64;            // gfx950 wavefront size
constexpr int kSeg = 512;            // tokens per draw segment (one wave: 8 tokens per lane)
constexpr int kMaxLen = 1024;        // max verify rows per request (chain) / nodes per tree
constexpr int kMaxCand = 1024;       // max candidates per draft row (sparse q)
constexpr int64_t kMaxVocab = int64_t(1) << 22;
// Per-request completion counters sit 256 bytes apart: a request's workgroups all update its counter at
// the end of the kernel, and counters sharing a cache line would serialise every request's updates on
// one memory channel while the logits stream saturates HBM.
constexpr size_t kCounterStride = 256;
constexpr size_t kCounterWords = kCounterStride / sizeof(unsigned long long);
constexpr float kNear = 1e-5f;       // |u - alpha| / CDF-gap band reported as NEAR_*
constexpr float kNearMass = 1e-6f;   // CDF-gap band in probability mass (gap * total weight)

// Partial statistics of one vocab chunk of one row (16 bytes).
//   greedy:   a = max logit, idx = lowest index attaining it (INT32_MAX if none), flags bit0 = NaN seen
//   sampling: a = m = max of x*coef (log2 units), b = z = sum exp2(x*coef - m)
struct alignas(16) Part {
  float a;
  float b;
  int32_t idx;
  uint32_t flags;
};

// What the final draw of a request needs; written by the request's scan, consumed by k_draw.
struct alignas(16) DrawDesc {
  uint32_t state;    // == the call's epoch: a draw is pending for this call
  int32_t row_t;     // global target row the token is drawn from
  int32_t row_q;     // draft row of the residual [p - q]_+ (logits, or sparse candidates), or -1 (from p)
  int32_t out_pos;   // out_tokens index of the drawn token
  float m_t, l_t;    // target row: max m (log2 units) and normaliser z of softmax = exp2(x*coef - m) / z
  float m_q, l_q;    // draft row, same meaning (dense rejection)
  float coef;        // log2(e) / temperature
  float u;           // sanitized u_final
  uint32_t status;   // request status bits so far
  int32_t n_seen;    // tree TARGET_ONLY: number of tokens excluded from the draw (in the seen buffer)
};

struct Layout {
  int32_t L = 0;         // row slots per request (chain: max_verify_len, tree: n_nodes)
  int32_t P = 1;         // 2 when draft rows are streamed too (rejection)
  int32_t S = 1;         // vocab chunks per row in k_stats
  int64_t chunk = 0;     // tokens per chunk in k_stats
  int32_t S2 = 1;        // vocab chunks per request in k_draw
  int32_t spc = 1;       // segments per k_draw chunk
  int32_t n_seg = 0;     // segments per row
  size_t off_cnt = 0, off_cnt2 = 0, off_part = 0, off_desc = 0, off_seg = 0, off_seen = 0;
  size_t bytes = 0;
};

// Workspace carve-up and launch shapes; the same function serves spec_workspace_bytes and the calls.
inline Layout make_layout(int kind, int mode, int64_t total_rows, int64_t vocab, int32_t batch, int32_t L) {
  Layout lo;
  const bool sampling = mode != SPEC_MODE_GREEDY;
  lo.L = L;
  lo.P = (kind == SPEC_KIND_CHAIN && mode == SPEC_MODE_REJECTION) ? 2 : 1;
  const int64_t slots = int64_t(batch) * L * lo.P;
  // One workgroup per row once there are >= 512 rows (measured best on MI355X: fewer partials and
  // counter updates per request, long streams per workgroup); smaller batches split rows into chunks of
  // at least 8192 tokens to keep ~512 workgroups streaming.
  int64_t s = slots > 0 ? (512 + slots - 1) / slots : 1;
  int64_t max_s = vocab / 8192;
  if (max_s < 1) max_s = 1;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  int64_t chunk = (vocab + s - 1) / s;
  chunk = (chunk + 63) / 64 * 64;
  lo.chunk = chunk;
  lo.S = int32_t((vocab + chunk - 1) / chunk);
  lo.n_seg = int32_t((vocab + kSeg - 1) / kSeg);
  // k_draw: ~2048 workgroups, each covering at least 16 segments (4 per wave).
  int64_t s2 = batch > 0 ? (2048 + batch - 1) / batch : 1;
  const int64_t max_s2 = (lo.n_seg + 15) / 16;
  if (s2 > max_s2) s2 = max_s2;
  if (s2 < 1) s2 = 1;
  lo.spc = int32_t((lo.n_seg + s2 - 1) / s2);
  lo.S2 = (lo.n_seg + lo.spc - 1) / lo.spc;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t o = 0;
  lo.off_cnt = o;  o = up(o + kCounterStride * size_t(batch));
  lo.off_cnt2 = o; o = up(o + kCounterStride * size_t(batch));
  lo.off_part = o; o = up(o + sizeof(Part) * size_t(slots) * size_t(lo.S));
  lo.off_desc = o; o = up(o + sizeof(DrawDesc) * size_t(batch));
  lo.off_seg = o;  o = up(o + (sampling ? sizeof(float2) * size_t(batch) * size_t(lo.n_seg) : 0));
  lo.off_seen = o; o = up(o + ((kind == SPEC_KIND_TREE && sampling) ? sizeof(int32_t) * size_t(batch) * L : 0));
  lo.bytes = o;
  (void)total_rows;
  return lo;
}

// Kernel parameter block of k_stats (passed by value).
struct StatsParams {
  const void* target;
  const void* draft;
  const int32_t* offsets;
  const int32_t* draft_tokens;
  const int32_t* parents;
  const int32_t* tokens;
  const int32_t* cand_ids;    // sparse q: [draft rows, K]
  const float* cand_q;
  const float* u_accept;
  const float* u_final;
  int32_t* accept_len;
  int32_t* bonus;
  int32_t* out_tokens;
  int32_t* accept_index;
  uint32_t* status;
  float* accept_prob;
  float* residual_mass;
  unsigned long long* cnt;
  unsigned long long* cnt2;   // draw-pass counters, armed by each request's scan
  Part* part;
  DrawDesc* desc;
  int32_t* seen;
  int64_t V;
  int64_t total_rows;
  int64_t chunk;
  int32_t B, L, P, S;
  int32_t K;                  // sparse q: candidates per draft row (0 otherwise)
  float coef;
  uint32_t epoch;
};

struct DrawParams {
  const void* target;
  const void* draft;
  int32_t* bonus;
  int32_t* out_tokens;
  uint32_t* status;
  float* residual_mass;
  unsigned long long* cnt2;
  DrawDesc* desc;
  float2* seg;
  const int32_t* seen;
  const int32_t* cand_ids;    // sparse q: the candidates of desc.row_q adjust the draw
  const float* cand_q;
  int64_t V;
  int32_t B, S2, spc, n_seg, seen_stride, K;
  uint32_t epoch;
};

struct CommitParams {
  spec_commit_args a;
};

// Host-side launchers (each in the translation unit of its kernel). They return hipSuccess or the
// launch error.
hipError_t launch_stats(int dtype, int mode, bool tree, const StatsParams& p, const Layout& lo,
                        hipStream_t stream);
hipError_t launch_draw(int dtype, const DrawParams& p, const Layout& lo, hipStream_t stream);
hipError_t launch_commit(const spec_commit_args& a, hipStream_t stream);
hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream);

}  // namespace sv
