// Internal definitions shared by the HIP translation units of libspecverify (not part of the ABI).
//
// Workspace state across calls: none is kept. The draw pass's per-request completion counters are reset
// to 0 by the logits stream of the same call (a kernel boundary before the draw counts), and every other
// workspace word a call reads was written earlier in that call, so whatever a previous call (of any shape)
// left in the workspace does not matter, and a captured call replays correctly.
//
// Data flow of one verify call (all on the caller's stream, no host synchronisation):
//   k_stats   one workgroup per (request, row slot, target|draft, vocab chunk): streams its slice of a
//             logits row once from HBM and stores a partial (greedy: max + lowest argmax; sampling: online
//             max + sum of exp2, and the logit at the token the row judges). Nothing else: no counters and
//             no waits, so the stream ends when its last loads land.
//   k_scan    greedy only: one workgroup per request merges the request's partials and runs its accept
//             scan (chain) or tree walk, and writes every output.
//   k_draw    sampling modes: workgroup (request, vocab chunk) first runs the request's scan itself (it is
//             small: one round of loads of partials, tokens and uniforms), which names the single row (or
//             target/draft row pair) the final token is drawn from; chunk 0 writes the scan's outputs.
//             Then it re-reads its slice of that row with the per-token adjustments of a short list (tried
//             tree tokens, sparse q candidates) and stores per-512-token segment sums; the last workgroup
//             of the request locates the inverse-CDF step (fp64 prefix over segments, then inside one
//             segment) and writes the token and the status.
//   k_commit  one workgroup: exclusive scan of accept_len + 1 and the slot gathers of the KV commit.
//   A fused commit (a verify call given commit arguments) runs the same commit inside k_scan / k_draw /
//   k_match: every request's accept scan publishes its result and counts itself; the workgroup that counts
//   last writes the commit lists for the whole batch (no extra launch).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

// Launch shape of the logits stream (k_stats). Tuned on MI355X; each may be overridden at build time.
#ifndef SV_STATS_THREADS
#define SV_STATS_THREADS 256         // threads per k_stats workgroup
#endif
#ifndef SV_STATS_WGS
#define SV_STATS_WGS 512             // streaming workgroups aimed for per call, sampling modes (rows are
#endif                               // split into chunks)
#ifndef SV_MATCH_WGS
#define SV_MATCH_WGS 1024            // the same, sample-then-match (each wave reduces every piece it reads
#endif                               // across the wave: more waves keep enough loads in flight)
#ifndef SV_STATS_WGS_GREEDY
#define SV_STATS_WGS_GREEDY 1024     // the same, greedy (less work per token: more loads in flight needed)
#endif
#ifndef SV_STATS_MIN_CHUNK
#define SV_STATS_MIN_CHUNK 8192      // fewest tokens per chunk
#endif
#ifndef SV_MATCH_CHUNK
#define SV_MATCH_CHUNK 8192          // sample-then-match: tokens per stream chunk at most (the draw narrows
#endif                               // its row from the chunk partials, so their size bounds its reads)
#ifndef SV_STATS_UNROLL
#define SV_STATS_UNROLL 4            // 16-byte loads in flight per thread per loop trip
#endif

#ifndef SV_DRAW_THREADS
#define SV_DRAW_THREADS 256          // threads per workgroup of k_draw and k_scan
#endif
#ifndef SV_DRAW_TRIP
#define SV_DRAW_TRIP 2               // draw segments each wave has in flight per trip
#endif
#ifndef SV_DRAW_WGS
#define SV_DRAW_WGS 1024             // draw workgroups aimed for per call
#endif

constexpr int kThreads = SV_DRAW_THREADS;
constexpr int kStatsThreads = SV_STATS_THREADS;
constexpr int kWave = 64;            // gfx950 wavefront size
// The request scan stages every partial of its request in LDS when there are at most this many (one load
// round); the launch shape keeps row slots x parts x chunks within it.
constexpr int kMaxStagedParts = 1024;
constexpr int kSeg = 512;            // tokens per draw segment (one wave: 8 tokens per lane)
// Sample-then-match on 16-byte aligned rows: the stream stores the (m, z) of every piece of a row, a piece
// being what one wave reads in one trip (SV_STATS_UNROLL runs per lane: 2048 tokens in bf16, 1024 in fp32).
// Chunks are then whole multiples of kPieceChunk tokens (a bf16 piece, two fp32 pieces).
constexpr int kPieceMin = 1024;      // smallest piece (fp32): sizes the workspace
constexpr int64_t kPieceChunk = 2048;
constexpr int kMaxLen = 1024;        // max verify rows per request (chain) / nodes per tree
constexpr int kMatchSplitMaxLen = 16;   // sample-then-match: requests of up to this many rows are drawn by
                                        // several workgroups (four rows each), longer ones by one
constexpr int kMaxCand = 1024;       // max candidates per draft row (sparse q)
constexpr int64_t kMaxVocab = int64_t(1) << 22;
// Per-request completion counters sit 256 bytes apart: a request's workgroups all update its counter at
// the end of the kernel, and counters sharing a cache line would serialise every request's updates on
// one memory channel while the logits stream saturates HBM.
constexpr size_t kCounterStride = 256;
constexpr size_t kCounterWords = kCounterStride / sizeof(unsigned long long);
constexpr size_t kBatchWord = kCounterWords / 2;   // draw: the request's next segment batch (own 128-byte half)
#ifndef SV_DRAW_BATCHES
#define SV_DRAW_BATCHES 4
#endif
constexpr int kDrawBatchesPerWg = SV_DRAW_BATCHES;  // draw: segment batches per workgroup aimed for
constexpr float kNear = 1e-5f;       // |u - alpha| / CDF-gap band reported as NEAR_*
constexpr float kNearMass = 1e-6f;   // CDF-gap band in probability mass (gap * total weight)

// Partial statistics of one vocab chunk of one row (32 bytes).
//   greedy:   a = max logit, idx = lowest index attaining it (INT32_MAX if none), flags bit0 = NaN seen
//   sampling: a = m = max of x*coef (log2 units), b = z = sum exp2(x*coef - m);
//             g = the row's logit at the token it judges (chain: d_{j+1}), read by the workgroup whose
//             chunk holds that token (flags kPartGathered); sparse q, chunk 0 of a target row: q = q(d), the
//             summed mass of the draft row's valid candidates with id d, and flags kPartBadCandId /
//             kPartBadCandQ for its malformed candidate entries.
struct alignas(16) Part {
  float a;
  float b;
  int32_t idx;
  uint32_t flags;
  float g;
  float q;
  uint32_t pad0, pad1;
};
constexpr uint32_t kPartNaN = 1u;
constexpr uint32_t kPartGathered = 2u;
constexpr uint32_t kPartBadCandId = 4u;
constexpr uint32_t kPartBadCandQ = 8u;

struct Layout {
  int32_t L = 0;         // row slots per request (chain: max_verify_len, tree: n_nodes)
  int32_t P = 1;         // 2 when draft rows are streamed too (rejection)
  int32_t S = 1;         // vocab chunks per row in k_stats
  int64_t chunk = 0;     // tokens per chunk in k_stats
  int32_t S2 = 1;        // vocab chunks per request in k_draw
  int32_t spc = 1;       // segments per k_draw workgroup on average
  int32_t bseg = 1;      // segments per batch that a k_draw workgroup takes at a time
  int32_t n_seg = 0;     // segments per row
  int32_t n_piece = 0;   // sample-then-match: piece slots per row (0: no piece partials)
  size_t off_cnt2 = 0, off_part = 0, off_seg = 0, off_piece = 0;
  size_t off_cm = 0;     // fused commit: counter, then the published accept lengths and tree paths
  size_t off_mrow = 0;   // sample-then-match on short requests: each row's published result (16 B)
  size_t bytes = 0;
};

// Workspace carve-up and launch shapes; the same function serves spec_workspace_bytes and the calls.
inline Layout make_layout(int kind, int mode, int64_t total_rows, int64_t vocab, int32_t batch, int32_t L) {
  Layout lo;
  const bool sampling = mode != SPEC_MODE_GREEDY;
  lo.L = L;
  lo.P = (kind == SPEC_KIND_CHAIN && mode == SPEC_MODE_REJECTION) ? 2 : 1;
  const int64_t slots = int64_t(batch) * L * lo.P;
  // Rows are split into S chunks so that about SV_STATS_WGS (SV_MATCH_WGS, SV_STATS_WGS_GREEDY) workgroups
  // stream, with at least SV_STATS_MIN_CHUNK tokens per chunk and all of a request's partials fitting the
  // scan's LDS.
  const int64_t wgs = mode == SPEC_MODE_SAMPLE_MATCH ? SV_MATCH_WGS : sampling ? SV_STATS_WGS : SV_STATS_WGS_GREEDY;
  int64_t s = slots > 0 ? (wgs + slots - 1) / slots : 1;
  const int64_t min_chunk = (mode == SPEC_MODE_SAMPLE_MATCH && SV_MATCH_CHUNK < SV_STATS_MIN_CHUNK)
                                ? int64_t(SV_MATCH_CHUNK) : int64_t(SV_STATS_MIN_CHUNK);
  int64_t max_s = vocab / min_chunk;
  const int64_t lds_s = kMaxStagedParts / (int64_t(L) * lo.P);
  if (max_s > lds_s) max_s = lds_s;
  if (max_s < 1) max_s = 1;
  // Sample-then-match: rows whose length is a multiple of 16 bytes (vocab % 8 == 0) get piece partials from
  // the stream; other rows fall back to fine chunks, which bound what the draw reads.
  const bool pieces = mode == SPEC_MODE_SAMPLE_MATCH && kind == SPEC_KIND_CHAIN && vocab % 8 == 0;
  if (mode == SPEC_MODE_SAMPLE_MATCH && !pieces) {
    const int64_t fine = (vocab + SV_MATCH_CHUNK - 1) / SV_MATCH_CHUNK;
    if (s < fine) s = fine;
  }
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  int64_t chunk = (vocab + s - 1) / s;
  chunk = (chunk + 63) / 64 * 64;
  if (pieces) chunk = (chunk + kPieceChunk - 1) / kPieceChunk * kPieceChunk;
  lo.chunk = chunk;
  lo.S = int32_t((vocab + chunk - 1) / chunk);
  lo.n_seg = int32_t((vocab + kSeg - 1) / kSeg);
  // k_draw: ~SV_DRAW_WGS workgroups, each covering at least one segment per wave.
  int64_t s2 = batch > 0 ? (SV_DRAW_WGS + batch - 1) / batch : 1;
  const int64_t min_segs = kThreads / kWave;
  const int64_t max_s2 = (lo.n_seg + min_segs - 1) / min_segs;
  if (s2 > max_s2) s2 = max_s2;
  if (s2 < 1) s2 = 1;
  lo.spc = int32_t((lo.n_seg + s2 - 1) / s2);
  lo.S2 = (lo.n_seg + lo.spc - 1) / lo.spc;
  // Batches of whole trips (every wave SV_DRAW_TRIP segments), about kDrawBatchesPerWg per workgroup.
  const int64_t trip_segs = int64_t(kThreads / kWave) * SV_DRAW_TRIP;
  const int64_t trips = (lo.spc + trip_segs * kDrawBatchesPerWg - 1) / (trip_segs * kDrawBatchesPerWg);
  lo.bseg = int32_t(trip_segs * (trips > 0 ? trips : 1));
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t o = 0;
  lo.off_cnt2 = o; o = up(o + (sampling ? kCounterStride * size_t(batch) : 0));
  lo.off_part = o; o = up(o + sizeof(Part) * size_t(slots) * size_t(lo.S));
  lo.off_seg = o;  o = up(o + (sampling ? sizeof(float2) * size_t(batch) * size_t(lo.n_seg) : 0));
  lo.n_piece = pieces ? int32_t((vocab + kPieceMin - 1) / kPieceMin) : 0;
  lo.off_piece = o; o = up(o + sizeof(float2) * size_t(batch) * size_t(L) * size_t(lo.n_piece));
  // fused commit: one counter line, an accept length per request and (trees) the accepted path of each
  lo.off_cm = o; o = up(o + kCounterStride + sizeof(int32_t) * size_t(batch) *
                                                (1 + (kind == SPEC_KIND_TREE ? size_t(L) : 0)));
  lo.off_mrow = o;
  o = up(o + (mode == SPEC_MODE_SAMPLE_MATCH && kind == SPEC_KIND_CHAIN && L <= kMatchSplitMaxLen
                  ? 16 * size_t(batch) * size_t(L) : 0));
  lo.bytes = o;
  (void)total_rows;
  return lo;
}

// Kernel parameter block of k_stats, k_scan and k_draw (passed by value).
struct VerifyParams {
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
  unsigned long long* cnt2;   // draw-pass counters, armed by the logits stream
  Part* part;
  float2* seg;                // draw-pass segment sums
  int64_t V;
  int64_t total_rows;
  int64_t chunk;
  int32_t B, L, P, S;
  int32_t K;                  // sparse q: candidates per draft row (0 otherwise)
  int32_t S2, n_seg;          // draw pass: workgroups per request, segments per row
  int32_t bseg;               // draw pass: segments per batch
  float coef;                 // log2(e) / temperature (sampling modes)
  int32_t tree;               // 1: tree verify (rows node-major, B * L of them)
  const uint32_t* mask;       // vocab mask of the target rows, [rows, mask_words], or NULL
  int64_t mask_words;         // ceil(V / 32)
  float2* piece;              // sample-then-match: (m, z) per piece of each target row slot, or NULL
  uint4* mrow;                // sample-then-match on short requests: published row results [B, L]
  int32_t n_piece;            // piece slots per row slot
  // Fused KV commit (cm_on): each request's accept scan publishes its accept length (trees: and its path)
  // in pub_r / pub_path and counts itself on ccnt (reset by the logits stream); the workgroup that counts
  // last writes the commit outputs for the whole batch.
  int32_t cm_on;
  unsigned long long* ccnt;
  int32_t* pub_r;             // [B]
  int32_t* pub_path;          // trees: [B, L] node indices of the accepted path
  const int64_t* verify_slots;
  const int32_t* seq_lens;
  int32_t* commit_offsets;
  int64_t* src_slots;
  int32_t* dst_pos;
  int32_t* new_seq_lens;
  uint32_t* cstatus;
  int64_t* evict_slots;       // optional
  int32_t* evict_offsets;     // optional
};

struct CommitParams {
  spec_commit_args a;
};

// Host-side launchers (each in the translation unit of its kernel). They return hipSuccess or the
// launch error.
// Launch `kernel` on `stream`. With ev0 / ev1 the launch goes through hipExtLaunchKernelGGL, which sets
// the events to the kernel's own start and stop timestamps (what a kernel trace reports), not to points
// between launches.
template <typename P>
hipError_t launch_kernel(void (*kernel)(P), dim3 grid, dim3 block, size_t smem, hipStream_t stream, hipEvent_t ev0,
                         hipEvent_t ev1, const P& p) {
  if (ev0 || ev1) hipExtLaunchKernelGGL(kernel, grid, block, uint32_t(smem), stream, ev0, ev1, 0u, p);
  else hipLaunchKernelGGL(kernel, grid, block, smem, stream, p);
  return hipGetLastError();
}

// ev0 / ev1: optional events that take the kernel's own start / stop timestamps.
hipError_t launch_stats(int dtype, int mode, const VerifyParams& p, hipStream_t stream, hipEvent_t ev0,
                        hipEvent_t ev1);
// The second kernel of a verify call: k_scan (greedy) or k_draw (sampling modes).
hipError_t launch_scan(int dtype, const VerifyParams& p, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_draw(int dtype, int mode, const VerifyParams& p, hipStream_t stream, hipEvent_t ev0,
                       hipEvent_t ev1);
// The second kernel of a sample-then-match call: per request, one sample per row and the match scan.
hipError_t launch_match(int dtype, const VerifyParams& p, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_commit(const spec_commit_args& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_plan(const spec_plan_args& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_cap_trim(const spec_cap_trim_args& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_kv_move(const spec_kv_move_args& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_tree_build(const spec_tree_build_args& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
size_t tree_build_smem(int topk, int n_steps, int n_nodes, bool* q_cached);
spec_status plan_budget_host(const float* conf, int32_t R, int32_t W, const double* sps_rows, const double* sps,
                             int32_t n_sps, float eps, int32_t* budget, double* theta, int32_t* n_entries);
spec_status plan_budget_cost_host(const float* conf, int32_t R, int32_t W, const double* req_rows,
                                  const double* req_cost, int32_t n_req, const double* tok_rows,
                                  const double* tok_cost, int32_t n_tok, float eps, int32_t* budget, double* theta,
                                  int32_t* n_entries);
hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream);
hipError_t launch_read_fold(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream, hipEvent_t ev0,
                            hipEvent_t ev1);

}  // namespace sv
