/*
 * specverify.h — C ABI of the speculative-decoding verify / accept / commit path (gfx950, HIP).
 *
 * Sources (web pages; cited by page and section):
 *   [EAGLE→DFlash2]  tom-jerr.github.io, "从 EAGLE 到 DFlash 2：SGLang 与 SpecForge 的投机解码训练和推理"
 *   [DSpark]         ggaaooppeenngg.github.io, "DSpark：半自回归 + 置信度调度的 Speculative Decoding 深度分析"
 *   [DFlash]         astro-wiki.dev.mem.ac, "DFlash"
 *   [SpecDec]        zdszero.github.io, "speculative_decoding"
 *
 * One verify round (the draft → verify → commit loop of [SpecDec] "抽象：draft → verify → commit" and
 * [EAGLE→DFlash2] §1.1): the target has scored the verify rows [anchor, d1 .. dm] in one forward, so row j
 * holds the logits that judge d_{j+1} and the last row yields the bonus token. This library decides the
 * accepted prefix, draws the correction / bonus token and produces the KV-slot lists to commit.
 *
 * Conventions shared by every entry point
 *   - Every pointer in an argument struct is a DEVICE pointer owned by the caller, except where noted.
 *     The library never allocates device memory and never synchronises: all work is enqueued on `stream`
 *     (NULL = the null stream) and outputs are valid once the stream reaches that point.
 *   - Logits are row-major [rows, vocab] with row stride == vocab elements, dtype SPEC_DTYPE_F32 (IEEE
 *     float) or SPEC_DTYPE_BF16 (bfloat16 bit patterns, 2 bytes). Token ids are int32 in [0, vocab).
 *   - The return code reports only what the host can see (argument shapes, null pointers, enums,
 *     workspace size, launch failures). Problems in the DATA never abort: they set bits in the per-request
 *     `status` output (SPEC_ST_*), and the call still runs to completion.
 *   - Random decisions use caller-supplied uniforms in [0,1) (fp32). Given the uniforms the result is a
 *     deterministic function of the inputs: one uniform per row under test (`u_accept`) and one per
 *     request for the single final draw (`u_final`).
 *   - A workspace (scratch device memory sized by spec_workspace_bytes) serves one call at a time; calls
 *     that overlap on one workspace race. Its contents between calls do not matter: a call resets or
 *     overwrites every word it reads, so one workspace can be reused by later calls of any shape it is
 *     large enough for, and a call captured in a HIP graph replays correctly (no memset nodes are
 *     recorded). spec_workspace_init zero-fills one (optional).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same opaque types as the HIP runtime headers declare. */
typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

#define SPEC_ABI_VERSION 8

/* Host-visible return codes. */
typedef enum spec_status {
  SPEC_OK = 0,
  SPEC_EINVAL = 1,        /* null pointer where one is required, or a size / count out of range          */
  SPEC_EDTYPE = 2,        /* dtype is neither SPEC_DTYPE_F32 nor SPEC_DTYPE_BF16                          */
  SPEC_EUNSUPPORTED = 3,  /* valid request this library does not implement (mode/kind pair, thresholds) */
  SPEC_EWORKSPACE = 4,    /* workspace NULL or smaller than spec_workspace_bytes()                        */
  SPEC_ELAUNCH = 5,       /* a kernel launch or event record returned an error                           */
  SPEC_ESCRATCH = 6,      /* spec_verify_chain_noalloc: the call needs more than SPEC_NOALLOC_SCRATCH_BYTES */
} spec_status;

typedef enum spec_dtype { SPEC_DTYPE_F32 = 0, SPEC_DTYPE_BF16 = 1 } spec_dtype;

/*
 * Verify modes.
 *   GREEDY       accept d_j while d_j == argmax(row j-1); the first mismatch is replaced by that argmax and
 *                a fully accepted draft gets argmax(row m) as bonus. Ties go to the LOWEST token id.
 *                Chain or tree. [SpecDec] "为什么结果不受 draft 影响" (verify_tree_greedy; a chain is a
 *                tree with one child per node); [EAGLE→DFlash2] §1.2 (same numerics and tie-breaking).
 *   REJECTION    chain only: accept d_j iff u_j < alpha_j = min(1, p_{j-1}(d_j)/q_{j-1}(d_j)); on the first
 *                rejection draw from [p-q]_+ / sum[p-q]_+, after full acceptance draw the bonus from p_m.
 *                p, q = softmax(logits / temperature). [EAGLE→DFlash2] §1.2 (alpha, residual p'),
 *                §1.1 (m+1 tokens on full acceptance); [SpecDec] (chain_speculative_sampling, topk = 1).
 *   TARGET_ONLY  tree only: judge children with the target probabilities alone (draft probabilities taken
 *                as zero), thresholds single/acc = 1.0 only. [SpecDec] "为什么结果不受 draft 影响"
 *                (tree_speculative_sampling_target_only). Rule used: walking down from the root, at node
 *                `cur` add p_cur(token) of each child in ascending node order (a token already seen among
 *                earlier siblings adds nothing) into acc and accept the first child with u_cur < acc; if
 *                none is accepted draw from p_cur with the tried tokens zeroed; at a leaf draw from p_cur.
 *   REJECTION_SPARSE
 *                chain only: REJECTION where each draft row's q arrives as K (candidate id, probability)
 *                pairs instead of draft logits: q is that candidate distribution scattered into vocab
 *                coordinates and zero elsewhere, so [p-q]_+ still covers the whole vocab and tokens
 *                outside the candidates remain reachable ([EAGLE→DFlash2] §6.5, sampling verify with the
 *                selector's q; greedy rows carry a one-hot q, i.e. K = 1 with probability 1). A repeated id
 *                adds its masses. The temperature divides the target logits only.
 *   SAMPLE_MATCH chain only: sample-then-match. Every target row j draws its own token t_j from p_j =
 *                softmax(logits / temperature) by inverse CDF (row j < m with u_accept of d_{j+1}, row m with
 *                u_final); d_{j+1} is accepted while it equals t_j, and the first mismatch (or row m) emits t_j.
 *                Every emitted token is a draw from its row's p. [DFlash] decode loop step 4 (compare each
 *                draft token with a sample of the posterior, longest matching prefix, first mismatch replaced
 *                by the posterior sample); [EAGLE→DFlash2] §1.2 (independent target sampling then prefix
 *                matching is a different implementation from p/q rejection). accept_prob reports p_j(d_{j+1})
 *                at the compared positions; residual_mass is -1 (no residual).
 *
 * Vocab (grammar) mask, every mode, optional: `vocab_mask` holds ceil(vocab/32) 32-bit words per target
 * row; token v of a row is allowed iff bit (v % 32) of word v / 32 is 1. A masked logit counts as -inf
 * whatever its value (before temperature, softmax and argmax); draft rows are not masked.
 * [EAGLE→DFlash2] §5.6.6 (the grammar mask is applied after the target forward, before acceptance) and
 * §8.4 (sampling reads the distribution after the mask). A row that leaves no token with a finite logit
 * sets SPEC_ST_NONFINITE in every mode.
 */
typedef enum spec_mode {
  SPEC_MODE_GREEDY = 0,
  SPEC_MODE_REJECTION = 1,
  SPEC_MODE_TARGET_ONLY = 2,
  SPEC_MODE_REJECTION_SPARSE = 3,
  SPEC_MODE_SAMPLE_MATCH = 4,
} spec_mode;

typedef enum spec_kind {
  SPEC_KIND_CHAIN = 0,
  SPEC_KIND_TREE = 1,
  SPEC_KIND_COMMIT = 2,
  SPEC_KIND_PLAN = 3,
  SPEC_KIND_CAP_TRIM = 4,
  SPEC_KIND_KV_MOVE = 5,
  SPEC_KIND_TREE_BUILD = 6,
} spec_kind;

/* Per-request status bits (output `status[b]`). */
#define SPEC_ST_NONFINITE     (1u << 0) /* a NaN logit in one of the request's rows; in sampling modes also
                                           +inf, or a row whose logits are all -inf                         */
#define SPEC_ST_BAD_TOKEN     (1u << 1) /* a draft / node token outside [0, vocab); it is never accepted    */
#define SPEC_ST_BAD_OFFSETS   (1u << 2) /* off[b] / off[b+1] fail the request's own checks (non-empty, at
                                           most max_verify_len rows, b <= off[b], off[b+1] <= T - B + b + 1,
                                           off[0] = 0, off[B] = T): the whole batch's outputs are then
                                           unspecified (no memory outside the given buffers is touched)    */
#define SPEC_ST_BAD_PARENT    (1u << 3) /* tree: parent[0] != -1 or parent[i] not in [0, i); such a node is
                                           nobody's child                                                   */
#define SPEC_ST_BAD_UNIFORM   (1u << 4) /* a uniform that is NaN or outside [0,1); it is used as 0 if NaN,
                                           else clamped to [0, 1 - 2^-24]                                    */
#define SPEC_ST_ZERO_Q        (1u << 5) /* rejection: q(d) == 0 at an examined position (alpha = 1 if
                                           p(d) > 0, else 0)                                                 */
#define SPEC_ST_ZERO_RESIDUAL (1u << 6) /* the final draw's weights summed to 0; drawn from p instead        */
#define SPEC_ST_NEAR_ALPHA    (1u << 7) /* diagnostic: |u - alpha| < 1e-5 at an examined accept test        */
#define SPEC_ST_NEAR_CDF      (1u << 8) /* diagnostic: the final draw's u lies within 1e-5 of a CDF step, or
                                           that margin times the weights' total mass Z is below 1e-6        */
#define SPEC_ST_BAD_ACCEPT    (1u << 9) /* commit: accept_len / accept_index outside the request's rows     */
#define SPEC_ST_BAD_Q         (1u << 10) /* REJECTION_SPARSE: a candidate probability that is negative or not
                                            finite; the entry is left out (an out-of-range candidate id
                                            sets SPEC_ST_BAD_TOKEN and is left out too)                     */
#define SPEC_ST_BAD_CONF      (1u << 11) /* planner / tree build: a confidence or draft probability that is NaN
                                            (used as 0) or outside [0, 1] (clamped into it)                 */
#define SPEC_ST_BAD_SLOT      (1u << 12) /* KV move: a slot, position, request row or commit range outside the
                                            given tables; the entry (or the request's range) is skipped     */

/*
 * Chain verify (GREEDY, REJECTION, REJECTION_SPARSE or SAMPLE_MATCH).
 *
 * Request b owns target rows [off[b], off[b+1]) (the ragged packing of [EAGLE→DFlash2] §5.6.5: verify
 * lens [4,2,6] -> offsets [0,4,6,12]); m_b = off[b+1] - off[b] - 1 >= 0 drafts. Draft-side arrays are
 * packed with m_b entries per request starting at off[b] - b; entry j of request b belongs to d_{j+1}:
 * draft_tokens[off[b]-b+j] = d_{j+1}, draft_logits row off[b]-b+j = the draft logits q_j that proposed
 * d_{j+1}, u_accept[off[b]-b+j] = the uniform of the test of d_{j+1}.
 *
 * Outputs (indexed like the verify rows unless noted; entries past the accepted part are -1):
 *   accept_len[b]             r = number of accepted drafts, 0 <= r <= m_b
 *   bonus[b]                  the token emitted after the accepted drafts (correction or bonus)
 *   out_tokens[off[b]+k]      k < r: d_{k+1}; k == r: bonus; k > r: -1
 *   accept_index[off[b]+k]    k <= r: off[b]+k (global verify row whose KV is committed); else -1
 *   status[b]                 SPEC_ST_* bits
 *   accept_prob[off[b]-b+j]   opt.: alpha_{j+1} where tested (sampling modes), else -1
 *   residual_mass[b]          opt.: sum of the final draw's weights (sampling modes), -1 in GREEDY
 */
typedef struct spec_commit_args spec_commit_args;

/*
 * Fused KV commit (optional, chain and tree verify): `commit` (a HOST pointer, NULL = none) asks the verify call
 * to also produce this round's KV commit lists in the same launches ([EAGLE→DFlash2] §5.6: the accept step
 * returns the accept lengths, bonus tokens and commit lengths together; §5.6.6 commit_lens = correct_len + 1).
 * The outputs are exactly those spec_commit_indices would give for row_offsets = target_offsets (chain) or
 * [0, N, 2N, ..] (tree), accept_len / accept_index = this call's outputs, total_rows, batch and
 * max_verify_len = this call's (tree: n_nodes). From *commit only verify_slots, seq_lens, the outputs
 * (commit_offsets, src_slots, dst_pos, new_seq_lens, status and the optional evict_slots / evict_offsets) and
 * capacity (>= total_rows) are used; its row_offsets, accept_len, accept_index, total_rows, batch,
 * max_verify_len and profile events are ignored. The commit runs in the call's second kernel, in the
 * workgroup that finishes its request's accept scan last, so it adds no launch and no kernel to
 * spec_kernel_count. A NULL verify_slots / seq_lens / output, or capacity < total_rows, is SPEC_EINVAL. When
 * requests report SPEC_ST_BAD_OFFSETS (the batch's verify outputs are then unspecified) every request whose own
 * offsets pass still commits its first accept_len + 1 rows; batch 0 launches nothing (commit_offsets untouched).
 */
typedef struct spec_chain_args {
  const void* target_logits;     /* [total_rows, vocab]                                   */
  const int32_t* target_offsets; /* [batch+1], off[0] = 0, off[batch] = total_rows           */
  const void* draft_logits;      /* [total_rows - batch, vocab]; REJECTION only (else NULL) */
  const int32_t* draft_tokens;   /* [total_rows - batch]                                   */
  const float* u_accept;         /* [total_rows - batch]; sampling modes only              */
  const float* u_final;          /* [batch]; sampling modes only                           */
  int32_t* accept_len;           /* [batch]                                                */
  int32_t* bonus;                /* [batch]                                                */
  int32_t* out_tokens;           /* [total_rows]                                           */
  int32_t* accept_index;         /* [total_rows]                                           */
  uint32_t* status;              /* [batch]                                                */
  float* accept_prob;            /* optional [total_rows - batch]                          */
  float* residual_mass;          /* optional [batch]                                       */
  void* workspace;               /* >= spec_workspace_bytes(SPEC_KIND_CHAIN, ...) bytes    */
  size_t workspace_bytes;
  hipEvent_t* profile_events;    /* HOST array, optional: n_profile_events = 2 * kernels events
                                    (see spec_kernel_count); events 2k and 2k+1 take the start
                                    and stop timestamps of kernel k itself (its dispatch on
                                    `stream`, as a kernel trace reports it)                    */
  int64_t total_rows;            /* T_rows = sum_b (m_b + 1)                                */
  int64_t vocab;                 /* V, 1 <= V <= 2^22                                       */
  int32_t batch;                 /* B >= 0 (B == 0: nothing is launched)                    */
  int32_t max_verify_len;        /* upper bound on m_b + 1, 1..1024; a longer request is
                                    reported as SPEC_ST_BAD_OFFSETS                        */
  int32_t dtype;                 /* spec_dtype                                             */
  int32_t mode;                  /* SPEC_MODE_GREEDY, _REJECTION, _REJECTION_SPARSE or
                                    _SAMPLE_MATCH                                            */
  float temperature;             /* sampling modes: finite, > 0; logits are divided by it    */
  int32_t n_profile_events;
  /* REJECTION_SPARSE only (else NULL / 0): candidate k of draft row i sits at [i * n_cand + k]     */
  const int32_t* cand_ids;       /* [total_rows - batch, n_cand] candidate token ids        */
  const float* cand_q;           /* [total_rows - batch, n_cand] their probabilities        */
  int32_t n_cand;                /* K, 1..1024                                             */
  int32_t reserved;
  const uint32_t* vocab_mask;    /* optional [total_rows, ceil(vocab/32)] allowed-token bits of
                                    the target rows (see "Vocab (grammar) mask"); NULL: none   */
  const spec_commit_args* commit; /* optional HOST pointer: fused KV commit (see above)        */
} spec_chain_args;

/*
 * Tree verify (GREEDY or TARGET_ONLY). Request b owns n_nodes verify rows b*N .. b*N+N-1 (node-major),
 * node 0 is the anchor (root), node i > 0 has parent[b*N+i] in [0, i) and token tokens[b*N+i]; row i
 * holds the target logits that judge node i's children ([EAGLE→DFlash2] §2.4 and §3.4: tree attention
 * gives every node its own distribution in one forward). Among equal candidates the lowest node index
 * wins. accept_index lists the path [0, n_1, .., n_r] as global rows b*N + n_k (compaction source for
 * the topk > 1 accepted path, [EAGLE→DFlash2] §8.2).
 *
 * Outputs as for the chain, sized batch*N (accept_prob[b*N+c] = acc when child c was tested in
 * TARGET_ONLY, else -1; residual_mass is -1 in GREEDY).
 */
typedef struct spec_tree_args {
  const void* target_logits; /* [batch*n_nodes, vocab]                          */
  const int32_t* parents;    /* [batch*n_nodes]                                 */
  const int32_t* tokens;     /* [batch*n_nodes] (node 0's entry is ignored)     */
  const float* u_accept;     /* [batch*n_nodes]: uniform used at node cur; TARGET_ONLY */
  const float* u_final;      /* [batch]; TARGET_ONLY                            */
  int32_t* accept_len;       /* [batch]                                         */
  int32_t* bonus;            /* [batch]                                         */
  int32_t* out_tokens;       /* [batch*n_nodes]                                 */
  int32_t* accept_index;     /* [batch*n_nodes]                                 */
  uint32_t* status;          /* [batch]                                         */
  float* accept_prob;        /* optional [batch*n_nodes]                        */
  float* residual_mass;      /* optional [batch]                                */
  void* workspace;
  size_t workspace_bytes;
  hipEvent_t* profile_events; /* HOST array, optional (see spec_chain_args)      */
  int64_t vocab;
  int32_t batch;
  int32_t n_nodes;           /* N, 1..1024                                      */
  int32_t dtype;
  int32_t mode;              /* SPEC_MODE_GREEDY or SPEC_MODE_TARGET_ONLY        */
  float temperature;         /* TARGET_ONLY: finite, > 0                         */
  float threshold_single;    /* TARGET_ONLY: must be 1.0 (else SPEC_EUNSUPPORTED) */
  float threshold_acc;       /* TARGET_ONLY: must be 1.0 (else SPEC_EUNSUPPORTED) */
  int32_t n_profile_events;
  const uint32_t* vocab_mask; /* optional [batch*n_nodes, ceil(vocab/32)] allowed-token bits of
                                 every node row; NULL: none                      */
  const spec_commit_args* commit; /* optional HOST pointer: fused KV commit (see spec_chain_args) */
} spec_tree_args;

/*
 * KV commit compaction ([EAGLE→DFlash2] §5.6.6 and §8.1: commit_lens = correct_len + 1, the KV of the
 * old anchor plus the r accepted drafts; [SpecDec] "实现：共享的骨架": accepted KV moves to contiguous
 * positions after seq_lens, rejected slots are reused later).
 *   commit_offsets[b]            exclusive scan of (accept_len[b] + 1); commit_offsets[batch] = total
 *   src_slots[commit_offsets[b]+k] = verify_slots[accept_index[row_offsets[b]+k]],  k = 0..accept_len[b]
 *   dst_pos[commit_offsets[b]+k]   = seq_lens[b] + k
 *   new_seq_lens[b]              = seq_lens[b] + accept_len[b] + 1
 *   evict_offsets[b], evict_slots  optional: the request's verify rows NOT listed in its accept_index, in
 *                                  ascending row order (their KV must stop being visible, §8.2)
 * row_offsets has the chain meaning (trees: [0, N, 2N, ...]). capacity (length of src_slots / dst_pos /
 * evict_slots) must be >= total_rows. Invalid accept_len / accept_index set SPEC_ST_BAD_ACCEPT: an
 * accept_len outside [0, rows) is clamped into it; an accept_index entry outside the request's rows commits
 * src_slots = -1; an entry naming a row a second time commits that row's slot again; the request evicts
 * exactly the rows no entry names (so its evict count is rows - distinct named rows).
 */
struct spec_commit_args {
  const int32_t* row_offsets;  /* [batch+1]                    */
  const int32_t* accept_len;   /* [batch]                      */
  const int32_t* accept_index; /* [total_rows]                 */
  const int64_t* verify_slots; /* [total_rows] KV slot per verify row */
  const int32_t* seq_lens;     /* [batch] committed length before this round */
  int32_t* commit_offsets;     /* [batch+1]                    */
  int64_t* src_slots;          /* [capacity]                   */
  int32_t* dst_pos;            /* [capacity]                   */
  int32_t* new_seq_lens;       /* [batch]                      */
  uint32_t* status;            /* [batch]                      */
  int64_t* evict_slots;        /* optional [capacity]          */
  int32_t* evict_offsets;      /* optional [batch+1]           */
  hipEvent_t* profile_events;  /* HOST array, optional          */
  int64_t total_rows;
  int64_t capacity;
  int32_t batch;
  int32_t max_verify_len;      /* upper bound on rows per request, 1..1024 */
  int32_t n_profile_events;
  int32_t reserved;
};

/*
 * Verify-length planner, device side: how many of each request's W proposed drafts this round verifies
 * ([EAGLE→DFlash2] §5.6.4 device allocation, §5.6.5 ragged layout; [DSpark] confidence truncation).
 *
 * confidence[r*W + j] = c_{r,j}, the draft head's estimate that draft j+1 of request r survives given that
 * draft j did; the prefix survival is A_{r,j} = c_{r,0} * .. * c_{r,j} (float32 products in position order).
 *   SPEC_PLAN_TOPK       rank every (r, j) with A_{r,j} >= survival_eps by A descending, then position j
 *                        ascending, then request r ascending; the first `budget` of them are verified, so
 *                        request r verifies selected[r] drafts (a prefix, since A falls along j). budget < 0
 *                        means no budget: every request verifies all W drafts.
 *   SPEC_PLAN_THRESHOLD  request r verifies the drafts before its first position with c_{r,j} < threshold
 *                        (all W if none).
 * Then verify_lens[r] = clamp(1 + selected[r], min_verify_len, max_verify_len) (the anchor row plus the
 * drafts), offsets = [0, verify_lens[0], ..] (exclusive prefix sum, total offsets[batch]; the layout
 * spec_verify_chain takes), and row_index[offsets[r] + j] = r*(W+1) + j maps each compact verify row to its
 * place in the uniform (W+1)-wide block [anchor, d_1 .. d_W] of request r. One workgroup, one kernel.
 * A NaN confidence counts as 0 and one outside [0, 1] is clamped into it (SPEC_ST_BAD_CONF).
 */
typedef enum spec_plan_mode { SPEC_PLAN_TOPK = 0, SPEC_PLAN_THRESHOLD = 1 } spec_plan_mode;

typedef struct spec_plan_args {
  const float* confidence;     /* [batch, width]                                                  */
  int32_t* selected;           /* [batch] drafts verified beyond the anchor                        */
  int32_t* verify_lens;        /* [batch]                                                         */
  int32_t* offsets;            /* [batch+1]                                                       */
  int64_t* row_index;          /* optional [batch*(width+1)]; entries past offsets[batch] untouched */
  uint32_t* status;            /* optional [batch]: SPEC_ST_BAD_CONF                               */
  hipEvent_t* profile_events;  /* HOST array, optional (2 events: the kernel's start / stop)        */
  int32_t batch;               /* R, 0..2^20-1                                                    */
  int32_t width;               /* W drafts proposed per request, 0..4095                           */
  int32_t mode;                /* spec_plan_mode                                                  */
  int32_t budget;              /* TOPK: drafts to verify over the batch (K); < 0: all of them       */
  int32_t min_verify_len;      /* 1 <= min_verify_len <= max_verify_len <= width + 1               */
  int32_t max_verify_len;
  float survival_eps;          /* TOPK: entries with survival below it are never selected (>= 0)   */
  float threshold;             /* THRESHOLD                                                       */
  int32_t n_profile_events;
  int32_t reserved;
} spec_plan_args;

spec_status spec_plan_layout(const spec_plan_args* args, hipStream_t stream);

/*
 * Verify-length planner, host side: the budget K ([EAGLE→DFlash2] §5.6.3; [DSpark] Hardware-Aware Prefix
 * Scheduler). From lagged confidences (HOST memory, [batch, width]) it takes the survival products as
 * spec_plan_layout does, drops those below survival_eps, sorts the rest descending a_1 >= .. >= a_n and
 * returns K* = argmax over 0 <= K <= n of (batch + a_1 + .. + a_K) * SPS(batch + K) (the smallest K among
 * equal values), where SPS(M), the engine's steps per second at M target rows, is linear between the
 * table points (sps_rows ascending, sps) and the nearest end value outside them. theta (optional, at least
 * batch*width + 1 doubles) receives the predicted throughput of K = 0 .. n, n_entries (optional) n.
 * Pure host function; SPEC_EINVAL for bad sizes, null pointers or a table whose rows do not increase.
 */
spec_status spec_plan_budget(const float* confidence_hist, int32_t batch, int32_t width, const double* sps_rows,
                             const double* sps, int32_t n_sps, float survival_eps, int32_t* budget,
                             double* theta, int32_t* n_entries);

/*
 * The same host budget under an additive cost table ([EAGLE→DFlash2] §5.6.3: with an additive cost table the
 * objective becomes N(K) / T(R, R + K)): K* = argmax over 0 <= K <= n of (batch + a_1 + .. + a_K) /
 * (T_req(batch) + T_tok(batch + K)), the smallest K among equal values. The pages name the table without
 * defining T; here a step's predicted time is the sum of a per-batch term read from (req_rows, req_cost) at
 * the request count and a per-row term read from (tok_rows, tok_cost) at the target row count, each linear
 * between its points and the nearest end value outside them (as for SPS). With T_req = 0 and T_tok = 1 / SPS
 * at every row count it is spec_plan_budget. theta receives N(K) / T for K = 0 .. n (output per unit of the
 * tables' time). Rows must increase strictly, req_cost >= 0 and tok_cost > 0 (every step time positive),
 * all finite; else SPEC_EINVAL, as for bad sizes or null pointers. Pure host function.
 */
spec_status spec_plan_budget_cost(const float* confidence_hist, int32_t batch, int32_t width,
                                  const double* req_rows, const double* req_cost, int32_t n_req,
                                  const double* tok_rows, const double* tok_cost, int32_t n_tok,
                                  float survival_eps, int32_t* budget, double* theta, int32_t* n_entries);

/*
 * Accept cutoff of a verify run over the full proposal width ([EAGLE→DFlash2] §5.6.6: the accept kernel's
 * cap_trim / commit_lens / block_accept_lens). For request b with rows [row_offsets[b], row_offsets[b+1])
 * of a full-width verify (raw_accept_len, raw_bonus, out_tokens from spec_verify_chain) and the plan's
 * verify_lens[b]:
 *   ell = verify_lens[b] - 1, correct_len = min(raw, ell), cap_trim_lens = raw - correct_len,
 *   commit_lens = correct_len + 1, block_accept_lens = commit_lens + cap_trim_lens.
 * A cut request (cap_trim_lens > 0) emits the token at position ell (the accepted draft d_{ell+1}) as its
 * bonus and its out_tokens after position ell become -1; otherwise bonus = raw_bonus. Requests whose rows
 * or lengths are invalid get SPEC_ST_BAD_ACCEPT, -1 outputs and untouched tokens. Feed correct_len to
 * spec_commit_indices as the accept length.
 */
typedef struct spec_cap_trim_args {
  const int32_t* row_offsets;     /* [batch+1] rows of the full-width verify                        */
  const int32_t* verify_lens;     /* [batch]                                                        */
  const int32_t* raw_accept_len;  /* [batch]                                                        */
  const int32_t* raw_bonus;       /* [batch]                                                        */
  int32_t* out_tokens;            /* [total_rows], read and rewritten in place                      */
  int32_t* correct_len;           /* [batch]                                                        */
  int32_t* cap_trim_lens;         /* [batch]                                                        */
  int32_t* commit_lens;           /* [batch]                                                        */
  int32_t* block_accept_lens;     /* [batch]                                                        */
  int32_t* bonus;                 /* [batch]                                                        */
  uint32_t* status;               /* [batch]                                                        */
  hipEvent_t* profile_events;     /* HOST array, optional (2 events)                                */
  int64_t total_rows;
  int32_t batch;
  int32_t n_profile_events;
} spec_cap_trim_args;

spec_status spec_cap_trim(const spec_cap_trim_args* args, hipStream_t stream);

/*
 * KV data move of a commit ([EAGLE→DFlash2] §8.2: a tree's accepted path is not contiguous in the flattened
 * tree, so its KV is compacted to the positions after seq_lens; the engineering note on
 * move_accept_tokens_to_target_kvcache: the accepted tokens' KV moves to the contiguous positions after
 * seq_lens, rejected slots are overwritten later). Takes the lists of spec_commit_indices. For request b,
 * entries e = commit_offsets[b] .. commit_offsets[b+1]-1 are moved in that order (path order):
 *   dst_slot = req_to_token[req_pool_indices[b] * max_context + dst_pos[e]],
 *   for every buffer: row dst_slot <- row src_slots[e]   (nothing when src == dst, e.g. a chain).
 * For a tree path this equals reading every source before writing any destination. Buffers are raw bytes:
 * buffers[i] is the device base address of buffer i, [n_slots, row_bytes] (e.g. K and V of every layer of
 * the target and of the draft). An entry outside the tables, or a request whose commit range is outside
 * [0, capacity], is skipped and sets SPEC_ST_BAD_SLOT.
 */
typedef struct spec_kv_move_args {
  const uint64_t* buffers;          /* device [n_buffers] base addresses                               */
  const int32_t* commit_offsets;    /* [batch+1]                                                       */
  const int64_t* src_slots;         /* [capacity]                                                      */
  const int32_t* dst_pos;           /* [capacity]                                                      */
  const int64_t* req_to_token;      /* [n_req_rows, max_context] slot of each (request row, position)   */
  const int32_t* req_pool_indices;  /* [batch] row of req_to_token of each request                     */
  uint32_t* status;                 /* optional [batch]                                                */
  hipEvent_t* profile_events;       /* HOST array, optional (2 events)                                 */
  int64_t n_slots;
  int64_t max_context;
  int64_t n_req_rows;
  int64_t capacity;                 /* entries of src_slots / dst_pos                                  */
  int32_t row_bytes;                /* bytes per slot per buffer: a multiple of 16, 16 .. 2^20         */
  int32_t n_buffers;                /* 1 .. 65535                                                      */
  int32_t batch;
  int32_t n_profile_events;
} spec_kv_move_args;

spec_status spec_kv_move(const spec_kv_move_args* args, hipStream_t stream);

/*
 * EAGLE-2 dynamic draft-tree construction ([EAGLE→DFlash2] §2.3–§2.4; [SpecDec] EAGLE tree build: topk^2 ->
 * topk per step, then the best n_nodes - 1 nodes plus the root). Per request: the draft's top-k children of
 * each frontier node at each of S steps, draft_tokens / draft_probs [batch, S, topk, topk] (step s, frontier
 * slot f, child rank c; step 0 expands the root only, slot 0). A candidate's score is the float32 product of
 * the probabilities along its path; candidate ids are c at step 0 and topk + (s-1) topk^2 + f topk + c at
 * step s. Every selection ranks by score descending, then candidate id ascending: the frontier after step s is
 * the top topk of step s's candidates (frontier slot = rank), and the tree's nodes are the root (node 0, token
 * = anchors[b]) and the top n_nodes - 1 of all candidates, in candidate-id order (a parent precedes its
 * children; the ancestor closure holds since a child never outranks its parent).
 * Outputs, [batch, n_nodes] unless noted: tokens, parents (root -1; the input spec_verify_tree takes),
 * positions = seq_lens[b] + depth (depth, not the flattened index), mask [batch, n_nodes, n_nodes] uint8
 * (mask[i][j] = 1 iff j is i or an ancestor of i: a node sees the committed history, its ancestors and
 * itself), first_child / next_sibling (-1 if none), cand_index (candidate id of each node, -1 for the root),
 * status (SPEC_ST_BAD_CONF). One workgroup per request.
 */
typedef struct spec_tree_build_args {
  const int32_t* anchors;           /* [batch]                                                        */
  const int32_t* draft_tokens;      /* [batch, n_steps, topk, topk]                                   */
  const float* draft_probs;         /* [batch, n_steps, topk, topk]                                   */
  const int32_t* seq_lens;          /* [batch]                                                        */
  int32_t* tokens;                  /* [batch, n_nodes]                                               */
  int32_t* parents;                 /* [batch, n_nodes]                                               */
  int32_t* positions;               /* [batch, n_nodes]                                               */
  uint8_t* mask;                    /* optional [batch, n_nodes, n_nodes]                             */
  int32_t* first_child;             /* optional [batch, n_nodes]                                      */
  int32_t* next_sibling;            /* optional [batch, n_nodes]                                      */
  int32_t* cand_index;              /* optional [batch, n_nodes]                                      */
  uint32_t* status;                 /* [batch]                                                        */
  hipEvent_t* profile_events;       /* HOST array, optional (2 events)                                */
  int32_t batch;
  int32_t n_steps;                  /* S >= 1                                                         */
  int32_t topk;                     /* 1 .. 64; topk + (S-1) topk^2 candidates, at most 4096            */
  int32_t n_nodes;                  /* 1 .. min(1024, candidates + 1)                                 */
  int32_t n_profile_events;
  int32_t reserved;
} spec_tree_build_args;

spec_status spec_tree_build(const spec_tree_build_args* args, hipStream_t stream);

spec_status spec_verify_chain(const spec_chain_args* args, hipStream_t stream);

/* spec_verify_chain for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same kernels and results, with the workspace taken
 * from a static device array of SPEC_NOALLOC_SCRATCH_BYTES bytes inside the library instead of
 * args->workspace (workspace / workspace_bytes are ignored and may be NULL / 0). The caller still passes
 * every input and output. The array exists once per GPU and stays until the process ends; its address is
 * looked up on the first call on each GPU (the GPU of `stream`). Nothing in it has to start at zero (each
 * call resets what it counts with), but every call on one GPU shares it: calls that overlap on one GPU
 * (other streams, other threads) race. A call whose spec_workspace_bytes exceeds the array returns
 * SPEC_ESCRATCH and launches nothing. No allocation or free of any kind is made. */
#define SPEC_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
spec_status spec_verify_chain_noalloc(const spec_chain_args* args, hipStream_t stream);

spec_status spec_verify_tree(const spec_tree_args* args, hipStream_t stream);
spec_status spec_commit_indices(const spec_commit_args* args, hipStream_t stream);

/* Workspace size in bytes for a call of this kind/mode and size (0 for SPEC_KIND_COMMIT). For trees pass
   total_rows = batch * n_nodes. Returns 0 for invalid arguments. Pure host function. */
size_t spec_workspace_bytes(int32_t kind, int32_t mode, int64_t total_rows, int64_t vocab, int32_t batch,
                            int32_t max_verify_len);

/* Zero-fills `bytes` of device memory at `workspace` with a kernel on `stream` (no memset node).
   Returns SPEC_EINVAL for a NULL workspace with bytes > 0, SPEC_ELAUNCH if the launch fails. */
spec_status spec_workspace_init(void* workspace, size_t bytes, hipStream_t stream);

/* A plain read of `bytes` of device memory at `src` (16-byte loads, every byte once, as the logits stream
   reads its rows), on `stream`: the reference for the stream's rate, this GPU's achievable HBM read rate at
   the same size, measured beside the verify kernels. Each of its workgroups (at most SPEC_READ_SINK_WORDS)
   stores the XOR of the 32-bit words it read into its own word of `sink` (device memory, SPEC_READ_SINK_WORDS
   uint32 words, zeroed by the caller): the XOR of all sink words is the XOR of every word read. events:
   NULL, or a HOST array of 2 events that take the kernel's own start and stop timestamps (as profile_events
   do for a verify call). src 16-byte aligned and bytes a multiple of 16, else SPEC_EINVAL (bytes = 0:
   nothing to do); SPEC_ELAUNCH if the launch fails. Not part of a verify call. */
#define SPEC_READ_SINK_WORDS 8192
spec_status spec_read_probe(const void* src, size_t bytes, uint32_t* sink, hipEvent_t* events, hipStream_t stream);

/* Number of kernels a call of this kind/mode launches (events: kernels + 1). Pure host function. */
int32_t spec_kernel_count(int32_t kind, int32_t mode);

/* Static string naming a return code (any int: codes that are no spec_status get "unknown spec_status").
   Pure host function. */
const char* spec_status_string(int32_t code);

/* SPEC_ABI_VERSION the library was built with, and sizeof of the argument structs (ABI checks). */
int32_t spec_abi_version(void);
size_t spec_args_size(int32_t kind);

#ifdef __cplusplus
}
#endif
#endif /* SPECVERIFY_H */
