// The steps on either side of a tree verify:
//   k_kv_move     the KV data move of a commit ([EAGLE→DFlash2] §8.2; move_accept_tokens_to_target_kvcache):
//                 accepted rows go to the slots of positions seq_len + k, in every KV buffer.
//   k_tree_build  EAGLE-2 dynamic draft-tree construction ([EAGLE→DFlash2] §2.3–§2.4): path-product scores,
//                 topk^2 -> topk frontier per step, rerank of all candidates, then the tree arrays the
//                 verify and the tree attention take (parents, depth positions, ancestor mask, first child,
//                 next sibling).
#include "sv_device.h"

namespace sv {

namespace {

// ---------------------------------------------------------------------------------------------------
// KV move. Workgroup (request, buffer, row chunk); thread t owns 16-byte lane t of the chunk in every row
// it copies, so entries are applied in path order by each thread's program order (a later entry never
// overwrites a row an earlier one still has to read, and no barrier is needed).
// ---------------------------------------------------------------------------------------------------
constexpr int kMoveLanes = 256;   // 16-byte lanes per workgroup (4 KB of a row)

struct MoveParams {
  spec_kv_move_args a;
  int chunks;
};

__global__ __launch_bounds__(kMoveLanes) void k_kv_move(MoveParams mp) {
  const spec_kv_move_args& a = mp.a;
  const int chunks = mp.chunks;
  const int c = blockIdx.x % chunks;
  const int buf = (blockIdx.x / chunks) % a.n_buffers;
  const int b = blockIdx.x / (chunks * a.n_buffers);
  const bool reporter = buf == 0 && c == 0 && threadIdx.x == 0;
  const int64_t e0 = a.commit_offsets[b], e1 = a.commit_offsets[b + 1];
  const int32_t pool = a.req_pool_indices[b];
  uint32_t st = 0;
  if (!(0 <= e0 && e0 <= e1 && e1 <= a.capacity) || !(pool >= 0 && pool < a.n_req_rows)) {
    st = SPEC_ST_BAD_SLOT;
  } else {
    char* base = reinterpret_cast<char*>(a.buffers[buf]);
    const int64_t lane = int64_t(c) * kMoveLanes + threadIdx.x;
    const bool active = lane * 16 < a.row_bytes;
    const int64_t* r2t = a.req_to_token + int64_t(pool) * a.max_context;
    for (int64_t e = e0; e < e1; ++e) {
      const int64_t src = a.src_slots[e];
      const int32_t pos = a.dst_pos[e];
      if (!(pos >= 0 && pos < a.max_context)) {
        st |= SPEC_ST_BAD_SLOT;
        continue;
      }
      const int64_t dst = r2t[pos];
      if (!(src >= 0 && src < a.n_slots && dst >= 0 && dst < a.n_slots)) {
        st |= SPEC_ST_BAD_SLOT;
        continue;
      }
      if (src == dst || !active) continue;
      const uint4 v = *reinterpret_cast<const uint4*>(base + src * a.row_bytes + lane * 16);
      *reinterpret_cast<uint4*>(base + dst * a.row_bytes + lane * 16) = v;
    }
  }
  if (reporter && a.status) a.status[b] = st;
}

// ---------------------------------------------------------------------------------------------------
// Tree build: one workgroup of 1024 threads per request, everything in LDS.
//
// Order. Candidate a ranks before candidate b when its score is higher, or equal with a lower id. Scores are
// non-negative floats, whose bit patterns order like unsigned integers, so the 64-bit key
// (score bits << 32) | ~id orders candidates exactly and is unique: a ranks before b iff key(a) > key(b), and
// a candidate's rank is the number of larger keys.
//
// Steps. Each step's keys are ranked among themselves by lane groups that count larger keys, and stored in
// rank order, so every step leaves a descending list whose head is the frontier. The lane group that ranks a
// frontier candidate also writes its k children's keys (score = its score times the child's probability)
// into the other of two key buffers, one child per lane, so the next step's keys are ready after one
// barrier. A step costs a few dependent LDS round trips: the lanes are spent on making each one short.
//
// Final selection: each candidate's rank among all of them is the sum over the step lists of how many keys
// of each are larger, by binary search in each (a candidate's own list gives its rank within the step).
// ---------------------------------------------------------------------------------------------------
constexpr int kTreeThreads = 1024;
constexpr int kTreeWaves = kTreeThreads / kWave;
constexpr int kTreeLdsMax = 64 * 1024 - 256;   // dynamic LDS (the static arrays take the rest)
constexpr int kRankPer = 4;                    // keys per thread at most (4096 candidates over 1024 threads)
constexpr int kMergeLists = 8;                 // step lists searched in lockstep in the final rank
constexpr int kMaxGroup = 16;                  // lanes sharing one key in the per-step rank

__device__ __forceinline__ float sanitize_q(float q, bool& bad) {
  if (!(q == q)) {
    bad = true;
    return 0.f;
  }
  if (q < 0.f) bad = true;
  if (q > 1.f) {
    bad = true;
    return 1.f;
  }
  return q > 0.f ? q : 0.f;
}

__device__ __forceinline__ uint64_t cand_key(float score, int id) {
  return (uint64_t(__float_as_uint(score)) << 32) | uint64_t(~uint32_t(id));
}
__device__ __forceinline__ int key_id(uint64_t key) { return int(~uint32_t(key)); }
__device__ __forceinline__ float key_score(uint64_t key) { return __uint_as_float(uint32_t(key >> 32)); }

// Sum over aligned groups of r lanes (r = 1, 2, 4, 8 or 16; every lane active): a butterfly through DPP quad
// permutes [1,0,3,2] and [2,3,0,1], then the half-row and row mirrors, each pairing a lane with one in the
// other half of its group.
__device__ __forceinline__ int group_sum(int v, int r) {
  if (r >= 2) v += __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
  if (r >= 4) v += __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
  if (r >= 8) v += __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);
  if (r >= 16) v += __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false);
  return v;
}

// LDS layout of one request (byte offsets). The 8-byte arrays come first. Optional parts, taken when they fit:
// the ancestor masks (trees of at most 64 nodes); two zero-padded key buffers of `pad` keys (without them
// each step's keys sit in the step's own list, bounds are checked, and a barrier separates reading them from
// the sorted writes); the staged probabilities.
struct TreeLayout {
  int sorted, ukeys, pad, anc, par, npar, depth, fc, q, bytes;
  bool sep, anc_masks, q_cached;
};

__host__ __device__ inline TreeLayout tree_layout(int k, int S, int N) {
  TreeLayout L{};
  const int kk = k * k;
  const int n_cand = k + (S - 1) * kk;
  L.pad = (kk + 2 * kMaxGroup - 1) / (2 * kMaxGroup) * (2 * kMaxGroup);
  L.anc_masks = N <= 64;
  const int fixed = ((8 * n_cand + 15) & ~15) + (L.anc_masks ? 8 * N : 0) + 4 * n_cand + 12 * N;
  L.sep = fixed + 16 * L.pad <= kTreeLdsMax;
  int at = 0;
  L.sorted = at;
  at += 8 * n_cand;                 // later reused as the int32 node index of every candidate
  at = (at + 15) & ~15;
  L.ukeys = at;
  if (L.sep) at += 16 * L.pad;
  L.anc = at;
  if (L.anc_masks) at += 8 * N;
  L.par = at;
  at += 4 * n_cand;
  L.npar = at;
  at += 4 * N;
  L.depth = at;
  at += 4 * N;
  L.fc = at;
  at += 4 * N;
  L.q_cached = at + 4 * S * kk <= kTreeLdsMax;
  L.q = at;
  if (L.q_cached) at += 4 * S * kk;
  L.bytes = at;
  return L;
}

struct TreeParams {
  spec_tree_build_args a;
};

template <bool QC>   // QC: the draft probabilities are staged in LDS
__global__ __launch_bounds__(kTreeThreads) void k_tree_build(TreeParams tp) {
  extern __shared__ __align__(16) char smem[];
  const spec_tree_build_args& a = tp.a;
  const int k = a.topk, S = a.n_steps, N = a.n_nodes;
  const int kk = k * k;
  const int n_cand = k + (S - 1) * kk;
  const TreeLayout L = tree_layout(k, S, N);
  uint64_t* s_sorted = reinterpret_cast<uint64_t*>(smem + L.sorted);  // per step: keys in rank order
  int32_t* s_node = reinterpret_cast<int32_t*>(smem + L.sorted);      // after the selection: node or 0
  uint64_t* s_u = reinterpret_cast<uint64_t*>(smem + L.ukeys);        // [2][pad] unsorted keys (sep)
  uint64_t* s_anc = reinterpret_cast<uint64_t*>(smem + L.anc);        // [N] ancestor-or-self bits
  int32_t* s_par = reinterpret_cast<int32_t*>(smem + L.par);          // [n_cand] parent candidate (-1: root)
  int32_t* s_npar = reinterpret_cast<int32_t*>(smem + L.npar);        // [N] parent node of each node
  int32_t* s_depth = reinterpret_cast<int32_t*>(smem + L.depth);      // [N]
  int32_t* s_fc = reinterpret_cast<int32_t*>(smem + L.fc);            // [N] first child
  float* s_q = reinterpret_cast<float*>(smem + L.q);                  // [S * kk] sanitized probabilities
  __shared__ uint32_t s_bad;
  __shared__ int32_t s_red[kTreeWaves];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t in0 = int64_t(b) * S * kk;
  if (tid == 0) s_bad = 0u;
  for (int i = tid; i < N; i += kTreeThreads) s_fc[i] = -1;
  // Every step's probabilities in one round of coalesced loads (the steps depend on each other; reading them
  // step by step would cost a memory round trip per step). Step 0 uses frontier slot 0 only.
  bool bad = false;
  if (QC) {
    for (int i = tid; i < S * kk; i += kTreeThreads) {
      const bool used = i >= kk || i < k;
      const float q = a.draft_probs[in0 + i];
      s_q[i] = used ? sanitize_q(q, bad) : 0.f;
    }
  }
  // Step 0's keys (the root's children, score = q) and the zero padding of the key buffers (a zero key ranks
  // after every real one).
  if (L.sep) {
    for (int i = tid; i < 2 * L.pad; i += kTreeThreads)
      s_u[i] = i < k ? cand_key(sanitize_q(a.draft_probs[in0 + i], bad), i) : 0ull;
  } else {
    for (int i = tid; i < k; i += kTreeThreads) s_sorted[i] = cand_key(sanitize_q(a.draft_probs[in0 + i], bad), i);
  }
  for (int i = tid; i < k; i += kTreeThreads) s_par[i] = -1;

  for (int s = 0; s < S; ++s) {
    const int cnt = s == 0 ? k : kk;
    const int base = s == 0 ? 0 : k + (s - 1) * kk;
    const int nbase = k + s * kk;   // first candidate id of step s + 1
    uint64_t* u = L.sep ? s_u + (s & 1) * L.pad : s_sorted + base;
    uint64_t* un = L.sep ? s_u + ((s + 1) & 1) * L.pad : s_sorted + nbase;
    // r lanes per key (up to 16, as many as the block holds), each counting a strided share; kRankPer keys
    // per thread at most.
    int r = 1;
    while (r < kMaxGroup && cnt * (2 * r) <= kTreeThreads) r *= 2;
    const int groups = kTreeThreads / r, sub = tid & (r - 1);
    __syncthreads();   // this step's keys are in place
    int rank[kRankPer];
    uint64_t key[kRankPer];
#pragma unroll
    for (int v = 0; v < kRankPer; ++v) {
      rank[v] = -1;
      key[v] = 0;
      if (v * groups >= cnt) continue;   // uniform
      const int i = v * groups + tid / r;
      const bool live = i < cnt;
      const uint64_t x = u[live ? i : 0];
      int n = 0;
      if (L.sep) {
        // Padded to whole pairs per lane group: every lane makes the same number of 16-byte reads.
        const int npairs = (cnt + 2 * r - 1) / (2 * r) * r;
        const ulonglong2* u2 = reinterpret_cast<const ulonglong2*>(u);
#pragma unroll 4
        for (int pp = sub; pp < npairs; pp += r) {
          const ulonglong2 y = u2[pp];
          n += (y.x > x ? 1 : 0) + (y.y > x ? 1 : 0);
        }
      } else {
        for (int j = sub; j < cnt; j += r) n += u[j] > x ? 1 : 0;
      }
      n = group_sum(n, r);   // every lane of the group holds the rank
      if (live) {
        rank[v] = n;
        key[v] = x;
      }
    }
    if (!L.sep) __syncthreads();   // every unsorted key has been read before the list overwrites them
#pragma unroll
    for (int v = 0; v < kRankPer; ++v) {
      if (rank[v] < 0) continue;
      if (sub == 0) s_sorted[base + rank[v]] = key[v];
      if (rank[v] < k && s + 1 < S) {
        // Frontier slot rank[v]: its children are step s + 1's candidates rank[v] * k + c, shared out
        // over the group's lanes.
        const float ps = key_score(key[v]);
        const int pid = key_id(key[v]);
        const int j0 = rank[v] * k;
        for (int c = sub; c < k; c += r) {
          const int qi = (s + 1) * kk + j0 + c;
          const float q = QC ? s_q[qi] : sanitize_q(a.draft_probs[in0 + qi], bad);
          un[j0 + c] = cand_key(ps * q, nbase + j0 + c);
          s_par[nbase + j0 + c] = pid;
        }
      }
    }
  }
  __syncthreads();
  if (bad) atomicOr(&s_bad, SPEC_ST_BAD_CONF);

  // The tree: the top N - 1 of all candidates. Rank among all = sum over the step lists of the larger keys,
  // found in each by a binary search whose halving sequence depends only on the list's length (the same for
  // every lane), so its probes need no bounds checks. A search keeps (start of its range - 8) as an LDS byte
  // address, so a probe is one add, one load, one compare and one select; kMergeLists lists are searched in
  // lockstep so that their loads overlap.
  const auto at = [&](int addr) -> uint64_t { return *reinterpret_cast<const uint64_t*>(smem + addr); };
  bool chosen_v[kRankPer];
  int id_v[kRankPer];
#pragma unroll
  for (int v = 0; v < kRankPer; ++v) {
    chosen_v[v] = false;
    id_v[v] = -1;
    const int p = v * kTreeThreads + tid;
    if (p >= n_cand) continue;
    const uint64_t x = s_sorted[p];
    int total;
    {   // step 0's list (k keys)
      int lm = L.sorted - 8;
      for (int len = k; len > 1; len -= len >> 1) {
        const int pa = lm + (len >> 1) * 8;
        lm = at(pa) > x ? pa : lm;
      }
      total = ((lm + 8 - L.sorted) >> 3) + (at(lm + 8) > x ? 1 : 0);
    }
    for (int s0 = 1; s0 < S && total < N - 1; s0 += kMergeLists) {
      const int nl = min(kMergeLists, S - s0);
      const int start0 = L.sorted + 8 * (k + (s0 - 1) * kk);
      int lm[kMergeLists];
#pragma unroll
      for (int w = 0; w < kMergeLists; ++w) lm[w] = start0 + (w < nl ? w * 8 * kk : 0) - 8;
      for (int len = kk; len > 1; len -= len >> 1) {
        const int hb = (len >> 1) * 8;
        uint64_t y[kMergeLists];
#pragma unroll
        for (int w = 0; w < kMergeLists; ++w) y[w] = at(lm[w] + hb);
#pragma unroll
        for (int w = 0; w < kMergeLists; ++w) lm[w] = y[w] > x ? lm[w] + hb : lm[w];
      }
      uint64_t y[kMergeLists];
#pragma unroll
      for (int w = 0; w < kMergeLists; ++w) y[w] = at(lm[w] + 8);
#pragma unroll
      for (int w = 0; w < kMergeLists; ++w)
        if (w < nl) total += ((lm[w] + 8 - start0 - w * 8 * kk) >> 3) + (y[w] > x ? 1 : 0);
    }
    chosen_v[v] = total < N - 1;
    id_v[v] = key_id(x);
  }
  __syncthreads();   // the lists are read; their memory now holds the node index of every candidate
#pragma unroll
  for (int v = 0; v < kRankPer; ++v)
    if (id_v[v] >= 0) s_node[id_v[v]] = chosen_v[v] ? 1 : 0;
  __syncthreads();

  // Nodes are numbered in candidate order (block scan of the chosen flags), so a parent precedes its children.
  // A thread's count is at most 4: the wave prefix takes three bit-plane ballots.
  const int per = (n_cand + kTreeThreads - 1) / kTreeThreads;
  const int c_lo = min(n_cand, tid * per), c_hi = min(n_cand, c_lo + per);
  int chosen = 0;
  for (int i = c_lo; i < c_hi; ++i) chosen += s_node[i];
  const int lane = tid & (kWave - 1), w = tid / kWave;
  int excl = 0, wave_total = 0;
#pragma unroll
  for (int bit = 0; bit < 3; ++bit) {
    const uint64_t m = __ballot((chosen >> bit) & 1);
    excl += int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u))) << bit;
    wave_total += __popcll(m) << bit;
  }
  if (lane == 0) s_red[w] = wave_total;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < w; ++i) before += s_red[i];
  int node = 1 + before + excl;
  for (int i = c_lo; i < c_hi; ++i)
    if (s_node[i]) s_node[i] = node++;
  __syncthreads();

  // Node fields. A candidate's depth is its step + 1.
  const int64_t out0 = int64_t(b) * N;
  const int32_t seq = a.seq_lens[b];
  for (int i = tid; i < n_cand; i += kTreeThreads) {
    const int nd = s_node[i];
    if (!nd) continue;
    const int step = i < k ? 0 : 1 + (i - k) / kk;
    const int pc = s_par[i];
    const int pn = pc < 0 ? 0 : s_node[pc];   // chosen: a child never outranks its parent
    s_npar[nd] = pn;
    s_depth[nd] = step + 1;
    a.tokens[out0 + nd] = a.draft_tokens[in0 + (step == 0 ? i : int64_t(step) * kk + (i - k - (step - 1) * kk))];
    a.parents[out0 + nd] = pn;
    a.positions[out0 + nd] = seq + step + 1;
    if (a.cand_index) a.cand_index[out0 + nd] = i;
  }
  if (tid == 0) {
    s_npar[0] = -1;
    s_depth[0] = 0;
    a.tokens[out0] = a.anchors[b];
    a.parents[out0] = -1;
    a.positions[out0] = seq;
    if (a.cand_index) a.cand_index[out0] = -1;
  }
  __syncthreads();
  // A node's children come from one frontier slot of one step, so their candidate ids, and hence their node
  // numbers, are consecutive: a node is its parent's first child when the node before it has another parent,
  // and its next sibling is the node after it when that one has the same parent.
  for (int i = 1 + tid; i < N; i += kTreeThreads)
    if (s_npar[i - 1] != s_npar[i]) s_fc[s_npar[i]] = i;
  if (a.next_sibling) {
    for (int i = tid; i < N; i += kTreeThreads)
      a.next_sibling[out0 + i] = (i > 0 && i + 1 < N && s_npar[i + 1] == s_npar[i]) ? i + 1 : -1;
  }
  // Visibility: j is i or one of its ancestors. Up to 64 nodes, each node's ancestor-or-self set is a bit mask
  // (one walk to the root per node); above, each entry walks up from i to j's depth.
  if (a.mask && L.anc_masks) {
    for (int i = tid; i < N; i += kTreeThreads) {
      uint64_t m = 0;
      for (int x = i; x >= 0; x = s_npar[x]) m |= 1ull << x;
      s_anc[i] = m;
    }
  }
  __syncthreads();
  if (a.first_child)
    for (int i = tid; i < N; i += kTreeThreads) a.first_child[out0 + i] = s_fc[i];
  if (a.mask) {
    uint8_t* m = a.mask + out0 * N;
    if (L.anc_masks) {
      for (int idx = tid; idx < N * N; idx += kTreeThreads)
        m[idx] = uint8_t((s_anc[idx / N] >> (idx % N)) & 1u);
    } else {
      for (int64_t idx = tid; idx < int64_t(N) * N; idx += kTreeThreads) {
        const int i = int(idx / N), j = int(idx % N);
        int x = i;
        while (s_depth[x] > s_depth[j]) x = s_npar[x];
        m[idx] = x == j ? 1 : 0;
      }
    }
  }
  if (tid == 0) a.status[b] = s_bad;
}

}  // namespace

hipError_t launch_kv_move(const spec_kv_move_args& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int lanes = (a.row_bytes + 15) / 16;
  const int chunks = (lanes + kMoveLanes - 1) / kMoveLanes;
  const int64_t blocks = int64_t(a.batch) * a.n_buffers * chunks;
  if (blocks <= 0) return hipSuccess;
  // a row shorter than one chunk runs with fewer threads (whole waves)
  const int threads = chunks > 1 ? kMoveLanes : (lanes + kWave - 1) / kWave * kWave;
  return launch_kernel(k_kv_move, dim3(unsigned(blocks)), dim3(threads), 0, stream, ev0, ev1, MoveParams{a, chunks});
}

// LDS of k_tree_build (the optional parts are reported through q_cached: the staged probabilities).
size_t tree_build_smem(int k, int S, int N, bool* q_cached) {
  const TreeLayout L = tree_layout(k, S, N);
  if (q_cached) *q_cached = L.q_cached;
  return size_t(L.bytes);
}

hipError_t launch_tree_build(const spec_tree_build_args& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.batch <= 0) return hipSuccess;
  bool qc = false;
  const size_t smem = tree_build_smem(a.topk, a.n_steps, a.n_nodes, &qc);
  return launch_kernel(qc ? k_tree_build<true> : k_tree_build<false>, dim3(unsigned(a.batch)), dim3(kTreeThreads),
                       smem, stream, ev0, ev1, TreeParams{a});
}

}  // namespace sv
