// Fused KV commit: the commit lists of a verify round produced inside the verify call's second kernel.
//   commit_len_b = accept_len_b + 1 ([EAGLE→DFlash2] §5.6.6 commit_lens = correct_len + 1; §8.1: the committed
//   KV is the old anchor plus the accepted drafts); src = the KV slot of each accepted row in path order,
//   dst = seq_lens[b] + k ([SpecDec] "实现：共享的骨架", move_accept_tokens_to_target_kvcache); the other
//   verify rows of the request are listed for eviction, in row order (§8.2).
// The results equal what k_commit computes from the verify outputs. They are simpler to reach here: the
// accepted entries of a chain request are its first r + 1 rows, those of a tree request its accepted path
// (node indices increasing from the root), so no entry is ever out of range or repeated.
//
// Hand-off: every request's accept scan publishes r (trees: the path) with agent-scope stores, waits for them
// to complete and counts itself on one counter (reset by the logits stream of the same call); the workgroup
// whose count is the last reads the published values with agent-scope loads and writes every commit output.
#pragma once

#include "sv_scan.h"

namespace sv {

constexpr int kFcTile = 256;   // requests per tile of the fused commit (one thread each)

__device__ __forceinline__ void store_agent32(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t load_agent32(int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publishes request b's accepted length r (-1: the request's offsets failed) and, for a tree, its path
// (LDS, r + 1 node indices), then counts the request. Every thread of the workgroup calls it; it returns true
// in the one workgroup of the call that counted last.
template <int NT>
__device__ bool commit_arrive(const VerifyParams& p, int b, int r, const int32_t* path) {
  __shared__ int s_last_commit;
  const int tid = threadIdx.x;
  if (tid == 0) store_agent32(p.pub_r + b, r);
  if (p.tree && path)
    for (int k = tid; k <= r; k += NT) store_agent32(p.pub_path + size_t(b) * p.L + k, path[k]);
  complete_memory_ops();   // the published words are stored before the request is counted
  __syncthreads();
  if (tid == 0) s_last_commit = uint32_t(atomicAdd(p.ccnt, 1ull)) + 1u == uint32_t(p.B);
  __syncthreads();
  return s_last_commit != 0;
}

constexpr int kFcWindow = 1024;     // verify rows whose slots a tile loads up front (with the request words):
                                    // the default, sized for the LDS of kernels whose every workgroup holds it

// The request of the tile that holds flat row i, given the inclusive row prefix `incl` over its nb requests.
__device__ __forceinline__ int fc_owner(const int32_t* incl, int nb, int i) {
  int lo = 0, hi = nb - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (incl[mid] > i) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// The commit lists of the whole batch, written by one workgroup of NT threads (NT a multiple of kFcTile).
// Requests go in tiles (a thread each). A tile costs one round of loads: its requests' words (offsets, seq_len,
// published accept length) and the slots of the WIN verify rows that follow the previous tile's rows (for
// trees also the published path entries, laid out like the rows), all issued before any is used and parked
// in LDS. When the tile's requests are packed (each request's rows follow the previous one's, as in every valid
// batch) those rows are exactly the tile's; otherwise (inconsistent offsets) each row is gathered on its own.
template <int NT, bool TREE, int WIN = kFcWindow>
__device__ void fused_commit(const VerifyParams& p) {
  constexpr int TW = kFcTile / kWave;   // waves that hold one request each in the tile's scan
  constexpr int K = WIN / NT;           // window rows loaded per thread
  __shared__ int32_t f_off0[kFcTile], f_r[kFcTile], f_seq[kFcTile], f_co[kFcTile], f_eo[kFcTile];
  __shared__ int32_t f_rows[kFcTile];    // inclusive prefix of the tile's rows
  __shared__ uint64_t f_wsum[TW];
  __shared__ int f_unpacked;
  __shared__ int64_t f_vs[WIN];    // verify_slots of the window rows
  __shared__ int32_t f_node[TREE ? WIN : 1];        // trees: published path entries of the window rows
  __shared__ uint32_t f_bits[TREE ? WIN / 32 : 1];  // trees: the tile's accepted nodes, by row
  __shared__ uint8_t f_acc[TREE ? NT : 1];          // trees of at most 64 nodes: per wave, the accepted flags
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int B = p.B;
  const int64_t T = TREE ? int64_t(B) * p.L : p.total_rows;
  const int tile_n = min(kFcTile, max(1, WIN / p.L));   // a packed tile's rows fit the window
  int64_t carry_c = 0, carry_e = 0, row0 = 0;
  for (int t0 = 0; t0 < B; t0 += tile_n) {
    const int nb = min(tile_n, B - t0);
    // ---- one round of loads ----
    const int b = t0 + tid;
    const bool has = tid < nb;
    int32_t o_lo = 0, o_hi = 0, seq = 0, r = 0;
    if (has) {
      if (!TREE) {
        o_lo = p.offsets[b];
        o_hi = p.offsets[b + 1];
      }
      seq = p.seq_lens[b];
      r = load_agent32(p.pub_r + b);
    }
    {
      int64_t vs[K];
      int32_t node[K];
#pragma unroll
      for (int j = 0; j < K; ++j) {
        const int64_t row = row0 + tid + j * NT;
        vs[j] = 0;
        node[j] = -1;
        if (row < T) {
          vs[j] = p.verify_slots[row];
          if (TREE) node[j] = load_agent32(p.pub_path + row);
        }
      }
#pragma unroll
      for (int j = 0; j < K; ++j) {
        f_vs[tid + j * NT] = vs[j];
        if (TREE) f_node[tid + j * NT] = node[j];
      }
    }
    // ---- per request: offsets check, commit / evict counts and their exclusive scan ----
    // (every thread takes part in the wave scans and barriers; threads past the tile hold no request)
    int64_t off0 = 0, len = 0;
    bool ok = false;
    if (has) {
      if (TREE) {
        off0 = int64_t(b) * p.L;
        len = p.L;
        ok = true;
      } else {
        off0 = o_lo;
        len = int64_t(o_hi) - o_lo;
        ok = chain_offsets_ok(p, b, o_lo, o_hi);
      }
      if (ok) r = r < 0 ? 0 : (r >= len ? int32_t(len) - 1 : r);   // never out of range from the scans
      else len = 0;
    }
    const uint64_t c = ok ? uint64_t(r) + 1 : 0;
    const uint64_t e = ok ? uint64_t(len) - c : 0;
    const uint64_t mine = (c << 32) | e;   // both sums stay below 2^31: no carry between the halves
    const uint64_t inc = wave_inclusive_sum_dpp(mine);
    if (lane == kWave - 1 && wv < TW) f_wsum[wv] = inc;
    if (tid == 0) f_unpacked = 0;
    if (TREE)
      for (int w = tid; w < WIN / 32; w += NT) f_bits[w] = 0u;
    __syncthreads();
    uint64_t base = 0;
    for (int w = 0; w < min(wv, TW); ++w) base += f_wsum[w];
    const uint64_t ex = base + inc - mine;
    if (has) {
      const int64_t co = carry_c + int64_t(ex >> 32);
      const int64_t eo = carry_e + int64_t(uint32_t(ex));
      p.commit_offsets[b] = int32_t(co);
      p.new_seq_lens[b] = seq + int32_t(c);
      if (p.evict_offsets) p.evict_offsets[b] = int32_t(eo);
      p.cstatus[b] = ok ? 0u : SPEC_ST_BAD_OFFSETS;
      const int32_t excl_rows = int32_t((ex >> 32) + uint32_t(ex));
      f_off0[tid] = int32_t(off0);
      f_r[tid] = r;
      f_seq[tid] = seq;
      f_co[tid] = int32_t(co);
      f_eo[tid] = int32_t(eo);
      f_rows[tid] = excl_rows + int32_t(len);
      if (len > 0 && off0 != row0 + excl_rows) f_unpacked = 1;   // rows not where the window has them
    }
    __syncthreads();
    uint64_t tile = 0;
    for (int w = 0; w < TW; ++w) tile += f_wsum[w];
    const int n_rows = int((tile >> 32) + uint32_t(tile));
    const bool packed = f_unpacked == 0;
    const bool tree_lanes = TREE && p.L <= kWave;   // trees of at most 64 nodes: a lane per node, below
    if (TREE && !tree_lanes) {
      // the accepted path entries of the tile's requests as bits, by the tile row of the node they name
      for (int i = tid; i < n_rows; i += NT) {
        const int q = i / p.L;
        const int32_t nd = f_node[i];
        if (i - q * p.L <= f_r[q] && nd >= 0 && nd < p.L) {
          const int nr = q * p.L + nd;
          atomicOr(&f_bits[nr >> 5], 1u << (nr & 31));
        }
      }
      __syncthreads();
    }
    // ---- the tile's rows: committed (src, dst) or evicted ----
    if (!packed) {   // inconsistent offsets (rare): each row's slot gathered on its own
      for (int i = tid; i < n_rows; i += NT) {
        const int q = fc_owner(f_rows, nb, i);
        f_vs[i] = p.verify_slots[int64_t(f_off0[q]) + i - (q ? f_rows[q - 1] : 0)];
      }
      __syncthreads();
    }
    if (tree_lanes) {
      // A request per segment of Lp lanes (Lp the smallest power of two >= L), a lane per node: the lanes
      // holding path entries flag the nodes they name in the wave's slice of f_acc (distinct nodes, so no
      // atomics; one wave's LDS operations complete in order), each lane reads its own node's flag, and a
      // ballot of those flags gives each accepted node its place on the path (the accepted nodes below it)
      // and each other node its place among the evicted ones. No bitmap over the tile, no division.
      constexpr int NW = NT / kWave;
      const int Lp = 1 << (32 - __clz(p.L - 1));
      const int G = kWave / Lp;
      const int seg = lane / Lp;
      const int k = lane - seg * Lp;
      const uint64_t seg_below = lanes_below(lane) & ~lanes_below(seg * Lp);   // this segment's lanes below
      uint8_t* acc = f_acc + wv * kWave;
      for (int q0 = wv * G; q0 < nb; q0 += NW * G) {   // uniform in the wave
        const int q = q0 + seg;
        const bool on = q < nb && k < p.L;
        acc[lane] = 0;
        if (on && k <= f_r[q]) {
          const int32_t nd = f_node[q * p.L + k];
          if (nd >= 0 && nd < p.L) acc[seg * Lp + nd] = 1;
        }
        __builtin_amdgcn_wave_barrier();
        const bool hit = on && acc[lane] != 0;
        const uint64_t hits = __ballot(hit);
        __builtin_amdgcn_wave_barrier();   // every lane has read its flag before the next request clears them
        if (on) {
          const int below = __popcll(hits & seg_below);
          const int64_t v = f_vs[q * p.L + k];
          if (hit) {
            p.src_slots[int64_t(f_co[q]) + below] = v;
            p.dst_pos[int64_t(f_co[q]) + below] = f_seq[q] + below;
          } else if (p.evict_slots) {
            p.evict_slots[int64_t(f_eo[q]) + (k - below)] = v;
          }
        }
      }
    }
    const bool chain_lanes = !TREE && packed && p.L <= kWave;   // packed chains of at most 64 rows
    if (chain_lanes) {
      // A request per segment of Lp lanes, a lane per row: row k of request q sits at the window row after
      // the requests before it, and it is committed at place k (k <= r) or evicted at place k - r - 1.
      constexpr int NW = NT / kWave;
      const int Lp = 1 << (32 - __clz(p.L - 1));
      const int G = kWave / Lp;
      const int seg = lane / Lp;
      const int k = lane - seg * Lp;
      for (int q0 = wv * G; q0 < nb; q0 += NW * G) {
        const int q = q0 + seg;
        if (q >= nb) continue;
        const int r0 = q ? f_rows[q - 1] : 0;
        if (k >= f_rows[q] - r0) continue;
        const int64_t v = f_vs[r0 + k];
        const int rq = f_r[q];
        if (k <= rq) {
          p.src_slots[int64_t(f_co[q]) + k] = v;
          p.dst_pos[int64_t(f_co[q]) + k] = f_seq[q] + k;
        } else if (p.evict_slots) {
          p.evict_slots[int64_t(f_eo[q]) + (k - rq - 1)] = v;
        }
      }
    }
    for (int i = tid; i < (tree_lanes || chain_lanes ? 0 : n_rows); i += NT) {
      const int q = TREE ? i / p.L : fc_owner(f_rows, nb, i);
      const int r0 = TREE ? q * p.L : (q ? f_rows[q - 1] : 0);   // the request's first row in the tile
      const int k = i - r0;
      const int64_t v = f_vs[i];
      int pos;   // place on the accepted path, or -1 - (place among the evicted rows)
      if (TREE) {
        // accepted nodes of request q below this one: bits [r0, i) of the tile's bitmap
        int below = 0;
        for (int w = r0 >> 5; w <= (i >> 5); ++w) {
          uint32_t m = f_bits[w];
          if (w == (r0 >> 5)) m &= ~((1u << (r0 & 31)) - 1u);
          if (w == (i >> 5)) m &= (1u << (i & 31)) - 1u;
          below += __popc(m);
        }
        pos = (f_bits[i >> 5] >> (i & 31)) & 1u ? below : -1 - (k - below);
      } else {
        pos = k <= f_r[q] ? k : -1 - (k - f_r[q] - 1);
      }
      if (pos >= 0) {
        p.src_slots[int64_t(f_co[q]) + pos] = v;
        p.dst_pos[int64_t(f_co[q]) + pos] = f_seq[q] + pos;
      } else if (p.evict_slots) {
        p.evict_slots[int64_t(f_eo[q]) + (-1 - pos)] = v;
      }
    }
    carry_c += int64_t(tile >> 32);
    carry_e += int64_t(uint32_t(tile));
    row0 += n_rows;
    __syncthreads();   // the tile's LDS is rewritten by the next tile
  }
  if (tid == 0) {
    p.commit_offsets[B] = int32_t(carry_c);
    if (p.evict_offsets) p.evict_offsets[B] = int32_t(carry_e);
  }
}

}  // namespace sv
