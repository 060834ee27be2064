// k_commit: KV commit compaction of one verify round, in one workgroup.
//   commit_len_b = accept_len_b + 1: the KV of the old anchor plus the accepted drafts
//   ([EAGLE→DFlash2] §5.6.6 commit_lens = correct_len + 1; §8.1: output E F X, committed KV D E F);
//   the accepted rows' slots move to contiguous positions after seq_lens ([SpecDec] "实现：共享的骨架",
//   move_accept_tokens_to_target_kvcache); the other verify rows are listed for eviction (§8.2: rejected
//   KV must stop being visible, when it is freed is the caller's choice).
// Requests are handled in tiles of up to 1024 requests and 8192 verify rows: thread per request for the
// scan, thread per verify row for the gathers. Each tile's window of accept_index and verify_slots entries
// (the rows that follow the previous tile's) is loaded into LDS together with the request data, so that a
// tile costs one round trip to memory; rows outside the window (only with inconsistent offsets) are read
// from memory directly. Any batch size works in one launch.
#include "sv_device.h"

namespace sv {

namespace {

constexpr int kCommitThreads = 1024;
constexpr int kTileRows = 8192;                       // verify rows staged in LDS at once
constexpr int kRowsPerThread = kTileRows / kCommitThreads;

struct CommitTile {
  int64_t w0;       // first global row of the staged window
  int n_st;         // rows staged
  const int32_t* s_ai;
  const int64_t* s_vs;
  const int32_t* accept_index;
  const int64_t* verify_slots;
  __device__ int32_t ai(int64_t row) const {
    const int64_t i = row - w0;
    return i >= 0 && i < n_st ? s_ai[i] : accept_index[row];
  }
  __device__ int64_t vs(int64_t row) const {
    const int64_t i = row - w0;
    return i >= 0 && i < n_st ? s_vs[i] : verify_slots[row];
  }
};

__global__ __launch_bounds__(kCommitThreads) void k_commit(spec_commit_args a) {
  // Per request of the tile: inclusive prefix of (rows << 32 | committed rows), its rows, accept length,
  // first row, seq_len and status.
  __shared__ uint64_t red[kCommitThreads / kWave];
  __shared__ uint64_t t_incl[kCommitThreads];
  __shared__ int32_t t_len[kCommitThreads];
  __shared__ int32_t t_r[kCommitThreads];
  __shared__ int32_t t_o0[kCommitThreads];
  __shared__ int32_t t_seq[kCommitThreads];
  __shared__ uint32_t t_st[kCommitThreads];
  __shared__ uint8_t t_id[kCommitThreads];   // the request's accepted entries are its first r + 1 rows
  __shared__ uint8_t t_win[kCommitThreads];  // all of the request's rows are staged
  __shared__ int32_t t_x[kCommitThreads];    // entries naming no new row of the request (extra)
  __shared__ int32_t t_xex[kCommitThreads];  // exclusive prefix of extra over the tile's requests
  __shared__ uint32_t s_idw[kTileRows / 32];  // bit i: staged row i's accept_index entry is the row itself
  __shared__ uint32_t s_accb[kTileRows / 32]; // bit i: staged row i is named by an entry of its request
  __shared__ int s_fit[kCommitThreads / kWave];
  __shared__ int s_xred[kCommitThreads / kWave];
  __shared__ int s_xtot;
  __shared__ int32_t s_ai[kTileRows];
  __shared__ int64_t s_vs[kTileRows];

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = tid / kWave;
  const int B = a.batch;
  const int64_t T = a.total_rows;
  const int L = a.max_verify_len;
  int64_t carry_c = 0, carry_e = 0, w0 = 0;
  for (int t0 = 0; t0 < B;) {
    const int n_st = int(min(int64_t(kTileRows), max(int64_t(0), T - w0)));
    // ---- one round of loads: the request and the window of rows after the previous tile's ----
    int32_t ai_r[kRowsPerThread];
    int64_t vs_r[kRowsPerThread];
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
      const int i = tid + j * kCommitThreads;
      ai_r[j] = -1;
      if (i < n_st) {
        ai_r[j] = a.accept_index[w0 + i];
        vs_r[j] = a.verify_slots[w0 + i];
      }
    }
    if (tid < kTileRows / 32) s_accb[tid] = 0u;
    const int b = t0 + tid;
    // the request's words, loaded with the rows (its accept length too, used only if its offsets pass)
    const int bc = min(b, B - 1);
    const int32_t off0_ld = a.row_offsets[bc];
    const int32_t off1_ld = a.row_offsets[bc + 1];
    const int32_t seq_ld = a.seq_lens[bc];
    const int32_t r_ld = a.accept_len[bc];
    int32_t off0 = 0, len = 0, r = 0, seq = 0;
    uint32_t st = 0;
    if (b < B) {
      off0 = off0_ld;
      const int32_t off1 = off1_ld;
      len = off1 - off0;
      bool ok = off0 >= b && off1 > off0 && off1 <= T - B + b + 1 && len <= L;
      if (b == 0 && off0 != 0) ok = false;
      if (b == B - 1 && off1 != T) ok = false;
      seq = seq_ld;
      if (!ok) {
        st = SPEC_ST_BAD_OFFSETS;
        len = 0;
      } else {
        r = r_ld;
        if (r < 0 || r >= len) {
          st |= SPEC_ST_BAD_ACCEPT;
          r = r < 0 ? 0 : len - 1;
        }
      }
    }
    const uint64_t mine = (uint64_t(uint32_t(len)) << 32) | uint32_t(len > 0 ? r + 1 : 0);
    const uint64_t inc = wave_inclusive_sum_dpp(mine);
    if (lane == kWave - 1) red[wv] = inc;
    t_len[tid] = len;
    t_r[tid] = r;
    t_o0[tid] = off0;
    t_seq[tid] = seq;
    t_st[tid] = st;
#pragma unroll
    for (int j = 0; j < kRowsPerThread; ++j) {
      const int i = tid + j * kCommitThreads;
      if (i < n_st) {
        s_ai[i] = ai_r[j];
        s_vs[i] = vs_r[j];
      }
      // rows i .. i + 63 of this wave: which entries name their own row
      const uint64_t idm = __ballot(i < n_st && int64_t(ai_r[j]) == w0 + i);
      if (lane == 0) {
        s_idw[i / 32] = uint32_t(idm);
        s_idw[i / 32 + 1] = uint32_t(idm >> 32);
      }
    }
    __syncthreads();
    uint64_t base = 0;
    for (int i = 0; i < wv; ++i) base += red[i];
    const uint64_t incl = base + inc;
    t_incl[tid] = incl;
    // ---- the request's entries: the usual form (its first r + 1 rows in order) or any other ----
    const CommitTile tw0{w0, n_st, s_ai, s_vs, a.accept_index, a.verify_slots};
    const int64_t lo_r = int64_t(off0) - w0;
    // All of the request's rows are staged AND sit at their packed place in the tile (the rows of the requests
    // before it in this tile come first). Packed places of different requests never overlap, so such requests
    // can share the bitmap s_accb. A request whose own offsets pass but overlap another's (inconsistent
    // offsets elsewhere in the batch) takes the per-request loops instead.
    const bool inwin = len > 0 && lo_r >= 0 && lo_r + len <= n_st && lo_r == int64_t(incl >> 32) - len;
    bool ident = inwin;
    if (ident) {
      // The form the verify kernels write: the bits of rows lo_r .. lo_r + r in s_idw all set. Every entry
      // is then inside the request and distinct, and the gathers need no scans.
      const int64_t hi_r = lo_r + r;
      for (int64_t wd = lo_r >> 5; wd <= (hi_r >> 5); ++wd) {
        const int a0 = wd == (lo_r >> 5) ? int(lo_r & 31) : 0;
        const int a1 = wd == (hi_r >> 5) ? int(hi_r & 31) : 31;
        const uint32_t need = (a1 == 31 ? ~0u : ((1u << (a1 + 1)) - 1u)) & ~((1u << a0) - 1u);
        ident &= (s_idw[wd] & need) == need;
      }
    }
    // Any other form: an entry outside the request's rows or naming a row twice is reported; the request
    // commits its entries in order (those outside its rows as -1) and evicts the rows no entry names.
    int distinct = len > 0 ? r + 1 : 0;   // rows of the request named by its entries
    if (len > 0 && !ident) {
      bool bad = false;
      distinct = 0;
      for (int k = 0; k <= r; ++k) {
        const int32_t ai = tw0.ai(int64_t(off0) + k);
        if (!(ai >= off0 && ai < off0 + len)) {
          bad = true;
          continue;
        }
        bool first = true;
        if (inwin) {   // ai - w0 lies in the staged rows of the request
          const uint32_t bit = 1u << ((ai - w0) & 31);
          first = !(atomicOr(&s_accb[(ai - w0) >> 5], bit) & bit);
        } else {
          for (int j = 0; j < k; ++j)
            if (tw0.ai(int64_t(off0) + j) == ai) first = false;
        }
        if (first) ++distinct;
        else bad = true;
      }
      if (bad) t_st[tid] |= SPEC_ST_BAD_ACCEPT;
    }
    t_id[tid] = ident;
    t_win[tid] = inwin;
    // The request evicts len - distinct rows; the scan above counted len - (r + 1), so the entries that name
    // no new row (extra) are summed separately.
    const int extra = (len > 0 ? r + 1 : 0) - distinct;
    t_x[tid] = extra;
    const int xinc = __ballot(extra != 0) ? wave_inclusive_sum(extra) : 0;   // usually none in the wave
    if (lane == kWave - 1) s_xred[wv] = xinc;
    // This tile: the longest prefix of the next min(1024, B - t0) requests with at most kTileRows rows
    // (never empty, since a request has at most 1024 rows). Row counts only grow, so the requests that fit
    // are a prefix: count them.
    const int avail = min(kCommitThreads, B - t0);
    const uint64_t fm = __ballot(tid < avail && (incl >> 32) <= uint64_t(kTileRows));
    if (lane == 0) s_fit[wv] = __popcll(fm);
    __syncthreads();
    int nb = 0, xbase = 0, xany = 0;
#pragma unroll
    for (int w = 0; w < kCommitThreads / kWave; ++w) {
      nb += s_fit[w];
      if (w < wv) xbase += s_xred[w];
      xany |= s_xred[w];
    }
    const int xex = xbase + xinc - extra;   // this request's exclusive prefix of extra (tid < nb)
    if (tid == nb - 1) s_xtot = xex + extra;
    const uint64_t tile_tot = t_incl[nb - 1];
    const int n_rows = int(tile_tot >> 32);
    if (tid < nb) {
      const int64_t co = carry_c + int64_t(uint32_t(incl - mine));
      const int64_t eo = carry_e + int64_t((incl - mine) >> 32) - int64_t(uint32_t(incl - mine)) + xex;
      a.commit_offsets[b] = int32_t(co);
      a.new_seq_lens[b] = seq + (len > 0 ? r + 1 : 0);
      if (a.evict_offsets) a.evict_offsets[b] = int32_t(eo);
    }
    if (xany) {   // uniform: some request of the lot has extra entries
      t_xex[tid] = xex;
      __syncthreads();
    }
    // ---- gathers, one thread per verify row of the tile ----
    const CommitTile tw{w0, n_st, s_ai, s_vs, a.accept_index, a.verify_slots};
    for (int i = tid; i < n_rows; i += kCommitThreads) {
      // owning request: the first lb whose inclusive row count exceeds i (it has rows)
      int l2 = 0, h2 = nb - 1;
      while (l2 < h2) {
        const int mid = (l2 + h2) >> 1;
        if ((t_incl[mid] >> 32) > uint64_t(i)) h2 = mid;
        else l2 = mid + 1;
      }
      const int lb = l2;
      const uint64_t inc_b = t_incl[lb];
      const int32_t len_b = t_len[lb];
      const int32_t r_b = t_r[lb];
      const int k = i - (int(inc_b >> 32) - len_b);
      const int64_t o0 = t_o0[lb];
      const int64_t row = o0 + k;   // < T: the request's offsets passed their checks
      const int64_t co_b = carry_c + int64_t(uint32_t(inc_b)) - (r_b + 1);
      const bool ident_b = t_id[lb];
      if (k <= r_b) {
        const int32_t ai = ident_b ? int32_t(row) : tw.ai(row);
        const bool in_req = ai >= o0 && ai < o0 + len_b;
        if (co_b + k < a.capacity) {   // always true unless the offsets are inconsistent
          a.src_slots[co_b + k] = in_req ? tw.vs(ai) : int64_t(-1);
          a.dst_pos[co_b + k] = t_seq[lb] + k;
        }
      }
      if (a.evict_slots) {
        // whether an entry names this row, and how many rows of the request below it are named
        bool accepted;
        int below;
        if (ident_b) {
          accepted = k <= r_b;
          below = min(k, r_b + 1);
        } else if (t_win[lb]) {
          const int64_t q = row - w0, q0 = o0 - w0;
          accepted = (s_accb[q >> 5] >> (q & 31)) & 1u;
          below = 0;
          for (int64_t wd = q0 >> 5; wd <= (q >> 5); ++wd) {   // bits q0 .. q - 1
            uint32_t m = s_accb[wd];
            if (wd == (q0 >> 5)) m &= ~((1u << (q0 & 31)) - 1u);
            if (wd == (q >> 5)) m &= (1u << (q & 31)) - 1u;
            below += __popc(m);
          }
        } else {
          accepted = false;
          below = 0;
          for (int j = 0; j <= r_b; ++j) {
            const int32_t aj = tw.ai(o0 + j);
            accepted |= aj == row;
            if (aj >= o0 && aj < row) {
              bool first = true;
              for (int jj = 0; jj < j; ++jj)
                if (tw.ai(o0 + jj) == aj) first = false;
              below += first;
            }
          }
        }
        if (!accepted) {
          const int32_t x_b = xany ? t_x[lb] : 0;
          const int64_t eo_b = carry_e + (int64_t(inc_b >> 32) - len_b) - (co_b - carry_c) + (xany ? t_xex[lb] : 0);
          const int64_t pos = eo_b + (k - below);
          if (pos >= eo_b && pos < eo_b + (len_b - r_b - 1 + x_b) && pos < a.capacity) a.evict_slots[pos] = tw.vs(row);
        }
      }
    }
    __syncthreads();
    // Each thread reads back only its own status entry before the next tile rewrites the tile arrays.
    if (tid < nb) a.status[b] = t_st[tid];
    carry_c += int64_t(uint32_t(tile_tot));
    carry_e += int64_t(tile_tot >> 32) - int64_t(uint32_t(tile_tot)) + (xany ? s_xtot : 0);
    w0 += n_rows;
    t0 += nb;
  }
  if (tid == 0) {
    a.commit_offsets[B] = int32_t(carry_c);
    if (a.evict_offsets) a.evict_offsets[B] = int32_t(carry_e);
  }
}

__global__ void k_fill_zero(uint4* p, size_t n16, uint8_t* tail, size_t ntail) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

hipError_t launch_commit(const spec_commit_args& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  return launch_kernel(k_commit, dim3(1), dim3(kCommitThreads), 0, stream, ev0, ev1, a);
}

hipError_t launch_fill_zero(void* ptr, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  // Zero the 16-byte aligned interior with vector stores; the unaligned ends byte by byte.
  uint8_t* p8 = static_cast<uint8_t*>(ptr);
  const size_t lead = (16 - (reinterpret_cast<uintptr_t>(p8) & 15)) & 15;
  if (lead >= bytes) {
    hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(64), 0, stream, static_cast<uint4*>(nullptr), size_t(0), p8, bytes);
    return hipGetLastError();
  }
  if (lead) {
    hipLaunchKernelGGL(k_fill_zero, dim3(1), dim3(64), 0, stream, static_cast<uint4*>(nullptr), size_t(0), p8, lead);
  }
  uint8_t* body = p8 + lead;
  const size_t n16 = (bytes - lead) / 16;
  const size_t ntail = (bytes - lead) - n16 * 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_fill_zero, dim3(unsigned(blocks)), dim3(256), 0, stream, reinterpret_cast<uint4*>(body), n16,
                     body + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace sv
