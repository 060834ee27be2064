// k_commit: KV commit compaction of one verify round, in one workgroup.
//   commit_len_b = accept_len_b + 1: the KV of the old anchor plus the accepted drafts
//   ([EAGLE→DFlash2] §5.6.6 commit_lens = correct_len + 1; §8.1: output E F X, committed KV D E F);
//   the accepted rows' slots move to contiguous positions after seq_lens ([SpecDec] "实现：共享的骨架",
//   move_accept_tokens_to_target_kvcache); the other verify rows are listed for eviction (§8.2: rejected
//   KV must stop being visible, when it is freed is the caller's choice).
// Requests are handled in tiles of up to 1024 requests and 8192 verify rows: thread per request for the
// scans, thread per verify row for the gathers, with the tile's accept_index entries staged in LDS for the
// duplicate and eviction checks. Any batch size works in one launch.
#include "sv_device.h"

namespace sv {

namespace {

constexpr int kCommitThreads = 1024;

__device__ __forceinline__ int64_t block_excl_scan_i64(int64_t v, int64_t* red, int64_t& total) {
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  int64_t inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int64_t n = __shfl_up(inc, o);
    if (lane >= o) inc += n;
  }
  __syncthreads();
  if (lane == kWave - 1) red[w] = inc;
  __syncthreads();
  int64_t base = 0, tot = 0;
  for (int i = 0; i < kCommitThreads / kWave; ++i) {
    if (i < w) base += red[i];
    tot += red[i];
  }
  __syncthreads();
  total = tot;
  return base + inc - v;
}

constexpr int kTileRows = 8192;   // verify rows whose accept_index entries are staged in LDS at once

__global__ __launch_bounds__(kCommitThreads) void k_commit(spec_commit_args a) {
  __shared__ int64_t red[kCommitThreads / kWave];
  __shared__ int32_t t_off[kCommitThreads + 1];
  __shared__ int32_t t_len[kCommitThreads];
  __shared__ int32_t t_r[kCommitThreads];
  __shared__ int32_t t_co[kCommitThreads];
  __shared__ int32_t t_eo[kCommitThreads];
  __shared__ int32_t t_seq[kCommitThreads];
  __shared__ uint32_t t_st[kCommitThreads];
  __shared__ int32_t s_ai[kTileRows];
  __shared__ int s_nb;

  const int tid = threadIdx.x;
  const int B = a.batch;
  const int64_t T = a.total_rows;
  const int L = a.max_verify_len;
  int64_t carry_c = 0, carry_e = 0;
  for (int t0 = 0; t0 < B; t0 += s_nb) {
    const int b = t0 + tid;
    int64_t clen = 0, elen = 0;
    int32_t off0 = 0, len = 0, r = 0, seq = 0;
    uint32_t st = 0;
    if (b < B) {
      off0 = a.row_offsets[b];
      const int32_t off1 = a.row_offsets[b + 1];
      len = off1 - off0;
      bool ok = off0 >= b && off1 > off0 && off1 <= T - B + b + 1 && len <= L;
      if (b == 0 && off0 != 0) ok = false;
      if (b == B - 1 && off1 != T) ok = false;
      seq = a.seq_lens[b];
      if (!ok) {
        st = SPEC_ST_BAD_OFFSETS;
        len = 0;
      } else {
        r = a.accept_len[b];
        if (r < 0 || r >= len) {
          st |= SPEC_ST_BAD_ACCEPT;
          r = r < 0 ? 0 : len - 1;
        }
        clen = r + 1;
        elen = len - clen;
      }
    }
    // This tile: as many of the next 1024 requests as have at most kTileRows rows in total (the rows
    // of a valid batch are consecutive; at least one request always fits since len <= 1024).
    int64_t tl;
    const int64_t rows_before = block_excl_scan_i64(int64_t(len), red, tl);
    const bool fits = b < B && rows_before + len <= kTileRows;
    if (tid == 0) s_nb = 0;
    __syncthreads();
    if (fits) atomicMax(&s_nb, tid + 1);
    __syncthreads();
    const int nb = s_nb;
    const bool in_tile = tid < nb;
    int64_t tc, te;
    const int64_t co = carry_c + block_excl_scan_i64(in_tile ? clen : 0, red, tc);
    const int64_t eo = carry_e + block_excl_scan_i64(in_tile ? elen : 0, red, te);
    t_off[tid] = int32_t(rows_before);   // row index relative to the tile's first row
    if (tid == nb - 1) t_off[nb] = int32_t(rows_before + len);
    t_len[tid] = len;
    t_r[tid] = r;
    t_co[tid] = int32_t(co);
    t_eo[tid] = int32_t(eo);
    t_seq[tid] = seq;
    t_st[tid] = st;
    if (in_tile) {
      a.commit_offsets[b] = int32_t(co);
      a.new_seq_lens[b] = seq + int32_t(clen);
      if (a.evict_offsets) a.evict_offsets[b] = int32_t(eo);
    }
    __syncthreads();
    // Rows of the tile: global rows [row0, row0 + n_rows) (consecutive for valid offsets; requests with
    // bad offsets own no rows).
    const int n_rows = t_off[nb];
    int32_t row0 = 0;
    {
      // first valid request's off0 minus its relative position gives the tile's first global row
      __shared__ int32_t s_row0;
      if (tid == 0) s_row0 = 0;
      __syncthreads();
      if (in_tile && len > 0 && t_off[tid] == 0) s_row0 = off0;
      __syncthreads();
      row0 = s_row0;
    }
    for (int i = tid; i < n_rows; i += kCommitThreads) s_ai[i] = row0 + i < T ? a.accept_index[row0 + i] : -1;
    __syncthreads();
    for (int i = tid; i < n_rows; i += kCommitThreads) {
      // request owning relative row i: the last lb with t_off[lb] <= i and t_len[lb] > 0
      int lo = 0, hi = nb - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (t_off[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      int lb = lo;
      while (lb > 0 && t_len[lb] == 0) --lb;
      const int32_t rel0 = t_off[lb];
      const int32_t len_b = t_len[lb];
      const int k = i - rel0;
      if (k < 0 || k >= len_b) continue;
      const int32_t r_b = t_r[lb];
      const int32_t o0 = row0 + rel0;
      const int32_t row = o0 + k;
      if (row >= T) continue;   // only when the offsets are inconsistent (the batch reports BAD_OFFSETS)
      if (k <= r_b) {
        const int32_t ai = s_ai[i];
        bool valid = ai >= o0 && ai < o0 + len_b && ai < T;
        for (int j = 0; j < k && valid; ++j)
          if (s_ai[rel0 + j] == ai) valid = false;   // listed twice
        if (!valid) atomicOr(&t_st[lb], SPEC_ST_BAD_ACCEPT);
        if (int64_t(t_co[lb]) + k < a.capacity) {   // always true unless the offsets are inconsistent
          a.src_slots[t_co[lb] + k] = valid ? a.verify_slots[ai] : int64_t(-1);
          a.dst_pos[t_co[lb] + k] = t_seq[lb] + k;
        }
      }
      if (a.evict_slots) {
        int below = 0;
        bool accepted = false;
        for (int j = 0; j <= r_b; ++j) {
          const int32_t ai = s_ai[rel0 + j];
          below += ai < row;
          accepted |= ai == row;
        }
        if (!accepted) {
          const int64_t pos = int64_t(t_eo[lb]) + (k - below);
          if (pos >= t_eo[lb] && pos < int64_t(t_eo[lb]) + (len_b - r_b - 1) && pos < a.capacity)
            a.evict_slots[pos] = a.verify_slots[row];
        }
      }
    }
    __syncthreads();
    if (in_tile) a.status[b] = t_st[tid];
    carry_c += tc;
    carry_e += te;
    __syncthreads();
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

hipError_t launch_commit(const spec_commit_args& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_commit, dim3(1), dim3(kCommitThreads), 0, stream, a);
  return hipGetLastError();
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
