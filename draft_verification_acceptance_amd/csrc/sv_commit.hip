// k_commit: KV commit compaction of one verify round, in one workgroup.
//   commit_len_b = accept_len_b + 1: the KV of the old anchor plus the accepted drafts
//   ([EAGLE→DFlash2] §5.6.6 commit_lens = correct_len + 1; §8.1: output E F X, committed KV D E F);
//   the accepted rows' slots move to contiguous positions after seq_lens ([SpecDec] "实现：共享的骨架",
//   move_accept_tokens_to_target_kvcache); the other verify rows are listed for eviction (§8.2: rejected
//   KV must stop being visible, when it is freed is the caller's choice).
// Requests are handled in tiles of 1024 (thread per request for the scans, thread per (request, row) for
// the gathers), so any batch size works in one launch.
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

__global__ __launch_bounds__(kCommitThreads) void k_commit(spec_commit_args a) {
  __shared__ int64_t red[kCommitThreads / kWave];
  __shared__ int32_t t_off[kCommitThreads];
  __shared__ int32_t t_len[kCommitThreads];
  __shared__ int32_t t_r[kCommitThreads];
  __shared__ int64_t t_co[kCommitThreads];
  __shared__ int64_t t_eo[kCommitThreads];
  __shared__ int32_t t_seq[kCommitThreads];
  __shared__ uint32_t t_st[kCommitThreads];

  const int tid = threadIdx.x;
  const int B = a.batch;
  const int64_t T = a.total_rows;
  const int L = a.max_verify_len;
  int64_t carry_c = 0, carry_e = 0;
  for (int t0 = 0; t0 < B; t0 += kCommitThreads) {
    const int b = t0 + tid;
    int64_t clen = 0, elen = 0;
    int32_t off0 = 0, len = 0, r = 0, seq = 0;
    uint32_t st = 0;
    if (b < B) {
      off0 = a.row_offsets[b];
      const int32_t off1 = a.row_offsets[b + 1];
      len = off1 - off0;
      bool ok = off0 >= 0 && off1 > off0 && off1 <= T && len <= L;
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
    int64_t tc, te;
    const int64_t co = carry_c + block_excl_scan_i64(clen, red, tc);
    const int64_t eo = carry_e + block_excl_scan_i64(elen, red, te);
    t_off[tid] = off0;
    t_len[tid] = len;
    t_r[tid] = r;
    t_co[tid] = co;
    t_eo[tid] = eo;
    t_seq[tid] = seq;
    t_st[tid] = st;
    if (b < B) {
      a.commit_offsets[b] = int32_t(co);
      a.new_seq_lens[b] = seq + int32_t(clen);
      if (a.evict_offsets) a.evict_offsets[b] = int32_t(eo);
    }
    __syncthreads();
    const int nb = min(kCommitThreads, B - t0);
    for (int64_t idx = tid; idx < int64_t(nb) * L; idx += kCommitThreads) {
      const int lb = int(idx / L);
      const int k = int(idx % L);
      const int32_t len_b = t_len[lb];
      if (k >= len_b) continue;
      const int32_t o0 = t_off[lb];
      const int32_t r_b = t_r[lb];
      const int32_t row = o0 + k;
      if (k <= r_b) {
        const int32_t ai = a.accept_index[row];
        bool valid = ai >= o0 && ai < o0 + len_b;
        for (int j = 0; j < k && valid; ++j)
          if (a.accept_index[o0 + j] == ai) valid = false;   // listed twice
        if (!valid) atomicOr(&t_st[lb], SPEC_ST_BAD_ACCEPT);
        a.src_slots[t_co[lb] + k] = valid ? a.verify_slots[ai] : int64_t(-1);
        a.dst_pos[t_co[lb] + k] = t_seq[lb] + k;
      }
      if (a.evict_slots) {
        int below = 0;
        bool accepted = false;
        for (int j = 0; j <= r_b; ++j) {
          const int32_t ai = a.accept_index[o0 + j];
          below += ai < row;
          accepted |= ai == row;
        }
        if (!accepted) {
          const int64_t pos = t_eo[lb] + (k - below);
          if (pos >= t_eo[lb] && pos < t_eo[lb] + (len_b - r_b - 1)) a.evict_slots[pos] = a.verify_slots[row];
        }
      }
    }
    __syncthreads();
    if (b < B) a.status[b] = t_st[tid];
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
