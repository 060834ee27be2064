// k_read_fold: a plain streaming read, the reference the logits stream's rate is compared with. Each
// thread reads 16-byte words (kReadUnroll of them in flight per loop trip, consecutive threads on
// consecutive words, workgroups on consecutive tiles) and XORs their 32-bit parts; workgroup k stores the
// XOR of everything it read into word k of the caller's sink (a plain store: no load can be dropped, the
// fold is checkable, and no two workgroups touch one word).
#include "sv_device.h"

namespace sv {

namespace {

// The fastest plain read measured at the stream's size (291.7 MB, cold): 512-thread workgroups, 4 loads in
// flight per thread, up to 4096 workgroups striding over 32 KB tiles (256 threads x 8192 workgroups: +1.5 %;
// one contiguous chunk per workgroup: +4 to +9 %).
constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 4;
constexpr size_t kReadTile = size_t(kReadThreads) * kReadUnroll;   // 16-byte words per workgroup trip
constexpr size_t kReadMaxBlocks = 4096;
static_assert(kReadMaxBlocks <= SPEC_READ_SINK_WORDS, "one sink word per workgroup");

struct ReadArgs {
  const uint4* src;
  size_t n16;        // 16-byte words to read
  uint32_t* sink;
};

__global__ __launch_bounds__(kReadThreads) void k_read_fold(ReadArgs a) {
  const uint4* __restrict__ src = a.src;
  const size_t n16 = a.n16;
  uint32_t acc = 0;
  for (size_t t0 = size_t(blockIdx.x) * kReadTile; t0 < n16; t0 += size_t(gridDim.x) * kReadTile) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const size_t i = t0 + size_t(u) * kReadThreads + threadIdx.x;
      const uint4 x = src[i < n16 ? i : n16 - 1];   // every lane loads: no branch among the loads
      v[u] = i < n16 ? x : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t s_acc[kReadThreads / kWave];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if (lane_id() == 0) s_acc[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kReadThreads / kWave; ++w) x ^= s_acc[w];
    a.sink[blockIdx.x] = x;
  }
}

}  // namespace

hipError_t launch_read_fold(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream, hipEvent_t ev0,
                            hipEvent_t ev1) {
  const ReadArgs a{static_cast<const uint4*>(src), bytes / 16, sink};
  if (a.n16 == 0) return hipSuccess;
  size_t blocks = (a.n16 + kReadTile - 1) / kReadTile;
  if (blocks > kReadMaxBlocks) blocks = kReadMaxBlocks;
  return launch_kernel(k_read_fold, dim3(unsigned(blocks)), dim3(kReadThreads), 0, stream, ev0, ev1, a);
}

}  // namespace sv
