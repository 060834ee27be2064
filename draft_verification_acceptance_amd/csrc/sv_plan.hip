// Verify-length planner and accept cutoff.
//
//   k_plan      one workgroup: the device allocation of [EAGLE→DFlash2] §5.6.4 (the first `budget` entries
//               of the batch in the order survival descending, position ascending, request ascending) or
//               [DSpark]'s confidence-threshold truncation, then verify_lens, the ragged offsets of §5.6.5
//               and the compact-row index.
//   k_cap_trim  one thread per request: the cutoff of §5.6.6 (cap_trim / commit_lens / block_accept_lens).
//   spec_plan_budget  (host) the budget K* of §5.6.3.
//
// The ranking is exact and needs no sort: each (request, position) entry gets a unique 64-bit key whose
// order is the ranking order (high word: the bits of the survival inverted, as survival >= 0 orders like
// its bit pattern; then the position; then the request), and a most-significant-digit radix select with
// 8-bit digits finds the budget-th smallest key T in 8 passes over the entries; the selected entries are the
// keys <= T. The survival products are float32 in position order, so every decision is a function of
// the inputs alone.
#include <string.h>

#include <vector>

#include "sv_device.h"

namespace sv {

namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / kWave;
constexpr int kPlanCache = 15360;   // survival values kept in LDS (60 KB; else recomputed each pass)
constexpr int kPlanPer = kPlanCache / kPlanThreads;   // cached entries per thread
constexpr int kPlanBatch = 16;   // confidences of one request read from LDS per round
static_assert(kPlanCache % kPlanThreads == 0, "whole entries per thread");

struct PlanParams {
  spec_plan_args a;
};

// A NaN confidence counts as 0 and one outside [0, 1] is clamped (bad = true); -0 becomes +0.
__host__ __device__ __forceinline__ float sanitize_conf(float c, bool& bad) {
  if (!(c == c)) {
    bad = true;
    return 0.f;
  }
  if (c < 0.f) bad = true;
  if (c > 1.f) {
    bad = true;
    return 1.f;
  }
  return c > 0.f ? c : 0.f;
}

__device__ __forceinline__ unsigned long long plan_key(float s, int j, int r) {
  return ((unsigned long long)(~__float_as_uint(s)) << 32) | ((unsigned long long)j << 20) | (unsigned long long)r;
}

// Block-wide exclusive prefix of int64 values over kPlanThreads threads; `red` holds kPlanWaves int64.
__device__ __forceinline__ long long plan_block_excl(long long v, long long* red, long long& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  long long inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const long long n = __shfl_up(inc, o);
    if (lane >= o) inc += n;
  }
  __syncthreads();
  if (lane == kWave - 1) red[w] = inc;
  __syncthreads();
  long long base = 0, tot = 0;
  for (int i = 0; i < kPlanWaves; ++i) {
    if (i < w) base += red[i];
    tot += red[i];
  }
  total = tot;
  return base + inc - v;
}

// Histogram add by a whole wave: lanes that share a digit (the common case) add it with one atomic.
__device__ __forceinline__ void hist_add(unsigned int* h, bool valid, unsigned int bin) {
  const uint64_t vm = __ballot(valid);
  if (!vm) return;
  const int leader = __ffsll((unsigned long long)vm) - 1;
  const unsigned int b0 = unsigned(__builtin_amdgcn_readlane(int(bin), leader));
  const bool same = valid && bin == b0;
  const uint64_t sm = __ballot(same);
  if (lane_id() == leader) atomicAdd(&h[b0], unsigned(__popcll(sm)));
  if (valid && !same) atomicAdd(&h[bin], 1u);
}

// Run by every wave on the same histogram: the digit d whose bin holds the k-th key (1-based), k's rank
// within that bin and the bin's count.
__device__ __forceinline__ void find_digit(const unsigned int* h, int k, int& digit, int& k_in_bin, int& bin_n) {
  const int lane = lane_id();
  unsigned int c[4];
  int c4 = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = h[lane * 4 + i];
    c4 += int(c[i]);
  }
  const int before0 = wave_inclusive_sum_dpp(c4) - c4;
  int found = -1, kn = 0, cn = 0, before = before0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (before < k && k <= before + int(c[i])) {
      found = lane * 4 + i;
      kn = k - before;
      cn = int(c[i]);
    }
    before += int(c[i]);
  }
  const uint64_t m = __ballot(found >= 0);
  const int src = __ffsll((unsigned long long)m) - 1;
  digit = __builtin_amdgcn_readlane(found, src);
  k_in_bin = __builtin_amdgcn_readlane(kn, src);
  bin_n = __builtin_amdgcn_readlane(cn, src);
}

// PER: the entries per thread the cached top-K keeps in registers (at least ceil(R*W / kPlanThreads)).
// PAD: the width is even and the LDS rows are padded to the odd stride W + 1.
template <int PER, bool PAD>
__global__ __launch_bounds__(kPlanThreads) void k_plan(PlanParams pp) {
  const spec_plan_args& a = pp.a;
  // [R][Wp] when R*W fits kPlanCache (at most 2 * kPlanCache floats): even rows padded to the odd stride W + 1,
  // so that threads walking consecutive requests read different LDS banks
  extern __shared__ __align__(16) float s_surv[];
  __shared__ unsigned int s_hist[3][256];
  __shared__ long long s_red[kPlanWaves];

  const int R = a.batch, W = a.width;
  const int n = R * W;
  const int tid = threadIdx.x;
  // Thread tid owns the contiguous requests [r_lo, r_hi) in the per-request passes.
  const int per = (R + kPlanThreads - 1) / kPlanThreads;
  const int r_lo = min(R, tid * per);
  const int r_hi = min(R, r_lo + per);
  const int Wp = PAD ? W + 1 : W;
  const bool cached = n <= kPlanCache;
  const bool topk = a.mode == SPEC_PLAN_TOPK && a.budget >= 0;
  const bool in_place = cached && a.mode == SPEC_PLAN_TOPK;
  const float eps = a.survival_eps;

  // The confidences go to LDS when they fit, with coalesced loads issued 8 per thread at a time (a
  // thread walking its own request's row load by load would wait a memory round trip per position).
  if (cached && n > 0) {
    constexpr int U = 8;
    // entry i = r * W + j goes to r * Wp + j; (r, j) advance by (kPlanThreads / W, kPlanThreads % W) per
    // kPlanThreads entries, no division
    const int step_r = kPlanThreads / W, step_j = kPlanThreads % W;
    int r = tid / W, j = tid % W;
    for (int base = 0; base < n; base += kPlanThreads * U) {
      float v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * kPlanThreads + tid;
        v[u] = i < n ? a.confidence[i] : 0.f;
      }
      if (!PAD) {   // odd rows are stored unpadded
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = base + u * kPlanThreads + tid;
          if (i < n) s_surv[i] = v[u];
        }
        continue;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = base + u * kPlanThreads + tid;
        if (i < n) s_surv[r * Wp + j] = v[u];
        r += step_r;
        j += step_j;
        if (j >= W) {
          j -= W;
          ++r;
        }
      }
    }
  }
  for (int i = tid; i < 3 * 256; i += kPlanThreads) (&s_hist[0][0])[i] = 0u;
  __syncthreads();
  // Confidence flags; in top-K mode the cached values become the survival products (in place), and the
  // selectable ones (survival >= eps) are counted on the way. A request's cached row is read kPlanBatch values
  // per LDS round (indices clamped into the row, so the reads need no branch).
  long long cnt = 0;
  bool dummy = false;
  for (int r = r_lo; r < r_hi; ++r) {
    bool bad = false;
    if (cached) {
      float s = 1.f;
      for (int j0 = 0; j0 < W; j0 += kPlanBatch) {
        float c[kPlanBatch];
#pragma unroll
        for (int t = 0; t < kPlanBatch; ++t) c[t] = s_surv[r * Wp + min(j0 + t, W - 1)];
#pragma unroll
        for (int t = 0; t < kPlanBatch; ++t) {
          if (j0 + t >= W) break;
          s = s * sanitize_conf(c[t], bad);
          if (in_place) {
            s_surv[r * Wp + j0 + t] = s;
            cnt += s >= eps;
          }
        }
      }
    } else {
      for (int j = 0; j < W; ++j) sanitize_conf(a.confidence[int64_t(r) * W + j], bad);
    }
    if (a.status) a.status[r] = bad ? SPEC_ST_BAD_CONF : 0u;
  }
  __syncthreads();

  // Survival of entry (r, j) while walking request r in position order (batches too large for LDS): the
  // running product `run` of the sanitized confidences in global memory.
#define SV_PLAN_SURV(r, j, run) (run = run * sanitize_conf(a.confidence[int64_t(r) * W + (j)], dummy))

  // Top-K: the budget-th smallest key T among the selectable entries: a radix select with 8-bit digits,
  // most significant first, one barrier per digit (three histogram buffers rotate: the one a pass fills,
  // the one it clears for the next pass, and the one the slowest wave may still be reading). Cached, each
  // thread keeps the keys of its entries tid + v * kPlanThreads in registers for every pass.
  unsigned long long T = 0;
  bool any = false;
  if (topk) {
    if (!cached) {
      for (int r = r_lo; r < r_hi; ++r) {
        float run = 1.f;
        for (int j = 0; j < W; ++j) cnt += SV_PLAN_SURV(r, j, run) >= eps;
      }
    }
    long long total;
    plan_block_excl(cnt, s_red, total);
    const int K = int(min((long long)a.budget, total));
    any = K > 0;
    if (any) {   // uniform; then n > 0 and W > 0
      const int nv = (n + kPlanThreads - 1) / kPlanThreads;   // at most PER when cached
      unsigned long long key[PER];   // 0: not selectable (every selectable key is nonzero)
      if (cached) {
        // entry e = r * W + j (at r * Wp + j in LDS); (r, j) advance as in the load above. Unpadded rows are
        // read at e (one base address and immediate offsets), padded ones at r * Wp + j.
        const int step_r = kPlanThreads / W, step_j = kPlanThreads % W;
        const auto build = [&](auto at) {
          int r = tid / W, j = tid % W;
#pragma unroll
          for (int v = 0; v < PER; ++v) {
            key[v] = 0ull;
            const int e = v * kPlanThreads + tid;
            if (v < nv && e < n) {
              const float sv = s_surv[at(e, r, j)];
              if (sv >= eps) key[v] = plan_key(sv, j, r);
            }
            r += step_r;
            j += step_j;
            if (j >= W) {
              j -= W;
              ++r;
            }
          }
        };
        if (!PAD) build([](int e, int, int) { return e; });
        else build([Wp](int, int r, int j) { return r * Wp + j; });
      }
      unsigned long long prefix = 0ull, mask = 0ull;
      int k = K;
      for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        unsigned int* H = s_hist[pass % 3];
        unsigned int* Z = s_hist[(pass + 1) % 3];
        for (int i = tid; i < 256; i += kPlanThreads) Z[i] = 0u;
        if (cached) {
#pragma unroll
          for (int v = 0; v < PER; ++v) {
            if (v < nv) {   // uniform: whole waves call hist_add
              const bool ok = key[v] != 0ull && (key[v] & mask) == prefix;
              hist_add(H, ok, unsigned((key[v] >> shift) & 255u));
            }
          }
        } else {
          // per thread, its requests in position order: count runs of equal digits, one atomic per run
          unsigned int run_bin = 256u, run_n = 0u;
          for (int r = r_lo; r < r_hi; ++r) {
            float run = 1.f;
            for (int j = 0; j < W; ++j) {
              const float sv = SV_PLAN_SURV(r, j, run);
              if (!(sv >= eps)) continue;
              const unsigned long long key2 = plan_key(sv, j, r);
              if ((key2 & mask) != prefix) continue;
              const unsigned int bin = unsigned((key2 >> shift) & 255u);
              if (bin != run_bin) {
                if (run_n) atomicAdd(&H[run_bin], run_n);
                run_bin = bin;
                run_n = 0u;
              }
              ++run_n;
            }
          }
          if (run_n) atomicAdd(&H[run_bin], run_n);
        }
        __syncthreads();
        int d, kn, bn;
        find_digit(H, k, d, kn, bn);
        prefix |= (unsigned long long)d << shift;
        mask |= 255ull << shift;
        k = kn;
        if (k == bn) {   // every key in this bin is selected: T is the bin's upper end (keys are unique)
          prefix |= shift ? (1ull << shift) - 1ull : 0ull;
          break;
        }
      }
      T = prefix;
    }
  }

  // Per request: selected drafts and the verify length; then the offsets.
  long long sum = 0;
  for (int r = r_lo; r < r_hi; ++r) {
    int sel = 0;
    if (a.mode == SPEC_PLAN_THRESHOLD) {   // the first position whose own confidence is below the threshold
      sel = W;
      if (cached) {
        for (int j0 = 0; j0 < W && sel == W; j0 += kPlanBatch) {
          float c[kPlanBatch];
#pragma unroll
          for (int t = 0; t < kPlanBatch; ++t) c[t] = s_surv[r * Wp + min(j0 + t, W - 1)];
#pragma unroll
          for (int t = kPlanBatch - 1; t >= 0; --t)   // the lowest position below the threshold wins
            if (j0 + t < W && sanitize_conf(c[t], dummy) < a.threshold) sel = j0 + t;
        }
      } else {
        for (int j = 0; j < W; ++j)
          if (sanitize_conf(a.confidence[int64_t(r) * W + j], dummy) < a.threshold) {
            sel = j;
            break;
          }
      }
    } else if (!topk) {
      sel = W;
    } else if (any) {
      if (cached) {
        for (int j0 = 0; j0 < W; j0 += kPlanBatch) {
          float c[kPlanBatch];
#pragma unroll
          for (int t = 0; t < kPlanBatch; ++t) c[t] = s_surv[r * Wp + min(j0 + t, W - 1)];
#pragma unroll
          for (int t = 0; t < kPlanBatch; ++t)
            if (j0 + t < W && c[t] >= eps && plan_key(c[t], j0 + t, r) <= T) ++sel;
        }
      } else {
        float run = 1.f;
        for (int j = 0; j < W; ++j) {
          const float sv = SV_PLAN_SURV(r, j, run);
          if (sv >= eps && plan_key(sv, j, r) <= T) ++sel;
        }
      }
    }
    const int vl = min(max(1 + sel, a.min_verify_len), a.max_verify_len);
    a.selected[r] = sel;
    a.verify_lens[r] = vl;
    sum += vl;
  }
#undef SV_PLAN_SURV
  long long total;
  long long off = plan_block_excl(sum, s_red, total);
  for (int r = r_lo; r < r_hi; ++r) {
    const int vl = a.verify_lens[r];   // written by this thread above
    a.offsets[r] = int32_t(off);
    if (a.row_index)
      for (int j = 0; j < vl; ++j) a.row_index[off + j] = int64_t(r) * (W + 1) + j;
    off += vl;
  }
  if (tid == 0) a.offsets[R] = int32_t(total);
}

__global__ void k_cap_trim(spec_cap_trim_args a) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.batch) return;
  const int64_t o0 = a.row_offsets[b];
  const int64_t rows = int64_t(a.row_offsets[b + 1]) - o0;
  const int v = a.verify_lens[b];
  const int raw = a.raw_accept_len[b];
  if (o0 < 0 || rows < 1 || o0 + rows > a.total_rows || v < 1 || raw < 0 || raw > rows - 1) {
    a.status[b] = SPEC_ST_BAD_ACCEPT;
    a.correct_len[b] = a.cap_trim_lens[b] = a.commit_lens[b] = a.block_accept_lens[b] = a.bonus[b] = -1;
    return;
  }
  const int ell = v - 1;
  const int capped = min(raw, ell);
  const int trim = raw - capped;
  a.correct_len[b] = capped;
  a.cap_trim_lens[b] = trim;
  a.commit_lens[b] = capped + 1;
  a.block_accept_lens[b] = capped + 1 + trim;
  a.status[b] = 0u;
  if (trim > 0) {
    a.bonus[b] = a.out_tokens[o0 + ell];
    for (int64_t k = ell + 1; k < rows; ++k) a.out_tokens[o0 + k] = -1;
  } else {
    a.bonus[b] = a.raw_bonus[b];
  }
}

// Steps per second at M target rows: linear between the table points, the nearest end value outside. `i` is
// the table segment of the previous call, M never smaller (the search only moves forward); slope[i] =
// (ys[i + 1] - ys[i]) / (xs[i + 1] - xs[i]).
double sps_at(double M, const double* xs, const double* ys, const double* slope, int n, int& i) {
#pragma clang fp contract(off)
  if (M <= xs[0]) return ys[0];
  if (M >= xs[n - 1]) return ys[n - 1];
  while (!(xs[i] <= M && M < xs[i + 1])) ++i;
  return slope[i] * (M - xs[i]) + ys[i];
}

// Non-negative floats in descending order: their bit patterns order like their values, so an LSD radix sort
// (8-bit digits, ascending) of the complemented patterns does it; a digit that is the same for every value is
// skipped. Equal values are interchangeable, so any correct sort leaves the same sequence.
void sort_desc_nonneg(std::vector<float>& a) {
  const size_t n = a.size();
  std::vector<uint32_t> k(n), t(n);
  for (size_t i = 0; i < n; ++i) {
    uint32_t b;
    memcpy(&b, &a[i], 4);
    k[i] = ~b;
  }
  for (int sh = 0; sh < 32; sh += 8) {
    size_t cnt[257] = {0};
    for (size_t i = 0; i < n; ++i) ++cnt[((k[i] >> sh) & 255u) + 1];
    if (n && cnt[((k[0] >> sh) & 255u) + 1] == n) continue;
    for (int d = 0; d < 256; ++d) cnt[d + 1] += cnt[d];
    for (size_t i = 0; i < n; ++i) t[cnt[(k[i] >> sh) & 255u]++] = k[i];
    k.swap(t);
  }
  for (size_t i = 0; i < n; ++i) {
    const uint32_t b = ~k[i];
    memcpy(&a[i], &b, 4);
  }
}

}  // namespace

hipError_t launch_plan(const spec_plan_args& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int64_t n = int64_t(a.batch) * a.width;
  const bool cached = n <= kPlanCache;
  // even rows padded to the odd stride W + 1: at most 2 * kPlanCache floats (120 KB of gfx950's 160 KB)
  const size_t smem = cached && n > 0 ? size_t(a.batch) * size_t(a.width | 1) * sizeof(float) : 0;
  // the smallest register set that holds a thread's cached entries (uncached batches keep none)
  const int64_t nv = cached ? (n + kPlanThreads - 1) / kPlanThreads : 1;
  const PlanParams pp{a};
  const dim3 g(1), blk(kPlanThreads);
  if (a.width % 2 == 0) {
    if (nv <= 1) return launch_kernel(k_plan<1, true>, g, blk, smem, stream, ev0, ev1, pp);
    if (nv <= 2) return launch_kernel(k_plan<2, true>, g, blk, smem, stream, ev0, ev1, pp);
    if (nv <= 4) return launch_kernel(k_plan<4, true>, g, blk, smem, stream, ev0, ev1, pp);
    if (nv <= 8) return launch_kernel(k_plan<8, true>, g, blk, smem, stream, ev0, ev1, pp);
    return launch_kernel(k_plan<kPlanPer, true>, g, blk, smem, stream, ev0, ev1, pp);
  }
  if (nv <= 1) return launch_kernel(k_plan<1, false>, g, blk, smem, stream, ev0, ev1, pp);
  if (nv <= 2) return launch_kernel(k_plan<2, false>, g, blk, smem, stream, ev0, ev1, pp);
  if (nv <= 4) return launch_kernel(k_plan<4, false>, g, blk, smem, stream, ev0, ev1, pp);
  if (nv <= 8) return launch_kernel(k_plan<8, false>, g, blk, smem, stream, ev0, ev1, pp);
  return launch_kernel(k_plan<kPlanPer, false>, g, blk, smem, stream, ev0, ev1, pp);
}

hipError_t launch_cap_trim(const spec_cap_trim_args& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const unsigned blocks = unsigned((a.batch + 255) / 256);
  return launch_kernel(k_cap_trim, dim3(blocks), dim3(256), 0, stream, ev0, ev1, a);
}

namespace {

// The sorted survival list of the host budget: the products of the sanitized confidences in position order
// (float32, as the device takes them), the ones below eps dropped, descending.
std::vector<float> sorted_survival(const float* conf, int32_t R, int32_t W, float eps) {
#pragma clang fp contract(off)
  std::vector<float> a;
  a.reserve(size_t(R) * W);
  for (int64_t r = 0; r < R; ++r) {
    float s = 1.f;
    bool bad = false;
    for (int64_t j = 0; j < W; ++j) {
      s = s * sanitize_conf(conf[r * W + j], bad);
      if (s >= eps) a.push_back(s);
    }
  }
  sort_desc_nonneg(a);   // the survival products are >= 0 (sanitized confidences)
  return a;
}

// A table read by the planner's rule, with its slopes computed once.
struct Table {
  const double* xs;
  const double* ys;
  int n;
  std::vector<double> slope;
  int seg = 0;   // the segment of the previous read; reads only move forward
  Table(const double* x, const double* y, int n_) : xs(x), ys(y), n(n_), slope(size_t(n_), 0.0) {
#pragma clang fp contract(off)
    for (int i = 0; i + 1 < n; ++i) slope[i] = (ys[i + 1] - ys[i]) / (xs[i + 1] - xs[i]);
  }
  double at(double M) { return sps_at(M, xs, ys, slope.data(), n, seg); }
};

// K* = argmax over 0 <= K <= n of value(N(K), R + K), N(K) = R + a_1 + .. + a_K (float64 prefix sums in the
// sorted order), the smallest K among equal values.
template <typename F>
void budget_search(const std::vector<float>& a, int32_t R, F value, int32_t* budget, double* theta,
                   int32_t* n_entries) {
#pragma clang fp contract(off)
  double N = double(R);
  double best = value(N, double(R));
  int32_t k_best = 0;
  if (theta) theta[0] = best;
  for (size_t k = 1; k <= a.size(); ++k) {
    N += double(a[k - 1]);
    const double th = value(N, double(R) + double(k));
    if (theta) theta[k] = th;
    if (th > best) {
      best = th;
      k_best = int32_t(k);
    }
  }
  *budget = k_best;
  if (n_entries) *n_entries = int32_t(a.size());
}

}  // namespace

spec_status plan_budget_host(const float* conf, int32_t R, int32_t W, const double* sps_rows, const double* sps,
                             int32_t n_sps, float eps, int32_t* budget, double* theta, int32_t* n_entries) {
  const std::vector<float> a = sorted_survival(conf, R, W, eps);
  Table t(sps_rows, sps, n_sps);
  budget_search(a, R, [&](double N, double M) {
#pragma clang fp contract(off)
    return N * t.at(M);
  }, budget, theta, n_entries);
  return SPEC_OK;
}

spec_status plan_budget_cost_host(const float* conf, int32_t R, int32_t W, const double* req_rows,
                                  const double* req_cost, int32_t n_req, const double* tok_rows,
                                  const double* tok_cost, int32_t n_tok, float eps, int32_t* budget, double* theta,
                                  int32_t* n_entries) {
  const std::vector<float> a = sorted_survival(conf, R, W, eps);
  Table tr(req_rows, req_cost, n_req), tt(tok_rows, tok_cost, n_tok);
  const double c = tr.at(double(R));
  budget_search(a, R, [&](double N, double M) {
#pragma clang fp contract(off)
    return N / (c + tt.at(M));
  }, budget, theta, n_entries);
  return SPEC_OK;
}

}  // namespace sv
