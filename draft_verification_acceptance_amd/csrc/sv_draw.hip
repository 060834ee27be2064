// k_draw: the final token of a sampling verify, drawn by inverse CDF from the one row (or row pair) that
// the request's scan named.
//   rejection at position j   w = [p_{j-1} - q_{j-1}]_+        ([EAGLE→DFlash2] §1.2, residual p')
//   every draft accepted      w = p_m                           ([EAGLE→DFlash2] §1.1, bonus)
//   tree target-only          w = p_cur with the tried child tokens set to 0 ([SpecDec]
//                             "为什么结果不受 draft 影响", target-only sampling; leaf: w = p_cur)
//   sparse q, rejection at j  w = [p_{j-1} - q_{j-1}]_+ where q_{j-1} is zero off its K candidates
//                             ([EAGLE→DFlash2] §6.5), so w = p except at the candidates
// The last two are one rule: w = [p - a]_+ with a per-token adjustment list a (a tried token carries
// a = +inf, a candidate its probability, repeated ids adding up) and a = 0 elsewhere.
// With a vocab mask the target row's disallowed tokens have p = 0 (so w = 0).
// The token is the number of cumulative probabilities u has reached, i.e. the smallest v with
// sum_{t<=v} w_t > u * sum w ([EAGLE→DFlash2] §6.2, inverse-CDF rule); if rounding leaves u past the last
// step the last positive-weight token is taken. Weights summing to 0 fall back to p (flagged).
//
// Layout of the work: S2 workgroups per request take batches of 512-token segments of request b's row from
// the request's counter until none is left; each wave reduces whole segments (8 consecutive tokens per lane,
// 16-byte loads) and stores sum w per segment. The request's last workgroup takes a float64 prefix over the
// segments (when the weights sum to 0 it first forms sum p per segment itself), then rescans the single
// segment holding u * Z in float64, token by token. With a fused
// KV commit each request has one more workgroup that only scans and counts the request for the commit.
#include "sv_fused.h"

namespace sv {

namespace {

struct RowCtx {
  const void* xt;
  const void* xq;
  const uint32_t* mt;   // vocab mask of the target row, or NULL
  int64_t mw;           // its words
  float coef, m_t, inv_zt, m_q, inv_zq;
  bool vec;   // both rows 16-byte aligned: whole 8-token runs load as one (bf16) or two (fp32) vectors
};

// Raw 16-bit (bf16) or 32-bit (fp32) bit patterns of 8 consecutive logits: loaded first, unpacked later,
// so that a wave can have every segment of its trip in flight at once.
struct Raw8 {
  uint4 a, b;   // bf16: a holds 8 values; fp32: a holds 4, b holds 4
};

template <typename DT>
__device__ __forceinline__ void load_raw8(const void* base, int64_t e, int64_t V, bool vec, Raw8& w) {
  const DT* row = static_cast<const DT*>(base);
  if (vec && e + 8 <= V) {
    const uint4* vp = reinterpret_cast<const uint4*>(row + e);
    w.a = load_stream(vp);
    if (sizeof(DT) == 4) w.b = load_stream(vp + 1);
    return;
  }
  // unaligned row or the row's last 8 tokens: element by element, -inf past the end
  uint32_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (sizeof(DT) == 2) v[j] = e + j < V ? uint32_t(reinterpret_cast<const uint16_t*>(row)[e + j]) : 0xFF80u;
    else v[j] = e + j < V ? __float_as_uint(reinterpret_cast<const float*>(row)[e + j]) : 0xFF800000u;
  }
  if (sizeof(DT) == 2) {
    w.a = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
  } else {
    w.a = make_uint4(v[0], v[1], v[2], v[3]);
    w.b = make_uint4(v[4], v[5], v[6], v[7]);
  }
}

template <typename DT>
__device__ __forceinline__ void unpack_raw8(const Raw8& w, float* x) {
  Elem<DT>::unpack(w.a, x);
  if (sizeof(DT) == 4) Elem<DT>::unpack(w.b, x + 4);
}

// The vocab mask word holding tokens [e, e + 8) of the target row (e % 8 == 0, so they lie in one word), all
// ones without a mask (always so when MASK is false). One load, its word index clamped into the row (bits past
// V are not used), issued with the logits' loads; the shift to token e happens where the bits are used
// (weights8), so that nothing waits for the load before then.
template <bool MASK>
__device__ __forceinline__ uint32_t row_mask_word(const RowCtx& r, int64_t e) {
  if (!MASK) return ~0u;
  return r.mt ? r.mt[min(e >> 5, r.mw - 1)] : ~0u;
}

// Weights of tokens [e, e+8) from their logits and mask word mw8 (row_mask_word): w (residual [p - q]_+ from
// a draft row, or [p - a]_+ with the adjustment list (seen, seen_a)) and p. The same arithmetic serves the
// segment sums and the token-by-token search, so both see identical values.
__device__ __forceinline__ void weights8(const RowCtx& r, int64_t e, int64_t V, uint32_t mw8, const float* x_in,
                                         const float* y, const int32_t* seen, const float* seen_a, int n_seen,
                                         float* w, float* pv) {
  float x[8];   // the target logits, disallowed ones (vocab mask) at -inf
  const uint32_t mb = mw8 >> uint32_t(e & 31);   // bit j = token e + j
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (mb >> j) & 1u ? x_in[j] : -INFINITY;
  if (r.xq) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float et = exp2_fast(fmaf(x[j], r.coef, -r.m_t));
      const float qv = exp2_fast(fmaf(y[j], r.coef, -r.m_q)) * r.inv_zq;
      pv[j] = et * r.inv_zt;
      // max(p - q, 0) with one rounding; p - q <= p <= 1, so clamping to [0, 1] is that max (one instruction
      // with the multiply-add; NaN becomes 0 as in fmaxf)
      w[j] = __builtin_amdgcn_fmed3f(fmaf(et, r.inv_zt, -qv), 0.f, 1.f);
    }
  } else {
    float adj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      pv[j] = exp2_fast(fmaf(x[j], r.coef, -r.m_t)) * r.inv_zt;
      adj[j] = 0.f;
    }
    for (int i = 0; i < n_seen; ++i) {
      const int64_t d = int64_t(seen[i]) - e;
      if (d >= 0 && d < 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j == d) adj[j] += seen_a[i];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = adj[j] > 0.f ? fmaxf(pv[j] - adj[j], 0.f) : pv[j];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (e + j >= V) { w[j] = 0.f; pv[j] = 0.f; }
}

template <typename DT, bool MASK>
__device__ __forceinline__ void load_weights8(const RowCtx& r, int64_t e, int64_t V, const int32_t* seen,
                                              const float* seen_a, int n_seen, float* w, float* pv) {
  Raw8 rt, rq;
  load_raw8<DT>(r.xt, e, V, r.vec, rt);
  if (r.xq) load_raw8<DT>(r.xq, e, V, r.vec, rq);
  const uint32_t mb = row_mask_word<MASK>(r, e);
  float x[8], y[8];
  unpack_raw8<DT>(rt, x);
  if (r.xq) unpack_raw8<DT>(rq, y);
  weights8(r, e, V, mb, x, y, seen, seen_a, n_seen, w, pv);
}

// The adjustment list entries whose token lies in [lo, hi), copied to LDS in list order (ids outside the
// vocab and masses that are negative, zero or not finite are left out). Returns the count (uniform).
__device__ int collect_adjust(const int32_t* ids, const float* as, int n, int64_t lo, int64_t hi, int32_t* s_t,
                              float* s_a, int* s_wcnt) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  int total = 0;
  for (int i0 = 0; i0 < n; i0 += kThreads) {
    const int i = i0 + tid;
    bool keep = false;
    int32_t t = 0;
    float a = INFINITY;   // tried tree tokens: removed entirely
    if (i < n) {
      t = ids[i];
      if (as) a = as[i];
      keep = t >= lo && t < hi && (as == nullptr || (a > 0.f && a < INFINITY));
    }
    const uint64_t mask = __ballot(keep);
    if (lane == 0) s_wcnt[wv] = __popcll(mask);
    __syncthreads();
    int before = total, here = 0;
    for (int w = 0; w < kThreads / kWave; ++w) {
      if (w < wv) before += s_wcnt[w];
      here += s_wcnt[w];
    }
    if (keep) {
      const int pos = before + __popcll(mask & lanes_below(lane));
      s_t[pos] = t;
      s_a[pos] = a;
    }
    total += here;
    __syncthreads();
  }
  return total;
}

// Segment sums are published and read as agent-scope 64-bit atomics (see complete_memory_ops).
__device__ __forceinline__ void store_seg(float2* dst, float w, float pv) {
  store_agent(reinterpret_cast<unsigned long long*>(dst),
              (unsigned long long)__float_as_uint(w) | ((unsigned long long)__float_as_uint(pv) << 32));
}

struct SegView {
  float2* base;
  __device__ __forceinline__ float2 operator[](int s) const {
    const unsigned long long v = load_agent(reinterpret_cast<unsigned long long*>(base + s));
    return make_float2(__uint_as_float(uint32_t(v)), __uint_as_float(uint32_t(v >> 32)));
  }
};

// Entries the adjustment list of a draw can hold.
template <bool TREE, bool SPARSE>
__host__ __device__ __forceinline__ int adjust_cap(const VerifyParams& p) {
  return TREE ? p.L : (SPARSE ? p.K : 0);
}

template <typename DT, bool TREE, bool SPARSE, bool MASK>
__global__ __launch_bounds__(kThreads) void k_draw(VerifyParams p) {
  extern __shared__ __align__(16) char smem[];
  __shared__ int s_wcnt[kThreads / kWave];
  __shared__ double red_d[kThreads / kWave];
  __shared__ int red_i[kThreads / kWave];
  __shared__ int s_last;
  __shared__ int s_batch;
  __shared__ int s_sel;
  __shared__ double s_sel_excl;

  // Workgroups per request: S2 that draw and, with a fused commit, one more in front that only runs the
  // scan, writes its outputs and takes part in the commit. The commit's last arrival does the batch's commit
  // while the memory system is busy with the draws (each of its loads then waits long): in a workgroup without
  // draw work that delays no draw. The scan-only workgroups come first in the grid (b = blockIdx): they start
  // at once, and they leave early, so draw workgroups that did not fit beside them start soon after.
  // Draw workgroup c of request b has index c * B + b for even c and c * B + (B - 1 - b) for odd c: a
  // request's workgroups are spread over the dispatch order, early and late places paired. Waves are served
  // oldest first, so the earlier workgroups stream faster; taking the segments in batches from a counter lets
  // them take more, and every request ends at about the same time (with two workgroups per request the pairing
  // evens out what the counter cannot move between requests).
  const int lead = p.cm_on ? 1 : 0;
  const bool scan_only = lead && int(blockIdx.x) < p.B;
  const int dw = int(blockIdx.x) - lead * p.B;   // draw workgroup index
  const int c = scan_only ? -1 : dw / p.B;
  const int b = scan_only ? int(blockIdx.x) : ((c & 1) ? p.B - 1 - dw % p.B : dw % p.B);
  const bool writes = lead ? scan_only : c == 0;   // the workgroup that writes the scan's outputs
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;

  // The request's scan (every workgroup of the request computes the same plan).
  const int nst = staged_parts(p.L, p.P, p.S);
  Part* stage = nst ? reinterpret_cast<Part*>(smem) : nullptr;
  char* rows = smem + size_t(nst) * sizeof(Part);
  // The adjustment list entries inside the current token range (LDS after the scan's arrays; room for every
  // entry: a tree's tried tokens are fewer than its nodes, a sparse row has K candidates).
  int32_t* s_seen = reinterpret_cast<int32_t*>(smem + scan_smem_bytes(TREE, true, p.L, p.P, p.S));
  float* s_seen_a = reinterpret_cast<float*>(s_seen + adjust_cap<TREE, SPARSE>(p));
  // Sparse q: the drawn row's whole candidate list, copied from global memory once (after the filtered list).
  int32_t* s_cand = reinterpret_cast<int32_t*>(s_seen_a + adjust_cap<TREE, SPARSE>(p));
  float* s_cand_a = reinterpret_cast<float*>(s_cand + adjust_cap<TREE, SPARSE>(p));
  DrawPlan d;
  if (TREE) {
    d = scan_tree<DT, true>(p, b, rows, stage, writes);
  } else {
    int64_t off0, len;
    if (!chain_request(p, b, off0, len)) {
      if (writes && tid == 0) write_bad_offsets(p, b);
      if (scan_only && commit_arrive<kThreads>(p, b, -1, nullptr)) fused_commit<kThreads, TREE>(p);
      return;   // no draw for b: all of b's workgroups agree
    }
    d = scan_chain_rejection<SPARSE>(p, b, off0, int(len), rows, stage, writes);
  }
  if (scan_only) {
    if (commit_arrive<kThreads>(p, b, d.r, d.path)) fused_commit<kThreads, TREE>(p);
    return;
  }

  RowCtx r;
  r.xt = static_cast<const DT*>(p.target) + int64_t(d.row_t) * p.V;
  r.xq = d.row_q >= 0 && p.draft ? static_cast<const DT*>(p.draft) + int64_t(d.row_q) * p.V : nullptr;
  r.mt = MASK && p.mask ? p.mask + int64_t(d.row_t) * p.mask_words : nullptr;
  r.mw = p.mask_words;
  r.coef = p.coef;
  r.m_t = d.m_t;
  r.inv_zt = 1.f / d.z_t;
  r.m_q = d.m_q;
  r.inv_zq = 1.f / d.z_q;
  r.vec = (reinterpret_cast<uintptr_t>(r.xt) & 15) == 0 && (reinterpret_cast<uintptr_t>(r.xq) & 15) == 0;

  // The adjustment list: the sparse candidates of the draft row, or the tokens the tree walk tried (LDS).
  const bool sparse = SPARSE && d.row_q >= 0;
  const int32_t* adj_ids = d.seen;
  const float* adj_a = nullptr;
  const int n_adj = sparse ? p.K : (TREE ? d.n_seen : 0);   // dense rejection: none (known at compile time)
  if (sparse) {   // uniform in the workgroup: every batch and the final search filter the list from LDS
    const int32_t* g_ids = p.cand_ids + int64_t(d.row_q) * p.K;
    const float* g_a = p.cand_q + int64_t(d.row_q) * p.K;
    for (int i = tid; i < p.K; i += kThreads) {
      s_cand[i] = g_ids[i];
      s_cand_a[i] = g_a[i];
    }
    __syncthreads();
    adj_ids = s_cand;
    adj_a = s_cand_a;
  }

  // Lane l of a wave owns tokens [s*512 + 8l, s*512 + 8l + 8) of segment s; wave w takes segments
  // s_begin + w, s_begin + w + kW, ... A trip covers kTrip segments per wave with all of their loads issued
  // before any is used.
  constexpr int kW = kThreads / kWave;
  constexpr int kTrip = SV_DRAW_TRIP;
  constexpr int kStep = kTrip * kW;
  const int64_t seg_base = int64_t(b) * p.n_seg;
  auto reduce_seg = [&](const Raw8& at, const Raw8& aq, uint32_t mb, int s, int n_seen) {
    const int64_t e = int64_t(s) * kSeg + 8 * lane;
    float x[8], y[8], w[8], pv[8];
    unpack_raw8<DT>(at, x);
    if (r.xq) unpack_raw8<DT>(aq, y);
    weights8(r, e, p.V, mb, x, y, s_seen, s_seen_a, n_seen, w, pv);
    float sw = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) sw += w[j];
    sw = wave_sum_dpp(sw);   // the wave is whole here: s is the same in all of its lanes
    if (lane == 0) store_seg(p.seg + seg_base + s, sw, 0.f);   // (p's sums only if the weights sum to 0)
  };
  // Batches of p.bseg segments (whole trips): draw workgroup c starts with batch c, then takes batches S2, S2 + 1,
  // ... from the request's counter, which the logits stream of this call reset to 0; the next batch is asked for
  // while this one streams. A workgroup stops at the first number past the last batch: every batch is taken by
  // exactly one workgroup, which stores its segment sums before it counts itself below.
  unsigned long long* next_batch = p.cnt2 + size_t(b) * kCounterWords + kBatchWord;
  const int n_batch = (p.n_seg + p.bseg - 1) / p.bseg;
  int batch = c;
  while (batch < n_batch) {
    const int s_begin = batch * p.bseg;
    const int s_end = min(p.n_seg, s_begin + p.bseg);
    const int n_seen = n_adj ? collect_adjust(adj_ids, adj_a, n_adj, int64_t(s_begin) * kSeg,
                                              int64_t(s_end) * kSeg, s_seen, s_seen_a, s_wcnt)
                             : 0;
    // The claim of the next batch: its atomic goes out behind the first trip's loads, and nothing uses its
    // result before the end of the batch (an add or a lane read of it here would wait for every load in flight).
    unsigned long long claim = 0ull;
    for (int t0 = s_begin + wv; t0 < s_end; t0 += kStep) {
      Raw8 rt[kTrip], rq[kTrip];
      uint32_t mk[kTrip];
#pragma unroll
      for (int u = 0; u < kTrip; ++u) {
        const int s = t0 + u * kW;
        mk[u] = ~0u;
        if (s < s_end) {
          load_raw8<DT>(r.xt, int64_t(s) * kSeg + 8 * lane, p.V, r.vec, rt[u]);
          if (r.xq) load_raw8<DT>(r.xq, int64_t(s) * kSeg + 8 * lane, p.V, r.vec, rq[u]);
          mk[u] = row_mask_word<MASK>(r, int64_t(s) * kSeg + 8 * lane);
        }
      }
      if (t0 == s_begin && tid == 0) claim = atomicAdd(next_batch, 1ull);
#pragma unroll
      for (int u = 0; u < kTrip; ++u) {
        const int s = t0 + u * kW;
        if (s >= s_end) break;
        reduce_seg(rt[u], rq[u], mk[u], s, n_seen);
      }
    }
    __syncthreads();   // every wave is past this batch's adjustment list and s_batch
    if (tid == 0) s_batch = p.S2 + int(claim);
    __syncthreads();
    batch = s_batch;
  }

  complete_memory_ops();   // every wave's segment sums are stored before the workgroup is counted
  __syncthreads();
  // The logits stream of this call reset this counter to 0 (previous kernel).
  if (tid == 0) s_last = uint32_t(atomicAdd(p.cnt2 + size_t(b) * kCounterWords, 1ull)) + 1u == uint32_t(p.S2);
  __syncthreads();
  if (!s_last) return;

  // ---- selection: float64 prefix over segments, then one segment token by token ----
  SegView seg{p.seg + int64_t(b) * p.n_seg};
  const int R = (p.n_seg + kThreads - 1) / kThreads;
  const int r_lo = min(p.n_seg, tid * R);
  const int r_hi = min(p.n_seg, r_lo + R);
  // A thread's segment sums are loaded once, all together, and kept in registers (rows of up to
  // kThreads * kSegRegs segments); longer rows read them again where they are used.
  constexpr int kSegRegs = 4;
  const bool regs = R <= kSegRegs;
  float2 sv[kSegRegs];
  if (regs) {
#pragma unroll
    for (int k = 0; k < kSegRegs; ++k) sv[k] = r_lo + k < r_hi ? seg[r_lo + k] : make_float2(0.f, 0.f);
  }
  // f(s, sums of segment s) for the thread's segments in order, until f returns true.
  auto for_segs = [&](auto&& f) {
    if (regs) {
#pragma unroll
      for (int k = 0; k < kSegRegs; ++k)
        if (r_lo + k < r_hi && f(r_lo + k, sv[k])) return;
    } else {
      for (int s = r_lo; s < r_hi; ++s)
        if (f(s, seg[s])) return;
    }
  };
  uint32_t flags = 0;
  bool use_p = false;
  double excl, incl, Z;
  {
    double loc = 0.0;
    for_segs([&](int, float2 v) { loc += double(v.x); return false; });
    block_scan_d(loc, red_d, excl, incl, Z);
  }
  if (!(Z > 0.0)) {   // weights summed to zero: draw from p instead
    use_p = true;
    flags |= SPEC_ST_ZERO_RESIDUAL;
    // The pass sums only the weights: this workgroup forms p's segment sums (the target row alone), a wave per
    // segment, kTrip segments' loads at a time, and stores them beside the weights' sums.
    RowCtx rp = r;
    rp.xq = nullptr;
    for (int t0 = wv; t0 < p.n_seg; t0 += kStep) {
      Raw8 rt[kTrip];
      uint32_t mk[kTrip];
#pragma unroll
      for (int u = 0; u < kTrip; ++u) {
        const int s = t0 + u * kW;
        mk[u] = ~0u;
        if (s < p.n_seg) {
          load_raw8<DT>(rp.xt, int64_t(s) * kSeg + 8 * lane, p.V, rp.vec, rt[u]);
          mk[u] = row_mask_word<MASK>(rp, int64_t(s) * kSeg + 8 * lane);
        }
      }
#pragma unroll
      for (int u = 0; u < kTrip; ++u) {
        const int s = t0 + u * kW;
        if (s >= p.n_seg) break;
        float x[8], w[8], pv[8];
        unpack_raw8<DT>(rt[u], x);
        weights8(rp, int64_t(s) * kSeg + 8 * lane, p.V, mk[u], x, x, s_seen, s_seen_a, 0, w, pv);
        float sp = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) sp += pv[j];
        sp = wave_sum_dpp(sp);
        if (lane == 0) store_seg(p.seg + seg_base + s, 0.f, sp);
      }
    }
    complete_memory_ops();
    __syncthreads();
    if (regs) {
#pragma unroll
      for (int k = 0; k < kSegRegs; ++k) sv[k] = r_lo + k < r_hi ? seg[r_lo + k] : make_float2(0.f, 0.f);
    }
    double loc = 0.0;
    for_segs([&](int, float2 v) { loc += double(v.y); return false; });
    block_scan_d(loc, red_d, excl, incl, Z);
  }
  const double target = double(d.u) * Z;
  if (tid == 0) s_sel = -1;
  __syncthreads();
  if (excl <= target && target < incl) {
    double acc = excl;
    int sel = -1, last_pos = -1;
    double sel_excl = 0.0, last_excl = 0.0;
    for_segs([&](int s, float2 v) {
      const double ws = double(use_p ? v.y : v.x);
      if (ws > 0.0) { last_pos = s; last_excl = acc; }
      if (target < acc + ws && ws > 0.0) { sel = s; sel_excl = acc; return true; }
      acc += ws;
      return false;
    });
    if (sel < 0) { sel = last_pos; sel_excl = last_excl; }
    if (sel >= 0) { s_sel = sel; s_sel_excl = sel_excl; }
  }
  __syncthreads();
  int sel = s_sel;
  double sel_excl = s_sel_excl;
  if (sel < 0) {
    // u * Z beyond every range (rounding or a non-finite row): the last segment with positive weight.
    int lastpos = -1;
    for_segs([&](int s, float2 v) {
      if ((use_p ? v.y : v.x) > 0.f) lastpos = s;
      return false;
    });
    lastpos = block_max_i(lastpos, red_i);
    sel = lastpos < 0 ? 0 : lastpos;
    // its start: recompute the prefix below it
    double loc = 0.0;
    for_segs([&](int s, float2 v) {
      if (s < sel) loc += double(use_p ? v.y : v.x);
      return false;
    });
    double e2, i2, t2;
    block_scan_d(loc, red_d, e2, i2, t2);
    sel_excl = t2;
  }
  // Adjustment list entries inside the selected segment.
  __syncthreads();
  const int64_t g_lo = int64_t(sel) * kSeg;
  const int n_sel = collect_adjust(adj_ids, adj_a, n_adj, g_lo, g_lo + kSeg, s_seen, s_seen_a, s_wcnt);
  if (tid < kWave) {
    // Token by token in float64, ascending: lane l holds tokens g_lo + 8l .. g_lo + 8l + 7.
    float w[8], pv[8];
    load_weights8<DT, MASK>(r, g_lo + 8 * lane, p.V, s_seen, s_seen_a, use_p ? 0 : n_sel, w, pv);
    double inc[8];
    double run = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      run += double(use_p ? pv[j] : w[j]);
      inc[j] = run;
    }
    const double lane_incl = wave_inclusive_sum_dpp(run);
    const double base = sel_excl + (lane_incl - run);
    int hit = -1, lastpos = -1;
#pragma unroll
    for (int j = 7; j >= 0; --j) {
      const double wj = double(use_p ? pv[j] : w[j]);
      if (wj > 0.0 && target < base + inc[j]) hit = j;
      if (wj > 0.0 && lastpos < 0) lastpos = j;
    }
    const uint64_t hmask = __ballot(hit >= 0);
    int64_t x;
    double c_lo, c_hi;
    if (hmask) {
      const int f = __ffsll((unsigned long long)hmask) - 1;
      const int j = __builtin_amdgcn_readlane(hit, f);
      double hi = 0.0, wj = 0.0;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k == j) { hi = base + inc[k]; wj = double(use_p ? pv[k] : w[k]); }
      c_hi = row_lanes_d(hi, f);
      c_lo = row_lanes_d(hi - wj, f);
      x = g_lo + 8 * f + j;
    } else {
      // rounding left u * Z past the segment: its last token with positive weight
      const uint64_t pmask = __ballot(lastpos >= 0);
      const int l = pmask ? 63 - __clzll((long long)pmask) : 0;
      const int j = __builtin_amdgcn_readlane(lastpos, l);
      double hi = 0.0, wj = 0.0;
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (k == j) { hi = base + inc[k]; wj = double(use_p ? pv[k] : w[k]); }
      c_hi = row_lanes_d(hi, l);
      c_lo = row_lanes_d(hi - wj, l);
      x = g_lo + 8 * l + (j < 0 ? 0 : j);
    }
    if (lane == 0) {
      const double u = double(d.u);
      // Too close to call: within 1e-5 of a step of the normalised CDF, or within 1e-6 in probability
      // mass (the resolution of fp32 probabilities; matters when the weights' total Z is small).
      const double gap = fmin(u - c_lo / Z, c_hi / Z - u);
      if (!(gap >= double(kNear)) || !(gap * Z >= double(kNearMass))) flags |= SPEC_ST_NEAR_CDF;
      const uint32_t st = d.status | flags;
      p.bonus[b] = int32_t(x);
      p.out_tokens[d.out_pos] = int32_t(x);
      p.status[b] = st;
      if (p.residual_mass) p.residual_mass[b] = float(Z);
    }
  }
}

// Chains: the maskless calls run an instantiation with no mask code at all (MASK false); masked calls and every
// tree call run the one that reads the mask row when there is one (MASK true, checked at run time). The tree
// kernel is kept on the latter: the maskless build of it measured 0.6 µs slower on the 64-node tree workload.
template <typename DT, bool MASK>
hipError_t launch_chain_draw(int mode, const VerifyParams& p, size_t smem, dim3 grid, dim3 block, hipStream_t stream,
                             hipEvent_t ev0, hipEvent_t ev1) {
  const size_t adj = sizeof(int32_t) + sizeof(float);   // per adjustment list entry
  if (mode == SPEC_MODE_REJECTION_SPARSE)   // the filtered list and the whole candidate list
    return launch_kernel(k_draw<DT, false, true, MASK>, grid, block, smem + 2 * adj * adjust_cap<false, true>(p),
                         stream, ev0, ev1, p);
  return launch_kernel(k_draw<DT, false, false, MASK>, grid, block, smem, stream, ev0, ev1, p);
}

template <typename DT>
hipError_t launch_draw_t(int mode, const VerifyParams& p, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int64_t blocks = int64_t(p.B) * (p.S2 + (p.cm_on ? 1 : 0));
  if (blocks <= 0) return hipSuccess;
  const size_t smem = scan_smem_bytes(p.tree != 0, true, p.L, p.P, p.S);
  const dim3 grid{unsigned(blocks)}, block{unsigned(kThreads)};
  if (p.tree) {
    const size_t adj = sizeof(int32_t) + sizeof(float);
    return launch_kernel(k_draw<DT, true, false, true>, grid, block, smem + adj * adjust_cap<true, false>(p), stream,
                         ev0, ev1, p);
  }
  if (p.mask) return launch_chain_draw<DT, true>(mode, p, smem, grid, block, stream, ev0, ev1);
  return launch_chain_draw<DT, false>(mode, p, smem, grid, block, stream, ev0, ev1);
}

}  // namespace

hipError_t launch_draw(int dtype, int mode, const VerifyParams& p, hipStream_t stream, hipEvent_t ev0,
                       hipEvent_t ev1) {
  if (dtype == SPEC_DTYPE_BF16) return launch_draw_t<uint16_t>(mode, p, stream, ev0, ev1);
  return launch_draw_t<float>(mode, p, stream, ev0, ev1);
}

}  // namespace sv
