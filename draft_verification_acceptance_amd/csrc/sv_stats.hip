// k_stats: one streaming pass over every verify row (target, and draft rows in rejection mode); each
// workgroup publishes a partial of its row chunk and ends. k_scan: the greedy request scans (a workgroup per
// request); k_scan_one / k_tree_one: the same for a small chain / tree batch in one workgroup.
//
// What is computed per row (the verify step scores all positions in one parallel pass; the rows after the
// first rejection are read too: [EAGLE→DFlash2] §1.1, [SpecDec] "抽象：draft → verify → commit"):
//   greedy    argmax with the lowest index among equal maxima ([SpecDec] "为什么结果不受 draft 影响":
//             verify_tree_greedy; [EAGLE→DFlash2] §1.2: same numerics and tie-breaking as plain greedy)
//   sampling  m = max(x) * log2(e)/T and z = sum exp2(x * log2(e)/T - m), i.e. softmax(x / T) = exp2(x*c - m)/z
//             ([EAGLE→DFlash2] §1.2: p_j and q_j are the distributions actually used), and for a chain the
//             logit at the token the row judges; sparse q ([EAGLE→DFlash2] §6.5): also q(d) from the draft
//             row's candidates.
// A vocab mask ([EAGLE→DFlash2] §5.6.6, §8.4: applied to the target logits after the forward, before
// acceptance) turns the disallowed logits of a target row into -inf as they stream.
#include "sv_fused.h"

namespace sv {

namespace {

constexpr int NT = kStatsThreads;         // threads per workgroup
constexpr int kW = NT / kWave;            // waves per workgroup
constexpr int kUnroll = SV_STATS_UNROLL;  // 16-byte loads in flight per thread per loop trip

struct Split {
  int64_t body_lo, nvec, body_hi, head;
};

template <typename DT>
__device__ __forceinline__ Split split_chunk(const DT* row, int64_t lo, int64_t hi) {
  constexpr int E = Elem<DT>::kPerVec;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row + lo);
  int64_t head = int64_t(((16u - unsigned(addr & 15u)) & 15u) / sizeof(DT));
  if (head > hi - lo) head = hi - lo;
  Split s;
  s.head = head;
  s.body_lo = lo + head;
  s.nvec = (hi - s.body_lo) / E;
  s.body_hi = s.body_lo + s.nvec * E;
  return s;
}

// Loads of one row chunk end with at most one partial trip whose loads are all issued together (a trip of
// single dependent loads would cost a full memory round trip each at the end of every workgroup). The
// unaligned head and tail elements (rows whose byte offset is not a multiple of 16) are loaded before the
// stream and folded in after it.

// Greedy partial of row[lo, hi) reduced over the workgroup (result valid in thread 0). MASK (0: none) applies
// the row's vocab mask `mrow` (nw words): disallowed logits become -inf as they are unpacked. 1: the chunk's
// 16-byte runs start at token multiples of the run length, so a run's bits lie in one word (one 4-byte
// load per 16-byte load, issued with it); 2: any alignment (two word loads).
template <int MASK>
__device__ __forceinline__ uint32_t run_mask(const uint32_t* mrow, int64_t v, int64_t nw) {
  return MASK == 1 ? mask_bits8_aligned(mrow, v) : MASK == 2 ? mask_bits8(mrow, v, nw) : ~0u;
}

// x[e] = bit e of mb set ? x[e] : -inf. Two instructions per element: the bit sign-extended into a full word
// (v_bfe_i32), then -inf's bits inserted where that word is clear (v_bfi_b32).
template <int N>
__device__ __forceinline__ void apply_run_mask(float* x, uint32_t mb) {
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const uint32_t keep = uint32_t(int32_t(mb << (31 - e)) >> 31);
    x[e] = __uint_as_float((keep & __float_as_uint(x[e])) | (~keep & 0xff800000u));
  }
}

template <typename DT, int MASK>
__device__ __forceinline__ void chunk_argmax(const DT* __restrict__ row, int64_t lo, int64_t hi, Part& out,
                                             float* red_f, int* red_i, uint32_t* red_u, const uint32_t* mrow,
                                             int64_t nw) {
  constexpr int E = Elem<DT>::kPerVec;
  const int tid = threadIdx.x;
  const Split sp = split_chunk(row, lo, hi);
  const uint4* __restrict__ vp = reinterpret_cast<const uint4*>(row + sp.body_lo);
  const bool has_h = tid < sp.head;
  const bool has_t = tid < hi - sp.body_hi;
  float vh = has_h ? Elem<DT>::load(row, lo + tid) : 0.f;
  float vt = has_t ? Elem<DT>::load(row, sp.body_hi + tid) : 0.f;
  if (MASK && has_h && !mask_allows(mrow, lo + tid)) vh = -INFINITY;
  if (MASK && has_t && !mask_allows(mrow, sp.body_hi + tid)) vt = -INFINITY;

  // Per thread: the largest vector maximum, the first vector attaining it and that vector's raw bits (the
  // lowest index inside it is recovered at the end without another load).
  float best = -INFINITY;
  int64_t bestk = -1;
  uint4 bestq = make_uint4(0u, 0u, 0u, 0u);
  uint32_t bestmb = ~0u;
  bool nan = false;
  auto consume = [&](const uint4& qv, int64_t kk, uint32_t mb) {
    float x[E];
    Elem<DT>::unpack(qv, x);
    if (MASK) {
      apply_run_mask<E>(x, mb);
    }
    float vm = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) vm = fmaxf(vm, x[e]);
#pragma unroll
    for (int e = 0; e < E; e += 2) nan |= __builtin_isunordered(x[e], x[e + 1]);
    if (vm > best || bestk < 0) {
      best = vm;
      bestk = kk;
      bestq = qv;
      bestmb = mb;
    }
  };
  int64_t k = tid;
  for (; k + (kUnroll - 1) * NT < sp.nvec; k += kUnroll * NT) {
    uint4 q[kUnroll];
    uint32_t mb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = load_stream(vp + k + u * NT);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) mb[u] = run_mask<MASK>(mrow, sp.body_lo + (k + u * NT) * E, nw);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) consume(q[u], k + u * NT, mb[u]);
  }
  if (k < sp.nvec) {
    uint4 q[kUnroll];
    uint32_t mb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      q[u] = k + u * NT < sp.nvec ? load_stream(vp + k + u * NT) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      mb[u] = k + u * NT < sp.nvec ? run_mask<MASK>(mrow, sp.body_lo + (k + u * NT) * E, nw) : ~0u;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (k + u * NT < sp.nvec) consume(q[u], k + u * NT, mb[u]);
  }
  int32_t idx = INT32_MAX;
  if (bestk >= 0) {  // lowest index of the thread's maximum inside its winning vector
    float x[E];
    Elem<DT>::unpack(bestq, x);
    if (MASK) {
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = (bestmb >> e) & 1u ? x[e] : -INFINITY;
    }
#pragma unroll
    for (int e = E - 1; e >= 0; --e)
      if (x[e] == best) idx = int32_t(sp.body_lo + bestk * E + e);
  }
  if (has_h) {
    if (vh != vh) nan = true;
    else if (better(vh, int32_t(lo + tid), best, idx)) { best = vh; idx = int32_t(lo + tid); }
  }
  if (has_t) {
    const int32_t i = int32_t(sp.body_hi + tid);
    if (vt != vt) nan = true;
    else if (better(vt, i, best, idx)) { best = vt; idx = i; }
  }
  // wave then workgroup reduction
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float v2 = __shfl_xor(best, o);
    const int32_t i2 = __shfl_xor(idx, o);
    if (better(v2, i2, best, idx)) { best = v2; idx = i2; }
  }
  const uint64_t nb = __ballot(nan);
  const int w = tid / kWave;
  if ((tid & (kWave - 1)) == 0) {
    red_f[w] = best;
    red_i[w] = idx;
    red_u[w] = nb != 0;
  }
  __syncthreads();
  if (tid == 0) {
    float bv = red_f[0];
    int32_t bi = red_i[0];
    uint32_t fl = red_u[0];
    for (int i = 1; i < kW; ++i) {
      if (better(red_f[i], red_i[i], bv, bi)) { bv = red_f[i]; bi = red_i[i]; }
      fl |= red_u[i];
    }
    out.a = bv;
    out.b = 0.f;
    out.idx = bi;
    out.flags = fl;
  }
}

// One element outside the 16-byte body as an (m, z) pair in log2 units: NaN poisons the sum, +inf makes the
// softmax undefined (z = NaN), -inf contributes nothing.
__device__ __forceinline__ void single_mz(float x, float coef, float& m2, float& z2) {
  m2 = x * coef;
  z2 = 1.f;
  if (x != x) { m2 = -INFINITY; z2 = x; }
  else if (m2 == -INFINITY) z2 = 0.f;
  else if (m2 == INFINITY) z2 = __builtin_nanf("");
}

// Sampling partial of row[lo, hi): (m, z) with m in log2 units, reduced over the workgroup (thread 0). MASK as
// for chunk_argmax.
template <typename DT, int MASK>
__device__ __forceinline__ void chunk_lse(const DT* __restrict__ row, int64_t lo, int64_t hi, float coef, Part& out,
                                          float* red_f, float* red_g, const uint32_t* mrow, int64_t nw) {
  constexpr int E = Elem<DT>::kPerVec;
  const int tid = threadIdx.x;
  const Split sp = split_chunk(row, lo, hi);
  const uint4* __restrict__ vp = reinterpret_cast<const uint4*>(row + sp.body_lo);
  const bool has_h = tid < sp.head;
  const bool has_t = tid < hi - sp.body_hi;
  float vh = has_h ? Elem<DT>::load(row, lo + tid) : 0.f;
  float vt = has_t ? Elem<DT>::load(row, sp.body_hi + tid) : 0.f;
  if (MASK && has_h && !mask_allows(mrow, lo + tid)) vh = -INFINITY;
  if (MASK && has_t && !mask_allows(mrow, sp.body_hi + tid)) vt = -INFINITY;

  float m = -INFINITY, z = 0.f;
  // Online update with kUnroll vectors: one rescale of z per trip.
  auto consume = [&](float* x) {
    float vm = x[0];
#pragma unroll
    for (int e = 1; e < kUnroll * E; ++e) vm = fmaxf(vm, x[e]);
    const float mn = fmaxf(m, vm * coef);
    z *= (mn == m) ? 1.f : exp2_fast(m - mn);
    m = mn;
    const float nm = (m == -INFINITY) ? 0.f : -m;
#pragma unroll
    for (int e = 0; e < kUnroll * E; ++e) z += exp2_fast(fmaf(x[e], coef, nm));
  };
  auto apply_mask = [&](float* xv, uint32_t mb) {
    if (MASK) {
      apply_run_mask<E>(xv, mb);
    }
  };
  int64_t k = tid;
  for (; k + (kUnroll - 1) * NT < sp.nvec; k += kUnroll * NT) {
    uint4 q[kUnroll];
    uint32_t mb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = load_stream(vp + k + u * NT);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) mb[u] = run_mask<MASK>(mrow, sp.body_lo + (k + u * NT) * E, nw);
    float x[kUnroll * E];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      Elem<DT>::unpack(q[u], x + u * E);
      apply_mask(x + u * E, mb[u]);
    }
    consume(x);
  }
  if (k < sp.nvec) {
    uint4 q[kUnroll];
    uint32_t mb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      q[u] = k + u * NT < sp.nvec ? load_stream(vp + k + u * NT) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      mb[u] = k + u * NT < sp.nvec ? run_mask<MASK>(mrow, sp.body_lo + (k + u * NT) * E, nw) : ~0u;
    float x[kUnroll * E];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      Elem<DT>::unpack(q[u], x + u * E);
      apply_mask(x + u * E, mb[u]);
      if (!(k + u * NT < sp.nvec)) {   // past the chunk: contributes nothing
#pragma unroll
        for (int e = 0; e < E; ++e) x[u * E + e] = -INFINITY;
      }
    }
    consume(x);
  }
  if (has_h) {
    float m2, z2;
    single_mz(vh, coef, m2, z2);
    merge_mz(m, z, m2, z2);
  }
  if (has_t) {
    float m2, z2;
    single_mz(vt, coef, m2, z2);
    merge_mz(m, z, m2, z2);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o);
    const float z2 = __shfl_xor(z, o);
    merge_mz(m, z, m2, z2);
  }
  const int w = tid / kWave;
  if ((tid & (kWave - 1)) == 0) {
    red_f[w] = m;
    red_g[w] = z;
  }
  __syncthreads();
  if (tid == 0) {
    float M = red_f[0], Z = red_g[0];
    for (int i = 1; i < kW; ++i) merge_mz(M, Z, red_f[i], red_g[i]);
    out.a = M;
    out.b = Z;
    out.idx = 0;
    out.flags = 0;
  }
}

// Sampling partial of row[lo, hi) that also stores the (m, z) of every piece (sample-then-match). The row is
// 16-byte aligned and lo a multiple of kPieceChunk (a whole number of pieces): wave w streams pieces w,
// w + kW, ... of the chunk (the workgroup's waves side by side), each trip one piece (kUnroll runs per lane,
// 64 lanes side by side, the next trip's loads issued before this one is reduced): the piece max m over the
// wave first, then z = sum exp2(x * coef - m), stored at prow[piece]. The chunk's (m, z) merges each wave's
// pieces in order, then the waves.
template <typename DT, int MASK>
__device__ __forceinline__ void chunk_lse_pieces(const DT* __restrict__ row, int64_t lo, int64_t hi, float coef,
                                                 Part& out, float* red_f, float* red_g, const uint32_t* mrow,
                                                 int64_t nw, float2* prow) {
  constexpr int E = Elem<DT>::kPerVec;
  constexpr int PW = kUnroll * kWave * E;   // tokens per piece
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  constexpr int64_t kStride = int64_t(kW) * PW;   // wave w takes pieces w, w + kW, ... of the chunk
  const int64_t wlo = lo + int64_t(w) * PW;
  const int64_t whi = hi;
  const uint4* __restrict__ vp = reinterpret_cast<const uint4*>(row);
  // Every lane loads (past the wave's range it reloads the range's last run and discards it): a load under a
  // branch would make the wait for this trip's data also wait for the next trip's, which the loop issues
  // before reducing this one.
  auto load_trip = [&](int64_t p0, uint4* q, uint32_t* mb) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = p0 + int64_t(u * kWave + lane) * E;
      const uint4 x = load_stream(vp + (v < whi ? v : whi - E) / E);
      q[u] = v < whi ? x : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = p0 + int64_t(u * kWave + lane) * E;
      const uint32_t x = run_mask<MASK>(mrow, v < whi ? v : whi - E, nw);
      mb[u] = v < whi ? x : 0u;   // past the chunk: nothing
    }
  };
  auto piece = [&](const uint4* q, const uint32_t* mb, bool whole, float& pm, float& pz) {
    float x[kUnroll * E];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      Elem<DT>::unpack(q[u], x + u * E);
      if (MASK || !whole) {
        apply_run_mask<E>(x + u * E, mb[u]);
      }
    }
    float vm = x[0];
#pragma unroll
    for (int e = 1; e < kUnroll * E; ++e) vm = fmaxf(vm, x[e]);
    pm = wave_max_dpp(vm * coef);
    const float nm = pm == -INFINITY ? 0.f : -pm;
    float lz = 0.f;
#pragma unroll
    for (int e = 0; e < kUnroll * E; ++e) lz += exp2_fast(fmaf(x[e], coef, nm));
    pz = wave_sum_dpp(lz);
  };
  float m = -INFINITY, z = 0.f;
  uint4 q[kUnroll];
  uint32_t mb[kUnroll];
  if (wlo < whi) load_trip(wlo, q, mb);
  int64_t p0 = wlo;
  // Every piece but the wave's last is whole and has a successor, whose loads go out first.
  for (; p0 + kStride < whi; p0 += kStride) {
    uint4 qn[kUnroll];
    uint32_t mbn[kUnroll];
    load_trip(p0 + kStride, qn, mbn);
    __builtin_amdgcn_sched_barrier(0);   // keep the successor's loads ahead of this piece's reduction
    float pm, pz;
    piece(q, mb, true, pm, pz);
    if (lane == 0) prow[p0 / PW] = make_float2(pm, pz);
    merge_mz(m, z, pm, pz);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      q[u] = qn[u];
      mb[u] = mbn[u];
    }
  }
  if (p0 < whi) {
    float pm, pz;
    if (p0 + PW <= whi) piece(q, mb, true, pm, pz);
    else piece(q, mb, false, pm, pz);
    if (lane == 0) prow[p0 / PW] = make_float2(pm, pz);
    merge_mz(m, z, pm, pz);
  }
  if (lane == 0) {
    red_f[w] = m;
    red_g[w] = z;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float M = red_f[0], Z = red_g[0];
    for (int i = 1; i < kW; ++i) merge_mz(M, Z, red_f[i], red_g[i]);
    out.a = M;
    out.b = Z;
    out.idx = 0;
    out.flags = 0;
  }
}

// ---------------------------------------------------------------------------------------------------
// The logits stream.
// ---------------------------------------------------------------------------------------------------
// PIECES: sample-then-match with piece partials (chain sampling only).
template <typename DT, bool SAMPLING, bool TREE, bool MASK, bool PIECES>
__global__ __launch_bounds__(NT) void k_stats(VerifyParams p) {
  __shared__ float red_f[kW];
  __shared__ float red_g[kW];
  __shared__ int red_i[kW];
  __shared__ uint32_t red_u[kW];
  __shared__ Part s_part;
  __shared__ float s_g;
  __shared__ uint32_t s_gf;

  // The fused commit of this call counts its requests from 0.
  if (p.cm_on && blockIdx.x == 0 && threadIdx.x == 0) store_agent(p.ccnt, 0ull);
  // Workgroup ids go round-robin over the XCDs. A request's (slot, part, chunk) order is rotated by its
  // index, so that the slots short requests leave empty do not always fall on the same XCDs.
  const int per_req = p.L * p.P * p.S;
  const int b = int(blockIdx.x / per_req);
  int64_t t = (int64_t(blockIdx.x % unsigned(per_req)) + b) % per_req;
  const int chunk = int(t % p.S);
  t /= p.S;
  const int part = int(t % p.P);
  const int slot = int(t / p.P);

  int64_t off0, len;
  if (TREE) {
    off0 = int64_t(b) * p.L;
    len = p.L;
  } else if (!chain_request(p, b, off0, len)) {
    return;   // reported by the request's scan
  }
  const int rows_here = part == 0 ? int(len) : int(len) - 1;
  if (slot >= rows_here) return;   // slot beyond this request's rows
  if (SAMPLING && slot == 0 && part == 0 && chunk == 0 && threadIdx.x == 0) {
    // the draw pass of this call counts its workgroups and hands out its segment batches from 0
    store_agent(p.cnt2 + size_t(b) * kCounterWords, 0ull);
    store_agent(p.cnt2 + size_t(b) * kCounterWords + kBatchWord, 0ull);
  }

  const int64_t lo = int64_t(chunk) * p.chunk;
  const int64_t hi = lo + p.chunk < p.V ? lo + p.chunk : p.V;
  const int64_t row = part == 0 ? off0 + slot : off0 - b + slot;
  const DT* base = static_cast<const DT*>(part == 0 ? p.target : p.draft) + row * p.V;
  // The vocab mask applies to target rows only.
  const uint32_t* mrow = MASK && part == 0 ? p.mask + row * p.mask_words : nullptr;

  // Chain sampling: row `slot` (target or draft) judges d_{slot+1}. The chunk holding that token reads the
  // logit there while the row streams (one thread), so the request scan needs no gathers of its own.
  const bool judge = SAMPLING && !TREE && slot < len - 1;
  float gv = 0.f;
  uint32_t gf = 0;
  if (judge && threadIdx.x == NT - 1) {
    const int32_t d = p.draft_tokens[off0 - b + slot];
    if (d >= lo && d < hi) {
      gv = Elem<DT>::load(base, d);
      if (MASK && mrow && !mask_allows(mrow, d)) gv = -INFINITY;
      gf = kPartGathered;
    }
  }
  // Sparse q: chunk 0 of the target row also sums q(d) over the draft row's candidates (wave 0) and flags
  // malformed entries.
  float qd = 0.f;
  uint32_t qf = 0;
  if (judge && p.K > 0 && part == 0 && chunk == 0 && threadIdx.x < kWave) {
    const int64_t drow = off0 - b + slot;
    const int32_t d = p.draft_tokens[drow];
    const int64_t cb = drow * int64_t(p.K);
    float acc = 0.f;
    uint32_t f = 0;
    for (int k = threadIdx.x; k < p.K; k += kWave) {
      const int32_t id = p.cand_ids[cb + k];
      const float qv = p.cand_q[cb + k];
      if (id < 0 || int64_t(id) >= p.V) f |= kPartBadCandId;
      else if (!(qv >= 0.f && qv < INFINITY)) f |= kPartBadCandQ;
      else if (id == d) acc += qv;
    }
    qd = wave_sum(acc);
    qf = (__ballot(f & kPartBadCandId) ? kPartBadCandId : 0u) | (__ballot(f & kPartBadCandQ) ? kPartBadCandQ : 0u);
  }

  // A 16-byte aligned row start (and chunk starts at multiples of 64 tokens) keeps every run's mask bits in
  // one word.
  const bool runs_aligned = (reinterpret_cast<uintptr_t>(base) & 15) == 0 && (lo & 63) == 0;
  // Sample-then-match with piece partials (aligned target rows; chunks are whole multiples of kPieceChunk).
  float2* prow = PIECES && part == 0 && runs_aligned && lo % kPieceChunk == 0
                     ? p.piece + (size_t(b) * p.L + slot) * p.n_piece
                     : nullptr;
  if (PIECES && prow) {
    if (MASK && mrow) chunk_lse_pieces<DT, 1>(base, lo, hi, p.coef, s_part, red_f, red_g, mrow, p.mask_words, prow);
    else chunk_lse_pieces<DT, 0>(base, lo, hi, p.coef, s_part, red_f, red_g, nullptr, 0, prow);
  } else if (MASK && mrow && runs_aligned) {
    if (SAMPLING) chunk_lse<DT, 1>(base, lo, hi, p.coef, s_part, red_f, red_g, mrow, p.mask_words);
    else chunk_argmax<DT, 1>(base, lo, hi, s_part, red_f, red_i, red_u, mrow, p.mask_words);
  } else if (MASK && mrow) {
    if (SAMPLING) chunk_lse<DT, 2>(base, lo, hi, p.coef, s_part, red_f, red_g, mrow, p.mask_words);
    else chunk_argmax<DT, 2>(base, lo, hi, s_part, red_f, red_i, red_u, mrow, p.mask_words);
  } else {
    if (SAMPLING) chunk_lse<DT, 0>(base, lo, hi, p.coef, s_part, red_f, red_g, nullptr, 0);
    else chunk_argmax<DT, 0>(base, lo, hi, s_part, red_f, red_i, red_u, nullptr, 0);
  }

  if (SAMPLING) {
    if (threadIdx.x == NT - 1) {
      s_g = gv;
      s_gf = gf;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    Part pt = s_part;
    if (SAMPLING) {
      pt.g = s_g;
      pt.q = qd;
      pt.flags |= s_gf | qf;
    }
    store_part(p.part + ((size_t(b) * p.L + slot) * p.P + part) * p.S + chunk, pt, SAMPLING);
  }
}

// ---------------------------------------------------------------------------------------------------
// Greedy request scans: one workgroup per request.
// ---------------------------------------------------------------------------------------------------
template <typename DT>
__global__ __launch_bounds__(kThreads) void k_scan(VerifyParams p) {
  extern __shared__ __align__(16) char smem[];
  const int b = blockIdx.x;
  const int nst = staged_parts(p.L, p.P, p.S);
  Part* stage = nst ? reinterpret_cast<Part*>(smem) : nullptr;
  char* rows = smem + size_t(nst) * sizeof(Part);
  int r = -1;
  const int32_t* path = nullptr;
  int64_t off0, len;
  if (p.tree) {
    const DrawPlan d = scan_tree<DT, false>(p, b, rows, stage, true);
    r = d.r;
    path = d.path;
  } else if (!chain_request(p, b, off0, len)) {
    if (threadIdx.x == 0) write_bad_offsets(p, b);
  } else {
    r = scan_chain_greedy(p, b, off0, int(len), rows, stage);
  }
  if (p.cm_on && commit_arrive<kThreads>(p, b, r, path)) {
    // k_scan has B workgroups, so the tree commit can hold a wider window (one tile for 32 requests of 64
    // nodes) without costing the kernel occupancy that matters.
    if (p.tree) fused_commit<kThreads, true, 2 * kFcWindow>(p);
    else fused_commit<kThreads, false>(p);
  }
}

// ---------------------------------------------------------------------------------------------------
// Greedy chains of a small batch in one workgroup. Every input that the batch's scans and its commit read
// (offsets, row partials, draft tokens; with a fused commit also seq_lens and verify_slots) goes into LDS in
// one load round; the scans run a request per segment of a wave's lanes (several short requests to a wave),
// and the commit lists follow from LDS, with no hand-off between workgroups. The outputs are those of k_scan
// and its fused commit.
// ---------------------------------------------------------------------------------------------------
#ifndef SV_ONE_THREADS
#define SV_ONE_THREADS 1024               // threads of k_scan_one / k_tree_one
#endif
constexpr int kOneThreads = SV_ONE_THREADS;
constexpr int kOneWaves = kOneThreads / kWave;
constexpr int kOneMaxB = kOneThreads;   // requests (a thread each in the commit's scan)
constexpr int kOneMaxParts = 2048;      // B * L * S row partials
constexpr int kOneMaxRows = 2048;       // verify rows of the batch
constexpr int kOneMaxLen = kWave;       // rows per request (a lane each)
constexpr int kOnePer = kOneMaxParts / kOneThreads;   // loads per thread and array in the load round
static_assert(kOneMaxRows == kOneMaxParts, "one load loop covers partials and rows");

struct GreedyPart {   // the greedy fields of a row partial
  float a;
  int32_t idx;
  uint32_t flags;
};

// A wave holds kWave / Lp requests at a time, Lp (the smallest power of two >= L) lanes each, a lane per row.
struct WaveSegs {
  int Lp, G, seg, j;
  uint64_t mask;   // the lanes of this lane's request
  __device__ __forceinline__ explicit WaveSegs(int L) {
    const int lane = threadIdx.x & (kWave - 1);
    Lp = 1 << (32 - __clz(L - 1));
    G = kWave / Lp;
    seg = lane / Lp;
    j = lane - seg * Lp;
    mask = (Lp == kWave ? ~0ull : (1ull << Lp) - 1) << (seg * Lp);
  }
};

// The scans of the batch by NW waves, a request per segment of lanes (WaveSegs). Every request output is
// written; s_r[b] takes the accepted length (-1: the request's offsets failed).
template <int NW>
__device__ __forceinline__ void greedy_chain_scans(const VerifyParams& p, const GreedyPart* pt, const int32_t* s_tok,
                                                   const int32_t* s_off, int32_t* s_r) {
  const int wv = threadIdx.x / kWave;
  const int S = p.S;
  const WaveSegs sg(p.L);
  const int j = sg.j;
  for (int b0 = wv * sg.G; b0 < p.B; b0 += NW * sg.G) {
    const int b = b0 + sg.seg;
    int64_t o0 = 0, o1 = 0;
    bool act = false;
    if (b < p.B) {
      o0 = s_off[b];
      o1 = s_off[b + 1];
      act = chain_offsets_ok(p, b, o0, o1);
      if (!act && j == 0) {
        write_bad_offsets(p, b);
        s_r[b] = -1;
      }
    }
    const int len = act ? int(o1 - o0) : 0;
    const int m = len - 1;
    const int64_t dr0 = o0 - b;
    GreedyPart row{-INFINITY, INT32_MAX, 0u};
    uint32_t f = 0;
    int32_t d = -1;
    bool fails = false;
    if (j < len) {
      const int base = (b * p.L + j) * S;
      row = pt[base];
      for (int c = 1; c < S; ++c) {
        const GreedyPart q = pt[base + c];
        if (better(q.a, q.idx, row.a, row.idx)) {
          row.a = q.a;
          row.idx = q.idx;
        }
        row.flags |= q.flags;
      }
      if (row.flags & kPartNaN) f |= SPEC_ST_NONFINITE;
      if (p.mask && row.a == -INFINITY) f |= SPEC_ST_NONFINITE;   // the mask left no finite logit
      if (j < m) {   // test of d_{j+1} against row j
        d = s_tok[dr0 + j];
        const bool ok = d >= 0 && int64_t(d) < p.V;
        if (!ok) f |= SPEC_ST_BAD_TOKEN;
        fails = !ok || d != row.idx;
      }
    }
    const uint64_t fm = __ballot(fails) & sg.mask;
    const int r = fm ? min(__ffsll((unsigned long long)fm) - 1 - sg.seg * sg.Lp, m) : m;
    const uint32_t fl = ((__ballot(f & SPEC_ST_NONFINITE) & sg.mask) ? uint32_t(SPEC_ST_NONFINITE) : 0u) |
                        ((__ballot(f & SPEC_ST_BAD_TOKEN) & sg.mask) ? uint32_t(SPEC_ST_BAD_TOKEN) : 0u);
    const int32_t bonus = __shfl(row.idx, sg.seg * sg.Lp + max(r, 0));
    if (j < len) {
      p.out_tokens[o0 + j] = j < r ? d : (j == r ? bonus : -1);
      p.accept_index[o0 + j] = j <= r ? int32_t(o0 + j) : -1;
    }
    if (p.accept_prob && j < m) p.accept_prob[dr0 + j] = -1.f;
    if (act && j == 0) {
      p.accept_len[b] = r;
      p.bonus[b] = bonus;
      p.status[b] = fl;
      if (p.residual_mass) p.residual_mass[b] = -1.f;
      s_r[b] = r;
    }
  }
}

// The commit lists from LDS, by NTH threads (B <= NTH): per request counts and their exclusive scan (a thread
// each), then the rows (a request per segment of lanes, as in the scans). s_co / s_eo take the per-request
// list offsets; s_wsum holds a word per wave. The caller synchronises after the scans (s_r complete, and
// s_co / s_eo may reuse their LDS).
template <int NTH>
__device__ __forceinline__ void greedy_chain_commit(const VerifyParams& p, const int32_t* s_off, const int32_t* s_seq,
                                                    const int32_t* s_r, const int64_t* s_vs, int32_t* s_co,
                                                    int32_t* s_eo, uint64_t* s_wsum) {
  constexpr int NW = NTH / kWave;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int B = p.B;
  {
    const int b = tid;
    const bool has = b < B;
    const int r = has ? s_r[b] : -1;
    const bool ok = r >= 0;
    const uint64_t c = ok ? uint64_t(r) + 1 : 0;
    const uint64_t e = ok ? uint64_t(s_off[b + 1] - s_off[b]) - c : 0;
    const uint64_t mine = (c << 32) | e;   // both sums stay below 2^31: no carry between the halves
    const uint64_t inc = wave_inclusive_sum_dpp(mine);
    if (lane == kWave - 1) s_wsum[wv] = inc;
    __syncthreads();
    uint64_t base = 0;
    for (int w = 0; w < wv; ++w) base += s_wsum[w];
    const uint64_t ex = base + inc - mine;
    if (has) {
      const int32_t co = int32_t(ex >> 32), eo = int32_t(uint32_t(ex));
      p.commit_offsets[b] = co;
      p.new_seq_lens[b] = s_seq[b] + int32_t(c);
      if (p.evict_offsets) p.evict_offsets[b] = eo;
      p.cstatus[b] = ok ? 0u : SPEC_ST_BAD_OFFSETS;
      s_co[b] = co;
      s_eo[b] = eo;
      if (b == B - 1) {
        const uint64_t tot = ex + mine;
        p.commit_offsets[B] = int32_t(tot >> 32);
        if (p.evict_offsets) p.evict_offsets[B] = int32_t(uint32_t(tot));
      }
    }
  }
  __syncthreads();
  const WaveSegs sg(p.L);
  for (int b0 = wv * sg.G; b0 < B; b0 += NW * sg.G) {
    const int b = b0 + sg.seg;
    const int r = b < B ? s_r[b] : -1;
    if (r < 0) continue;
    const int64_t o0 = s_off[b];
    const int len = int(s_off[b + 1] - o0);
    const int k = sg.j;
    if (k < len) {
      const int64_t v = s_vs[o0 + k];
      if (k <= r) {
        p.src_slots[int64_t(s_co[b]) + k] = v;
        p.dst_pos[int64_t(s_co[b]) + k] = s_seq[b] + k;
      } else if (p.evict_slots) {
        p.evict_slots[int64_t(s_eo[b]) + (k - r - 1)] = v;
      }
    }
  }
}

template <typename DT>
__global__ __launch_bounds__(kOneThreads) void k_scan_one(VerifyParams p) {
  __shared__ GreedyPart s_pt[kOneMaxParts];
  __shared__ int32_t s_tok[kOneMaxRows];
  __shared__ int64_t s_vs[kOneMaxRows];
  __shared__ int32_t s_off[kOneMaxB + 1];
  __shared__ int32_t s_seq[kOneMaxB];
  __shared__ int32_t s_r[kOneMaxB];       // accepted drafts of request b, -1: its offsets failed
  __shared__ uint64_t s_wsum[kOneWaves];
  const int tid = threadIdx.x;
  const int B = p.B;
  const int64_t T = p.total_rows;
  const int n_parts = B * p.L * p.S;   // the part area of request b starts at b * L * S (P = 1)

  // ---- the load round: every load of this thread issued before any is used ----
  {
    Part pv[kOnePer];
    int32_t tv[kOnePer], ov[kOnePer];
    int64_t vv[kOnePer];
#pragma unroll
    for (int k = 0; k < kOnePer; ++k) {
      const int i = tid + k * kOneThreads;
      pv[k] = i < n_parts ? load_part(p.part + i, false) : Part{};
      tv[k] = i < T - B ? p.draft_tokens[i] : 0;
      vv[k] = p.cm_on && i < T ? p.verify_slots[i] : 0;
      ov[k] = i <= B ? p.offsets[i] : 0;
    }
    const int32_t sq = p.cm_on && tid < B ? p.seq_lens[tid] : 0;
#pragma unroll
    for (int k = 0; k < kOnePer; ++k) {
      const int i = tid + k * kOneThreads;
      if (i < n_parts) s_pt[i] = GreedyPart{pv[k].a, pv[k].idx, pv[k].flags};
      if (i < T - B) s_tok[i] = tv[k];
      if (p.cm_on && i < T) s_vs[i] = vv[k];
      if (i <= B) s_off[i] = ov[k];
    }
    if (tid < B) s_seq[tid] = sq;
  }
  __syncthreads();

  greedy_chain_scans<kOneWaves>(p, s_pt, s_tok, s_off, s_r);
  if (!p.cm_on) return;
  __syncthreads();
  int32_t* s_co = reinterpret_cast<int32_t*>(s_pt);   // the partials are no longer needed
  greedy_chain_commit<kOneThreads>(p, s_off, s_seq, s_r, s_vs, s_co, s_co + kOneMaxB, s_wsum);
}

// Greedy trees of a small batch in one workgroup, the same way: partials, parents, tokens (and with a fused
// commit seq_lens and verify slots) in LDS from one load round, a wave per tree with a lane per node (the walk
// of scan_tree: from the root, the lowest-index child whose token is its parent's argmax, by ballot), and the
// commit lists from LDS (accepted nodes in path order, the others evicted in node order).
template <typename DT>
__global__ __launch_bounds__(kOneThreads) void k_tree_one(VerifyParams p) {
  __shared__ GreedyPart s_pt[kOneMaxParts];
  __shared__ int32_t s_par[kOneMaxRows];
  __shared__ int32_t s_tok[kOneMaxRows];
  __shared__ int64_t s_vs[kOneMaxRows];
  __shared__ int32_t s_seq[kOneMaxB];
  __shared__ int32_t s_r[kOneMaxB];
  __shared__ uint64_t s_path[kOneMaxB];   // the accepted nodes of each tree, one bit per node
  __shared__ uint64_t s_wsum[kOneWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int B = p.B, N = p.L, S = p.S;
  const int T = B * N;
  const int n_parts = T * S;

  // ---- the load round: every load of this thread issued before any is used ----
  {
    Part pv[kOnePer];
    int32_t av[kOnePer], tv[kOnePer];
    int64_t vv[kOnePer];
#pragma unroll
    for (int k = 0; k < kOnePer; ++k) {
      const int i = tid + k * kOneThreads;
      pv[k] = i < n_parts ? load_part(p.part + i, false) : Part{};
      av[k] = i < T ? p.parents[i] : 0;
      tv[k] = i < T ? p.tokens[i] : 0;
      vv[k] = p.cm_on && i < T ? p.verify_slots[i] : 0;
    }
    const int32_t sq = p.cm_on && tid < B ? p.seq_lens[tid] : 0;
#pragma unroll
    for (int k = 0; k < kOnePer; ++k) {
      const int i = tid + k * kOneThreads;
      if (i < n_parts) s_pt[i] = GreedyPart{pv[k].a, pv[k].idx, pv[k].flags};
      if (i < T) {
        s_par[i] = av[k];
        s_tok[i] = tv[k];
        if (p.cm_on) s_vs[i] = vv[k];
      }
    }
    if (tid < B) s_seq[tid] = sq;
  }
  __syncthreads();

  // ---- the walks: a wave per tree, a lane per node (the rules of scan_tree) ----
  for (int b = wv; b < B; b += kOneWaves) {
    const int i = lane;
    const int64_t base = int64_t(b) * N;
    uint32_t f = 0;
    int32_t arg = INT32_MAX, par = -2, tok = -1;
    if (i < N) {
      const GreedyPart* rp = s_pt + (size_t(b) * N + i) * S;
      GreedyPart row = rp[0];
      for (int c = 1; c < S; ++c) {
        const GreedyPart q = rp[c];
        if (better(q.a, q.idx, row.a, row.idx)) {
          row.a = q.a;
          row.idx = q.idx;
        }
        row.flags |= q.flags;
      }
      arg = row.idx;
      if (row.flags & kPartNaN) f |= SPEC_ST_NONFINITE;
      if (p.mask && row.a == -INFINITY) f |= SPEC_ST_NONFINITE;   // the mask left no finite logit
      const int32_t a = s_par[base + i];
      const int32_t t = s_tok[base + i];
      if (i == 0) {
        if (a != -1) f |= SPEC_ST_BAD_PARENT;
      } else {
        const bool pok = a >= 0 && a < i;
        if (!pok) f |= SPEC_ST_BAD_PARENT;
        const bool tok_ok = t >= 0 && int64_t(t) < p.V;
        if (!tok_ok) f |= SPEC_ST_BAD_TOKEN;
        par = pok ? a : -2;
        tok = tok_ok ? t : -1;
      }
    }
    // Node i may follow its parent on the path iff its token is the parent's argmax: one shuffle for every
    // node at once, so each step of the walk is a compare and a ballot (no shuffle on the chain of steps).
    const int32_t want = __shfl(arg, par < 0 ? 0 : par);
    const uint64_t ok = __ballot(i < N && par >= 0 && tok == want);
    uint64_t path = 1;   // node 0, the root
    int cur = 0, r = 0;
    while (true) {
      const uint64_t hit = __ballot(par == cur) & ok;   // children of cur (par < i: all past cur) that match
      if (!hit) break;
      cur = __ffsll((unsigned long long)hit) - 1;
      path |= 1ull << cur;
      ++r;
    }
    uint32_t fl = 0;
#pragma unroll
    for (uint32_t bit = 1; bit <= SPEC_ST_BAD_PARENT; bit <<= 1)
      if (__ballot(f & bit)) fl |= bit;
    const int32_t bonus = __shfl(arg, cur);
    // Lane i writes as node i (on the path at position k = the accepted nodes below it, since node indices
    // grow along the path: accept_index[k] = node i, out_tokens[k - 1] = its token) and as output row i (past
    // r: -1; at r: the bonus).
    if (i < N) {
      if ((path >> i) & 1ull) {
        const int k = __popcll(path & lanes_below(i));
        p.accept_index[base + k] = int32_t(base + i);
        if (k > 0) p.out_tokens[base + k - 1] = tok;
      }
      if (i == r) p.out_tokens[base + r] = bonus;
      if (i > r) {
        p.out_tokens[base + i] = -1;
        p.accept_index[base + i] = -1;
      }
      if (p.accept_prob) p.accept_prob[base + i] = -1.f;
    }
    if (lane == 0) {
      p.accept_len[b] = r;
      p.bonus[b] = bonus;
      p.status[b] = fl;
      if (p.residual_mass) p.residual_mass[b] = -1.f;
      s_r[b] = r;
      s_path[b] = path;
    }
  }
  if (!p.cm_on) return;
  __syncthreads();

  // ---- the commit lists: per tree counts and their exclusive scan, then the nodes ----
  int32_t* s_co = reinterpret_cast<int32_t*>(s_pt);   // the partials are no longer needed
  int32_t* s_eo = s_co + kOneMaxB;
  {
    const int b = tid;
    const bool has = b < B;
    const uint64_t c = has ? uint64_t(s_r[b]) + 1 : 0;
    const uint64_t e = has ? uint64_t(N) - c : 0;
    const uint64_t mine = (c << 32) | e;   // both sums stay below 2^31: no carry between the halves
    const uint64_t inc = wave_inclusive_sum_dpp(mine);
    if (lane == kWave - 1) s_wsum[wv] = inc;
    __syncthreads();
    uint64_t pre = 0;
    for (int w = 0; w < wv; ++w) pre += s_wsum[w];
    const uint64_t ex = pre + inc - mine;
    if (has) {
      const int32_t co = int32_t(ex >> 32), eo = int32_t(uint32_t(ex));
      p.commit_offsets[b] = co;
      p.new_seq_lens[b] = s_seq[b] + int32_t(c);
      if (p.evict_offsets) p.evict_offsets[b] = eo;
      p.cstatus[b] = 0u;
      s_co[b] = co;
      s_eo[b] = eo;
      if (b == B - 1) {
        const uint64_t tot = ex + mine;
        p.commit_offsets[B] = int32_t(tot >> 32);
        if (p.evict_offsets) p.evict_offsets[B] = int32_t(uint32_t(tot));
      }
    }
  }
  __syncthreads();
  for (int b = wv; b < B; b += kOneWaves) {
    const int i = lane;
    if (i < N) {
      const uint64_t path = s_path[b];
      const int below = __popcll(path & lanes_below(i));
      const int64_t v = s_vs[int64_t(b) * N + i];
      if ((path >> i) & 1ull) {
        p.src_slots[int64_t(s_co[b]) + below] = v;
        p.dst_pos[int64_t(s_co[b]) + below] = s_seq[b] + below;
      } else if (p.evict_slots) {
        p.evict_slots[int64_t(s_eo[b]) + (i - below)] = v;
      }
    }
  }
}

template <typename DT>
hipError_t launch_stats_t(int mode, const VerifyParams& p, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int64_t blocks = int64_t(p.B) * p.L * p.P * p.S;
  if (blocks <= 0) return hipSuccess;
  const bool sampling = mode != SPEC_MODE_GREEDY;
  const dim3 grid{unsigned(blocks)}, block{unsigned(NT)};
  if (sampling && !p.tree && mode == SPEC_MODE_SAMPLE_MATCH && p.piece) {
    if (p.mask) return launch_kernel(k_stats<DT, true, false, true, true>, grid, block, 0, stream, ev0, ev1, p);
    return launch_kernel(k_stats<DT, true, false, false, true>, grid, block, 0, stream, ev0, ev1, p);
  }
  if (p.mask) {
    if (p.tree) {
      if (sampling) return launch_kernel(k_stats<DT, true, true, true, false>, grid, block, 0, stream, ev0, ev1, p);
      return launch_kernel(k_stats<DT, false, true, true, false>, grid, block, 0, stream, ev0, ev1, p);
    }
    if (sampling) return launch_kernel(k_stats<DT, true, false, true, false>, grid, block, 0, stream, ev0, ev1, p);
    return launch_kernel(k_stats<DT, false, false, true, false>, grid, block, 0, stream, ev0, ev1, p);
  }
  if (p.tree) {
    if (sampling) return launch_kernel(k_stats<DT, true, true, false, false>, grid, block, 0, stream, ev0, ev1, p);
    return launch_kernel(k_stats<DT, false, true, false, false>, grid, block, 0, stream, ev0, ev1, p);
  }
  if (sampling) return launch_kernel(k_stats<DT, true, false, false, false>, grid, block, 0, stream, ev0, ev1, p);
  return launch_kernel(k_stats<DT, false, false, false, false>, grid, block, 0, stream, ev0, ev1, p);
}

// Whether a greedy batch goes to one workgroup (k_scan_one, k_tree_one): its partials, tokens and rows fit the
// LDS arrays, and a request's rows (a tree's nodes) fit a wave.
bool scan_one_fits(const VerifyParams& p) {
  const int64_t rows = p.tree ? int64_t(p.B) * p.L : p.total_rows;
  return p.P == 1 && p.B <= kOneMaxB && p.L <= kOneMaxLen && int64_t(p.B) * p.L * p.S <= kOneMaxParts &&
         rows <= kOneMaxRows;
}

}  // namespace

hipError_t launch_stats(int dtype, int mode, const VerifyParams& p, hipStream_t stream, hipEvent_t ev0,
                        hipEvent_t ev1) {
  if (dtype == SPEC_DTYPE_BF16) return launch_stats_t<uint16_t>(mode, p, stream, ev0, ev1);
  return launch_stats_t<float>(mode, p, stream, ev0, ev1);
}

hipError_t launch_scan(int dtype, const VerifyParams& p, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (p.B <= 0) return hipSuccess;
  if (scan_one_fits(p)) {   // a small greedy batch: one workgroup
    const dim3 grid{1u}, block{unsigned(kOneThreads)};
    if (p.tree) {
      if (dtype == SPEC_DTYPE_BF16) return launch_kernel(k_tree_one<uint16_t>, grid, block, 0, stream, ev0, ev1, p);
      return launch_kernel(k_tree_one<float>, grid, block, 0, stream, ev0, ev1, p);
    }
    if (dtype == SPEC_DTYPE_BF16) return launch_kernel(k_scan_one<uint16_t>, grid, block, 0, stream, ev0, ev1, p);
    return launch_kernel(k_scan_one<float>, grid, block, 0, stream, ev0, ev1, p);
  }
  const size_t smem = scan_smem_bytes(p.tree != 0, false, p.L, p.P, p.S);
  const dim3 grid{unsigned(p.B)}, block{unsigned(kThreads)};
  if (dtype == SPEC_DTYPE_BF16) return launch_kernel(k_scan<uint16_t>, grid, block, smem, stream, ev0, ev1, p);
  return launch_kernel(k_scan<float>, grid, block, smem, stream, ev0, ev1, p);
}

}  // namespace sv
