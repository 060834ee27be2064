// k_match: the second kernel of a sample-then-match verify. Every target row j draws its own token t_j from
// p_j by inverse CDF with its uniform; d_{j+1} is accepted while it equals t_j, and the first mismatch (or
// row m) emits t_j ([DFlash] decode loop, step 4: compare each draft token with a sample of the posterior,
// longest matching prefix, the first mismatch replaced by the posterior's sample; [EAGLE→DFlash2] §1.2:
// independent target sampling then prefix matching is a different implementation from p/q rejection).
//
// Requests of up to 16 rows: k_match_split, four rows (a wave each) per workgroup, the request's rows spread
// over several workgroups that hand their results to the last of them. Longer requests: k_match, one workgroup
// of 1024 threads per request, one wave per row, 16 rows at a time in row order; the request stops after the
// first group of rows that holds a mismatch. A draw does not read the whole row: the stream
// stored the (m, z) of every piece of the row (2048 tokens in bf16) or, for rows that are not 16-byte
// aligned, of its chunks, so the unit holding u * Z is known from those masses z_i 2^(m_i - m); the wave
// then narrows that unit down (each lane sums a contiguous range of it in float64, a wave scan picks the
// lane whose range holds the target, and so on until a lane holds at most 8 tokens; a unit of at most 2048
// tokens, a bf16 piece, is decided in one round: each lane holds its 32 tokens and the picked lane walks
// them). Only that unit of the row is read (4 KB per row for a bf16 piece).
#include "sv_fused.h"

namespace sv {

namespace {

constexpr int kMatchThreads = 1024;
constexpr int kMatchWaves = kMatchThreads / kWave;
constexpr int kSumUnrollStream = SV_STATS_UNROLL;   // runs per lane in one trip of the stream: a piece
// 8-token runs in flight per lane while a range is summed (16 VGPRs of raw words for either type; the
// multi-level draw serves units wider than a piece, which only rows without piece partials have)
template <typename DT>
constexpr int sum_unroll() {
  return sizeof(DT) == 2 ? 4 : 2;
}

// Raw bits of the logits of tokens [e, e + 8) of a row (bf16: one 16-byte word, fp32: two), -inf from `end`
// on: vector loads when the run is whole and aligned, element by element otherwise. Plain (cached) loads:
// the narrower levels of a draw read the same bytes again.
struct Raw8 {
  uint4 a, b;
};

template <typename DT>
__device__ __forceinline__ void load_raw8(const DT* row, int e, int end, Raw8& w) {
  if (e + 8 <= end && (reinterpret_cast<uintptr_t>(row + e) & 15) == 0) {
    const uint4* vp = reinterpret_cast<const uint4*>(row + e);
    w.a = vp[0];
    if (sizeof(DT) == 4) w.b = vp[1];
    return;
  }
  uint32_t v[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (sizeof(DT) == 2) v[j] = e + j < end ? uint32_t(reinterpret_cast<const uint16_t*>(row)[e + j]) : 0xFF80u;
    else v[j] = e + j < end ? __float_as_uint(reinterpret_cast<const float*>(row)[e + j]) : 0xFF800000u;
  }
  if (sizeof(DT) == 2) {
    w.a = make_uint4(v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16));
  } else {
    w.a = make_uint4(v[0], v[1], v[2], v[3]);
    w.b = make_uint4(v[4], v[5], v[6], v[7]);
  }
}

// The weights exp2(x * coef - m) of the run at e (0 where the vocab mask disallows or past the row).
template <typename DT>
__device__ __forceinline__ void weights8(const Raw8& r, int e, float coef, float m, const uint32_t* mrow, int64_t mw,
                                         float* w) {
  float x[8];
  Elem<DT>::unpack(r.a, x);
  if (sizeof(DT) == 4) Elem<DT>::unpack(r.b, x + 4);
  const uint32_t mb = mrow ? mask_bits8(mrow, e, mw) : ~0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = (mb >> j) & 1u ? exp2_fast(fmaf(x[j], coef, -m)) : 0.f;
}

// Sum of the weights of tokens [la, lb), ascending, in float64 (sum_unroll runs in flight).
template <typename DT>
__device__ double range_sum(const DT* row, int la, int lb, float coef, float m, const uint32_t* mrow, int64_t mw) {
  constexpr int kSumUnroll = sum_unroll<DT>();
  double s = 0.0;
  for (int e0 = la; e0 < lb; e0 += 8 * kSumUnroll) {
    Raw8 r[kSumUnroll];
#pragma unroll
    for (int u = 0; u < kSumUnroll; ++u)
      if (e0 + 8 * u < lb) load_raw8<DT>(row, e0 + 8 * u, lb, r[u]);
#pragma unroll
    for (int u = 0; u < kSumUnroll; ++u) {
      const int e = e0 + 8 * u;
      if (e >= lb) break;
      float w[8];
      weights8<DT>(r[u], e, coef, m, mrow, mw, w);
#pragma unroll
      for (int j = 0; j < 8; ++j) s += double(w[j]);
    }
  }
  return s;
}

// Inverse-CDF draw inside tokens [a, a + n) of a row (one wave, every lane active): t = the target mass
// measured from a. Returns the token (the first whose cumulative weight exceeds t; if rounding leaves t past
// the range, the last token with positive weight); cum = the mass before it, measured from a; w_tok = its
// weight.
template <typename DT>
__device__ int wave_draw(const DT* row, int a, int n, double t, float coef, float m, const uint32_t* mrow, int64_t mw,
                         double& cum, double& w_tok) {
  const int lane = lane_id();
  cum = 0.0;
  w_tok = 0.0;
  while (n > 0) {
    int per = (n + kWave - 1) / kWave;
    if (per > 8) per = (per + 7) / 8 * 8;   // 8-token runs stay 16-byte aligned
    const int la = a + min(n, lane * per);
    const int lb = a + min(n, (lane + 1) * per);
    float wl[8];
    double s = 0.0;
    if (per <= 8) {
      if (la < lb) {
        Raw8 r;
        load_raw8<DT>(row, la, lb, r);
        weights8<DT>(r, la, coef, m, mrow, mw, wl);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) wl[j] = 0.f;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) s += double(wl[j]);
    } else {
      s = range_sum<DT>(row, la, lb, coef, m, mrow, mw);
    }
    const double incl = wave_inclusive_sum_dpp(s);
    const double excl = incl - s;
    const uint64_t hit = __ballot(s > 0.0 && t < incl);
    int f;
    if (hit) {
      f = __ffsll((unsigned long long)hit) - 1;
    } else {
      const uint64_t pos = __ballot(s > 0.0);
      f = pos ? 63 - __clzll((long long)pos) : 0;
    }
    const double ex_f = row_lanes_d(excl, f);
    t -= ex_f;
    cum += ex_f;
    if (per <= 8) {
      // lane f holds the token among its (at most 8) weights
      int pick = 0;
      double before = 0.0, wp = 0.0;
      if (lane == f) {
        int first = -1, last = -1;
        double acc = 0.0, b_first = 0.0, b_last = 0.0, w_first = 0.0, w_last = 0.0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const double wj = double(wl[j]);
          if (wj > 0.0) {
            if (first < 0 && t < acc + wj) { first = j; b_first = acc; w_first = wj; }
            last = j;
            b_last = acc;
            w_last = wj;
          }
          acc += wj;
        }
        if (first >= 0) { pick = first; before = b_first; wp = w_first; }
        else if (last >= 0) { pick = last; before = b_last; wp = w_last; }
      }
      const int tok = __builtin_amdgcn_readlane(la + pick, f);
      cum += row_lanes_d(before, f);
      w_tok = row_lanes_d(wp, f);
      return tok;
    }
    a = __builtin_amdgcn_readlane(la, f);
    n = __builtin_amdgcn_readlane(lb, f) - a;
  }
  return a;
}

// wave_draw for a unit of at most kWave * 32 tokens (a stream piece) in one round of loads: every lane holds
// its whole range (at most 4 runs of 8) in registers; a wave scan of the lane sums picks the lane, whose
// words are then read out (readlane) so that lane l weighs its l-th token, and a second wave scan picks the
// token. Same contract as wave_draw.
template <typename DT>
__device__ int wave_draw_small(const DT* row, int a, int n, double t, float coef, float m, const uint32_t* mrow,
                               int64_t mw, double& cum, double& w_tok) {
  constexpr int kRuns = 4;
  constexpr int kWords = sizeof(DT) == 2 ? 4 : 8;   // 32-bit words per 8-token run
  constexpr int kTokPerWord = 4 / int(sizeof(DT));
  const int lane = lane_id();
  int per = (n + kWave - 1) / kWave;
  if (per > 8) per = (per + 7) / 8 * 8;   // 8-token runs stay 16-byte aligned
  const int la = a + min(n, lane * per);
  const int lb = a + min(n, (lane + 1) * per);
  Raw8 r[kRuns];
#pragma unroll
  for (int k = 0; k < kRuns; ++k) {
    r[k].a = make_uint4(0u, 0u, 0u, 0u);
    r[k].b = r[k].a;
    if (la + 8 * k < lb) load_raw8<DT>(row, la + 8 * k, lb, r[k]);
  }
  // Lane sums: each run of 8 weights added in fp32 (relative error below 1e-6, far inside the 1e-5 band a
  // draw is flagged in), the runs in float64.
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kRuns; ++k) {
    if (la + 8 * k < lb) {
      float w[8];
      weights8<DT>(r[k], la + 8 * k, coef, m, mrow, mw, w);
      s += double(((w[0] + w[1]) + (w[2] + w[3])) + ((w[4] + w[5]) + (w[6] + w[7])));
    }
  }
  double incl = wave_inclusive_sum_dpp(s);
  uint64_t hit = __ballot(s > 0.0 && t < incl);
  int f;
  if (hit) {
    f = __ffsll((unsigned long long)hit) - 1;
  } else {
    const uint64_t pos = __ballot(s > 0.0);
    f = pos ? 63 - __clzll((long long)pos) : 0;
  }
  const double ex_f = row_lanes_d(incl - s, f);
  t -= ex_f;
  // Second level: lane l weighs token la_f + l of lane f's range (its word read out of lane f's registers).
  const int la_f = __builtin_amdgcn_readlane(la, f);
  const int nt = __builtin_amdgcn_readlane(lb, f) - la_f;   // at most 32
  const int widx = lane / kTokPerWord;
  uint32_t word = 0u;
#pragma unroll
  for (int k = 0; k < kRuns; ++k) {
    const uint32_t rw[8] = {r[k].a.x, r[k].a.y, r[k].a.z, r[k].a.w, r[k].b.x, r[k].b.y, r[k].b.z, r[k].b.w};
#pragma unroll
    for (int q = 0; q < kWords; ++q) {
      const uint32_t v = uint32_t(__builtin_amdgcn_readlane(int(rw[q]), f));
      if (widx == k * kWords + q) word = v;
    }
  }
  float x;
  if (sizeof(DT) == 2) x = __uint_as_float((lane & 1) ? (word & 0xFFFF0000u) : (word << 16));
  else x = __uint_as_float(word);
  const int tok_l = la_f + lane;
  const bool allowed = lane < nt && (mrow == nullptr || mask_allows(mrow, tok_l));
  const double w1 = allowed ? double(exp2_fast(fmaf(x, coef, -m))) : 0.0;
  incl = wave_inclusive_sum_dpp(w1);
  hit = __ballot(w1 > 0.0 && t < incl);
  int g;
  if (hit) {
    g = __ffsll((unsigned long long)hit) - 1;
  } else {   // rounding left t past the range: its last token with positive weight
    const uint64_t pos = __ballot(w1 > 0.0);
    g = pos ? 63 - __clzll((long long)pos) : 0;
  }
  cum = ex_f + row_lanes_d(incl - w1, g);
  w_tok = row_lanes_d(w1, g);
  return la_f + g;
}

// Masses of the units a row's CDF is first split into, in row order: the stream's pieces (when it stored
// them) or its chunks. unit_mass(i) = z_i 2^(m_i - m) for the row max m, as a float64.
struct RowUnits {
  const Part* chunks;     // the row's S chunk partials
  const float2* pieces;   // or its piece partials (NULL: chunks)
  int n;                  // units in the row
  int64_t width;          // tokens per unit
  __device__ __forceinline__ double mass(int i, float m) const {
    float mi, zi;
    if (pieces) {
      const float2 v = pieces[i];
      mi = v.x;
      zi = v.y;
    } else {
      const Part pt = load_part(chunks + i, true);
      mi = pt.a;
      zi = pt.b;
    }
    return zi > 0.f ? double(zi) * double(exp2_fast(mi - m)) : 0.0;
  }
};

// unit_mass of a unit whose (m_i, z_i) is already loaded. 2^(m_i - m) in fp32 (m_i <= m: a factor in
// (0, 1], as accurate as the fp32 z_i it scales).
__device__ __forceinline__ double unit_mass(float2 mz, float m) {
  return mz.y > 0.f ? double(mz.y) * double(exp2_fast(mz.x - m)) : 0.0;
}

// Unit masses each lane keeps in registers (units lane + 64 k): rows of up to 128 units never reload them.
constexpr int kUnitRegs = 4;

// One row's result, valid in lane 0 of the wave that computed it.
struct MatchRow {
  int32_t d;     // d_{j+1} (-1 for the last row)
  int32_t t;     // the row's sample (when drawn)
  uint32_t f;    // the row's status bits
  bool near;     // the sample lies within 1e-5 of a step of the normalised CDF (when drawn)
  float m, z, g;   // row max (log2 units), normaliser, the logit gathered at d_{j+1} (0 if none)
};

// Row j of request b, one wave: one round of loads (its chunk partials, the raw (m, z) of its units, its draft
// token and uniforms; every lane loads at clamped indices and discards what is out of range), the partials
// merged (status, row max, normaliser, the gathered logit), the unit masses totalled in float64 and, if
// `draw`, the sample: the unit holding u * Z from the masses in registers, then the token inside that unit.
template <typename DT>
__device__ MatchRow match_row(const VerifyParams& p, int b, int j, int64_t off0, int m, bool draw) {
  constexpr int PW = kSumUnrollStream * kWave * Elem<DT>::kPerVec;   // tokens per stream piece
  const int lane = threadIdx.x & (kWave - 1);
  const int S = p.S;
  const int64_t dr0 = off0 - b;
  RowUnits ru;
  ru.chunks = p.part + (size_t(b) * p.L + j) * S;   // P = 1: target rows only
  ru.pieces = p.piece ? p.piece + (size_t(b) * p.L + j) * p.n_piece : nullptr;
  ru.n = p.piece ? int((p.V + PW - 1) / PW) : S;
  ru.width = p.piece ? int64_t(PW) : p.chunk;
  const Part* rowp = ru.chunks;
  const bool regs = ru.pieces ? ru.n <= kWave * kUnitRegs : S <= kWave;
  // ---- one round of loads
  const Part pt0 = load_part(rowp + min(lane, S - 1), true);
  float2 ur[kUnitRegs];
#pragma unroll
  for (int k = 0; k < kUnitRegs; ++k)
    ur[k] = ru.pieces ? ru.pieces[min(lane + kWave * k, ru.n - 1)] : make_float2(pt0.a, pt0.b);
  const int jd = m > 0 ? min(j, m - 1) : 0;
  const int32_t d_ld = m > 0 ? p.draft_tokens[dr0 + jd] : -1;
  const float ua_ld = m > 0 ? p.u_accept[dr0 + jd] : 0.f;
  const float uf_ld = p.u_final[b];
  // ---- the chunk partials, merged lane-parallel
  float mj = -INFINITY, zj = 0.f, gj = 0.f;
  bool gathered = false;
  for (int c0 = 0; c0 < S; c0 += kWave) {
    const int c = c0 + lane;
    const Part pt = c0 == 0 ? pt0 : load_part(rowp + min(c, S - 1), true);
    float cm = c < S ? pt.a : -INFINITY, cz = c < S ? pt.b : 0.f;
    // butterfly inside each 16-lane row (DPP), then the four row results
    merge_mz(cm, cz, dpp_f<0xB1>(cm), dpp_f<0xB1>(cz));
    merge_mz(cm, cz, dpp_f<0x4E>(cm), dpp_f<0x4E>(cz));
    merge_mz(cm, cz, dpp_f<0x141>(cm), dpp_f<0x141>(cz));
    merge_mz(cm, cz, dpp_f<0x140>(cm), dpp_f<0x140>(cz));
    float rm = row_lanes(cm, 0), rz = row_lanes(cz, 0);
    merge_mz(rm, rz, row_lanes(cm, 16), row_lanes(cz, 16));
    merge_mz(rm, rz, row_lanes(cm, 32), row_lanes(cz, 32));
    merge_mz(rm, rz, row_lanes(cm, 48), row_lanes(cz, 48));
    merge_mz(mj, zj, rm, rz);
    const uint64_t gm = __ballot(c < S && (pt.flags & kPartGathered));
    if (gm) {
      gj = row_lanes(pt.g, __ffsll((unsigned long long)gm) - 1);
      gathered = true;
    }
  }
  // ---- unit masses (float64) and their total Z
  double ms[kUnitRegs];
  double Z = 0.0;
  if (regs) {
#pragma unroll
    for (int k = 0; k < kUnitRegs; ++k) {
      ms[k] = lane + kWave * k < ru.n ? unit_mass(ur[k], mj) : 0.0;
      if (kWave * k < ru.n) Z += wave_sum_dpp(ms[k]);
    }
  } else {
    for (int i0 = 0; i0 < ru.n; i0 += kWave) Z += wave_sum_dpp(i0 + lane < ru.n ? ru.mass(i0 + lane, mj) : 0.0);
  }
  MatchRow out;
  out.d = j < m ? d_ld : -1;
  bool ubad = false;
  const float u = sanitize_u(j < m ? ua_ld : uf_ld, ubad);
  out.f = 0;
  if (j < m && !(out.d >= 0 && int64_t(out.d) < p.V)) out.f |= SPEC_ST_BAD_TOKEN;
  if (ubad) out.f |= SPEC_ST_BAD_UNIFORM;
  if (z_bad(zj)) out.f |= SPEC_ST_NONFINITE;
  out.m = mj;
  out.z = zj;
  out.g = gathered ? gj : 0.f;
  out.t = -1;
  out.near = false;
  if (draw) {
    const double T = double(u) * Z;
    // the unit holding T (the first with positive mass whose cumulative mass passes T; rounding past the
    // end: the last with positive mass)
    int usel = -1, ulast = -1;
    double cum0 = 0.0, cum_last = 0.0, carry = 0.0;
    auto scan_block = [&](int i0, double mass) {
      const double incl = carry + wave_inclusive_sum_dpp(mass);
      const uint64_t hit = __ballot(mass > 0.0 && T < incl);
      if (hit) {
        const int f = __ffsll((unsigned long long)hit) - 1;
        usel = i0 + f;
        cum0 = row_lanes_d(incl - mass, f);
      }
      const uint64_t pos = __ballot(mass > 0.0);
      if (pos) {
        const int f = 63 - __clzll((long long)pos);
        ulast = i0 + f;
        cum_last = row_lanes_d(incl - mass, f);
      }
      carry = row_lanes_d(incl, kWave - 1);
    };
    if (regs) {
#pragma unroll
      for (int k = 0; k < kUnitRegs; ++k)
        if (usel < 0 && kWave * k < ru.n) scan_block(kWave * k, ms[k]);
    } else {
      for (int i0 = 0; i0 < ru.n && usel < 0; i0 += kWave)
        scan_block(i0, i0 + lane < ru.n ? ru.mass(i0 + lane, mj) : 0.0);
    }
    if (usel < 0) {   // rounding left u * Z past every unit (or nothing has mass)
      usel = ulast < 0 ? 0 : ulast;
      cum0 = ulast < 0 ? 0.0 : cum_last;
    }
    const int a = int(int64_t(usel) * ru.width);
    const int n = int(min(p.V, int64_t(usel + 1) * ru.width)) - a;
    const DT* row = static_cast<const DT*>(p.target) + (off0 + j) * p.V;
    const uint32_t* mrow = p.mask ? p.mask + (off0 + j) * p.mask_words : nullptr;
    double cum1, w_tok;
    out.t = n <= kWave * 32 ? wave_draw_small<DT>(row, a, n, T - cum0, p.coef, mj, mrow, p.mask_words, cum1, w_tok)
                            : wave_draw<DT>(row, a, n, T - cum0, p.coef, mj, mrow, p.mask_words, cum1, w_tok);
    // Too close to call: u within 1e-5 of a step of the normalised CDF.
    const double lo = (cum0 + cum1) / Z;
    const double gap = fmin(double(u) - lo, lo + w_tok / Z - double(u));
    out.near = !(gap >= double(kNear));
  }
  return out;
}

// p_k(d_{k+1}) where compared, the accept_prob output: the same fp32 arithmetic as the rejection scans.
__device__ __forceinline__ float match_prob(const VerifyParams& p, const MatchRow& r) {
  return r.d >= 0 && int64_t(r.d) < p.V ? exp2_fast(fmaf(r.g, p.coef, -r.m)) / r.z : 0.f;
}

template <typename DT>
__global__ __launch_bounds__(kMatchThreads) void k_match(VerifyParams p) {
  __shared__ int32_t s_d[kMaxLen];     // d_{j+1} per row j < m
  __shared__ int32_t s_t[kMaxLen];     // the sample t_j of row j
  __shared__ float s_pk[kMaxLen];      // p_j(d_{j+1})
  __shared__ uint8_t s_near[kMaxLen];
  __shared__ uint32_t s_flags;
  __shared__ int s_r, s_stop;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  int64_t off0, len64;
  if (!chain_request(p, b, off0, len64)) {
    if (tid == 0) write_bad_offsets(p, b);
    if (p.cm_on && commit_arrive<kMatchThreads>(p, b, -1, nullptr)) fused_commit<kMatchThreads, false>(p);
    return;
  }
  const int len = int(len64);
  const int m = len - 1;
  const int64_t dr0 = off0 - b;
  if (tid == 0) {
    s_flags = 0;
    s_r = m;
    s_stop = 0;
  }

  // Rows in groups of 16 in row order, one wave per row (match_row). Until a group has held a mismatch
  // each row draws its sample; later groups still merge their partials (their status bits count).
  uint32_t fl = 0;
  bool stopped = false;
  for (int j0 = 0; j0 < len; j0 += kMatchWaves) {
    const int j = j0 + wv;
    if (j < len) {
      const MatchRow mr = match_row<DT>(p, b, j, off0, m, !stopped);
      if (lane == 0) {
        s_d[j] = mr.d;
        s_pk[j] = match_prob(p, mr);
        fl |= mr.f;
        if (!stopped) {
          s_t[j] = mr.t;
          s_near[j] = mr.near;
        }
      }
    }
    __syncthreads();
    if (!stopped && tid == 0) {
      for (int jj = j0; jj < min(len, j0 + kMatchWaves); ++jj) {
        const int32_t dd = s_d[jj];
        if (jj == m || !(dd >= 0 && int64_t(dd) < p.V && dd == s_t[jj])) {
          s_r = jj;
          s_stop = 1;
          break;
        }
      }
    }
    __syncthreads();
    stopped = s_stop != 0;
  }
  if (fl) atomicOr(&s_flags, fl);
  const int r = s_r;
  const int32_t bonus = s_t[r];
  uint32_t near = 0;
  for (int k = tid; k < len; k += kMatchThreads) {
    p.out_tokens[off0 + k] = k < r ? s_d[k] : (k == r ? bonus : -1);
    p.accept_index[off0 + k] = k <= r ? int32_t(off0 + k) : -1;
    if (k <= r && s_near[k]) near = SPEC_ST_NEAR_CDF;
    if (k < m && p.accept_prob) p.accept_prob[dr0 + k] = k <= r ? s_pk[k] : -1.f;
  }
  if (near) atomicOr(&s_flags, near);
  __syncthreads();
  if (tid == 0) {
    p.accept_len[b] = r;
    p.bonus[b] = bonus;
    p.status[b] = s_flags;
    if (p.residual_mass) p.residual_mass[b] = -1.f;
  }
  if (p.cm_on && commit_arrive<kMatchThreads>(p, b, r, nullptr)) fused_commit<kMatchThreads, false>(p);
}

// Sample-then-match on short requests (at most kMatchSplitMaxLen rows): workgroup g of request b draws rows
// 4g .. 4g + 3 (a wave each), so that a request's rows run on several compute units instead of sharing one;
// each row's result is published (agent-scope stores), and the request's last workgroup to count itself on
// the request's counter (reset by the logits stream of the same call) reads them, finds the first mismatch
// and writes the request's outputs, as k_match does.
template <typename DT>
__global__ __launch_bounds__(kThreads) void k_match_split(VerifyParams p) {
  constexpr int kRows = kThreads / kWave;
  __shared__ int s_last;
  __shared__ uint32_t s_flags;
  const int G = (p.L + kRows - 1) / kRows;
  const int b = int(blockIdx.x) / G;
  const int g = int(blockIdx.x) % G;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  int64_t off0, len64;
  if (!chain_request(p, b, off0, len64)) {   // every workgroup of b agrees; one reports it
    if (g == 0) {
      if (tid == 0) write_bad_offsets(p, b);
      if (p.cm_on && commit_arrive<kThreads>(p, b, -1, nullptr)) fused_commit<kThreads, false>(p);
    }
    return;
  }
  const int len = int(len64);
  const int m = len - 1;
  const int64_t dr0 = off0 - b;
  uint4* pub = p.mrow + size_t(b) * p.L;
  const int j = g * kRows + wv;
  if (j < len) {
    const MatchRow mr = match_row<DT>(p, b, j, off0, m, true);
    if (lane == 0) {
      const float pk = match_prob(p, mr);
      store_agent(reinterpret_cast<unsigned long long*>(pub + j),
                  (unsigned long long)uint32_t(mr.t) | ((unsigned long long)uint32_t(mr.d) << 32));
      store_agent(reinterpret_cast<unsigned long long*>(pub + j) + 1,
                  (unsigned long long)(mr.f | (mr.near ? SPEC_ST_NEAR_CDF : 0u)) |
                      ((unsigned long long)__float_as_uint(pk) << 32));
    }
  }
  complete_memory_ops();   // the published rows are stored before the workgroup is counted
  __syncthreads();
  if (tid == 0) s_last = uint32_t(atomicAdd(p.cnt2 + size_t(b) * kCounterWords, 1ull)) + 1u == uint32_t(G);
  __syncthreads();
  if (!s_last) return;

  // The request's last workgroup: wave 0 reads every row (a lane each; len <= 64).
  int r = m;
  if (tid < kWave) {
    const int k = lane;
    int32_t t = -1, d = -1;
    uint32_t f = 0;
    float pk = 0.f;
    if (k < len) {
      const unsigned long long w0 = load_agent(reinterpret_cast<unsigned long long*>(pub + k));
      const unsigned long long w1 = load_agent(reinterpret_cast<unsigned long long*>(pub + k) + 1);
      t = int32_t(uint32_t(w0));
      d = int32_t(uint32_t(w0 >> 32));
      f = uint32_t(w1);
      pk = __uint_as_float(uint32_t(w1 >> 32));
    }
    const uint64_t stop = __ballot(k < len && (k == m || !(d >= 0 && int64_t(d) < p.V && d == t)));
    r = stop ? __ffsll((unsigned long long)stop) - 1 : m;
    uint32_t fl = 0;
#pragma unroll
    for (uint32_t bit = 1; bit <= SPEC_ST_NEAR_CDF; bit <<= 1) {
      const bool any = bit == SPEC_ST_NEAR_CDF ? __ballot(k <= r && (f & bit)) : __ballot(k < len && (f & bit));
      if (any) fl |= bit;
    }
    const int32_t bonus = __shfl(t, r);
    if (k < len) {
      p.out_tokens[off0 + k] = k < r ? d : (k == r ? bonus : -1);
      p.accept_index[off0 + k] = k <= r ? int32_t(off0 + k) : -1;
      if (k < m && p.accept_prob) p.accept_prob[dr0 + k] = k <= r ? pk : -1.f;
    }
    if (k == 0) {
      p.accept_len[b] = r;
      p.bonus[b] = bonus;
      p.status[b] = fl;
      if (p.residual_mass) p.residual_mass[b] = -1.f;
      s_flags = uint32_t(r);
    }
  }
  __syncthreads();
  r = int(s_flags);
  if (p.cm_on && commit_arrive<kThreads>(p, b, r, nullptr)) fused_commit<kThreads, false>(p);
}

}  // namespace

hipError_t launch_match(int dtype, const VerifyParams& p, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (p.B <= 0) return hipSuccess;
  if (p.L <= kMatchSplitMaxLen) {
    constexpr int kRows = kThreads / kWave;
    const dim3 grid{unsigned(p.B * ((p.L + kRows - 1) / kRows))}, block{unsigned(kThreads)};
    if (dtype == SPEC_DTYPE_BF16) return launch_kernel(k_match_split<uint16_t>, grid, block, 0, stream, ev0, ev1, p);
    return launch_kernel(k_match_split<float>, grid, block, 0, stream, ev0, ev1, p);
  }
  const dim3 grid{unsigned(p.B)}, block{unsigned(kMatchThreads)};
  if (dtype == SPEC_DTYPE_BF16) return launch_kernel(k_match<uint16_t>, grid, block, 0, stream, ev0, ev1, p);
  return launch_kernel(k_match<float>, grid, block, 0, stream, ev0, ev1, p);
}

}  // namespace sv
