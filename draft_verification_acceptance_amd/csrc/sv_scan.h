// Request scans of libspecverify: merge a request's row partials and decide its accepted prefix.
//
//   chain greedy     d_{j+1} is accepted while it equals the lowest-index argmax of row j; the first
//                    mismatch (or row m) gives the bonus ([SpecDec] "为什么结果不受 draft 影响":
//                    verify_tree_greedy with one child per node; [EAGLE→DFlash2] §1.2)
//   chain rejection  alpha_j = min(1, p_j(d_{j+1}) / q_j(d_{j+1})), accepted iff u_j < alpha_j, up to the first
//                    rejection ([EAGLE→DFlash2] §1.2); sparse q: q_j(d) is the summed mass of the
//                    candidates with id d ([EAGLE→DFlash2] §6.5)
//   tree             walk down from the root taking the lowest-index child that matches the argmax (greedy)
//                    or whose cumulative sibling mass passes u (target-only) ([SpecDec], target-only
//                    sampling; a token already tried among earlier siblings adds nothing)
// Every scan reads memory in one round (the request's partials, staged in LDS, with its tokens and
// uniforms); the logits at the judged tokens of a chain arrive in the partials (read while the rows
// stream). A scan runs in one workgroup of kThreads threads: k_scan (greedy, one workgroup per request) or
// every k_draw workgroup of the request (sampling modes: each needs the scan's result to know which row
// to draw from, and recomputing it costs less than handing it over).
#pragma once

#include "sv_device.h"

namespace sv {

// Partials: stored by k_stats and read by a later kernel (k_scan or k_draw) on the same stream, so plain
// stores and loads suffice (the kernel boundary makes the stores visible on every XCD). Greedy rows use the
// first 16 bytes, sampling rows 24 (with the gathered logit and q(d)).
__device__ __forceinline__ void store_part(Part* dst, const Part& v, bool sampling) {
  uint4* d = reinterpret_cast<uint4*>(dst);
  d[0] = make_uint4(__float_as_uint(v.a), __float_as_uint(v.b), uint32_t(v.idx), v.flags);
  if (sampling) reinterpret_cast<uint2*>(d + 1)[0] = make_uint2(__float_as_uint(v.g), __float_as_uint(v.q));
}

__device__ __forceinline__ Part load_part(const Part* src, bool sampling) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  const uint4 w0 = s[0];
  const uint2 w1 = sampling ? reinterpret_cast<const uint2*>(s + 1)[0] : make_uint2(0u, 0u);
  Part r;
  r.a = __uint_as_float(w0.x);
  r.b = __uint_as_float(w0.y);
  r.idx = int32_t(w0.z);
  r.flags = w0.w;
  r.g = __uint_as_float(w1.x);
  r.q = __uint_as_float(w1.y);
  r.pad0 = r.pad1 = 0;
  return r;
}

// Row slots x parts x chunks of one request, if a scan stages them all in LDS (else 0).
__host__ __device__ __forceinline__ int staged_parts(int L, int P, int S) {
  const int n = L * P * S;
  return n <= kMaxStagedParts ? n : 0;
}

// Dynamic LDS of a scan: the staged partials, then its per-row arrays.
__host__ __device__ __forceinline__ size_t scan_smem_bytes(bool tree, bool sampling, int L, int P, int S) {
  const size_t per_row = tree ? 11 * 4 : (sampling ? 7 * 4 + 1 : 2 * 4);
  return size_t(staged_parts(L, P, S)) * sizeof(Part) + (per_row * size_t(L) + 15) / 16 * 16;
}

// The partials of one request, indexed (slot * P + part) * S + chunk: staged in LDS by the scan's load
// round, or read from the workspace when the launch shape has more than kMaxStagedParts per request.
struct ReqParts {
  const Part* lds;
  const Part* glob;
  bool sampling;
  __device__ __forceinline__ Part operator[](int i) const { return lds ? lds[i] : load_part(glob + i, sampling); }
};

// Merge the S chunk partials of one row in chunk order (deterministic).
__device__ __forceinline__ Part merge_greedy(const ReqParts& rp, int i0, int S) {
  Part r = rp[i0];
  for (int c = 1; c < S; ++c) {
    const Part q = rp[i0 + c];
    if (better(q.a, q.idx, r.a, r.idx)) { r.a = q.a; r.idx = q.idx; }
    r.flags |= q.flags;
  }
  return r;
}

// Sampling row: (m, z) merged in chunk order; g = the logit gathered by the chunk holding the judged token;
// q and the candidate flags come from chunk 0.
struct RowStats {
  float m, z, g, q;
  uint32_t flags;
};

__device__ __forceinline__ RowStats merge_sampling(const ReqParts& rp, int i0, int S) {
  const Part first = rp[i0];
  RowStats r{first.a, first.b, first.g, first.q, first.flags};
  for (int c = 1; c < S; ++c) {
    const Part q = rp[i0 + c];
    merge_mz(r.m, r.z, q.a, q.b);
    if (q.flags & kPartGathered) r.g = q.g;
    r.flags |= q.flags;
  }
  return r;
}

// A sampling row is usable iff its normaliser is a positive finite number (NaN: a NaN or +inf logit;
// 0: every logit is -inf).
__device__ __forceinline__ bool z_bad(float z) { return !(z > 0.f && z < INFINITY); }

// Request b of a chain batch: [off0, off0 + len) is usable iff its offsets pass the request's own checks
// (non-empty, at most L rows, and the bounds every valid batch meets that keep its draft rows inside
// [0, total_rows - B): off[b] >= b, off[b+1] <= total_rows - B + b + 1; off[0] = 0, off[B] = total_rows).
__device__ __forceinline__ bool chain_offsets_ok(const VerifyParams& p, int b, int64_t off0, int64_t off1) {
  bool ok = off0 >= b && off1 > off0 && off1 <= p.total_rows - p.B + b + 1 && off1 - off0 <= p.L;
  if (b == 0 && off0 != 0) ok = false;
  if (b == p.B - 1 && off1 != p.total_rows) ok = false;
  return ok;
}

__device__ __forceinline__ bool chain_request(const VerifyParams& p, int b, int64_t& off0, int64_t& len) {
  off0 = p.offsets[b];
  const int64_t off1 = p.offsets[b + 1];
  len = off1 - off0;
  return chain_offsets_ok(p, b, off0, off1);
}

// Outputs indexed by request for a request whose offsets fail their checks.
__device__ __forceinline__ void write_bad_offsets(const VerifyParams& p, int b) {
  p.status[b] = SPEC_ST_BAD_OFFSETS;
  p.accept_len[b] = 0;
  p.bonus[b] = -1;
  if (p.residual_mass) p.residual_mass[b] = -1.f;
}

// What the final draw of a sampling request needs (the result of its scan).
struct DrawPlan {
  int32_t row_t;        // global target row the token is drawn from
  int32_t row_q;        // draft row of the residual [p - q]_+ (logits, or sparse candidates), or -1 (from p)
  int32_t out_pos;      // out_tokens index of the drawn token
  float m_t, z_t;       // target row: max m (log2 units) and normaliser z of softmax = exp2(x*coef - m) / z
  float m_q, z_q;       // draft row, same meaning (dense rejection)
  float u;              // sanitized u_final
  uint32_t status;      // request status bits of the scan
  int32_t n_seen;       // tree target-only: tokens excluded from the draw (listed in `seen`, LDS)
  const int32_t* seen;
  int32_t r;            // accepted drafts
  const int32_t* path;  // tree: the accepted path's node indices, root first (LDS); chain: NULL
};

// Load round of a chain scan: the request's n partials (when staged) and its n_tok draft tokens and
// uniforms, every load issued before any is waited for. Ends with a workgroup barrier.
__device__ __forceinline__ void chain_load_round(const VerifyParams& p, const Part* gp, int n, Part* stage,
                                                 bool sampling, int64_t tok0, int n_tok, int32_t* s_d,
                                                 float* s_u) {
  const int cnt = max(stage ? n : 0, n_tok);
  for (int i = threadIdx.x; i < cnt; i += kThreads) {
    const bool hp = stage && i < n;
    const bool ht = i < n_tok;
    Part pt{};
    int32_t d = 0;
    float u = 0.f;
    if (hp) pt = load_part(gp + i, sampling);
    if (ht) {
      d = p.draft_tokens[tok0 + i];
      if (s_u) u = p.u_accept[tok0 + i];
    }
    if (hp) stage[i] = pt;
    if (ht) {
      s_d[i] = d;
      if (s_u) s_u[i] = u;
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------------------------------
// Chain greedy: writes every output of request b.
// ---------------------------------------------------------------------------------------------------
__device__ int scan_chain_greedy(const VerifyParams& p, int b, int64_t off0, int len, char* smem, Part* stage) {
  __shared__ int s_red[kThreads / kWave];
  __shared__ uint32_t s_flags;
  const int tid = threadIdx.x;
  const int m = len - 1;
  const int64_t dr0 = off0 - b;
  int* s_arg = reinterpret_cast<int*>(smem);
  int32_t* s_d = s_arg + p.L;
  const Part* gp = p.part + size_t(b) * p.L * p.S;
  if (tid == 0) s_flags = 0;
  chain_load_round(p, gp, len * p.S, stage, false, dr0, m, s_d, nullptr);
  const ReqParts rp{stage, gp, false};
  uint32_t fl = 0;
  int fail = INT32_MAX;
  for (int j = tid; j < len; j += kThreads) {
    const Part r = merge_greedy(rp, j * p.S, p.S);
    s_arg[j] = r.idx;
    if (r.flags & kPartNaN) fl |= SPEC_ST_NONFINITE;
    if (p.mask && r.a == -INFINITY) fl |= SPEC_ST_NONFINITE;   // the mask left no finite logit
    if (j < m) {   // test of d_{j+1} against row j
      const int32_t d = s_d[j];
      const bool ok = d >= 0 && int64_t(d) < p.V;
      if (!ok) fl |= SPEC_ST_BAD_TOKEN;
      if (!ok || d != r.idx) fail = min(fail, j);
    }
  }
  if (fl) atomicOr(&s_flags, fl);
  fail = block_min_i(fail, s_red);
  const int r = min(fail, m);
  const int32_t bonus = s_arg[r];
  for (int k = tid; k < len; k += kThreads) {
    p.out_tokens[off0 + k] = k < r ? s_d[k] : (k == r ? bonus : -1);
    p.accept_index[off0 + k] = k <= r ? int32_t(off0 + k) : -1;
  }
  if (p.accept_prob)
    for (int j = tid; j < m; j += kThreads) p.accept_prob[dr0 + j] = -1.f;
  if (tid == 0) {
    p.accept_len[b] = r;
    p.bonus[b] = bonus;
    p.status[b] = s_flags;
    if (p.residual_mass) p.residual_mass[b] = -1.f;
  }
  return r;
}

// ---------------------------------------------------------------------------------------------------
// Chain rejection, dense (q from draft logits) or SPARSE (q from K candidate (id, probability) pairs per draft
// row, zero off the candidates). Writes the outputs known before the draw iff write_out; returns the plan.
// ---------------------------------------------------------------------------------------------------
template <bool SPARSE>
__device__ DrawPlan scan_chain_rejection(const VerifyParams& p, int b, int64_t off0, int len, char* smem,
                                         Part* stage, bool write_out) {
  __shared__ int s_red[kThreads / kWave];
  __shared__ uint32_t s_flags;
  __shared__ float s_uf;
  const int tid = threadIdx.x;
  const int m = len - 1;
  const int64_t dr0 = off0 - b;
  const int L = p.L;
  const int PS = p.P * p.S;
  float* s_mt = reinterpret_cast<float*>(smem);
  float* s_zt = s_mt + L;
  float* s_mq = s_zt + L;
  float* s_zq = s_mq + L;
  float* s_a = s_zq + L;
  float* s_u = s_a + L;
  int32_t* s_d = reinterpret_cast<int32_t*>(s_u + L);
  uint8_t* s_acc = reinterpret_cast<uint8_t*>(s_d + L);   // bit0 accepted, bit1 near, bit2 q == 0
  const Part* gp = p.part + size_t(b) * L * PS;
  if (tid == 0) s_flags = 0;
  const float uf_raw = p.u_final[b];   // one address for the workgroup, in flight with the load round
  chain_load_round(p, gp, len * PS, stage, true, dr0, m, s_d, s_u);
  const ReqParts rp{stage, gp, true};
  if (len <= kWave) {
    // A lane per row in wave 0, the same arithmetic as below: the first failure, the flags and the plan's
    // row values come from ballots and lane reads, and one barrier hands the plan to the other waves.
    __shared__ DrawPlan s_plan;
    if (tid < kWave) {
      const int j = tid;
      uint32_t f = 0;
      float a = 0.f;
      bool acc = false, near = false, zq = false;
      RowStats t{0.f, 1.f, 0.f, 0.f, 0u}, qr{0.f, 1.f, 0.f, 0.f, 0u};
      int32_t d = 0;
      if (j < len) {
        t = merge_sampling(rp, j * PS, p.S);
        if (z_bad(t.z)) f |= SPEC_ST_NONFINITE;
      }
      if (j < m) {
        if (!SPARSE) {
          qr = merge_sampling(rp, j * PS + p.S, p.S);
          if (z_bad(qr.z)) f |= SPEC_ST_NONFINITE;
        } else {
          if (t.flags & kPartBadCandId) f |= SPEC_ST_BAD_TOKEN;
          if (t.flags & kPartBadCandQ) f |= SPEC_ST_BAD_Q;
        }
        d = s_d[j];
        const bool ok = d >= 0 && int64_t(d) < p.V;
        if (!ok) f |= SPEC_ST_BAD_TOKEN;
        bool ubad = false;
        const float u = sanitize_u(s_u[j], ubad);
        if (ubad) f |= SPEC_ST_BAD_UNIFORM;
        if (ok && SPARSE) {
          const float qd = t.q;
          if (!(qd > 0.f)) {
            zq = true;
            a = t.g > -INFINITY ? 1.f : 0.f;
          } else {
            a = fminf(1.f, exp2_fast(fmaf(t.g, p.coef, -t.m)) / (t.z * qd));
          }
        } else if (ok) {
          if (qr.g == -INFINITY) {
            zq = true;
            a = t.g > -INFINITY ? 1.f : 0.f;
          } else {
            const float et = fmaf(t.g, p.coef, -t.m);
            const float eq = fmaf(qr.g, p.coef, -qr.m);
            a = fminf(1.f, exp2_fast(et - eq) * (qr.z / t.z));
          }
        }
        acc = u < a;
        near = fabsf(u - a) < kNear;
      }
      const uint64_t fails = __ballot(j < m && !acc);
      const int r = fails ? min(__ffsll((unsigned long long)fails) - 1, m) : m;
      const float mt = __shfl(t.m, r), zt = __shfl(t.z, r), mq = __shfl(qr.m, r), zqr = __shfl(qr.z, r);
      const bool examined = j < m && j <= r;
      uint32_t fl = 0;
#pragma unroll
      for (uint32_t bit = 1; bit <= SPEC_ST_BAD_Q; bit <<= 1)
        if (__ballot(f & bit)) fl |= bit;
      if (__ballot(examined && near)) fl |= SPEC_ST_NEAR_ALPHA;
      if (__ballot(examined && zq)) fl |= SPEC_ST_ZERO_Q;
      bool ubad = false;
      const float uf = sanitize_u(uf_raw, ubad);
      if (ubad) fl |= SPEC_ST_BAD_UNIFORM;
      if (write_out) {
        if (p.accept_prob && j < m) p.accept_prob[dr0 + j] = examined ? a : -1.f;
        // out_tokens[off0 + r] belongs to the draw's last workgroup, possibly on another XCD: no other
        // workgroup may store to it.
        if (j < len) {
          if (j != r) p.out_tokens[off0 + j] = j < r ? d : -1;
          p.accept_index[off0 + j] = j <= r ? int32_t(off0 + j) : -1;
        }
        if (j == 0) p.accept_len[b] = r;
      }
      if (j == 0) {
        DrawPlan pl;
        pl.row_t = int32_t(off0 + r);
        pl.row_q = r < m ? int32_t(dr0 + r) : -1;
        pl.out_pos = int32_t(off0 + r);
        pl.m_t = mt;
        pl.z_t = zt;
        pl.m_q = r < m && !SPARSE ? mq : 0.f;
        pl.z_q = r < m && !SPARSE ? zqr : 1.f;
        pl.u = uf;
        pl.status = fl;
        pl.n_seen = 0;
        pl.seen = nullptr;
        pl.r = r;
        pl.path = nullptr;
        s_plan = pl;
      }
    }
    __syncthreads();
    return s_plan;
  }
  uint32_t fl = 0;
  int fail = INT32_MAX;
  for (int j = tid; j < len; j += kThreads) {
    const RowStats t = merge_sampling(rp, j * PS, p.S);
    s_mt[j] = t.m;
    s_zt[j] = t.z;
    if (z_bad(t.z)) fl |= SPEC_ST_NONFINITE;
    if (j >= m) continue;
    RowStats q{0.f, 1.f, 0.f, 0.f, 0u};
    if (!SPARSE) {
      q = merge_sampling(rp, j * PS + p.S, p.S);
      if (z_bad(q.z)) fl |= SPEC_ST_NONFINITE;
    } else {
      if (t.flags & kPartBadCandId) fl |= SPEC_ST_BAD_TOKEN;
      if (t.flags & kPartBadCandQ) fl |= SPEC_ST_BAD_Q;
    }
    s_mq[j] = q.m;
    s_zq[j] = q.z;
    const int32_t d = s_d[j];
    const bool ok = d >= 0 && int64_t(d) < p.V;
    if (!ok) fl |= SPEC_ST_BAD_TOKEN;
    bool ubad = false;
    const float u = sanitize_u(s_u[j], ubad);
    if (ubad) fl |= SPEC_ST_BAD_UNIFORM;
    float a = 0.f;
    uint8_t bits = 0;
    if (ok && SPARSE) {
      const float qd = t.q;        // q(d): the masses of the valid candidate entries with id d
      if (!(qd > 0.f)) {           // q(d) = 0: alpha = 1 if p(d) > 0 else 0
        bits |= 4;
        a = t.g > -INFINITY ? 1.f : 0.f;
      } else {
        a = fminf(1.f, exp2_fast(fmaf(t.g, p.coef, -t.m)) / (t.z * qd));
      }
    } else if (ok) {
      if (q.g == -INFINITY) {      // q(d) = 0: alpha = 1 if p(d) > 0 else 0
        bits |= 4;
        a = t.g > -INFINITY ? 1.f : 0.f;
      } else {
        // alpha = min(1, p(d)/q(d)) with p(d) = exp2(gt*c - m_t)/z_t, q(d) = exp2(gq*c - m_q)/z_q
        const float et = fmaf(t.g, p.coef, -t.m);
        const float eq = fmaf(q.g, p.coef, -q.m);
        a = fminf(1.f, exp2_fast(et - eq) * (q.z / t.z));
      }
    }
    if (u < a) bits |= 1;
    else fail = min(fail, j);
    if (fabsf(u - a) < kNear) bits |= 2;
    s_a[j] = a;
    s_acc[j] = bits;
  }
  fail = block_min_i(fail, s_red);   // contains __syncthreads
  const int r = min(fail, m);
  for (int j = tid; j < m; j += kThreads) {
    const bool examined = j <= r;
    if (examined && (s_acc[j] & 2)) fl |= SPEC_ST_NEAR_ALPHA;
    if (examined && (s_acc[j] & 4)) fl |= SPEC_ST_ZERO_Q;
    if (write_out && p.accept_prob) p.accept_prob[dr0 + j] = examined ? s_a[j] : -1.f;
  }
  if (tid == 0) {
    bool ubad = false;
    s_uf = sanitize_u(uf_raw, ubad);
    if (ubad) fl |= SPEC_ST_BAD_UNIFORM;
  }
  if (fl) atomicOr(&s_flags, fl);
  if (write_out) {
    // out_tokens[off0 + r] belongs to the draw's last workgroup, possibly on another XCD: no other
    // workgroup may store to it.
    for (int k = tid; k < len; k += kThreads) {
      if (k != r) p.out_tokens[off0 + k] = k < r ? s_d[k] : -1;
      p.accept_index[off0 + k] = k <= r ? int32_t(off0 + k) : -1;
    }
    if (tid == 0) p.accept_len[b] = r;
  }
  __syncthreads();
  DrawPlan d;
  d.row_t = int32_t(off0 + r);
  d.row_q = r < m ? int32_t(dr0 + r) : -1;
  d.out_pos = int32_t(off0 + r);
  d.m_t = s_mt[r];
  d.z_t = s_zt[r];
  d.m_q = r < m && !SPARSE ? s_mq[r] : 0.f;
  d.z_q = r < m && !SPARSE ? s_zq[r] : 1.f;
  d.u = s_uf;
  d.status = s_flags;
  d.n_seen = 0;
  d.seen = nullptr;
  d.r = r;
  d.path = nullptr;
  return d;
}

// ---------------------------------------------------------------------------------------------------
// Tree walk. Children are examined in ascending node index. Greedy: writes every output. Target-only:
// writes the outputs known before the draw iff write_out and returns the plan (the tried tokens of the
// final node stay in LDS).
// ---------------------------------------------------------------------------------------------------
template <typename DT, bool SAMPLING>
__device__ DrawPlan scan_tree(const VerifyParams& p, int b, char* smem, Part* stage, bool write_out) {
  __shared__ uint32_t s_flags;
  __shared__ int s_path_len;
  __shared__ int s_cur;
  __shared__ int s_nseen;
  const int tid = threadIdx.x;
  const int N = p.L;
  const int64_t base = int64_t(b) * N;
  int32_t* s_par = reinterpret_cast<int32_t*>(smem);     // parent, or -2 when the node is nobody's child
  int32_t* s_tok = s_par + N;                             // token, or -1 when out of range
  int32_t* s_arg = s_tok + N;                             // greedy: argmax of the node's row
  float* s_m = reinterpret_cast<float*>(s_arg + N);       // sampling: row max (log2 units)
  float* s_z = s_m + N;                                   // sampling: row normaliser
  float* s_pv = s_z + N;                                  // sampling: p_parent(token) of each node
  float* s_prob = s_pv + N;                               // accept_prob output staging
  float* s_u = s_prob + N;                                // sanitized u_accept per node
  int32_t* s_path = reinterpret_cast<int32_t*>(s_u + N);
  int32_t* s_list = s_path + N;                           // children of the current node (ascending)
  int32_t* s_seen = s_list + N;                           // distinct tokens tried at the current node
  const Part* gp = p.part + size_t(b) * N * p.S;
  if (tid == 0) { s_flags = 0; s_nseen = 0; }
  const float uf_raw = SAMPLING ? p.u_final[b] : 0.f;   // in flight with the load round
  // Load round: partials (when staged), parents, tokens and uniforms.
  {
    const int np = N * p.S;
    const int cnt = max(stage ? np : 0, N);
    for (int i = tid; i < cnt; i += kThreads) {
      const bool hp = stage && i < np;
      const bool hn = i < N;
      Part pt{};
      int32_t par = 0, tok = 0;
      float u = 0.f;
      if (hp) pt = load_part(gp + i, SAMPLING);
      if (hn) {
        par = p.parents[base + i];
        tok = p.tokens[base + i];
        if (SAMPLING) u = p.u_accept[base + i];
      }
      if (hp) stage[i] = pt;
      if (hn) {
        s_par[i] = par;
        s_tok[i] = tok;
        s_u[i] = u;
      }
    }
    __syncthreads();
  }
  const ReqParts rp{stage, gp, SAMPLING};
  uint32_t fl = 0;
  for (int i = tid; i < N; i += kThreads) {
    if (SAMPLING) {
      const RowStats r = merge_sampling(rp, i * p.S, p.S);
      s_m[i] = r.m;
      s_z[i] = r.z;
      if (z_bad(r.z)) fl |= SPEC_ST_NONFINITE;
      bool ubad = false;
      s_u[i] = sanitize_u(s_u[i], ubad);
      if (ubad) fl |= SPEC_ST_BAD_UNIFORM;
    } else {
      const Part r = merge_greedy(rp, i * p.S, p.S);
      s_arg[i] = r.idx;
      if (r.flags & kPartNaN) fl |= SPEC_ST_NONFINITE;
      if (p.mask && r.a == -INFINITY) fl |= SPEC_ST_NONFINITE;   // the mask left no finite logit
    }
    const int32_t par = s_par[i];
    const int32_t tok = s_tok[i];
    if (i == 0) {
      if (par != -1) fl |= SPEC_ST_BAD_PARENT;
      s_par[0] = -2;
    } else {
      const bool pok = par >= 0 && par < i;
      if (!pok) fl |= SPEC_ST_BAD_PARENT;
      const bool tok_ok = tok >= 0 && int64_t(tok) < p.V;
      if (!tok_ok) fl |= SPEC_ST_BAD_TOKEN;
      s_par[i] = pok ? par : -2;
      s_tok[i] = tok_ok ? tok : -1;
    }
    s_prob[i] = -1.f;
  }
  __syncthreads();
  if (SAMPLING) {
    // p_parent(token) for every valid child (one parallel round of gathers).
    for (int i = tid; i < N; i += kThreads) {
      const int32_t par = s_par[i];
      const int32_t tok = s_tok[i];
      float pv = 0.f;
      if (i > 0 && par >= 0 && tok >= 0) {
        float g = Elem<DT>::load(static_cast<const DT*>(p.target) + (base + par) * p.V, tok);
        if (p.mask && !mask_allows(p.mask + (base + par) * p.mask_words, tok)) g = -INFINITY;
        pv = exp2_fast(fmaf(g, p.coef, -s_m[par])) / s_z[par];
      }
      s_pv[i] = pv;
    }
    __syncthreads();
  }
  // The walk itself: wave 0, one lane per candidate child.
  if (tid < kWave) {
    const int lane = tid;
    int cur = 0;
    int plen = 1;
    if (lane == 0) s_path[0] = 0;
    uint32_t wfl = 0;
    while (true) {
      int next = -1;
      if (!SAMPLING) {
        const int32_t want = s_arg[cur];
        for (int c0 = cur + 1; c0 < N && next < 0; c0 += kWave) {
          const int c = c0 + lane;
          const bool hit = c < N && s_par[c] == cur && s_tok[c] == want;
          const uint64_t mask = __ballot(hit);
          if (mask) next = c0 + __ffsll((unsigned long long)mask) - 1;
        }
      } else {
        // Collect the valid children of cur in ascending order.
        int nch = 0;
        for (int c0 = cur + 1; c0 < N; c0 += kWave) {
          const int c = c0 + lane;
          const bool isc = c < N && s_par[c] == cur && s_tok[c] >= 0;
          const uint64_t mask = __ballot(isc);
          if (isc) s_list[nch + __popcll(mask & lanes_below(lane))] = c;
          nch += __popcll(mask);
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        const float u = s_u[cur];
        float carry = 0.f;
        int nseen = 0;
        for (int i0 = 0; i0 < nch && next < 0; i0 += kWave) {
          const int i = i0 + lane;
          bool fresh = false;
          int c = -1;
          int32_t t = -1;
          if (i < nch) {
            c = s_list[i];
            t = s_tok[c];
            fresh = true;
            for (int j = 0; j < i; ++j)
              if (s_tok[s_list[j]] == t) { fresh = false; break; }
          }
          const float mass = fresh ? s_pv[c] : 0.f;
          const float acc = carry + wave_inclusive_sum(mass);
          const bool take = fresh && u < acc;
          const uint64_t tmask = __ballot(take);
          const int first = tmask ? __ffsll((unsigned long long)tmask) - 1 : kWave;
          // children up to (and including) the accepted one were examined
          if (fresh && lane <= first) {
            s_prob[c] = acc;
            if (fabsf(u - acc) < kNear) wfl |= SPEC_ST_NEAR_ALPHA;
          }
          const uint64_t fmask = __ballot(fresh && lane <= first);
          if (fresh && lane <= first) s_seen[nseen + __popcll(fmask & lanes_below(lane))] = t;
          nseen += __popcll(fmask);
          if (tmask) next = __shfl(c, first);
          carry = __shfl(acc, kWave - 1);
        }
        if (lane == 0) s_nseen = next < 0 ? nseen : 0;
      }
      if (next < 0) break;
      cur = next;
      if (lane == 0) s_path[plen] = cur;
      ++plen;
    }
    if (lane == 0) {
      s_path_len = plen;
      s_cur = cur;
    }
    fl |= wfl;
  }
  if (fl) atomicOr(&s_flags, fl);
  __syncthreads();
  const int r = s_path_len - 1;
  const int cur = s_cur;
  int32_t bonus = -1;
  if (!SAMPLING) bonus = s_arg[cur];
  if (write_out) {
    for (int k = tid; k < N; k += kThreads) {
      // target-only: out_tokens[base + r] belongs to the draw's last workgroup (no other store to it)
      if (!SAMPLING || k != r) p.out_tokens[base + k] = k < r ? s_tok[s_path[k + 1]] : (k == r ? bonus : -1);
      p.accept_index[base + k] = k <= r ? int32_t(base + s_path[k]) : -1;
      if (p.accept_prob) p.accept_prob[base + k] = s_prob[k];
    }
    if (tid == 0) {
      p.accept_len[b] = r;
      if (!SAMPLING) {
        p.bonus[b] = bonus;
        p.status[b] = s_flags;
        if (p.residual_mass) p.residual_mass[b] = -1.f;
      }
    }
  }
  DrawPlan d;
  d.row_t = int32_t(base + cur);
  d.row_q = -1;
  d.out_pos = int32_t(base + r);
  d.m_t = SAMPLING ? s_m[cur] : 0.f;
  d.z_t = SAMPLING ? s_z[cur] : 1.f;
  d.m_q = 0.f;
  d.z_q = 1.f;
  d.u = 0.f;
  d.status = s_flags;
  d.n_seen = SAMPLING ? s_nseen : 0;
  d.seen = s_seen;
  d.r = r;
  d.path = s_path;
  if (SAMPLING) {
    bool ubad = false;
    d.u = sanitize_u(uf_raw, ubad);
    if (ubad) d.status |= SPEC_ST_BAD_UNIFORM;
  }
  return d;
}

}  // namespace sv
