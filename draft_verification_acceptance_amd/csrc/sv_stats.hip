// k_stats: one streaming pass over every verify row (target, and draft rows in rejection mode), fused with
// the per-request accept scan (chains) or tree walk, run by the workgroup that finishes a request last.
//
// What is computed per row (the verify step scores all positions in one parallel pass; the rows after the
// first rejection are read too: [EAGLE→DFlash2] §1.1, [SpecDec] "抽象：draft → verify → commit"):
//   greedy    argmax with the lowest index among equal maxima ([SpecDec] "为什么结果不受 draft 影响":
//             verify_tree_greedy; [EAGLE→DFlash2] §1.2: same numerics and tie-breaking as plain greedy)
//   sampling  m = max(x) * log2(e)/T and z = sum exp2(x * log2(e)/T - m), i.e. softmax(x / T) = exp2(x*c - m)/z
//             ([EAGLE→DFlash2] §1.2: p_j and q_j are the distributions actually used).
#include "sv_device.h"

namespace sv {

namespace {

constexpr int kUnroll = 4;   // 16-byte loads in flight per thread per loop trip

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

// Greedy partial of row[lo, hi) reduced over the workgroup (result valid in thread 0).
template <typename DT>
__device__ void chunk_argmax(const DT* __restrict__ row, int64_t lo, int64_t hi, Part& out, float* red_f,
                             int* red_i, uint32_t* red_u) {
  constexpr int E = Elem<DT>::kPerVec;
  const int tid = threadIdx.x;
  const Split sp = split_chunk(row, lo, hi);
  const uint4* __restrict__ vp = reinterpret_cast<const uint4*>(row + sp.body_lo);

  float best = -INFINITY;
  int64_t bestk = tid < sp.nvec ? tid : -1;
  bool nan = false;
  int64_t k = tid;
  for (; k + (kUnroll - 1) * kThreads < sp.nvec; k += kUnroll * kThreads) {
    uint4 q[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = load_stream(vp + k + u * kThreads);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float x[E];
      Elem<DT>::unpack(q[u], x);
      float vm = x[0];
#pragma unroll
      for (int e = 1; e < E; ++e) vm = fmaxf(vm, x[e]);
#pragma unroll
      for (int e = 0; e < E; e += 2) nan |= __builtin_isunordered(x[e], x[e + 1]);
      if (vm > best) {
        best = vm;
        bestk = k + u * kThreads;
      }
    }
  }
  for (; k < sp.nvec; k += kThreads) {
    float x[E];
    Elem<DT>::unpack(load_stream(vp + k), x);
    float vm = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) vm = fmaxf(vm, x[e]);
#pragma unroll
    for (int e = 0; e < E; e += 2) nan |= __builtin_isunordered(x[e], x[e + 1]);
    if (vm > best) {
      best = vm;
      bestk = k;
    }
  }
  int32_t idx = INT32_MAX;
  if (bestk >= 0) {  // recover the lowest index of the thread's maximum inside its winning vector
    float x[E];
    Elem<DT>::unpack(vp[bestk], x);
#pragma unroll
    for (int e = E - 1; e >= 0; --e)
      if (x[e] == best) idx = int32_t(sp.body_lo + bestk * E + e);
  }
  if (tid < sp.head) {
    const int64_t i = lo + tid;
    const float v = Elem<DT>::load(row, i);
    if (v != v) nan = true;
    else if (better(v, int32_t(i), best, idx)) { best = v; idx = int32_t(i); }
  }
  if (tid < hi - sp.body_hi) {
    const int64_t i = sp.body_hi + tid;
    const float v = Elem<DT>::load(row, i);
    if (v != v) nan = true;
    else if (better(v, int32_t(i), best, idx)) { best = v; idx = int32_t(i); }
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
    for (int i = 1; i < kThreads / kWave; ++i) {
      if (better(red_f[i], red_i[i], bv, bi)) { bv = red_f[i]; bi = red_i[i]; }
      fl |= red_u[i];
    }
    out.a = bv;
    out.b = 0.f;
    out.idx = bi;
    out.flags = fl;
  }
}

// Sampling partial of row[lo, hi): (m, z) with m in log2 units, reduced over the workgroup (thread 0).
template <typename DT>
__device__ void chunk_lse(const DT* __restrict__ row, int64_t lo, int64_t hi, float coef, Part& out, float* red_f,
                          float* red_g) {
  constexpr int E = Elem<DT>::kPerVec;
  const int tid = threadIdx.x;
  const Split sp = split_chunk(row, lo, hi);
  const uint4* __restrict__ vp = reinterpret_cast<const uint4*>(row + sp.body_lo);

  float m = -INFINITY, z = 0.f;
  int64_t k = tid;
  for (; k + (kUnroll - 1) * kThreads < sp.nvec; k += kUnroll * kThreads) {
    uint4 q[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) q[u] = load_stream(vp + k + u * kThreads);
    float x[kUnroll * E];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) Elem<DT>::unpack(q[u], x + u * E);
    float vm = x[0];
#pragma unroll
    for (int e = 1; e < kUnroll * E; ++e) vm = fmaxf(vm, x[e]);
    const float mn = fmaxf(m, vm * coef);
    z *= (mn == m) ? 1.f : exp2_fast(m - mn);
    m = mn;
    const float nm = (m == -INFINITY) ? 0.f : -m;
#pragma unroll
    for (int e = 0; e < kUnroll * E; ++e) z += exp2_fast(fmaf(x[e], coef, nm));
  }
  for (; k < sp.nvec; k += kThreads) {
    float x[E];
    Elem<DT>::unpack(load_stream(vp + k), x);
    float vm = x[0];
#pragma unroll
    for (int e = 1; e < E; ++e) vm = fmaxf(vm, x[e]);
    const float mn = fmaxf(m, vm * coef);
    z *= (mn == m) ? 1.f : exp2_fast(m - mn);
    m = mn;
    const float nm = (m == -INFINITY) ? 0.f : -m;
#pragma unroll
    for (int e = 0; e < E; ++e) z += exp2_fast(fmaf(x[e], coef, nm));
  }
  if (tid < sp.head) {
    const float x = Elem<DT>::load(row, lo + tid);
    float m2 = x * coef, z2 = 1.f;
    if (x != x) { m2 = -INFINITY; z2 = x; }            // NaN poisons the sum
    else if (m2 == -INFINITY) z2 = 0.f;
    else if (m2 == INFINITY) z2 = __builtin_nanf("");  // +inf: softmax undefined
    merge_mz(m, z, m2, z2);
  }
  if (tid < hi - sp.body_hi) {
    const float x = Elem<DT>::load(row, sp.body_hi + tid);
    float m2 = x * coef, z2 = 1.f;
    if (x != x) { m2 = -INFINITY; z2 = x; }
    else if (m2 == -INFINITY) z2 = 0.f;
    else if (m2 == INFINITY) z2 = __builtin_nanf("");
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
    for (int i = 1; i < kThreads / kWave; ++i) merge_mz(M, Z, red_f[i], red_g[i]);
    out.a = M;
    out.b = Z;
    out.idx = 0;
    out.flags = 0;
  }
}

template <typename DT>
__device__ __forceinline__ float gather(const void* base, int64_t row, int64_t V, int64_t col) {
  return Elem<DT>::load(static_cast<const DT*>(base) + row * V, col);
}

// Partials are published and read as two agent-scope 64-bit atomics (see complete_memory_ops).
__device__ __forceinline__ void store_part(Part* dst, const Part& v) {
  unsigned long long* d = reinterpret_cast<unsigned long long*>(dst);
  store_agent(d, (unsigned long long)__float_as_uint(v.a) | ((unsigned long long)__float_as_uint(v.b) << 32));
  store_agent(d + 1, (unsigned long long)uint32_t(v.idx) | ((unsigned long long)v.flags << 32));
}

__device__ __forceinline__ Part load_part(const Part* src) {
  unsigned long long* s = reinterpret_cast<unsigned long long*>(const_cast<Part*>(src));
  const unsigned long long w0 = load_agent(s);
  const unsigned long long w1 = load_agent(s + 1);
  Part r;
  r.a = __uint_as_float(uint32_t(w0));
  r.b = __uint_as_float(uint32_t(w0 >> 32));
  r.idx = int32_t(uint32_t(w1));
  r.flags = uint32_t(w1 >> 32);
  return r;
}

// Merge the S partials of one row slot.
__device__ __forceinline__ Part merge_greedy(const Part* p, int S) {
  Part r = load_part(p);
  for (int c = 1; c < S; ++c) {
    const Part q = load_part(p + c);
    if (better(q.a, q.idx, r.a, r.idx)) { r.a = q.a; r.idx = q.idx; }
    r.flags |= q.flags;
  }
  return r;
}

__device__ __forceinline__ void merge_sampling(const Part* p, int S, float& m, float& z) {
  const Part first = load_part(p);
  m = first.a;
  z = first.b;
  for (int c = 1; c < S; ++c) {
    const Part q = load_part(p + c);
    merge_mz(m, z, q.a, q.b);
  }
}

// A sampling row is usable iff its normaliser is a positive finite number (NaN: a NaN or +inf logit;
// 0: every logit is -inf).
__device__ __forceinline__ bool z_bad(float z) { return !(z > 0.f && z < INFINITY); }

// ---------------------------------------------------------------------------------------------------
// Chain scans (run by the last workgroup of request b).
// ---------------------------------------------------------------------------------------------------
template <typename DT>
__device__ void scan_chain_greedy(const StatsParams& p, int b, int64_t off0, int len, char* smem) {
  __shared__ int s_red[kThreads / kWave];
  __shared__ uint32_t s_flags;
  const int tid = threadIdx.x;
  const int m = len - 1;
  const int64_t dr0 = off0 - b;
  int* s_arg = reinterpret_cast<int*>(smem);
  if (tid == 0) s_flags = 0;
  __syncthreads();
  uint32_t fl = 0;
  for (int j = tid; j < len; j += kThreads) {
    const Part r = merge_greedy(p.part + (size_t(b) * p.L + j) * p.P * p.S, p.S);
    s_arg[j] = r.idx;
    if (r.flags) fl |= SPEC_ST_NONFINITE;
  }
  int fail = INT32_MAX;
  __syncthreads();
  for (int j = tid; j < m; j += kThreads) {  // test of d_{j+1} against row j
    const int32_t d = p.draft_tokens[dr0 + j];
    const bool ok = d >= 0 && int64_t(d) < p.V;
    if (!ok) fl |= SPEC_ST_BAD_TOKEN;
    if (!ok || d != s_arg[j]) fail = min(fail, j);
  }
  if (fl) atomicOr(&s_flags, fl);
  fail = block_min_i(fail, s_red);
  const int r = min(fail, m);
  const int32_t bonus = s_arg[r];
  for (int k = tid; k < len; k += kThreads) {
    p.out_tokens[off0 + k] = k < r ? p.draft_tokens[dr0 + k] : (k == r ? bonus : -1);
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
}

// Dense rejection (q from draft logits) or SPARSE (q from K candidate (id, probability) pairs per draft row,
// zero off the candidates: [EAGLE→DFlash2] §6.5).
template <typename DT, bool SPARSE>
__device__ void scan_chain_rejection(const StatsParams& p, int b, int64_t off0, int len, char* smem) {
  __shared__ int s_red[kThreads / kWave];
  __shared__ uint32_t s_flags;
  const int tid = threadIdx.x;
  const int m = len - 1;
  const int64_t dr0 = off0 - b;
  const int L = p.L;
  float* s_mt = reinterpret_cast<float*>(smem);
  float* s_zt = s_mt + L;
  float* s_mq = s_zt + L;
  float* s_zq = s_mq + L;
  float* s_a = s_zq + L;
  uint8_t* s_acc = reinterpret_cast<uint8_t*>(s_a + L);   // bit0 accepted, bit1 near, bit2 q == 0
  if (tid == 0) s_flags = 0;
  __syncthreads();
  uint32_t fl = 0;
  for (int j = tid; j < len; j += kThreads) {
    float mm, zz;
    merge_sampling(p.part + (size_t(b) * p.L + j) * p.P * p.S, p.S, mm, zz);
    s_mt[j] = mm;
    s_zt[j] = zz;
    if (z_bad(zz)) fl |= SPEC_ST_NONFINITE;
  }
  if (!SPARSE) {
    for (int j = tid; j < m; j += kThreads) {
      float mm, zz;
      merge_sampling(p.part + ((size_t(b) * p.L + j) * p.P + 1) * p.S, p.S, mm, zz);
      s_mq[j] = mm;
      s_zq[j] = zz;
      if (z_bad(zz)) fl |= SPEC_ST_NONFINITE;
    }
  } else {
    // every candidate entry of the request's draft rows: ids in [0, V), probabilities finite and >= 0
    const int64_t n_ent = int64_t(m) * p.K;
    const int64_t e0 = dr0 * int64_t(p.K);
    for (int64_t i = tid; i < n_ent; i += kThreads) {
      const int32_t id = p.cand_ids[e0 + i];
      const float qv = p.cand_q[e0 + i];
      if (id < 0 || int64_t(id) >= p.V) fl |= SPEC_ST_BAD_TOKEN;
      else if (!(qv >= 0.f && qv < INFINITY)) fl |= SPEC_ST_BAD_Q;
    }
  }
  __syncthreads();
  int fail = INT32_MAX;
  for (int j = tid; j < m; j += kThreads) {
    const int32_t d = p.draft_tokens[dr0 + j];
    const bool ok = d >= 0 && int64_t(d) < p.V;
    if (!ok) fl |= SPEC_ST_BAD_TOKEN;
    bool ubad = false;
    const float u = sanitize_u(p.u_accept[dr0 + j], ubad);
    if (ubad) fl |= SPEC_ST_BAD_UNIFORM;
    float a = 0.f;
    uint8_t bits = 0;
    if (ok && SPARSE) {
      const float gt = gather<DT>(p.target, off0 + j, p.V, d);
      // q(d): the masses of the valid candidate entries with id d, in entry order
      const int64_t cb = (dr0 + j) * int64_t(p.K);
      float qd = 0.f;
      for (int k = 0; k < p.K; ++k) {
        const float qv = p.cand_q[cb + k];
        if (p.cand_ids[cb + k] == d && qv >= 0.f && qv < INFINITY) qd += qv;
      }
      if (!(qd > 0.f)) {           // q(d) = 0: alpha = 1 if p(d) > 0 else 0
        bits |= 4;
        a = gt > -INFINITY ? 1.f : 0.f;
      } else {
        a = fminf(1.f, exp2_fast(fmaf(gt, p.coef, -s_mt[j])) / (s_zt[j] * qd));
      }
    } else if (ok) {
      const float gt = gather<DT>(p.target, off0 + j, p.V, d);
      const float gq = gather<DT>(p.draft, dr0 + j, p.V, d);
      if (gq == -INFINITY) {       // q(d) = 0: alpha = 1 if p(d) > 0 else 0
        bits |= 4;
        a = gt > -INFINITY ? 1.f : 0.f;
      } else {
        // alpha = min(1, p(d)/q(d)) with p(d) = exp2(gt*c - m_t)/z_t, q(d) = exp2(gq*c - m_q)/z_q
        const float et = fmaf(gt, p.coef, -s_mt[j]);
        const float eq = fmaf(gq, p.coef, -s_mq[j]);
        a = fminf(1.f, exp2_fast(et - eq) * (s_zq[j] / s_zt[j]));
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
    if (p.accept_prob) p.accept_prob[dr0 + j] = examined ? s_a[j] : -1.f;
  }
  bool ubad = false;
  float uf = 0.f;
  if (tid == 0) uf = sanitize_u(p.u_final[b], ubad);
  if (ubad) fl |= SPEC_ST_BAD_UNIFORM;
  if (fl) atomicOr(&s_flags, fl);
  for (int k = tid; k < len; k += kThreads) {
    p.out_tokens[off0 + k] = k < r ? p.draft_tokens[dr0 + k] : -1;   // k == r: written by k_draw
    p.accept_index[off0 + k] = k <= r ? int32_t(off0 + k) : -1;
  }
  __syncthreads();
  if (tid == 0) {
    p.accept_len[b] = r;
    DrawDesc d;
    d.state = p.epoch;
    d.row_t = int32_t(off0 + r);
    d.row_q = r < m ? int32_t(dr0 + r) : -1;
    d.out_pos = int32_t(off0 + r);
    d.m_t = s_mt[r];
    d.l_t = s_zt[r];
    d.m_q = r < m && !SPARSE ? s_mq[r] : 0.f;
    d.l_q = r < m && !SPARSE ? s_zq[r] : 1.f;
    d.coef = p.coef;
    d.u = uf;
    d.status = s_flags;
    d.n_seen = 0;
    p.desc[b] = d;
    p.cnt2[size_t(b) * kCounterWords] = (unsigned long long)p.epoch << 32;   // the draw pass counts from 0
    p.status[b] = s_flags;
  }
}

// ---------------------------------------------------------------------------------------------------
// Tree walk (run by the last workgroup of request b). Children are examined in ascending node index.
// ---------------------------------------------------------------------------------------------------
template <typename DT, bool SAMPLING>
__device__ void scan_tree(const StatsParams& p, int b, char* smem) {
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
  if (tid == 0) { s_flags = 0; s_nseen = 0; }
  __syncthreads();
  uint32_t fl = 0;
  for (int i = tid; i < N; i += kThreads) {
    const Part* pp = p.part + (size_t(b) * N + i) * p.S;
    if (SAMPLING) {
      float mm, zz;
      merge_sampling(pp, p.S, mm, zz);
      s_m[i] = mm;
      s_z[i] = zz;
      if (z_bad(zz)) fl |= SPEC_ST_NONFINITE;
      bool ubad = false;
      s_u[i] = sanitize_u(p.u_accept[base + i], ubad);
      if (ubad) fl |= SPEC_ST_BAD_UNIFORM;
    } else {
      const Part r = merge_greedy(pp, p.S);
      s_arg[i] = r.idx;
      if (r.flags) fl |= SPEC_ST_NONFINITE;
    }
    const int32_t par = p.parents[base + i];
    const int32_t tok = p.tokens[base + i];
    if (i == 0) {
      if (par != -1) fl |= SPEC_ST_BAD_PARENT;
      s_par[0] = -2;
      s_tok[0] = tok;
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
        const float g = gather<DT>(p.target, base + par, p.V, tok);
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
  for (int k = tid; k < N; k += kThreads) {
    p.out_tokens[base + k] = k < r ? p.tokens[base + s_path[k + 1]] : (k == r ? bonus : -1);
    p.accept_index[base + k] = k <= r ? int32_t(base + s_path[k]) : -1;
    if (p.accept_prob) p.accept_prob[base + k] = s_prob[k];
  }
  if (SAMPLING) {
    const int ns = s_nseen;
    for (int k = tid; k < ns; k += kThreads) p.seen[base + k] = s_seen[k];
  }
  __syncthreads();
  if (tid == 0) {
    p.accept_len[b] = r;
    if (!SAMPLING) {
      p.bonus[b] = bonus;
      if (p.residual_mass) p.residual_mass[b] = -1.f;
    } else {
      bool ubad = false;
      const float uf = sanitize_u(p.u_final[b], ubad);
      uint32_t st = s_flags | (ubad ? SPEC_ST_BAD_UNIFORM : 0u);
      DrawDesc d;
      d.state = p.epoch;
      d.row_t = int32_t(base + cur);
      d.row_q = -1;
      d.out_pos = int32_t(base + r);
      d.m_t = s_m[cur];
      d.l_t = s_z[cur];
      d.m_q = 0.f;
      d.l_q = 1.f;
      d.coef = p.coef;
      d.u = uf;
      d.status = st;
      d.n_seen = s_nseen;
      p.desc[b] = d;
      p.cnt2[size_t(b) * kCounterWords] = (unsigned long long)p.epoch << 32;   // the draw pass counts from 0
      s_flags = st;
    }
    p.status[b] = s_flags;
  }
}

// ---------------------------------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------------------------------
template <typename DT, bool SAMPLING, bool TREE>
__global__ __launch_bounds__(kThreads) void k_stats(StatsParams p) {
  extern __shared__ __align__(16) char smem[];
  __shared__ float red_f[kThreads / kWave];
  __shared__ float red_g[kThreads / kWave];
  __shared__ int red_i[kThreads / kWave];
  __shared__ uint32_t red_u[kThreads / kWave];
  __shared__ Part s_part;
  __shared__ int s_last;

  int64_t t = blockIdx.x;
  const int chunk = int(t % p.S);
  t /= p.S;
  const int part = int(t % p.P);
  t /= p.P;
  const int slot = int(t % p.L);
  const int b = int(t / p.L);

  int64_t off0, len;
  if (TREE) {
    off0 = int64_t(b) * p.L;
    len = p.L;
  } else {
    off0 = p.offsets[b];
    const int64_t off1 = p.offsets[b + 1];
    len = off1 - off0;
    // Besides its own range, a request checks the conditions every valid batch meets that keep its draft
    // rows inside [0, total_rows - B): off[b] >= b and off[b+1] <= total_rows - B + b + 1.
    bool ok = off0 >= b && off1 > off0 && off1 <= p.total_rows - p.B + b + 1 && len <= p.L;
    if (b == 0 && off0 != 0) ok = false;
    if (b == p.B - 1 && off1 != p.total_rows) ok = false;
    if (!ok) {
      // Offsets this request cannot be processed with: report and write what is indexed by request.
      if (slot == 0 && part == 0 && chunk == 0 && threadIdx.x == 0) {
        p.status[b] = SPEC_ST_BAD_OFFSETS;
        p.accept_len[b] = 0;
        p.bonus[b] = -1;
        if (p.residual_mass) p.residual_mass[b] = -1.f;
      }
      return;
    }
  }
  const int rows_here = part == 0 ? int(len) : int(len) - 1;
  if (slot >= rows_here) return;   // slot beyond this request's rows

  const int64_t lo = int64_t(chunk) * p.chunk;
  const int64_t hi = lo + p.chunk < p.V ? lo + p.chunk : p.V;
  const int64_t row = part == 0 ? off0 + slot : off0 - b + slot;
  const DT* base = static_cast<const DT*>(part == 0 ? p.target : p.draft) + row * p.V;

  if (SAMPLING) chunk_lse<DT>(base, lo, hi, p.coef, s_part, red_f, red_g);
  else chunk_argmax<DT>(base, lo, hi, s_part, red_f, red_i, red_u);

  if (threadIdx.x == 0) {
    store_part(p.part + ((size_t(b) * p.L + slot) * p.P + part) * p.S + chunk, s_part);
    complete_memory_ops();   // the partial is stored before it is counted
    const uint32_t expected = uint32_t((TREE ? len : (p.P == 2 ? 2 * len - 1 : len)) * p.S);
    s_last = count_done(p.cnt + size_t(b) * kCounterWords, p.epoch) == expected;
  }
  __syncthreads();
  if (!s_last) return;
  if (TREE) scan_tree<DT, SAMPLING>(p, b, smem);
  else if (SAMPLING && p.P == 2) scan_chain_rejection<DT, false>(p, b, off0, int(len), smem);
  else if (SAMPLING) scan_chain_rejection<DT, true>(p, b, off0, int(len), smem);
  else scan_chain_greedy<DT>(p, b, off0, int(len), smem);
}

template <typename DT>
hipError_t launch_stats_t(int mode, bool tree, const StatsParams& p, const Layout& lo, hipStream_t stream) {
  const int64_t blocks = int64_t(p.B) * p.L * p.P * p.S;
  if (blocks <= 0) return hipSuccess;
  const bool sampling = mode != SPEC_MODE_GREEDY;
  // Dynamic LDS serves only the request scan; it is sized for the actual rows per request.
  const size_t per_row = tree ? 11 * 4 : (sampling ? 5 * 4 + 1 : 4);
  const size_t smem = (per_row * size_t(p.L) + 15) / 16 * 16;
  const dim3 grid{unsigned(blocks)}, block{unsigned(kThreads)};
  if (tree) {
    if (sampling) hipLaunchKernelGGL((k_stats<DT, true, true>), grid, block, smem, stream, p);
    else hipLaunchKernelGGL((k_stats<DT, false, true>), grid, block, smem, stream, p);
  } else {
    if (sampling) hipLaunchKernelGGL((k_stats<DT, true, false>), grid, block, smem, stream, p);
    else hipLaunchKernelGGL((k_stats<DT, false, false>), grid, block, smem, stream, p);
  }
  (void)lo;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_stats(int dtype, int mode, bool tree, const StatsParams& p, const Layout& lo,
                        hipStream_t stream) {
  if (dtype == SPEC_DTYPE_BF16) return launch_stats_t<uint16_t>(mode, tree, p, lo, stream);
  return launch_stats_t<float>(mode, tree, p, lo, stream);
}

}  // namespace sv
