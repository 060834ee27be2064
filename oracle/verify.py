"""Oracle for the speculative-decoding verify / accept / commit step: plain, slow, fp64, CPU only.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may import
or call this module. It shares no code with the HIP library (draft_verification_acceptance_amd/) and
imports nothing from it; both sides only consume the same seeded inputs.

Every request is handled on its own, one row at a time, in float64 numpy. The steps follow the pages in
their order and notation:

  [EAGLE→DFlash2]  tom-jerr.github.io, "从 EAGLE 到 DFlash 2：SGLang 与 SpecForge 的投机解码训练和推理"
  [DFlash]         astro-wiki.dev.mem.ac, "DFlash"
  [SpecDec]        zdszero.github.io, "speculative_decoding"

Verify rows are [a, d1 .. dm]: row j is the target's distribution for the token after d_j (row 0: after the
anchor a), so row j-1 judges d_j and row m yields the bonus ([EAGLE→DFlash2] §1.1). Readings taken where
the pages leave a step open are marked READING.

Pins: every function here is checked in tests/test_oracle_pins.py against values the pages print, closed
forms, brute force and textbook special cases. No function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

# Per-request status bits (values fixed by the C ABI of the library under test).
ST_NONFINITE = 1 << 0
ST_BAD_TOKEN = 1 << 1
ST_BAD_OFFSETS = 1 << 2
ST_BAD_PARENT = 1 << 3
ST_BAD_UNIFORM = 1 << 4
ST_ZERO_Q = 1 << 5
ST_ZERO_RESIDUAL = 1 << 6
ST_NEAR_ALPHA = 1 << 7
ST_NEAR_CDF = 1 << 8
ST_BAD_ACCEPT = 1 << 9
ST_BAD_Q = 1 << 10

NEAR = 1e-5          # width of the "too close to call" band for accept tests and CDF steps
NEAR_MASS = 1e-6     # the same band measured in probability mass for a draw (gap * Z), see near_cdf()
U_MAX = 1.0 - 2.0 ** -24   # largest float32 below 1


# ----------------------------------------------------------------------------------------------------
# Common definitions
# ----------------------------------------------------------------------------------------------------
def decode_row(row: np.ndarray) -> np.ndarray:
    """One logits row -> float64. uint16 rows hold bfloat16 bit patterns: the float32 with those 16 bits
    on top and zeros below, which is exact; float32 rows convert exactly too."""
    if row.dtype == np.uint16:
        return (row.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if row.dtype == np.float32:
        return row.astype(np.float64)
    raise TypeError(f"logits must be uint16 (bf16 bits) or float32, got {row.dtype}")


def row_nonfinite(x: np.ndarray, sampling: bool) -> bool:
    """NaN anywhere; for sampling also +inf or a row of only -inf (softmax undefined)."""
    if np.isnan(x).any():
        return True
    if sampling and (np.isposinf(x).any() or np.isneginf(x).all()):
        return True
    return False


def mask_row(x: np.ndarray, words) -> np.ndarray:
    """Vocab (grammar) mask on one target row ([EAGLE→DFlash2] §5.6.6 and §8.4: the grammar mask is applied to
    the target logits after the target forward and before acceptance, and sampling reads the masked
    distribution). `words` holds the row's allowed-token bits: token v is allowed iff bit (v mod 32) of word
    v // 32 is 1 (READING: the packed bitmask layout; None = every token allowed). A masked logit becomes -inf
    whatever its value, so a NaN or +inf there no longer counts."""
    if words is None:
        return x
    v = np.arange(len(x))
    allowed = (np.asarray(words, np.uint64)[v >> 5] >> (v & 31).astype(np.uint64)) & np.uint64(1)
    return np.where(allowed == 1, x, -np.inf)


def softmax_T(x: np.ndarray, temperature: float) -> np.ndarray:
    """p = softmax(x / T) in float64 ([EAGLE→DFlash2] §1.2: p_j, q_j are the distributions actually used,
    READING: the same temperature divides target and draft logits). -inf entries get p = 0."""
    z = x / temperature
    zmax = np.max(z)
    with np.errstate(invalid="ignore"):       # an all -inf row is reported as non-finite by the caller
        e = np.exp(z - zmax)
        return e / np.sum(e)


def argmax_lowest(x: np.ndarray) -> int:
    """Greedy argmax with the lowest id among equal maxima (READING: the pages ask for the same
    tie-breaking as plain greedy, [EAGLE→DFlash2] §1.2). NaN entries never win."""
    y = np.where(np.isnan(x), -np.inf, x)
    best = np.max(y)
    return int(np.flatnonzero(y == best)[0])


def sanitize_uniform(u) -> tuple[float, bool]:
    """Caller uniforms lie in [0,1) and are used as exact float64 values. Returns (value, was_bad): NaN is
    used as 0 and a value outside [0,1) is clamped to [0, 1 - 2^-24]."""
    v = float(u)
    if np.isnan(v):
        return 0.0, True
    if 0.0 <= v < 1.0:
        return v, False
    return min(max(v, 0.0), U_MAX), True


def residual_weights(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Rejection branch weights [p - q]_+ ([EAGLE→DFlash2] §1.2: after a rejection draw from
    [p(v) - q(v)]_+ / sum_u [p(u) - q(u)]_+; the accept branch carries min(p, q), the two add up to p)."""
    return np.maximum(p - q, 0.0)


def accept_probability(pd: float, qd: float) -> float:
    """alpha = min(1, p(d) / q(d)) ([EAGLE→DFlash2] §1.2). READING for q(d) = 0 (p/0): alpha = 1 if p(d) > 0
    else 0; the caller flags the case."""
    if qd == 0.0:
        return 1.0 if pd > 0.0 else 0.0
    return min(1.0, pd / qd)


def sparse_q(ids: np.ndarray, probs: np.ndarray, V: int) -> tuple[np.ndarray, int]:
    """Proposal q over the vocab from K (candidate id, probability) pairs: the candidate distribution is
    scattered into target vocab coordinates and q is zero everywhere else ([EAGLE→DFlash2] §6.5, sampling
    verify with the selector's candidate q; greedy rows carry a one-hot q). Returns (q, status bits).
    READING: a repeated id adds its masses (top-K ids are distinct, so this only concerns malformed
    input); an id outside [0, V) sets BAD_TOKEN and a negative or non-finite probability sets BAD_Q, and
    such an entry is left out."""
    q = np.zeros(V)
    st = 0
    for i, w in zip(np.asarray(ids).tolist(), np.asarray(probs, np.float64).tolist()):
        if not 0 <= i < V:
            st |= ST_BAD_TOKEN
            continue
        if not (np.isfinite(w) and w >= 0.0):
            st |= ST_BAD_Q
            continue
        q[i] += w
    return q, st


def draw(w: np.ndarray, u: float) -> tuple[int, float, float]:
    """Inverse-CDF draw from nonnegative weights w ([EAGLE→DFlash2] §6.2, the selector's rule: the index is
    the number of cumulative probabilities that u has reached). Returns (token, gap, Z) where Z = sum w
    (ascending order), gap = distance from u to the nearer edge of the chosen step.
    READING: when rounding leaves u past the last step, the largest id with positive weight is taken, so a
    zero-weight id is never drawn."""
    c = np.cumsum(w)
    Z = float(c[-1])
    C = c / Z
    k = int(np.count_nonzero(C <= u))
    if k == len(w):
        k = int(np.flatnonzero(w > 0)[-1])
    lo = float(C[k - 1]) if k > 0 else 0.0
    gap = min(u - lo, float(C[k]) - u)
    return k, gap, Z


def near_cdf_band(gap: float) -> bool:
    """The draw's u lies within 1e-5 of a step of the normalised CDF: too close to call, flagged and counted
    (the band the verify step's contract fixes for residual-CDF gaps)."""
    return gap < NEAR


def near_cdf_mass(gap: float, Z: float) -> bool:
    """READING (an accommodation of fp32 arithmetic, not a rule of the pages): the draw's margin measured in
    probability mass, gap * Z, is below 1e-6. A verifier that forms p and q in fp32 knows each probability to
    about 1e-7 relative, so the steps of the normalised residual CDF of a residual with small total mass Z
    are known only to about 1e-6 / Z. This widens the 1e-5 band only where Z < 0.1, i.e. for rejections
    between nearly equal p and q; on the seeded workloads it adds no exemption (tested)."""
    return gap * Z < NEAR_MASS


def near_cdf(gap: float, Z: float) -> bool:
    """A final draw too close to call: near_cdf_band or near_cdf_mass."""
    return near_cdf_band(gap) or near_cdf_mass(gap, Z)


def sample_then_match(ps: list, toks: list, tok_ok: list, us: list) -> tuple[int, int, list, int | None]:
    """Sample-then-match over one request's rows ([DFlash] decode loop, step 4: each draft token is compared
    with a sample of the target posterior at its position, the accept length is the longest matching prefix,
    and the first mismatch is replaced by that sample; [EAGLE→DFlash2] §1.2: sampling the target
    independently and matching the prefix is a different implementation from p/q rejection). Every emitted
    token is a draw from its row's p, so the output follows the target.
    ps[j] = p_j (rows 0..m), toks[j] = d_{j+1}, us[j] = the uniform of row j.
    READING: row j's sample is draw(p_j, us[j]) with us[j] = the uniform of d_{j+1}'s test for j < m and
    u_final for row m; the compared positions report p_j(d_{j+1}) as their accept probability; there is no
    residual. Returns (r, emitted sample at row r, accept probabilities of the compared positions, index of
    the first sample too close to a CDF step or None)."""
    m = len(toks)
    alphas = []
    near = None
    for j in range(m + 1):
        t, gap, Z = draw(ps[j], us[j])
        if near_cdf_band(gap) and near is None:   # p_j itself: Z = 1, the mass clause adds nothing
            near = j
        if j < m:
            alphas.append(ps[j][toks[j]] if tok_ok[j] else 0.0)
            if tok_ok[j] and t == toks[j]:
                continue
        return j, t, alphas, near
    raise AssertionError("unreachable")


def _sentinel_outputs(n_rows: int, n_draft: int, batch: int) -> dict:
    return {
        "accept_len": np.full(batch, -2, np.int64),
        "bonus": np.full(batch, -2, np.int64),
        "out_tokens": np.full(n_rows, -2, np.int64),
        "accept_index": np.full(n_rows, -2, np.int64),
        "status": np.zeros(batch, np.uint32),
        "accept_prob": np.full(n_draft, np.nan),
        "residual_mass": np.full(batch, np.nan),
        "flag_pos": np.full(batch, -2, np.int64),
        "near_mass_only": np.zeros(batch, bool),
        "evaluated": np.zeros(batch, bool),
    }


# ----------------------------------------------------------------------------------------------------
# Chain verify
# ----------------------------------------------------------------------------------------------------
def verify_chain(target: np.ndarray, offsets: np.ndarray, draft_tokens: np.ndarray, mode: str, *,
                 draft: np.ndarray | None = None, u_accept: np.ndarray | None = None,
                 u_final: np.ndarray | None = None, temperature: float = 1.0,
                 max_verify_len: int = 1024, requests=None, cand_ids: np.ndarray | None = None,
                 cand_q: np.ndarray | None = None, vocab_mask: np.ndarray | None = None) -> dict:
    """Chain verify for mode "greedy", "rejection", "rejection_sparse" or "sample_match".

    target [T_rows, V] (uint16 bf16 bits or float32); offsets [B+1]: request b owns target rows
    off[b]..off[b+1]-1 (ragged layout of [EAGLE→DFlash2] §5.6.5). Draft-side arrays hold m_b entries per
    request from off[b]-b on; entry j is about d_{j+1}. "rejection" takes q_j = softmax(draft row / T);
    "rejection_sparse" takes q_j from the K candidate pairs cand_ids[entry], cand_q[entry] ([D_rows, K]) of
    sparse_q (the temperature then divides the target logits only: q arrives as probabilities).
    "sample_match" draws a sample from every target row and accepts while it equals the draft token.
    vocab_mask [T_rows, ceil(V/32)] (optional) masks the target rows (mask_row); draft rows are not masked.
    `requests` limits the work to some requests (the others keep sentinel values: -2 / NaN).

    Returns accept_len, bonus, out_tokens, accept_index, status, accept_prob, residual_mass, and (oracle
    only) flag_pos = the position of the first decision too close to call (NEAR_ALPHA at the test of d_j:
    j-1; NEAR_CDF at the final draw: r; a sample-then-match sample at row j: j), i.e. the number of leading
    emitted tokens that no such decision can change; r+1 if none. near_mass_only: the request's only flag is
    a final draw caught by near_cdf_mass alone.
    """
    assert mode in ("greedy", "rejection", "rejection_sparse", "sample_match")
    T, V = target.shape
    B = len(offsets) - 1
    out = _sentinel_outputs(T, max(T - B, 0), B)
    cand = (cand_ids, cand_q) if mode == "rejection_sparse" else None
    for b in (range(B) if requests is None else requests):
        _chain_request(out, b, target, offsets, draft_tokens, mode, draft, u_accept, u_final,
                       temperature, max_verify_len, T, V, B, cand, vocab_mask)
    return out


def _chain_offsets_ok(offsets, b, T, B, max_len) -> bool:
    """Request b's rows [off[b], off[b+1]) checked on their own: non-empty, at most max_len rows, and the
    bounds every strictly increasing offsets array from 0 to T obeys (off[b] >= b, off[b+1] <= T-B+b+1)."""
    lo, hi = int(offsets[b]), int(offsets[b + 1])
    ok = b <= lo < hi <= T - B + b + 1 and hi - lo <= max_len
    if b == 0 and lo != 0:
        ok = False
    if b == B - 1 and hi != T:
        ok = False
    return ok


def _chain_request(out, b, target, offsets, draft_tokens, mode, draft, u_accept, u_final, temperature,
                   max_len, T, V, B, cand=None, vocab_mask=None):
    out["evaluated"][b] = True
    if not _chain_offsets_ok(offsets, b, T, B, max_len):
        out["status"][b] = ST_BAD_OFFSETS
        out["accept_len"][b] = 0
        out["bonus"][b] = -1
        out["flag_pos"][b] = 0
        return
    off = int(offsets[b])
    m = int(offsets[b + 1]) - off - 1
    dr0 = off - b                      # first draft-side entry of this request
    sampling = mode != "greedy"
    st = 0

    t_rows = [mask_row(decode_row(target[off + j]), None if vocab_mask is None else vocab_mask[off + j])
              for j in range(m + 1)]
    s_rows = [decode_row(draft[dr0 + j]) for j in range(m)] if mode == "rejection" else []
    for x in t_rows + s_rows:
        if row_nonfinite(x, sampling):
            st |= ST_NONFINITE
    if vocab_mask is not None and any(np.isneginf(x).all() for x in t_rows):
        st |= ST_NONFINITE     # READING: a masked row with no allowed finite logit, in every mode
    toks = [int(draft_tokens[dr0 + j]) for j in range(m)]      # toks[j-1] = d_j
    tok_ok = [0 <= d < V for d in toks]
    if not all(tok_ok):
        st |= ST_BAD_TOKEN

    alphas = np.full(m, -1.0)
    flag_pos = None
    resid = -1.0
    if not sampling:
        # Greedy ([SpecDec] "为什么结果不受 draft 影响"; [DFlash] decode loop step 4): accept d_j while it
        # equals the argmax of row j-1; the first mismatch is replaced by that argmax.
        r = 0
        for j in range(1, m + 1):
            if tok_ok[j - 1] and toks[j - 1] == argmax_lowest(t_rows[j - 1]):
                r = j
            else:
                break
        x = argmax_lowest(t_rows[r])
    elif mode == "sample_match":
        us = [sanitize_uniform(u_accept[dr0 + j]) for j in range(m)] + [sanitize_uniform(u_final[b])]
        if any(bad for _, bad in us):
            st |= ST_BAD_UNIFORM
        ps = [softmax_T(x, temperature) for x in t_rows]
        r, x, a, near = sample_then_match(ps, toks, tok_ok, [u for u, _ in us])
        alphas[:len(a)] = a
        if near is not None:
            st |= ST_NEAR_CDF
            flag_pos = near
    else:
        us = [sanitize_uniform(u_accept[dr0 + j]) for j in range(m)]
        uf, uf_bad = sanitize_uniform(u_final[b])
        if uf_bad or any(bad for _, bad in us):
            st |= ST_BAD_UNIFORM
        ps = [softmax_T(x, temperature) for x in t_rows]
        if cand is None:
            qs = [softmax_T(x, temperature) for x in s_rows]
        else:
            qs = []
            for j in range(m):
                q, qst = sparse_q(cand[0][dr0 + j], cand[1][dr0 + j], V)
                qs.append(q)
                st |= qst
        r = m
        w = None
        for j in range(1, m + 1):
            # alpha_j = min(1, p_{j-1}(d_j) / q_{j-1}(d_j))   ([EAGLE→DFlash2] §1.2)
            if tok_ok[j - 1]:
                pd = ps[j - 1][toks[j - 1]]
                qd = qs[j - 1][toks[j - 1]]
                if qd == 0.0:
                    st |= ST_ZERO_Q
                a = accept_probability(pd, qd)
            else:
                a = 0.0          # an out-of-range token is never accepted
            alphas[j - 1] = a
            u = us[j - 1][0]
            if abs(u - a) < NEAR:
                st |= ST_NEAR_ALPHA
                flag_pos = j - 1 if flag_pos is None else flag_pos
            if u < a:            # READING: accept iff u < alpha
                continue
            # Rejected at j: draw from the residual [p - q]_+ / sum [p - q]_+ of row j-1.
            r = j - 1
            w = residual_weights(ps[j - 1], qs[j - 1])
            break
        if w is None:
            # Every draft passed: bonus from the last row, m+1 new tokens ([EAGLE→DFlash2] §1.1).
            w = ps[m]
        if np.sum(w) == 0.0:
            st |= ST_ZERO_RESIDUAL  # READING: an all-zero residual (rounding, or a sparse q whose masses reach p
            #                         wherever p > 0) leaves the draw undefined -> draw from p
            w = ps[r]
        x, gap, resid = draw(w, uf)
        if near_cdf(gap, resid):
            out["near_mass_only"][b] = flag_pos is None and not near_cdf_band(gap)
            st |= ST_NEAR_CDF
            flag_pos = r if flag_pos is None else flag_pos

    out["accept_len"][b] = r
    out["bonus"][b] = x
    for k in range(m + 1):
        out["out_tokens"][off + k] = toks[k] if k < r else (x if k == r else -1)
        out["accept_index"][off + k] = off + k if k <= r else -1
    out["accept_prob"][dr0:dr0 + m] = alphas
    out["residual_mass"][b] = resid
    out["status"][b] = st
    out["flag_pos"][b] = r + 1 if flag_pos is None else flag_pos


# ----------------------------------------------------------------------------------------------------
# Tree verify
# ----------------------------------------------------------------------------------------------------
def verify_tree(target: np.ndarray, parents: np.ndarray, tokens: np.ndarray, n_nodes: int, mode: str, *,
                u_accept: np.ndarray | None = None, u_final: np.ndarray | None = None,
                temperature: float = 1.0, requests=None, vocab_mask: np.ndarray | None = None) -> dict:
    """Tree verify for mode "greedy" or "target_only".

    Request b owns rows b*N .. b*N+N-1; node 0 is the anchor, node i > 0 has parent in [0, i) and token
    tokens[b*N+i]. Row i is the target distribution after the path to node i (tree attention,
    [EAGLE→DFlash2] §2.4). Children are examined in ascending node index (READING). vocab_mask [B*N,
    ceil(V/32)] (optional) masks every node row (mask_row).
    """
    assert mode in ("greedy", "target_only")
    rows, V = target.shape
    N = int(n_nodes)
    B = rows // N
    out = _sentinel_outputs(rows, rows, B)
    for b in (range(B) if requests is None else requests):
        _tree_request(out, b, target, parents, tokens, N, mode, u_accept, u_final, temperature, V, vocab_mask)
    return out


def _tree_request(out, b, target, parents, tokens, N, mode, u_accept, u_final, temperature, V, vocab_mask=None):
    out["evaluated"][b] = True
    base = b * N
    sampling = mode == "target_only"
    st = 0
    rows = [mask_row(decode_row(target[base + i]), None if vocab_mask is None else vocab_mask[base + i])
            for i in range(N)]
    for x in rows:
        if row_nonfinite(x, sampling):
            st |= ST_NONFINITE
    if vocab_mask is not None and any(np.isneginf(x).all() for x in rows):
        st |= ST_NONFINITE
    par = [int(parents[base + i]) for i in range(N)]
    tok = [int(tokens[base + i]) for i in range(N)]
    if par[0] != -1:
        st |= ST_BAD_PARENT
    parent_ok = [False] + [0 <= par[i] < i for i in range(1, N)]
    if not all(parent_ok[1:]):
        st |= ST_BAD_PARENT
    tok_ok = [True] + [0 <= tok[i] < V for i in range(1, N)]
    if not all(tok_ok):
        st |= ST_BAD_TOKEN

    def children(c):
        return [i for i in range(c + 1, N) if parent_ok[i] and par[i] == c]

    probs = np.full(N, -1.0)
    flag_pos = None
    resid = -1.0
    path = [0]
    cur = 0
    if not sampling:
        # verify_tree_greedy semantics ([SpecDec] "为什么结果不受 draft 影响"): follow the child whose token
        # equals the argmax of the current node's row; the lowest index wins among equal children.
        while True:
            a = argmax_lowest(rows[cur])
            hits = [c for c in children(cur) if tok_ok[c] and tok[c] == a]
            if not hits:
                break
            cur = hits[0]
            path.append(cur)
        x = argmax_lowest(rows[cur])
    else:
        uf, uf_bad = sanitize_uniform(u_final[b])
        bad_u = uf_bad
        for i in range(N):
            bad_u |= sanitize_uniform(u_accept[base + i])[1]
        if bad_u:
            st |= ST_BAD_UNIFORM
        # Target-only tree sampling with thresholds 1.0 ([SpecDec] "为什么结果不受 draft 影响": only target
        # probabilities judge, draft probabilities passed as 0). READING: sibling-by-sibling rejection with
        # a one-hot proposal: child c is accepted with the target mass of its token, the residual is p
        # restricted to the tokens not yet tried, so every emitted token is distributed as p.
        while True:
            p = softmax_T(rows[cur], temperature)
            u = sanitize_uniform(u_accept[base + cur])[0]
            acc = 0.0
            seen: list[int] = []
            nxt = None
            for c in children(cur):
                if not tok_ok[c] or tok[c] in seen:
                    continue
                seen.append(tok[c])
                acc += p[tok[c]]
                probs[c] = acc
                if abs(u - acc) < NEAR:
                    st |= ST_NEAR_ALPHA
                    flag_pos = len(path) - 1 if flag_pos is None else flag_pos
                if u < acc:
                    nxt = c
                    break
            if nxt is None:
                break
            cur = nxt
            path.append(cur)
        w = p.copy()
        if seen:
            w[seen] = 0.0
        if np.sum(w) == 0.0:
            st |= ST_ZERO_RESIDUAL
            w = p
        x, gap, resid = draw(w, uf)
        if near_cdf(gap, resid):
            out["near_mass_only"][b] = flag_pos is None and not near_cdf_band(gap)
            st |= ST_NEAR_CDF
            flag_pos = len(path) - 1 if flag_pos is None else flag_pos

    r = len(path) - 1
    out["accept_len"][b] = r
    out["bonus"][b] = x
    for k in range(N):
        out["out_tokens"][base + k] = tok[path[k + 1]] if k < r else (x if k == r else -1)
        out["accept_index"][base + k] = base + path[k] if k <= r else -1
    out["accept_prob"][base:base + N] = probs
    out["residual_mass"][b] = resid
    out["status"][b] = st
    out["flag_pos"][b] = r + 1 if flag_pos is None else flag_pos


# ----------------------------------------------------------------------------------------------------
# Commit
# ----------------------------------------------------------------------------------------------------
def commit_indices(row_offsets: np.ndarray, accept_len: np.ndarray, accept_index: np.ndarray,
                   verify_slots: np.ndarray, seq_lens: np.ndarray, max_verify_len: int = 1024) -> dict:
    """KV commit compaction ([EAGLE→DFlash2] §5.6.6: commit_lens = correct_len + 1; §8.1: the committed KV
    rows are the old anchor plus the accepted drafts, in path order; [SpecDec] "实现：共享的骨架": they
    move to contiguous positions after seq_lens). Also lists the rows to evict (not on the path)."""
    B = len(row_offsets) - 1
    T = len(verify_slots)
    status = np.zeros(B, np.uint32)
    clen = np.zeros(B, np.int64)
    elen = np.zeros(B, np.int64)
    per_req = []
    for b in range(B):
        ok = _chain_offsets_ok(row_offsets, b, T, B, max_verify_len)
        if not ok:
            status[b] |= ST_BAD_OFFSETS
            per_req.append(None)
            continue
        lo, hi = int(row_offsets[b]), int(row_offsets[b + 1])
        r = int(accept_len[b])
        if not 0 <= r < hi - lo:
            status[b] |= ST_BAD_ACCEPT
            r = min(max(r, 0), hi - lo - 1)
        idx = [int(accept_index[lo + k]) for k in range(r + 1)]
        if any(not lo <= i < hi for i in idx) or len(set(idx)) != len(idx):
            status[b] |= ST_BAD_ACCEPT
        clen[b] = r + 1
        acc = set(idx)
        ev = [i for i in range(lo, hi) if i not in acc]
        elen[b] = len(ev)
        per_req.append((lo, r, idx, ev))
    commit_offsets = np.zeros(B + 1, np.int64)
    commit_offsets[1:] = np.cumsum(clen)
    evict_offsets = np.zeros(B + 1, np.int64)
    evict_offsets[1:] = np.cumsum(elen)
    total = int(commit_offsets[-1])
    src = np.full(total, -1, np.int64)
    dst = np.full(total, -1, np.int64)
    evict = np.full(int(evict_offsets[-1]), -1, np.int64)
    new_seq = np.array(seq_lens, np.int64).copy()
    for b in range(B):
        if per_req[b] is None:
            continue
        lo, r, idx, ev = per_req[b]
        for k in range(r + 1):
            i = idx[k]
            src[commit_offsets[b] + k] = int(verify_slots[i]) if lo <= i < int(row_offsets[b + 1]) else -1
            dst[commit_offsets[b] + k] = int(seq_lens[b]) + k
        for k, i in enumerate(ev):
            evict[evict_offsets[b] + k] = int(verify_slots[i])
        new_seq[b] = int(seq_lens[b]) + r + 1
    return {"commit_offsets": commit_offsets, "src_slots": src, "dst_pos": dst, "new_seq_lens": new_seq,
            "status": status, "evict_offsets": evict_offsets, "evict_slots": evict}
