"""Oracle for the DSpark verify-length planner and the accept cutoff (cap_trim): plain, slow, CPU only.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may import
or call this module. It shares no code with the HIP library and imports nothing from it.

Steps, in the pages' order and notation:

  [EAGLE→DFlash2]  tom-jerr.github.io, "从 EAGLE 到 DFlash 2：SGLang 与 SpecForge 的投机解码训练和推理",
                   §5.5 (throughput model), §5.6.3 (host budget K*), §5.6.4 (device top-K allocation),
                   §5.6.5 (ragged layout), §5.6.6 (cap_trim / commit_lens / block_accept_lens)
  [DSpark]         ggaaooppeenngg.github.io, "DSpark：半自回归 + 置信度调度的 Speculative Decoding 深度分析",
                   confidence head and threshold truncation, Hardware-Aware Prefix Scheduler

R requests each propose W drafts with per-position confidences c_{r,j} (the head's estimate that position j
survives given j-1 did). The prefix survival is A_{r,j} = prod_{i<=j} c_{r,i}. A plan verifies l_r of them:
M = sum_r (1 + l_r) target rows, expected output N = sum_r (1 + sum_{j<=l_r} A_{r,j}), throughput N * SPS(M).

Precision: the survival products are taken in float32 in position order, as the library's kernel takes them,
because they decide integers (the ranking and the budget); sums and the throughput model are float64.

READINGS (where the pages leave a step open):
  * a confidence that is NaN counts as 0 and one outside [0, 1] is clamped into it (flagged);
  * survival_eps: entries with A < eps are dropped from the history sort and are never selected;
  * K* is the argmax of N(K) * SPS(R + K) over every prefix budget 0 <= K <= n ([EAGLE→DFlash2] §5.6.3
    evaluates all prefix budgets with one cumulative sum); on equal values the smallest K wins;
  * SPS(M) between table points is linear in M, and outside the table it is the nearest end value;
  * the additive cost table's T(R, M) = T_req(R) + T_tok(M), two tables read by the same rule
    (budget_from_survival_cost);
  * budget < 0 stands for "no budget" (the relay had nothing): every request verifies all W drafts;
  * threshold truncation compares each position's own confidence c_{r,j}, not the survival, and verifies the
    drafts before the first one below the threshold (all W if none is);
  * cap_trim: when the accepted prefix is cut at ell, the emitted token at position ell (the accepted draft
    d_{ell+1}) becomes the bonus; positions after it are cleared.
"""
from __future__ import annotations

import numpy as np

ST_BAD_ACCEPT = 1 << 9
ST_BAD_CONF = 1 << 11


def sanitize_confidence(c) -> tuple[np.float32, bool]:
    """NaN -> 0, outside [0, 1] -> clamped; returns (value as float32, whether it was changed)."""
    c = np.float32(c)
    if np.isnan(c):
        return np.float32(0.0), True
    if c < 0:
        return np.float32(0.0), True
    if c > 1:
        return np.float32(1.0), True
    return c, False


def survival(conf: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """A_{r,j} = prod_{i<=j} c_{r,i}, float32 products in position order; also per-request BAD_CONF flags."""
    conf = np.asarray(conf, np.float32)
    R, W = conf.shape
    A = np.zeros((R, W), np.float32)
    flags = np.zeros(R, np.uint32)
    for r in range(R):
        s = np.float32(1.0)
        for j in range(W):
            c, bad = sanitize_confidence(conf[r, j])
            if bad:
                flags[r] |= ST_BAD_CONF
            s = np.float32(s * c)
            A[r, j] = s
    return A, flags


def sps_at(M: float, sps_rows: np.ndarray, sps: np.ndarray) -> float:
    """Steps per second at M target rows: linear between table points, the end value outside (the same
    rule reads the additive cost tables)."""
    xs = [float(x) for x in sps_rows]
    ys = [float(y) for y in sps]
    if M <= xs[0]:
        return ys[0]
    if M >= xs[-1]:
        return ys[-1]
    i = 0
    while not (xs[i] <= M < xs[i + 1]):
        i += 1
    slope = (ys[i + 1] - ys[i]) / (xs[i + 1] - xs[i])
    return slope * (M - xs[i]) + ys[i]


def budget_from_survival(A_hist: np.ndarray, sps_rows, sps, eps: float = 0.0) -> tuple[int, np.ndarray]:
    """Host budget ([EAGLE→DFlash2] §5.6.3): flatten the history survival, drop entries below eps, sort
    descending a_1 >= .. >= a_n, N(K) = R + a_1 + .. + a_K, K* = argmax_{0<=K<=n} N(K) * SPS(R + K).
    Returns (K*, theta[0..n])."""
    A_hist = np.asarray(A_hist, np.float32)
    R = A_hist.shape[0]
    a = sorted((float(v) for v in A_hist.ravel() if v >= np.float32(eps)), reverse=True)
    theta = np.zeros(len(a) + 1)
    N = float(R)
    theta[0] = N * sps_at(R, sps_rows, sps)
    best, k_best = theta[0], 0
    for K in range(1, len(a) + 1):
        N += a[K - 1]
        theta[K] = N * sps_at(R + K, sps_rows, sps)
        if theta[K] > best:
            best, k_best = theta[K], K
    return k_best, theta


def plan_budget(conf_hist: np.ndarray, sps_rows, sps, eps: float = 0.0) -> tuple[int, np.ndarray]:
    """The host budget from lagged confidences (survival taken first)."""
    A, _ = survival(conf_hist)
    return budget_from_survival(A, sps_rows, sps, eps)


def budget_from_survival_cost(A_hist: np.ndarray, req_rows, req_cost, tok_rows, tok_cost,
                              eps: float = 0.0) -> tuple[int, np.ndarray]:
    """Host budget under an additive cost table ([EAGLE→DFlash2] §5.6.3: with an additive cost table the
    objective N(K) * SPS(R + K) becomes N(K) / T(R, R + K)). READING: the pages name the table but do not
    define T; here T(R, M) = T_req(R) + T_tok(M), the predicted time of one step with R requests and M target
    rows as the sum of a per-batch term and a per-row term, each read from its own table (linear between
    points, the end value outside, as for SPS). With T_req = 0 and T_tok = 1 / SPS at every integer M this is
    the SPS objective. Same sort, prefix sums and tie rule as budget_from_survival. Returns (K*, theta)."""
    A_hist = np.asarray(A_hist, np.float32)
    R = A_hist.shape[0]
    a = sorted((float(v) for v in A_hist.ravel() if v >= np.float32(eps)), reverse=True)
    c = sps_at(R, req_rows, req_cost)
    theta = np.zeros(len(a) + 1)
    N = float(R)
    theta[0] = N / (c + sps_at(R, tok_rows, tok_cost))
    best, k_best = theta[0], 0
    for K in range(1, len(a) + 1):
        N += a[K - 1]
        theta[K] = N / (c + sps_at(R + K, tok_rows, tok_cost))
        if theta[K] > best:
            best, k_best = theta[K], K
    return k_best, theta


def plan_budget_cost(conf_hist: np.ndarray, req_rows, req_cost, tok_rows, tok_cost,
                     eps: float = 0.0) -> tuple[int, np.ndarray]:
    """The additive-cost host budget from lagged confidences (survival taken first)."""
    A, _ = survival(conf_hist)
    return budget_from_survival_cost(A, req_rows, req_cost, tok_rows, tok_cost, eps)


def ragged_offsets(verify_lens) -> np.ndarray:
    """[EAGLE→DFlash2] §5.6.5: verify lens [4,2,6] -> offsets [0,4,6,12] (exclusive prefix sum, total last)."""
    out = [0]
    for v in verify_lens:
        out.append(out[-1] + int(v))
    return np.asarray(out, np.int32)


def _finish_layout(selected, W, min_len, max_len, flags):
    verify_lens = np.array([min(max(1 + int(s), min_len), max_len) for s in selected], np.int32)
    offsets = ragged_offsets(verify_lens)
    row_index = np.full(int(offsets[-1]), -1, np.int64)
    for r, v in enumerate(verify_lens):
        for j in range(int(v)):
            row_index[offsets[r] + j] = r * (W + 1) + j
    return {"selected": np.asarray(selected, np.int32), "verify_lens": verify_lens, "offsets": offsets,
            "row_index": row_index, "status": flags}


def plan_from_survival(A: np.ndarray, budget: int, *, min_len: int = 1, max_len: int | None = None,
                       eps: float = 0.0, flags=None) -> dict:
    """Device allocation ([EAGLE→DFlash2] §5.6.4): rank every (request, position) by current survival
    descending, then position ascending, then request ascending; the first `budget` of them are verified;
    verify_lens = clamp(1 + selected_r, min_len, max_len); ragged offsets follow. row_index maps each
    compact verify row to r * (W + 1) + j, j = 0 being the anchor."""
    A = np.asarray(A, np.float32)
    R, W = A.shape
    max_len = W + 1 if max_len is None else max_len
    flags = np.zeros(R, np.uint32) if flags is None else flags
    if budget < 0:   # no budget: the uniform full layout
        return _finish_layout([W] * R, W, min_len, max_len, flags)
    entries = [(r, j) for r in range(R) for j in range(W) if A[r, j] >= np.float32(eps)]
    order = sorted(entries, key=lambda e: (-float(A[e[0], e[1]]), e[1], e[0]))
    selected = [0] * R
    for r, _ in order[:budget]:
        selected[r] += 1
    return _finish_layout(selected, W, min_len, max_len, flags)


def plan_layout(conf: np.ndarray, budget: int, *, min_len: int = 1, max_len: int | None = None,
                eps: float = 0.0) -> dict:
    """The device allocation from current confidences (survival taken first)."""
    A, flags = survival(conf)
    return plan_from_survival(A, budget, min_len=min_len, max_len=max_len, eps=eps, flags=flags)


def threshold_layout(conf: np.ndarray, threshold: float, *, min_len: int = 1, max_len: int | None = None) -> dict:
    """[DSpark] threshold truncation: verify the drafts before the first position whose confidence is below
    the threshold (every draft if none is), then clamp as the top-K layout does."""
    conf = np.asarray(conf, np.float32)
    R, W = conf.shape
    max_len = W + 1 if max_len is None else max_len
    _, flags = survival(conf)
    selected = []
    for r in range(R):
        first_below = W
        for j in range(W):
            c, _ = sanitize_confidence(conf[r, j])
            if c < np.float32(threshold):
                first_below = j
                break
        selected.append(first_below)
    return _finish_layout(selected, W, min_len, max_len, flags)


def cap_trim(row_offsets, verify_lens, raw_accept_len, raw_bonus, out_tokens) -> dict:
    """[EAGLE→DFlash2] §5.6.6: ell = verify_len - 1; capped = min(raw, ell); cap_trim = raw - capped;
    correct_len = capped; commit_lens = correct_len + 1; block_accept_lens = commit_lens + cap_trim. A cut
    prefix takes its bonus at position ell and clears the emitted tokens after it (READING above). Invalid
    lengths set BAD_ACCEPT and leave the request's entries at -1 (its tokens untouched)."""
    B = len(verify_lens)
    out = {k: np.full(B, -1, np.int32) for k in ("correct_len", "cap_trim", "commit_lens", "block_accept_lens",
                                                   "bonus")}
    out["status"] = np.zeros(B, np.uint32)
    toks = np.array(out_tokens, np.int32)
    for b in range(B):
        o0 = int(row_offsets[b])
        rows = int(row_offsets[b + 1]) - o0
        v, raw = int(verify_lens[b]), int(raw_accept_len[b])
        if rows < 1 or v < 1 or raw < 0 or raw > rows - 1:
            out["status"][b] = ST_BAD_ACCEPT
            continue
        ell = v - 1
        capped = min(raw, ell)
        trim = raw - capped
        out["correct_len"][b] = capped
        out["cap_trim"][b] = trim
        out["commit_lens"][b] = capped + 1
        out["block_accept_lens"][b] = capped + 1 + trim
        if trim > 0:
            out["bonus"][b] = toks[o0 + ell]
            for k in range(ell + 1, rows):
                toks[o0 + k] = -1
        else:
            out["bonus"][b] = int(raw_bonus[b])
    out["out_tokens"] = toks
    return out
