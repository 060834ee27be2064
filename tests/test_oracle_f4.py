"""Pins for the oracle's sample-then-match verify and vocab (grammar) mask (oracle/verify.py).

  * exact integration: for every fixed draft pair, one sample-then-match round followed by exact continuation
    from the target gives the target's own distribution over 3-token sequences (also under a vocab mask, where
    the target is the masked one); chain rejection with masked target rows and unmasked draft rows is
    lossless with respect to the masked target; the first token of a masked target-only tree follows the
    masked p;
  * hand checks: which uniform serves which row (equal logits: the inverse CDF of u on V equal steps is
    floor(V u)); the packed mask layout (tests/golden/vocab_mask_layout.json);
  * special cases and identities: at a very low temperature sample-then-match equals greedy; an all-ones mask
    equals no mask in every mode; greedy under a mask equals the argmax over the allowed id set; masked
    draft tokens are never accepted; a row with nothing allowed is non-finite;
  * planted mistakes (monkeypatch) that the pins catch.
"""
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import verify as ov
from test_oracle_pins import pieces, _tables

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def words_from_allowed(allowed_rows, V):
    """Packed allowed-token bits, built with plain integer shifts (token v: bit v % 32 of word v // 32)."""
    W = (V + 31) // 32
    out = np.zeros((len(allowed_rows), W), np.uint32)
    for i, allowed in enumerate(allowed_rows):
        for v in allowed:
            out[i, v // 32] |= np.uint32(1 << (v % 32))
    return out


def chain(t_rows, toks, mode, us=None, uf=0.5, T=1.0, s_rows=None, mask=None):
    t = np.asarray(t_rows, np.float32)
    n = len(t)
    s = None if s_rows is None else np.asarray(s_rows, np.float32).reshape(n - 1, t.shape[1])
    return oracle.verify_chain(t, np.array([0, n], np.int32), np.asarray(toks, np.int32), mode, draft=s,
                               u_accept=None if us is None else np.asarray(us, np.float64),
                               u_final=np.array([uf], np.float64), temperature=T, vocab_mask=mask)


def emitted(o):
    r = int(o["accept_len"][0])
    return tuple(int(x) for x in o["out_tokens"][:r + 1])


# ----------------------------------------------------------------------------------------------------
# sample-then-match: exact integration
# ----------------------------------------------------------------------------------------------------
def _masked_p(logits, T, allowed=None):
    x = np.asarray(logits, np.float64) / T
    if allowed is None:
        return softmax(x)
    p = np.zeros(len(x))
    p[list(allowed)] = softmax(x[list(allowed)])
    return p


def sample_match_integration_error(seed=0, V=4, T=1.0, masked=False):
    """Max over fixed drafts (d1, d2) of max |P_spec - P_target| over 3-token sequences: one sample-then-match
    round (m = 2) plus exact continuation from the target. With `masked`, row k of every prefix disallows
    token (k + seed) % V and the target is the masked distribution."""
    t, _ = _tables(seed, V)
    allowed = [None, None, None]
    if masked:
        allowed = [[v for v in range(V) if v != (k + seed) % V] for k in range(3)]
    words = None if not masked else words_from_allowed(allowed, V)

    def p_true(prefix):
        k = len(prefix)
        row = t[0] if k == 0 else (t[1][prefix[0]] if k == 1 else t[2][prefix[0], prefix[1]])
        return _masked_p(row, T, allowed[k])

    target = np.zeros((V, V, V))
    for a in range(V):
        for b in range(V):
            target[a, b] = p_true([])[a] * p_true([a])[b] * p_true([a, b])
    worst = 0.0
    for d1 in range(V):
        for d2 in range(V):
            rows = [t[0], t[1][d1], t[2][d1, d2]]

            def run(u0, u1, uf):
                return chain(rows, [d1, d2], "sample_match", [u0, u1], uf, T, mask=words)

            def key(o, n):   # the first n emitted tokens and whether n drafts were accepted
                return emitted(o)[:n] + (int(o["accept_len"][0]) >= n,)

            spec = np.zeros((V, V, V))
            for a0, b0, _ in pieces(lambda u: key(run(u, 0.5, 0.5), 1)):
                m0 = 0.5 * (a0 + b0)
                o0 = run(m0, 0.5, 0.5)
                if int(o0["accept_len"][0]) == 0:
                    y0 = emitted(o0)[0]
                    pa = p_true([y0])
                    for b in range(V):
                        spec[y0, b] += (b0 - a0) * pa[b] * p_true([y0, b])
                    continue
                for a1, b1, _ in pieces(lambda u: key(run(m0, u, 0.5), 2)):
                    m1 = 0.5 * (a1 + b1)
                    o1 = run(m0, m1, 0.5)
                    if int(o1["accept_len"][0]) == 1:
                        y = emitted(o1)
                        spec[y[0], y[1]] += (b0 - a0) * (b1 - a1) * p_true(list(y))
                        continue
                    for af, bf, _ in pieces(lambda u: int(run(m0, m1, u)["bonus"][0])):
                        y = emitted(run(m0, m1, 0.5 * (af + bf)))
                        spec[y[0], y[1], y[2]] += (b0 - a0) * (b1 - a1) * (bf - af)
            worst = max(worst, float(np.max(np.abs(spec - target))))
    return worst


@pytest.mark.parametrize("seed,T,masked", [(0, 1.0, False), (1, 0.7, False), (2, 1.0, True)])
def test_sample_match_exact_integration_is_lossless(seed, T, masked):
    assert sample_match_integration_error(seed, 4, T, masked) < 1e-12


def test_sample_match_uniform_assignment_hand_check():
    # Equal logits over V = 4: p = 1/4 each, draw(u) = floor(4u). Row 0 takes u_accept[0] = 0.1 -> 0, row 1
    # u_accept[1] = 0.6 -> 2, row 2 u_final = 0.9 -> 3.
    rows = np.zeros((3, 4), np.float32)
    o = chain(rows, [0, 2], "sample_match", [0.1, 0.6], 0.9)
    assert emitted(o) == (0, 2, 3) and o["bonus"][0] == 3 and o["accept_len"][0] == 2
    assert np.allclose(o["accept_prob"], [0.25, 0.25]) and o["residual_mass"][0] == -1 and o["status"][0] == 0
    o = chain(rows, [0, 1], "sample_match", [0.1, 0.6], 0.9)
    assert emitted(o) == (0, 2) and o["bonus"][0] == 2 and list(o["out_tokens"]) == [0, 2, -1]
    o = chain(rows, [3, 1], "sample_match", [0.1, 0.6], 0.9)
    assert emitted(o) == (0,) and list(o["accept_prob"]) == [0.25, -1.0]


def test_sample_match_low_temperature_equals_greedy():
    rng = np.random.default_rng(5)
    V, B = 50, 24
    for b in range(B):
        m = int(rng.integers(0, 7))
        rows = rng.normal(0, 1, (m + 1, V)).astype(np.float32)
        top = rows.argmax(1)
        rows[np.arange(m + 1), top] += 1.0            # a clear winner per row
        k = int(rng.integers(0, m + 1))
        toks = [int(top[j]) if j < k else int((top[j] + 1) % V) for j in range(m)]
        us = rng.uniform(0.01, 0.99, m)
        g = chain(rows, toks, "greedy")
        s = chain(rows, toks, "sample_match", us, float(rng.uniform(0.01, 0.99)), T=0.02)
        assert emitted(g) == emitted(s) and g["bonus"][0] == s["bonus"][0]
        assert s["status"][0] == 0


def test_sample_match_reports_match_probability_and_flags():
    rng = np.random.default_rng(9)
    V = 30
    rows = rng.normal(0, 1.5, (4, V)).astype(np.float32)
    toks = [3, 7, V + 5]                      # the last draft token is out of range
    T = 0.8
    o = chain(rows, toks, "sample_match", [0.0, 0.0, 0.2], 0.3, T=T)
    r = int(o["accept_len"][0])
    for j in range(min(r + 1, 3)):
        want = softmax(rows[j].astype(np.float64) / T)[toks[j]] if toks[j] < V else 0.0
        assert abs(o["accept_prob"][j] - want) < 1e-12
    assert o["status"][0] & ov.ST_BAD_TOKEN
    o = chain(rows[:3], toks[:2], "sample_match", [np.nan, 0.5], 1.5, T=T)
    assert o["status"][0] & ov.ST_BAD_UNIFORM


# ----------------------------------------------------------------------------------------------------
# vocab mask
# ----------------------------------------------------------------------------------------------------
def _golden_rows(g):
    V = g["vocab"]
    rows = np.zeros((2, V), np.float32)
    for i, key in enumerate(("row_a", "row_b")):
        for tok, val in g[key].items():
            rows[i, int(tok)] = val
    return rows


def test_mask_layout_golden():
    with open(os.path.join(GOLDEN, "vocab_mask_layout.json")) as f:
        g = json.load(f)
    V = g["vocab"]
    words = np.array([g["mask_words"], g["mask_words"]], np.uint32)
    assert np.array_equal(words[0], words_from_allowed([g["allowed"]], V)[0])
    rows = _golden_rows(g)
    for i in range(2):
        x = ov.mask_row(rows[i].astype(np.float64), words[i])
        assert sorted(np.flatnonzero(np.isfinite(x)).tolist()) == g["allowed"]
        assert ov.argmax_lowest(x) == g["expected_masked_argmax"][i]
    for d1, key in ((33, "greedy_d1_33"), (10, "greedy_d1_10")):
        o = chain(rows, [d1], "greedy", mask=words)
        assert o["accept_len"][0] == g[key]["accept_len"]
        assert list(o["out_tokens"]) == g[key]["out_tokens"] and o["bonus"][0] == g[key]["bonus"]
        assert o["status"][0] == 0


def _random_chain_batch(rng, B, V, max_m):
    lens = rng.integers(1, max_m + 2, B)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(offs[-1])
    target = rng.normal(0, 2, (T, V)).astype(np.float32)
    draft = target[np.concatenate([np.arange(offs[b], offs[b + 1] - 1) for b in range(B)])] \
        + rng.normal(0, 1, (T - B, V)).astype(np.float32)
    toks = rng.integers(0, V, T - B).astype(np.int32)
    u = rng.random(T - B)
    uf = rng.random(B)
    return target, offs, draft, toks, u, uf


def test_all_ones_mask_equals_no_mask():
    rng = np.random.default_rng(11)
    V, B = 45, 6
    target, offs, draft, toks, u, uf = _random_chain_batch(rng, B, V, 4)
    ones = np.full((len(target), (V + 31) // 32), 0xFFFFFFFF, np.uint32)
    K = 5
    ids = np.stack([rng.choice(V, K, replace=False) for _ in range(len(draft))]).astype(np.int32)
    qs = rng.dirichlet(np.ones(K), len(draft)).astype(np.float32)
    for mode in ("greedy", "rejection", "rejection_sparse", "sample_match"):
        kw = dict(draft=draft if mode == "rejection" else None, u_accept=u, u_final=uf, temperature=0.9,
                  cand_ids=ids, cand_q=qs)
        a = oracle.verify_chain(target, offs, toks, mode, **kw)
        b = oracle.verify_chain(target, offs, toks, mode, vocab_mask=ones, **kw)
        for key in ("accept_len", "bonus", "out_tokens", "accept_index", "status", "accept_prob", "residual_mass"):
            assert np.array_equal(a[key], b[key], equal_nan=True), (mode, key)
    N = 7
    parents = np.array([-1, 0, 0, 1, 1, 2, 3] * 2, np.int32)
    ttoks = rng.integers(0, V, 2 * N).astype(np.int32)
    trows = rng.normal(0, 2, (2 * N, V)).astype(np.float32)
    ones = np.full((2 * N, (V + 31) // 32), 0xFFFFFFFF, np.uint32)
    for mode in ("greedy", "target_only"):
        kw = dict(u_accept=rng.random(2 * N), u_final=rng.random(2), temperature=1.0)
        a = oracle.verify_tree(trows, parents, ttoks, N, mode, **kw)
        b = oracle.verify_tree(trows, parents, ttoks, N, mode, vocab_mask=ones, **kw)
        for key in ("accept_len", "bonus", "out_tokens", "accept_index", "status", "accept_prob", "residual_mass"):
            assert np.array_equal(a[key], b[key], equal_nan=True), (mode, key)


def test_greedy_under_mask_is_argmax_over_allowed_set():
    rng = np.random.default_rng(12)
    V = 70
    for trial in range(30):
        m = int(rng.integers(0, 5))
        rows = rng.integers(-3, 4, (m + 1, V)).astype(np.float32)    # integer logits: many ties
        allowed = [sorted(rng.choice(V, int(rng.integers(1, V)), replace=False).tolist()) for _ in range(m + 1)]
        words = words_from_allowed(allowed, V)
        best = [max(al, key=lambda v: (rows[j, v], -v)) for j, al in enumerate(allowed)]
        k = int(rng.integers(0, m + 1))
        toks = [best[j] if j < k else (best[j] + 1) % V for j in range(m)]
        o = chain(rows, toks, "greedy", mask=words)
        r = int(o["accept_len"][0])
        assert r == k and o["bonus"][0] == best[k]
        assert o["status"][0] == 0


def masked_rejection_integration_error(seed=0, V=4, T=1.0):
    """Chain rejection (m = 2) with masked target rows and unmasked draft rows, drafts drawn from the
    unmasked q: the emitted 3-token distribution equals the masked target's (row k disallows token
    (k + seed + 1) % V; a masked draft token has p(d) = 0 and is always rejected)."""
    t, s = _tables(seed, V)
    allowed = [[v for v in range(V) if v != (k + seed + 1) % V] for k in range(3)]
    words = words_from_allowed(allowed, V)

    def p_true(prefix):
        k = len(prefix)
        row = t[0] if k == 0 else (t[1][prefix[0]] if k == 1 else t[2][prefix[0], prefix[1]])
        return _masked_p(row, T, allowed[k])

    target = np.zeros((V, V, V))
    for a in range(V):
        for b in range(V):
            target[a, b] = p_true([])[a] * p_true([a])[b] * p_true([a, b])
    spec = np.zeros((V, V, V))
    q0 = softmax(s[0].astype(np.float64) / T)
    for d1 in range(V):
        q1 = softmax(s[1][d1].astype(np.float64) / T)
        for d2 in range(V):
            wq = q0[d1] * q1[d2]
            rows = [t[0], t[1][d1], t[2][d1, d2]]
            srows = [s[0], s[1][d1]]

            def run(u1, u2, uf):
                return chain(rows, [d1, d2], "rejection", [u1, u2], uf, T, s_rows=srows, mask=words)

            for a1, b1, acc1 in pieces(lambda u: int(run(u, 0.5, 0.5)["accept_len"][0]) >= 1):
                m1 = 0.5 * (a1 + b1)
                regions = [(b1 - a1, m1, 0.5)] if not acc1 else [
                    ((b1 - a1) * (b2 - a2), m1, 0.5 * (a2 + b2))
                    for a2, b2, _ in pieces(lambda u: int(run(m1, u, 0.5)["accept_len"][0]) >= 2)]
                for meas, u1, u2 in regions:
                    for af, bf, _ in pieces(lambda u: int(run(u1, u2, u)["bonus"][0])):
                        y = emitted(run(u1, u2, 0.5 * (af + bf)))
                        mass = wq * meas * (bf - af)
                        if len(y) == 3:
                            spec[y] += mass
                        elif len(y) == 2:
                            spec[y[0], y[1]] += mass * p_true(list(y))
                        else:
                            pa = p_true(list(y))
                            for b in range(V):
                                spec[y[0], b] += mass * pa[b] * p_true([y[0], b])
    return float(np.max(np.abs(spec - target)))


@pytest.mark.parametrize("seed,T", [(0, 1.0), (3, 0.8)])
def test_masked_rejection_exact_integration_is_lossless(seed, T):
    assert masked_rejection_integration_error(seed, 4, T) < 1e-12


def test_masked_tree_target_only_first_token_follows_masked_p():
    # Root with children 1 (token 0) and 2 (token 2); row 0 disallows token 0. Integrate over (u_root, u_final):
    # the first emitted token follows the masked p_root, and child 1 (masked token) is never accepted.
    rng = np.random.default_rng(21)
    V, T = 4, 1.0
    rows = rng.normal(0, 1.5, (3, V)).astype(np.float32)
    allowed = [[1, 2, 3], list(range(V)), list(range(V))]
    words = words_from_allowed(allowed, V)
    parents = np.array([-1, 0, 0], np.int32)
    toks = np.array([0, 0, 2], np.int32)

    def run(u0, uf):
        return oracle.verify_tree(rows, parents, toks, 3, "target_only", u_accept=np.array([u0, 0.5, 0.5]),
                                  u_final=np.array([uf]), temperature=T, vocab_mask=words)

    dist = np.zeros(V)
    def key(o):
        return int(o["accept_len"][0]), int(o["out_tokens"][0])

    for a0, b0, _ in pieces(lambda u: key(run(u, 0.5))):
        o = run(0.5 * (a0 + b0), 0.5)
        if int(o["accept_len"][0]) >= 1:
            assert int(o["accept_index"][1]) == 2          # only the allowed child can be accepted
            dist[int(o["out_tokens"][0])] += b0 - a0
            continue
        for af, bf, _ in pieces(lambda u: int(run(0.5 * (a0 + b0), u)["bonus"][0])):
            dist[int(run(0.5 * (a0 + b0), 0.5 * (af + bf))["bonus"][0])] += (b0 - a0) * (bf - af)
    assert np.max(np.abs(dist - _masked_p(rows[0], T, allowed[0]))) < 1e-12


def test_mask_statuses():
    V = 40
    rows = np.zeros((3, V), np.float32)
    rows[0, 5] = np.nan                       # NaN and +inf at masked positions are erased by the mask
    rows[1, 6] = np.inf
    allowed = [[1, 2, 3], [7, 8], [0, 39]]
    words = words_from_allowed(allowed, V)
    for mode, kw in (("greedy", {}), ("sample_match", {"us": [0.3, 0.3]}),
                     ("rejection", {"us": [0.3, 0.3], "s_rows": np.zeros((2, V))})):
        o = chain(rows, [5, 7], mode, mask=words, **kw)
        assert o["status"][0] & ov.ST_NONFINITE == 0, mode
        assert o["accept_len"][0] == 0, mode           # d1 = 5 is masked: never accepted
        if mode != "greedy":
            assert o["accept_prob"][0] == 0.0
        assert o["out_tokens"][0] in allowed[0]
    empty = words.copy()
    empty[1] = 0                                        # row 1 allows nothing
    for mode, kw in (("greedy", {}), ("sample_match", {"us": [0.3, 0.3]})):
        o = chain(rows, [1, 7], mode, mask=empty, **kw)
        assert o["status"][0] & ov.ST_NONFINITE, mode
    trows = np.zeros((3, V), np.float32)
    o = oracle.verify_tree(trows, np.array([-1, 0, 0], np.int32), np.array([0, 1, 2], np.int32), 3, "greedy",
                           vocab_mask=np.array([words[0], words[1], np.zeros_like(words[0])]))
    assert o["status"][0] & ov.ST_NONFINITE


# ----------------------------------------------------------------------------------------------------
# planted mistakes
# ----------------------------------------------------------------------------------------------------
def test_pins_catch_match_against_the_previous_draft(monkeypatch):
    def shifted(ps, toks, tok_ok, us):
        m = len(toks)
        alphas = []
        for j in range(m + 1):
            t, _, _ = ov.draw(ps[j], us[j])
            if j < m:
                prev = toks[j - 1] if j > 0 else toks[0]           # off by one draft position
                alphas.append(ps[j][prev])
                if t == prev:
                    continue
            return j, t, alphas, None
    monkeypatch.setattr(ov, "sample_then_match", shifted)
    assert sample_match_integration_error(0, 4, 1.0) > 1e-3


def test_pins_catch_reversed_cdf(monkeypatch):
    real = ov.draw
    monkeypatch.setattr(ov, "draw", lambda w, u: real(w, ov.U_MAX - u))
    with pytest.raises(AssertionError):
        test_sample_match_uniform_assignment_hand_check()


def test_pins_catch_reversed_mask_bit_order(monkeypatch):
    def reversed_bits(x, words):
        if words is None:
            return x
        v = np.arange(len(x))
        allowed = (np.asarray(words, np.uint64)[v >> 5] >> (31 - (v & 31)).astype(np.uint64)) & np.uint64(1)
        return np.where(allowed == 1, x, -np.inf)
    monkeypatch.setattr(ov, "mask_row", reversed_bits)
    with pytest.raises(AssertionError):
        test_mask_layout_golden()


def test_pins_catch_an_ignored_mask(monkeypatch):
    monkeypatch.setattr(ov, "mask_row", lambda x, words: x)
    assert masked_rejection_integration_error(0, 4, 1.0) > 1e-3
    assert sample_match_integration_error(2, 4, 1.0, True) > 1e-3
