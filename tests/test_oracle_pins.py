"""Pins for the fp64 CPU oracle: what the pages and the mathematics fix, independent of the oracle's code.

Kinds of pin used here (each cites the passage it comes from):
  * worked examples the pages print (tests/golden/*.json);
  * closed forms: acceptance mass min(p,q) plus rejection mass [p-q]_+ equals p; E[accept] = sum min(p,q);
    mean accept length from the survival product; q = p accepts everything and emits m+1 tokens;
  * exact integration: the output is a piecewise-constant function of the uniforms, so its distribution is
    integrated exactly by locating every step with bisection on the oracle itself and weighting by the
    step widths; it must equal the target's own autoregressive distribution (the lossless property);
  * textbook special cases: greedy speculative decoding equals plain greedy decoding (np.argmax) on a toy
    language model, a chain is a tree with one child per node;
  * statistics: chi-square of emitted tokens against p, binomial acceptance rates.
The last section plants plausible mistakes in the oracle (monkeypatch) and checks that the pins catch them.
"""
import json
import os

import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

import oracle
from oracle import verify as ov
from draft_verification_acceptance_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------------------------------
def one_hot_logits(V, tok, hi=5.0, lo=0.0):
    x = np.full(V, lo, np.float32)
    x[tok] = hi
    return x


def pieces(f, lo=0.0, hi=1.0, grid=9, tol=1e-15):
    """Steps of a piecewise-constant, step-monotone f on [lo, hi): list of (a, b, value)."""
    xs = np.linspace(lo, hi, grid)
    xs[-1] = np.nextafter(hi, lo)
    vals = [f(x) for x in xs]
    out = []

    def rec(a, fa, b, fb):
        if fa == fb:
            out.append((a, b, fa))
            return
        if b - a < tol:
            out.append((a, b, fb))
            return
        m = 0.5 * (a + b)
        fm = f(m)
        rec(a, fa, m, fm)
        rec(m, fm, b, fb)

    for i in range(grid - 1):
        rec(xs[i], vals[i], xs[i + 1], vals[i + 1])
    out[-1] = (out[-1][0], hi, out[-1][2])
    merged = [out[0]]
    for a, b, v in out[1:]:
        if v == merged[-1][2]:
            merged[-1] = (merged[-1][0], b, v)
        else:
            merged.append((a, b, v))
    return merged


def chain_call(t_rows, s_rows, toks, us, uf, T, mode="rejection"):
    t = np.asarray(t_rows, np.float32)
    n = len(t)
    s = np.asarray(s_rows, np.float32).reshape(n - 1, t.shape[1]) if s_rows is not None else None
    return oracle.verify_chain(t, np.array([0, n], np.int32), np.asarray(toks, np.int32), mode, draft=s,
                               u_accept=np.asarray(us, np.float64), u_final=np.array([uf], np.float64),
                               temperature=T)


def emitted(o):
    r = int(o["accept_len"][0])
    return tuple(int(x) for x in o["out_tokens"][:r + 1])


# ----------------------------------------------------------------------------------------------------
# worked examples from the pages
# ----------------------------------------------------------------------------------------------------
def _letters(names):
    return [ord(c) - ord("A") for c in names]


def test_commit_worked_example_defgh():
    g = golden("commit_defgh.json")
    V = 32
    X = ord("X") - ord("A")
    verify_in = _letters(g["verify_input"])
    drafts = _letters(g["drafts"])
    # Target rows: row D predicts E, row E predicts F, row F predicts X (so G is rejected); G, H arbitrary.
    nxt = _letters(g["accepted"]) + [X, 0, 0]
    rows = [one_hot_logits(V, t) for t in nxt]
    o = chain_call(rows, None, drafts, [0.5] * 4, 0.5, 1.0, mode="greedy")
    assert int(o["accept_len"][0]) == g["r"]
    assert [chr(ord("A") + t) for t in emitted(o)] == g["new_output"]
    assert int(o["bonus"][0]) == X and g["next_anchor"] == "X"
    slots = np.array([100 + i for i in range(len(verify_in))], np.int64)
    committed_before = len(g["committed_before"])
    c = oracle.commit_indices(np.array([0, 5]), o["accept_len"], o["accept_index"], slots,
                              np.array([committed_before]))
    assert int(c["commit_offsets"][-1]) == g["commit_len"]
    kv_rows = [int(s) - 100 for s in c["src_slots"]]
    assert [g["verify_input"][i] for i in kv_rows] == g["new_valid_kv"]
    assert list(c["dst_pos"]) == list(range(committed_before, committed_before + g["commit_len"]))
    assert int(c["new_seq_lens"][0]) == len(g["committed_after"])
    assert [g["verify_input"][int(s) - 100] for s in c["evict_slots"]] == g["temporary_kv"]


def test_commit_invalid_accept_index_by_hand():
    """Invalid accept_index forms, worked by hand: two requests of 5 rows (rows 0-4 and 5-9, slots 100 + row).
    Request 0 (r = 3) lists rows 2, 2, 4, 7: row 2 twice (committed twice), row 7 outside it (committed as -1);
    the rows it names are {2, 4}, so it evicts rows 0, 1, 3. Request 1 (accept_len 9, clamped to 4) lists its
    rows 5..9 in order: all committed, nothing evicted. Both are flagged BAD_ACCEPT."""
    offs = np.array([0, 5, 10])
    acc = np.array([2, 2, 4, 7, -1, 5, 6, 7, 8, 9])
    slots = np.arange(100, 110, dtype=np.int64)
    c = oracle.commit_indices(offs, np.array([3, 9]), acc, slots, np.array([40, 60]), 5)
    assert list(c["commit_offsets"]) == [0, 4, 9]
    assert list(c["src_slots"]) == [102, 102, 104, -1, 105, 106, 107, 108, 109]
    assert list(c["dst_pos"]) == [40, 41, 42, 43, 60, 61, 62, 63, 64]
    assert list(c["new_seq_lens"]) == [44, 65]
    assert list(c["evict_offsets"]) == [0, 3, 3]
    assert list(c["evict_slots"]) == [100, 101, 103]
    assert all(int(st) & oracle.ST_BAD_ACCEPT for st in c["status"])


def test_verify_len_cutoff_example():
    g = golden("verify_len_cutoff.json")
    V = 32
    drafts = _letters(["E", "F", "G"])
    gstar = 30
    rows = [one_hot_logits(V, t) for t in _letters(["E", "F"]) + [gstar, 7]]
    assert len(rows) == g["verify_len"]
    o = chain_call(rows, None, drafts, [0.5] * 3, 0.5, 1.0, mode="greedy")
    assert int(o["accept_len"][0]) == g["correct_len"]
    out = emitted(o)
    assert len(out) == len(g["output"]) and out[:2] == tuple(_letters(g["accepted"])) and out[2] == gstar
    c = oracle.commit_indices(np.array([0, 4]), o["accept_len"], o["accept_index"], np.arange(4), np.array([0]))
    assert int(c["commit_offsets"][-1]) == g["commit_lens"]
    assert list(c["src_slots"]) == [0, 1, 2]          # rows D, E, F


def test_ragged_offsets_example():
    g = golden("ragged_offsets.json")
    lens = np.array(g["verify_lens"])
    offs = np.zeros(len(lens) + 1, np.int32)
    offs[1:] = np.cumsum(lens)
    assert list(offs) == g["offsets"] and offs[-1] == g["target_rows"]
    V = 16
    rng = np.random.default_rng(0)
    T = int(offs[-1])
    B = len(lens)
    assert T - B == g["extra_draft_budget"]       # draft rows = sum of m_b
    target = rng.standard_normal((T, V)).astype(np.float32)
    toks = np.array([int(np.argmax(target[offs[b] + j])) for b in range(B) for j in range(lens[b] - 1)], np.int32)
    o = oracle.verify_chain(target, offs, toks, "greedy")
    # Drafts equal every argmax: all accepted, so every request commits its whole verify length.
    assert list(o["accept_len"]) == list(lens - 1)
    c = oracle.commit_indices(offs, o["accept_len"], o["accept_index"], np.arange(T), np.zeros(B, np.int32))
    assert list(c["commit_offsets"]) == g["offsets"]


def test_hand_listed_tree():
    g = golden("tree7.json")
    V, N = g["vocab"], len(g["parents"])
    rows = np.stack([one_hot_logits(V, a) for a in g["row_argmax"]])
    o = oracle.verify_tree(rows, np.array(g["parents"]), np.array(g["tokens"]), N, "greedy")
    assert int(o["accept_len"][0]) == g["expected_accept_len"]
    assert int(o["bonus"][0]) == g["expected_bonus"]
    assert list(o["out_tokens"][:g["expected_accept_len"] + 1]) == g["expected_out_tokens"]
    assert list(o["accept_index"][:len(g["expected_path"])]) == g["expected_path"]
    assert all(v == -1 for v in o["accept_index"][len(g["expected_path"]):])


# ----------------------------------------------------------------------------------------------------
# draw
# ----------------------------------------------------------------------------------------------------
def test_draw_special_cases():
    V = 10
    w = np.zeros(V)
    w[6] = 3.0
    for u in (0.0, 0.3, 0.999999):
        assert ov.draw(w, u)[0] == 6
    w = np.ones(V)
    for u in (0.0, 0.05, 0.1 + 1e-9, 0.55, 0.95, 0.999):
        assert ov.draw(w, u)[0] == int(np.floor(u * V))
    # u past the last step through rounding: the largest id with positive weight, never a zero-weight id.
    w = np.array([0.2, 0.8, 0.0, 0.0])
    assert ov.draw(w, ov.U_MAX)[0] == 1
    k, gap, Z = ov.draw(np.array([1.0, 1.0, 2.0]), 0.5)
    assert k == 2 and Z == 4.0 and gap == 0.0


# ----------------------------------------------------------------------------------------------------
# exact integration: lossless chain rejection sampling
# ----------------------------------------------------------------------------------------------------
def _tables(seed, V):
    rng = np.random.default_rng(seed)
    t = [rng.normal(0, 1.5, (V,)), rng.normal(0, 1.5, (V, V)), rng.normal(0, 1.5, (V, V, V))]
    s = [t[0] + rng.normal(0, 1.0, (V,)), t[1] + rng.normal(0, 1.0, (V, V))]
    return [x.astype(np.float32) for x in t], [x.astype(np.float32) for x in s]


def _p(logits, T):
    return softmax(np.asarray(logits, np.float64) / T)


def chain_integration_error(seed=0, V=4, T=1.0):
    """Max |P_spec - P_target| over 3-token sequences for one m=2 rejection round plus exact
    continuation from the target."""
    t, s = _tables(seed, V)

    def p_true(prefix):
        if len(prefix) == 0:
            return _p(t[0], T)
        if len(prefix) == 1:
            return _p(t[1][prefix[0]], T)
        return _p(t[2][prefix[0], prefix[1]], T)

    target = np.zeros((V, V, V))
    for a in range(V):
        for b in range(V):
            target[a, b] = p_true([]) [a] * p_true([a])[b] * p_true([a, b])
    spec = np.zeros((V, V, V))
    q0 = _p(s[0], T)
    for d1 in range(V):
        q1 = _p(s[1][d1], T)
        for d2 in range(V):
            wq = q0[d1] * q1[d2]
            trows = [t[0], t[1][d1], t[2][d1, d2]]
            srows = [s[0], s[1][d1]]

            def run(u1, u2, uf):
                return chain_call(trows, srows, [d1, d2], [u1, u2], uf, T)

            for a1, b1, acc1 in pieces(lambda u: int(run(u, 0.5, 0.5)["accept_len"][0]) >= 1):
                m1 = 0.5 * (a1 + b1)
                regions = [(b1 - a1, m1, 0.5)] if not acc1 else [
                    ((b1 - a1) * (b2 - a2), m1, 0.5 * (a2 + b2))
                    for a2, b2, _ in pieces(lambda u: int(run(m1, u, 0.5)["accept_len"][0]) >= 2)]
                for meas, u1, u2 in regions:
                    for af, bf, _ in pieces(lambda u: int(run(u1, u2, u)["bonus"][0])):
                        y = list(emitted(run(u1, u2, 0.5 * (af + bf))))
                        mass = wq * meas * (bf - af)
                        if len(y) >= 3:
                            spec[y[0], y[1], y[2]] += mass
                        elif len(y) == 2:
                            spec[y[0], y[1]] += mass * p_true(y)
                        else:
                            pa = p_true(y)
                            for b in range(V):
                                spec[y[0], b] += mass * pa[b] * p_true([y[0], b])
    assert abs(target.sum() - 1) < 1e-12
    return float(np.max(np.abs(spec - target)))


@pytest.mark.parametrize("seed,T", [(0, 1.0), (1, 0.7)])
def test_chain_rejection_exact_integration_is_lossless(seed, T):
    assert chain_integration_error(seed, 4, T) < 1e-12


def mass_decomposition_error(seed=3, V=5, T=1.0):
    """One draft position: accept mass of token v must be min(p,q)(v), rejection mass [p-q]_+(v), and
    they add to p(v) (the pages' acceptance / rejection mass identity)."""
    rng = np.random.default_rng(seed)
    t0 = rng.normal(0, 1.5, V).astype(np.float32)
    t1 = rng.normal(0, 1.5, V).astype(np.float32)
    s0 = (t0 + rng.normal(0, 1.0, V)).astype(np.float32)
    p, q = _p(t0, T), _p(s0, T)
    A = np.zeros(V)
    R = np.zeros(V)
    for d in range(V):
        def run(u1, uf):
            return chain_call([t0, t1], [s0], [d], [u1], uf, T)
        for a1, b1, acc in pieces(lambda u: int(run(u, 0.5)["accept_len"][0]) >= 1):
            if acc:
                A[d] += q[d] * (b1 - a1)
            else:
                m1 = 0.5 * (a1 + b1)
                for af, bf, x in pieces(lambda u: int(run(m1, u)["bonus"][0])):
                    R[x] += q[d] * (b1 - a1) * (bf - af)
    err_a = np.max(np.abs(A - np.minimum(p, q)))
    err_r = np.max(np.abs(R - np.maximum(p - q, 0)))
    err_p = np.max(np.abs(A + R - p))
    return max(err_a, err_r, err_p)


def test_accept_plus_reject_mass_is_p():
    assert mass_decomposition_error() < 1e-12


def test_residual_identity_elementwise():
    rng = np.random.default_rng(5)
    for _ in range(20):
        p = softmax(rng.normal(0, 2, 100))
        q = softmax(rng.normal(0, 2, 100))
        w = ov.residual_weights(p, q)
        assert np.max(np.abs(np.minimum(p, q) + w - p)) <= 1e-15
        # sum [p-q]_+ = 1 - sum min(p,q) = TV(p,q)
        assert abs(w.sum() - (1 - np.minimum(p, q).sum())) < 1e-14
        assert abs(w.sum() - 0.5 * np.abs(p - q).sum()) < 1e-14


def test_residual_mass_output_equals_total_variation():
    w = W.tiny_chain(seed=1000)
    o = oracle.verify_chain(w.target, w.offsets, w.draft_tokens, "rejection", draft=w.draft,
                            u_accept=w.u_accept, u_final=w.u_final)
    for b in range(w.batch):
        r = int(o["accept_len"][b])
        m = int(w.offsets[b + 1] - w.offsets[b] - 1)
        p = _p(w.target[w.offsets[b] + r], 1.0)
        if r < m:
            q = _p(w.draft[w.offsets[b] - b + r], 1.0)
            assert abs(o["residual_mass"][b] - 0.5 * np.abs(p - q).sum()) < 1e-12
        else:
            assert abs(o["residual_mass"][b] - 1.0) < 1e-12


# ----------------------------------------------------------------------------------------------------
# statistics on i.i.d. rows
# ----------------------------------------------------------------------------------------------------
def _iid_batch(seed, N, m, V, T):
    rng = np.random.default_rng(seed)
    tl = rng.normal(0, 1.5, (m + 1, V)).astype(np.float32)
    sl = (tl[:m] + rng.normal(0, 1.0, (m, V))).astype(np.float32)
    p = [_p(x, T) for x in tl]
    q = [_p(x, T) for x in sl]
    target = np.tile(tl, (N, 1))
    draft = np.tile(sl, (N, 1))
    toks = np.stack([rng.choice(V, size=N, p=q[j]) for j in range(m)], 1).reshape(-1).astype(np.int32)
    offs = (np.arange(N + 1) * (m + 1)).astype(np.int32)
    ua = rng.random(N * m)
    uf = rng.random(N)
    o = oracle.verify_chain(target, offs, toks, "rejection", draft=draft, u_accept=ua, u_final=uf,
                            temperature=T)
    return o, p, q, offs


def chi_square_pvalues(o, p, offs, m, V):
    N = len(offs) - 1
    pv = []
    r = o["accept_len"]
    for k in range(m + 1):
        sel = np.flatnonzero(r >= k)
        toks = o["out_tokens"][offs[sel] + k]
        obs = np.bincount(toks, minlength=V).astype(float)
        exp = p[k] * len(sel)
        keep = exp >= 5
        o2 = np.append(obs[keep], obs[~keep].sum())
        e2 = np.append(exp[keep], exp[~keep].sum())
        if e2[-1] == 0:
            o2, e2 = o2[:-1], e2[:-1]
        pv.append(stats.chisquare(o2, e2).pvalue)
    return pv


def test_statistics_emitted_tokens_follow_p_and_accept_rates():
    N, m, V, T = 20000, 3, 8, 1.0
    o, p, q, offs = _iid_batch(11, N, m, V, T)
    r = o["accept_len"]
    # Chi-square per emitted position (given the round reached it) against p_k; Bonferroni over positions.
    pv = chi_square_pvalues(o, p, offs, m, V)
    assert min(pv) > 1e-3 / (m + 1), pv
    # P(accept d_j | reached) = sum min(p_{j-1}, q_{j-1}) = 1 - TV, binomial 4 sigma.
    beta = [np.minimum(p[j], q[j]).sum() for j in range(m)]
    for j in range(1, m + 1):
        reached = np.sum(r >= j - 1)
        acc = np.sum(r >= j)
        se = np.sqrt(beta[j - 1] * (1 - beta[j - 1]) / reached)
        assert abs(acc / reached - beta[j - 1]) < 4 * se
    # E[r] = sum_k prod_{j<=k} beta_j (survival product).
    er = sum(np.prod(beta[:k]) for k in range(1, m + 1))
    assert abs(r.mean() - er) < 4 * r.std() / np.sqrt(N)


def test_q_equal_p_accepts_everything():
    rng = np.random.default_rng(2)
    V, m = 32, 6
    tl = rng.normal(0, 2, (m + 1, V)).astype(np.float32)
    for T in (0.05, 0.7, 1.0, 5.0):
        toks = [int(np.argsort(tl[j])[-1 - j % 3]) for j in range(m)]
        o = chain_call(tl, tl[:m], toks, rng.random(m) * 0.999, 0.3, T)
        assert int(o["accept_len"][0]) == m
        assert len(emitted(o)) == m + 1
        assert np.allclose(o["accept_prob"], 1.0)


# ----------------------------------------------------------------------------------------------------
# greedy: speculative greedy == plain greedy on a toy language model
# ----------------------------------------------------------------------------------------------------
def toy_greedy_mismatches(seed, V, L=64, m=4, quantize=True):
    """Run speculative greedy decoding (oracle verify + oracle commit) on a toy LM whose logits depend on
    the last two tokens, with a noisy toy drafter; count positions that differ from plain greedy."""
    rng = np.random.default_rng(seed)
    table = rng.integers(0, 4, (V, V, V)).astype(np.float32) if quantize else \
        rng.normal(0, 1, (V, V, V)).astype(np.float32)
    drafter = table + rng.normal(0, 1.0, table.shape).astype(np.float32)
    plain = [1, 2]
    while len(plain) < L + 2:
        plain.append(int(np.argmax(table[plain[-2], plain[-1]])))
    seq = [1, 2]
    kv_len = 1                      # target KV holds seq[:-1]; seq[-1] is the anchor
    while len(seq) < L + 2:
        ctx = list(seq)
        drafts = []
        for _ in range(m):
            d = int(np.argmax(drafter[ctx[-2], ctx[-1]])) if rng.random() < 0.8 else int(rng.integers(V))
            drafts.append(d)
            ctx.append(d)
        rows = [table[ctx[len(seq) - 2 + j], ctx[len(seq) - 1 + j]] for j in range(m + 1)]
        o = chain_call(rows, None, drafts, [0.5] * m, 0.5, 1.0, mode="greedy")
        r = int(o["accept_len"][0])
        c = oracle.commit_indices(np.array([0, m + 1]), o["accept_len"], o["accept_index"],
                                  np.arange(m + 1), np.array([kv_len]))
        assert list(c["src_slots"]) == list(range(r + 1))
        kv_len = int(c["new_seq_lens"][0])
        seq += list(emitted(o))
        assert kv_len == len(seq) - 1
    return sum(a != b for a, b in zip(seq[:L + 2], plain))


@pytest.mark.parametrize("V,quantize", [(8, True), (32, True), (32, False)])
def test_speculative_greedy_equals_plain_greedy(V, quantize):
    for seed in range(6):
        assert toy_greedy_mismatches(seed, V, quantize=quantize) == 0


def test_block_greedy_planted_prefix():
    # The generator fixes the accept length by construction (np.argmax, forced ties: 30% of rows here).
    w = W.block_greedy(seed=3001, batch=24, vocab=2048, tie_rate=0.3, parallel=False)
    assert w.meta["tie_rows"] > 50
    o = oracle.verify_chain(w.target, w.offsets, w.draft_tokens, "greedy", max_verify_len=16)
    assert list(o["accept_len"]) == list(w.planted_r)


def test_block_greedy_planted_prefix_full_vocab():
    w = W.block_greedy(seed=3000, batch=4, parallel=False)
    o = oracle.verify_chain(w.target, w.offsets, w.draft_tokens, "greedy", max_verify_len=16)
    assert list(o["accept_len"]) == list(w.planted_r)


# ----------------------------------------------------------------------------------------------------
# trees
# ----------------------------------------------------------------------------------------------------
def test_chain_shaped_tree_equals_chain_greedy():
    w = W.tiny_chain(seed=1234, batch=6, m=6, vocab=16)
    oc = oracle.verify_chain(w.target, w.offsets, w.draft_tokens, "greedy")
    N = 7
    parents = np.tile(np.arange(-1, N - 1), w.batch)
    tokens = np.concatenate([[0] + list(w.draft_tokens[b * 6:(b + 1) * 6]) for b in range(w.batch)])
    ot = oracle.verify_tree(w.target, parents, tokens, N, "greedy")
    for k in ("accept_len", "bonus", "out_tokens", "accept_index"):
        assert np.array_equal(oc[k], ot[k]), k
    # also with drafts forced to the argmax prefix of random length
    rng = np.random.default_rng(3)
    tok2 = w.draft_tokens.copy()
    for b in range(w.batch):
        for j in range(rng.integers(0, 7)):
            tok2[b * 6 + j] = np.argmax(w.target[b * 7 + j])
    oc = oracle.verify_chain(w.target, w.offsets, tok2, "greedy")
    tokens = np.concatenate([[0] + list(tok2[b * 6:(b + 1) * 6]) for b in range(w.batch)])
    ot = oracle.verify_tree(w.target, parents, tokens, N, "greedy")
    assert np.array_equal(oc["accept_len"], ot["accept_len"]) and np.array_equal(oc["bonus"], ot["bonus"])
    assert oc["accept_len"].max() > 0


def test_tree_greedy_set_formulation():
    # With distinct sibling tokens the accepted nodes are exactly those whose whole ancestor chain matches
    # the argmax of the parent's row; the accept length is the deepest such node's depth.
    rng = np.random.default_rng(9)
    V, N, B = 6, 24, 40
    target = rng.integers(0, 3, (B * N, V)).astype(np.float32)   # many ties
    parents = np.empty(B * N, np.int64)
    tokens = np.empty(B * N, np.int64)
    for b in range(B):
        used = {}
        parents[b * N] = -1
        tokens[b * N] = 0
        for i in range(1, N):
            while True:
                p = int(rng.integers(0, i))
                free = [t for t in range(V) if t not in used.get(p, set())]
                if free:
                    break
            t = int(rng.choice(free)) if rng.random() < 0.5 else int(np.argmax(target[b * N + p]))
            if t in used.get(p, set()):
                t = int(rng.choice(free))
            used.setdefault(p, set()).add(t)
            parents[b * N + i], tokens[b * N + i] = p, t
    o = oracle.verify_tree(target, parents, tokens, N, "greedy")
    for b in range(B):
        good = {0}
        depth = {0: 0}
        for i in range(1, N):
            p = int(parents[b * N + i])
            depth[i] = depth[p] + 1
            if p in good and tokens[b * N + i] == np.argmax(target[b * N + p]):
                good.add(i)
        r = max(depth[i] for i in good)
        assert int(o["accept_len"][b]) == r
        path = [int(x) - b * N for x in o["accept_index"][b * N:b * N + r + 1]]
        assert sorted(good) == path


def test_chain_shaped_tree_target_only_equals_rejection_with_one_hot_q():
    rng = np.random.default_rng(21)
    V, m, B = 12, 5, 30
    for T in (0.7, 1.0):
        tl = rng.normal(0, 1.5, (B * (m + 1), V)).astype(np.float32)
        toks = rng.integers(0, V, B * m).astype(np.int32)
        for b in range(B):       # make some drafts likely: the row's argmax
            for j in range(m):
                if rng.random() < 0.6:
                    toks[b * m + j] = np.argmax(tl[b * (m + 1) + j])
        draft = np.full((B * m, V), -np.inf, np.float32)
        draft[np.arange(B * m), toks] = 0.0              # q = one-hot(d_{j+1})
        ua = rng.random(B * m)
        uf = rng.random(B)
        offs = (np.arange(B + 1) * (m + 1)).astype(np.int32)
        oc = oracle.verify_chain(tl, offs, toks, "rejection", draft=draft, u_accept=ua, u_final=uf, temperature=T)
        N = m + 1
        parents = np.tile(np.arange(-1, N - 1), B)
        tokens = np.concatenate([[0] + list(toks[b * m:(b + 1) * m]) for b in range(B)])
        u_nodes = np.concatenate([list(ua[b * m:(b + 1) * m]) + [0.5] for b in range(B)])
        ot = oracle.verify_tree(tl, parents, tokens, N, "target_only", u_accept=u_nodes, u_final=uf, temperature=T)
        for k in ("accept_len", "bonus", "out_tokens", "accept_index", "residual_mass"):
            assert np.array_equal(oc[k], ot[k]), k
        assert ((oc["status"] & np.uint32(~oracle.ST_ZERO_Q & 0xFFFFFFFF)) == ot["status"]).all()


def tree_target_only_integration_error(seed=4, V=4, T=1.0, dup=False):
    """Exact integration over (u_root, u_node1, u_final) for a 4-node tree: the first two emitted tokens
    (with exact continuation) must follow p_root(x1) p(x2 | x1)."""
    rng = np.random.default_rng(seed)
    t0 = rng.normal(0, 1.5, V).astype(np.float32)
    t1 = rng.normal(0, 1.5, (V, V)).astype(np.float32)        # row after token a
    parents = np.array([-1, 0, 0, 1])
    a, bb = (1, 1) if dup else (1, 3)
    c = 2
    tokens = np.array([0, a, bb, c])
    rows = np.stack([t0, t1[a], t1[bb], t1[a]])                 # node 3's row is never used at L = 2
    p0 = _p(t0, T)
    target = np.outer(p0, np.ones(V)) * np.stack([_p(t1[x], T) for x in range(V)])
    spec = np.zeros((V, V))

    def run(u0, u1, uf):
        return oracle.verify_tree(rows, parents, tokens, 4, "target_only", u_accept=np.array([u0, u1, 0.5, 0.5]),
                                  u_final=np.array([uf]), temperature=T)

    def path_key(o):
        return tuple(int(x) for x in o["accept_index"][:int(o["accept_len"][0]) + 1])

    for a0, b0, key0 in pieces(lambda u: path_key(run(u, 0.5, 0.5))[:2]):
        m0 = 0.5 * (a0 + b0)
        for a1, b1, _ in pieces(lambda u: path_key(run(m0, u, 0.5))):
            m1 = 0.5 * (a1 + b1)
            for af, bf, _ in pieces(lambda u: int(run(m0, m1, u)["bonus"][0])):
                o = run(m0, m1, 0.5 * (af + bf))
                y = [int(x) for x in o["out_tokens"][:int(o["accept_len"][0]) + 1]]
                mass = (b0 - a0) * (b1 - a1) * (bf - af)
                if len(y) >= 2:
                    spec[y[0], y[1]] += mass
                else:
                    spec[y[0]] += mass * _p(t1[y[0]], T)
    return float(np.max(np.abs(spec - target)))


@pytest.mark.parametrize("dup", [False, True])
def test_tree_target_only_exact_integration_is_lossless(dup):
    assert tree_target_only_integration_error(dup=dup) < 1e-12


def test_tree_target_only_chi_square():
    rng = np.random.default_rng(31)
    V, Bn = 6, 12000
    t0 = rng.normal(0, 1.0, V).astype(np.float32)
    tA = rng.normal(0, 1.0, V).astype(np.float32)
    tB = rng.normal(0, 1.0, V).astype(np.float32)
    # root -> children tokens 0, 1 (nodes 1, 2); node 1 -> children tokens 2, 3 (nodes 3, 4); node 2 leaf
    parents = np.array([-1, 0, 0, 1, 1])
    tokens = np.array([0, 0, 1, 2, 3])
    rows = np.stack([t0, tA, tB, tA, tA])
    N = 5
    o = oracle.verify_tree(np.tile(rows, (Bn, 1)), np.tile(parents, Bn), np.tile(tokens, Bn), N, "target_only",
                           u_accept=rng.random(Bn * N), u_final=rng.random(Bn), temperature=1.0)
    first = o["out_tokens"][np.arange(Bn) * N]
    p0 = _p(t0, 1.0)
    assert stats.chisquare(np.bincount(first, minlength=V), p0 * Bn).pvalue > 1e-3 / 2
    # given the first token was the draft token 0 (node 1 accepted), the second follows node 1's row
    sel = np.flatnonzero(o["accept_len"] >= 1)
    sel = sel[o["accept_index"][sel * N + 1] % N == 1]
    second = o["out_tokens"][sel * N + 1]
    assert stats.chisquare(np.bincount(second, minlength=V), _p(tA, 1.0) * len(sel)).pvalue > 1e-3 / 2


# ----------------------------------------------------------------------------------------------------
# commit invariants and edge cases
# ----------------------------------------------------------------------------------------------------
def test_commit_invariants_on_ragged_workload():
    w = W.ragged(seed=5005, batch=40, vocab=64, parallel=False)
    o = oracle.verify_chain(w.target, w.offsets, w.draft_tokens, "rejection", draft=w.draft, u_accept=w.u_accept,
                            u_final=w.u_final, temperature=w.temperature, max_verify_len=16)
    slots = W.verify_slots_for(w.total_rows)
    seq = W.seq_lens_for(w.batch)
    c = oracle.commit_indices(w.offsets, o["accept_len"], o["accept_index"], slots, seq, 16)
    assert int(c["commit_offsets"][-1]) == int((o["accept_len"] + 1).sum())
    assert int(c["commit_offsets"][-1]) + int(c["evict_offsets"][-1]) == w.total_rows
    for b in range(w.batch):
        lo, r = int(w.offsets[b]), int(o["accept_len"][b])
        s = c["src_slots"][c["commit_offsets"][b]:c["commit_offsets"][b + 1]]
        assert list(s) == list(slots[lo:lo + r + 1])            # path order = the verify prefix
        d = c["dst_pos"][c["commit_offsets"][b]:c["commit_offsets"][b + 1]]
        assert list(d) == list(range(seq[b], seq[b] + r + 1))   # contiguous after seq_lens
        assert c["new_seq_lens"][b] == seq[b] + r + 1
        ev = c["evict_slots"][c["evict_offsets"][b]:c["evict_offsets"][b + 1]]
        assert list(ev) == list(slots[lo + r + 1:int(w.offsets[b + 1])])
    assert not c["status"].any()


def test_edge_cases_statuses():
    V = 16
    rng = np.random.default_rng(4)
    t = rng.normal(0, 1, (3, V)).astype(np.float32)
    s = rng.normal(0, 1, (2, V)).astype(np.float32)
    # m = 0: the anchor row alone, r = 0, bonus drawn from p_0 (or argmax in greedy)
    o = chain_call(t[:1], np.zeros((0, V)), [], [], 0.4, 1.0)
    assert int(o["accept_len"][0]) == 0 and int(o["bonus"][0]) == ov.draw(_p(t[0], 1.0), 0.4)[0]
    o = chain_call(t[:1], None, [], [], 0.4, 1.0, mode="greedy")
    assert int(o["bonus"][0]) == int(np.argmax(t[0]))
    # NaN -> status bit; out-of-range token -> status bit and never accepted; bad uniform -> status bit
    tn = t.copy()
    tn[1, 3] = np.nan
    assert chain_call(tn, s, [1, 2], [0.1, 0.1], 0.5, 1.0)["status"][0] & oracle.ST_NONFINITE
    assert chain_call(tn, None, [1, 2], [0.1, 0.1], 0.5, 1.0, mode="greedy")["status"][0] & oracle.ST_NONFINITE
    o = chain_call(t, s, [V + 3, 2], [0.0, 0.0], 0.5, 1.0)
    assert o["status"][0] & oracle.ST_BAD_TOKEN and int(o["accept_len"][0]) == 0
    assert chain_call(t, s, [1, 2], [1.5, 0.1], 0.5, 1.0)["status"][0] & oracle.ST_BAD_UNIFORM
    assert chain_call(t, s, [1, 2], [0.1, 0.1], np.nan, 1.0)["status"][0] & oracle.ST_BAD_UNIFORM
    # -inf masking: masked ids are never drawn; an all -inf row is non-finite for sampling, fine for greedy
    tm = t.copy()
    tm[:, ::2] = -np.inf
    o = chain_call(tm, s, [1, 3], [0.9, 0.9], 0.7, 1.0)
    assert int(o["bonus"][0]) % 2 == 1 and not o["status"][0] & oracle.ST_NONFINITE
    ta = t.copy()
    ta[2] = -np.inf
    assert chain_call(ta, s, [1, 2], [0.1, 0.1], 0.5, 1.0)["status"][0] & oracle.ST_NONFINITE
    assert not chain_call(ta, None, [1, 2], [0.1, 0.1], 0.5, 1.0, mode="greedy")["status"][0]
    # q(d) = 0 at a draft token with p(d) > 0: alpha = 1, flagged
    sz = s.copy()
    sz[0, 5] = -np.inf
    o = chain_call(t, sz, [5, 2], [0.99, 0.1], 0.5, 1.0)
    assert o["status"][0] & oracle.ST_ZERO_Q and o["accept_prob"][0] == 1.0
    # bad offsets
    o = oracle.verify_chain(t, np.array([0, 2]), np.array([1, 2], np.int32), "greedy")
    assert o["status"][0] & oracle.ST_BAD_OFFSETS
    # bad parent
    o = oracle.verify_tree(t, np.array([-1, 0, 5]), np.array([0, 1, 2]), 3, "greedy")
    assert o["status"][0] & oracle.ST_BAD_PARENT


# ----------------------------------------------------------------------------------------------------
# sparse-q rejection ([EAGLE→DFlash2] §6.5: the selector's K-candidate q is scattered into vocab
# coordinates, zero elsewhere; the residual still spans the whole vocab; greedy rows carry a one-hot q)
# ----------------------------------------------------------------------------------------------------
def chain_call_sparse(t_rows, ids_rows, q_rows, toks, us, uf, T):
    t = np.asarray(t_rows, np.float32)
    n = len(t)
    return oracle.verify_chain(t, np.array([0, n], np.int32), np.asarray(toks, np.int32), "rejection_sparse",
                               u_accept=np.asarray(us, np.float64), u_final=np.array([uf], np.float64),
                               temperature=T, cand_ids=np.asarray(ids_rows).reshape(n - 1, -1),
                               cand_q=np.asarray(q_rows, np.float64).reshape(n - 1, -1))


def _top_candidates(s_logits, K, T):
    """K highest draft logits (distinct ids, descending) and the softmax over just those K at T: the
    selector's candidate set and its normalised conditional q."""
    ids = np.argsort(-np.asarray(s_logits, np.float64), kind="stable")[:K]
    return ids, _p(np.asarray(s_logits, np.float64)[ids], T)


def test_sparse_full_support_equals_dense_rejection():
    # K = V with q = softmax(draft / T): the same proposal as dense rejection, so every output agrees.
    # The candidate order is a random permutation, so a scatter by candidate position would fail.
    rng = np.random.default_rng(41)
    V, T = 24, 0.8
    lens = rng.integers(1, 7, 40)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    R, B = int(offs[-1]), len(lens)
    tl = rng.normal(0, 1.5, (R, V)).astype(np.float32)
    dl = np.concatenate([tl[offs[b]:offs[b + 1] - 1] for b in range(B)]) + rng.normal(0, 0.7, (R - B, V))
    dl = dl.astype(np.float32)
    q = np.stack([_p(x, T) for x in dl])
    toks = np.array([rng.choice(V, p=qq) for qq in q], np.int32)
    ids = np.stack([rng.permutation(V) for _ in range(R - B)]).astype(np.int32)
    ua, uf = rng.random(R - B), rng.random(B)
    od = oracle.verify_chain(tl, offs, toks, "rejection", draft=dl, u_accept=ua, u_final=uf, temperature=T)
    osp = oracle.verify_chain(tl, offs, toks, "rejection_sparse", u_accept=ua, u_final=uf, temperature=T,
                              cand_ids=ids, cand_q=np.take_along_axis(q, ids, 1))
    for k in ("accept_len", "bonus", "out_tokens", "accept_index", "status"):
        assert np.array_equal(od[k], osp[k]), k
    assert np.allclose(od["accept_prob"], osp["accept_prob"], rtol=0, atol=1e-15)
    assert np.allclose(od["residual_mass"], osp["residual_mass"], rtol=0, atol=1e-15)


def test_sparse_one_hot_equals_tree_target_only_on_a_chain():
    # Greedy rows: q = one-hot(d). Rejection with that q is the target-only rule on a chain-shaped tree
    # (each node has one child), pinned separately by exact integration.
    rng = np.random.default_rng(43)
    V, m, B = 10, 4, 40
    for T in (0.6, 1.0):
        tl = rng.normal(0, 1.5, (B * (m + 1), V)).astype(np.float32)
        toks = rng.integers(0, V, B * m).astype(np.int32)
        for i in range(B * m):
            if rng.random() < 0.6:
                toks[i] = np.argmax(tl[(i // m) * (m + 1) + i % m])
        ua, uf = rng.random(B * m), rng.random(B)
        offs = (np.arange(B + 1) * (m + 1)).astype(np.int32)
        osp = oracle.verify_chain(tl, offs, toks, "rejection_sparse", u_accept=ua, u_final=uf, temperature=T,
                                  cand_ids=toks[:, None], cand_q=np.ones((B * m, 1)))
        N = m + 1
        parents = np.tile(np.arange(-1, N - 1), B)
        tokens = np.concatenate([[0] + list(toks[b * m:(b + 1) * m]) for b in range(B)])
        u_nodes = np.concatenate([list(ua[b * m:(b + 1) * m]) + [0.5] for b in range(B)])
        ot = oracle.verify_tree(tl, parents, tokens, N, "target_only", u_accept=u_nodes, u_final=uf, temperature=T)
        for k in ("accept_len", "bonus", "out_tokens", "accept_index", "residual_mass", "status"):
            assert np.array_equal(osp[k], ot[k]), k


def test_sparse_q_covering_p_draws_from_p():
    # p = 1/4 on four tokens (all other logits -inf) and a sparse q of mass 1/2 on each of them: alpha = 1/2, and
    # after a rejection [p - q]_+ is 0 everywhere, so the draw falls back to p (reading R6, ZERO_RESIDUAL): the
    # token is the (floor(4 u) + 1)-th of the four, residual_mass p's total (1), accept_prob 1/2.
    V, sup = 12, [1, 4, 7, 11]
    t0 = np.full(V, -np.inf, np.float32)
    t0[sup] = 0.0
    t1 = np.zeros(V, np.float32)
    for uf in (0.05, 0.3, 0.55, 0.99):
        for u1, rejected in ((0.7, True), (0.2, False)):
            o = chain_call_sparse([t0, t1], [sup], [[0.5] * 4], [sup[2]], [u1], uf, 1.0)
            assert o["accept_prob"][0] == 0.5
            if rejected:
                assert o["accept_len"][0] == 0 and o["status"][0] & oracle.ST_ZERO_RESIDUAL
                assert o["bonus"][0] == sup[int(4 * uf)] and o["residual_mass"][0] == 1.0
            else:
                assert o["accept_len"][0] == 1 and not o["status"][0] & oracle.ST_ZERO_RESIDUAL


def sparse_mass_decomposition_error(seed=7, V=6, K=3, T=0.9):
    """One draft position with a K-candidate q: accept mass of v is min(p, q)(v), rejection mass
    [p - q]_+(v) (equal to p(v) off the candidates), and the two add up to p(v)."""
    rng = np.random.default_rng(seed)
    t0 = rng.normal(0, 1.5, V).astype(np.float32)
    t1 = rng.normal(0, 1.5, V).astype(np.float32)
    ids, qc = _top_candidates(t0 + rng.normal(0, 1.0, V), K, T)
    p = _p(t0, T)
    q = np.zeros(V)
    q[ids] = qc
    A = np.zeros(V)
    R = np.zeros(V)
    for d, qd in zip(ids, qc):
        def run(u1, uf):
            return chain_call_sparse([t0, t1], [ids], [qc], [d], [u1], uf, T)
        for a1, b1, acc in pieces(lambda u: int(run(u, 0.5)["accept_len"][0]) >= 1):
            if acc:
                A[d] += qd * (b1 - a1)
            else:
                m1 = 0.5 * (a1 + b1)
                for af, bf, x in pieces(lambda u: int(run(m1, u)["bonus"][0])):
                    R[x] += qd * (b1 - a1) * (bf - af)
    off = np.setdiff1d(np.arange(V), ids)
    assert np.all(R[off] > 0)          # tokens outside the candidates stay reachable
    return max(np.max(np.abs(A - np.minimum(p, q))), np.max(np.abs(R - np.maximum(p - q, 0))),
               np.max(np.abs(A + R - p)))


def test_sparse_accept_plus_reject_mass_is_p():
    assert sparse_mass_decomposition_error() < 1e-12


def sparse_chain_integration_error(seed=0, V=4, K=2, T=1.0):
    """Exact integration of one m = 2 round with K-candidate proposals (d ~ q over the candidates of the
    row each draft came from) plus exact continuation: the 3-token distribution must be the target's."""
    t, s = _tables(seed, V)

    def p_true(prefix):
        if len(prefix) == 0:
            return _p(t[0], T)
        if len(prefix) == 1:
            return _p(t[1][prefix[0]], T)
        return _p(t[2][prefix[0], prefix[1]], T)

    target = np.zeros((V, V, V))
    for a in range(V):
        for b in range(V):
            target[a, b] = p_true([])[a] * p_true([a])[b] * p_true([a, b])
    spec = np.zeros((V, V, V))
    ids0, q0 = _top_candidates(s[0], K, T)
    for d1, w1 in zip(ids0, q0):
        ids1, q1 = _top_candidates(s[1][d1], K, T)
        for d2, w2 in zip(ids1, q1):
            trows = [t[0], t[1][d1], t[2][d1, d2]]

            def run(u1, u2, uf):
                return chain_call_sparse(trows, [ids0, ids1], [q0, q1], [d1, d2], [u1, u2], uf, T)

            for a1, b1, acc1 in pieces(lambda u: int(run(u, 0.5, 0.5)["accept_len"][0]) >= 1):
                m1 = 0.5 * (a1 + b1)
                regions = [(b1 - a1, m1, 0.5)] if not acc1 else [
                    ((b1 - a1) * (b2 - a2), m1, 0.5 * (a2 + b2))
                    for a2, b2, _ in pieces(lambda u: int(run(m1, u, 0.5)["accept_len"][0]) >= 2)]
                for meas, u1, u2 in regions:
                    for af, bf, _ in pieces(lambda u: int(run(u1, u2, u)["bonus"][0])):
                        y = list(emitted(run(u1, u2, 0.5 * (af + bf))))
                        mass = w1 * w2 * meas * (bf - af)
                        if len(y) >= 3:
                            spec[y[0], y[1], y[2]] += mass
                        elif len(y) == 2:
                            spec[y[0], y[1]] += mass * p_true(y)
                        else:
                            pa = p_true(y)
                            for b in range(V):
                                spec[y[0], b] += mass * pa[b] * p_true([y[0], b])
    return float(np.max(np.abs(spec - target)))


@pytest.mark.parametrize("seed,T", [(0, 1.0), (2, 0.6)])
def test_sparse_rejection_exact_integration_is_lossless(seed, T):
    assert sparse_chain_integration_error(seed, 4, 2, T) < 1e-12


def test_sparse_duplicate_and_invalid_candidates():
    rng = np.random.default_rng(47)
    V = 16
    tl = rng.normal(0, 1.5, (3, V)).astype(np.float32)
    toks = np.array([3, 5], np.int32)
    base_ids = np.array([[3, 7, 9], [5, 1, 2]])
    base_q = np.array([[0.5, 0.3, 0.2], [0.6, 0.3, 0.1]])
    ref = chain_call_sparse(tl, base_ids, base_q, toks, [0.4, 0.9], 0.3, 1.0)
    # a repeated id adds its masses
    dup = chain_call_sparse(tl, [[3, 7, 3, 9], [5, 1, 2, 2]], [[0.2, 0.3, 0.3, 0.2], [0.6, 0.3, 0.05, 0.05]],
                            toks, [0.4, 0.9], 0.3, 1.0)
    for k in ("accept_len", "bonus", "out_tokens", "status"):
        assert np.array_equal(ref[k], dup[k]), k
    assert np.allclose(ref["accept_prob"], dup["accept_prob"], rtol=0, atol=1e-15)
    # entries with an id outside [0, V) or a negative / non-finite mass are reported and left out
    for bad_id, bad_q, bit in ((V, 0.4, oracle.ST_BAD_TOKEN), (-1, 0.4, oracle.ST_BAD_TOKEN),
                               (4, -0.1, oracle.ST_BAD_Q), (4, np.nan, oracle.ST_BAD_Q), (4, np.inf, oracle.ST_BAD_Q)):
        o = chain_call_sparse(tl, np.concatenate([base_ids, [[bad_id], [4]]], 1),
                              np.concatenate([base_q, [[bad_q], [0.0]]], 1), toks, [0.4, 0.9], 0.3, 1.0)
        assert o["status"][0] & bit
        for k in ("accept_len", "bonus", "out_tokens"):
            assert np.array_equal(ref[k], o[k]), k
    # a draft token that is no candidate has q(d) = 0
    o = chain_call_sparse(tl, base_ids, base_q, [4, 5], [0.4, 0.9], 0.3, 1.0)
    assert o["status"][0] & oracle.ST_ZERO_Q and o["accept_prob"][0] == 1.0


# ----------------------------------------------------------------------------------------------------
# the "too close to call" bands and flag_pos, placed by hand
# ----------------------------------------------------------------------------------------------------
# Decisions within 1e-5 of their threshold are flagged and counted instead of compared: |u - alpha| < 1e-5
# for an accept test, a CDF gap < 1e-5 for a draw. Each case below puts u 0.9e-5 or 1.1e-5 from a threshold
# whose value is known in closed form (probabilities 1/4, 1/2, 2/3 ... from logits ln p), so a band of the
# wrong width, a flag on an unexamined test or a flag_pos one position off fails. flag_pos = the position of
# the first flagged decision (the test of d_j: j - 1; the final draw: r; a sample at row j: j), r + 1 if none.
LN = lambda *p: [float(np.log(x)) for x in p]  # noqa: E731


def _flag_cases():
    """(name, oracle call, expected (status NEAR bits, flag_pos, accept_len, first emitted tokens))."""
    A, C = oracle.ST_NEAR_ALPHA, oracle.ST_NEAR_CDF
    cases = []
    # final draw of a lone anchor row, p = [1/4, 1/4, 1/2]: CDF steps at 1/4 and 1/2
    for u, near, tok in ((0.5 - 0.9e-5, True, 1), (0.5 - 1.1e-5, False, 1), (0.5 + 0.9e-5, True, 2),
                         (0.5 + 1.1e-5, False, 2), (0.25 - 0.9e-5, True, 0), (0.25 + 1.1e-5, False, 1),
                         (0.75, False, 2)):
        cases.append((f"anchor draw u={u}", lambda u=u: chain_call([LN(.25, .25, .5)], None, [], [], u, 1.0),
                      (C if near else 0, 0 if near else 1, 0, (tok,))))
    # residual draw: p = [.4, .3, .3], q = [.2, .1, .7], d1 = 2 rejected (alpha 3/7, u .9); w = [.2, .2, 0],
    # Z = .4, normalised step at 1/2 (gap * Z stays above 1e-6: only the 1e-5 band decides)
    for u, near, tok in ((0.5 - 0.9e-5, True, 0), (0.5 - 1.1e-5, False, 0), (0.5 + 0.9e-5, True, 1),
                         (0.5 + 1.1e-5, False, 1)):
        cases.append((f"residual draw u={u}", lambda u=u: chain_call([LN(.4, .3, .3), LN(.5, .25, .25)],
                                                                     [LN(.2, .1, .7)], [2], [0.9], u, 1.0),
                      (C if near else 0, 0 if near else 1, 0, (tok,))))
    # accept test: p = [1/2, 1/2], q = [3/4, 1/4], d1 = 0: alpha = 2/3; row 1 p = [1/2, 1/2], u_final 1/4
    a23 = 2.0 / 3.0
    for du, near, r in ((-0.9e-5, True, 1), (0.9e-5, True, 0), (-1.1e-5, False, 1), (1.1e-5, False, 0)):
        tok = (0, 0) if r == 1 else (1,)           # rejected: residual [0, 1/4] -> token 1
        cases.append((f"accept test du={du}", lambda du=du: chain_call([LN(.5, .5), LN(.5, .5)], [LN(.75, .25)], [0],
                                                                       [a23 + du], 0.25, 1.0),
                      (A if near else 0, 0 if near else r + 1, r, tok)))
    # the third test of a chain is the near one: d = [1, 1, 0] (alpha 1, 1, 2/3) -> flag_pos 2
    rows, drows = [LN(.5, .5)] * 4, [LN(.75, .25)] * 3
    cases.append(("third test near", lambda: chain_call(rows, drows, [1, 1, 0], [0.3, 0.3, a23 - 0.5e-5], 0.25, 1.0),
                  (A, 2, 3, (1, 1, 0, 0))))
    cases.append(("third test clear", lambda: chain_call(rows, drows, [1, 1, 0], [0.3, 0.3, a23 - 2e-5], 0.25, 1.0),
                  (0, 4, 3, (1, 1, 0, 0))))
    # tests after the first rejection are never examined, so never flagged
    cases.append(("unexamined", lambda: chain_call(rows, drows, [0, 0, 0], [0.9, a23 + 1e-7, a23 - 1e-7], 0.5, 1.0),
                  (0, 1, 0, (1,))))
    # the mass clause: p = [.2, .3, .5], q = [.195, .295, .51], d1 = 2 rejected (alpha .98, u .99); w = [.005,
    # .005, 0], Z = .01, normalised step at 1/2: 5e-5 from it is outside the 1e-5 band but gap * Z = 5e-7 < 1e-6
    for u, near in ((0.5 - 5e-5, True), (0.5 - 2e-4, False), (0.5 + 5e-5, True), (0.5 + 2e-4, False)):
        cases.append((f"mass clause u={u}", lambda u=u: chain_call([LN(.2, .3, .5), LN(.3, .3, .4)], [LN(.195, .295, .51)],
                                                                   [2], [0.99], u, 1.0),
                      (C if near else 0, 0 if near else 1, 0, (0 if u < 0.5 else 1,))))
    # tree target-only: root p = [1/4, 1/4, 1/2], children tokens 0 (node 1) and 1 (node 2); node 2 has child
    # token 2 (node 3), node 2's row p = [1/4, 1/4, 1/2]: cumulative masses 1/4, 1/2 at the root, 1/2 at node 2
    rows_t = np.array([LN(.25, .25, .5)] * 4, np.float32)
    par, toks = np.array([-1, 0, 0, 2]), np.array([0, 0, 1, 2])

    def tree(u0, u2, uf):
        ua = np.array([u0, 0.5, u2, 0.5])
        return oracle.verify_tree(rows_t, par, toks, 4, "target_only", u_accept=ua, u_final=np.array([uf]))
    cases.append(("tree root near", lambda: tree(0.25 + 0.9e-5, 0.3, 0.9), (A, 0, 2, (1, 2, 2))))
    cases.append(("tree root clear", lambda: tree(0.25 + 1.1e-5, 0.3, 0.9), (0, 3, 2, (1, 2, 2))))
    cases.append(("tree depth-1 near", lambda: tree(0.3, 0.5 - 0.9e-5, 0.9), (A, 1, 2, (1, 2, 2))))
    cases.append(("tree depth-1 clear", lambda: tree(0.3, 0.5 - 1.1e-5, 0.9), (0, 3, 2, (1, 2, 2))))
    # sample-then-match: p = [1/4, 1/4, 1/2] on every row, drafts [1, 1]: row 1's sample u .5 - 0.9e-5 (token 1,
    # matches d2) is near -> flag_pos 1; all matched, row 2 samples token 2
    rows_s = [LN(.25, .25, .5)] * 3
    for u1, near in ((0.5 - 0.9e-5, True), (0.5 - 1.1e-5, False)):
        cases.append((f"sample-then-match u={u1}",
                      lambda u1=u1: chain_call(rows_s, None, [1, 1], [0.3, u1], 0.9, 1.0, mode="sample_match"),
                      (C if near else 0, 1 if near else 3, 2, (1, 1, 2))))
    return cases


def flag_pin_failures():
    fails = []
    for name, call, (bits, fpos, r, toks) in _flag_cases():
        o = call()
        got = (int(o["status"][0]) & (oracle.ST_NEAR_ALPHA | oracle.ST_NEAR_CDF), int(o["flag_pos"][0]),
               int(o["accept_len"][0]), emitted(o))
        if got != (bits, fpos, r, toks):
            fails.append((name, got, (bits, fpos, r, toks)))
    return fails


def test_flag_bands_and_flag_pos_by_hand():
    assert flag_pin_failures() == []


def test_mass_clause_is_marked():
    """near_mass_only marks exactly the requests whose only flag is the mass clause."""
    o = chain_call([LN(.2, .3, .5), LN(.3, .3, .4)], [LN(.195, .295, .51)], [2], [0.99], 0.5 - 5e-5, 1.0)
    assert o["near_mass_only"][0] and abs(o["residual_mass"][0] - 0.01) < 1e-6
    o = chain_call([LN(.4, .3, .3), LN(.5, .25, .25)], [LN(.2, .1, .7)], [2], [0.9], 0.5 - 0.9e-5, 1.0)
    assert not o["near_mass_only"][0] and o["status"][0] & oracle.ST_NEAR_CDF


# ----------------------------------------------------------------------------------------------------
# planted mistakes: each plausible bug in the oracle must fail one of the pins above
# ----------------------------------------------------------------------------------------------------
def test_pins_catch_swapped_residual(monkeypatch):
    monkeypatch.setattr(ov, "residual_weights", lambda p, q: np.maximum(q - p, 0.0))
    assert mass_decomposition_error() > 1e-3


def test_pins_catch_inverted_ratio(monkeypatch):
    monkeypatch.setattr(ov, "accept_probability", lambda pd, qd: min(1.0, qd / pd) if pd > 0 else 1.0)
    assert mass_decomposition_error() > 1e-3


def test_pins_catch_dropped_min(monkeypatch):
    # alpha = p/q without the min: decisions unchanged for u < 1 but the residual branch is still right;
    # the pin that sees it is the alpha output (accept_prob must stay in [0, 1]).
    monkeypatch.setattr(ov, "accept_probability", lambda pd, qd: pd / qd if qd > 0 else 1.0)
    rng = np.random.default_rng(2)
    tl = rng.normal(0, 2, (3, 8)).astype(np.float32)
    sl = (tl[:2] + rng.normal(0, 2, (2, 8))).astype(np.float32)
    probs = [chain_call(tl, sl, [d, 0], [0.5, 0.5], 0.5, 1.0)["accept_prob"][0] for d in range(8)]
    assert max(probs) > 1.0


def test_pins_catch_draw_off_by_one(monkeypatch):
    orig = ov.draw

    def bad_draw(w, u):
        k, gap, Z = orig(w, u)
        return min(k + 1, len(w) - 1), gap, Z
    monkeypatch.setattr(ov, "draw", bad_draw)
    assert mass_decomposition_error() > 1e-3


def test_pins_catch_strict_vs_nonstrict_cdf(monkeypatch):
    def bad_draw(w, u):           # count(C < u) instead of count(C <= u): only differs on exact steps
        c = np.cumsum(w)
        C = c / c[-1]
        k = int(np.count_nonzero(C < u))
        return min(k, len(w) - 1), 0.0, float(c[-1])
    monkeypatch.setattr(ov, "draw", bad_draw)
    assert ov.draw(np.ones(4), 0.25)[0] == 0      # the rule itself: u on a step edge takes the next id
    monkeypatch.undo()
    assert ov.draw(np.ones(4), 0.25)[0] == 1


def test_pins_catch_highest_index_ties(monkeypatch):
    def bad_argmax(x):
        y = np.where(np.isnan(x), -np.inf, x)
        return int(np.flatnonzero(y == np.max(y))[-1])
    monkeypatch.setattr(ov, "argmax_lowest", bad_argmax)
    assert sum(toy_greedy_mismatches(s, 8) for s in range(4)) > 0


def test_pins_catch_missing_temperature(monkeypatch):
    monkeypatch.setattr(ov, "softmax_T", lambda x, T: softmax(x))
    assert chain_integration_error(1, 4, 0.7) > 1e-3


def test_pins_catch_residual_restricted_to_candidates(monkeypatch):
    # a residual that drops the mass outside the candidate set makes those tokens unreachable
    monkeypatch.setattr(ov, "residual_weights", lambda p, q: np.where(q > 0, np.maximum(p - q, 0.0), 0.0))
    with pytest.raises(AssertionError):
        sparse_mass_decomposition_error()
    assert sparse_chain_integration_error(0, 4, 2, 1.0) > 1e-3


def test_pins_catch_q_indexed_by_candidate_position(monkeypatch):
    def bad_sparse_q(ids, probs, V):
        q = np.zeros(V)
        q[:len(probs)] = probs
        return q, 0
    monkeypatch.setattr(ov, "sparse_q", bad_sparse_q)
    assert sparse_chain_integration_error(0, 4, 2, 1.0) > 1e-3


def test_p_zero_is_never_accepted():
    # accept iff u < alpha: with p(d) = 0 even u = 0 rejects (u <= alpha would accept it).
    V = 8
    t = np.zeros((2, V), np.float32)
    t[0, 3] = -np.inf
    s = np.zeros((1, V), np.float32)
    o = chain_call(t, s, [3], [0.0], 0.5, 1.0)
    assert int(o["accept_len"][0]) == 0 and o["accept_prob"][0] == 0.0


def test_pins_catch_flag_band_ten_times_too_wide(monkeypatch):
    monkeypatch.setattr(ov, "NEAR", 1e-4)
    assert any(n.startswith(("anchor", "residual", "accept", "tree", "sample")) for n, _, _ in flag_pin_failures())


def test_pins_catch_flag_band_ten_times_too_narrow(monkeypatch):
    monkeypatch.setattr(ov, "NEAR", 1e-6)
    assert len(flag_pin_failures()) >= 5


def test_pins_catch_mass_clause_dropped_or_widened(monkeypatch):
    monkeypatch.setattr(ov, "near_cdf_mass", lambda gap, Z: False)
    assert any(n.startswith("mass clause") for n, _, _ in flag_pin_failures())
    monkeypatch.setattr(ov, "near_cdf_mass", lambda gap, Z: gap * Z < 1e-5)
    assert any(n.startswith("mass clause") for n, _, _ in flag_pin_failures())


@pytest.mark.parametrize("shift", [1, -1])
def test_pins_catch_flag_pos_off_by_one(monkeypatch, shift):
    """flag_pos one position late or early (on flagged requests) fails the hand-placed cases."""
    def shifted(fn):
        def call(*a, **k):
            o = fn(*a, **k)
            near = (o["status"] & (oracle.ST_NEAR_ALPHA | oracle.ST_NEAR_CDF)) != 0
            o["flag_pos"] = np.where(near, o["flag_pos"] + shift, o["flag_pos"])
            return o
        return call
    monkeypatch.setattr(oracle, "verify_chain", shifted(ov.verify_chain))
    monkeypatch.setattr(oracle, "verify_tree", shifted(ov.verify_tree))
    fails = {n.split(" u=")[0].split(" du=")[0] for n, _, _ in flag_pin_failures()}
    assert {"anchor draw", "residual draw", "accept test", "third test near", "tree root near",
            "tree depth-1 near", "sample-then-match"} <= fails
