"""CPU pins of the planner / cap_trim oracle (oracle/plan.py).

Each function is checked against what the pages and the mathematics fix: the pages' worked examples
(golden files, each with its citation), brute force over every per-request length vector on tiny inputs, an
independent formulation of the ranking (the pairwise count the pages describe for the device kernel),
special cases (flat SPS table, empty and full budgets) and invariants. The last section plants plausible
mistakes in the oracle and checks that a pin catches each.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import plan as op

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------------------------------
# worked examples
# ----------------------------------------------------------------------------------------------------
def test_budget_k_table():
    g = _golden("dspark_budget_k4.json")
    K, theta = op.budget_from_survival(g["history_survival"], g["sps_rows"], g["sps"])
    assert K == g["K_star"]
    assert np.allclose(theta, g["predicted_tokens_per_s"], atol=1e-5)
    # the columns of the table: target rows R + K and predicted output N(K)
    R = len(g["history_survival"])
    for k, rows, n, t in zip(g["K"], g["target_rows"], g["predicted_output"], g["predicted_tokens_per_s"]):
        assert rows == R + k
        assert abs(n * op.sps_at(rows, g["sps_rows"], g["sps"]) - t) < 1e-9


def test_topk_allocation_example():
    g = _golden("dspark_topk_allocation.json")
    o = op.plan_from_survival(g["current_survival"], g["budget"])
    assert list(o["selected"]) == g["selected_extra"]
    assert list(o["verify_lens"]) == g["verify_lens"]
    assert int(o["offsets"][-1]) == g["target_rows"]
    # the historical winners of the same budget belong to other requests (only K is carried over)
    h = op.plan_from_survival(_golden("dspark_budget_k4.json")["history_survival"], g["budget"])
    assert list(h["selected"]) == [g["history_top4_owners"]["A"], g["history_top4_owners"]["B"]]


def test_ragged_offsets_example():
    g = _golden("ragged_offsets.json")
    assert list(op.ragged_offsets(g["verify_lens"])) == g["offsets"]
    assert int(op.ragged_offsets(g["verify_lens"])[-1]) == g["target_rows"]
    assert sum(v - 1 for v in g["verify_lens"]) == g["extra_draft_budget"]


def test_cap_trim_examples():
    g = _golden("verify_len_cutoff.json")
    for ex in g["cap_trim_examples"]:
        ell, raw = ex["ell"], ex["raw_correct_len"]
        rows = 8
        offs = np.array([0, rows], np.int32)
        toks = np.arange(100, 100 + rows, dtype=np.int32)
        toks[raw] = 900                      # the correction / bonus of the full-width verify
        toks[raw + 1:] = -1
        o = op.cap_trim(offs, [ell + 1], [raw], [900], toks)
        assert o["cap_trim"][0] == ex["cap_trim"]
        assert o["correct_len"][0] == min(raw, ell)
        assert o["commit_lens"][0] == min(raw, ell) + 1
        assert o["block_accept_lens"][0] == o["commit_lens"][0] + ex["cap_trim"]
        if ex["cap_trim"] == 0:
            assert o["bonus"][0] == 900
        else:   # cut at ell: the accepted draft at position ell is emitted as the bonus
            assert o["bonus"][0] == toks[ell]
            assert list(o["out_tokens"][ell + 1:]) == [-1] * (rows - ell - 1)
    # the D E F G example: verify_len 4, E F accepted, G rejected -> correct_len 2, commit 3
    o = op.cap_trim(np.array([0, 4]), [g["verify_len"]], [g["correct_len"]], [7], np.array([1, 2, 7, -1]))
    assert o["correct_len"][0] == g["correct_len"] and o["commit_lens"][0] == g["commit_lens"]


# ----------------------------------------------------------------------------------------------------
# brute force and independent formulations
# ----------------------------------------------------------------------------------------------------
def _theta(A, lens, sps_rows, sps):
    R = A.shape[0]
    N = R + sum(float(A[r, :lens[r]].astype(np.float64).sum()) for r in range(R))
    return N * op.sps_at(R + sum(lens), sps_rows, sps)


@pytest.mark.parametrize("seed", range(12))
def test_budget_is_the_best_of_every_length_vector(seed):
    """max over every l in {0..W}^R of N(l) * SPS(M(l)) equals the prefix-budget argmax, and the top-K
    allocation at K* reaches it (survival non-increasing along positions, as a product of confidences)."""
    rng = np.random.default_rng(seed)
    R, W = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    conf = rng.uniform(0.05, 1.0, (R, W)).astype(np.float32)
    A, _ = op.survival(conf)
    rows = np.arange(R, R * (W + 1) + 1)
    sps = np.cumsum(-rng.uniform(0, 30, len(rows))) + 1000.0      # steps/s falls as rows grow
    best = max(_theta(A, lens, rows, sps) for lens in itertools.product(range(W + 1), repeat=R))
    K, theta = op.budget_from_survival(A, rows, sps)
    assert abs(theta[K] - best) <= 1e-9 * best
    lay = op.plan_from_survival(A, K)
    assert abs(_theta(A, list(lay["selected"]), rows, sps) - best) <= 1e-9 * best


# ----------------------------------------------------------------------------------------------------
# the additive cost-table budget: K* = argmax N(K) / T(R, R + K), T(R, M) = T_req(R) + T_tok(M)
# ----------------------------------------------------------------------------------------------------
def test_cost_budget_reproduces_the_k_table():
    """With no per-batch term and T_tok = 1 / SPS at every table point (the table has a point at every M
    the search visits) the additive objective is the SPS objective: the pages' K table, K* = 4."""
    g = _golden("dspark_budget_k4.json")
    tok = 1.0 / np.asarray(g["sps"], np.float64)
    K, theta = op.budget_from_survival_cost(g["history_survival"], [1.0], [0.0], g["sps_rows"], tok)
    assert K == g["K_star"]
    assert np.allclose(theta, g["predicted_tokens_per_s"], atol=1e-5)   # survival in float32, as printed
    Ks, theta_s = op.budget_from_survival(g["history_survival"], g["sps_rows"], g["sps"])
    assert Ks == K and np.allclose(theta, theta_s, rtol=1e-14)


def _theta_cost(A, lens, R, req_rows, req_cost, tok_rows, tok_cost):
    N = R + sum(float(A[r, j]) for r in range(A.shape[0]) for j in range(lens[r]))
    return N / (op.sps_at(R, req_rows, req_cost) + op.sps_at(R + sum(lens), tok_rows, tok_cost))


@pytest.mark.parametrize("seed", range(10))
def test_cost_budget_is_the_best_of_every_length_vector(seed):
    """max over every l in {0..W}^R of N(l) / T(R, M(l)) equals the prefix-budget argmax; the top-K allocation
    at K* reaches it."""
    rng = np.random.default_rng(100 + seed)
    R, W = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    conf = rng.uniform(0.05, 1.0, (R, W)).astype(np.float32)
    A, _ = op.survival(conf)
    req_rows, req_cost = np.array([1.0, 4.0]), np.sort(rng.uniform(0.0, 5e-3, 2))
    tok_rows = np.arange(R, R * (W + 1) + 1, dtype=np.float64)
    tok_cost = np.cumsum(rng.uniform(0, 2e-3, len(tok_rows))) + 1e-3     # time grows with the rows
    best = max(_theta_cost(A, lens, R, req_rows, req_cost, tok_rows, tok_cost)
               for lens in itertools.product(range(W + 1), repeat=R))
    K, theta = op.budget_from_survival_cost(A, req_rows, req_cost, tok_rows, tok_cost)
    assert abs(theta[K] - best) <= 1e-12 * best
    lay = op.plan_from_survival(A, K)
    assert abs(_theta_cost(A, list(lay["selected"]), R, req_rows, req_cost, tok_rows, tok_cost) - best) <= 1e-12 * best


def test_cost_budget_special_cases():
    A = np.array([[0.9, 0.6, 0.2], [0.8, 0.5, 0.1]], np.float32)
    rows = np.array([2.0, 8.0])
    # a per-row cost that does not grow: every positive-survival draft pays
    assert op.budget_from_survival_cost(A, [1.0], [1e-3], rows, [1e-3, 1e-3])[0] == 6
    # a per-row cost that grows steeply: none pays
    assert op.budget_from_survival_cost(A, [1.0], [0.0], rows, [1e-3, 1.0])[0] == 0
    # a larger fixed per-batch cost makes extra rows relatively cheaper: K* never falls as it grows, and
    # with a per-batch cost far above the per-row one every draft pays
    ks = [op.budget_from_survival_cost(A, [1.0], [c], rows, [1e-3, 3e-3])[0] for c in (0.0, 1e-3, 1e-2, 1e-1, 10.0)]
    assert ks == sorted(ks) and ks[0] < 6 and ks[-1] == 6
    # eps drops entries from the sort
    assert op.budget_from_survival_cost(A, [1.0], [1e-3], rows, [1e-3, 1e-3], eps=0.55)[0] == 3


def _pairwise_selected(A, K, eps=0.0):
    """The device kernel's formulation on the pages: rank(e) = number of entries before e (survival greater,
    or equal and position smaller, or equal position and request smaller); e is selected iff rank < K."""
    R, W = A.shape
    sel = np.zeros(R, np.int32)
    ents = [(r, j) for r in range(R) for j in range(W) if A[r, j] >= np.float32(eps)]
    for (r, j) in ents:
        rank = 0
        for (r2, j2) in ents:
            gt = A[r2, j2] > A[r, j]
            eq = A[r2, j2] == A[r, j]
            if gt or (eq and (j2 < j or (j2 == j and r2 < r))):
                rank += 1
        if rank < K:
            sel[r] += 1
    return sel


@pytest.mark.parametrize("seed", range(10))
def test_allocation_equals_pairwise_rank_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    R, W = int(rng.integers(1, 7)), int(rng.integers(1, 6))
    levels = np.array([1.0, 0.75, 0.5, 0.5, 0.25], np.float32)       # quantised: many exact ties
    conf = rng.choice(levels, (R, W)).astype(np.float32)
    A, _ = op.survival(conf)
    eps = float(rng.choice([0.0, 0.1]))
    for K in range(0, R * W + 2):
        o = op.plan_from_survival(A, K, eps=eps)
        assert list(o["selected"]) == list(_pairwise_selected(A, K, eps)), (K, A)


@pytest.mark.parametrize("seed", range(8))
def test_allocation_selects_prefixes_and_respects_the_budget(seed):
    rng = np.random.default_rng(200 + seed)
    R, W = 9, 6
    conf = rng.uniform(0.0, 1.0, (R, W)).astype(np.float32)
    A, _ = op.survival(conf)
    n = R * W
    for K in (0, 1, 5, 17, n - 1, n, n + 10):
        o = op.plan_from_survival(A, K)
        sel = o["selected"]
        assert sel.sum() == min(K, n)
        # prefix property: every selected entry's predecessors in its request are selected, i.e. the
        # chosen positions of request r are exactly 0 .. sel[r]-1
        thr = sorted(((-float(A[r, j]), j, r) for r in range(R) for j in range(W)))[:K]
        chosen = {(r, j) for (_, j, r) in thr}
        for r in range(R):
            assert {j for (rr, j) in chosen if rr == r} == set(range(sel[r]))
        assert np.array_equal(o["verify_lens"], 1 + sel)
        assert np.array_equal(o["offsets"], np.concatenate([[0], np.cumsum(1 + sel)]))
        # row_index maps compact rows back to (request, position) of the uniform (W + 1)-wide layout
        for r in range(R):
            for j in range(int(o["verify_lens"][r])):
                assert o["row_index"][o["offsets"][r] + j] == r * (W + 1) + j


def test_flat_sps_verifies_everything_and_no_budget_is_uniform():
    rng = np.random.default_rng(7)
    conf = rng.uniform(0.01, 1.0, (5, 7)).astype(np.float32)
    A, _ = op.survival(conf)
    K, theta = op.budget_from_survival(A, [1, 100], [50.0, 50.0])
    assert K == A.size and np.all(np.diff(theta) > 0)
    # a table that only falls: verify nothing beyond the anchors
    K0, _ = op.budget_from_survival(A, [5, 6], [100.0, 1.0])
    assert K0 == 0
    u = op.plan_from_survival(A, -1, max_len=6)
    assert list(u["verify_lens"]) == [6] * 5 and list(u["selected"]) == [7] * 5
    assert list(op.plan_from_survival(A, 0)["verify_lens"]) == [1] * 5
    assert list(op.plan_from_survival(A, 0, min_len=3)["verify_lens"]) == [3] * 5
    # equal predicted throughput for every K (all survival 0): the smallest budget wins
    Kz, thz = op.budget_from_survival(np.zeros((2, 2), np.float32), [1, 9], [5.0, 5.0])
    assert Kz == 0 and np.all(thz == thz[0])


def test_sps_interpolation_and_eps():
    assert op.sps_at(2, [2, 4], [100.0, 80.0]) == 100.0
    assert op.sps_at(3, [2, 4], [100.0, 80.0]) == 90.0
    assert op.sps_at(1, [2, 4], [100.0, 80.0]) == 100.0
    assert op.sps_at(9, [2, 4], [100.0, 80.0]) == 80.0
    A = np.array([[0.9, 0.05], [0.5, 0.01]], np.float32)
    K, theta = op.budget_from_survival(A, [1, 100], [10.0, 10.0], eps=0.1)
    assert K == 2 and len(theta) == 3                  # the two entries below eps are dropped
    o = op.plan_from_survival(A, 10, eps=0.1)
    assert list(o["selected"]) == [1, 1]


def test_threshold_truncation():
    conf = np.array([[0.9, 0.8, 0.3, 0.9], [0.9, 0.9, 0.9, 0.9], [0.2, 0.9, 0.9, 0.9], [0.5, 0.49, 1, 1]],
                    np.float32)
    o = op.threshold_layout(conf, 0.5)
    assert list(o["selected"]) == [2, 4, 0, 1]
    assert list(o["verify_lens"]) == [3, 5, 1, 2]
    assert list(op.threshold_layout(conf, 0.5, max_len=3)["verify_lens"]) == [3, 3, 1, 2]


def test_confidence_sanitising():
    conf = np.array([[np.nan, 0.5], [1.5, 0.5], [-0.1, 0.9], [0.5, 0.5]], np.float32)
    A, flags = op.survival(conf)
    assert list(flags) == [op.ST_BAD_CONF] * 3 + [0]
    assert A[0, 1] == 0 and A[1, 0] == 1 and A[1, 1] == np.float32(0.5) and A[2, 1] == 0


def test_cap_trim_invalid_lengths():
    o = op.cap_trim(np.array([0, 3, 6, 6]), [0, 3, 1], [1, 5, 0], [1, 2, 3], np.zeros(6, np.int32))
    assert list(o["status"]) == [op.ST_BAD_ACCEPT] * 3


# ----------------------------------------------------------------------------------------------------
# planted mistakes
# ----------------------------------------------------------------------------------------------------
def test_pins_catch_request_before_position_ties(monkeypatch):
    def bad(A, budget, *, min_len=1, max_len=None, eps=0.0, flags=None):
        A = np.asarray(A, np.float32)
        R, W = A.shape
        order = sorted(((r, j) for r in range(R) for j in range(W)), key=lambda e: (-float(A[e]), e[0], e[1]))
        sel = [0] * R
        for r, _ in order[:budget]:
            sel[r] += 1
        return op._finish_layout(sel, W, min_len, W + 1 if max_len is None else max_len, np.zeros(R, np.uint32))
    monkeypatch.setattr(op, "plan_from_survival", bad)
    with pytest.raises(AssertionError):
        test_allocation_equals_pairwise_rank_with_ties(0)


def test_pins_catch_missing_anchor(monkeypatch):
    orig = op._finish_layout

    def bad(selected, W, min_len, max_len, flags):
        o = orig(selected, W, min_len, max_len, flags)
        o["verify_lens"] = np.maximum(o["verify_lens"] - 1, 0)
        return o
    monkeypatch.setattr(op, "_finish_layout", bad)
    with pytest.raises(AssertionError):
        test_topk_allocation_example()


def test_pins_catch_last_of_equal_budgets(monkeypatch):
    def bad(A_hist, sps_rows, sps, eps=0.0):
        K, theta = orig(A_hist, sps_rows, sps, eps)
        return int(len(theta) - 1 - np.argmax(theta[::-1])), theta
    orig = op.budget_from_survival
    monkeypatch.setattr(op, "budget_from_survival", bad)
    with pytest.raises(AssertionError):
        test_flat_sps_verifies_everything_and_no_budget_is_uniform()


def test_pins_catch_sum_instead_of_product(monkeypatch):
    def bad(conf):
        conf = np.asarray(conf, np.float32)
        return np.cumsum(conf, axis=1).astype(np.float32), np.zeros(conf.shape[0], np.uint32)
    monkeypatch.setattr(op, "survival", bad)
    with pytest.raises(AssertionError):
        test_confidence_sanitising()
    with pytest.raises(AssertionError):
        for seed in range(12):
            test_budget_is_the_best_of_every_length_vector(seed)


def test_pins_catch_trim_with_the_wrong_sign(monkeypatch):
    orig = op.cap_trim

    def bad(row_offsets, verify_lens, raw, raw_bonus, out_tokens):
        o = orig(row_offsets, verify_lens, raw, raw_bonus, out_tokens)
        o["block_accept_lens"] = o["commit_lens"] - o["cap_trim"]
        return o
    monkeypatch.setattr(op, "cap_trim", bad)
    with pytest.raises(AssertionError):
        test_cap_trim_examples()


def test_plan_status_bits_match_the_library_abi_values():
    assert op.ST_BAD_ACCEPT == oracle.ST_BAD_ACCEPT


def test_pins_catch_cost_multiplied_instead_of_divided(monkeypatch):
    monkeypatch.setattr(op, "budget_from_survival_cost", _bad_cost)
    with pytest.raises(AssertionError):
        test_cost_budget_reproduces_the_k_table()


def _bad_cost(A_hist, req_rows, req_cost, tok_rows, tok_cost, eps=0.0):
    """N(K) * T(R, R + K): the cost read as a rate."""
    A_hist = np.asarray(A_hist, np.float32)
    R = A_hist.shape[0]
    a = sorted((float(v) for v in A_hist.ravel() if v >= np.float32(eps)), reverse=True)
    theta = [R * (op.sps_at(R, req_rows, req_cost) + op.sps_at(R, tok_rows, tok_cost))]
    N = float(R)
    for K in range(1, len(a) + 1):
        N += a[K - 1]
        theta.append(N * (op.sps_at(R, req_rows, req_cost) + op.sps_at(R + K, tok_rows, tok_cost)))
    return int(np.argmax(theta)), np.array(theta)


def test_pins_catch_cost_without_the_batch_term(monkeypatch):
    orig = op.budget_from_survival_cost
    monkeypatch.setattr(op, "budget_from_survival_cost",
                        lambda A, rr, rc, tr, tc, eps=0.0: orig(A, rr, [0.0] * len(rc), tr, tc, eps))
    with pytest.raises(AssertionError):
        test_cost_budget_special_cases()
