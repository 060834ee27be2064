"""The library's host budget function (spec_plan_budget) against the oracle: it is host code, so these run
on the CPU. The budget is an integer decided by float comparisons; both sides take the survival products in
float32 in position order and the sums and the throughput model in float64, so K* and every predicted
throughput must agree exactly."""
import json
import os

import numpy as np
import pytest

import draft_verification_acceptance_amd as dva
from oracle import plan as op

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
pytestmark = pytest.mark.skipif(not os.path.exists(dva.library_path), reason="libspecverify.so not built")


def test_host_budget_worked_example():
    with open(os.path.join(GOLDEN, "dspark_budget_k4.json")) as f:
        g = json.load(f)
    A = np.asarray(g["history_survival"], np.float32)
    # confidences whose float32 running products are the table's survival values
    conf = np.empty_like(A)
    for r in range(A.shape[0]):
        prev = np.float32(1.0)
        for j in range(A.shape[1]):
            conf[r, j] = np.float32(A[r, j] / prev)
            prev = np.float32(prev * conf[r, j])
    K, theta = dva.plan_budget(conf, g["sps_rows"], g["sps"])
    assert K == g["K_star"]
    assert np.allclose(theta, g["predicted_tokens_per_s"], atol=1e-4)
    Ko, tho = op.plan_budget(conf, g["sps_rows"], g["sps"])
    assert K == Ko and np.array_equal(np.asarray(theta), tho)


@pytest.mark.parametrize("seed", range(20))
def test_host_budget_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    R, W = int(rng.integers(1, 64)), int(rng.integers(1, 16))
    conf = rng.beta(4, 1.5, (R, W)).astype(np.float32)
    if seed % 4 == 0:
        conf[rng.random((R, W)) < 0.05] = np.nan                  # sanitised as 0
    if seed % 5 == 0:
        conf = np.round(conf * 4) / 4                               # exact ties in the sort
    n_pts = int(rng.integers(1, 6))
    rows = np.sort(rng.choice(np.arange(1, R * (W + 1) + 4), n_pts, replace=False)).astype(np.float64)
    sps = np.sort(rng.uniform(10, 200, n_pts))[::-1].copy()
    eps = float(rng.choice([0.0, 0.05, 0.3]))
    K, theta = dva.plan_budget(conf, rows, sps, survival_eps=eps)
    Ko, tho = op.plan_budget(conf, rows, sps, eps)
    assert K == Ko
    assert np.array_equal(np.asarray(theta), tho)


def test_host_budget_at_the_ragged_shape():
    """The planner workload's shape (512 requests x 15 drafts): every digit of the descending sort is in use."""
    from draft_verification_acceptance_amd import workloads as W
    w = W.planner_inputs()
    for eps, quant in ((0.0, False), (0.05, False), (0.0, True)):
        conf = np.round(w.conf_hist * 8) / 8 if quant else w.conf_hist     # quant: thousands of exact ties
        K, theta = dva.plan_budget(conf.astype(np.float32), w.sps_rows, w.sps, survival_eps=eps)
        Ko, tho = op.plan_budget(conf.astype(np.float32), w.sps_rows, w.sps, eps)
        assert K == Ko
        assert np.array_equal(theta, tho)


@pytest.mark.parametrize("case", ["zeros", "ones", "single", "all_below_eps", "nan_rows", "powers_of_two"])
def test_host_budget_degenerate_inputs(case):
    """Inputs whose sorted survival list is degenerate: every value equal, one value, none selectable, NaNs
    sanitised to 0, and values that differ only in their exponent (a single digit of the descending sort)."""
    rng = np.random.default_rng(7)
    conf = {"zeros": np.zeros((9, 4), np.float32),
            "ones": np.ones((9, 4), np.float32),
            "single": np.array([[0.7]], np.float32),
            "all_below_eps": np.full((6, 5), 0.2, np.float32),
            "nan_rows": np.where(rng.random((8, 6)) < 0.5, np.nan, 0.9).astype(np.float32),
            "powers_of_two": np.float32(2.0) ** -rng.integers(0, 6, (12, 7)).astype(np.float32)}[case]
    rows = np.array([1.0, 20.0, 60.0, 200.0])
    sps = np.array([120.0, 100.0, 70.0, 30.0])
    for eps in (0.0, 0.3):
        K, theta = dva.plan_budget(conf, rows, sps, survival_eps=eps)
        Ko, tho = op.plan_budget(conf, rows, sps, eps)
        assert K == Ko
        assert np.array_equal(theta, tho)


@pytest.mark.parametrize("seed", range(16))
def test_host_cost_budget_matches_oracle(seed):
    """spec_plan_budget_cost against oracle.plan.plan_budget_cost: K* and every N(K) / T agree exactly."""
    rng = np.random.default_rng(50 + seed)
    R, W = int(rng.integers(1, 64)), int(rng.integers(1, 16))
    conf = rng.beta(4, 1.5, (R, W)).astype(np.float32)
    if seed % 4 == 0:
        conf = np.round(conf * 4) / 4                               # exact ties in the sort
    n_req, n_tok = int(rng.integers(1, 4)), int(rng.integers(1, 6))
    req_rows = np.sort(rng.choice(np.arange(1, 80), n_req, replace=False)).astype(np.float64)
    req_cost = rng.uniform(0.0, 2e-3, n_req) * (seed % 3 != 0)       # some tables with no per-batch term
    tok_rows = np.sort(rng.choice(np.arange(1, R * (W + 1) + 4), n_tok, replace=False)).astype(np.float64)
    tok_cost = np.sort(rng.uniform(1e-4, 5e-3, n_tok))
    eps = float(rng.choice([0.0, 0.05, 0.3]))
    K, theta = dva.plan_budget_cost(conf, req_rows, req_cost, tok_rows, tok_cost, survival_eps=eps)
    Ko, tho = op.plan_budget_cost(conf, req_rows, req_cost, tok_rows, tok_cost, eps)
    assert K == Ko
    assert np.array_equal(np.asarray(theta), tho)


def test_host_cost_budget_k_table_and_checks():
    with open(os.path.join(GOLDEN, "dspark_budget_k4.json")) as f:
        g = json.load(f)
    A = np.asarray(g["history_survival"], np.float32)
    conf = np.empty_like(A)
    for r in range(A.shape[0]):
        prev = np.float32(1.0)
        for j in range(A.shape[1]):
            conf[r, j] = np.float32(A[r, j] / prev)
            prev = np.float32(prev * conf[r, j])
    K, theta = dva.plan_budget_cost(conf, [1.0], [0.0], g["sps_rows"], 1.0 / np.asarray(g["sps"], np.float64))
    assert K == g["K_star"] and np.allclose(theta, g["predicted_tokens_per_s"], atol=1e-4)
    for bad in (dict(tok_cost=[0.0, 1e-3]), dict(req_cost=[-1e-3]), dict(tok_rows=[5.0, 5.0]),
                dict(tok_cost=[np.inf, 1e-3])):
        kw = dict(req_rows=[1.0], req_cost=[0.0], tok_rows=[2.0, 8.0], tok_cost=[1e-3, 2e-3])
        kw.update(bad)
        with pytest.raises(dva.SpecError):
            dva.plan_budget_cost(conf, kw["req_rows"], kw["req_cost"], kw["tok_rows"], kw["tok_cost"])
