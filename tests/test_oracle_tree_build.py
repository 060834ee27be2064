"""CPU pins of the EAGLE-2 tree-construction oracle (oracle/tree_build.py): the pages' hand-checked
visibility tree (golden file), topk = 1 giving a chain, an independent whole-set formulation of the selection
(full sort of every path product in float64 over distinct scores), structural invariants (ancestor closure,
parent before child, mask = ancestor relation, positions = depth, first child / next sibling from the parent
array), and planted mistakes."""
import json
import os

import numpy as np
import pytest

from oracle import tree_build as otb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_hand_checked_tree():
    g = _golden("tree_mask_hand_check.json")
    t = otb.build_tree(g["anchor"], np.array(g["tokens"]), np.array(g["probs"], np.float32), g["n_nodes"], g["seq_len"])
    assert list(t["tokens"]) == g["expected_tokens"]
    assert list(t["parents"]) == g["expected_parents"]
    assert list(t["depth"]) == g["expected_depth"]
    assert list(t["positions"]) == g["expected_positions"]
    names = g["names"]
    for i, name in enumerate(names):
        vis = sorted(names[j] for j in range(len(names)) if t["mask"][i, j])
        assert vis == sorted(g["expected_visible"][name]), name
    assert list(t["first_child"]) == g["expected_first_child"]
    assert list(t["next_sibling"]) == g["expected_next_sibling"]


def test_topk_one_is_a_chain():
    rng = np.random.default_rng(3)
    S = 6
    toks = rng.integers(0, 1000, (S, 1, 1))
    probs = rng.uniform(0.1, 1.0, (S, 1, 1)).astype(np.float32)
    t = otb.build_tree(7, toks, probs, S + 1, 20)
    assert list(t["parents"]) == [-1] + list(range(S))
    assert list(t["tokens"]) == [7] + list(toks[:, 0, 0])
    assert list(t["positions"]) == list(range(20, 21 + S))
    assert np.array_equal(t["mask"], np.tril(np.ones((S + 1, S + 1), np.uint8)))


def _random_inputs(rng, S, k):
    toks = rng.integers(0, 50000, (S, k, k))
    # distinct, well separated probabilities: no two path products within float32 rounding of each other
    probs = rng.uniform(0.05, 1.0, (S, k, k)).astype(np.float32)
    return toks, probs


@pytest.mark.parametrize("S,k,N,seed", [(3, 2, 6, 0), (5, 4, 20, 1), (8, 8, 64, 2), (4, 3, 10, 3), (6, 5, 31, 4),
                                         (2, 8, 72, 5), (1, 8, 9, 6), (7, 2, 2, 7)])
def test_selection_equals_best_paths_and_structure(S, k, N, seed):
    rng = np.random.default_rng(seed)
    toks, probs = _random_inputs(rng, S, k)
    t = otb.build_tree(11, toks, probs, N, 100)
    c = otb.candidates(toks, probs)
    # independent formulation: every candidate's path product in float64 from its explicit parent chain,
    # then the N - 1 best by a full sort
    n = len(c["score"])
    prod64 = np.ones(n)
    for i in range(n):
        j, q = i, 1.0
        while j >= 0:
            s, f, cc = _coords(j, k)
            q *= float(probs[s, f, cc])
            j = int(c["parent"][j])
        prod64[i] = q
    assert np.allclose(prod64, c["score"], rtol=1e-5)
    best = set(np.argsort(-prod64, kind="stable")[:N - 1].tolist())
    assert set(t["cand_index"][1:].tolist()) == best
    # frontier after each step = the k best candidates of that step
    for s, fr in enumerate(c["frontiers"]):
        ids = [i for i in range(n) if c["step"][i] == s]
        assert fr == sorted(ids, key=lambda i: -prod64[i])[:k]
    # structure
    for i in range(1, N):
        p = t["parents"][i]
        assert 0 <= p < i and t["depth"][i] == t["depth"][p] + 1
        assert t["positions"][i] == 100 + t["depth"][i]
        assert t["cand_index"][i] > t["cand_index"][p] or p == 0
    anc = np.eye(N, dtype=np.uint8)
    for i in range(N):
        j = t["parents"][i]
        while j >= 0:
            anc[i, j] = 1
            j = t["parents"][j]
    assert np.array_equal(anc, t["mask"])
    for i in range(N):
        kids = [j for j in range(N) if t["parents"][j] == i]
        assert t["first_child"][i] == (kids[0] if kids else -1)
        if i > 0:
            sibs = [j for j in range(i + 1, N) if t["parents"][j] == t["parents"][i]]
            assert t["next_sibling"][i] == (sibs[0] if sibs else -1)


def _coords(cid, k):
    if cid < k:
        return 0, 0, cid
    r = cid - k
    s = 1 + r // (k * k)
    r %= k * k
    return s, r // k, r % k


def test_ties_go_to_the_lower_candidate_id_and_bad_probs_are_flagged():
    toks = np.arange(2 * 2 * 2).reshape(2, 2, 2)
    probs = np.full((2, 2, 2), 0.5, np.float32)
    t = otb.build_tree(0, toks, probs, 4, 0)
    # all step-0 scores tie (0.5), all step-1 scores tie (0.25): ids 0, 1 then the lowest step-1 id 2
    assert list(t["cand_index"]) == [-1, 0, 1, 2]
    probs[1, 0, 0] = np.nan
    probs[0, 0, 1] = 1.5
    assert otb.build_tree(0, toks, probs, 4, 0)["status"] == otb.ST_BAD_CONF


def test_pins_catch_frontier_by_own_probability(monkeypatch):
    orig = otb.candidates

    def bad(tokens, probs):
        c = orig(tokens, probs)
        S, k, _ = tokens.shape
        # rank each step by the child's own probability instead of the path product
        for s in range(1, S):
            ids = [i for i in range(len(c["score"])) if c["step"][i] == s]
            c["frontiers"][s] = sorted(ids, key=lambda i: -float(probs[s].ravel()[i - (k + (s - 1) * k * k)]))[:k]
        return c
    monkeypatch.setattr(otb, "candidates", bad)
    with pytest.raises(AssertionError):
        test_selection_equals_best_paths_and_structure(5, 4, 20, 1)


def test_pins_catch_flattened_positions(monkeypatch):
    orig = otb.build_tree

    def bad(anchor, tokens, probs, n_nodes, seq_len):
        t = orig(anchor, tokens, probs, n_nodes, seq_len)
        t["positions"] = seq_len + np.arange(n_nodes)
        return t
    monkeypatch.setattr(otb, "build_tree", bad)
    with pytest.raises(AssertionError):
        test_hand_checked_tree()


def test_pins_catch_sibling_visibility(monkeypatch):
    orig = otb.build_tree

    def bad(anchor, tokens, probs, n_nodes, seq_len):
        t = orig(anchor, tokens, probs, n_nodes, seq_len)
        t["mask"] = np.tril(np.ones((n_nodes, n_nodes), np.uint8))     # plain causal mask over the flat order
        return t
    monkeypatch.setattr(otb, "build_tree", bad)
    with pytest.raises(AssertionError):
        test_hand_checked_tree()
