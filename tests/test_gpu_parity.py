"""GPU parity: the HIP library (through its C ABI) against the fp64 CPU oracle on the same seeded inputs.

Sizes: every workload at a reduced vocabulary that still spans several chunks per row and an unaligned
ragged tail, then at full size in the launch configuration the benchmark times; every request is compared
at both sizes. Edge cases and statistics follow.

SPECVERIFY_FUZZ_SEEDS=n widens the seeded random tests (random shapes, random trees, fault injection, corrupt
candidate lists) by n more seeds each, for a longer sweep than the default run.
"""
import os

import numpy as np
import pytest
import torch
from scipy import stats

import draft_verification_acceptance_amd as dva
import oracle
from draft_verification_acceptance_amd import workloads as W
from gpu_util import (compare_chain, compare_tree, dev, dev_logits, np_out, oracle_chain, oracle_tree, run_chain,
                      run_tree)
from test_oracle_flag_counts import EXPECTED as FLAGGED

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


_FUZZ = range(100, 100 + int(os.environ.get("SPECVERIFY_FUZZ_SEEDS", "0")))   # extra seeds of the random tests


# ----------------------------------------------------------------------------------------------------
# the five workloads
# ----------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("mode", ["greedy", "rejection"])
def test_tiny_chain(mode):
    w = W.tiny_chain()
    _say("tiny_chain", mode)
    g = run_chain(w, mode)
    o = oracle_chain(w, mode)
    assert compare_chain(w, mode, o, g, expect=FLAGGED[("tiny_chain", mode)]) == 0


def test_chain_rejection_small_vocab():
    w = W.chain_rejection(seed=2001, vocab=20011)
    _say("chain_rejection V=20011")
    g = run_chain(w, "rejection")
    o = oracle_chain(w, "rejection")
    compare_chain(w, "rejection", o, g)
    assert o["accept_len"].max() >= 2


def test_block_greedy_small_vocab():
    w = W.block_greedy(seed=3001, vocab=20011, tie_rate=0.2)
    _say("block_greedy V=20011")
    g = run_chain(w, "greedy")
    o = oracle_chain(w, "greedy")
    assert compare_chain(w, "greedy", o, g) == 0
    assert np.array_equal(g["accept_len"], w.planted_r)


@pytest.mark.parametrize("mode", ["greedy", "target_only"])
def test_tree_small_vocab(mode):
    w = W.tree(seed=4001, vocab=12007)
    _say("tree V=12007", mode)
    g = run_tree(w, mode)
    o = oracle_tree(w, mode)
    compare_tree(w, mode, o, g)


def test_ragged_small_vocab():
    w = W.ragged(seed=5001, vocab=4099)
    _say("ragged V=4099")
    g = run_chain(w, "rejection")
    o = oracle_chain(w, "rejection")
    compare_chain(w, "rejection", o, g)


@pytest.mark.parametrize("K,T,sigma", [(16, 1.0, 1.0), (1, 0.7, 1.0), (64, 0.5, 0.2)])
def test_chain_sparse_small_vocab(K, T, sigma):
    w = W.chain_sparse(seed=6001, vocab=20011, K=K, temperature=T, greedy_frac=0.3, batch=40, draft_sigma=sigma)
    _say("chain_sparse V=20011", K, T, w.meta)
    g = run_chain(w, "rejection_sparse")
    o = oracle_chain(w, "rejection_sparse")
    compare_chain(w, "rejection_sparse", o, g)
    # tokens outside the candidates are emitted after rejections (the residual spans the vocab)
    D = w.total_rows - w.batch
    outside = 0
    for b in range(w.batch):
        r = int(o["accept_len"][b])
        if r < 7:
            outside += int(int(o["bonus"][b]) not in set(w.cand_ids[int(w.offsets[b]) - b + r].tolist()))
    assert D > 0 and (outside > 0 or K == 64)


def test_chain_sparse_fp32_and_ragged():
    w = W.chain_sparse(seed=6002, vocab=999, K=8, temperature=0.8, greedy_frac=0.5, batch=24, bf16=False,
                       ragged=True, parallel=False)
    _say("chain_sparse fp32 V=999")
    assert compare_chain(w, "rejection_sparse", oracle_chain(w, "rejection_sparse"), run_chain(w, "rejection_sparse")) <= 12
    # duplicates, invalid entries and q(d) = 0 on the device as in the oracle
    ids = w.cand_ids.copy()
    q = w.cand_q.copy()
    D = w.total_rows - w.batch
    assert D >= 8
    ids[0, 1] = ids[0, 0]                     # repeated id: masses add
    ids[D // 4, 2] = w.vocab + 3              # out of range: BAD_TOKEN, left out
    q[D // 2, 3] = -0.5                       # negative: BAD_Q, left out
    q[D - 1, 0] = np.nan
    w.draft_tokens[3] = int(np.setdiff1d(np.arange(w.vocab), ids[3])[0])   # not a candidate: q(d) = 0
    w.cand_ids, w.cand_q = ids, q
    o = oracle_chain(w, "rejection_sparse")
    g = run_chain(w, "rejection_sparse")
    assert np.any(o["status"] & oracle.ST_BAD_TOKEN) and np.any(o["status"] & oracle.ST_BAD_Q)
    compare_chain(w, "rejection_sparse", o, g)


@pytest.mark.parametrize("seed", [61, 62, *(1000 + s for s in _FUZZ)])
def test_chain_sparse_random_corrupt_candidates(seed):
    """Seeded corruption of sparse candidate lists (ragged fp32 chains): ids outside [0, V), duplicated ids
    (the drafted token's among them), masses that are negative, NaN, infinite or sum past 1, a row whose
    entries are all invalid, and drafted tokens that are no candidate. Device = oracle for every request."""
    rng = np.random.default_rng(seed)
    w = W.chain_sparse(seed=6100 + seed, vocab=997, K=8, temperature=0.8, greedy_frac=0.3, batch=24, bf16=False,
                       ragged=True, parallel=False)
    ids, q = w.cand_ids.copy(), w.cand_q.copy()
    D, K = ids.shape
    for i in range(D):
        kind = int(rng.integers(0, 10))
        c = int(rng.integers(0, K))
        if kind == 0:
            ids[i, c] = int(rng.choice([-1, w.vocab, w.vocab + 50]))
        elif kind == 1:
            ids[i, c] = ids[i, (c + 1) % K]
        elif kind == 2:
            q[i, c] = rng.choice([-0.25, np.nan, np.inf, -np.inf])
        elif kind == 3:
            q[i] *= 3.0                                  # masses past 1
        elif kind == 4:
            ids[i, :] = -5                               # nothing valid
        elif kind == 5:
            w.draft_tokens[i] = int(np.setdiff1d(np.arange(w.vocab), ids[i])[0])
        elif kind == 6:
            ids[i, c] = w.draft_tokens[i]                # the drafted token listed (again)
    w.cand_ids, w.cand_q = ids, q
    _say("chain_sparse corrupt candidates", seed)
    compare_chain(w, "rejection_sparse", oracle_chain(w, "rejection_sparse"), run_chain(w, "rejection_sparse"))


@pytest.mark.parametrize("V", [20011, 151936])
def test_zero_residual_falls_back_to_p(V):
    """A rejected row whose residual weights are all zero: request 0's first target row puts p = 0.2 on five
    tokens spread over the vocabulary (every other logit -inf), and its sparse q lists those five
    with mass 0.5 each, so the drafted one is rejected (alpha = 0.4 < u = 0.9) and [p - q]_+ = 0 everywhere.
    The draw then falls back to p (ZERO_RESIDUAL), whose segment sums the drawing workgroup forms itself:
    the token and residual_mass (the mass of p) equal the oracle's."""
    w = W.chain_sparse(seed=6301, batch=4, vocab=V, K=8, temperature=0.8, bf16=False, parallel=False)
    toks5 = np.array([3, V // 7, V // 2 + 1, V - 2000, V - 1], np.int32)
    w.target[0, :] = -np.inf
    w.target[0, toks5] = 0.0
    ids, q = w.cand_ids.copy(), w.cand_q.copy()
    ids[0, :5], q[0, :5] = toks5, 0.5
    ids[0, 5:], q[0, 5:] = toks5[0], 0.0
    w.cand_ids, w.cand_q = ids, q
    w.draft_tokens[0] = toks5[2]
    w.u_accept[0] = 0.9
    for uf in (0.1, 0.5, 0.95):
        w.u_final[0] = uf
        _say("zero residual", V, uf)
        o = oracle_chain(w, "rejection_sparse")
        g = run_chain(w, "rejection_sparse")
        assert o["status"][0] & oracle.ST_ZERO_RESIDUAL and g["status"][0] & oracle.ST_ZERO_RESIDUAL
        assert g["accept_len"][0] == 0 and g["bonus"][0] == toks5[int(uf / 0.2)]
        compare_chain(w, "rejection_sparse", o, g)


# Full sizes, the benchmark's launch configuration; every request is compared with the oracle and the
# flagged ones are exactly the oracle's count for the seeded workload.
def test_full_chain_sparse():
    w = W.chain_sparse()
    _say("chain_sparse full", w.meta)
    g = run_chain(w, "rejection_sparse")
    o = oracle_chain(w, "rejection_sparse")
    compare_chain(w, "rejection_sparse", o, g, expect=FLAGGED[("chain_sparse", "rejection_sparse")])
    assert np.all((g["accept_len"] >= 0) & (g["accept_len"] <= 7))
    assert not np.any(g["status"] & ~np.uint32(oracle.ST_NEAR_ALPHA | oracle.ST_NEAR_CDF))



def test_full_chain_rejection():
    w = W.chain_rejection()
    _say("chain_rejection full")
    g = run_chain(w, "rejection")
    o = oracle_chain(w, "rejection")
    compare_chain(w, "rejection", o, g, expect=FLAGGED[("chain_rejection", "rejection")])
    # properties that hold for every request at any size
    assert np.all((g["accept_len"] >= 0) & (g["accept_len"] <= 7))
    assert np.all((g["bonus"] >= 0) & (g["bonus"] < w.vocab))
    assert not np.any(g["status"] & ~np.uint32(oracle.ST_NEAR_ALPHA | oracle.ST_NEAR_CDF))
    assert np.all((g["residual_mass"] > 0) & (g["residual_mass"] <= 1.0 + 1e-6))


def test_full_block_greedy():
    w = W.block_greedy()
    _say("block_greedy full")
    g = run_chain(w, "greedy")
    o = oracle_chain(w, "greedy")
    assert compare_chain(w, "greedy", o, g, expect=FLAGGED[("block_greedy", "greedy")]) == 0
    assert np.array_equal(g["accept_len"], w.planted_r)


@pytest.mark.parametrize("mode", ["greedy", "target_only"])
def test_full_tree(mode):
    w = W.tree()
    _say("tree full", mode)
    g = run_tree(w, mode)
    o = oracle_tree(w, mode)
    compare_tree(w, mode, o, g, expect=FLAGGED[("tree", mode)])


def test_full_ragged():
    w = W.ragged()
    _say("ragged full", w.total_rows)
    g = run_chain(w, "rejection")
    o = oracle_chain(w, "rejection")
    compare_chain(w, "rejection", o, g, expect=FLAGGED[("ragged", "rejection")])
    m = np.diff(w.offsets) - 1
    assert np.all((g["accept_len"] >= 0) & (g["accept_len"] <= m))


# ----------------------------------------------------------------------------------------------------
# edge cases
# ----------------------------------------------------------------------------------------------------
def _chain_from(target, draft, offsets, tokens, ua, uf, T, max_len):
    return W.ChainWorkload("edge", target.shape[1], len(offsets) - 1, np.asarray(offsets, np.int32), target, draft,
                           np.asarray(tokens, np.int32), np.asarray(ua, np.float32), np.asarray(uf, np.float32),
                           T, ("greedy", "rejection"), max_len)


@pytest.mark.parametrize("V", [1, 7, 32, 1000, 8195, 151937])
def test_vocab_sizes(V):
    w = W.tiny_chain(seed=77 + V, batch=6, m=3, vocab=V)
    for mode in ("greedy", "rejection"):
        _say("vocab", V, mode)
        for bf16 in (False, True):
            ww = w
            if bf16:
                ww = _chain_from(W.bf16_bits(w.target), W.bf16_bits(w.draft), w.offsets, w.draft_tokens, w.u_accept,
                                 w.u_final, 1.0, w.max_verify_len)
            g = run_chain(ww, mode)
            o = oracle_chain(ww, mode)
            compare_chain(ww, mode, o, g)


def test_draw_over_1024_segments():
    """A vocab of more than 1024 draw segments of 512 tokens (more than one per thread of the final
    workgroup's prefix): peaked rows, so that the draws are not all within the CDF tolerance."""
    w = W.chain_rejection(seed=2003, batch=6, m=3, vocab=600_001, parallel=False)
    _say("chain_rejection V=600001")
    compare_chain(w, "rejection", oracle_chain(w, "rejection"), run_chain(w, "rejection"))


def test_long_rejection_request_reads_partials_unstaged():
    """A rejection request of 700 rows has 1400 row partials, more than the scan stages in LDS (1024): it reads
    them from the workspace instead. With draft = target every draft is accepted (alpha = 1, r = m = 699); with
    a noisy draft the first rejection falls somewhere. Both against the oracle, next to short requests."""
    rng = np.random.default_rng(70)
    V = 509
    lens = np.array([700, 1, 40])
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, B = int(offs[-1]), 3
    tl = rng.normal(0, 2, (T, V)).astype(np.float32)
    same = np.concatenate([tl[offs[b]:offs[b + 1] - 1] for b in range(B)])   # draft row j = target row j
    for noisy in (False, True):
        dl = same + (rng.normal(0, 1.0, same.shape).astype(np.float32) if noisy else 0.0)
        toks = np.array([int(np.argmax(r)) for r in dl], np.int32)
        w = _chain_from(tl, dl, offs, toks, rng.random(T - B), rng.random(B), 1.0, 700)
        _say("long rejection request, noisy draft" if noisy else "long rejection request, draft = target")
        g = run_chain(w, "rejection")
        compare_chain(w, "rejection", oracle_chain(w, "rejection"), g)
        if not noisy:
            assert int(g["accept_len"][0]) == 699


def test_maximum_vocab():
    """V = 2^22, the largest vocab the library accepts (8192 draw segments, 2048 sample-then-match pieces per
    row): rows of zeros with a few raised tokens (so that draws land on wide CDF steps), fp32 and bf16, chain
    greedy / rejection / sample-then-match and a 3-node tree, against the oracle."""
    rng = np.random.default_rng(22)
    V = 1 << 22
    offs = np.array([0, 3, 5], np.int32)
    T, B = 5, 2
    spikes = rng.integers(0, V, (T, 3))
    tl = np.zeros((T, V), np.float32)
    dl = np.zeros((T - B, V), np.float32)
    for i in range(T):
        tl[i, spikes[i]] = [21.0, 20.0, 19.0]
    for i in range(T - B):
        row = i + int(np.searchsorted(offs - np.arange(B + 1), i, "right")) - 1   # draft row j of b: target row j of b
        dl[i, spikes[row]] = [19.0, 21.0, 20.0]
    toks = np.array([spikes[0, 0], spikes[1, 1], spikes[3, 0]], np.int32)
    for bf16 in (False, True):
        t_ = W.bf16_bits(tl) if bf16 else tl
        d_ = W.bf16_bits(dl) if bf16 else dl
        w = W.ChainWorkload("maxvocab", V, B, offs, t_, d_, toks, rng.random(T - B).astype(np.float32),
                            rng.random(B).astype(np.float32), 1.0, ("greedy", "rejection", "sample_match"), 3)
        for mode in ("greedy", "rejection", "sample_match"):
            _say("maximum vocab", mode, "bf16" if bf16 else "fp32")
            compare_chain(w, mode, oracle_chain(w, mode), run_chain(w, mode))
    tt = np.zeros((3, V), np.float32)
    for i in range(3):
        tt[i, spikes[i]] = [21.0, 20.0, 19.0]
    tw = W.TreeWorkload("maxvocab tree", V, 1, 3, tt, np.array([-1, 0, 0], np.int32),
                        np.array([0, spikes[0, 1], spikes[0, 0]], np.int32), rng.random(3).astype(np.float32),
                        rng.random(1).astype(np.float32), 1.0)
    for mode in ("greedy", "target_only"):
        _say("maximum vocab tree", mode)
        compare_tree(tw, mode, oracle_tree(tw, mode), run_tree(tw, mode))


@pytest.mark.parametrize("T", [0.05, 0.7, 5.0])
def test_temperatures(T):
    w = W.chain_rejection(seed=2100, batch=16, m=5, vocab=3001, parallel=False)
    w.temperature = T
    _say("temperature", T)
    g = run_chain(w, "rejection")
    o = oracle_chain(w, "rejection")
    compare_chain(w, "rejection", o, g)


def test_ragged_lengths_including_zero_drafts():
    rng = np.random.default_rng(5)
    V = 513
    lens = np.array([1, 1, 5, 1, 9, 2, 1, 16, 3], np.int64)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, B = int(offs[-1]), len(lens)
    tl = rng.normal(0, 2, (T, V)).astype(np.float32)
    dl = (tl[:T - B] + rng.normal(0, 1, (T - B, V))).astype(np.float32)
    toks = np.array([np.argmax(tl[offs[b] + j]) if rng.random() < 0.7 else rng.integers(V)
                     for b in range(B) for j in range(lens[b] - 1)], np.int32)
    w = _chain_from(tl, dl, offs, toks, rng.random(T - B), rng.random(B), 0.9, 16)
    for mode in ("greedy", "rejection"):
        g = run_chain(w, mode)
        o = oracle_chain(w, mode)
        compare_chain(w, mode, o, g)
        assert np.all(g["accept_len"][lens == 1] == 0)


@pytest.mark.parametrize("seed", [*range(8), *_FUZZ])
def test_random_shapes_match_the_oracle(seed):
    """Seeded random batch shapes across the launch paths (one-workgroup and per-request scans, split and
    whole-request matches, draw workgroup counts): 1..300 requests of 1..40 rows (ragged), vocab 1..5000
    (fewer for large batches), fp32 or bf16 logits, temperature 0.3..1.5, every chain mode (the sparse q: the
    draft row's top 1..8 tokens with their softmax mass). Every request is compared with the oracle."""
    rng = np.random.default_rng(900 + seed)
    B = int(rng.integers(1, 301))
    L = int(rng.integers(1, 41))
    lens = rng.integers(1, L + 1, B)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, D = int(offs[-1]), int(offs[-1]) - B
    V = int(max(1, min(int(rng.integers(1, 5001)), 12_000_000 // (2 * T))))
    temp = float(rng.uniform(0.3, 1.5))
    tl = (rng.normal(0, 2, (T, V)) * rng.uniform(0.5, 2.0)).astype(np.float32)
    rows = np.concatenate([np.arange(offs[b], offs[b + 1] - 1) for b in range(B)]).astype(np.int64)
    dl = (tl[rows] + rng.normal(0, 0.8, (D, V))).astype(np.float32)
    toks = np.where(rng.random(D) < 0.6, np.argmax(tl[rows], axis=1) if D else 0,
                    rng.integers(0, V, D)).astype(np.int32)
    w = _chain_from(tl, dl, offs, toks, rng.random(D), rng.random(B), temp, L)
    K = int(rng.integers(1, 9))
    ids = np.stack([W.top_candidates(x, min(K, V)) for x in dl]) if D else np.zeros((0, min(K, V)), np.int32)
    q = np.exp((dl[np.arange(D)[:, None], ids] - dl.max(axis=1, keepdims=True)) / temp) if D else np.zeros(ids.shape)
    w.cand_ids, w.cand_q = ids.astype(np.int32), (q / np.maximum(q.sum(axis=1, keepdims=True), 1e-30)).astype(np.float32)
    bf16 = bool(rng.integers(0, 2))
    if bf16:
        w = _chain_from(W.bf16_bits(tl), W.bf16_bits(dl), offs, toks, w.u_accept, w.u_final, temp, L)
        w.cand_ids, w.cand_q = ids.astype(np.int32), (q / np.maximum(q.sum(axis=1, keepdims=True), 1e-30)).astype(np.float32)
    for mode in ("greedy", "rejection", "rejection_sparse", "sample_match"):
        _say("random shape", seed, B, L, T, V, round(temp, 2), "bf16" if bf16 else "fp32", mode)
        compare_chain(w, mode, oracle_chain(w, mode), run_chain(w, mode))


def test_masked_logits_ties_and_special_rows():
    rng = np.random.default_rng(11)
    V, B, m = 700, 12, 4
    T = B * (m + 1)
    offs = np.arange(B + 1, dtype=np.int32) * (m + 1)
    tl = rng.integers(-3, 4, (T, V)).astype(np.float32)        # many exact ties
    tl[:, rng.random(V) < 0.5] = -np.inf                       # masked vocabulary entries
    tl[0:5, 5] = 100.0                                          # one-hot-like p (alpha = p(d)/q(d) huge)
    dl = tl[:T - B].copy() + rng.normal(0, 0.5, (T - B, V)).astype(np.float32)
    dl[10:14] = tl[12:16]                                       # identical p and q rows for request 2
    dl[20:24] *= 10.0                                           # very peaked q for request 5
    toks = np.empty(T - B, np.int32)
    for b in range(B):
        for j in range(m):
            row = tl[offs[b] + j]
            toks[b * m + j] = np.flatnonzero(row == row.max())[0] if rng.random() < 0.8 else rng.integers(V)
    w = _chain_from(tl, dl, offs, toks, rng.random(T - B), rng.random(B), 1.0, m + 1)
    for mode in ("greedy", "rejection"):
        for bf16 in (False, True):
            ww = w if not bf16 else _chain_from(W.bf16_bits(tl), W.bf16_bits(dl), offs, toks, w.u_accept, w.u_final,
                                                1.0, m + 1)
            g = run_chain(ww, mode)
            o = oracle_chain(ww, mode)
            compare_chain(ww, mode, o, g)


def test_status_bits_nan_bad_token_bad_uniform_bad_offsets():
    rng = np.random.default_rng(12)
    V, B, m = 300, 6, 3
    T = B * (m + 1)
    offs = np.arange(B + 1, dtype=np.int32) * (m + 1)
    tl = rng.normal(0, 1, (T, V)).astype(np.float32)
    dl = rng.normal(0, 1, (T - B, V)).astype(np.float32)
    toks = rng.integers(0, V, T - B).astype(np.int32)
    ua = rng.random(T - B).astype(np.float32)
    uf = rng.random(B).astype(np.float32)
    tl[1, 17] = np.nan          # request 0: NaN in a target row
    dl[5, 3] = np.nan           # request 1: NaN in a draft row
    toks[8] = V + 5             # request 2: out-of-range token
    ua[13] = 1.5                # request 4: bad uniform
    uf[5] = np.nan              # request 5: bad final uniform
    w = _chain_from(tl, dl, offs, toks, ua, uf, 1.0, m + 1)
    for mode in ("greedy", "rejection"):
        g = run_chain(w, mode)
        o = oracle_chain(w, mode)
        compare_chain(w, mode, o, g)
        assert g["status"][0] & oracle.ST_NONFINITE
        assert g["status"][2] & oracle.ST_BAD_TOKEN
        if mode == "rejection":
            assert g["status"][1] & oracle.ST_NONFINITE
            assert g["status"][4] & oracle.ST_BAD_UNIFORM
            assert g["status"][5] & oracle.ST_BAD_UNIFORM
    # offsets that do not describe the rows: reported, nothing else checked
    bad = offs.copy()
    bad[3] = bad[2]
    wb = _chain_from(tl, dl, bad, toks, ua, uf, 1.0, m + 1)
    g = run_chain(wb, "greedy")
    assert g["status"][2] & oracle.ST_BAD_OFFSETS


@pytest.mark.parametrize("seed,max_len", [(41, 6), (42, 6), (43, 6), (41, 100),
                                          *((1000 + s, 6 if s % 2 == 0 else 100) for s in _FUZZ)])
def test_random_faults_match_the_oracle(seed, max_len):
    """Seeded fault injection over ragged requests: NaN, +inf and -inf logits (a few, or a whole row), draft
    tokens outside [0, V), uniforms that are NaN, negative or >= 1; greedy, rejection and sample-then-match.
    Every request's status and outputs equal the oracle's (a NONFINITE request: its flag). max_verify_len 6
    runs small greedy batches in one workgroup, 100 (more rows per request than a wave has lanes) in one
    workgroup per request."""
    rng = np.random.default_rng(seed)
    V, B = 257, 24
    lens = rng.integers(1, 7, B)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(offs[-1])
    tl = rng.normal(0, 2, (T, V)).astype(np.float32)
    dl = rng.normal(0, 2, (T - B, V)).astype(np.float32)
    toks = rng.integers(0, V, T - B).astype(np.int32)
    for b in range(B):                           # half the drafts agree with the target's argmax
        o0, n = int(offs[b]), int(lens[b])
        for j in range(n - 1):
            if rng.random() < 0.5:
                toks[o0 - b + j] = int(np.argmax(tl[o0 + j]))
    ua = rng.random(T - B).astype(np.float32)
    uf = rng.random(B).astype(np.float32)
    for b in range(B):
        o0, n = int(offs[b]), int(lens[b])
        d0 = o0 - b
        kind = int(rng.integers(0, 14))
        row = o0 + int(rng.integers(0, n))
        if kind == 5:
            tl[row, rng.integers(0, V)] = np.nan
        elif kind == 6 and n > 1:
            dl[d0 + int(rng.integers(0, n - 1)), rng.integers(0, V)] = np.nan
        elif kind == 7:
            tl[row, rng.integers(0, V)] = np.inf
        elif kind == 8:
            tl[row, :] = -np.inf
        elif kind == 9 and n > 1:
            toks[d0 + int(rng.integers(0, n - 1))] = int(rng.choice([-1, V, V + 7]))
        elif kind == 10 and n > 1:
            ua[d0 + int(rng.integers(0, n - 1))] = rng.choice([np.nan, 1.0, -0.25, 3.0])
        elif kind == 11:
            uf[b] = rng.choice([np.nan, 1.0, -0.5])
        elif kind == 12:
            tl[row, rng.integers(0, V, 20)] = -np.inf
        elif kind == 13 and n > 1:
            dl[d0 + int(rng.integers(0, n - 1)), :] = -np.inf
    w = W.ChainWorkload("faults", V, B, offs, tl, dl, toks, ua, uf, 0.9, ("greedy", "rejection", "sample_match"),
                        max_len)
    for mode in ("greedy", "rejection", "sample_match"):
        _say("random faults", seed, max_len, mode)
        g = run_chain(w, mode)
        o = oracle_chain(w, mode)
        compare_chain(w, mode, o, g)


def test_tree_edge_cases():
    rng = np.random.default_rng(13)
    V = 50
    # N = 1 (root only), chain-shaped, duplicate sibling tokens, bad parents, one-hot rows
    for N in (1, 2, 9, 64, 130):
        B = 5
        target = rng.integers(-2, 3, (B * N, V)).astype(np.float32)
        parents = np.zeros(B * N, np.int32)
        tokens = np.zeros(B * N, np.int32)
        for b in range(B):
            parents[b * N] = -1
            for i in range(1, N):
                parents[b * N + i] = i - 1 if b == 1 else rng.integers(0, i)
                p = parents[b * N + i]
                row = target[b * N + p]
                tokens[b * N + i] = np.flatnonzero(row == row.max())[0] if rng.random() < 0.6 else rng.integers(V)
            if b == 2 and N > 3:        # duplicate sibling tokens
                parents[b * N + 1: b * N + 4] = 0
                tokens[b * N + 1: b * N + 4] = tokens[b * N + 1]
            if b == 3 and N > 3:
                parents[b * N + 3] = 7 if N > 7 else N - 1    # parent not before the node
        tw = W.TreeWorkload("edge", V, B, N, target, parents, tokens, rng.random(B * N).astype(np.float32),
                            rng.random(B).astype(np.float32), 1.0)
        for mode in ("greedy", "target_only"):
            _say("tree edge N", N, mode)
            g = run_tree(tw, mode)
            o = oracle_tree(tw, mode)
            compare_tree(tw, mode, o, g)
            if N > 7:
                assert g["status"][3] & oracle.ST_BAD_PARENT


@pytest.mark.parametrize("seed", [51, 52, *(1000 + s for s in _FUZZ)])
def test_random_tree_faults_match_the_oracle(seed):
    """Seeded fault injection on trees of 12 nodes: NaN, +inf and -inf logits (a few, or a whole row), node
    tokens outside [0, V), parents that do not precede their node, uniforms that are NaN or outside [0, 1);
    greedy and target-only against the oracle."""
    rng = np.random.default_rng(seed)
    V, B, N = 97, 20, 12
    target = rng.normal(0, 2, (B * N, V)).astype(np.float32)
    parents = np.zeros(B * N, np.int32)
    tokens = np.zeros(B * N, np.int32)
    for b in range(B):
        parents[b * N] = -1
        for i in range(1, N):
            p = int(rng.integers(0, i))
            parents[b * N + i] = p
            row = target[b * N + p]
            tokens[b * N + i] = int(np.argmax(row)) if rng.random() < 0.5 else int(rng.integers(V))
    ua = rng.random(B * N).astype(np.float32)
    uf = rng.random(B).astype(np.float32)
    for b in range(B):
        kind = int(rng.integers(0, 12))
        node = b * N + int(rng.integers(0, N))
        child = b * N + int(rng.integers(1, N))
        if kind == 4:
            target[node, rng.integers(0, V)] = np.nan
        elif kind == 5:
            target[node, rng.integers(0, V)] = np.inf
        elif kind == 6:
            target[node, :] = -np.inf
        elif kind == 7:
            tokens[child] = int(rng.choice([-3, V, V + 1]))
        elif kind == 8:
            parents[child] = int(rng.integers(child - b * N, N + 2))   # not before the node (or past N)
        elif kind == 9:
            ua[child] = rng.choice([np.nan, 1.0, -0.5])
        elif kind == 10:
            uf[b] = rng.choice([np.nan, 2.0])
        elif kind == 11:
            target[node, rng.integers(0, V, 10)] = -np.inf
    tw = W.TreeWorkload("tree faults", V, B, N, target, parents, tokens, ua, uf, 0.8)
    for mode in ("greedy", "target_only"):
        _say("random tree faults", seed, mode)
        compare_tree(tw, mode, oracle_tree(tw, mode), run_tree(tw, mode))


@pytest.mark.parametrize("seed", [*range(6), *_FUZZ])
def test_random_tree_shapes_match_the_oracle(seed):
    """Seeded random tree batches across the launch paths (one-workgroup walks, per-request scans, draw
    workgroup counts): 1..200 trees of 1..100 nodes (parents uniform over the earlier nodes, each token the
    parent's argmax with probability 0.6, else uniform), vocab 1..5000 (fewer for large batches), fp32 or
    bf16 logits, temperature 0.3..1.5; greedy and target-only, every tree compared with the oracle."""
    rng = np.random.default_rng(950 + seed)
    B = int(rng.integers(1, 201))
    N = int(rng.integers(1, 101))
    V = int(max(1, min(int(rng.integers(1, 5001)), 8_000_000 // (B * N))))
    target = (rng.normal(0, 2, (B * N, V)) * rng.uniform(0.5, 2.0)).astype(np.float32)
    parents = np.full(B * N, -1, np.int32)
    tokens = np.zeros(B * N, np.int32)
    for b in range(B):
        for i in range(1, N):
            par = int(rng.integers(0, i))
            parents[b * N + i] = par
            tokens[b * N + i] = int(np.argmax(target[b * N + par])) if rng.random() < 0.6 else int(rng.integers(V))
    if rng.integers(0, 2):
        target = W.bf16_bits(target)
    tw = W.TreeWorkload("random tree", V, B, N, target, parents, tokens, rng.random(B * N).astype(np.float32),
                        rng.random(B).astype(np.float32), float(rng.uniform(0.3, 1.5)))
    for mode in ("greedy", "target_only"):
        _say("random tree shape", seed, B, N, V, target.dtype, mode)
        compare_tree(tw, mode, oracle_tree(tw, mode), run_tree(tw, mode))


def test_chain_shaped_tree_matches_chain_on_gpu():
    w = W.block_greedy(seed=3003, batch=16, vocab=5003, parallel=False)
    N = 16
    parents = np.tile(np.arange(-1, N - 1, dtype=np.int32), w.batch)
    tokens = np.concatenate([[0] + list(w.draft_tokens[b * 15:(b + 1) * 15]) for b in range(w.batch)]).astype(np.int32)
    tw = W.TreeWorkload("chain_tree", w.vocab, w.batch, N, w.target, parents, tokens,
                        np.zeros(w.batch * N, np.float32), np.zeros(w.batch, np.float32), 1.0)
    gc = run_chain(w, "greedy")
    gt = run_tree(tw, "greedy")
    for k in ("accept_len", "bonus", "out_tokens", "accept_index"):
        assert np.array_equal(gc[k], gt[k]), k


# ----------------------------------------------------------------------------------------------------
# determinism, unwritten outputs, workspace reuse across calls
# ----------------------------------------------------------------------------------------------------
def test_determinism_poisoned_outputs_and_workspace_reuse():
    wa = W.ragged(seed=5002, batch=64, vocab=30011)
    wb = W.chain_rejection(seed=2002, batch=8, vocab=30011, parallel=False)
    ws = dva.workspace("chain", "rejection", wa.total_rows, wa.vocab, wa.batch, 16)
    outs = []
    for rep in range(2):
        for w in (wa, wb):
            out = {k: torch.full((n,), 0x7EEEEEEE, dtype=torch.int32, device="cuda") for k, n in
                   (("accept_len", w.batch), ("bonus", w.batch), ("out_tokens", w.total_rows),
                    ("accept_index", w.total_rows), ("status", w.batch))}
            g = run_chain(w, "rejection", ws=ws, out=out)
            for k in ("accept_len", "bonus", "out_tokens", "accept_index", "status"):
                assert not np.any(g[k].view(np.int32) == 0x7EEEEEEE), k
            outs.append(g)
    for a, b in ((outs[0], outs[2]), (outs[1], outs[3])):
        for k in a:
            assert np.array_equal(a[k], b[k]), k
    o = oracle_chain(wb, "rejection")
    compare_chain(wb, "rejection", o, outs[3])


def _poisoned(n_req, n_rows, n_prob):
    out = {k: torch.full((n,), 0x7EEEEEEE, dtype=torch.int32, device="cuda") for k, n in
           (("accept_len", n_req), ("bonus", n_req), ("out_tokens", n_rows), ("accept_index", n_rows),
            ("status", n_req))}
    out["accept_prob"] = torch.full((n_prob,), float("nan"), dtype=torch.float32, device="cuda")
    out["residual_mass"] = torch.full((n_req,), float("nan"), dtype=torch.float32, device="cuda")
    return out


def _all_written(g):
    for k in ("accept_len", "bonus", "out_tokens", "accept_index", "status"):
        assert not np.any(g[k].view(np.int32) == 0x7EEEEEEE), k
    assert not np.isnan(g["accept_prob"]).any() and not np.isnan(g["residual_mass"]).any()


@pytest.mark.parametrize("mode", ["target_only", "greedy"])
def test_tree_determinism_poisoned_outputs_and_workspace_reuse(mode):
    """spec_verify_tree run twice on the same inputs, with a call of another shape in between on the same
    workspace and every output poisoned before each call: bitwise identical results, every output written,
    and the oracle's results."""
    ta = W.tree(seed=4011, batch=24, vocab=30011)
    tb = W.tree(seed=4012, batch=6, n_nodes=17, vocab=20011, parallel=False)
    ws = torch.empty(max(dva.workspace_bytes("tree", mode, w.total_rows, w.vocab, w.batch, w.n_nodes)
                         for w in (ta, tb)), dtype=torch.uint8, device="cuda")
    outs = []
    for rep in range(2):
        for w in (ta, tb):
            outs.append(run_tree(w, mode, ws=ws, out=_poisoned(w.batch, w.total_rows, w.total_rows)))
            _all_written(outs[-1])
    for a, b in ((outs[0], outs[2]), (outs[1], outs[3])):
        for k in a:
            assert np.array_equal(a[k], b[k], equal_nan=True), k
    compare_tree(tb, mode, oracle_tree(tb, mode), outs[3])
    compare_tree(ta, mode, oracle_tree(ta, mode), outs[2])


def test_sample_match_determinism_poisoned_outputs_and_workspace_reuse():
    """The same for sample-then-match chains (piece partials and the per-row draws)."""
    wa = W.block_sample(seed=7021, batch=16, vocab=30016)
    wb = W.ragged(seed=5021, batch=20, vocab=4099, parallel=False)
    ws = torch.empty(max(dva.workspace_bytes("chain", "sample_match", w.total_rows, w.vocab, w.batch, 16)
                         for w in (wa, wb)), dtype=torch.uint8, device="cuda")
    outs = []
    for rep in range(2):
        for w in (wa, wb):
            outs.append(run_chain(w, "sample_match", ws=ws,
                                  out=_poisoned(w.batch, w.total_rows, w.total_rows - w.batch)))
            _all_written(outs[-1])
    for a, b in ((outs[0], outs[2]), (outs[1], outs[3])):
        for k in a:
            assert np.array_equal(a[k], b[k], equal_nan=True), k
    compare_chain(wb, "sample_match", oracle_chain(wb, "sample_match"), outs[3])
    compare_chain(wa, "sample_match", oracle_chain(wa, "sample_match"), outs[2])


# ----------------------------------------------------------------------------------------------------
# statistics on the GPU: emitted tokens follow p
# ----------------------------------------------------------------------------------------------------
def test_gpu_chi_square_emitted_tokens_follow_p():
    rng = np.random.default_rng(41)
    N, m, V, T = 200_000, 3, 16, 0.8
    tl = rng.normal(0, 1.5, (m + 1, V)).astype(np.float32)
    sl = (tl[:m] + rng.normal(0, 1.0, (m, V))).astype(np.float32)
    p = [np.exp(x / T - (x / T).max()) / np.exp(x / T - (x / T).max()).sum() for x in tl.astype(np.float64)]
    q = [np.exp(x / T - (x / T).max()) / np.exp(x / T - (x / T).max()).sum() for x in sl.astype(np.float64)]
    target = torch.from_numpy(tl).cuda().repeat(N, 1)
    draft = torch.from_numpy(sl).cuda().repeat(N, 1)
    toks = np.stack([rng.choice(V, size=N, p=q[j]) for j in range(m)], 1).reshape(-1).astype(np.int32)
    offs = (np.arange(N + 1) * (m + 1)).astype(np.int32)
    o = dva.verify_chain(target, dev(offs), dev(toks), "rejection", draft_logits=draft,
                         u_accept=dev(rng.random(N * m).astype(np.float32)), u_final=dev(rng.random(N).astype(np.float32)),
                         temperature=T, max_verify_len=m + 1)
    g = np_out(o)
    r = g["accept_len"]
    pv = []
    for k in range(m + 1):
        sel = np.flatnonzero(r >= k)
        t = g["out_tokens"][offs[sel] + k]
        pv.append(stats.chisquare(np.bincount(t, minlength=V), p[k] * len(sel)).pvalue)
    assert min(pv) > 1e-3 / (m + 1), pv
    beta = [np.minimum(p[j], q[j]).sum() for j in range(m)]
    er = sum(np.prod(beta[:k]) for k in range(1, m + 1))
    assert abs(r.mean() - er) < 4 * r.std() / np.sqrt(N)


# ----------------------------------------------------------------------------------------------------
# commit
# ----------------------------------------------------------------------------------------------------
def _commit_check(offsets, accept_len, accept_index, slots, seq, max_len):
    g = np_out(dva.commit_indices(dev(offsets, torch.int32), dev(accept_len, torch.int32),
                                  dev(accept_index, torch.int32), dev(slots, torch.int64), dev(seq, torch.int32),
                                  max_verify_len=max_len))
    o = oracle.commit_indices(offsets, accept_len, accept_index, slots, seq, max_len)
    n = int(o["commit_offsets"][-1])
    ne = int(o["evict_offsets"][-1])
    assert np.array_equal(g["commit_offsets"], o["commit_offsets"])
    assert np.array_equal(g["src_slots"][:n], o["src_slots"])
    assert np.array_equal(g["dst_pos"][:n], o["dst_pos"])
    assert np.array_equal(g["new_seq_lens"], o["new_seq_lens"])
    assert np.array_equal(g["status"], o["status"])
    assert np.array_equal(g["evict_offsets"], o["evict_offsets"])
    assert np.array_equal(g["evict_slots"][:ne], o["evict_slots"])
    return g


def test_commit_parity_chain_and_tree():
    w = W.ragged(seed=5003, batch=1500, vocab=64, parallel=False)     # > one tile of 1024 requests
    g = run_chain(w, "rejection")
    slots = W.verify_slots_for(w.total_rows)
    seq = W.seq_lens_for(w.batch)
    _commit_check(w.offsets, g["accept_len"], g["accept_index"], slots, seq, 16)
    tw = W.tree(seed=4003, batch=8, vocab=2000, parallel=False)
    gt = run_tree(tw, "greedy")
    offs = (np.arange(tw.batch + 1) * tw.n_nodes).astype(np.int32)
    _commit_check(offs, gt["accept_len"], gt["accept_index"], W.verify_slots_for(tw.total_rows), W.seq_lens_for(8),
                  tw.n_nodes)
    # worked example: verify D E F G H, E F accepted -> commit D E F after 3 committed tokens
    _commit_check(np.array([0, 5], np.int32), np.array([2], np.int32), np.array([0, 1, 2, -1, -1], np.int32),
                  np.arange(100, 105), np.array([3], np.int32), 5)
    # invalid accept lengths / indices are reported
    g2 = np_out(dva.commit_indices(dev(np.array([0, 3, 6], np.int32)), dev(np.array([5, 1], np.int32)),
                                   dev(np.array([0, 1, 2, 3, 3, -1], np.int32)), dev(np.arange(6, dtype=np.int64)),
                                   dev(np.array([0, 0], np.int32)), max_verify_len=4))
    assert g2["status"][0] & oracle.ST_BAD_ACCEPT and g2["status"][1] & oracle.ST_BAD_ACCEPT


@pytest.mark.parametrize("seed", [31, 32])
def test_commit_random_accept_index(seed):
    """Seeded commit inputs that mix the form the verify kernels write (accept_index = the request's first r + 1
    rows) with scrambled ones: other rows of the request, rows listed twice, rows of other requests, -1, and
    accept lengths out of range. Every output equals the oracle's."""
    rng = np.random.default_rng(seed)
    B = 300
    lens = rng.integers(1, 17, B)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(offs[-1])
    acc = np.full(T, -1, np.int32)
    alen = np.zeros(B, np.int32)
    for b in range(B):
        o0, n = int(offs[b]), int(lens[b])
        r = int(rng.integers(0, n))
        kind = rng.integers(0, 6)
        if kind == 0:                       # accept length out of range (clamped and reported)
            alen[b] = int(rng.choice([-1, n, n + 3]))
            acc[o0:o0 + n] = np.arange(o0, o0 + n)
            continue
        alen[b] = r
        if kind <= 2:                       # the verify kernels' form
            acc[o0:o0 + r + 1] = np.arange(o0, o0 + r + 1)
        elif kind == 3:                     # a permutation of the request's rows
            acc[o0:o0 + r + 1] = o0 + rng.permutation(n)[: r + 1]
        elif kind == 4:                     # duplicates
            acc[o0:o0 + r + 1] = o0 + rng.integers(0, max(1, r), r + 1)
        else:                               # rows outside the request, or -1
            acc[o0:o0 + r + 1] = rng.choice([-1, 0, T - 1, o0 + n], r + 1)
    print("commit random", seed, flush=True)
    _commit_check(offs, alen, acc, rng.integers(0, 1 << 40, T).astype(np.int64),
                  rng.integers(0, 4096, B).astype(np.int32), 16)


def test_inconsistent_offsets_are_reported_and_stay_in_bounds():
    # Offsets that describe no valid packing; every request checks its own bounds (draft rows inside
    # [0, T - B)), reports BAD_OFFSETS, and the kernels touch nothing outside the given buffers.
    rng = np.random.default_rng(21)
    V, T, B = 300, 10, 3
    tl = rng.normal(0, 1, (T, V)).astype(np.float32)
    dl = rng.normal(0, 1, (T - B, V)).astype(np.float32)
    toks = rng.integers(0, V, T - B).astype(np.int32)
    for offs in ([0, 10, 5, 10], [0, 2, 2, 10], [1, 4, 7, 10], [0, 4, 7, 9]):
        w = _chain_from(tl, dl, np.array(offs, np.int32), toks, rng.random(T - B), rng.random(B), 1.0, 16)
        o = oracle_chain(w, "rejection")
        for mode in ("greedy", "rejection"):
            g = run_chain(w, mode)
            for b in range(B):
                assert bool(g["status"][b] & oracle.ST_BAD_OFFSETS) == bool(o["status"][b] & oracle.ST_BAD_OFFSETS)
            assert np.any(g["status"] & oracle.ST_BAD_OFFSETS)
        # the commit pass handles the requests whose own offsets pass exactly as the oracle does
        gc = _commit_check(np.array(offs, np.int32), np.zeros(B, np.int32), np.arange(T, dtype=np.int32),
                           np.arange(T, dtype=np.int64), np.zeros(B, np.int32), 16)
        assert np.any(gc["status"] & oracle.ST_BAD_OFFSETS)


def _overlapping_commit_case(rng):
    """Offsets where one interior offset jumps past the next: that request fails its checks, and the requests
    on either side of it both pass while their rows overlap. accept_index holds permutations of each passing
    request's rows (later requests overwrite the entries they share), so entries name rows twice, rows of the
    neighbour, or rows in scrambled order. Returns None when the case would need more than T output entries."""
    B = int(rng.integers(3, 9))
    lens = rng.integers(1, 7, B)
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(offs[-1])
    k = int(rng.integers(1, B - 1))
    offs[k] = min(int(offs[k + 1]) + int(rng.integers(1, 4)), T - B + k)
    if not offs[k] > offs[k + 1]:
        return None
    ok = [oracle.verify._chain_offsets_ok(offs, b, T, B, 16) for b in range(B)]
    if not (ok[k - 1] and ok[k + 1]):
        return None
    acc = rng.integers(-1, T, T).astype(np.int32)
    alen = np.zeros(B, np.int32)
    for b in range(B):
        if not ok[b]:
            continue
        lo, hi = int(offs[b]), int(offs[b + 1])
        r = int(rng.integers(0, hi - lo))
        alen[b] = r
        acc[lo:lo + r + 1] = lo + rng.permutation(hi - lo)[: r + 1]
    slots = rng.integers(0, 1 << 40, T).astype(np.int64)
    seq = rng.integers(0, 4096, B).astype(np.int32)
    o = oracle.commit_indices(offs, alen, acc, slots, seq, 16)
    if o["commit_offsets"][-1] > T or o["evict_offsets"][-1] > T:
        return None
    return offs.astype(np.int32), alen, acc, slots, seq


def test_commit_overlapping_passing_requests():
    """Two requests whose own offsets pass but whose rows overlap (the request between them is bad), with
    permuted accept_index entries: each is committed and evicted exactly as the oracle does (no spurious
    BAD_ACCEPT from the other's entries)."""
    # the hand case: offsets [0, 4, 2, 6], requests 0 and 2 share rows 2-3
    _commit_check(np.array([0, 4, 2, 6], np.int32), np.array([3, 0, 1], np.int32),
                  np.array([1, 0, 3, 2, 5, 4], np.int32), np.arange(10, 16, dtype=np.int64),
                  np.array([7, 0, 9], np.int32), 16)
    rng = np.random.default_rng(41)
    done = 0
    while done < 40:
        c = _overlapping_commit_case(rng)
        if c is None:
            continue
        _commit_check(*c, 16)
        done += 1


def _ln(*p):
    return [float(np.log(x)) if x > 0 else -np.inf for x in p]


def test_near_flags_match_the_oracle_by_hand():
    """The device's own NEAR_ALPHA / NEAR_CDF estimates against the oracle's on requests whose u sits 0.9e-5 or
    1.1e-5 from an accept threshold or a CDF step of known value (the hand-placed cases of the oracle pins,
    V = 3, fp32): the bits agree request by request, and everything compares by the parity contract."""
    a23 = 2.0 / 3.0
    reqs = []   # (target rows, draft rows, drafts, u_accept, u_final)
    for u in (0.5 - 0.9e-5, 0.5 - 1.1e-5, 0.5 + 0.9e-5, 0.5 + 1.1e-5, 0.25 - 0.9e-5, 0.25 + 1.1e-5, 0.75):
        reqs.append(([_ln(.25, .25, .5)], [], [], [], u))
    for u in (0.5 - 0.9e-5, 0.5 - 1.1e-5, 0.5 + 0.9e-5, 0.5 + 1.1e-5):
        reqs.append(([_ln(.4, .3, .3), _ln(.5, .25, .25)], [_ln(.2, .1, .7)], [2], [0.9], u))
    for du in (-0.9e-5, 0.9e-5, -1.1e-5, 1.1e-5):
        reqs.append(([_ln(.5, .5, 0), _ln(.5, .5, 0)], [_ln(.75, .25, 0)], [0], [a23 + du], 0.25))
    rows, drows = [_ln(.5, .5, 0)] * 4, [_ln(.75, .25, 0)] * 3
    reqs.append((rows, drows, [1, 1, 0], [0.3, 0.3, a23 - 0.5e-5], 0.25))
    reqs.append((rows, drows, [1, 1, 0], [0.3, 0.3, a23 - 2e-5], 0.25))
    reqs.append((rows, drows, [0, 0, 0], [0.9, a23 + 1e-7, a23 - 1e-7], 0.5))
    for u in (0.5 - 5e-5, 0.5 - 2e-4, 0.5 + 5e-5, 0.5 + 2e-4):
        reqs.append(([_ln(.2, .3, .5), _ln(.3, .3, .4)], [_ln(.195, .295, .51)], [2], [0.99], u))
    offs = np.concatenate([[0], np.cumsum([len(r[0]) for r in reqs])]).astype(np.int32)
    tl = np.array([x for r in reqs for x in r[0]], np.float32)
    dl = np.array([x for r in reqs for x in r[1]], np.float32)
    w = _chain_from(tl, dl, offs, [d for r in reqs for d in r[2]], [u for r in reqs for u in r[3]],
                    [r[4] for r in reqs], 1.0, 4)
    o, g = oracle_chain(w, "rejection"), run_chain(w, "rejection")
    near = np.uint32(oracle.ST_NEAR_ALPHA | oracle.ST_NEAR_CDF)
    assert np.array_equal(g["status"] & near, o["status"] & near), (g["status"], o["status"])
    assert int(np.count_nonzero(o["status"] & near)) == 10
    compare_chain(w, "rejection", o, g)
    # tree target-only: cumulative child masses 1/4, 1/2 at the root and 1/2 at node 2
    cases = [(0.25 + 0.9e-5, 0.3), (0.25 + 1.1e-5, 0.3), (0.3, 0.5 - 0.9e-5), (0.3, 0.5 - 1.1e-5)]
    B, N = len(cases), 4
    tw = W.TreeWorkload("edge", 3, B, N, np.tile(np.array([_ln(.25, .25, .5)] * N, np.float32), (B, 1)),
                        np.tile(np.array([-1, 0, 0, 2], np.int32), B), np.tile(np.array([0, 0, 1, 2], np.int32), B),
                        np.array([[u0, 0.5, u2, 0.5] for u0, u2 in cases], np.float32).ravel(),
                        np.full(B, 0.9, np.float32), 1.0, ("greedy", "target_only"))
    o, g = oracle_tree(tw, "target_only"), run_tree(tw, "target_only")
    assert np.array_equal(g["status"] & near, o["status"] & near), (g["status"], o["status"])
    assert list(o["flag_pos"]) == [0, 3, 1, 3]
    compare_tree(tw, "target_only", o, g)


def test_gpu_tree_target_only_chi_square():
    """Target-only tree sampling on the GPU emits tokens distributed as p at depth 1 and 2 ([SpecDec], only the
    target's probabilities judge): root children tokens 0, 1 (nodes 1, 2), node 1's children tokens 2, 3
    (nodes 3, 4), node 2 a leaf; 200k requests with independent uniforms. The first emitted token follows
    the root's p; given node 1 was accepted the second follows node 1's row, given node 2 node 2's row."""
    rng = np.random.default_rng(43)
    V, Bn, N = 12, 200_000, 5
    rows = rng.normal(0, 1.0, (N, V)).astype(np.float32)
    p = [np.exp(x - x.max()) / np.exp(x - x.max()).sum() for x in rows.astype(np.float64)]
    parents = np.array([-1, 0, 0, 1, 1], np.int32)
    tokens = np.array([0, 0, 1, 2, 3], np.int32)
    target = torch.from_numpy(rows).cuda().repeat(Bn, 1)
    g = np_out(dva.verify_tree(target, dev(np.tile(parents, Bn)), dev(np.tile(tokens, Bn)), N, "target_only",
                               u_accept=dev(rng.random(Bn * N).astype(np.float32)),
                               u_final=dev(rng.random(Bn).astype(np.float32)), temperature=1.0))
    base = np.arange(Bn) * N
    first = g["out_tokens"][base]
    pv = [stats.chisquare(np.bincount(first, minlength=V), p[0] * Bn).pvalue]
    for node in (1, 2):
        sel = np.flatnonzero((g["accept_len"] >= 1) & (g["accept_index"][base + 1] == base + node))
        second = g["out_tokens"][base[sel] + 1]
        pv.append(stats.chisquare(np.bincount(second, minlength=V), p[node] * len(sel)).pvalue)
        assert len(sel) > 1000
    print("tree target-only chi-square p-values", pv, flush=True)
    assert min(pv) > 1e-3 / len(pv), pv
