"""GPU parity of sample-then-match and of the vocab (grammar) mask: the HIP library through its C ABI against
the fp64 oracle on the same seeded inputs (small vocabularies that span several chunks with an unaligned tail,
then full size), long requests, statuses, a chi-square of the sampled tokens, and an all-ones mask that must
leave every output of every mode unchanged on the GPU."""
import numpy as np
import pytest
import torch
from scipy import stats

import draft_verification_acceptance_amd as dva
import oracle
from draft_verification_acceptance_amd import workloads as W
from gpu_util import (compare_chain, compare_tree, dev, dev_logits, dev_mask, np_out, oracle_chain, oracle_tree,
                      run_chain, run_tree)
from test_oracle_flag_counts import EXPECTED as FLAGGED

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _f32(row):
    return W.bf16_to_f32(row) if row.dtype == np.uint16 else row


def _allowed(mask_row, v):
    return (int(mask_row[v >> 5]) >> (v & 31)) & 1 == 1


def _chain_from(w, target, draft, tokens=None, ua=None, uf=None):
    return W.ChainWorkload(w.name, target.shape[1], w.batch, w.offsets, target, draft,
                           w.draft_tokens if tokens is None else np.asarray(tokens, np.int32),
                           w.u_accept if ua is None else np.asarray(ua, np.float32),
                           w.u_final if uf is None else np.asarray(uf, np.float32), w.temperature, w.modes,
                           w.max_verify_len, cand_ids=w.cand_ids, cand_q=w.cand_q)


# ----------------------------------------------------------------------------------------------------
# sample-then-match
# ----------------------------------------------------------------------------------------------------
def test_sample_match_tiny():
    w = W.tiny_chain()
    _say("sample_match tiny")
    compare_chain(w, "sample_match", oracle_chain(w, "sample_match"), run_chain(w, "sample_match"))


def test_sample_match_small_vocab():
    w = W.chain_rejection(seed=2001, vocab=20011)
    _say("sample_match chain V=20011")
    compare_chain(w, "sample_match", oracle_chain(w, "sample_match"), run_chain(w, "sample_match"))


def test_sample_match_block_small_vocab():
    w = W.block_sample(seed=7001, vocab=20011)
    _say("sample_match block V=20011")
    g = run_chain(w, "sample_match")
    o = oracle_chain(w, "sample_match")
    compare_chain(w, "sample_match", o, g)
    assert o["accept_len"].max() >= 3


def test_sample_match_block_full():
    w = W.block_sample()
    _say("sample_match block full")
    g = run_chain(w, "sample_match")
    o = oracle_chain(w, "sample_match")
    compare_chain(w, "sample_match", o, g, expect=FLAGGED[("block_sample", "sample_match")])
    assert np.all((g["accept_len"] >= 0) & (g["accept_len"] <= 15))
    assert np.all((g["bonus"] >= 0) & (g["bonus"] < w.vocab))
    assert np.all(g["residual_mass"] == -1)
    assert g["accept_len"].mean() >= 1.0


def test_sample_match_ragged_small_vocab():
    w = W.ragged(seed=5001, vocab=4099)
    _say("sample_match ragged V=4099")
    compare_chain(w, "sample_match", oracle_chain(w, "sample_match"), run_chain(w, "sample_match"))


@pytest.mark.parametrize("V", [1, 7, 4096, 8195, 151936, 151937])   # multiples of 8: piece partials
def test_sample_match_vocab_sizes(V):
    # peaked rows (block_sample): most draws land on a wide CDF step, so few are too close to call
    w = W.block_sample(seed=91 + V, batch=12, block=4, vocab=V, parallel=False)
    for bf16 in (True, False):
        _say("sample_match vocab", V, "bf16" if bf16 else "fp32")
        ww = w if bf16 else _chain_from(w, W.bf16_to_f32(w.target), None)
        compare_chain(ww, "sample_match", oracle_chain(ww, "sample_match"), run_chain(ww, "sample_match"))


@pytest.mark.parametrize("V", [600_008, 600_001])
def test_sample_match_many_units(V):
    """Rows with more units than the draw keeps in registers: 600008 (bf16 pieces of 2048 tokens: 293 of them;
    fp32 pieces of 1024: 586) and 600001 (not 16-byte aligned: 73 stream chunks, more than one per lane)."""
    w = W.block_sample(seed=95, batch=6, block=3, vocab=V, temperature=0.6, parallel=False)
    for bf16 in (True, False):
        _say("sample_match many units", V, "bf16" if bf16 else "fp32")
        ww = w if bf16 else _chain_from(w, W.bf16_to_f32(w.target), None)
        compare_chain(ww, "sample_match", oracle_chain(ww, "sample_match"), run_chain(ww, "sample_match"))


def _long_workload(seed, B, L, V, breaks):
    """Requests of L rows whose rows are all but certain (one token raised by 60): the draft copies that token
    except at the positions in `breaks[b]` (None: never), so the accepted prefix crosses the kernel's groups
    of 16 rows."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (B * L, V)).astype(np.float32)
    top = rng.integers(0, V, B * L)
    x[np.arange(B * L), top] += 60.0
    toks = []
    for b in range(B):
        for j in range(L - 1):
            t = int(top[b * L + j])
            toks.append((t + 1) % V if breaks[b] == j else t)
    offs = (np.arange(B + 1) * L).astype(np.int32)
    return W.ChainWorkload("long", V, B, offs, x, None, np.array(toks, np.int32),
                           rng.uniform(0.01, 0.99, B * (L - 1)).astype(np.float32),
                           rng.uniform(0.01, 0.99, B).astype(np.float32), 1.0, ("sample_match",), L)


def test_sample_match_long_requests():
    breaks = [None, 0, 15, 16, 17, 31, 40, None]
    w = _long_workload(5, len(breaks), 45, 3001, breaks)
    _say("sample_match long requests")
    g = run_chain(w, "sample_match")
    o = oracle_chain(w, "sample_match")
    compare_chain(w, "sample_match", o, g)
    want = [44 if br is None else br for br in breaks]
    assert list(g["accept_len"]) == want


def test_sample_match_statuses():
    w = W.tiny_chain(seed=12, batch=5, m=3, vocab=64)
    t = w.target.copy()
    t[2, 5] = np.nan                               # request 0, row 2
    toks = w.draft_tokens.copy()
    toks[4] = 64                                   # request 1: out-of-range draft token
    ua = w.u_accept.copy()
    ua[7] = 1.5                                    # request 2: bad uniform
    uf = w.u_final.copy()
    uf[3] = np.nan                                 # request 3: bad final uniform
    ww = _chain_from(w, t, w.draft, toks, ua, uf)
    _say("sample_match statuses")
    g = run_chain(ww, "sample_match")
    o = oracle_chain(ww, "sample_match")
    compare_chain(ww, "sample_match", o, g)
    assert g["status"][0] & oracle.ST_NONFINITE
    assert g["status"][1] & oracle.ST_BAD_TOKEN and g["accept_len"][1] <= 1
    assert g["status"][2] & oracle.ST_BAD_UNIFORM and g["status"][3] & oracle.ST_BAD_UNIFORM
    # zero-draft requests: the sample of row 0 is the bonus
    z = W.ragged(seed=5003, batch=40, m_max=0, vocab=1001)
    compare_chain(z, "sample_match", oracle_chain(z, "sample_match"), run_chain(z, "sample_match"))


@pytest.mark.parametrize("masked", [False, True])
def test_sample_match_chi_square(masked):
    """4000 one-row requests share one row; their samples (u_final uniform) follow p (or the masked p)."""
    rng = np.random.default_rng(31)
    V, B, T = 50, 4000, 0.8
    row = rng.normal(0, 1.5, V).astype(np.float32)
    target = np.tile(row, (B, 1))
    offs = np.arange(B + 1, dtype=np.int32)
    w = W.ChainWorkload("chi", V, B, offs, target, None, np.zeros(0, np.int32), np.zeros(0, np.float32),
                        rng.random(B, dtype=np.float32), T, ("sample_match",), 1)
    allowed = np.ones(V, bool)
    mask = None
    if masked:
        allowed[rng.choice(V, 20, replace=False)] = False
        mask = W.vocab_masks(0, B, V, 0.0, keep=[np.flatnonzero(allowed)] * B)
    _say("sample_match chi-square", masked)
    g = run_chain(w, "sample_match", mask=mask)
    x = row.astype(np.float64) / T
    p = np.where(allowed, np.exp(x - x.max()), 0.0)
    p /= p.sum()
    counts = np.bincount(g["bonus"], minlength=V)
    assert counts[~allowed].sum() == 0
    exp = p[allowed] * B
    assert stats.chisquare(counts[allowed], exp).pvalue > 1e-4


# ----------------------------------------------------------------------------------------------------
# vocab mask
# ----------------------------------------------------------------------------------------------------
def _chain_keep(w):
    """Per target row: its judged draft token and its argmax stay allowed, so acceptances still happen."""
    return W.chain_keep(w)


def _check_allowed_outputs(g, mask, rows_of):
    for b, rows in rows_of:
        for k, t in zip(rows, g["out_tokens"][rows]):
            if t >= 0:
                assert _allowed(mask[k], int(t)), (b, k, int(t))


@pytest.mark.parametrize("mode", ["greedy", "rejection", "rejection_sparse", "sample_match"])
def test_mask_chain_modes_small_vocab(mode):
    if mode == "greedy":
        w = W.block_greedy(seed=3001, vocab=20011, tie_rate=0.2)
    elif mode == "rejection_sparse":
        w = W.chain_sparse(seed=6001, vocab=20011)
    else:
        w = W.chain_rejection(seed=2001, vocab=20011)
    mask = W.vocab_masks(11, w.total_rows, w.vocab, 0.3, _chain_keep(w))
    _say("mask chain", mode)
    g = run_chain(w, mode, mask=mask)
    o = oracle_chain(w, mode, mask=mask)
    compare_chain(w, mode, o, g)
    assert o["accept_len"].max() >= 1
    rows = [(b, np.arange(int(w.offsets[b]), int(w.offsets[b + 1]))) for b in range(w.batch)]
    _check_allowed_outputs(g, mask, rows)


@pytest.mark.parametrize("mode", ["greedy", "target_only"])
def test_mask_tree_small_vocab(mode):
    w = W.tree(seed=4001, vocab=12007)
    N = w.n_nodes
    keep = []
    for i in range(w.batch * N):
        b, n = divmod(i, N)
        kids = [int(w.tokens[b * N + c]) for c in range(n + 1, N) if int(w.parents[b * N + c]) == n]
        keep.append(kids + [int(np.argmax(_f32(w.target[i])))])
    mask = W.vocab_masks(12, w.batch * N, w.vocab, 0.2, keep)
    _say("mask tree", mode)
    g = run_tree(w, mode, mask=mask)
    o = oracle_tree(w, mode, mask=mask)
    compare_tree(w, mode, o, g)
    assert o["accept_len"].max() >= 1
    # the bonus (drawn or argmax) is allowed in its row
    for b in range(w.batch):
        r = int(g["accept_len"][b])
        node = int(g["accept_index"][b * N + r]) if r >= 0 else b * N
        if not g["status"][b] & oracle.ST_NONFINITE:
            assert _allowed(mask[node], int(g["bonus"][b]))


def test_mask_full_chain_rejection_and_block_sample():
    w = W.chain_rejection()
    mask = W.vocab_masks(13, w.total_rows, w.vocab, 0.05, _chain_keep(w))
    _say("mask full chain_rejection")
    g = run_chain(w, "rejection", mask=mask)
    o = oracle_chain(w, "rejection", mask=mask)
    compare_chain(w, "rejection", o, g, expect=FLAGGED[("chain_rejection+mask13", "rejection")])
    assert not np.any(g["status"] & ~np.uint32(oracle.ST_NEAR_ALPHA | oracle.ST_NEAR_CDF))
    rows = [(b, np.arange(int(w.offsets[b]), int(w.offsets[b + 1]))) for b in range(w.batch)]
    _check_allowed_outputs(g, mask, rows)
    s = W.block_sample()
    smask = W.vocab_masks(14, s.total_rows, s.vocab, 0.05, _chain_keep(s))
    _say("mask full block_sample")
    gs = run_chain(s, "sample_match", mask=smask)
    compare_chain(s, "sample_match", oracle_chain(s, "sample_match", mask=smask), gs,
                  expect=FLAGGED[("block_sample+mask14", "sample_match")])
    rows = [(b, np.arange(int(s.offsets[b]), int(s.offsets[b + 1]))) for b in range(s.batch)]
    _check_allowed_outputs(gs, smask, rows)


def test_mask_edge_cases():
    w = W.tiny_chain(seed=17, batch=4, m=3, vocab=96)
    t = w.target.copy()
    t[0, 7] = np.nan                       # masked NaN and +inf: ignored
    t[1, 8] = np.inf
    keep = _chain_keep(w)
    mask = W.vocab_masks(15, w.total_rows, w.vocab, 0.5, keep)
    mask[0, 0] &= ~np.uint32(1 << 7)
    mask[1, 0] &= ~np.uint32(1 << 8)
    mask[6] = 0                            # request 1, row 2: nothing allowed
    ww = _chain_from(w, t, w.draft)
    for mode in ("greedy", "rejection", "sample_match"):
        _say("mask edge", mode)
        g = run_chain(ww, mode, mask=mask)
        o = oracle_chain(ww, mode, mask=mask)
        compare_chain(ww, mode, o, g)
        assert not g["status"][0] & oracle.ST_NONFINITE
        assert g["status"][1] & oracle.ST_NONFINITE
    # unaligned vocab sizes, fp32 and bf16
    for V in (1, 8195):
        u = W.tiny_chain(seed=19 + V, batch=6, m=3, vocab=V)
        um = W.vocab_masks(16, u.total_rows, V, 0.4, _chain_keep(u))
        for bf16 in (False, True):
            uu = _chain_from(u, W.bf16_bits(u.target), W.bf16_bits(u.draft)) if bf16 else u
            for mode in ("greedy", "rejection", "sample_match"):
                _say("mask vocab", V, mode, bf16)
                compare_chain(uu, mode, oracle_chain(uu, mode, mask=um), run_chain(uu, mode, mask=um))
    # tree: a node row that allows nothing
    tw = W.tree(seed=4003, batch=3, vocab=1001)
    tm = W.vocab_masks(17, tw.batch * tw.n_nodes, tw.vocab, 0.5)
    tm[tw.n_nodes] = 0
    for mode in ("greedy", "target_only"):
        g = run_tree(tw, mode, mask=tm)
        o = oracle_tree(tw, mode, mask=tm)
        compare_tree(tw, mode, o, g)
        assert g["status"][1] & oracle.ST_NONFINITE


def test_all_ones_mask_equals_no_mask_on_gpu():
    w = W.chain_sparse(seed=6002, vocab=20011)
    ones = np.full((w.total_rows, (w.vocab + 31) // 32), 0xFFFFFFFF, np.uint32)
    for mode in ("greedy", "rejection_sparse", "sample_match"):
        a = run_chain(w, mode)
        b = run_chain(w, mode, mask=ones)
        for key in a:
            assert np.array_equal(a[key], b[key]), (mode, key)
    r = W.chain_rejection(seed=2002, vocab=20011)
    ones = np.full((r.total_rows, (r.vocab + 31) // 32), 0xFFFFFFFF, np.uint32)
    a, b = run_chain(r, "rejection"), run_chain(r, "rejection", mask=ones)
    for key in a:
        assert np.array_equal(a[key], b[key]), ("rejection", key)
    t = W.tree(seed=4002, vocab=12007)
    ones = np.full((t.batch * t.n_nodes, (t.vocab + 31) // 32), 0xFFFFFFFF, np.uint32)
    for mode in ("greedy", "target_only"):
        a, b = run_tree(t, mode), run_tree(t, mode, mask=ones)
        for key in a:
            assert np.array_equal(a[key], b[key]), (mode, key)
