"""GPU: the KV commit fused into the verify call against spec_commit_indices run on the verify's outputs.

The fused commit runs in the verify call's second kernel (the workgroup whose request finishes its accept scan
last). Its outputs must be bit-identical to the standalone commit's on the same round, for every verify mode,
for chains and trees, with bad offsets among the requests, over several tiles of requests, and when the call is
captured in a HIP graph and replayed.
"""
import numpy as np
import pytest
import torch

import draft_verification_acceptance_amd as dva
import oracle
from draft_verification_acceptance_amd import workloads as W
from gpu_util import compare_chain, compare_tree, dev, dev_logits, np_out, oracle_chain, oracle_tree

pytestmark = pytest.mark.gpu

KEYS = ("commit_offsets", "src_slots", "dst_pos", "new_seq_lens", "evict_offsets", "evict_slots")


def _chain_kw(w, mode):
    kw = dict(max_verify_len=w.max_verify_len)
    if mode != "greedy":
        kw.update(u_accept=dev(w.u_accept), u_final=dev(w.u_final), temperature=w.temperature)
    if mode == "rejection":
        kw.update(draft_logits=dev_logits(w.draft))
    if mode == "rejection_sparse":
        kw.update(cand_ids=dev(w.cand_ids, torch.int32), cand_q=dev(w.cand_q, torch.float32))
    return kw


def _check(g, offsets, max_len, slots, seq, accept_index=None):
    """Fused outputs g against spec_commit_indices on g's own accept_len / accept_index (or the given
    accept_index), and against the oracle's commit of them."""
    ai = g["accept_index"] if accept_index is None else accept_index
    s = np_out(dva.commit_indices(dev(offsets, torch.int32), dev(g["accept_len"]), dev(ai, torch.int32),
                                  dev(slots), dev(seq), max_verify_len=max_len))
    n, ne = int(s["commit_offsets"][-1]), int(s["evict_offsets"][-1])
    for k in KEYS:
        m = {"src_slots": n, "dst_pos": n, "evict_slots": ne}.get(k)
        a, b = g[k], s[k]
        if m is not None:
            a, b = a[:m], b[:m]
        assert np.array_equal(a, b), k
    assert np.array_equal(g["commit_status"].view(np.uint32), s["status"]), "status"
    o = oracle.commit_indices(offsets, g["accept_len"], ai, slots, seq, max_len)
    assert np.array_equal(g["commit_offsets"], o["commit_offsets"])
    assert np.array_equal(g["src_slots"][:n], o["src_slots"]) and np.array_equal(g["evict_slots"][:ne], o["evict_slots"])
    return n


@pytest.mark.parametrize("name,mode", [("tiny_chain", "greedy"), ("tiny_chain", "rejection"),
                                       ("chain_rejection", "rejection"), ("block_greedy", "greedy"),
                                       ("ragged", "rejection"), ("chain_sparse", "rejection_sparse"),
                                       ("block_sample", "sample_match"), ("ragged", "greedy")])
def test_fused_commit_chain_matches_standalone(name, mode):
    w = W.FULL[name]()
    print("fused commit", name, mode, w.batch, w.total_rows, flush=True)
    slots = W.verify_slots_for(w.total_rows)
    seq = W.seq_lens_for(w.batch)
    g = np_out(dva.verify_chain(dev_logits(w.target), dev(w.offsets, torch.int32), dev(w.draft_tokens, torch.int32),
                                mode, verify_slots=dev(slots), seq_lens=dev(seq), **_chain_kw(w, mode)))
    n = _check(g, w.offsets, w.max_verify_len, slots, seq)
    assert n == int(g["accept_len"].sum()) + w.batch


@pytest.mark.parametrize("mode", ["greedy", "target_only"])
def test_fused_commit_tree_matches_standalone(mode):
    for w in (W.tree(), W.tree(seed=4021, batch=300, n_nodes=9, vocab=4099, parallel=False)):   # > one tile
        print("fused commit tree", mode, w.batch, w.n_nodes, flush=True)
        slots = W.verify_slots_for(w.total_rows)
        seq = W.seq_lens_for(w.batch)
        kw = {}
        if mode == "target_only":
            kw = dict(u_accept=dev(w.u_accept), u_final=dev(w.u_final), temperature=w.temperature)
        g = np_out(dva.verify_tree(dev_logits(w.target), dev(w.parents), dev(w.tokens), w.n_nodes, mode,
                                   verify_slots=dev(slots), seq_lens=dev(seq), **kw))
        offs = (np.arange(w.batch + 1) * w.n_nodes).astype(np.int32)
        _check(g, offs, w.n_nodes, slots, seq)


@pytest.mark.parametrize("mode", ["rejection", "greedy", "sample_match"])
def test_fused_commit_many_tiles_and_bad_offsets(mode):
    """1500 requests (six tiles of the commit), then offsets where some requests fail their checks."""
    w = W.ragged(seed=5031, batch=1500, vocab=64, parallel=False)
    slots = np.random.default_rng(3).integers(0, 1 << 40, w.total_rows).astype(np.int64)
    seq = np.random.default_rng(4).integers(0, 4096, w.batch).astype(np.int32)
    g = np_out(dva.verify_chain(dev_logits(w.target), dev(w.offsets, torch.int32), dev(w.draft_tokens, torch.int32),
                                mode, verify_slots=dev(slots), seq_lens=dev(seq), **_chain_kw(w, mode)))
    _check(g, w.offsets, w.max_verify_len, slots, seq)
    offs = w.offsets.copy()
    offs[7] = offs[8] + 1            # request 7 fails; 6 and 8 pass with overlapping rows
    offs[300] = offs[299]            # request 299 empty
    g = np_out(dva.verify_chain(dev_logits(w.target), dev(offs, torch.int32), dev(w.draft_tokens, torch.int32),
                                mode, verify_slots=dev(slots), seq_lens=dev(seq), **_chain_kw(w, mode)))
    assert g["commit_status"][7] & oracle.ST_BAD_OFFSETS and g["commit_status"][299] & oracle.ST_BAD_OFFSETS
    # With bad offsets in the batch the verify outputs are unspecified (requests 6 and 8 share rows, and both
    # write accept_index there); each request whose own offsets pass still commits its first accept_len + 1
    # rows: the commit of accept_index[x] = x for every row x.
    _check(g, offs, w.max_verify_len, slots, seq, accept_index=np.arange(w.total_rows, dtype=np.int32))


@pytest.mark.parametrize("mode", ["greedy", "rejection"])
def test_fused_commit_small_batch_bad_offsets(mode):
    """40 requests (greedy: the one-workgroup path, which scans and commits the batch from LDS), with the
    same kinds of failing offsets."""
    w = W.ragged(seed=5033, batch=40, vocab=64, parallel=False)
    slots = np.random.default_rng(5).integers(0, 1 << 40, w.total_rows).astype(np.int64)
    seq = np.random.default_rng(6).integers(0, 4096, w.batch).astype(np.int32)
    g = np_out(dva.verify_chain(dev_logits(w.target), dev(w.offsets, torch.int32), dev(w.draft_tokens, torch.int32),
                                mode, verify_slots=dev(slots), seq_lens=dev(seq), **_chain_kw(w, mode)))
    _check(g, w.offsets, w.max_verify_len, slots, seq)
    offs = w.offsets.copy()
    offs[7] = offs[8] + 1            # request 7 fails; 6 and 8 pass with overlapping rows
    offs[20] = offs[19]              # request 19 empty
    g = np_out(dva.verify_chain(dev_logits(w.target), dev(offs, torch.int32), dev(w.draft_tokens, torch.int32),
                                mode, verify_slots=dev(slots), seq_lens=dev(seq), **_chain_kw(w, mode)))
    assert g["commit_status"][7] & oracle.ST_BAD_OFFSETS and g["commit_status"][19] & oracle.ST_BAD_OFFSETS
    _check(g, offs, w.max_verify_len, slots, seq, accept_index=np.arange(w.total_rows, dtype=np.int32))


def _poison(outs):
    for t in outs.values():
        t.fill_(-12345.0 if t.dtype == torch.float32 else -5)


@pytest.mark.parametrize("kind", ["chain", "tree", "greedy_chain", "sample_match"])
def test_fused_commit_graph_replay(kind):
    """Captured once, replayed several times with other library work and synchronisations between the replays;
    every replay's verify and commit outputs equal the eager call's (outputs poisoned before each run, so the
    capacity past the committed entries keeps the poison in all of them)."""
    if kind == "tree":
        w = W.tree(seed=4031, batch=24, vocab=30011, parallel=False)
        slots, seq = W.verify_slots_for(w.total_rows), W.seq_lens_for(w.batch)
        call = dva.prepare_verify_tree(dev_logits(w.target), dev(w.parents), dev(w.tokens), w.n_nodes, "target_only",
                                       u_accept=dev(w.u_accept), u_final=dev(w.u_final), temperature=1.0,
                                       verify_slots=dev(slots), seq_lens=dev(seq))
    else:
        mode = {"chain": "rejection", "greedy_chain": "greedy", "sample_match": "sample_match"}[kind]
        w = (W.block_sample(seed=7031, vocab=20008, parallel=False) if kind == "sample_match" else
             W.chain_rejection(seed=2031, batch=48, vocab=30011, parallel=False))
        slots, seq = W.verify_slots_for(w.total_rows), W.seq_lens_for(w.batch)
        call = dva.prepare_verify_chain(dev_logits(w.target), dev(w.offsets, torch.int32),
                                        dev(w.draft_tokens, torch.int32), mode, verify_slots=dev(slots),
                                        seq_lens=dev(seq), **_chain_kw(w, mode))
    other = W.chain_rejection(seed=2032, vocab=3001, parallel=False)
    o_slots, o_seq = W.verify_slots_for(other.total_rows), W.seq_lens_for(other.batch)
    other_call = dva.prepare_verify_chain(dev_logits(other.target), dev(other.offsets, torch.int32),
                                          dev(other.draft_tokens, torch.int32), "rejection", verify_slots=dev(o_slots),
                                          seq_lens=dev(o_seq), **_chain_kw(other, "rejection"))
    _poison(call.outputs)
    call.run()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in call.outputs.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call.run()
    for rep in range(4):
        _poison(call.outputs)
        other_call.run()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, t in ref.items():
            assert torch.equal(call.outputs[k], t), (kind, rep, k)


@pytest.mark.parametrize("batch,m_max", [(1024, 1), (30, 63)])
def test_one_workgroup_greedy_chain_limits(batch, m_max):
    """Greedy chain batches at the one-workgroup path's limits (1024 requests; requests of 64 rows): verify
    outputs equal the oracle's, the fused commit equals the standalone commit."""
    w = W.ragged(seed=5041, batch=batch, m_max=m_max, vocab=97, parallel=False)
    assert w.total_rows <= 2048 and w.max_verify_len <= 64
    print("one-workgroup greedy chain", batch, w.max_verify_len, w.total_rows, flush=True)
    slots = np.random.default_rng(7).integers(0, 1 << 40, w.total_rows).astype(np.int64)
    seq = np.random.default_rng(8).integers(0, 4096, w.batch).astype(np.int32)
    g = np_out(dva.verify_chain(dev_logits(w.target), dev(w.offsets, torch.int32), dev(w.draft_tokens, torch.int32),
                                "greedy", verify_slots=dev(slots), seq_lens=dev(seq), **_chain_kw(w, "greedy")))
    assert compare_chain(w, "greedy", oracle_chain(w, "greedy"), g) == 0
    _check(g, w.offsets, w.max_verify_len, slots, seq)


@pytest.mark.parametrize("batch,block", [(64, 16), (256, 4), (65, 16)])
def test_sample_match_short_request_batches(batch, block):
    """Sample-then-match batches of short requests (the split kernel: four rows per workgroup, each request
    finished by its last workgroup, the commit by the last request): 64 x 16 and 65 x 16 rows, 256 requests of
    4 rows. Verify outputs equal the oracle's, the fused commit the standalone commit."""
    w = W.block_sample(seed=7061 + batch, batch=batch, block=block, vocab=4099, parallel=False)
    print("sample_match", batch, block, w.total_rows, flush=True)
    slots = np.random.default_rng(12).integers(0, 1 << 40, w.total_rows).astype(np.int64)
    seq = np.random.default_rng(13).integers(0, 4096, w.batch).astype(np.int32)
    g = np_out(dva.verify_chain(dev_logits(w.target), dev(w.offsets, torch.int32), dev(w.draft_tokens, torch.int32),
                                "sample_match", verify_slots=dev(slots), seq_lens=dev(seq),
                                **_chain_kw(w, "sample_match")))
    compare_chain(w, "sample_match", oracle_chain(w, "sample_match"), g)
    _check(g, w.offsets, w.max_verify_len, slots, seq)


@pytest.mark.parametrize("max_len", [1, 2, 3, 5, 8, 9, 17, 33])
def test_one_workgroup_greedy_chain_segments(max_len):
    """The one-workgroup greedy path packs 64 / Lp requests into a wave (Lp: the smallest power of two >= the
    longest request): ragged batches whose longest request is 1 .. 33 rows, so segments of 1 .. 64 lanes,
    with requests shorter than their segment. Verify outputs equal the oracle's, the fused commit the
    standalone commit."""
    batch = min(1024, 2048 // max_len)
    w = W.ragged(seed=5070 + max_len, batch=batch, m_max=max_len - 1, vocab=61, parallel=False)
    assert w.max_verify_len == max_len and w.total_rows <= 2048
    print("one-workgroup greedy chain segments", batch, max_len, w.total_rows, flush=True)
    slots = np.random.default_rng(14).integers(0, 1 << 40, w.total_rows).astype(np.int64)
    seq = np.random.default_rng(15).integers(0, 4096, w.batch).astype(np.int32)
    g = np_out(dva.verify_chain(dev_logits(w.target), dev(w.offsets, torch.int32), dev(w.draft_tokens, torch.int32),
                                "greedy", verify_slots=dev(slots), seq_lens=dev(seq), **_chain_kw(w, "greedy")))
    assert compare_chain(w, "greedy", oracle_chain(w, "greedy"), g) == 0
    _check(g, w.offsets, w.max_verify_len, slots, seq)


@pytest.mark.parametrize("batch,n_nodes", [(1024, 2), (32, 64), (33, 62)])
def test_one_workgroup_greedy_tree_limits(batch, n_nodes):
    """Greedy tree batches at the one-workgroup path's limits (2048 nodes; trees of 64 nodes)."""
    w = W.tree(seed=4041, batch=batch, n_nodes=n_nodes, vocab=301, parallel=False)
    print("one-workgroup greedy tree", batch, n_nodes, flush=True)
    slots = np.random.default_rng(9).integers(0, 1 << 40, w.total_rows).astype(np.int64)
    seq = np.random.default_rng(10).integers(0, 4096, w.batch).astype(np.int32)
    g = np_out(dva.verify_tree(dev_logits(w.target), dev(w.parents), dev(w.tokens), w.n_nodes, "greedy",
                               verify_slots=dev(slots), seq_lens=dev(seq)))
    assert compare_tree(w, "greedy", oracle_tree(w, "greedy"), g) == 0
    offs = (np.arange(w.batch + 1) * w.n_nodes).astype(np.int32)
    _check(g, offs, w.n_nodes, slots, seq)
