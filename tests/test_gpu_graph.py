"""Verify + commit captured in a HIP graph (torch.cuda.CUDAGraph over the library's launches) and replayed
several times, with eager work (output poisoning and other library calls on other buffers) and host
synchronisation between replays. Every replay must reproduce the eager results exactly: the library
launches only kernels (no memset nodes, no allocation), and each call resets the workspace words it reads.
"""
import numpy as np
import pytest
import torch

import draft_verification_acceptance_amd as dva
from draft_verification_acceptance_amd import workloads as W
from gpu_util import dev, dev_logits

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A5A5A


def _chain_calls(w, mode, mask=None):
    kw = dict(max_verify_len=w.max_verify_len)
    if mode == "rejection":
        kw.update(draft_logits=dev_logits(w.draft), u_accept=dev(w.u_accept), u_final=dev(w.u_final),
                  temperature=w.temperature)
    elif mode == "rejection_sparse":
        kw.update(cand_ids=dev(w.cand_ids, torch.int32), cand_q=dev(w.cand_q), u_accept=dev(w.u_accept),
                  u_final=dev(w.u_final), temperature=w.temperature)
    elif mode == "sample_match":
        kw.update(u_accept=dev(w.u_accept), u_final=dev(w.u_final), temperature=w.temperature)
    if mask is not None:
        kw.update(vocab_mask=dev(np.ascontiguousarray(mask, np.uint32).view(np.int32)))
    offs = dev(w.offsets, torch.int32)
    v = dva.prepare_verify_chain(dev_logits(w.target), offs, dev(w.draft_tokens, torch.int32), mode, **kw)
    o = v.outputs
    c = dva.prepare_commit_indices(offs, o["accept_len"], o["accept_index"], dev(W.verify_slots_for(w.total_rows)),
                                   dev(W.seq_lens_for(w.batch)), max_verify_len=w.max_verify_len)
    return v, c


def _tree_calls(w, mode):
    kw = {}
    if mode == "target_only":
        kw = dict(u_accept=dev(w.u_accept), u_final=dev(w.u_final), temperature=w.temperature)
    v = dva.prepare_verify_tree(dev_logits(w.target), dev(w.parents, torch.int32), dev(w.tokens, torch.int32),
                                w.n_nodes, mode, **kw)
    o = v.outputs
    offs = dev((np.arange(w.batch + 1) * w.n_nodes).astype(np.int32))
    c = dva.prepare_commit_indices(offs, o["accept_len"], o["accept_index"], dev(W.verify_slots_for(w.total_rows)),
                                   dev(W.seq_lens_for(w.batch)), max_verify_len=w.n_nodes)
    return v, c


def _snapshot(v, c):
    torch.cuda.synchronize()
    return {**{"v." + k: t.clone() for k, t in v.outputs.items()}, **{"c." + k: t.clone() for k, t in c.outputs.items()}}


def _poison(v, c):
    for t in list(v.outputs.values()) + list(c.outputs.values()):
        if t.dtype == torch.float32:
            t.fill_(-12345.0)
        else:
            t.fill_(SENTINEL)


@pytest.mark.parametrize("case", ["chain_rejection", "block_greedy", "tree_target_only", "ragged", "block_sample",
                                  "chain_sparse", "chain_masked"])
def test_graph_replays_match_eager(case):
    print("graph replay", case, flush=True)
    if case == "chain_rejection":
        v, c = _chain_calls(W.chain_rejection(seed=2011, vocab=20011, parallel=False), "rejection")
    elif case == "block_greedy":
        v, c = _chain_calls(W.block_greedy(seed=3011, vocab=20011, parallel=False), "greedy")
    elif case == "tree_target_only":
        v, c = _tree_calls(W.tree(seed=4011, vocab=12007, parallel=False), "target_only")
    elif case == "ragged":
        v, c = _chain_calls(W.ragged(seed=5011, batch=96, vocab=4099, parallel=False), "rejection")
    elif case == "block_sample":
        v, c = _chain_calls(W.block_sample(seed=7011, vocab=20008, parallel=False), "sample_match")
    elif case == "chain_sparse":
        v, c = _chain_calls(W.chain_sparse(seed=6011, vocab=20011, parallel=False), "rejection_sparse")
    else:
        w = W.chain_rejection(seed=2013, vocab=20011, parallel=False)
        keep = [int(np.argmax(w.target[i])) for i in range(w.total_rows)]
        v, c = _chain_calls(w, "rejection", W.vocab_masks(13, w.total_rows, w.vocab, 0.3, keep))
    # other eager work on other buffers between replays: a different workload through the same library
    ov, oc = _chain_calls(W.chain_rejection(seed=2012, vocab=3001, parallel=False), "rejection")

    _poison(v, c)         # capacity past the committed entries keeps the sentinel in every run
    v.run()
    c.run()
    ref = _snapshot(v, c)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        v.run()
        c.run()
    for rep in range(4):
        _poison(v, c)
        ov.run()
        oc.run()
        torch.cuda.synchronize()
        g.replay()
        got = _snapshot(v, c)
        for k, t in ref.items():
            assert torch.equal(got[k], t), (case, rep, k)
