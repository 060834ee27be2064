"""spec_verify_chain_noalloc (the verify entry point whose workspace is the library's static per-GPU scratch)
against spec_verify_chain (caller workspace) through the C ABI: identical outputs, on calls in a row whose
second is smaller than the first, so whatever the first left in the scratch must not matter."""
import numpy as np
import pytest
import torch

import draft_verification_acceptance_amd as dva
from draft_verification_acceptance_amd import workloads as W
from gpu_util import dev, dev_logits, np_out

pytestmark = pytest.mark.gpu

OUTS = ("accept_len", "bonus", "out_tokens", "accept_index", "status", "accept_prob", "residual_mass")


def _call(w, mode, noalloc):
    kw = dict(max_verify_len=w.max_verify_len, noalloc=noalloc)
    if mode in ("rejection", "rejection_sparse", "sample_match"):
        kw.update(u_accept=dev(w.u_accept), u_final=dev(w.u_final), temperature=w.temperature)
    if mode == "rejection":
        kw.update(draft_logits=dev_logits(w.draft))
    if mode == "rejection_sparse":
        kw.update(cand_ids=dev(w.cand_ids, torch.int32), cand_q=dev(w.cand_q, torch.float32))
    T, B = w.total_rows, w.batch
    D = T - B
    # outputs poisoned first: every entry must be written by the call
    out = {k: torch.full((n,), -7, dtype=dt, device="cuda") for k, n, dt in
           (("accept_len", B, torch.int32), ("bonus", B, torch.int32), ("out_tokens", T, torch.int32),
            ("accept_index", T, torch.int32), ("status", B, torch.int32))}
    out["accept_prob"] = torch.full((D,), float("nan"), dtype=torch.float32, device="cuda")
    out["residual_mass"] = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
    o = dva.verify_chain(dev_logits(w.target), dev(w.offsets, torch.int32), dev(w.draft_tokens, torch.int32), mode,
                         out=out, **kw)
    return np_out(o)


def _same(a, b, name):
    for k in OUTS:
        assert np.array_equal(a[k], b[k], equal_nan=True), (name, k)


def _pair(w, mode, name):
    print("noalloc", name, mode, w.total_rows, w.vocab, flush=True)
    g0 = _call(w, mode, noalloc=True)
    g1 = _call(w, mode, noalloc=False)
    _same(g0, g1, name)
    assert not np.isnan(g0["accept_prob"]).any() and (g0["accept_len"] >= 0).all()
    return g0


@pytest.mark.parametrize("mode", ["rejection", "greedy", "sample_match", "rejection_sparse"])
def test_noalloc_matches_workspace_entry_point(mode):
    if mode == "rejection_sparse":
        big, small = W.chain_sparse(), W.chain_sparse(seed=6011, vocab=5003, batch=9)
    elif mode == "sample_match":
        big, small = W.block_sample(), W.block_sample(seed=7011, vocab=4096, batch=5)
    else:
        big, small = W.chain_rejection(), W.chain_rejection(seed=2011, batch=7, m=3, vocab=3001, parallel=False)
    _pair(big, mode, "full")
    _pair(small, mode, "smaller")      # the second call in a row, smaller than the first
    _pair(big, mode, "full again")


def test_noalloc_largest_workload_then_tiny():
    """The ragged workload (B 512, up to 16 rows, about 1.9 MB of workspace: the largest shape measured here)
    then the tiny one, in a row."""
    _pair(W.ragged(), "rejection", "ragged")
    t = W.tiny_chain()
    for mode in ("rejection", "greedy"):
        _pair(t, mode, "tiny")


def test_noalloc_refuses_calls_beyond_its_scratch():
    """A call whose workspace would exceed the scratch is refused on the host before any launch (the pointers
    below are never dereferenced)."""
    import ctypes
    B = 8192
    T = B * 16
    assert dva.workspace_bytes("chain", "rejection", T, 151936, B, 16) > dva.NOALLOC_SCRATCH_BYTES
    a = dva.ChainArgs()
    fake = 1 << 40
    for k in ("target_logits", "target_offsets", "draft_tokens", "accept_len", "bonus", "out_tokens",
              "accept_index", "status", "draft_logits", "u_accept", "u_final"):
        setattr(a, k, fake)
    a.total_rows, a.vocab, a.batch, a.max_verify_len, a.dtype, a.mode, a.temperature = T, 151936, B, 16, 1, 1, 1.0
    with pytest.raises(dva.SpecError) as e:
        dva._check(dva._lib().spec_verify_chain_noalloc(ctypes.byref(a), None))
    assert e.value.code == 6 and "SCRATCH" in str(e.value)
