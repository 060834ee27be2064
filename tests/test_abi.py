"""CPU checks of the C ABI library: it loads, exports every symbol include/specverify.h declares, its
argument structs match the binding, and host-side argument checks return the documented codes before any
device work (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

import draft_verification_acceptance_amd as dva

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dva.library_path), reason="libspecverify.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"spec_verify_chain", "spec_verify_tree", "spec_commit_indices", "spec_workspace_bytes",
            "spec_status_string", "spec_abi_version"} <= set(names)
    lib = ctypes.CDLL(dva.library_path)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_struct_sizes():
    lib = dva._lib()        # raises on ABI or struct-size mismatch
    assert dva.abi_version() == 8
    assert lib.spec_args_size(0) == ctypes.sizeof(dva.ChainArgs) == 208
    assert lib.spec_args_size(1) == ctypes.sizeof(dva.TreeArgs)
    assert lib.spec_args_size(2) == ctypes.sizeof(dva.CommitArgs)


def test_status_strings_and_kernel_counts():
    for code, word in [(0, "SPEC_OK"), (1, "EINVAL"), (2, "EDTYPE"), (3, "EUNSUPPORTED"), (4, "EWORKSPACE"),
                       (5, "ELAUNCH"), (6, "ESCRATCH")]:
        assert word in dva.status_string(code)
    assert "unknown" in dva.status_string(99)
    assert dva.kernel_count("chain", "greedy") == 2
    assert dva.kernel_count("chain", "rejection") == 2
    assert dva.kernel_count("chain", "rejection_sparse") == 2
    assert dva.kernel_count("chain", "sample_match") == 2
    assert dva.kernel_count("tree", "target_only") == 2
    assert dva.kernel_count("commit", "greedy") == 1


def test_workspace_bytes():
    b = dva.workspace_bytes("chain", "rejection", 512, 151936, 64, 8)
    assert b > 0 and b % 256 == 0
    assert dva.workspace_bytes("chain", "greedy", 512, 151936, 32, 16) > 0
    # sparse q streams no draft rows: never more partials than dense rejection
    assert 0 < dva.workspace_bytes("chain", "rejection_sparse", 512, 151936, 64, 8) <= b
    assert dva.workspace_bytes("tree", "target_only", 2048, 128256, 32, 64) > 0
    assert dva.workspace_bytes("chain", "greedy", 10, 0, 2, 5) == 0           # vocab < 1
    assert dva.workspace_bytes("chain", "greedy", 10, 1 << 23, 2, 5) == 0     # vocab too large
    assert dva.workspace_bytes("chain", "greedy", 10, 100, 2, 2000) == 0      # rows per request too large
    assert dva.workspace_bytes("tree", "greedy", 10, 100, 3, 0) == 0          # rows not a multiple of batch


def _chain(**kw):
    a = dva.ChainArgs()
    a.total_rows, a.vocab, a.batch, a.max_verify_len = 10, 100, 2, 8
    a.dtype, a.mode, a.temperature = 1, 0, 1.0
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _call_chain(a):
    return dva._lib().spec_verify_chain(ctypes.byref(a), None)


def test_chain_host_checks():
    lib = dva._lib()
    assert lib.spec_verify_chain(None, None) == 1
    assert _call_chain(_chain(dtype=7)) == 2                                  # EDTYPE
    assert _call_chain(_chain(mode=2)) == 3                                   # target-only on a chain
    assert _call_chain(_chain(mode=9)) == 1
    assert _call_chain(_chain(vocab=0)) == 1
    assert _call_chain(_chain(max_verify_len=0)) == 1
    assert _call_chain(_chain(total_rows=1)) == 1                             # fewer rows than requests
    assert _call_chain(_chain()) == 1                                         # null pointers
    assert _call_chain(_chain(batch=0, total_rows=0)) == 0                    # empty batch: nothing to do
    fake = 1 << 40                                                            # never dereferenced
    full = dict(target_logits=fake, target_offsets=fake, draft_tokens=fake, accept_len=fake, bonus=fake,
                out_tokens=fake, accept_index=fake, status=fake)
    assert _call_chain(_chain(**full)) == 4                                   # no workspace
    assert _call_chain(_chain(**full, workspace=fake, workspace_bytes=16)) == 4
    rej = dict(full, mode=1, draft_logits=fake, u_accept=fake, u_final=fake)
    assert _call_chain(_chain(**rej, temperature=0.0)) == 1                   # T must be > 0
    assert _call_chain(_chain(**rej, temperature=float("inf"))) == 1
    assert _call_chain(_chain(**dict(rej, u_final=None))) == 1
    assert _call_chain(_chain(**full, n_profile_events=2)) == 1               # events array missing
    sp = dict(full, mode=3, u_accept=fake, u_final=fake, cand_ids=fake, cand_q=fake)
    assert _call_chain(_chain(**sp, n_cand=0)) == 1                           # K in 1..1024
    assert _call_chain(_chain(**sp, n_cand=1025)) == 1
    assert _call_chain(_chain(**dict(sp, cand_q=None), n_cand=4)) == 1
    assert _call_chain(_chain(**sp, n_cand=4)) == 4                           # args fine, no workspace
    sm = dict(full, mode=4, u_accept=fake, u_final=fake)                       # sample-then-match
    assert _call_chain(_chain(**sm, temperature=0.0)) == 1
    assert _call_chain(_chain(**dict(sm, u_accept=None))) == 1
    assert _call_chain(_chain(**sm)) == 4                                     # args fine, no workspace
    assert _call_chain(_chain(**sm, vocab_mask=fake)) == 4                    # a mask changes no check
    assert dva.workspace_bytes("chain", "sample_match", 10, 100, 2, 5) > 0


def test_fused_commit_host_checks():
    """A verify call given commit arguments checks them as spec_commit_indices does, before any launch."""
    lib = dva._lib()
    fake = 1 << 40
    full = dict(target_logits=fake, target_offsets=fake, draft_tokens=fake, accept_len=fake, bonus=fake,
                out_tokens=fake, accept_index=fake, status=fake, workspace=fake, workspace_bytes=1 << 30)
    good = dict(verify_slots=fake, seq_lens=fake, commit_offsets=fake, src_slots=fake, dst_pos=fake,
                new_seq_lens=fake, status=fake, capacity=10)
    for bad in (dict(verify_slots=None), dict(seq_lens=None), dict(src_slots=None), dict(status=None),
                dict(capacity=9), dict(evict_slots=fake)):
        c = dva.CommitArgs(**dict(good, **bad))
        a = _chain(**full)
        a.commit = ctypes.addressof(c)
        assert lib.spec_verify_chain(ctypes.byref(a), None) == 1, bad
        t = dva.TreeArgs()
        t.vocab, t.batch, t.n_nodes, t.dtype, t.mode = 100, 2, 5, 1, 0
        for k in ("target_logits", "parents", "tokens", "accept_len", "bonus", "out_tokens", "accept_index", "status",
                  "workspace"):
            setattr(t, k, fake)
        t.workspace_bytes = 1 << 30
        t.commit = ctypes.addressof(c)
        assert lib.spec_verify_tree(ctypes.byref(t), None) == 1, bad


def test_noalloc_host_checks():
    """spec_verify_chain_noalloc checks the same arguments, ignores the workspace fields, and refuses a call whose
    workspace would not fit its static scratch with SPEC_ESCRATCH before touching any GPU."""
    lib = dva._lib()
    call = lambda a: lib.spec_verify_chain_noalloc(ctypes.byref(a), None)  # noqa: E731
    assert lib.spec_verify_chain_noalloc(None, None) == 1
    assert call(_chain(dtype=7)) == 2
    assert call(_chain(mode=2)) == 3
    assert call(_chain()) == 1                                                # null pointers
    assert call(_chain(batch=0, total_rows=0)) == 0
    fake = 1 << 40
    full = dict(target_logits=fake, target_offsets=fake, draft_tokens=fake, accept_len=fake, bonus=fake,
                out_tokens=fake, accept_index=fake, status=fake, mode=1, draft_logits=fake, u_accept=fake,
                u_final=fake)
    # 8192 requests x 16 rows at V 151936: more than SPEC_NOALLOC_SCRATCH_BYTES of workspace
    big = dict(total_rows=8192 * 16, vocab=151936, batch=8192, max_verify_len=16)
    need = dva.workspace_bytes("chain", "rejection", big["total_rows"], big["vocab"], big["batch"], 16)
    assert need > dva.NOALLOC_SCRATCH_BYTES
    assert call(_chain(**full, **big)) == 6                                   # ESCRATCH
    assert call(_chain(**full, **big, workspace=fake, workspace_bytes=1 << 40)) == 6   # workspace ignored
    # the chain rejection workload (B 64, m 7, V 151936) and the ragged one (B 512, up to 16 rows) fit
    assert dva.workspace_bytes("chain", "rejection", 512, 151936, 64, 8) <= dva.NOALLOC_SCRATCH_BYTES
    assert dva.workspace_bytes("chain", "rejection", 8192, 151936, 512, 16) <= dva.NOALLOC_SCRATCH_BYTES


def test_tree_and_commit_host_checks():
    lib = dva._lib()
    a = dva.TreeArgs()
    a.vocab, a.batch, a.n_nodes, a.dtype, a.mode, a.temperature = 100, 2, 4, 1, 1, 1.0
    assert lib.spec_verify_tree(ctypes.byref(a), None) == 3                   # rejection on a tree
    a.mode = 3
    assert lib.spec_verify_tree(ctypes.byref(a), None) == 3                   # sparse rejection on a tree
    a.mode = 4
    assert lib.spec_verify_tree(ctypes.byref(a), None) == 3                   # sample-then-match on a tree
    a.mode = 2
    a.threshold_single, a.threshold_acc = 0.9, 1.0
    assert lib.spec_verify_tree(ctypes.byref(a), None) == 3                   # thresholds other than 1.0
    a.threshold_single = 1.0
    a.n_nodes = 0
    assert lib.spec_verify_tree(ctypes.byref(a), None) == 1
    a.n_nodes = 4
    assert lib.spec_verify_tree(ctypes.byref(a), None) == 1                   # null pointers
    c = dva.CommitArgs()
    c.batch, c.total_rows, c.capacity, c.max_verify_len = 2, 10, 5, 8
    assert lib.spec_commit_indices(ctypes.byref(c), None) == 1                # capacity < total_rows
    c.capacity = 10
    assert lib.spec_commit_indices(ctypes.byref(c), None) == 1                # null pointers


def test_plan_and_cap_trim_argument_checks():
    lib = dva._lib()
    assert lib.spec_args_size(3) == ctypes.sizeof(dva.PlanArgs)
    assert lib.spec_args_size(4) == ctypes.sizeof(dva.CapTrimArgs)
    assert dva.kernel_count("plan", "topk") == 1 and dva.kernel_count("cap_trim", "greedy") == 1
    fake = 1 << 40                                                            # never dereferenced

    def plan(**kw):
        a = dva.PlanArgs()
        base = dict(confidence=fake, selected=fake, verify_lens=fake, offsets=fake, batch=4, width=7, mode=0,
                    budget=3, min_verify_len=1, max_verify_len=8, survival_eps=0.0, threshold=0.5)
        base.update(kw)
        for k, v in base.items():
            setattr(a, k, v)
        return lib.spec_plan_layout(ctypes.byref(a), None)
    assert plan(mode=2) == 1                                                  # unknown mode
    assert plan(max_verify_len=9) == 1                                        # more rows than anchor + drafts
    assert plan(min_verify_len=0) == 1
    assert plan(min_verify_len=5, max_verify_len=4) == 1
    assert plan(width=4096) == 1
    assert plan(batch=1 << 20) == 1
    assert plan(offsets=None) == 1
    assert plan(confidence=None) == 1
    assert plan(survival_eps=-1.0) == 1
    assert plan(n_profile_events=2) == 1                                      # events array missing

    def trim(**kw):
        a = dva.CapTrimArgs()
        base = dict(row_offsets=fake, verify_lens=fake, raw_accept_len=fake, raw_bonus=fake, out_tokens=fake,
                    correct_len=fake, cap_trim_lens=fake, commit_lens=fake, block_accept_lens=fake, bonus=fake,
                    status=fake, total_rows=16, batch=2)
        base.update(kw)
        for k, v in base.items():
            setattr(a, k, v)
        return lib.spec_cap_trim(ctypes.byref(a), None)
    assert trim(out_tokens=None) == 1
    assert trim(batch=-1) == 1
    assert trim(total_rows=-1) == 1


def test_plan_budget_host_argument_checks():
    import numpy as np
    c = np.full((2, 3), 0.5, np.float32)
    with pytest.raises(dva.SpecError):
        dva.plan_budget(c, [1.0, 1.0], [5.0, 4.0])                           # rows must increase
    with pytest.raises(dva.SpecError):
        dva.plan_budget(c, [1.0, 2.0], [5.0, float("nan")])
    with pytest.raises(dva.SpecError):
        dva.plan_budget(c, [1.0, 2.0], [5.0, 4.0], survival_eps=-0.5)
    K0, th0 = dva.plan_budget(np.zeros((0, 3), np.float32), [1.0], [5.0])
    assert K0 == 0 and th0.dtype == np.float64 and list(th0) == [0.0]


def test_read_probe_host_checks():
    lib = dva._lib()
    fake = 1 << 40                                                            # never dereferenced
    assert lib.spec_read_probe(fake, 0, fake, None, None) == 0                # nothing to read
    assert lib.spec_read_probe(None, 64, fake, None, None) == 1
    assert lib.spec_read_probe(fake, 64, None, None, None) == 1
    assert lib.spec_read_probe(fake + 4, 64, fake, None, None) == 1           # src not 16-byte aligned
    assert lib.spec_read_probe(fake, 60, fake, None, None) == 1               # not whole 16-byte words
