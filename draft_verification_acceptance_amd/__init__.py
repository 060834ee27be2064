"""Speculative-decoding verify / accept / commit on MI355X (gfx950).

Thin ctypes binding of libspecverify.so (the C ABI declared in include/specverify.h). Every step of the
verify path runs in the library's HIP kernels; this module only checks and marshals torch tensors (device
memory) and passes the current torch stream. There is no CPU fallback: without the built library every
entry point raises.

    verify_chain(...)    greedy or rejection-sampling verify of ragged chains (spec_verify_chain)
    verify_tree(...)     greedy or target-only verify of draft trees (spec_verify_tree)
    commit_indices(...)  KV commit compaction of a verify round (spec_commit_indices)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "SpecError", "verify_chain", "verify_tree", "commit_indices", "workspace", "workspace_bytes", "read_probe",
    "workspace_init", "kernel_count", "status_string", "abi_version", "library_path", "HipEvents",
    "MODES", "ST", "PreparedCall", "prepare_verify_chain", "prepare_verify_tree", "prepare_commit_indices",
    "plan_layout", "prepare_plan_layout", "plan_budget", "plan_budget_cost", "cap_trim", "prepare_cap_trim", "kv_move",
    "prepare_kv_move", "tree_build", "prepare_tree_build",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
# SPECVERIFY_LIBRARY: another build of the same library (the host-sanitizer build of build.py --sanitize)
library_path = os.environ.get("SPECVERIFY_LIBRARY") or os.path.join(_PKG, "libspecverify.so")

ABI_VERSION = 8
MODES = {"greedy": 0, "rejection": 1, "target_only": 2, "rejection_sparse": 3, "sample_match": 4}
KIND_CHAIN, KIND_TREE, KIND_COMMIT, KIND_PLAN, KIND_CAP_TRIM, KIND_KV_MOVE, KIND_TREE_BUILD = 0, 1, 2, 3, 4, 5, 6
PLAN_MODES = {"topk": 0, "threshold": 1}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}


class ST:
    """Per-request status bits (SPEC_ST_*)."""
    NONFINITE = 1 << 0
    BAD_TOKEN = 1 << 1
    BAD_OFFSETS = 1 << 2
    BAD_PARENT = 1 << 3
    BAD_UNIFORM = 1 << 4
    ZERO_Q = 1 << 5
    ZERO_RESIDUAL = 1 << 6
    NEAR_ALPHA = 1 << 7
    NEAR_CDF = 1 << 8
    BAD_ACCEPT = 1 << 9
    BAD_Q = 1 << 10
    BAD_CONF = 1 << 11
    BAD_SLOT = 1 << 12


class SpecError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{message} (code {code})")
        self.code = code


_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class ChainArgs(ctypes.Structure):
    _fields_ = [("target_logits", _vp), ("target_offsets", _vp), ("draft_logits", _vp), ("draft_tokens", _vp),
                ("u_accept", _vp), ("u_final", _vp), ("accept_len", _vp), ("bonus", _vp), ("out_tokens", _vp),
                ("accept_index", _vp), ("status", _vp), ("accept_prob", _vp), ("residual_mass", _vp),
                ("workspace", _vp), ("workspace_bytes", _sz), ("profile_events", _vp), ("total_rows", _i64),
                ("vocab", _i64), ("batch", _i32), ("max_verify_len", _i32), ("dtype", _i32), ("mode", _i32),
                ("temperature", _f32), ("n_profile_events", _i32), ("cand_ids", _vp), ("cand_q", _vp),
                ("n_cand", _i32), ("reserved", _i32), ("vocab_mask", _vp), ("commit", _vp)]


class TreeArgs(ctypes.Structure):
    _fields_ = [("target_logits", _vp), ("parents", _vp), ("tokens", _vp), ("u_accept", _vp), ("u_final", _vp),
                ("accept_len", _vp), ("bonus", _vp), ("out_tokens", _vp), ("accept_index", _vp), ("status", _vp),
                ("accept_prob", _vp), ("residual_mass", _vp), ("workspace", _vp), ("workspace_bytes", _sz),
                ("profile_events", _vp), ("vocab", _i64), ("batch", _i32), ("n_nodes", _i32), ("dtype", _i32),
                ("mode", _i32), ("temperature", _f32), ("threshold_single", _f32), ("threshold_acc", _f32),
                ("n_profile_events", _i32), ("vocab_mask", _vp), ("commit", _vp)]


class CommitArgs(ctypes.Structure):
    _fields_ = [("row_offsets", _vp), ("accept_len", _vp), ("accept_index", _vp), ("verify_slots", _vp),
                ("seq_lens", _vp), ("commit_offsets", _vp), ("src_slots", _vp), ("dst_pos", _vp),
                ("new_seq_lens", _vp), ("status", _vp), ("evict_slots", _vp), ("evict_offsets", _vp),
                ("profile_events", _vp), ("total_rows", _i64), ("capacity", _i64), ("batch", _i32),
                ("max_verify_len", _i32), ("n_profile_events", _i32), ("reserved", _i32)]


class PlanArgs(ctypes.Structure):
    _fields_ = [("confidence", _vp), ("selected", _vp), ("verify_lens", _vp), ("offsets", _vp), ("row_index", _vp),
                ("status", _vp), ("profile_events", _vp), ("batch", _i32), ("width", _i32), ("mode", _i32),
                ("budget", _i32), ("min_verify_len", _i32), ("max_verify_len", _i32), ("survival_eps", _f32),
                ("threshold", _f32), ("n_profile_events", _i32), ("reserved", _i32)]


class CapTrimArgs(ctypes.Structure):
    _fields_ = [("row_offsets", _vp), ("verify_lens", _vp), ("raw_accept_len", _vp), ("raw_bonus", _vp),
                ("out_tokens", _vp), ("correct_len", _vp), ("cap_trim_lens", _vp), ("commit_lens", _vp),
                ("block_accept_lens", _vp), ("bonus", _vp), ("status", _vp), ("profile_events", _vp),
                ("total_rows", _i64), ("batch", _i32), ("n_profile_events", _i32)]


class KvMoveArgs(ctypes.Structure):
    _fields_ = [("buffers", _vp), ("commit_offsets", _vp), ("src_slots", _vp), ("dst_pos", _vp),
                ("req_to_token", _vp), ("req_pool_indices", _vp), ("status", _vp), ("profile_events", _vp),
                ("n_slots", _i64), ("max_context", _i64), ("n_req_rows", _i64), ("capacity", _i64),
                ("row_bytes", _i32), ("n_buffers", _i32), ("batch", _i32), ("n_profile_events", _i32)]


class TreeBuildArgs(ctypes.Structure):
    _fields_ = [("anchors", _vp), ("draft_tokens", _vp), ("draft_probs", _vp), ("seq_lens", _vp), ("tokens", _vp),
                ("parents", _vp), ("positions", _vp), ("mask", _vp), ("first_child", _vp), ("next_sibling", _vp),
                ("cand_index", _vp), ("status", _vp), ("profile_events", _vp), ("batch", _i32), ("n_steps", _i32),
                ("topk", _i32), ("n_nodes", _i32), ("n_profile_events", _i32), ("reserved", _i32)]


_LIB = None


def _lib():
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(library_path):
        raise RuntimeError(f"{library_path} is not built; run `python -m draft_verification_acceptance_amd.build`")
    lib = ctypes.CDLL(library_path)
    lib.spec_verify_chain.argtypes = [ctypes.POINTER(ChainArgs), _vp]
    lib.spec_verify_chain_noalloc.argtypes = [ctypes.POINTER(ChainArgs), _vp]
    lib.spec_verify_tree.argtypes = [ctypes.POINTER(TreeArgs), _vp]
    lib.spec_commit_indices.argtypes = [ctypes.POINTER(CommitArgs), _vp]
    lib.spec_plan_layout.argtypes = [ctypes.POINTER(PlanArgs), _vp]
    lib.spec_cap_trim.argtypes = [ctypes.POINTER(CapTrimArgs), _vp]
    lib.spec_kv_move.argtypes = [ctypes.POINTER(KvMoveArgs), _vp]
    lib.spec_tree_build.argtypes = [ctypes.POINTER(TreeBuildArgs), _vp]
    for f in (lib.spec_verify_chain, lib.spec_verify_chain_noalloc, lib.spec_verify_tree, lib.spec_commit_indices, lib.spec_plan_layout,
              lib.spec_cap_trim, lib.spec_kv_move, lib.spec_tree_build):
        f.restype = ctypes.c_int
    import numpy as np
    _f32a = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
    _f64a = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
    lib.spec_plan_budget.argtypes = [_f32a, _i32, _i32, _f64a, _f64a, _i32, _f32, ctypes.POINTER(_i32), _f64a,
                                     ctypes.POINTER(_i32)]
    lib.spec_plan_budget.restype = ctypes.c_int
    lib.spec_plan_budget_cost.argtypes = [_f32a, _i32, _i32, _f64a, _f64a, _i32, _f64a, _f64a, _i32, _f32,
                                          ctypes.POINTER(_i32), _f64a, ctypes.POINTER(_i32)]
    lib.spec_plan_budget_cost.restype = ctypes.c_int
    lib.spec_workspace_bytes.argtypes = [_i32, _i32, _i64, _i64, _i32, _i32]
    lib.spec_workspace_bytes.restype = _sz
    lib.spec_workspace_init.argtypes = [_vp, _sz, _vp]
    lib.spec_workspace_init.restype = ctypes.c_int
    lib.spec_read_probe.argtypes = [_vp, _sz, _vp, _vp, _vp]
    lib.spec_read_probe.restype = ctypes.c_int
    lib.spec_kernel_count.argtypes = [_i32, _i32]
    lib.spec_kernel_count.restype = _i32
    lib.spec_status_string.argtypes = [ctypes.c_int]
    lib.spec_status_string.restype = ctypes.c_char_p
    lib.spec_abi_version.argtypes = []
    lib.spec_abi_version.restype = _i32
    lib.spec_args_size.argtypes = [_i32]
    lib.spec_args_size.restype = _sz
    if lib.spec_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libspecverify ABI {lib.spec_abi_version()} != binding ABI {ABI_VERSION}")
    for kind, st in ((KIND_CHAIN, ChainArgs), (KIND_TREE, TreeArgs), (KIND_COMMIT, CommitArgs), (KIND_PLAN, PlanArgs),
                     (KIND_CAP_TRIM, CapTrimArgs), (KIND_KV_MOVE, KvMoveArgs), (KIND_TREE_BUILD, TreeBuildArgs)):
        if lib.spec_args_size(kind) != ctypes.sizeof(st):
            raise RuntimeError(f"argument struct {st.__name__} size mismatch with the library")
    _LIB = lib
    return lib


def abi_version() -> int:
    return int(_lib().spec_abi_version())


def status_string(code: int) -> str:
    return _lib().spec_status_string(int(code)).decode()


def kernel_count(kind: str, mode: str) -> int:
    k = {"chain": KIND_CHAIN, "tree": KIND_TREE, "commit": KIND_COMMIT, "plan": KIND_PLAN,
         "cap_trim": KIND_CAP_TRIM, "kv_move": KIND_KV_MOVE, "tree_build": KIND_TREE_BUILD}[kind]
    return int(_lib().spec_kernel_count(k, MODES.get(mode, 0)))


def _check(code: int):
    if code != 0:
        raise SpecError(code, status_string(code))


def workspace_bytes(kind: str, mode: str, total_rows: int, vocab: int, batch: int, max_verify_len: int) -> int:
    k = {"chain": KIND_CHAIN, "tree": KIND_TREE}[kind]
    return int(_lib().spec_workspace_bytes(k, MODES[mode], int(total_rows), int(vocab), int(batch),
                                           int(max_verify_len)))


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def workspace_init(ws: torch.Tensor):
    _check(_lib().spec_workspace_init(ws.data_ptr(), ws.numel() * ws.element_size(), _stream(ws.device)))


READ_SINK_WORDS = 8192   # SPEC_READ_SINK_WORDS
NOALLOC_SCRATCH_BYTES = 4 << 20   # SPEC_NOALLOC_SCRATCH_BYTES


def read_probe(src: torch.Tensor, sink: torch.Tensor, nbytes: int | None = None, events: "HipEvents | None" = None):
    """spec_read_probe: a plain read of the first `nbytes` (default: all) bytes of `src` on the current stream.
    `sink`: an int32 device tensor of READ_SINK_WORDS words the caller zeroes; the XOR of its words is the XOR
    of every 32-bit word read. `events` (2 of them) take the kernel's start and stop timestamps."""
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if (sink.dtype != torch.int32 or sink.device != src.device or sink.numel() < READ_SINK_WORDS
            or n > src.numel() * src.element_size()):
        raise SpecError("read_probe: sink must be READ_SINK_WORDS int32 words on src's device, nbytes within src")
    _check(_lib().spec_read_probe(src.data_ptr(), n, sink.data_ptr(), events.pointer() if events else None,
                                  _stream(src.device)))


def workspace(kind: str, mode: str, total_rows: int, vocab: int, batch: int, max_verify_len: int,
              device="cuda") -> torch.Tensor:
    """A zero-filled workspace for calls up to this size (reusable by later calls on the same stream)."""
    n = workspace_bytes(kind, mode, total_rows, vocab, batch, max_verify_len)
    if n == 0:
        raise SpecError(1, "invalid workspace request")
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    workspace_init(ws)
    return ws


def _ptr(t):
    return None if t is None else t.data_ptr()


def _req(t: torch.Tensor, name: str, dtype, n=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if n is not None and t.numel() != n:
        raise ValueError(f"{name} must have {n} elements, got {t.numel()}")
    return t


class HipEvents:
    """Timing events created through the HIP runtime. Passed to a library call (2 per kernel), events 2k and
    2k+1 take the start and stop timestamps of the call's kernel k."""

    def __init__(self, n: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(_vp)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _vp, _vp]
        self._hip.hipEventSynchronize.argtypes = [_vp]
        self._hip.hipEventDestroy.argtypes = [_vp]
        self.arr = (_vp * n)()
        for i in range(n):
            h = _vp()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.arr[i] = h
        self.n = n

    def pointer(self):
        return ctypes.cast(self.arr, _vp)

    def elapsed_ms(self, i: int, j: int) -> float:
        self._hip.hipEventSynchronize(self.arr[j])
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[i], self.arr[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        try:
            for i in range(self.n):
                self._hip.hipEventDestroy(self.arr[i])
        except Exception:
            pass


def _outputs(out, device, batch, rows, draft_rows, want_prob, want_resid):
    if out is None:
        out = {}
    def get(name, n, dtype, fill=None):
        t = out.get(name)
        if t is None:
            t = torch.empty(n, dtype=dtype, device=device)
            out[name] = t
        return _req(t, name, dtype, n, device)
    get("accept_len", batch, torch.int32)
    get("bonus", batch, torch.int32)
    get("out_tokens", rows, torch.int32)
    get("accept_index", rows, torch.int32)
    get("status", batch, torch.int32)
    if want_prob:
        get("accept_prob", draft_rows, torch.float32)
    if want_resid:
        get("residual_mass", batch, torch.float32)
    return out


class PreparedCall:
    """A verify / commit call whose argument block is built once; run() launches it again on the current
    stream of its device (same tensors, same workspace). Keeps every tensor it points at alive."""

    def __init__(self, fn, args, outputs: dict, keep: list, device):
        self._fn = fn
        self._args = args
        self.outputs = outputs
        self._keep = keep
        self._device = device

    def run(self, events: "HipEvents | None" = None, stream: int | None = None) -> dict:
        a = self._args
        a.profile_events = events.pointer() if events is not None else None
        a.n_profile_events = events.n if events is not None else 0
        _check(self._fn(ctypes.byref(a), _stream(self._device) if stream is None else stream))
        return self.outputs


def _fused_commit(verify_slots, seq_lens, B: int, T: int, dev, evict: bool, o: dict, keep: list):
    """The CommitArgs of a fused commit (verify_slots int64 [T], seq_lens int32 [B]); its outputs are added to
    the verify outputs `o` as commit_offsets, src_slots, dst_pos, new_seq_lens, commit_status and (evict)
    evict_offsets, evict_slots. Returns the address of the struct, kept alive through `keep`."""
    _req(verify_slots, "verify_slots", torch.int64, T, dev)
    _req(seq_lens, "seq_lens", torch.int32, B, dev)

    def get(name, n, dtype):
        t = o.get(name)
        if t is None:
            t = torch.empty(n, dtype=dtype, device=dev)
            o[name] = t
        return _req(t, name, dtype, n, dev)
    get("commit_offsets", B + 1, torch.int32)
    get("src_slots", T, torch.int64)
    get("dst_pos", T, torch.int32)
    get("new_seq_lens", B, torch.int32)
    get("commit_status", B, torch.int32)
    if evict:
        get("evict_offsets", B + 1, torch.int32)
        get("evict_slots", T, torch.int64)
    c = CommitArgs()
    c.verify_slots, c.seq_lens = _ptr(verify_slots), _ptr(seq_lens)
    c.commit_offsets, c.src_slots, c.dst_pos = _ptr(o["commit_offsets"]), _ptr(o["src_slots"]), _ptr(o["dst_pos"])
    c.new_seq_lens, c.status = _ptr(o["new_seq_lens"]), _ptr(o["commit_status"])
    c.evict_slots = _ptr(o.get("evict_slots")) if evict else None
    c.evict_offsets = _ptr(o.get("evict_offsets")) if evict else None
    c.total_rows, c.capacity, c.batch = T, T, B
    keep += [verify_slots, seq_lens, c]
    return ctypes.addressof(c)


def prepare_verify_chain(target_logits: torch.Tensor, target_offsets: torch.Tensor, draft_tokens: torch.Tensor,
                         mode: str = "greedy", *, draft_logits: torch.Tensor | None = None,
                         u_accept: torch.Tensor | None = None, u_final: torch.Tensor | None = None,
                         temperature: float = 1.0, max_verify_len: int | None = None, workspace_tensor=None,
                         out: dict | None = None, accept_prob: bool = True, residual_mass: bool = True,
                         cand_ids: torch.Tensor | None = None, cand_q: torch.Tensor | None = None,
                         vocab_mask: torch.Tensor | None = None, noalloc: bool = False,
                         verify_slots: torch.Tensor | None = None, seq_lens: torch.Tensor | None = None,
                         commit_evict: bool = True) -> PreparedCall:
    """Checks and marshals the arguments of spec_verify_chain once (see verify_chain). noalloc: call
    spec_verify_chain_noalloc instead (the library's static per-GPU scratch serves as the workspace; no
    workspace tensor is made or passed). verify_slots / seq_lens: fuse the round's KV commit into the call
    (its outputs join the verify outputs, see _fused_commit)."""
    lib = _lib()
    dev = target_logits.device
    if target_logits.dim() != 2:
        raise ValueError("target_logits must be [rows, vocab]")
    if target_logits.dtype not in DTYPES:
        raise TypeError("target_logits must be bfloat16 or float32")
    _req(target_logits, "target_logits", target_logits.dtype, device=dev)
    T, V = target_logits.shape
    _req(target_offsets, "target_offsets", torch.int32, device=dev)
    B = target_offsets.numel() - 1
    D = T - B
    if max_verify_len is None:
        raise ValueError("max_verify_len (upper bound on m_b + 1) is required")
    _req(draft_tokens, "draft_tokens", torch.int32, D, dev)
    m = MODES[mode]
    K = 0
    if mode == "rejection":
        _req(draft_logits, "draft_logits", target_logits.dtype, D * V, dev)
    elif mode == "rejection_sparse":
        if cand_ids is None or cand_ids.dim() != 2 or cand_ids.shape[0] != D:
            raise ValueError("cand_ids must be [total_rows - batch, K]")
        K = int(cand_ids.shape[1])
        _req(cand_ids, "cand_ids", torch.int32, D * K, dev)
        _req(cand_q, "cand_q", torch.float32, D * K, dev)
    elif mode not in ("greedy", "sample_match"):
        raise SpecError(3, status_string(3))
    if vocab_mask is not None:
        _req(vocab_mask, "vocab_mask", torch.int32, T * ((V + 31) // 32), dev)
    if mode != "greedy":
        _req(u_accept, "u_accept", torch.float32, D, dev)
        _req(u_final, "u_final", torch.float32, B, dev)
    if noalloc:
        if workspace_tensor is not None:
            raise ValueError("noalloc calls take no workspace tensor")
    elif workspace_tensor is None:
        workspace_tensor = workspace("chain", mode, T, V, B, max_verify_len, dev)
    o = _outputs(out, dev, B, T, D, accept_prob, residual_mass)
    a = ChainArgs()
    a.target_logits = _ptr(target_logits)
    a.target_offsets = _ptr(target_offsets)
    a.draft_logits = _ptr(draft_logits)
    a.draft_tokens = _ptr(draft_tokens)
    a.u_accept = _ptr(u_accept)
    a.u_final = _ptr(u_final)
    a.accept_len, a.bonus = o["accept_len"].data_ptr(), o["bonus"].data_ptr()
    a.out_tokens, a.accept_index = o["out_tokens"].data_ptr(), o["accept_index"].data_ptr()
    a.status = o["status"].data_ptr()
    a.accept_prob = _ptr(o.get("accept_prob")) if accept_prob else None
    a.residual_mass = _ptr(o.get("residual_mass")) if residual_mass else None
    a.workspace = None if noalloc else workspace_tensor.data_ptr()
    a.workspace_bytes = 0 if noalloc else workspace_tensor.numel()
    a.total_rows, a.vocab, a.batch = T, V, B
    a.max_verify_len = int(max_verify_len)
    a.dtype = DTYPES[target_logits.dtype]
    a.mode = m
    a.temperature = float(temperature)
    a.cand_ids = _ptr(cand_ids) if K else None
    a.cand_q = _ptr(cand_q) if K else None
    a.n_cand = K
    a.vocab_mask = _ptr(vocab_mask)
    keep = [target_logits, target_offsets, draft_tokens, draft_logits, u_accept, u_final, cand_ids, cand_q,
            vocab_mask, workspace_tensor]
    if verify_slots is not None or seq_lens is not None:
        a.commit = _fused_commit(verify_slots, seq_lens, B, T, dev, commit_evict, o, keep)
    return PreparedCall(lib.spec_verify_chain_noalloc if noalloc else lib.spec_verify_chain, a, o, keep, dev)


def verify_chain(target_logits: torch.Tensor, target_offsets: torch.Tensor, draft_tokens: torch.Tensor,
                 mode: str = "greedy", *, events: "HipEvents | None" = None, **kw) -> dict:
    """spec_verify_chain on torch tensors (launched on the current stream; asynchronous).

    target_logits [T_rows, V] bf16/fp32; target_offsets int32 [B+1]; draft-side int32 tokens, float32
    uniforms and logits packed with m_b entries per request from off[b]-b; max_verify_len bounds m_b + 1.
    Keywords: draft_logits (rejection), cand_ids / cand_q ([T_rows - B, K] int32 / float32, rejection_sparse),
    u_accept, u_final, temperature, max_verify_len, workspace_tensor, out, accept_prob, residual_mass,
    vocab_mask (int32 [T_rows, ceil(V/32)] allowed-token bits of the target rows, bit v % 32 of word v // 32),
    noalloc (spec_verify_chain_noalloc: no workspace; calls needing more than NOALLOC_SCRATCH_BYTES raise),
    verify_slots (int64 [T_rows]) and seq_lens (int32 [B]) to fuse the KV commit of the round into the call
    (outputs commit_offsets, src_slots, dst_pos, new_seq_lens, commit_status, evict_offsets, evict_slots as
    commit_indices gives them; commit_evict=False drops the evict lists).
    Modes: greedy, rejection, rejection_sparse, sample_match. Returns the output tensors (accept_len, bonus,
    out_tokens, accept_index, status, accept_prob, residual_mass)."""
    return prepare_verify_chain(target_logits, target_offsets, draft_tokens, mode, **kw).run(events)


def prepare_verify_tree(target_logits: torch.Tensor, parents: torch.Tensor, tokens: torch.Tensor, n_nodes: int,
                        mode: str = "greedy", *, u_accept=None, u_final=None, temperature: float = 1.0,
                        threshold_single: float = 1.0, threshold_acc: float = 1.0, workspace_tensor=None,
                        out: dict | None = None, accept_prob: bool = True, residual_mass: bool = True,
                        vocab_mask: torch.Tensor | None = None, verify_slots: torch.Tensor | None = None,
                        seq_lens: torch.Tensor | None = None, commit_evict: bool = True) -> PreparedCall:
    """Checks and marshals the arguments of spec_verify_tree once (see verify_tree; verify_slots / seq_lens:
    fused KV commit as for prepare_verify_chain)."""
    lib = _lib()
    dev = target_logits.device
    if target_logits.dim() != 2 or target_logits.dtype not in DTYPES:
        raise ValueError("target_logits must be a 2-D bfloat16 / float32 tensor")
    _req(target_logits, "target_logits", target_logits.dtype, device=dev)
    rows, V = target_logits.shape
    N = int(n_nodes)
    if N < 1 or rows % N:
        raise ValueError("rows must be a multiple of n_nodes")
    B = rows // N
    _req(parents, "parents", torch.int32, rows, dev)
    _req(tokens, "tokens", torch.int32, rows, dev)
    if mode == "target_only":
        _req(u_accept, "u_accept", torch.float32, rows, dev)
        _req(u_final, "u_final", torch.float32, B, dev)
    elif mode != "greedy":
        raise SpecError(3, status_string(3))
    if vocab_mask is not None:
        _req(vocab_mask, "vocab_mask", torch.int32, rows * ((V + 31) // 32), dev)
    if workspace_tensor is None:
        workspace_tensor = workspace("tree", mode, rows, V, B, N, dev)
    o = _outputs(out, dev, B, rows, rows, accept_prob, residual_mass)
    a = TreeArgs()
    a.target_logits, a.parents, a.tokens = _ptr(target_logits), _ptr(parents), _ptr(tokens)
    a.u_accept, a.u_final = _ptr(u_accept), _ptr(u_final)
    a.accept_len, a.bonus = o["accept_len"].data_ptr(), o["bonus"].data_ptr()
    a.out_tokens, a.accept_index = o["out_tokens"].data_ptr(), o["accept_index"].data_ptr()
    a.status = o["status"].data_ptr()
    a.accept_prob = _ptr(o.get("accept_prob")) if accept_prob else None
    a.residual_mass = _ptr(o.get("residual_mass")) if residual_mass else None
    a.workspace = workspace_tensor.data_ptr()
    a.workspace_bytes = workspace_tensor.numel()
    a.vocab, a.batch, a.n_nodes = V, B, N
    a.dtype = DTYPES[target_logits.dtype]
    a.mode = MODES[mode]
    a.temperature = float(temperature)
    a.threshold_single, a.threshold_acc = float(threshold_single), float(threshold_acc)
    a.vocab_mask = _ptr(vocab_mask)
    keep = [target_logits, parents, tokens, u_accept, u_final, vocab_mask, workspace_tensor]
    if verify_slots is not None or seq_lens is not None:
        a.commit = _fused_commit(verify_slots, seq_lens, B, rows, dev, commit_evict, o, keep)
    return PreparedCall(lib.spec_verify_tree, a, o, keep, dev)


def verify_tree(target_logits: torch.Tensor, parents: torch.Tensor, tokens: torch.Tensor, n_nodes: int,
                mode: str = "greedy", *, events: "HipEvents | None" = None, **kw) -> dict:
    """spec_verify_tree on torch tensors: target_logits [B*N, V]; parents, tokens int32 [B*N]. Keywords:
    u_accept, u_final, temperature, threshold_single, threshold_acc, workspace_tensor, out, accept_prob,
    residual_mass, vocab_mask (int32 [B*N, ceil(V/32)], as for verify_chain)."""
    return prepare_verify_tree(target_logits, parents, tokens, n_nodes, mode, **kw).run(events)


def prepare_commit_indices(row_offsets: torch.Tensor, accept_len: torch.Tensor, accept_index: torch.Tensor,
                           verify_slots: torch.Tensor, seq_lens: torch.Tensor, *, max_verify_len: int,
                           evict: bool = True, out: dict | None = None) -> PreparedCall:
    """Checks and marshals the arguments of spec_commit_indices once (see commit_indices)."""
    lib = _lib()
    dev = row_offsets.device
    _req(row_offsets, "row_offsets", torch.int32, device=dev)
    B = row_offsets.numel() - 1
    _req(accept_len, "accept_len", torch.int32, B, dev)
    T = accept_index.numel()
    _req(accept_index, "accept_index", torch.int32, T, dev)
    _req(verify_slots, "verify_slots", torch.int64, T, dev)
    _req(seq_lens, "seq_lens", torch.int32, B, dev)
    o = {} if out is None else out

    def get(name, n, dtype):
        t = o.get(name)
        if t is None:
            t = torch.empty(n, dtype=dtype, device=dev)
            o[name] = t
        return _req(t, name, dtype, n, dev)
    get("commit_offsets", B + 1, torch.int32)
    get("src_slots", T, torch.int64)
    get("dst_pos", T, torch.int32)
    get("new_seq_lens", B, torch.int32)
    get("status", B, torch.int32)
    if evict:
        get("evict_offsets", B + 1, torch.int32)
        get("evict_slots", T, torch.int64)
    a = CommitArgs()
    a.row_offsets, a.accept_len, a.accept_index = _ptr(row_offsets), _ptr(accept_len), _ptr(accept_index)
    a.verify_slots, a.seq_lens = _ptr(verify_slots), _ptr(seq_lens)
    a.commit_offsets, a.src_slots, a.dst_pos = _ptr(o["commit_offsets"]), _ptr(o["src_slots"]), _ptr(o["dst_pos"])
    a.new_seq_lens, a.status = _ptr(o["new_seq_lens"]), _ptr(o["status"])
    a.evict_slots = _ptr(o.get("evict_slots")) if evict else None
    a.evict_offsets = _ptr(o.get("evict_offsets")) if evict else None
    a.total_rows, a.capacity, a.batch = T, T, B
    a.max_verify_len = int(max_verify_len)
    keep = [row_offsets, accept_len, accept_index, verify_slots, seq_lens]
    return PreparedCall(lib.spec_commit_indices, a, o, keep, dev)


def commit_indices(row_offsets: torch.Tensor, accept_len: torch.Tensor, accept_index: torch.Tensor,
                   verify_slots: torch.Tensor, seq_lens: torch.Tensor, *, max_verify_len: int,
                   evict: bool = True, out: dict | None = None, events: "HipEvents | None" = None) -> dict:
    """spec_commit_indices on torch tensors. Returns commit_offsets, src_slots, dst_pos, new_seq_lens,
    status (and evict_offsets, evict_slots). src_slots / dst_pos are sized total_rows; the valid part is
    commit_offsets[-1] entries long."""
    return prepare_commit_indices(row_offsets, accept_len, accept_index, verify_slots, seq_lens,
                                  max_verify_len=max_verify_len, evict=evict, out=out).run(events)


# ----------------------------------------------------------------------------------------------------
# verify-length planner and accept cutoff
# ----------------------------------------------------------------------------------------------------
def plan_budget(confidence_hist, sps_rows, sps, *, survival_eps: float = 0.0):
    """spec_plan_budget (host function): the verify budget K* from lagged confidences [batch, width] (a host
    array: numpy or CPU tensor, float32) and an SPS table. Returns (K*, predicted throughput for K = 0..n as a
    float64 numpy array)."""
    import numpy as np
    c = np.ascontiguousarray(confidence_hist.cpu().numpy() if isinstance(confidence_hist, torch.Tensor)
                             else confidence_hist, dtype=np.float32)
    if c.ndim != 2:
        raise ValueError("confidence_hist must be [batch, width]")
    R, W = c.shape
    xs = np.ascontiguousarray(sps_rows, dtype=np.float64)
    ys = np.ascontiguousarray(sps, dtype=np.float64)
    if xs.shape != ys.shape or xs.ndim != 1:
        raise ValueError("sps_rows and sps must be 1-D of equal length")
    theta = np.zeros(R * W + 1, np.float64)
    k, n = _i32(), _i32()
    _check(_lib().spec_plan_budget(c, R, W, xs, ys, len(xs), float(survival_eps), ctypes.byref(k), theta,
                                   ctypes.byref(n)))
    return int(k.value), theta[:n.value + 1]


def plan_budget_cost(confidence_hist, req_rows, req_cost, tok_rows, tok_cost, *, survival_eps: float = 0.0):
    """spec_plan_budget_cost (host function): the verify budget K* under an additive step-cost table (per-batch
    cost at the request count plus per-row cost at the target row count). Returns (K*, N(K) / T for K = 0..n)."""
    import numpy as np
    c = np.ascontiguousarray(confidence_hist.cpu().numpy() if isinstance(confidence_hist, torch.Tensor)
                             else confidence_hist, dtype=np.float32)
    if c.ndim != 2:
        raise ValueError("confidence_hist must be [batch, width]")
    R, W = c.shape
    tabs = [np.ascontiguousarray(t, dtype=np.float64) for t in (req_rows, req_cost, tok_rows, tok_cost)]
    if tabs[0].shape != tabs[1].shape or tabs[2].shape != tabs[3].shape or any(t.ndim != 1 for t in tabs):
        raise ValueError("each cost table is two 1-D arrays of equal length")
    theta = np.zeros(R * W + 1, np.float64)
    k, n = _i32(), _i32()
    _check(_lib().spec_plan_budget_cost(c, R, W, tabs[0], tabs[1], len(tabs[0]), tabs[2], tabs[3], len(tabs[2]),
                                        float(survival_eps), ctypes.byref(k), theta, ctypes.byref(n)))
    return int(k.value), theta[:n.value + 1]


def prepare_plan_layout(confidence: torch.Tensor, *, mode: str = "topk", budget: int = -1, threshold: float = 0.5,
                        min_verify_len: int = 1, max_verify_len: int | None = None, survival_eps: float = 0.0,
                        row_index: bool = True, out: dict | None = None) -> PreparedCall:
    """Checks and marshals the arguments of spec_plan_layout once (see plan_layout)."""
    lib = _lib()
    dev = confidence.device
    if confidence.dim() != 2:
        raise ValueError("confidence must be [batch, width]")
    _req(confidence, "confidence", torch.float32, device=dev)
    R, W = confidence.shape
    o = {} if out is None else out

    def get(name, n, dtype):
        t = o.get(name)
        if t is None:
            t = torch.empty(n, dtype=dtype, device=dev)
            o[name] = t
        return _req(t, name, dtype, n, dev)
    get("selected", R, torch.int32)
    get("verify_lens", R, torch.int32)
    get("offsets", R + 1, torch.int32)
    get("status", R, torch.int32)
    if row_index:
        get("row_index", R * (W + 1), torch.int64)
    a = PlanArgs()
    a.confidence = _ptr(confidence)
    a.selected, a.verify_lens, a.offsets = _ptr(o["selected"]), _ptr(o["verify_lens"]), _ptr(o["offsets"])
    a.row_index = _ptr(o.get("row_index")) if row_index else None
    a.status = _ptr(o["status"])
    a.batch, a.width, a.mode, a.budget = R, W, PLAN_MODES[mode], int(budget)
    a.min_verify_len = int(min_verify_len)
    a.max_verify_len = int(W + 1 if max_verify_len is None else max_verify_len)
    a.survival_eps, a.threshold = float(survival_eps), float(threshold)
    return PreparedCall(lib.spec_plan_layout, a, o, [confidence], dev)


def plan_layout(confidence: torch.Tensor, *, events: "HipEvents | None" = None, **kw) -> dict:
    """spec_plan_layout: per-request verify lengths from current confidences [batch, width] (float32). mode
    "topk" verifies the `budget` entries of highest prefix survival (budget < 0: every draft), "threshold" the
    drafts before the first confidence below `threshold`. Returns selected, verify_lens, offsets, status and
    row_index (compact verify row -> r * (width + 1) + j)."""
    return prepare_plan_layout(confidence, **kw).run(events)


def prepare_cap_trim(row_offsets: torch.Tensor, verify_lens: torch.Tensor, raw_accept_len: torch.Tensor,
                     raw_bonus: torch.Tensor, out_tokens: torch.Tensor, *, out: dict | None = None) -> PreparedCall:
    """Checks and marshals the arguments of spec_cap_trim once (see cap_trim)."""
    lib = _lib()
    dev = row_offsets.device
    _req(row_offsets, "row_offsets", torch.int32, device=dev)
    B = row_offsets.numel() - 1
    _req(verify_lens, "verify_lens", torch.int32, B, dev)
    _req(raw_accept_len, "raw_accept_len", torch.int32, B, dev)
    _req(raw_bonus, "raw_bonus", torch.int32, B, dev)
    T = out_tokens.numel()
    _req(out_tokens, "out_tokens", torch.int32, T, dev)
    o = {} if out is None else out
    for name in ("correct_len", "cap_trim_lens", "commit_lens", "block_accept_lens", "bonus", "status"):
        if o.get(name) is None:
            o[name] = torch.empty(B, dtype=torch.int32, device=dev)
        _req(o[name], name, torch.int32, B, dev)
    o["out_tokens"] = out_tokens
    a = CapTrimArgs()
    a.row_offsets, a.verify_lens = _ptr(row_offsets), _ptr(verify_lens)
    a.raw_accept_len, a.raw_bonus, a.out_tokens = _ptr(raw_accept_len), _ptr(raw_bonus), _ptr(out_tokens)
    a.correct_len, a.cap_trim_lens = _ptr(o["correct_len"]), _ptr(o["cap_trim_lens"])
    a.commit_lens, a.block_accept_lens = _ptr(o["commit_lens"]), _ptr(o["block_accept_lens"])
    a.bonus, a.status = _ptr(o["bonus"]), _ptr(o["status"])
    a.total_rows, a.batch = T, B
    keep = [row_offsets, verify_lens, raw_accept_len, raw_bonus, out_tokens]
    return PreparedCall(lib.spec_cap_trim, a, o, keep, dev)


def cap_trim(row_offsets, verify_lens, raw_accept_len, raw_bonus, out_tokens, *,
             events: "HipEvents | None" = None, out: dict | None = None) -> dict:
    """spec_cap_trim: cut a full-width verify's accepted prefix at each request's verify length. out_tokens is
    rewritten in place. Returns correct_len, cap_trim_lens, commit_lens, block_accept_lens, bonus, status."""
    return prepare_cap_trim(row_offsets, verify_lens, raw_accept_len, raw_bonus, out_tokens, out=out).run(events)


# ----------------------------------------------------------------------------------------------------
# the steps on either side of a tree verify: KV data move of the commit, draft-tree construction
# ----------------------------------------------------------------------------------------------------
def prepare_kv_move(buffers, commit_offsets: torch.Tensor, src_slots: torch.Tensor, dst_pos: torch.Tensor,
                    req_to_token: torch.Tensor, req_pool_indices: torch.Tensor) -> PreparedCall:
    """Checks and marshals the arguments of spec_kv_move once (see kv_move)."""
    lib = _lib()
    if not buffers:
        raise ValueError("at least one KV buffer is required")
    dev = buffers[0].device
    n_slots = buffers[0].shape[0]
    row_bytes = buffers[0][0].numel() * buffers[0].element_size() if n_slots else 0
    for t in buffers:
        if not (t.is_cuda and t.is_contiguous() and t.device == dev and t.shape[0] == n_slots):
            raise ValueError("KV buffers must be contiguous GPU tensors of equal slot count on one device")
        if t[0].numel() * t.element_size() != row_bytes:
            raise ValueError("KV buffers must have equal row bytes")
    addrs = torch.tensor([t.data_ptr() for t in buffers], dtype=torch.int64, device=dev)
    _req(commit_offsets, "commit_offsets", torch.int32, device=dev)
    B = commit_offsets.numel() - 1
    _req(src_slots, "src_slots", torch.int64, device=dev)
    _req(dst_pos, "dst_pos", torch.int32, src_slots.numel(), dev)
    _req(req_pool_indices, "req_pool_indices", torch.int32, B, dev)
    if req_to_token.dim() != 2:
        raise ValueError("req_to_token must be [rows, max_context]")
    _req(req_to_token, "req_to_token", torch.int64, device=dev)
    o = {"status": torch.empty(B, dtype=torch.int32, device=dev)}
    a = KvMoveArgs()
    a.buffers, a.commit_offsets = addrs.data_ptr(), _ptr(commit_offsets)
    a.src_slots, a.dst_pos = _ptr(src_slots), _ptr(dst_pos)
    a.req_to_token, a.req_pool_indices, a.status = _ptr(req_to_token), _ptr(req_pool_indices), _ptr(o["status"])
    a.n_slots, a.max_context, a.n_req_rows = n_slots, req_to_token.shape[1], req_to_token.shape[0]
    a.capacity, a.row_bytes, a.n_buffers, a.batch = src_slots.numel(), row_bytes, len(buffers), B
    keep = [addrs, commit_offsets, src_slots, dst_pos, req_to_token, req_pool_indices] + list(buffers)
    return PreparedCall(lib.spec_kv_move, a, o, keep, dev)


def kv_move(buffers, commit_offsets, src_slots, dst_pos, req_to_token, req_pool_indices, *,
            events: "HipEvents | None" = None) -> dict:
    """spec_kv_move: move the committed rows of every KV buffer (list of [n_slots, ...] GPU tensors, equal row
    bytes, a multiple of 16) to the slots of positions dst_pos through req_to_token. In place. Returns status."""
    return prepare_kv_move(buffers, commit_offsets, src_slots, dst_pos, req_to_token, req_pool_indices).run(events)


def prepare_tree_build(anchors: torch.Tensor, draft_tokens: torch.Tensor, draft_probs: torch.Tensor,
                       seq_lens: torch.Tensor, n_nodes: int, *, mask: bool = True,
                       out: dict | None = None) -> PreparedCall:
    """Checks and marshals the arguments of spec_tree_build once (see tree_build)."""
    lib = _lib()
    dev = anchors.device
    if draft_tokens.dim() != 4 or draft_tokens.shape[2] != draft_tokens.shape[3]:
        raise ValueError("draft_tokens must be [batch, n_steps, topk, topk]")
    B, S, k, _ = draft_tokens.shape
    _req(anchors, "anchors", torch.int32, B, dev)
    _req(draft_tokens, "draft_tokens", torch.int32, device=dev)
    _req(draft_probs, "draft_probs", torch.float32, B * S * k * k, dev)
    _req(seq_lens, "seq_lens", torch.int32, B, dev)
    N = int(n_nodes)
    o = {} if out is None else out
    for name in ("tokens", "parents", "positions", "first_child", "next_sibling", "cand_index"):
        if o.get(name) is None:
            o[name] = torch.empty(B * N, dtype=torch.int32, device=dev)
        _req(o[name], name, torch.int32, B * N, dev)
    if o.get("status") is None:
        o["status"] = torch.empty(B, dtype=torch.int32, device=dev)
    if mask and o.get("mask") is None:
        o["mask"] = torch.empty(B * N * N, dtype=torch.uint8, device=dev)
    a = TreeBuildArgs()
    a.anchors, a.draft_tokens, a.draft_probs, a.seq_lens = (_ptr(anchors), _ptr(draft_tokens), _ptr(draft_probs),
                                                           _ptr(seq_lens))
    a.tokens, a.parents, a.positions = _ptr(o["tokens"]), _ptr(o["parents"]), _ptr(o["positions"])
    a.mask = _ptr(o.get("mask")) if mask else None
    a.first_child, a.next_sibling, a.cand_index = (_ptr(o["first_child"]), _ptr(o["next_sibling"]),
                                                   _ptr(o["cand_index"]))
    a.status = _ptr(o["status"])
    a.batch, a.n_steps, a.topk, a.n_nodes = B, S, k, N
    return PreparedCall(lib.spec_tree_build, a, o, [anchors, draft_tokens, draft_probs, seq_lens], dev)


def tree_build(anchors, draft_tokens, draft_probs, seq_lens, n_nodes: int, *, mask: bool = True,
               events: "HipEvents | None" = None, out: dict | None = None) -> dict:
    """spec_tree_build: EAGLE-2 draft trees of n_nodes nodes from the draft's per-step top-k children
    (draft_tokens int32 / draft_probs float32 [batch, n_steps, topk, topk]). Returns tokens, parents,
    positions, mask ([batch * n_nodes * n_nodes] uint8), first_child, next_sibling, cand_index ([batch *
    n_nodes] int32 each; tokens and parents feed verify_tree) and status."""
    return prepare_tree_build(anchors, draft_tokens, draft_probs, seq_lens, n_nodes, mask=mask, out=out).run(events)

