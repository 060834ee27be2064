"""Oracle for the KV data move of a verify round's commit: plain, slow, CPU only.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may import
or call this module. It shares no code with the HIP library and imports nothing from it.

[EAGLE→DFlash2] tom-jerr.github.io, "从 EAGLE 到 DFlash 2：SGLang 与 SpecForge 的投机解码训练和推理", §8.1-§8.2 and
the engineering notes on move_accept_tokens_to_target_kvcache: after verify, the KV of the accepted tokens is
moved to the contiguous positions after seq_lens (a tree's accepted path sits at non-contiguous node rows);
rejected slots are simply overwritten later. The positions map to physical KV slots through the request's
row of the req_to_token table; draft and target share these slot ids but keep separate buffers (every
buffer listed is moved: K and V of every layer).

For request b with commit entries e = commit_offsets[b] .. commit_offsets[b+1]-1 (k = 0, 1, .. in path
order): dst_slot = req_to_token[req_pool_indices[b], dst_pos[e]] and, for every buffer, row dst_slot takes
the contents of row src_slots[e]. READING: entries are moved in path order k = 0, 1, .. (for a tree path the
destinations are positions seq_len + k and the sources the path nodes' rows seq_len + n_k with n_k >= k
strictly increasing, so a source is never a position written by an earlier entry: this equals reading every
source before writing any destination). An entry whose slots or position fall outside the tables is skipped
and flags BAD_SLOT; an entry with src == dst moves nothing.
"""
from __future__ import annotations

import numpy as np

ST_BAD_SLOT = 1 << 12


def kv_move(buffers: list[np.ndarray], commit_offsets, src_slots, dst_pos, req_to_token: np.ndarray,
            req_pool_indices) -> tuple[list[np.ndarray], np.ndarray]:
    """Returns the moved copies of `buffers` (each [n_slots, row]) and per-request status."""
    out = [b.copy() for b in buffers]
    B = len(commit_offsets) - 1
    status = np.zeros(B, np.uint32)
    n_slots = buffers[0].shape[0] if buffers else 0
    n_rows, max_ctx = req_to_token.shape
    for b in range(B):
        pool = int(req_pool_indices[b])
        for e in range(int(commit_offsets[b]), int(commit_offsets[b + 1])):
            src, pos = int(src_slots[e]), int(dst_pos[e])
            if not (0 <= pool < n_rows and 0 <= pos < max_ctx):
                status[b] |= ST_BAD_SLOT
                continue
            dst = int(req_to_token[pool, pos])
            if not (0 <= src < n_slots and 0 <= dst < n_slots):
                status[b] |= ST_BAD_SLOT
                continue
            if src == dst:
                continue
            for buf in out:
                buf[dst] = buf[src]
    return out, status
