"""CPU pins of the KV data-move oracle (oracle/kv.py): the pages' tree-path compaction on the hand-built
tree (golden file), the chain case where nothing moves, path order = gather-then-scatter on random tree
paths (an independent formulation), untouched rows, bad slots, and a planted mistake."""
import json
import os

import numpy as np
import pytest

from oracle import kv as okv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _labelled_buffers(n_slots, labels, row=4):
    """Two buffers (K and V of one layer) whose rows encode a label id."""
    ids = {lab: i + 1 for i, lab in enumerate(sorted(set(labels.values())))}
    k = np.zeros((n_slots, row), np.int32)
    for slot, lab in labels.items():
        k[int(slot)] = ids[lab]
    return [k, -k], ids


def test_tree_path_compaction_example():
    g = _golden("kv_move_tree7.json")
    n_slots = 128
    bufs, ids = _labelled_buffers(n_slots, g["rows_before"])
    r2t = np.full((1, 64), -1, np.int64)
    for i, s in enumerate(g["node_slots"]):
        r2t[0, g["seq_len"] + i] = s
    assert list(np.asarray(g["node_slots"])[g["accepted_path"]]) == g["src_slots"]
    out, st = okv.kv_move(bufs, [0, 3], g["src_slots"], g["dst_pos"], r2t, [0])
    assert st[0] == 0
    for slot, lab in g["rows_after"].items():
        assert np.all(out[0][int(slot)] == ids[lab]) and np.all(out[1][int(slot)] == -ids[lab])
    for pos, lab in g["committed_positions_after"].items():
        assert np.all(out[0][r2t[0, int(pos)]] == ids[lab])


def test_chain_commit_moves_nothing():
    # [EAGLE→DFlash2] §8.1: D E F G H verified, D E F committed: a chain's accepted rows already sit at
    # the positions after seq_len, so every entry has src == dst.
    g = _golden("commit_defgh.json")
    seq = len(g["committed_before"])
    r2t = np.arange(200, 264, dtype=np.int64)[None, :]
    labels = {str(r2t[0, seq + i]): t for i, t in enumerate(g["verify_input"])}
    bufs, ids = _labelled_buffers(300, labels)
    n = g["commit_len"]
    src = [int(r2t[0, seq + k]) for k in range(n)]
    out, st = okv.kv_move(bufs, [0, n], src, [seq + k for k in range(n)], r2t, [0])
    assert all(np.array_equal(a, b) for a, b in zip(out, bufs)) and st[0] == 0
    assert [int(out[0][r2t[0, seq + k]][0]) for k in range(n)] == [ids[t] for t in g["new_valid_kv"]]


def _gather_scatter(buffers, offs, src, dst_pos, r2t, pools):
    out = [b.copy() for b in buffers]
    for b in range(len(offs) - 1):
        es = range(offs[b], offs[b + 1])
        dsts = [int(r2t[pools[b], dst_pos[e]]) for e in es]
        rows = [[buf[int(src[e])].copy() for e in es] for buf in buffers]
        for bi, buf in enumerate(out):
            for i, d in enumerate(dsts):
                buf[d] = rows[bi][i]
    return out


def _random_paths(rng, B, N, seq_max=50):
    offs, src, dst = [0], [], []
    r2t = np.full((B + 3, seq_max + N + 4), -1, np.int64)
    pools = rng.permutation(B + 3)[:B]
    slots = rng.permutation(4096)
    nxt = 0
    for b in range(B):
        seq = int(rng.integers(0, seq_max))
        for p in range(seq + N):
            r2t[pools[b], p] = slots[nxt]
            nxt += 1
        r = int(rng.integers(0, min(N, 6)))
        path = [0] + sorted(rng.choice(np.arange(1, N), r, replace=False).tolist())
        for k, node in enumerate(path):
            src.append(int(r2t[pools[b], seq + node]))
            dst.append(seq + k)
        offs.append(len(src))
    return np.array(offs), np.array(src, np.int64), np.array(dst, np.int32), r2t, pools


@pytest.mark.parametrize("seed", range(10))
def test_path_order_equals_gather_then_scatter(seed):
    rng = np.random.default_rng(seed)
    offs, src, dst, r2t, pools = _random_paths(rng, 12, 16)
    bufs = [rng.integers(-1000, 1000, (4096, 6)).astype(np.int32) for _ in range(3)]
    out, st = okv.kv_move(bufs, offs, src, dst, r2t, pools)
    ref = _gather_scatter(bufs, offs, src, dst, r2t, pools)
    assert all(np.array_equal(a, b) for a, b in zip(out, ref)) and not st.any()
    # every committed position holds its source's original row; rows no entry writes are untouched
    written = {int(r2t[pools[b], dst[e]]) for b in range(12) for e in range(offs[b], offs[b + 1])}
    for b in range(12):
        for e in range(offs[b], offs[b + 1]):
            assert np.array_equal(out[0][r2t[pools[b], dst[e]]], bufs[0][src[e]])
    keep = np.setdiff1d(np.arange(4096), np.array(sorted(written)))
    assert np.array_equal(out[1][keep], bufs[1][keep])


def test_bad_slots_are_skipped_and_flagged():
    bufs = [np.arange(40).reshape(10, 4).astype(np.int32)]
    r2t = np.array([[0, 1, 2, 3, 4, 5, 6, 7, 8, 99]], np.int64)
    offs = [0, 2, 3, 4, 5]
    src = [5, 6, 42, 3, 1]
    dst = [0, 1, 2, 9, 2]
    out, st = okv.kv_move(bufs, offs, src, dst, r2t, [0, 0, 0, 1])
    assert list(st) == [0, okv.ST_BAD_SLOT, okv.ST_BAD_SLOT, okv.ST_BAD_SLOT]
    assert np.array_equal(out[0][0], bufs[0][5]) and np.array_equal(out[0][1], bufs[0][6])
    assert np.array_equal(out[0][2:], bufs[0][2:])


def test_pins_catch_reverse_order(monkeypatch):
    def bad(buffers, offs, src, dst_pos, r2t, pools):
        out = [b.copy() for b in buffers]
        for b in range(len(offs) - 1):
            for e in reversed(range(int(offs[b]), int(offs[b + 1]))):
                d = int(r2t[pools[b], dst_pos[e]])
                for buf in out:
                    buf[d] = buf[int(src[e])]
        return out, np.zeros(len(offs) - 1, np.uint32)
    monkeypatch.setattr(okv, "kv_move", bad)
    with pytest.raises(AssertionError):
        for seed in range(10):
            test_path_order_equals_gather_then_scatter(seed)
