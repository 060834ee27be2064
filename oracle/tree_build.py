"""Oracle for EAGLE-2 dynamic draft-tree construction: plain, slow, CPU only.

TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of bench.py may import
or call this module. It shares no code with the HIP library and imports nothing from it.

Steps, in the pages' order:
  [EAGLE→DFlash2]  tom-jerr.github.io, "从 EAGLE 到 DFlash 2：SGLang 与 SpecForge 的投机解码训练和推理",
                   §2.3 (a node's score is the product of the draft probabilities along its path; expand the
                   high-score frontier, rerank all generated candidates within the verify budget, keep the
                   ancestor closure), §2.4 (a node sees the committed history, its ancestors and itself, not
                   its siblings; its position id is its depth, not its index in the flattened array), §3.4
                   (the tree arrays: parents, mask, positions, first child / next sibling)
  [SpecDec]        zdszero.github.io, "speculative_decoding" (EAGLE tree build: each step keeps topk of the
                   topk^2 expansions, then the best num_draft_tokens - 1 nodes plus the root form the tree)

Inputs per request b: the anchor token (the root), the draft's top-k children of each frontier node at each of
S steps: tokens[b, s, f, c], probs[b, s, f, c] (f = frontier slot, c = child rank); step 0 expands the root
only (f = 0). Candidate ids: step 0's are 0 .. k-1 (c), step s >= 1's are k + (s-1) k^2 + f k + c.

READINGS (where the pages leave a step open):
  * score(candidate) = float32 product score(parent) * q in path order, the root's score being 1;
  * every selection ranks candidates by score descending, then candidate id ascending;
  * the frontier after step s is the top k of step s's candidates in that order (frontier slot = rank);
  * the tree's nodes are the root and the top N - 1 of all candidates, listed in candidate-id order, so a
    parent precedes its children; the ancestor closure holds because a child never outranks its parent
    (q <= 1 and a parent's id is smaller);
  * a probability that is NaN counts as 0 and one outside [0, 1] is clamped (BAD_CONF);
  * outputs: tokens (node 0 = anchor), parents (root -1), depth, positions = seq_len + depth, the
    visibility mask [N, N] (1 iff j is i or an ancestor of i), first child and next sibling (-1 if none),
    and the candidate id of every node (-1 for the root).
"""
from __future__ import annotations

import numpy as np

ST_BAD_CONF = 1 << 11


def _sanitize(q) -> tuple[np.float32, bool]:
    q = np.float32(q)
    if np.isnan(q):
        return np.float32(0.0), True
    if q < 0:
        return np.float32(0.0), True
    if q > 1:
        return np.float32(1.0), True
    return (q if q > 0 else np.float32(0.0)), False


def candidates(tokens: np.ndarray, probs: np.ndarray) -> dict:
    """Expand and select step by step for one request: tokens/probs [S, k, k]. Returns per candidate id its
    score, token, parent candidate id (-1: root) and step, the frontier after each step, and a BAD_CONF flag."""
    S, k, _ = tokens.shape
    n = k + (S - 1) * k * k
    score = np.zeros(n, np.float32)
    token = np.zeros(n, np.int64)
    parent = np.full(n, -1, np.int64)
    step = np.zeros(n, np.int64)
    bad = False
    frontier = [(-1, np.float32(1.0))]   # (candidate id, score) of the frontier, in slot order
    frontiers = []
    for s in range(S):
        ids = []
        for f, (pid, psc) in enumerate(frontier):
            for c in range(k):
                cid = c if s == 0 else k + (s - 1) * k * k + f * k + c
                q, b = _sanitize(probs[s, f, c])
                bad |= b
                score[cid] = np.float32(psc * q)
                token[cid] = tokens[s, f, c]
                parent[cid] = pid
                step[cid] = s
                ids.append(cid)
        ranked = sorted(ids, key=lambda i: (-float(score[i]), i))
        frontier = [(i, score[i]) for i in ranked[:k]]
        frontiers.append([i for i, _ in frontier])
    return {"score": score, "token": token, "parent": parent, "step": step, "frontiers": frontiers, "bad": bad}


def build_tree(anchor: int, tokens: np.ndarray, probs: np.ndarray, n_nodes: int, seq_len: int) -> dict:
    """One request's tree of n_nodes nodes (root included)."""
    c = candidates(np.asarray(tokens), np.asarray(probs))
    n_cand = len(c["score"])
    if not 1 <= n_nodes <= n_cand + 1:
        raise ValueError("n_nodes must be in [1, number of candidates + 1]")
    order = sorted(range(n_cand), key=lambda i: (-float(c["score"][i]), i))
    chosen = sorted(order[:n_nodes - 1])
    node_of = {cid: i + 1 for i, cid in enumerate(chosen)}
    N = n_nodes
    toks = np.zeros(N, np.int64)
    par = np.full(N, -1, np.int64)
    depth = np.zeros(N, np.int64)
    cand = np.full(N, -1, np.int64)
    toks[0] = anchor
    for i, cid in enumerate(chosen, start=1):
        pc = int(c["parent"][cid])
        par[i] = 0 if pc < 0 else node_of[pc]     # KeyError here would mean a broken ancestor closure
        toks[i] = c["token"][cid]
        depth[i] = depth[par[i]] + 1
        cand[i] = cid
    mask = np.zeros((N, N), np.uint8)
    for i in range(N):
        j = i
        while j >= 0:
            mask[i, j] = 1
            j = int(par[j])
    first_child = np.full(N, -1, np.int64)
    next_sibling = np.full(N, -1, np.int64)
    for i in range(1, N):
        p = int(par[i])
        if first_child[p] < 0:
            first_child[p] = i
        for j in range(i + 1, N):
            if par[j] == p:
                next_sibling[i] = j
                break
    return {"tokens": toks, "parents": par, "depth": depth, "positions": seq_len + depth, "mask": mask,
            "first_child": first_child, "next_sibling": next_sibling, "cand_index": cand,
            "status": ST_BAD_CONF if c["bad"] else 0, "frontiers": c["frontiers"], "score": c["score"]}


def build_trees(anchors, tokens, probs, n_nodes: int, seq_lens) -> dict:
    """Batch version: tokens/probs [B, S, k, k]. Outputs stacked per request."""
    B = len(anchors)
    res = [build_tree(int(anchors[b]), tokens[b], probs[b], n_nodes, int(seq_lens[b])) for b in range(B)]
    out = {}
    for key in ("tokens", "parents", "depth", "positions", "mask", "first_child", "next_sibling", "cand_index"):
        out[key] = np.stack([r[key] for r in res])
    out["status"] = np.array([r["status"] for r in res], np.uint32)
    return out
