"""Seeded synthetic verify workloads (inputs only; no verify / accept / commit arithmetic lives here).

Both the HIP library's tests / bench and the CPU oracle consume these arrays; neither side's code is used
to make them. Shapes follow the workloads the pages describe: Qwen-family vocab 151,936 and Llama-3 vocab
128,256; DFlash blocks of 16 (anchor + 15); DSpark / EAGLE chains of 7-8; EAGLE trees of 64 nodes;
high-concurrency ragged batches with per-request draft length 0..15.

Recipe (all numpy PCG64; seed = 1000*k for workload k; np.random.SeedSequence(seed).spawn(B + 1): child 0
drives the batch structure, child b+1 drives request b and is split again into logits / noise / tokens /
uniforms streams, so requests can be generated independently and in parallel):
  * target logits  3*N(0,1) per entry, plus 8 added to one uniformly chosen token per row
                   (tiny workload: N(0, 2^2), float32, no planted token);
  * draft logits   target (float32, before rounding) + N(0, sigma^2);
  * bf16           round-to-nearest-even of the float32 values (stored as uint16 bit patterns);
  * draft tokens   sampling workloads: d_{j+1} ~ q_j = softmax(stored draft row j / T), drawn in float64
                   with np.searchsorted over the cumulative sum (the drafter's own sampling, so d ~ q exactly
                   as the verifier sees q); greedy block workload: a planted accepted prefix (see
                   block_greedy); trees: EAGLE-style top-c expansion (see tree);
  * uniforms       Generator.random(dtype=float32), in [0, 1).
  * planner        (planner_inputs) per-request draft quality q_r ~ Beta(4, 1.5); current confidence
                   c_{r,j} = clip(q_r * 0.97^j + N(0, 0.05^2), 0, 1) (later positions a little less sure);
                   the lagged history = clip(c + N(0, 0.05^2), 0, 1); SPS table (rows -> steps/s) points
                   512:100, 2048:95, 4096:70, 8192:35 (flat at low load, falling at high load, the shape
                   the DSpark page describes); raw accept lengths of a full-width verify ~ U{0..W}.
  * tree round     (tree_round_inputs) draft top-k children per step: token ids uniform, probabilities a
                   sorted Dirichlet(0.7) top-k slice; accepted paths: the root and U{0..4} increasing node
                   ids; req_to_token a shuffled slot table, node i of request b at position seq_len + i.
  * sparse q       (chain_sparse) the drafter's candidate set of a draft row is the top-K of its float32
                   draft logits (distinct ids, descending, lowest id first among equal values) and q the
                   softmax over just those K at T, stored as float32; a greedy request takes the first
                   candidate with a one-hot q over the candidates, a sampling request draws d ~ q from the
                   stored float32 q (float64 inverse CDF).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

QWEN_VOCAB = 151936
LLAMA3_VOCAB = 128256


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _pool_map(fn, items, parallel: bool):
    items = list(items)
    if not parallel or len(items) < 4:
        return [fn(i) for i in items]
    workers = max(1, min(16, os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))


def _target_rows(rng: np.random.Generator, n: int, V: int, planted: bool, scale: float) -> np.ndarray:
    x = rng.standard_normal((n, V), dtype=np.float32)
    x *= np.float32(scale)
    if planted and n:
        cols = rng.integers(0, V, size=n)
        x[np.arange(n), cols] += np.float32(8.0)
    return x


def _draw_from_rows(rows_bits_or_f32: np.ndarray, temperature: float, u: np.ndarray) -> np.ndarray:
    """The drafter's sampling: token ~ softmax(row / T) per row (float64, inverse CDF via searchsorted)."""
    out = np.empty(len(rows_bits_or_f32), np.int32)
    for i, row in enumerate(rows_bits_or_f32):
        x = (bf16_to_f32(row) if row.dtype == np.uint16 else row).astype(np.float64) / temperature
        e = np.exp(x - x.max())
        cdf = np.cumsum(e)
        k = int(np.searchsorted(cdf, float(u[i]) * cdf[-1], side="right"))
        out[i] = min(k, len(cdf) - 1)
    return out


@dataclass
class ChainWorkload:
    name: str
    vocab: int
    batch: int
    offsets: np.ndarray          # int32 [B+1]
    target: np.ndarray           # [T_rows, V] uint16 (bf16 bits) or float32
    draft: np.ndarray | None     # [T_rows - B, V] or None (greedy-only workloads)
    draft_tokens: np.ndarray     # int32 [T_rows - B]
    u_accept: np.ndarray         # float32 [T_rows - B]
    u_final: np.ndarray          # float32 [B]
    temperature: float
    modes: tuple
    max_verify_len: int
    planted_r: np.ndarray | None = None     # block_greedy only: accept length fixed by construction
    meta: dict = field(default_factory=dict)
    cand_ids: np.ndarray | None = None      # chain_sparse only: int32 [T_rows - B, K]
    cand_q: np.ndarray | None = None        # chain_sparse only: float32 [T_rows - B, K]

    @property
    def total_rows(self) -> int:
        return int(self.offsets[-1])

    @property
    def dtype(self) -> str:
        return "bf16" if self.target.dtype == np.uint16 else "f32"

    def algorithmic_bytes(self, mode: str) -> int:
        """Every target row (and draft row in rejection mode, or the candidate pairs in sparse mode) read
        once."""
        rows = self.total_rows + (self.total_rows - self.batch if mode == "rejection" else 0)
        extra = self.cand_ids.nbytes + self.cand_q.nbytes if mode == "rejection_sparse" else 0
        return rows * self.vocab * self.target.itemsize + extra


@dataclass
class TreeWorkload:
    name: str
    vocab: int
    batch: int
    n_nodes: int
    target: np.ndarray           # [B*N, V]
    parents: np.ndarray          # int32 [B*N]
    tokens: np.ndarray           # int32 [B*N]
    u_accept: np.ndarray         # float32 [B*N]
    u_final: np.ndarray          # float32 [B]
    temperature: float
    modes: tuple = ("greedy", "target_only")
    meta: dict = field(default_factory=dict)

    @property
    def total_rows(self) -> int:
        return self.batch * self.n_nodes

    @property
    def dtype(self) -> str:
        return "bf16" if self.target.dtype == np.uint16 else "f32"

    def algorithmic_bytes(self, mode: str) -> int:
        return self.total_rows * self.vocab * self.target.itemsize


def _chain_from_lengths(name, seed, kids, lens, V, *, bf16, planted, scale, draft_sigma, temperature,
                        modes, max_len, parallel):
    B = len(lens)
    offsets = np.zeros(B + 1, np.int32)
    offsets[1:] = np.cumsum(lens)
    T = int(offsets[-1])
    D = T - B
    tdtype = np.uint16 if bf16 else np.float32
    target = np.empty((T, V), tdtype)
    draft = np.empty((D, V), tdtype) if draft_sigma is not None else None
    tokens = np.empty(D, np.int32)
    u_accept = np.empty(D, np.float32)
    u_final = np.empty(B, np.float32)

    def one(b):
        s_logit, s_noise, s_tok, s_unif = [np.random.Generator(np.random.PCG64(s)) for s in kids[b + 1].spawn(4)]
        n = int(lens[b])
        m = n - 1
        t = _target_rows(s_logit, n, V, planted, scale)
        lo, dlo = int(offsets[b]), int(offsets[b]) - b
        target[lo:lo + n] = bf16_bits(t) if bf16 else t
        if draft is not None and m > 0:
            d = t[:m] + s_noise.standard_normal((m, V), dtype=np.float32) * np.float32(draft_sigma)
            draft[dlo:dlo + m] = bf16_bits(d) if bf16 else d
            tokens[dlo:dlo + m] = _draw_from_rows(draft[dlo:dlo + m], temperature,
                                                  s_tok.random(m, dtype=np.float32))
        u_accept[dlo:dlo + m] = s_unif.random(m, dtype=np.float32)
        u_final[b] = s_unif.random(dtype=np.float32)

    _pool_map(one, range(B), parallel)
    return ChainWorkload(name, V, B, offsets, target, draft, tokens, u_accept, u_final, temperature, modes,
                         max_len, meta={"seed": seed})


def tiny_chain(seed: int = 1000, batch: int = 4, m: int = 4, vocab: int = 32) -> ChainWorkload:
    """Tiny chain: B 4, m 4 (verify length 5), V 32, float32 logits; target ~ N(0, 2^2), draft = target +
    N(0, 0.5^2), T 1.0; drafts drawn from q; both greedy and rejection run on the same inputs."""
    kids = np.random.SeedSequence(seed).spawn(batch + 1)
    lens = np.full(batch, m + 1, np.int64)
    return _chain_from_lengths("tiny_chain", seed, kids, lens, vocab, bf16=False, planted=False, scale=2.0,
                               draft_sigma=0.5, temperature=1.0, modes=("greedy", "rejection"),
                               max_len=m + 1, parallel=False)


def chain_rejection(seed: int = 2000, batch: int = 64, m: int = 7, vocab: int = QWEN_VOCAB,
                    parallel: bool = True) -> ChainWorkload:
    """Chain rejection sampling: B 64, m 7 (verify length 8), V 151,936, bf16; draft = target + N(0, 1),
    T 1.0, topk 1."""
    kids = np.random.SeedSequence(seed).spawn(batch + 1)
    lens = np.full(batch, m + 1, np.int64)
    return _chain_from_lengths("chain_rejection", seed, kids, lens, vocab, bf16=True, planted=True, scale=3.0,
                               draft_sigma=1.0, temperature=1.0, modes=("rejection",), max_len=m + 1,
                               parallel=parallel)


def ragged(seed: int = 5000, batch: int = 512, m_max: int = 15, vocab: int = QWEN_VOCAB,
           temperature: float = 0.7, parallel: bool = True) -> ChainWorkload:
    """High-concurrency ragged verify: B 512, m_i ~ U{0..15}, V 151,936, bf16 target and draft;
    draft = target + N(0, 0.8^2), T 0.7, rejection; rows packed by offsets."""
    kids = np.random.SeedSequence(seed).spawn(batch + 1)
    s_struct = np.random.Generator(np.random.PCG64(kids[0]))
    lens = s_struct.integers(0, m_max + 1, size=batch) + 1
    return _chain_from_lengths("ragged", seed, kids, lens, vocab, bf16=True, planted=True, scale=3.0,
                               draft_sigma=0.8, temperature=temperature, modes=("rejection",),
                               max_len=m_max + 1, parallel=parallel)


def top_candidates(x: np.ndarray, K: int) -> np.ndarray:
    """Ids of the K largest entries of x, by descending value and ascending id among equal values."""
    part = np.argpartition(-x, K - 1)[:K] if K < len(x) else np.arange(len(x))
    kth = x[part].min()
    pool = np.flatnonzero(x >= kth)                  # every id tied with the K-th value competes
    order = np.lexsort((pool, -x[pool].astype(np.float64)))
    return pool[order[:K]].astype(np.int32)


def chain_sparse(seed: int = 6000, batch: int = 64, m: int = 7, vocab: int = QWEN_VOCAB, K: int = 16,
                 temperature: float = 1.0, greedy_frac: float = 0.25, bf16: bool = True,
                 ragged: bool = False, draft_sigma: float = 1.0, parallel: bool = True) -> ChainWorkload:
    """Chain rejection with a sparse q (the DFlash 2 selector's K candidates): B 64, m 7, V 151,936, bf16
    target as chain_rejection; per draft row the top-16 of draft logits target + N(0, 1) and q = softmax
    over them at T 1.0; a quarter of the requests are greedy rows (one-hot q on the first candidate).
    ragged=True draws each request's m from U{0..m} instead."""
    kids = np.random.SeedSequence(seed).spawn(batch + 1)
    s_struct = np.random.Generator(np.random.PCG64(kids[0]))
    greedy = s_struct.random(batch) < greedy_frac
    lens = s_struct.integers(0, m + 1, size=batch) + 1 if ragged else np.full(batch, m + 1, np.int64)
    w = _chain_from_lengths("chain_sparse", seed, kids, lens, vocab, bf16=bf16, planted=True, scale=3.0,
                            draft_sigma=None, temperature=temperature, modes=("rejection_sparse",),
                            max_len=m + 1, parallel=parallel)
    D = w.total_rows - batch
    ids = np.empty((D, K), np.int32)
    qs = np.empty((D, K), np.float32)

    def one(b):
        # streams 4 and 5 of request b (0..3 made its target rows and uniforms)
        s_noise, s_tok = [np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(b + 1, i))))
                          for i in (4, 5)]
        lo, dlo = int(w.offsets[b]), int(w.offsets[b]) - b
        for j in range(int(lens[b]) - 1):
            t = bf16_to_f32(w.target[lo + j]) if bf16 else w.target[lo + j]
            d = t + s_noise.standard_normal(vocab, dtype=np.float32) * np.float32(draft_sigma)
            c = top_candidates(d, K)
            ids[dlo + j] = c
            if greedy[b]:
                qs[dlo + j] = 0.0
                qs[dlo + j, 0] = 1.0
                w.draft_tokens[dlo + j] = c[0]
            else:
                z = d[c].astype(np.float64) / temperature
                e = np.exp(z - z.max())
                qs[dlo + j] = (e / e.sum()).astype(np.float32)
                cdf = np.cumsum(qs[dlo + j].astype(np.float64))
                u = float(s_tok.random(dtype=np.float32))
                k = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
                w.draft_tokens[dlo + j] = c[min(k, K - 1)]

    _pool_map(one, range(batch), parallel)
    w.cand_ids, w.cand_q = ids, qs
    w.meta["greedy_requests"] = int(greedy.sum())
    return w


def block_greedy(seed: int = 3000, batch: int = 32, block: int = 16, vocab: int = QWEN_VOCAB,
                 tie_rate: float = 0.01, parallel: bool = True) -> ChainWorkload:
    """DFlash-shaped greedy verify: B 32, block 16 (anchor + 15 drafts), V 151,936, bf16 target only.

    Planted accept length r0 ~ Geometric(0.25) on {0, 1, ..} (P(r0 = k) = 0.75^k * 0.25) clipped to
    block-1. d_1..d_r0 equal the target argmax (lowest id among the row's maxima, np.argmax); d_{r0+1} is
    uniform over the ids outside the row's maximal set; later drafts are uniform. In `tie_rate` of the rows
    the max value is copied to another random id (an exact tie); inside the prefix, half of the tied rows
    make the draft use the HIGHER tied id, which ends the accepted prefix there. planted_r holds the accept
    length these choices fix."""
    kids = np.random.SeedSequence(seed).spawn(batch + 1)
    s_struct = np.random.Generator(np.random.PCG64(kids[0]))
    r0 = np.minimum(s_struct.geometric(0.25, size=batch) - 1, block - 1)
    m = block - 1
    offsets = (np.arange(batch + 1) * block).astype(np.int32)
    T = batch * block
    target = np.empty((T, vocab), np.uint16)
    tokens = np.empty(batch * m, np.int32)
    planted = np.empty(batch, np.int64)
    n_ties = np.zeros(batch, np.int64)

    def one(b):
        s_logit, s_noise, s_tok, s_unif = [np.random.Generator(np.random.PCG64(s)) for s in kids[b + 1].spawn(4)]
        rows = bf16_bits(_target_rows(s_logit, block, vocab, True, 3.0))
        tie = s_noise.random(block) < tie_rate
        use_high = s_noise.random(block) < 0.5
        r_exp = int(r0[b])
        for j in range(block):
            f = bf16_to_f32(rows[j])
            top = int(np.argmax(f))
            if tie[j]:
                other = int(s_noise.integers(0, vocab - 1))
                other += other >= top
                rows[j, other] = rows[j, top]
                n_ties[b] += 1
        for j in range(1, m + 1):           # d_j is judged by row j-1
            f = bf16_to_f32(rows[j - 1])
            maxset = np.flatnonzero(f == f.max())
            if j <= r0[b]:
                d = int(maxset[0])
                if tie[j - 1] and len(maxset) > 1 and use_high[j - 1]:
                    d = int(maxset[-1])
                    r_exp = min(r_exp, j - 1)
            elif j == r0[b] + 1:
                d = int(s_tok.integers(0, vocab - len(maxset)))
                for t in maxset:            # skip the maximal ids
                    d += d >= t
            else:
                d = int(s_tok.integers(0, vocab))
            tokens[b * m + j - 1] = d
        target[b * block:(b + 1) * block] = rows
        planted[b] = r_exp

    _pool_map(one, range(batch), parallel)
    wl = ChainWorkload("block_greedy", vocab, batch, offsets, target, None, tokens,
                       np.zeros(batch * m, np.float32), np.zeros(batch, np.float32), 1.0, ("greedy",), block,
                       planted_r=planted, meta={"seed": seed, "tie_rows": int(n_ties.sum())})
    return wl


def tree(seed: int = 4000, batch: int = 32, n_nodes: int = 64, vocab: int = LLAMA3_VOCAB, max_depth: int = 8,
         max_branch: int = 8, temperature: float = 1.0, bf16: bool = True, parallel: bool = True) -> TreeWorkload:
    """EAGLE-style tree verify: B 32, 64 nodes per request including the root, V 128,256, bf16 target.

    parent[i] is uniform over the earlier nodes j with depth(j) < max_depth and fewer than max_branch
    children. A node with c children gives them, in child-index order, the top-c ids (distinct, by value
    descending, lowest id first among equal values) of its own target row plus N(0, 1) noise (a stand-in
    for a draft's top-k expansion). The root's token is random and unused."""
    kids = np.random.SeedSequence(seed).spawn(batch + 1)
    N = n_nodes
    tdtype = np.uint16 if bf16 else np.float32
    target = np.empty((batch * N, vocab), tdtype)
    parents = np.empty(batch * N, np.int32)
    tokens = np.empty(batch * N, np.int32)
    u_accept = np.empty(batch * N, np.float32)
    u_final = np.empty(batch, np.float32)

    def one(b):
        s_logit, s_noise, s_tok, s_unif = [np.random.Generator(np.random.PCG64(s)) for s in kids[b + 1].spawn(4)]
        x = _target_rows(s_logit, N, vocab, True, 3.0)
        rows = bf16_bits(x) if bf16 else x
        par = np.full(N, -1, np.int64)
        depth = np.zeros(N, np.int64)
        nchild = np.zeros(N, np.int64)
        for i in range(1, N):
            cand = [j for j in range(i) if depth[j] < max_depth and nchild[j] < max_branch]
            p = int(cand[int(s_tok.integers(0, len(cand)))])
            par[i] = p
            depth[i] = depth[p] + 1
            nchild[p] += 1
        tok = np.zeros(N, np.int64)
        tok[0] = s_tok.integers(0, vocab)
        for j in range(N):
            kids_j = [i for i in range(j + 1, N) if par[i] == j]
            if not kids_j:
                continue
            base = bf16_to_f32(rows[j]) if bf16 else rows[j]
            noisy = base + s_noise.standard_normal(vocab, dtype=np.float32)
            c = len(kids_j)
            kth = np.partition(noisy, vocab - c)[vocab - c]
            cand = np.flatnonzero(noisy >= kth)
            order = np.lexsort((cand, -noisy[cand]))
            for i, t in zip(kids_j, cand[order][:c]):
                tok[i] = int(t)
        sl = slice(b * N, (b + 1) * N)
        target[sl] = rows
        parents[sl] = par
        tokens[sl] = tok
        u_accept[sl] = s_unif.random(N, dtype=np.float32)
        u_final[b] = s_unif.random(dtype=np.float32)

    _pool_map(one, range(batch), parallel)
    return TreeWorkload("tree", vocab, batch, N, target, parents, tokens, u_accept, u_final, temperature,
                        meta={"seed": seed})


def verify_slots_for(total_rows: int, seed: int = 7) -> np.ndarray:
    """Synthetic KV slot ids of the verify rows (a shuffled range, int64)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.permutation(np.arange(10_000, 10_000 + 4 * total_rows, 4, dtype=np.int64))[:total_rows]


def seq_lens_for(batch: int, seed: int = 8) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(16, 4096, size=batch).astype(np.int32)


@dataclass
class PlannerInputs:
    conf: np.ndarray            # [R, W] float32 current confidences
    conf_hist: np.ndarray       # [R, W] float32 lagged confidences (the host budget's history)
    sps_rows: np.ndarray        # SPS table: target rows ...
    sps: np.ndarray             # ... and steps per second there
    raw_accept_len: np.ndarray  # [R] int32 accept lengths of a full-width verify (for the cutoff)


def planner_inputs(seed: int = 7000, batch: int = 512, width: int = 15) -> PlannerInputs:
    """Confidences for the verify-length planner at the ragged workload's shape (see the module recipe)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.beta(4.0, 1.5, batch)
    decay = 0.97 ** np.arange(width)
    conf = np.clip(q[:, None] * decay[None, :] + rng.normal(0, 0.05, (batch, width)), 0, 1).astype(np.float32)
    hist = np.clip(conf + rng.normal(0, 0.05, (batch, width)), 0, 1).astype(np.float32)
    raw = rng.integers(0, width + 1, batch).astype(np.int32)
    return PlannerInputs(conf, hist, np.array([512.0, 2048.0, 4096.0, 8192.0]), np.array([100.0, 95.0, 70.0, 35.0]),
                         raw)


@dataclass
class TreeRoundInputs:
    anchors: np.ndarray         # [B] int32
    draft_tokens: np.ndarray    # [B, S, k, k] int32
    draft_probs: np.ndarray     # [B, S, k, k] float32
    seq_lens: np.ndarray        # [B] int32
    n_nodes: int
    commit_offsets: np.ndarray  # [B+1] int32: accepted paths of the tree (commit lists)
    src_slots: np.ndarray       # int64
    dst_pos: np.ndarray         # int32
    req_to_token: np.ndarray    # [B, max_context] int64
    n_slots: int


def tree_round_inputs(seed: int = 8000, batch: int = 32, steps: int = 8, topk: int = 8, n_nodes: int = 64,
                      vocab: int = LLAMA3_VOCAB, context: int = 256) -> TreeRoundInputs:
    """The draft side and the commit side of a tree round at the EAGLE tree workload's shape (B 32, 64 nodes,
    topk 8, 8 steps): the draft's per-step top-k children with probabilities drawn as top-k slices of a
    Dirichlet(0.7) softmax, and accepted paths (a root plus U{0..4} increasing node ids) to move, with slots of
    a shuffled req_to_token table (context positions per request, nodes at seq_len + i)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    toks = rng.integers(0, vocab, (batch, steps, topk, topk)).astype(np.int32)
    probs = np.sort(rng.dirichlet(np.ones(topk) * 0.7, (batch, steps, topk)), axis=-1)[..., ::-1]
    probs = np.ascontiguousarray(probs, dtype=np.float32)
    anchors = rng.integers(0, vocab, batch).astype(np.int32)
    seq = rng.integers(16, context - n_nodes - 1, batch).astype(np.int32)
    n_slots = batch * context
    r2t = rng.permutation(n_slots).reshape(batch, context).astype(np.int64)
    offs, src, dst = [0], [], []
    for b in range(batch):
        r = int(rng.integers(0, 5))
        path = [0] + sorted(rng.choice(np.arange(1, n_nodes), r, replace=False).tolist())
        for k, node in enumerate(path):
            src.append(int(r2t[b, seq[b] + node]))
            dst.append(int(seq[b]) + k)
        offs.append(len(src))
    return TreeRoundInputs(anchors, toks, probs, seq, n_nodes, np.array(offs, np.int32), np.array(src, np.int64),
                           np.array(dst, np.int32), r2t, n_slots)


def block_sample(seed: int = 7000, batch: int = 32, block: int = 16, vocab: int = QWEN_VOCAB,
                 temperature: float = 1.0, parallel: bool = True) -> ChainWorkload:
    """DFlash-shaped sampling verify for sample-then-match: B 32, block 16 (anchor + 15 drafts), V 151,936,
    bf16 target rows 3 N(0,1) with one token raised by U(14, 20) (its probability at T = 1 then spans about
    0.1 .. 0.97, a peaked next-token distribution); the draft proposes that token with probability 0.8 and a
    uniform token otherwise. Uniforms U[0,1) float32 per row (u_accept for rows 0..14, u_final for row 15)."""
    kids = np.random.SeedSequence(seed).spawn(batch + 1)
    m = block - 1
    offsets = (np.arange(batch + 1) * block).astype(np.int32)
    T = batch * block
    target = np.empty((T, vocab), np.uint16)
    tokens = np.empty(batch * m, np.int32)
    u_acc = np.empty(batch * m, np.float32)
    u_fin = np.empty(batch, np.float32)

    def one(b):
        s_logit, s_tok, s_unif = [np.random.Generator(np.random.PCG64(s)) for s in kids[b + 1].spawn(3)]
        x = s_logit.standard_normal((block, vocab), dtype=np.float32) * np.float32(3.0)
        top = s_logit.integers(0, vocab, block)
        x[np.arange(block), top] += s_logit.uniform(14.0, 20.0, block).astype(np.float32)
        target[b * block:(b + 1) * block] = bf16_bits(x)
        pick = s_tok.random(m) < 0.8
        tokens[b * m:(b + 1) * m] = np.where(pick, top[:m], s_tok.integers(0, vocab, m))
        u_acc[b * m:(b + 1) * m] = s_unif.random(m, dtype=np.float32)
        u_fin[b] = s_unif.random(dtype=np.float32)

    _pool_map(one, range(batch), parallel)
    return ChainWorkload("block_sample", vocab, batch, offsets, target, None, tokens, u_acc, u_fin, temperature,
                         ("sample_match",), block, meta={"seed": seed})


def chain_keep(w) -> list:
    """Per target row of a chain workload, the tokens a grammar-like mask keeps allowed: the row's argmax and
    the draft token the row judges (a grammar admits what the model predicts, so acceptances still happen)."""
    keep = []
    for b in range(w.batch):
        lo, hi = int(w.offsets[b]), int(w.offsets[b + 1])
        for j in range(hi - lo):
            row = w.target[lo + j]
            ks = [int(np.argmax(bf16_to_f32(row) if row.dtype == np.uint16 else row))]
            if j < hi - lo - 1:
                ks.append(int(w.draft_tokens[lo - b + j]))
            keep.append(ks)
    return keep


def vocab_masks(seed: int, rows: int, vocab: int, allowed: float, keep=None) -> np.ndarray:
    """Grammar-like vocab masks: uint32 [rows, ceil(vocab/32)], token v of row i allowed iff bit v % 32 of word
    v // 32 is set. Each token is allowed with probability `allowed`; keep[i] (an int or a list of ints, -1
    ignored) lists tokens forced allowed in row i (a grammar usually admits what the model predicts)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    W = (vocab + 31) // 32
    out = np.empty((rows, W), np.uint32)
    for i in range(rows):
        bits = rng.random(W * 32, dtype=np.float32) < np.float32(allowed)
        bits[vocab:] = False
        if keep is not None:
            for k in np.atleast_1d(keep[i]):
                if 0 <= int(k) < vocab:
                    bits[int(k)] = True
        # little bit order: bit j of byte k is token 8k + j, so little-endian word w holds tokens 32w .. 32w+31
        out[i] = np.packbits(bits, bitorder="little").view("<u4")
    return out


# Full-size workloads (name -> builder); each builder's defaults are the full shapes.
FULL = {
    "tiny_chain": tiny_chain,
    "chain_rejection": chain_rejection,
    "block_greedy": block_greedy,
    "tree": tree,
    "ragged": ragged,
    "chain_sparse": chain_sparse,
    "block_sample": block_sample,
}
