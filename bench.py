#!/usr/bin/env python3
"""Throughput of the speculative-decoding verify -> accept -> commit hot path on one MI355X.

One step = one verify round of the timed workload (K steps captured into a HIP graph and timed as one replay;
then K eager steps from Python for reference, and K more with per-kernel HIP events): spec_verify_chain (every
target and draft logit row streamed once, accept scan, residual / bonus draw, outputs) with the KV commit
compaction fused into the same call (--commit separate: spec_commit_indices as its own launch), through the
C ABI. Inputs are synthetic, seeded and resident in HBM before timing; a
rotation of input sets keeps the live footprint above twice the 256 MB Infinity Cache so HBM, not the
cache, serves the stream.

Prints ONE JSON line. value = verified positions per second (target rows judged, sum_b (m_b + 1)).
roofline: the dominant kernel (k_stats, the logits stream) timed with HIP events that take its own start and
stop timestamps on the launch stream (hipExtLaunchKernel), against its algorithmic bytes (every target and
draft row read once); read_floor: a plain read of the same byte count (spec_read_probe) timed the same way,
the rate HBM actually delivers at this size. cpu_baseline: the fp64 CPU oracle timed on this host on the
same inputs, one thread pinned to one core; cpu_baseline_parallel: the same oracle with the requests split over
one forked process per core of this process's CPU share (at most 16, each pinned), both run before the GPU is
touched.

    python bench.py [--steps K] [--warmup W]
                    [--workload chain_rejection|block_greedy|tree|ragged|chain_sparse|block_sample|chain_rejection_masked]
                    [--no-extra] [--no-cpu-baseline] [--copy-calibration]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor peak
MALL_BYTES = 256 << 20         # Infinity Cache
METRIC = "verified draft positions/sec (bf16 logits, V=151936) and % of HBM peak"
DEFAULT_WORKLOAD = "chain_rejection"


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


# What the verify kernels (k_stats and the second kernel with the fused commit) are compiled from, with the
# build flags: counter summaries taken on other sources are not reused.
VERIFY_SOURCES = ("csrc/sv_stats.hip", "csrc/sv_draw.hip", "csrc/sv_match.hip", "csrc/sv_scan.h", "csrc/sv_fused.h",
                  "csrc/sv_device.h", "csrc/sv_internal.h", "csrc/sv_api.hip", "build.py")


def kernel_source_hash() -> str:
    """Hash of the verify kernels' sources and build flags."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "draft_verification_acceptance_amd")
    for f in VERIFY_SOURCES:
        with open(os.path.join(pkg, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------------------------------
# workloads on the device
# ----------------------------------------------------------------------------------------------------
def _dev_logits(a):
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def _dev(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _grammar_mask(w):
    """A grammar-like vocab mask for a chain workload: 5 % of the tokens allowed per target row, plus the
    row's argmax and the draft token it judges (a grammar admits what the model predicts)."""
    from draft_verification_acceptance_amd import workloads as W
    return W.vocab_masks(int(w.meta.get("seed", 0)) + 17, w.total_rows, w.vocab, 0.05, W.chain_keep(w))


def build_sets(name: str):
    """Seeded input sets (seed 1000*k + i) until the live footprint exceeds 2x the Infinity Cache.
    chain_rejection_masked: the chain_rejection sets with a grammar-like vocab mask per target row."""
    from draft_verification_acceptance_amd import workloads as W
    masked = name == "chain_rejection_masked"
    gen = "chain_rejection" if masked else name
    base = {"tiny_chain": 1000, "chain_rejection": 2000, "block_greedy": 3000, "tree": 4000, "ragged": 5000,
            "chain_sparse": 6000, "block_sample": 7000}[gen]
    sets = []
    total = 0
    i = 0
    while total <= 2 * MALL_BYTES or len(sets) < 2:
        w = W.FULL[gen](seed=base + i)
        w.meta["seed"] = base + i
        if masked:
            w.name = name
            w.meta["seed"] = base + i
            w.meta["vocab_mask"] = _grammar_mask(w)
        mode = w.modes[-1]
        sets.append(w)
        total += w.algorithmic_bytes(mode)
        i += 1
    return sets


class ChainStep:
    def __init__(self, w, mode, fused=True):
        import torch

        import draft_verification_acceptance_amd as dva
        from draft_verification_acceptance_amd import workloads as W
        self.w = w
        t = _dev_logits(w.target)
        offs = _dev(w.offsets)
        kw = dict(max_verify_len=w.max_verify_len)
        if mode == "rejection":
            kw.update(draft_logits=_dev_logits(w.draft), u_accept=_dev(w.u_accept), u_final=_dev(w.u_final),
                      temperature=w.temperature)
        elif mode == "rejection_sparse":
            kw.update(cand_ids=_dev(w.cand_ids), cand_q=_dev(w.cand_q), u_accept=_dev(w.u_accept),
                      u_final=_dev(w.u_final), temperature=w.temperature)
        elif mode == "sample_match":
            kw.update(u_accept=_dev(w.u_accept), u_final=_dev(w.u_final), temperature=w.temperature)
        mask = w.meta.get("vocab_mask")
        if mask is not None:
            kw.update(vocab_mask=_dev(mask.view("<i4")))
        slots, seq = _dev(W.verify_slots_for(w.total_rows)), _dev(W.seq_lens_for(w.batch))
        if fused:   # the KV commit inside the verify call
            self.verify = dva.prepare_verify_chain(t, offs, _dev(w.draft_tokens), mode, verify_slots=slots,
                                                   seq_lens=seq, **kw)
            self.commit = None
        else:
            self.verify = dva.prepare_verify_chain(t, offs, _dev(w.draft_tokens), mode, **kw)
            o = self.verify.outputs
            self.commit = dva.prepare_commit_indices(offs, o["accept_len"], o["accept_index"], slots, seq,
                                                     max_verify_len=w.max_verify_len)
        self.mode = mode
        self.positions = w.total_rows
        self.draft_positions = w.total_rows - w.batch
        self.bytes = w.algorithmic_bytes(mode) + (mask.nbytes if mask is not None else 0)
        torch.cuda.synchronize()

    def draw_bytes(self, accept_len) -> float:
        """Logit bytes the second kernel reads by design for these results (row partials aside): rejection, the
        target and draft rows of the rejected slot (one target row when every draft is accepted; sparse q, that
        row's candidate pairs instead of a draft row); sample-then-match, one 2048-token piece of every row
        drawn (rows go in groups of 16 up to the group holding the first mismatch); greedy, none."""
        import numpy as np
        w = self.w
        mask = w.meta.get("vocab_mask")
        row = w.vocab * w.target.itemsize
        row_t = row + (mask.shape[1] * mask.itemsize if mask is not None else 0)   # with its mask words
        n_draft = np.diff(w.offsets.astype(np.int64)) - 1
        a = np.asarray(accept_len, np.int64)
        rejected = a < n_draft
        if self.mode == "rejection":
            return float(w.batch * row_t + np.count_nonzero(rejected) * row)
        if self.mode == "rejection_sparse":
            pair = w.cand_ids.shape[1] * (w.cand_ids.itemsize + w.cand_q.itemsize)
            return float(w.batch * row_t + np.count_nonzero(rejected) * pair)
        if self.mode == "sample_match":
            drawn = np.minimum(n_draft + 1, (a // 16 + 1) * 16)
            return float(np.sum(drawn) * min(row, 2048 * w.target.itemsize))
        return 0.0


class TreeStep:
    def __init__(self, w, mode, fused=True):
        import numpy as np
        import torch

        import draft_verification_acceptance_amd as dva
        from draft_verification_acceptance_amd import workloads as W
        self.w = w
        kw = {}
        if mode == "target_only":
            kw = dict(u_accept=_dev(w.u_accept), u_final=_dev(w.u_final), temperature=w.temperature)
        slots, seq = _dev(W.verify_slots_for(w.total_rows)), _dev(W.seq_lens_for(w.batch))
        if fused:
            kw.update(verify_slots=slots, seq_lens=seq)
        self.verify = dva.prepare_verify_tree(_dev_logits(w.target), _dev(w.parents), _dev(w.tokens), w.n_nodes, mode,
                                              **kw)
        self.commit = None
        if not fused:
            o = self.verify.outputs
            offs = _dev((np.arange(w.batch + 1) * w.n_nodes).astype(np.int32))
            self.commit = dva.prepare_commit_indices(offs, o["accept_len"], o["accept_index"], slots, seq,
                                                     max_verify_len=w.n_nodes)
        self.mode = mode
        self.positions = w.total_rows
        self.draft_positions = w.total_rows - w.batch
        self.bytes = w.algorithmic_bytes(mode)
        torch.cuda.synchronize()

    def draw_bytes(self, accept_len) -> float:
        """Logit bytes the second kernel reads by design (row partials aside): target_only, the one target row
        each request draws from (the residual at the node where it stopped, or the bonus row); greedy, none."""
        w = self.w
        return float(w.batch * w.vocab * w.target.itemsize) if self.mode == "target_only" else 0.0


def run_workload(name: str, mode: str | None, steps: int, warmup: int, fused: bool = True) -> dict:
    import numpy as np
    import torch

    import draft_verification_acceptance_amd as dva
    t0 = time.time()
    sets = build_sets(name)
    mode = mode or sets[0].modes[-1]
    kind = "tree" if name == "tree" else "chain"
    st = [(TreeStep if kind == "tree" else ChainStep)(w, mode, fused) for w in sets]

    def step(s, ev_v=None, ev_c=None):
        s.verify.run(ev_v)
        if s.commit is not None:
            s.commit.run(ev_c)
    _log(f"[bench] {name}/{mode}: {len(sets)} input sets, {sum(s.bytes for s in st) / 1e6:.0f} MB live, "
         f"setup {time.time() - t0:.1f}s")
    nk = dva.kernel_count(kind, mode)
    ev_v = [dva.HipEvents(2 * nk) for _ in range(steps)]   # start / stop of each kernel
    ev_c = [dva.HipEvents(2) for _ in range(steps)]
    for i in range(warmup):
        step(st[i % len(st)])
    torch.cuda.synchronize()
    # The K timed steps are captured once into a HIP graph (the library launches only kernels on the
    # caller's stream: no allocation, memset or synchronisation) and replayed with one host launch, so the
    # GPU, not Python and the launch path, sets the pace. One untimed replay first.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            step(st[i % len(st)])
    graph.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t1
    # The same steps issued eagerly from Python (host launch path included), for reference.
    t2 = time.perf_counter()
    for i in range(steps):
        step(st[i % len(st)])
    torch.cuda.synchronize()
    wall_eager = time.perf_counter() - t2
    del graph
    # Same steps again with HIP events taking each kernel's start / stop timestamps (per-kernel durations).
    for i in range(steps):
        step(st[i % len(st)], ev_v[i], ev_c[i])
    torch.cuda.synchronize()
    k_stats = np.array([e.elapsed_ms(0, 1) for e in ev_v])
    k_draw = np.array([e.elapsed_ms(2, 3) for e in ev_v]) if nk > 1 else np.zeros(steps)
    k_commit = np.array([e.elapsed_ms(0, 1) for e in ev_c]) if not fused else None
    verify_ms = k_stats + k_draw
    positions = np.mean([st[i % len(st)].positions for i in range(steps)])
    draft_positions = np.mean([st[i % len(st)].draft_positions for i in range(steps)])
    nbytes = np.mean([st[i % len(st)].bytes for i in range(steps)])
    # Sanity of the last results (no data faults in these synthetic inputs), and the device's own count of
    # decisions too close to call on the canonical input set (set 0, re-run eagerly).
    stat = st[(steps - 1) % len(st)].verify.outputs["status"].cpu().numpy().view(np.uint32)
    bad = int(np.count_nonzero(stat & ~np.uint32(dva.ST.NEAR_ALPHA | dva.ST.NEAR_CDF)))
    acc = st[(steps - 1) % len(st)].verify.outputs["accept_len"].float().mean().item()
    # Every set's outputs hold its last eager run: the second kernel's by-design logit bytes per step.
    draw_nbytes = np.mean([st[i % len(st)].draw_bytes(st[i % len(st)].verify.outputs["accept_len"].cpu().numpy())
                           for i in range(steps)])
    step(st[0])
    torch.cuda.synchronize()
    st0 = st[0].verify.outputs["status"].cpu().numpy().view(np.uint32)
    near = {"requests": int(st0.size), "near_alpha": int(np.count_nonzero(st0 & np.uint32(dva.ST.NEAR_ALPHA))),
            "near_cdf": int(np.count_nonzero(st0 & np.uint32(dva.ST.NEAR_CDF))),
            "flagged": int(np.count_nonzero(st0 & np.uint32(dva.ST.NEAR_ALPHA | dva.ST.NEAR_CDF))),
            "input_set_seed": int(sets[0].meta["seed"])}
    ms_step = wall * 1e3 / steps
    stats_ms = float(np.mean(k_stats))
    return {
        "workload": name, "mode": mode, "batch": sets[0].batch, "vocab": sets[0].vocab,
        "verify_positions_per_step": float(positions), "draft_positions_per_step": float(draft_positions),
        "algorithmic_bytes_per_step": float(nbytes), "draw_logit_bytes_per_step": float(draw_nbytes),
        "rotation_sets": len(sets),
        "ms_per_step": ms_step,
        "ms_per_step_eager": wall_eager * 1e3 / steps,
        "positions_per_s": positions / (ms_step * 1e-3),
        "draft_positions_per_s": draft_positions / (ms_step * 1e-3),
        "step_hbm_fraction": nbytes / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "kernel_ms": {"k_stats": {"mean": stats_ms, "p10": float(np.percentile(k_stats, 10)),
                                  "p50": float(np.median(k_stats)), "p90": float(np.percentile(k_stats, 90))},
                      "k_draw": float(np.mean(k_draw)),
                      "k_commit": float(np.mean(k_commit)) if k_commit is not None else "fused into k_draw / k_scan",
                      "verify_kernels_p50": float(np.median(verify_ms))},
        "commit": "fused" if fused else "separate launch",
        "device_flags": near,
        "stats_kernel_gbs": nbytes / (stats_ms * 1e-3) / 1e9,
        "mean_accept_len": acc,
        "status_faults": bad,
    }


def run_planner(steps: int) -> dict:
    """The verify-length planner at the ragged workload's shape (512 requests x 15 proposed drafts): the host
    budget from lagged confidences and a synthetic SPS table, the device allocation kernel, and the accept
    cutoff of a full-width verify. Latency-bound work (30 KB of confidences): times, not bandwidth."""
    import numpy as np
    import torch

    import draft_verification_acceptance_amd as dva
    from draft_verification_acceptance_amd import workloads as W
    w = W.planner_inputs()
    t0 = time.perf_counter()
    reps = 50
    for _ in range(reps):
        K, theta = dva.plan_budget(w.conf_hist, w.sps_rows, w.sps)
    host_us = (time.perf_counter() - t0) / reps * 1e6
    conf = torch.from_numpy(w.conf).cuda()
    plan = dva.prepare_plan_layout(conf, budget=K)
    R, Wd = w.conf.shape
    offs = torch.arange(0, (R + 1) * (Wd + 1), Wd + 1, dtype=torch.int32, device="cuda")
    raw = torch.from_numpy(w.raw_accept_len).cuda()
    toks = torch.zeros(R * (Wd + 1), dtype=torch.int32, device="cuda")
    trim = dva.prepare_cap_trim(offs, plan.outputs["verify_lens"], raw, raw.clone(), toks)
    for _ in range(10):
        plan.run()
        trim.run()
    torch.cuda.synchronize()
    ev_p = [dva.HipEvents(2) for _ in range(steps)]
    ev_t = [dva.HipEvents(2) for _ in range(steps)]
    for i in range(steps):
        plan.run(ev_p[i])
        trim.run(ev_t[i])
    torch.cuda.synchronize()
    kp = np.array([e.elapsed_ms(0, 1) for e in ev_p]) * 1e3
    kt = np.array([e.elapsed_ms(0, 1) for e in ev_t]) * 1e3
    vl = plan.outputs["verify_lens"].cpu().numpy()
    return {"requests": int(R), "proposed_drafts": int(R * Wd), "budget": int(K),
            "target_rows_planned": int(vl.sum()), "host_budget_us": host_us,
            "plan_kernel_us": {"mean": float(kp.mean()), "p50": float(np.median(kp))},
            "cap_trim_kernel_us": {"mean": float(kt.mean()), "p50": float(np.median(kt))},
            "bound": "latency (one workgroup; 30 KB of confidences)"}


def run_tree_round(steps: int) -> dict:
    """The steps on either side of a tree verify at the EAGLE tree workload's shape: draft-tree construction
    (B 32, topk 8, 8 steps: 456 candidates -> 64 nodes) and the KV data move of the accepted paths over 64
    KV buffers of 2 KB rows (K and V of 32 layers x 8 KV heads x 128 dims, bf16: a Llama-3-8B-sized cache).
    Tree build is latency work; the move's bytes are 2 x moved rows x 2 KB x 64 buffers."""
    import numpy as np
    import torch

    import draft_verification_acceptance_amd as dva
    from draft_verification_acceptance_amd import workloads as W
    w = W.tree_round_inputs()
    d = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    build = dva.prepare_tree_build(d(w.anchors), d(w.draft_tokens), d(w.draft_probs), d(w.seq_lens), w.n_nodes)
    n_buf, row_elems = 64, 1024
    bufs = [torch.empty((w.n_slots, row_elems), dtype=torch.bfloat16, device="cuda").normal_() for _ in range(n_buf)]
    move = dva.prepare_kv_move(bufs, d(w.commit_offsets), d(w.src_slots), d(w.dst_pos), d(w.req_to_token),
                               d(np.arange(len(w.anchors), dtype=np.int32)))
    for _ in range(10):
        build.run()
        move.run()
    torch.cuda.synchronize()
    eb = [dva.HipEvents(2) for _ in range(steps)]
    em = [dva.HipEvents(2) for _ in range(steps)]
    for i in range(steps):
        build.run(eb[i])
        move.run(em[i])
    torch.cuda.synchronize()
    kb = np.array([e.elapsed_ms(0, 1) for e in eb]) * 1e3
    km = np.array([e.elapsed_ms(0, 1) for e in em]) * 1e3
    moved = int(np.count_nonzero(w.src_slots != w.req_to_token[np.repeat(np.arange(len(w.anchors)),
                                                                         np.diff(w.commit_offsets)), w.dst_pos]))
    move_bytes = 2 * moved * row_elems * 2 * n_buf
    del bufs
    torch.cuda.empty_cache()
    return {"tree_build": {"requests": len(w.anchors), "candidates": int(8 + 7 * 64), "nodes": w.n_nodes,
                           "kernel_us": {"mean": float(kb.mean()), "p50": float(np.median(kb))},
                           "bound": "latency (one workgroup per request)"},
            "kv_move": {"commit_entries": int(w.src_slots.size), "rows_moved": moved, "buffers": n_buf,
                        "row_bytes": row_elems * 2, "bytes": move_bytes,
                        "kernel_us": {"mean": float(km.mean()), "p50": float(np.median(km))},
                        "gbs": move_bytes / (float(km.mean()) * 1e-6) / 1e9,
                        "bound": "hbm copy, latency-bound at this size"}}


def cpu_baseline(name: str, budget_s: float = 12.0) -> dict:
    """The fp64 oracle in this process, one thread, on the canonical input set of the timed workload (used for
    the tree workload; chains get the pinned runs of cpu_baselines)."""
    import numpy as np

    import oracle
    from draft_verification_acceptance_amd import workloads as W
    w = W.FULL[name](seed={"chain_rejection": 2000, "block_greedy": 3000, "tree": 4000, "ragged": 5000,
                           "chain_sparse": 6000}[name])
    mode = w.modes[-1]
    slots = W.verify_slots_for(w.total_rows)
    seq = W.seq_lens_for(w.batch)
    passes = 0
    rows = 0
    t0 = time.perf_counter()
    while True:
        if name == "tree":
            o = oracle.verify_tree(w.target, w.parents, w.tokens, w.n_nodes, mode, u_accept=w.u_accept,
                                   u_final=w.u_final, temperature=w.temperature)
            offs = np.arange(w.batch + 1) * w.n_nodes
            oracle.commit_indices(offs, o["accept_len"], o["accept_index"], slots, seq, w.n_nodes)
        else:
            o = oracle.verify_chain(w.target, w.offsets, w.draft_tokens, mode, draft=w.draft, u_accept=w.u_accept,
                                    u_final=w.u_final, temperature=w.temperature, max_verify_len=w.max_verify_len,
                                    cand_ids=w.cand_ids, cand_q=w.cand_q)
            oracle.commit_indices(w.offsets, o["accept_len"], o["accept_index"], slots, seq, w.max_verify_len)
        passes += 1
        rows += w.total_rows
        if time.perf_counter() - t0 >= budget_s or passes >= 20:
            break
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} full pass(es) over one input set of the timed workload ({w.batch} requests, "
                      f"{w.total_rows} verify rows, fp64 numpy, one thread) incl. commit; {dt:.1f} s"}


_PAR = {}   # the workload the forked oracle workers split (set before the pool forks)


def _oracle_requests(args):
    """One worker of the oracle runs: pinned to one CPU, full passes over requests [b0, b1) of the chain
    workload in _PAR until the time budget (at most max_passes), verify + commit."""
    import numpy as np

    import oracle
    from draft_verification_acceptance_amd import workloads as W
    b0, b1, budget_s, cpu, max_passes = args
    os.sched_setaffinity(0, {cpu})
    w, mode = _PAR["w"], _PAR["mode"]
    off = w.offsets
    r0, r1 = int(off[b0]), int(off[b1])
    d0, d1 = r0 - b0, r1 - b1
    offs = (off[b0:b1 + 1] - r0).astype(np.int32)
    sl = lambda a, lo, hi: None if a is None else a[lo:hi]
    slots = W.verify_slots_for(r1 - r0)
    seq = W.seq_lens_for(b1 - b0)
    rows = passes = 0
    t0 = time.perf_counter()
    while True:
        o = oracle.verify_chain(w.target[r0:r1], offs, w.draft_tokens[d0:d1], mode, draft=sl(w.draft, d0, d1),
                                u_accept=w.u_accept[d0:d1], u_final=w.u_final[b0:b1], temperature=w.temperature,
                                max_verify_len=w.max_verify_len, cand_ids=sl(w.cand_ids, d0, d1),
                                cand_q=sl(w.cand_q, d0, d1))
        oracle.commit_indices(offs, o["accept_len"], o["accept_index"], slots, seq, w.max_verify_len)
        passes += 1
        rows += r1 - r0
        if time.perf_counter() - t0 >= budget_s or passes >= max_passes:
            break
    return rows, time.perf_counter() - t0, passes


def cpu_baselines(name: str, budget_single: float = 8.0, budget_par: float = 8.0):
    """The fp64 oracle on this host, on the canonical input set of the timed workload (a chain workload):
    (single, parallel). single: one forked worker pinned to one core, repeated full passes over all
    requests (verify + commit). parallel: the requests split evenly over one forked worker per core of this
    process's CPU share (at most 16), each pinned to its own core and repeating full passes over its
    requests; value = the sum of the workers' rates. Call it before this process touches the GPU (the
    workers are forks of it)."""
    import multiprocessing as mp

    from draft_verification_acceptance_amd import workloads as W
    seeds = {"chain_rejection": 2000, "block_greedy": 3000, "ragged": 5000, "chain_sparse": 6000}
    if name not in seeds:
        return None, None
    w = W.FULL[name](seed=seeds[name])
    cpus = sorted(os.sched_getaffinity(0))
    n = max(1, min(16, len(cpus), w.batch))
    _PAR["w"], _PAR["mode"] = w, w.modes[-1]
    ctx = mp.get_context("fork")
    with ctx.Pool(1) as pool:
        # the last CPU of the share: CPU 0 also serves the system, which halved the rate there
        rows, dt, passes = pool.map(_oracle_requests, [(0, w.batch, budget_single, cpus[-1], 20)])[0]
    cuts = [round(i * w.batch / n) for i in range(n + 1)]
    with ctx.Pool(n) as pool:
        res = pool.map(_oracle_requests, [(cuts[i], cuts[i + 1], budget_par, cpus[i], 1 << 30) for i in range(n)])
    _PAR.clear()
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    single = {"value": rows / dt, "unit": "positions/s", "cores": 1, "kind": "oracle", "cpu": model,
              "sample": f"{passes} full pass(es) over one input set of the timed workload ({w.batch} requests, "
                        f"{w.total_rows} verify rows, fp64 numpy, one thread pinned to one core) incl. commit; "
                        f"{dt:.1f} s"}
    par = {"value": sum(r / t for r, t, _ in res), "unit": "positions/s", "cores": n, "kind": "oracle",
           "cpu": model,
           "sample": f"{n} forked workers pinned to one core each, requests split evenly over them, each "
                     f"repeating full passes over its requests (fp64 numpy, one thread each) incl. commit for "
                     f"~{budget_par:.0f} s; value = sum of the workers' rates"}
    return single, par


def load_traffic(name: str, mode: str):
    """HBM bytes per launch of the verify kernels for one workload, from its committed rocprofv3 counter summary
    (profiles/traffic_<workload>_<mode>.txt), if the counters were taken on the current kernel sources; None
    otherwise."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}_{mode}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or ":" not in line:
                continue
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_hash") != kernel_source_hash():
        return None
    return {"k_stats_hbm_bytes_per_launch": float(vals["k_stats_hbm_bytes_per_launch"]),
            "k_stats_ratio_to_algorithmic": float(vals["k_stats_ratio_to_algorithmic"]),
            "second_kernel": vals["second_kernel"],
            "second_kernel_hbm_bytes_per_launch": float(vals["second_kernel_hbm_bytes_per_launch"]),
            "source": os.path.relpath(path, ROOT)}


def read_floor(nbytes: int, reps: int = 20) -> dict:
    """This GPU's achievable HBM read rate at the stream's size: spec_read_probe (a plain read, 16-byte loads)
    over nbytes, alternating between two buffers of that size as the timed step alternates its input sets (so
    the 256 MB cache serves neither), each launch timed by events on its own dispatch like the verify
    kernels."""
    import torch
    import draft_verification_acceptance_amd as dva
    n = nbytes // 16 * 16
    bufs = [torch.full((n,), i + 1, dtype=torch.uint8, device="cuda") for i in range(2)]
    sink = torch.zeros(dva.READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    for i in range(4):
        dva.read_probe(bufs[i % 2], sink)
    evs = [dva.HipEvents(2) for _ in range(reps)]
    for i in range(reps):
        dva.read_probe(bufs[i % 2], sink, events=evs[i])
    torch.cuda.synchronize()
    ms = sum(e.elapsed_ms(0, 1) for e in evs) / reps
    del bufs
    torch.cuda.empty_cache()
    return {"kernel": "k_read_fold", "bytes": n, "avg_launch_ms": ms, "gbs": n / (ms * 1e-3) / 1e9, "launches": reps}


def copy_calibration():
    """A plain copy of known size, for scaling rocprofv3's FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=["chain_rejection", "block_greedy", "tree", "ragged", "chain_sparse", "block_sample",
                             "chain_rejection_masked"])
    ap.add_argument("--mode", default=None)
    ap.add_argument("--no-extra", action="store_true", help="skip the other full-size workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--commit", choices=["fused", "separate"], default="fused",
                    help="the KV commit inside the verify call (default) or as its own spec_commit_indices launch")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the verify path shards by request with no exchange, so N GPUs "
              "would each run this same step on B/N requests; N > 1 is not run.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    # The oracle runs fork their workers, so they go before anything in this process touches the GPU.
    cpu, cpu_par = (None, None) if args.no_cpu_baseline else cpu_baselines(args.workload)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    fused = args.commit == "fused"
    main_res = run_workload(args.workload, args.mode, args.steps, args.warmup, fused)
    extra = {}
    if not args.no_extra:
        for name, mode in (("block_greedy", None), ("ragged", None), ("tree", "greedy"), ("tree", "target_only"),
                           ("chain_sparse", None), ("block_sample", None), ("chain_rejection_masked", "rejection")):
            if name == args.workload and (mode or "") == (args.mode or ""):
                continue
            r = run_workload(name, mode, max(50, args.steps // 2), args.warmup, fused)
            e = {k: r[k] for k in ("verify_positions_per_step", "ms_per_step", "ms_per_step_eager",
                                   "positions_per_s", "step_hbm_fraction", "stats_kernel_gbs", "kernel_ms",
                                   "algorithmic_bytes_per_step", "draw_logit_bytes_per_step", "mean_accept_len",
                                   "status_faults", "device_flags", "commit")}
            e["traffic"] = load_traffic(name, r["mode"])
            extra[f"{name}/{r['mode']}"] = e
            torch.cuda.empty_cache()
        extra["planner"] = run_planner(max(50, args.steps // 2))
        extra["tree_round"] = run_tree_round(max(50, args.steps // 2))
    stats_ms = main_res["kernel_ms"]["k_stats"]["mean"]
    achieved = main_res["stats_kernel_gbs"]
    if cpu is None and not args.no_cpu_baseline and args.workload == "tree":
        cpu = cpu_baseline("tree")
    traffic = load_traffic(main_res["workload"], main_res["mode"])
    floor = read_floor(int(main_res["algorithmic_bytes_per_step"]))
    line = {
        "metric": METRIC,
        "value": main_res["positions_per_s"],
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "ms_per_step_eager": main_res["ms_per_step_eager"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, shaped like the pages' workloads)",
        "config": {"workload": f"{main_res['workload']}: B {main_res['batch']}, V {main_res['vocab']}, "
                               f"{main_res['mode']}, {main_res['verify_positions_per_step']:.0f} verify rows/step",
                   "mode": main_res["mode"], "batch": main_res["batch"], "vocab": main_res["vocab"],
                   "verify_positions_per_step": main_res["verify_positions_per_step"],
                   "draft_positions_per_step": main_res["draft_positions_per_step"],
                   "rotation_sets": main_res["rotation_sets"], "parallelism": "none (one GPU)"},
        "draft_positions_per_s": main_res["draft_positions_per_s"],
        "step_hbm_fraction": main_res["step_hbm_fraction"],
        "roofline": {"bound": "hbm", "kernel": "k_stats", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic["k_stats_hbm_bytes_per_launch"] if traffic else None,
                     "traffic_detail": traffic,
                     "algorithmic_bytes_per_launch": main_res["algorithmic_bytes_per_step"],
                     "draw_logit_bytes_per_launch": main_res["draw_logit_bytes_per_step"],
                     "avg_launch_ms": stats_ms,
                     "read_floor": dict(floor, frac=achieved / floor["gbs"])},
        "kernel_ms": main_res["kernel_ms"],
        "commit": main_res["commit"],
        "device_flags": main_res["device_flags"],
        "mean_accept_len": main_res["mean_accept_len"],
        "status_faults": main_res["status_faults"],
        "cpu_baseline": cpu,
        "cpu_baseline_parallel": cpu_par,
        "other_workloads": extra,
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
