#!/usr/bin/env python3
"""Benchmark of the batched draft-verification sampler on one MI355X.

Workload (one step = one exact verification call over one batch):
    B=32 requests, K=5 drafts, V=128256, bf16 logits; target 3*N(0,1), draft
    = target + 0.5*N(0,1), drafts sampled from the draft softmax, seeded fp32
    uniforms.  Inputs are resident in HBM before timing starts.

The timed loop rotates through enough distinct copies of the inputs that
their total size is at least twice the 256 MB last-level cache (MALL), so
logits are streamed from HBM, not from that cache.  The K timed calls are
captured into one HIP graph and replayed once between two events (launches
then cost no host time); the same loop run eagerly is reported alongside.

The exact call is one kernel launch (k_single).  Its duration is measured
with HIP start/stop events that its dispatch timestamps itself
(spec_verify_profile_next_call) over K further calls; the call's algorithmic
bytes (every logit read once, plus tokens, uniforms and outputs) divided by
that duration give the roofline figure.  The streaming kernel alone (k_stream,
no sweep or draw) is also timed back to back, as the floor under the
launch's streaming phase.  With the CPU leg on (the default), the outputs of
every timed workload are checked against the fp64 oracle on the same inputs
(mismatches, near-tie flags per decision, largest log-prob difference, mean
accepted length), and the oracle is timed on a bounded sample of the
benchmark batch on the host's cores.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-configs]
    python bench.py --copy-calibration     # plain 1 GiB device copy, for counters
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
POWER_ALPHA = 0.5  # exponent of the power-rule measurement
KERNEL_SRC = os.path.join(ROOT, "draft_verification_row_amd", "csrc", "spec_verify.hip")

# HBM traffic of one exact call's kernel dispatch (k_single) on this workload,
# from two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch,
# averaged over dispatches), scaled by what the same counters read for a
# plain 1 GiB device copy (FETCH_SIZE reads half the bytes, WRITE_SIZE all).
# Reported only while the kernel source file is the one the counters were
# taken on.
TRAFFIC = {"source_sha256": "1441fcbf327bf14362ce38490cafb7b69319bf392be1f853689cfe224b2212b9",
           "fetch_kib": 50959.9, "write_kib": 1120.3, "fetch_scale": 2.0, "write_scale": 1.0}

MALL_BYTES = 256 * 1024 * 1024
# What the profiling hook's start/stop events bracket in each entry point.
KERNEL_TIMED = {"exact": "k_single: the whole call (one launch)",
                "power": "k_single: the whole call (one launch)",
                "relaxed": "k_single: the whole call (one launch)",
                "greedy": "k_greedy: the whole call (one launch)",
                "sample": "k_sample_rows: the whole call (one launch)",
                "tree": "k_tree: the whole call (one launch)"}
RUNS = 3  # timed replays of the captured steps; the median is reported
METRIC = "verify rounds/s + achieved HBM GB/s (% of peak), B=32 K=5 V=128256 bf16"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-graph", action="store_true", help="time the eager loop only")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (greedy B=8, tree, relaxed/exact B=64)")
    return ap.parse_args()


class Hip:
    """The few HIP runtime calls used for event timing."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
        return e

    def elapsed_ms(self, a, b) -> float:
        assert self.lib.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)

    def destroy(self, e):
        self.lib.hipEventDestroy(e)


def copy_calibration():
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    reps = 5
    t0.record()
    for _ in range(reps):
        y.copy_(x)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "reps": reps,
                      "ms_per_copy": ms, "gbs_read_plus_write": 2 * n / ms / 1e6}))


class Case:
    """Resident input sets and prebuilt C-call arguments for one entry point.

    mode: exact, power, greedy or relaxed (chain inputs), sample (the draft
    rows of chain inputs), tree (tree inputs)."""

    def __init__(self, lib, mode, ci, sets, torch, dev):
        import draft_verification_row_amd as sv
        from numpy import int16
        self.lib, self.mode, self.ci, self.sets = lib, mode, ci, sets
        self.torch = torch

        def logits(a):
            return torch.from_numpy(a.view(int16)).view(torch.bfloat16).to(dev)

        def i32(shape):
            return torch.empty(shape, dtype=torch.int32, device=dev)

        def f32(shape):
            return torch.empty(shape, dtype=torch.float32, device=dev)

        self.inputs, self.outputs = [], []
        if mode == "tree":
            B, N, V = ci.B, ci.N, ci.V
            T0 = logits(ci.target)
            small = [torch.from_numpy(a).to(dev) for a in (ci.node_tok, ci.parents, ci.num_nodes)]
            self.ws = torch.zeros(sv.spec_verify_workspace_bytes(B, N, V), dtype=torch.uint8,
                                  device=dev)
            for s in range(sets):
                self.inputs.append((T0.clone(), *[a.clone() for a in small]))
                self.outputs.append(dict(path=i32((B, N)), tok=i32((B, N)), ln=i32(B), st=i32(B)))
            del T0
            return
        B, K, V = ci.B, ci.K, ci.V
        T0 = logits(ci.draft if mode == "sample" else ci.target)
        D0 = logits(ci.draft) if mode in ("exact", "power") else None
        x0 = torch.from_numpy(ci.tokens).to(dev)
        u0 = torch.from_numpy(ci.uniforms).to(dev)
        if mode == "sample":
            u0 = torch.from_numpy(ci.uniforms[:, :K].copy()).to(dev)
            nbytes = sv.spec_sample_workspace_bytes(B * K, V)
        else:
            rows = 2 * K + 1 if mode in ("exact", "power") else K + 1
            nbytes = sv.spec_verify_workspace_bytes(B, rows, V)
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        for s in range(sets):
            D = D0.clone() if D0 is not None else None
            self.inputs.append((T0.clone(), D, x0.clone(), u0.clone()))
            if mode == "sample":
                self.outputs.append(dict(tok=i32((B, K)), lq=f32((B, K)), st=i32((B, K))))
                continue
            out = dict(tok=i32((B, K + 1)), ln=i32(B), st=i32(B))
            if mode in ("exact", "power", "relaxed"):
                out["tlp"] = f32((B, K + 1))
                out["blp"] = f32((B, K + 1))
            self.outputs.append(out)
        del T0, D0

    def args(self, s, stream):
        P = ctypes.c_void_p
        o = self.outputs[s]
        ws = self.ws
        if self.mode == "tree":
            B, N, V = self.ci.B, self.ci.N, self.ci.V
            T, nt, par, nn = self.inputs[s]
            return (P(T.data_ptr()), 1, P(nt.data_ptr()), P(par.data_ptr()), P(nn.data_ptr()), B,
                    N, V, P(o["path"].data_ptr()), P(o["tok"].data_ptr()), P(o["ln"].data_ptr()),
                    None, None, P(o["st"].data_ptr()), P(ws.data_ptr()), ws.numel(), P(stream))
        B, K, V = self.ci.B, self.ci.K, self.ci.V
        T, D, x, u = self.inputs[s]
        if self.mode == "sample":
            return (P(T.data_ptr()), 1, P(u.data_ptr()), B * K, V, P(o["tok"].data_ptr()),
                    P(o["lq"].data_ptr()), P(o["st"].data_ptr()), P(ws.data_ptr()), ws.numel(),
                    P(stream))
        tail = (P(o["st"].data_ptr()), P(ws.data_ptr()), ws.numel(), P(stream))
        if self.mode == "greedy":
            return (P(T.data_ptr()), 1, P(x.data_ptr()), B, K, V, P(o["tok"].data_ptr()),
                    P(o["ln"].data_ptr()), None, None) + tail
        outs = (P(o["tok"].data_ptr()), P(o["ln"].data_ptr()), P(o["tlp"].data_ptr()),
                P(o["blp"].data_ptr()))
        if self.mode == "relaxed":
            return ((P(T.data_ptr()), 1, P(x.data_ptr()), P(u.data_ptr()), B, K, V,
                     ctypes.c_float(self.ci.tau), self.ci.top_k) + outs + tail)
        if self.mode == "power":
            return ((P(T.data_ptr()), P(D.data_ptr()), 1, P(x.data_ptr()), P(u.data_ptr()), B, K,
                     V, ctypes.c_float(POWER_ALPHA)) + outs + tail)
        return ((P(T.data_ptr()), P(D.data_ptr()), 1, P(x.data_ptr()), P(u.data_ptr()), B, K, V) +
                outs + tail)

    def fn(self):
        return {"exact": self.lib.spec_verify_exact, "greedy": self.lib.spec_verify_greedy,
                "relaxed": self.lib.spec_verify_relaxed, "tree": self.lib.spec_verify_tree,
                "sample": self.lib.spec_sample_drafts, "power": self.lib.spec_verify_power}[self.mode]

    def run(self, n, start=0, stream=None):
        torch = self.torch
        st = stream if stream is not None else torch.cuda.current_stream().cuda_stream
        f = self.fn()
        argv = [self.args(s, st) for s in range(self.sets)]
        for i in range(start, start + n):
            rc = f(*argv[i % self.sets])
            if rc != 0:
                raise RuntimeError(f"{self.mode} call failed with status {rc}")

    def snapshot(self):
        return [{k: v.clone() for k, v in o.items()} for o in self.outputs]


def time_case(case, steps, warmup, hip, use_graph):
    import torch
    case.run(warmup)
    torch.cuda.synchronize()
    res = {}
    # eager loop
    a, b = hip.event(), hip.event()
    stream = torch.cuda.current_stream().cuda_stream
    hip.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    torch.cuda.synchronize()
    hip.lib.hipEventRecord(a, ctypes.c_void_p(stream))
    case.run(steps, stream=stream)
    hip.lib.hipEventRecord(b, ctypes.c_void_p(stream))
    torch.cuda.synchronize()
    res["eager_ms_per_step"] = hip.elapsed_ms(a, b) / steps
    eager_out = case.snapshot()
    res["outputs"] = eager_out
    # graph replay of exactly `steps` calls
    if use_graph:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            case.run(steps, stream=torch.cuda.current_stream().cuda_stream)
        g.replay()  # untimed: first replay uploads the graph
        torch.cuda.synchronize()
        runs = []
        for _ in range(RUNS):
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0.record()
            g.replay()
            t1.record()
            torch.cuda.synchronize()
            runs.append(t0.elapsed_time(t1) / steps)
        res["graph_ms_per_step"] = sorted(runs)[len(runs) // 2]
        res["graph_ms_per_step_runs"] = runs
        # the timed replays must reproduce the eager results bit for bit
        res["outputs"] = case.snapshot()
        for o1, o2 in zip(eager_out, res["outputs"]):
            for k in o1:
                if not torch.equal(o1[k], o2[k]):
                    raise RuntimeError(f"graph replay output {k} differs from the eager call")
        del g
    # per-kernel durations through the library's event hook: the streaming
    # kernel's own start/stop timestamps, and the rest of the call
    evs = [(hip.event(), hip.event(), hip.event()) for _ in range(steps)]
    f = case.fn()
    argv = [case.args(s, stream) for s in range(case.sets)]
    torch.cuda.synchronize()
    for i in range(steps):
        case.lib.spec_verify_profile_next_call(*evs[i])
        assert f(*argv[i % case.sets]) == 0
    torch.cuda.synchronize()
    ks = [hip.elapsed_ms(x, y) for x, y, _ in evs]
    rest = [hip.elapsed_ms(y, z) for _, y, z in evs]
    res["kernel_ms_mean"] = sum(ks) / len(ks)
    res["kernel_ms_min"] = min(ks)
    res["rest_ms_mean"] = sum(rest) / len(rest)
    for e in evs:
        for x in e:
            hip.destroy(x)
    hip.destroy(a)
    hip.destroy(b)
    return res


def stream_alone(lib, case, steps, hip, torch):
    """The exact call's streaming kernel launched back to back with nothing
    between its launches (the vocabulary-sharded statistics step at one shard
    launches exactly this kernel), rotating over the case's input sets: the
    mean of the dispatches' own durations.  Inside a call the same kernel
    follows the previous call's sampling kernel; the difference between the
    two is the cost of starting the stream after another kernel."""
    import draft_verification_row_amd.sharded as sh
    B, K, V = case.ci.B, case.ci.K, case.ci.V
    rec = torch.empty(sh.shard_record_bytes(torch.bfloat16, B, 2 * K + 1, V, 1), dtype=torch.uint8,
                      device=case.ws.device)
    for i in range(20):
        T, D, x, _ = case.inputs[i % case.sets]
        sh.shard_stats_exact(T, D, x, 1, 0, rec)
    evs = [(hip.event(), hip.event(), hip.event()) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        T, D, x, _ = case.inputs[i % case.sets]
        lib.spec_verify_profile_next_call(*evs[i])
        sh.shard_stats_exact(T, D, x, 1, 0, rec)
    torch.cuda.synchronize()
    d = [hip.elapsed_ms(a, b) for a, b, _ in evs]
    for e in evs:
        for h in e:
            hip.destroy(h)
    return sum(d) / len(d)


def read_ceiling(lib, nbytes, steps, hip, torch, dev):
    """The library's read-only kernel (the streaming kernel's tiles and loads,
    no arithmetic) over nbytes, rotating over enough buffers to defeat the
    last-level cache: its mean dispatch duration and rate."""
    sets = math.ceil(2 * MALL_BYTES / nbytes)
    bufs = [torch.full((nbytes,), 1, dtype=torch.uint8, device=dev) for _ in range(sets)]
    words = lib.spec_read_ceiling_out_words(nbytes)
    out = torch.empty(words, dtype=torch.int32, device=dev)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i in range(20):
        assert lib.spec_read_ceiling(ctypes.c_void_p(bufs[i % sets].data_ptr()), nbytes,
                                     ctypes.c_void_p(out.data_ptr()), st) == 0
    evs = [(hip.event(), hip.event(), hip.event()) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        lib.spec_verify_profile_next_call(*evs[i])
        assert lib.spec_read_ceiling(ctypes.c_void_p(bufs[i % sets].data_ptr()), nbytes,
                                     ctypes.c_void_p(out.data_ptr()), st) == 0
    torch.cuda.synchronize()
    d = [hip.elapsed_ms(a, b) for a, b, _ in evs]
    for e in evs:
        for h in e:
            hip.destroy(h)
    del bufs
    us = sum(d) / len(d) * 1e3
    return {"kernel": "k_read: the streaming kernel's 16 KiB tiles and non-temporal 16-byte loads, "
                      "no arithmetic", "bytes": nbytes, "kernel_us_mean": us,
            "gbs": nbytes / (us * 1e-6) / 1e9, "frac_of_peak": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "input_sets": sets}


def oracle_rate(fn, seconds, max_calls):
    """Calls per second of an oracle call, over about `seconds` (at least one call)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= max_calls:
            return n / el


def other_workload(lib, mode, ci, nbytes, label, steps, warmup, hip, use_graph, torch, dev,
                   cpu=False):
    """Call rate, and the rate of the launch the library's profiling hook
    brackets (the whole call for the single-launch rules, the streaming kernel
    for the tree), of one more workload; with cpu, the oracle's rate on the
    same inputs beside it (a bounded sample)."""
    sets = math.ceil(2 * MALL_BYTES / nbytes)
    case = Case(lib, mode, ci, sets, torch, dev)
    r = time_case(case, steps, warmup, hip, use_graph)
    del case
    torch.cuda.synchronize()
    ms = r["graph_ms_per_step"] if use_graph else r["eager_ms_per_step"]
    logit_bytes = ci.target.nbytes + (ci.draft.nbytes if mode == "exact" else 0)
    out = {"workload": label, "entry_point": f"spec_verify_{mode}",
           "kernel": KERNEL_TIMED[mode],
           "rounds_per_s": 1000.0 / ms, "us_per_call": ms * 1e3,
           "hbm_gbs_call": nbytes / (ms * 1e-3) / 1e9,
           "hbm_frac_call": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "kernel_us_mean": r["kernel_ms_mean"] * 1e3,
           "kernel_gbs": logit_bytes / (r["kernel_ms_mean"] * 1e-3) / 1e9,
           "kernel_frac": logit_bytes / (r["kernel_ms_mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "rest_of_call_us_mean": r["rest_ms_mean"] * 1e3,
           "eager_us_per_call": r["eager_ms_per_step"] * 1e3,
           "graph_us_per_call_runs": [x * 1e3 for x in r.get("graph_ms_per_step_runs", [])],
           "algorithmic_bytes": nbytes, "input_sets": sets,
           "cpu_oracle_rounds_per_s": None, "cpu_oracle_gbs_equivalent": None}
    if cpu:
        rate = oracle_call_rate(mode, ci)
        out["cpu_oracle_rounds_per_s"] = rate
        out["cpu_oracle_gbs_equivalent"] = rate * nbytes / 1e9
        out["oracle_check"] = oracle_leg(mode, ci, r["outputs"])
    return out


def oracle_call(mode, ci):
    """The fp64 oracle's call on the inputs a workload times (CPU oracle leg)."""
    import oracle
    if mode == "tree":
        return lambda: oracle.tree(ci.target, ci.node_tok, ci.parents, "bf16",  # noqa: E731
                                   num_nodes=ci.num_nodes)
    if mode == "greedy":
        return lambda: oracle.greedy(ci.target, ci.tokens, "bf16")  # noqa: E731
    if mode == "relaxed":
        return lambda: oracle.relaxed(ci.target, ci.tokens, ci.uniforms, "bf16", ci.tau,  # noqa: E731
                                      ci.top_k)
    if mode == "power":
        return lambda: oracle.power(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16",  # noqa: E731
                                    POWER_ALPHA)
    if mode == "sample":
        return lambda: oracle.sample(ci.draft, ci.uniforms[:, :ci.K].copy(), "bf16")  # noqa: E731
    return lambda: oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16")  # noqa: E731


def oracle_call_rate(mode, ci):
    return oracle_rate(oracle_call(mode, ci), 2.0, 50)


def check_outputs(mode, outputs, orc):
    """Compares the outputs of the timed calls (every input set holds the same
    inputs) with the oracle's: a request mismatches when its accepted count,
    status or emitted tokens differ outside a flagged near-tie (from a flagged
    position on only the prefix must agree), or its log-probs differ by more
    than 1e-4.  Returns the counts, the largest log-prob difference and the
    mean accepted length on both sides."""
    import numpy as np
    mism, worst, lens = 0, 0.0, []
    if mode == "sample":
        ok = orc.flag == 0
        for o in outputs:
            tok, lq = o["tok"].cpu().numpy(), o["lq"].cpu().numpy()
            st = o["st"].cpu().numpy()
            bad = ((tok != orc.tokens) & ok) | (st != 0)
            d = np.abs(lq - orc.logq)[ok]
            dmax = float(d.max()) if d.size else 0.0
            worst = max(worst, dmax)
            mism += int(bad.sum()) + int((d >= 1e-4).sum())
        rows = orc.flag.size
        return {"calls_checked": len(outputs), "rows_per_call": rows, "mismatched_rows": mism,
                "flagged_rows_per_call": int(orc.flag.sum()),
                "flagged_per_draw": float(orc.flag.sum()) / rows, "max_abs_dlogprob": worst}
    for o in outputs:
        tok, ln, st = (o[k].cpu().numpy() for k in ("tok", "ln", "st"))
        lps = [(o[k].cpu().numpy(), ref) for k, ref in (("tlp", orc.target_logprob),
                                                       ("blp", orc.behavior_logprob)) if k in o]
        if mode == "tree":
            path = o["path"].cpu().numpy()
        lens.append(ln.astype(np.float64))
        for b in range(tok.shape[0]):
            f, n = int(orc.flag[b]), int(orc.accept_len[b])
            if f >= 0:
                good = ln[b] >= f and n >= f and (tok[b, :f] == orc.tokens[b, :f]).all()
                span = f
            else:
                good = (ln[b] == n and st[b] == orc.status[b] and
                        (tok[b, :n + 1] == orc.tokens[b, :n + 1]).all() and (tok[b, n + 1:] == -1).all())
                if mode == "tree":
                    good = good and (path[b] == orc.path[b]).all()
                span = n + 1
            for got, ref in lps:
                if span > 0:
                    d = float(np.abs(got[b, :span] - ref[b, :span]).max())
                    worst = max(worst, d)
                    good = good and d < 1e-4
            mism += 0 if good else 1
    B = orc.accept_len.size
    dec = int(orc.decisions.sum())
    flagged = int((orc.flag >= 0).sum())
    return {"calls_checked": len(outputs), "requests_per_call": B, "mismatched_requests": mism,
            "decisions_per_call": dec, "flagged_per_call": flagged,
            "flagged_per_decision": flagged / max(dec, 1), "max_abs_dlogprob": worst,
            "mean_accept_len": float(np.mean(lens)),
            "mean_accept_len_oracle": float(orc.accept_len.mean())}


def oracle_leg(mode, ci, outputs):
    """One oracle call on the timed inputs and the check of the timed outputs."""
    return check_outputs(mode, outputs, oracle_call(mode, ci)())


def sharded_block(lib, ci, G, steps, warmup, hip, torch, dev):
    """One shard's kernels of a vocabulary-sharded call at the workload's shape
    (G shards of V/G columns), all shards run on this device in turn.  Each
    step's kernel is timed by its own dispatch events; the exchanges between
    the steps (a few KB) are not part of this measurement."""
    import draft_verification_row_amd.sharded as sh
    from numpy import int16
    B, K, V = ci.B, ci.K, ci.V
    Vs = V // G
    sets = math.ceil(2 * MALL_BYTES / ci.algorithmic_bytes_exact)

    def split(a):
        t = torch.from_numpy(a.view(int16)).view(torch.bfloat16).to(dev)
        return [t[:, :, s * Vs:(s + 1) * Vs].contiguous() for s in range(G)]

    T0, D0 = split(ci.target), split(ci.draft)
    Ts = [[t.clone() for t in T0] for _ in range(sets)]
    Ds = [[d.clone() for d in D0] for _ in range(sets)]
    del T0, D0
    x = torch.from_numpy(ci.tokens).to(dev)
    u = torch.from_numpy(ci.uniforms).to(dev)
    slot = sh.shard_record_bytes(torch.bfloat16, B, 2 * K + 1, V, G)
    gslot = sh.shard_record_bytes(torch.bfloat16, B, K + 1, V, G)
    sslot = sh.shard_sums_bytes(B, V, G)
    rec = torch.empty(G * slot, dtype=torch.uint8, device=dev)
    grec = torch.empty(G * gslot, dtype=torch.uint8, device=dev)
    sums = torch.empty(G * sslot, dtype=torch.uint8, device=dev)
    ws = [torch.empty(sh.shard_workspace_bytes(B), dtype=torch.uint8, device=dev) for _ in range(G)]
    import draft_verification_row_amd as sv
    out = sv.VerifyResult(*sv._outs(B, K + 1, dev, True))
    own = torch.empty(B, dtype=torch.int32, device=dev)

    def stats(i, s):
        sh.shard_stats_exact(Ts[i][s], Ds[i][s], x, G, s, rec[s * slot:(s + 1) * slot])

    def sweep(i, s):
        sh.shard_sweep_exact(Ts[i][s], Ds[i][s], rec, x, u, G, s, out,
                             sums[s * sslot:(s + 1) * sslot], ws[s])

    def sample(i, s):
        sh.shard_sample_exact(Ts[i][s], Ds[i][s], sums, u, G, s, out, own, ws[s])

    def gstats(i, s):
        sh.shard_stats_greedy(Ts[i][s], G, s, grec[s * gslot:(s + 1) * gslot], logprobs=False)

    def gcombine(i, s):
        sh.shard_combine_greedy(grec, torch.bfloat16, x, V, G, logprobs=False)

    def timed(fn, i, s):
        e = (hip.event(), hip.event(), hip.event())
        lib.spec_verify_profile_next_call(*e)
        fn(i, s)
        return e

    evs = {k: [] for k in ("stats", "sweep", "sample")}
    for it in range(warmup + steps):
        i = it % sets
        for s in range(G):
            if it >= warmup:
                evs["stats"].append(timed(stats, i, s))
            else:
                stats(i, s)
        for s in range(G):
            if it >= warmup:
                evs["sweep"].append(timed(sweep, i, s))
            else:
                sweep(i, s)
        for s in range(G):
            if it >= warmup:
                evs["sample"].append(timed(sample, i, s))
            else:
                sample(i, s)
    torch.cuda.synchronize()
    res = {}
    for k, lst in evs.items():
        d = [hip.elapsed_ms(a, b) for a, b, _ in lst]
        res[k] = sum(d) / len(d) * 1e3
        for e in lst:
            for h in e:
                hip.destroy(h)
    # greedy, no log-probs: the greedy rows are the target rows of the same shards
    gevs = {"stats": [], "combine": []}
    for it in range(warmup + steps):
        i = it % sets
        for s in range(G):
            if it >= warmup:
                gevs["stats"].append(timed(gstats, i, s))
            else:
                gstats(i, s)
        if it >= warmup:
            gevs["combine"].append(timed(gcombine, i, 0))
        else:
            gcombine(i, 0)
    torch.cuda.synchronize()
    gres = {}
    for k, lst in gevs.items():
        d = [hip.elapsed_ms(a, b) for a, b, _ in lst]
        gres[k] = sum(d) / len(d) * 1e3
        for e in lst:
            for h in e:
                hip.destroy(h)
    shard_bytes = (ci.target.nbytes + ci.draft.nbytes) // G
    del Ts, Ds
    torch.cuda.synchronize()
    return {
        "workload": f"exact and greedy, B={B} K={K} V={V} bf16 split over {G} vocabulary shards of "
                    f"{Vs} columns; one shard's kernels, all shards run on this device in turn",
        "shards": G, "columns_per_shard": Vs,
        "exact": {"stats_kernel_us": res["stats"],
                  "stats_gbs": shard_bytes / (res["stats"] * 1e-6) / 1e9,
                  "sweep_kernel_us": res["sweep"], "sample_kernel_us": res["sample"],
                  "kernel_us_per_shard": res["stats"] + res["sweep"] + res["sample"],
                  "logit_bytes_per_shard": shard_bytes,
                  "exchange_bytes_per_shard": [slot, sslot, B * 12]},
        "greedy_no_logprobs": {"stats_kernel_us": gres["stats"],
                               "stats_gbs": ci.target.nbytes // G / (gres["stats"] * 1e-6) / 1e9,
                               "combine_kernel_us": gres["combine"],
                               "kernel_us_per_shard": gres["stats"] + gres["combine"],
                               "exchange_bytes_per_shard": [gslot]},
        "not_measured": "exchange latency (all-gathers of the slots, broadcast of the draw)",
        "input_sets": sets,
    }


def markov_block(torch, dev, rounds, with_cpu, use_graph=True):
    """The multi-round driver with toy Markov models (V=4096, B=32, K=4): the
    GPU loop's rate (all rounds in one captured graph, and the eager loop),
    the run's acceptance statistics, and the oracle's driver on a few rounds
    of the same inputs beside it."""
    import draft_verification_row_amd.markov as mk
    import synth
    from numpy import int16
    V, B, K = 4096, 32, 4
    m = synth.markov_inputs(V, B, K, rounds, "bf16", seed=4096)
    P = torch.from_numpy(m.target.view(int16)).view(torch.bfloat16).to(dev)
    Q = torch.from_numpy(m.draft.view(int16)).view(torch.bfloat16).to(dev)
    st = torch.from_numpy(m.start).to(dev)
    ud = torch.from_numpy(m.u_draft).to(dev)
    uv = torch.from_numpy(m.u_verify).to(dev)
    warm = min(10, rounds)
    mk.generate_speculative(P, Q, st, ud[:warm].contiguous(), uv[:warm].contiguous())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    tr = mk.generate_speculative(P, Q, st, ud, uv)
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - t0
    # every round captured in one HIP graph: the first replay uploads it, the
    # median of RUNS timed replays is reported, and each replay must equal the
    # eager loop's tokens bit for bit
    el = eager_s
    if use_graph:
        g = mk.SpeculativeGraph(P, Q, B, K, rounds)
        g.run(st, ud, uv)
        torch.cuda.synchronize()
        runs = []
        for _ in range(RUNS):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            gt = g.run(st, ud, uv)
            e1.record()
            torch.cuda.synchronize()
            runs.append(e0.elapsed_time(e1) * 1e-3)
            if not (torch.equal(gt.emitted, tr.emitted) and torch.equal(gt.accept_len, tr.accept_len)):
                raise RuntimeError("the graph-captured driver differs from the eager loop")
        el = sorted(runs)[len(runs) // 2]
        del g
    timed = (f"all rounds captured in one HIP graph (rounds_per_s: median of {RUNS} replays, "
             f"input copies included) and the eager loop (eager_rounds_per_s)" if use_graph
             else "the eager loop")
    res = {"workload": f"multi-round speculative sampling, toy Markov models V={V} (target "
                       f"2*N(0,1) logits per state, draft target+0.7*N(0,1)), B={B} sequences, "
                       f"K={K}, {rounds} rounds; per round K draft draws (spec_sample_drafts) and "
                       f"one exact verification; timed: {timed}",
           "rounds_per_s": rounds / el, "tokens_per_s": None, "ms_per_round": el / rounds * 1e3,
           "eager_rounds_per_s": rounds / eager_s, "eager_ms_per_round": eager_s / rounds * 1e3,
           **mk.trace_stats(tr.accept_len, K, 0.1), "cpu_oracle_rounds_per_s": None}
    res["tokens_per_s"] = res["tokens"] / el
    if with_cpu:
        import oracle
        n = min(20, rounds)
        t0 = time.perf_counter()
        oracle.speculative_generate(m.target, m.draft, m.start, m.u_draft[:n], m.u_verify[:n], "bf16")
        res["cpu_oracle_rounds_per_s"] = n / (time.perf_counter() - t0)
    return res


def kernel_source_sha256():
    """SHA-256 of the kernel source file (the counters below belong to it)."""
    import hashlib
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_bytes():
    """HBM bytes per dispatch of the exact call's kernel from the recorded
    counters, or None when none are recorded for the current kernel source."""
    if not TRAFFIC or TRAFFIC["source_sha256"] != kernel_source_sha256():
        return None
    return int(TRAFFIC["fetch_kib"] * TRAFFIC["fetch_scale"] * 1024 +
               TRAFFIC["write_kib"] * TRAFFIC["write_scale"] * 1024)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(ci, seconds):
    import oracle
    import synth
    oracle.load()
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16")
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = oracle.max_threads()
    oracle.set_threads(1)
    one = oracle_rate(lambda: oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16"),
                      3.0, 100)
    oracle.set_threads(threads)
    tiny = synth.tiny_exact_v32()
    tiny_rate = tiny.B * oracle_rate(lambda: oracle.exact(tiny.target, tiny.draft, tiny.tokens, tiny.uniforms,
                                                      "f32"), 1.0, 1000)
    return {"value": n / el, "unit": "rounds/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} exact verification calls of the benchmark batch (B=32, K=5, "
                      f"V=128256 bf16) on the same inputs, {el:.1f} s, fp64 C oracle, "
                      f"OpenMP over requests",
            "cpu_model": cpu_model(), "single_thread_value": one,
            "gbs_equivalent": n / el * ci.algorithmic_bytes_exact / 1e9,
            "tiny_exact_b1_k4_v32_rounds_per_s": tiny_rate}


def progress(msg: str) -> None:
    """One line per finished block on stderr (stdout carries only the result)."""
    print(f"bench: {msg} ({time.time() - _T0:.0f} s)", file=sys.stderr, flush=True)


_T0 = time.time()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU; --gpus {args.gpus} is not supported "
              "(requests shard across GPUs with no exchange, see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch

    import draft_verification_row_amd as sv
    import synth

    lib = sv.load_library()
    lib.spec_verify_profile_next_call.argtypes = [ctypes.c_void_p] * 3
    lib.spec_verify_power.argtypes = ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p] + [ctypes.c_int] * 3 + [ctypes.c_float] +
                                      [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p])
    lib.spec_sample_drafts.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
    lib.spec_verify_profile_next_call.restype = None
    dev = torch.device("cuda:0")
    hip = Hip()
    ci = synth.exact_b32_k5()
    bytes_exact = ci.algorithmic_bytes_exact
    bytes_greedy = ci.algorithmic_bytes_greedy
    sets_exact = math.ceil(2 * MALL_BYTES / bytes_exact)
    sets_greedy = math.ceil(2 * MALL_BYTES / bytes_greedy)
    use_graph = not args.no_graph

    ex = Case(lib, "exact", ci, sets_exact, torch, dev)
    r_ex = time_case(ex, args.steps, args.warmup, hip, use_graph)
    alone_ms = stream_alone(lib, ex, args.steps, hip, torch)
    del ex
    progress("exact timed")
    gr = Case(lib, "greedy", ci, sets_greedy, torch, dev)
    r_gr = time_case(gr, args.steps, args.warmup, hip, use_graph)
    del gr
    progress("greedy timed")
    pw = Case(lib, "power", ci, sets_exact, torch, dev)
    r_pw = time_case(pw, args.steps, args.warmup, hip, use_graph)
    del pw
    progress("power timed")
    sets_sample = math.ceil(2 * MALL_BYTES / ci.draft.nbytes)
    sa = Case(lib, "sample", ci, sets_sample, torch, dev)
    r_sa = time_case(sa, args.steps, args.warmup, hip, use_graph)
    del sa
    progress("draft sampler timed")
    torch.cuda.synchronize()
    ceiling = read_ceiling(lib, ci.target.nbytes + ci.draft.nbytes, args.steps, hip, torch, dev)
    ceiling_g = read_ceiling(lib, ci.target.nbytes, args.steps, hip, torch, dev)
    progress("read ceiling timed")
    cpu = not args.no_cpu_baseline
    others = None
    if not args.no_configs:
        others = {}
        greedy8 = synth.greedy_chain_b8()
        others["greedy_b8"] = other_workload(
            lib, "greedy", greedy8, greedy8.algorithmic_bytes_greedy,
            "greedy chain, B=8 K=5 V=128256 bf16, no log-probs", args.steps, args.warmup, hip,
            use_graph, torch, dev, cpu)
        del greedy8
        progress("greedy B=8 timed")
        tree8 = synth.tree_b8_n61()
        others["tree_b8_n61"] = other_workload(
            lib, "tree", tree8, tree8.algorithmic_bytes,
            "greedy tree (depth 5, top-k 4, 60 drafted nodes + root), B=8 V=128256 bf16, "
            "no log-probs", args.steps, args.warmup, hip, use_graph, torch, dev, cpu)
        del tree8
        progress("tree timed")
        large = synth.large_b64_k8()
        others["relaxed_b64_k8"] = other_workload(
            lib, "relaxed", large, large.algorithmic_bytes_relaxed,
            f"relaxed (p >= {large.tau} or top-{large.top_k}), B=64 K=8 V=151936 bf16", args.steps,
            args.warmup, hip, use_graph, torch, dev, cpu)
        others["exact_b64_k8"] = other_workload(
            lib, "exact", large, large.algorithmic_bytes_exact,
            "exact, B=64 K=8 V=151936 bf16, draft target+0.8*N(0,1)", args.steps, args.warmup,
            hip, use_graph, torch, dev, cpu)
        del large
        progress("B=64 relaxed and exact timed")
        others["sharded_exact_greedy_g8"] = sharded_block(lib, ci, 8, min(args.steps, 200),
                                                         min(args.warmup, 20), hip, torch, dev)
        progress("vocabulary shards timed")
        others["markov_driver"] = markov_block(torch, dev, min(args.steps, 200),
                                               not args.no_cpu_baseline, use_graph)
        progress("multi-round driver timed")

    ms = r_ex["graph_ms_per_step"] if use_graph else r_ex["eager_ms_per_step"]
    value = 1000.0 / ms
    k_ms = r_ex["kernel_ms_mean"]
    # the exact call is one kernel launch: its algorithmic bytes are the call's
    # (every logit read once, the tokens and uniforms, the outputs)
    stream_bytes = ci.target.nbytes + ci.draft.nbytes
    achieved = bytes_exact / (k_ms * 1e-3) / 1e9
    g_ms = r_gr["graph_ms_per_step"] if use_graph else r_gr["eager_ms_per_step"]
    s_ms = r_sa["graph_ms_per_step"] if use_graph else r_sa["eager_ms_per_step"]
    p_ms = r_pw["graph_ms_per_step"] if use_graph else r_pw["eager_ms_per_step"]
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "rounds/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "exact verification (min(1,p/q) + residual), B=32 K=5 V=128256 "
                               "bf16, target 3*N(0,1), draft target+0.5*N(0,1)",
                   "B": ci.B, "K": ci.K, "V": ci.V, "input_sets": sets_exact,
                   "launch": "hip graph replay of the timed calls" if use_graph else "eager"},
        "hbm_gbs_call": bytes_exact / (ms * 1e-3) / 1e9,
        "hbm_frac_call": bytes_exact / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_bytes(),
                     "kernel": "k_single<bf16, exact>: the whole call in one launch (streams every "
                               "logit once, decides, draws the terminal token)",
                     "kernel_us_mean": k_ms * 1e3, "kernel_us_min": r_ex["kernel_ms_min"] * 1e3,
                     "algorithmic_bytes_per_launch": bytes_exact,
                     "logit_bytes_per_launch": stream_bytes,
                     "rest_of_call_us_mean": r_ex["rest_ms_mean"] * 1e3,
                     "frac_of_read_ceiling": achieved / ceiling["gbs"],
                     "stream_alone_us_mean": alone_ms * 1e3,
                     "stream_alone_frac": stream_bytes / (alone_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "stream_alone_note": "k_stream alone (the same 16 KiB tile streaming with no "
                                          "sweep or draw, as the one-shard statistics step "
                                          "launches it), back to back: the floor under the "
                                          "single launch's streaming phase"},
        "read_ceiling": ceiling,
        "graph_ms_per_step_runs": r_ex.get("graph_ms_per_step_runs"),
        "eager": {"rounds_per_s": 1000.0 / r_ex["eager_ms_per_step"],
                  "ms_per_step": r_ex["eager_ms_per_step"]},
        "greedy_b32_k5": {
            "kernel": KERNEL_TIMED["greedy"],
            "rounds_per_s": 1000.0 / g_ms, "ms_per_step": g_ms,
            "hbm_gbs_call": bytes_greedy / (g_ms * 1e-3) / 1e9,
            "kernel_us_mean": r_gr["kernel_ms_mean"] * 1e3,
            "kernel_gbs": ci.target.nbytes / (r_gr["kernel_ms_mean"] * 1e-3) / 1e9,
            "kernel_frac": ci.target.nbytes / (r_gr["kernel_ms_mean"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kernel_frac_of_read_ceiling": ci.target.nbytes / (r_gr["kernel_ms_mean"] * 1e-3) / 1e9
                                           / ceiling_g["gbs"],
            "read_ceiling": ceiling_g,
            "rest_of_call_us_mean": r_gr["rest_ms_mean"] * 1e3,
            "eager_rounds_per_s": 1000.0 / r_gr["eager_ms_per_step"],
            "algorithmic_bytes": bytes_greedy, "input_sets": sets_greedy},
        "power_b32_k5": {
            "alpha": POWER_ALPHA, "rounds_per_s": 1000.0 / p_ms, "ms_per_step": p_ms,
            "hbm_gbs_call": bytes_exact / (p_ms * 1e-3) / 1e9,
            "kernel_us_mean": r_pw["kernel_ms_mean"] * 1e3,
            "kernel_gbs": stream_bytes / (r_pw["kernel_ms_mean"] * 1e-3) / 1e9,
            "rest_of_call_us_mean": r_pw["rest_ms_mean"] * 1e3, "input_sets": sets_exact},
        "draft_sampler_b32_k5_draft_rows": {
            "calls_per_s": 1000.0 / s_ms, "ms_per_call": s_ms, "rows": ci.B * ci.K,
            "hbm_gbs_call": ci.draft.nbytes / (s_ms * 1e-3) / 1e9,
            "kernel_us_mean": r_sa["kernel_ms_mean"] * 1e3,
            "kernel_gbs": ci.draft.nbytes / (r_sa["kernel_ms_mean"] * 1e-3) / 1e9,
            "rest_of_call_us_mean": r_sa["rest_ms_mean"] * 1e3,
            "logit_bytes": ci.draft.nbytes, "input_sets": sets_sample},
        "other_workloads": others,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        progress("oracle checks of the timed outputs start")
        checks = {"exact_b32_k5": oracle_leg("exact", ci, r_ex["outputs"]),
                  "greedy_b32_k5": oracle_leg("greedy", ci, r_gr["outputs"]),
                  "power_b32_k5": oracle_leg("power", ci, r_pw["outputs"]),
                  "draft_sampler_b32_k5_draft_rows": oracle_leg("sample", ci, r_sa["outputs"])}
        for k, v in (others or {}).items():
            if isinstance(v, dict) and "oracle_check" in v:
                checks[k] = v["oracle_check"]
        out["timed_outputs_vs_oracle"] = checks
        bad = {k: v.get("mismatched_requests", v.get("mismatched_rows")) for k, v in checks.items()}
        if any(bad.values()):
            print(f"bench: timed outputs differ from the oracle: {bad}", file=sys.stderr, flush=True)
        progress("CPU baseline starts")
        out["cpu_baseline"] = cpu_baseline(ci, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
