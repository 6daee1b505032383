"""Decisions placed next to their thresholds: how far from a threshold the HIP
library still decides as the oracle does.

Accept tests (spec-decode README, "How it works": draft j is accepted iff
u_j < min(1, p/q); nanospec README, acceptance rules: p >= tau or top-k, and
min(1, p/q)^alpha): the uniform, or tau, is set at float32 values next to the
oracle's ratio, from 2e-6 away down to the two float32 neighbours of the
ratio.  Beyond the 1e-6 near-tie window every decision must match the oracle
bit for bit; inside it the test records how close the GPU still matches, which
measures its error on the ratio.

Terminal draws (the same README: the residual normalize(relu(p - q)), or the
last target row after K acceptances): u_K is set at float32 values whose
distance from a boundary of the inverse CDF lies in each decade from 1e-14 to
1e-7 of the draw's total mass.  The expected token comes from an
extended-precision running sum of the oracle's weights.  Every draw at least
1e-12 of the total from a boundary must match it, a decade inside the
near-tie window of the terminal draws; the closest mismatch is recorded.

Inputs are seeded chain batches at the shapes and scales of the benchmark
workloads: 3*N(0,1) targets with 0.5 and 0.8 draft noise at V = 128256 and
151936, flat 0.3*N(0,1) rows, and small fp32 rows.
"""
import zlib

import numpy as np
import pytest
import torch

import draft_verification_row_amd as sv
import oracle
import synth
from parity import BINS, U_REJECT, dev, dev_logits, near_boundary_uniforms

pytestmark = pytest.mark.gpu

# offsets of u from the ratio r (absolute), besides r's own float32 neighbours
OFFSETS = [2e-6, -2e-6, 5e-7, -5e-7, 2e-7, -2e-7, 1e-7, -1e-7, 5e-8, -5e-8]
WINDOW = oracle.EPS_ACCEPT
SAMPLE_CHECK = 1e-12  # terminal draws this far (relative) from a boundary must match


def _workload(name):
    if name == "exact_b32_k5_rows":
        return synth.chain_inputs(6, 5, 128256, "bf16", seed=3031, useed=3032, d_noise=0.5)
    if name == "large_b64_k8_rows":
        return synth.chain_inputs(4, 8, 151936, "bf16", seed=5051, useed=5052, d_noise=0.8)
    if name == "flat_rows":
        return synth.chain_inputs(6, 5, 128256, "bf16", seed=6061, useed=6062, t_scale=0.3,
                                  d_noise=0.3)
    if name == "small_f32":
        return synth.chain_inputs(8, 5, 5003, "f32", seed=7071, useed=7072, t_scale=2.0,
                                  d_noise=0.7)
    raise KeyError(name)


def _rep(a, b, m):
    return np.repeat(a[b:b + 1], m, 0)


def _gpu(rule, ci, b, x, u, **kw):
    m = u.shape[0]
    T = dev_logits(_rep(ci.target, b, m), ci.dtype)
    if rule == "exact":
        r = sv.spec_verify_exact(T, dev_logits(_rep(ci.draft, b, m), ci.dtype), dev(x), dev(u))
    elif rule == "power":
        r = sv.spec_verify_power(T, dev_logits(_rep(ci.draft, b, m), ci.dtype), dev(x), dev(u),
                                 kw["alpha"])
    else:
        r = sv.spec_verify_relaxed(T, dev(x), dev(u), kw["tau"], kw["top_k"])
    torch.cuda.synchronize()
    return r.accept_len.cpu().numpy(), r.tokens.cpu().numpy()


def _oracle(rule, ci, b, x, u, **kw):
    m = u.shape[0]
    T = _rep(ci.target, b, m)
    if rule == "exact":
        return oracle.exact(T, _rep(ci.draft, b, m), x, u, ci.dtype)
    if rule == "power":
        return oracle.power(T, _rep(ci.draft, b, m), x, u, ci.dtype, kw["alpha"])
    return oracle.relaxed(T, x, u, ci.dtype, kw["tau"], kw["top_k"])


def _ratios(rule, ci, **kw):
    """The oracle's acceptance probabilities of every draft (all accepted at
    u = 0): min(1, p/q), or its alpha power."""
    z = np.zeros((ci.B, ci.K + 1), np.float32)
    if rule == "exact":
        o = oracle.exact(ci.target, ci.draft, ci.tokens, z, ci.dtype)
    else:
        o = oracle.power(ci.target, ci.draft, ci.tokens, z, ci.dtype, kw["alpha"])
    assert (o.accept_len == ci.K).all()
    return np.exp(o.behavior_logprob[:, :ci.K])


def _picks_near(r):
    """Float32 uniforms next to r: r + OFFSETS and r's two float32 neighbours."""
    f = np.float32(r)
    cand = [np.float32(r + d) for d in OFFSETS]
    lo = f if float(f) < r else np.nextafter(f, np.float32(0))
    hi = f if float(f) > r else np.nextafter(f, np.float32(1))
    cand += [lo, hi]
    return [(u, float(u) - r) for u in cand if 0 < u < 1]


@pytest.mark.parametrize("rule", ["exact", "power"])
@pytest.mark.parametrize("name", ["exact_b32_k5_rows", "large_b64_k8_rows", "flat_rows", "small_f32"])
def test_accept_test_window(rule, name):
    ci = _workload(name)
    kw = {"alpha": 0.5} if rule == "power" else {}
    print(f"accept window {rule} {name}", flush=True)
    r = _ratios(rule, ci, **kw)
    tested, worst_mismatch, closest = 0, 0.0, 1.0
    for b in range(ci.B):
        rows = []
        for j in range(ci.K):
            if not (1e-4 < r[b, j] < 0.999):
                continue
            for u, off in _picks_near(float(r[b, j])):
                rows.append((j, u, off))
        if not rows:
            continue
        m = len(rows)
        u = np.full((m, ci.K + 1), 0.5, np.float32)
        for i, (j, uu, _) in enumerate(rows):
            u[i, :j] = 0.0
            u[i, j] = uu
        x = _rep(ci.tokens, b, m)
        g_len, _ = _gpu(rule, ci, b, x, u, **kw)
        o = _oracle(rule, ci, b, x, u, **kw)
        for i, (j, uu, off) in enumerate(rows):
            precise = off < 0                      # u < r accepts
            gpu = bool(g_len[i] > j)
            closest = min(closest, abs(off))
            tested += 1
            if abs(off) >= WINDOW:
                assert o.flag[i] < 0 or o.flag[i] > j
                assert bool(o.accept_len[i] > j) == precise, (b, j, off)
                assert gpu == precise, f"{rule} {name} request {b} draft {j}: u - r = {off:.3e}"
            elif gpu != precise:
                worst_mismatch = max(worst_mismatch, abs(off))
    print(f"MEASURED accept window {rule} {name}: {tested} decisions, closest |u - r| {closest:.2e}, "
          f"largest |u - r| decided differently from the oracle {worst_mismatch:.2e}", flush=True)
    assert tested >= 20


@pytest.mark.parametrize("name", ["exact_b32_k5_rows", "flat_rows", "small_f32"])
def test_relaxed_tau_window(name):
    """tau set next to p_0(x_0) (top_k = 0, so only p >= tau accepts)."""
    ci = _workload(name)
    print(f"tau window {name}", flush=True)
    z = np.zeros((ci.B, ci.K + 1), np.float32)
    o0 = oracle.relaxed(ci.target, ci.tokens, z, ci.dtype, 0.0, 0)
    p0 = np.exp(o0.target_logprob[:, 0])
    tested, worst_mismatch = 0, 0.0
    for b in range(ci.B):
        for tau, off in _picks_near(float(p0[b])):
            x = ci.tokens[b:b + 1]
            g_len, _ = _gpu("relaxed", ci, b, x, z[b:b + 1], tau=float(tau), top_k=0)
            o = oracle.relaxed(ci.target[b:b + 1], x, z[b:b + 1], ci.dtype, float(tau), 0)
            precise = off <= 0                     # p >= tau accepts
            gpu = bool(g_len[0] > 0)
            tested += 1
            if abs(off) >= WINDOW:
                assert bool(o.accept_len[0] > 0) == precise
                assert gpu == precise, f"{name} request {b}: tau - p = {off:.3e}"
            elif gpu != precise:
                worst_mismatch = max(worst_mismatch, abs(off))
    print(f"MEASURED tau window {name}: {tested} decisions, largest |tau - p| decided differently "
          f"{worst_mismatch:.2e}", flush=True)


# ------------------------------------------------------------ terminal draws
def _terminal_case(rule, ci, rng):
    """Per request: the first-rejection position n, the uniforms and tokens
    that make the decisions stop there, and the rule's keyword arguments."""
    B, K = ci.B, ci.K
    x = ci.tokens.copy()
    u = np.zeros((B, K + 1), np.float32)
    n = np.full(B, K, np.int32)
    kw = {}
    if rule in ("exact_residual", "power"):
        kw = {"alpha": 0.5} if rule == "power" else {}
        r = _ratios("power" if rule == "power" else "exact", ci, **kw)
        for b in range(B):
            rej = np.flatnonzero(r[b] < 0.999)
            n[b] = rej[rng.integers(0, rej.size)]
            u[b, n[b]] = U_REJECT
    elif rule == "relaxed":
        kw = {"tau": 2.0, "top_k": 1}  # accept iff the draft is a row maximum
        Tw = synth.widen(ci.target, ci.dtype)
        for b in range(B):
            n[b] = rng.integers(0, K + 1)
            for j in range(K):
                row = Tw[b, j]
                if j < n[b]:
                    x[b, j] = int(np.argmax(row))
                elif j == n[b]:
                    below = np.flatnonzero(row < row.max())
                    x[b, j] = int(below[rng.integers(0, below.size)])
    return n, x, u, kw


def _terminal_weights(rule, ci, n):
    if rule in ("exact_residual", "exact_bonus"):
        return oracle.terminal_weights("exact", ci.target, ci.dtype, n, ci.draft)
    return oracle.terminal_weights("target", ci.target, ci.dtype, n)


@pytest.mark.parametrize("rule", ["exact_residual", "exact_bonus", "relaxed", "power"])
@pytest.mark.parametrize("name", ["exact_b32_k5_rows", "large_b64_k8_rows", "small_f32"])
def test_terminal_draw_window(rule, name):
    rng = np.random.default_rng(zlib.crc32(f"{rule}/{name}".encode()))
    ci = _workload(name)
    print(f"terminal window {rule} {name}", flush=True)
    n, x, u0, kw = _terminal_case(rule, ci, rng)
    tw = _terminal_weights(rule, ci, n)
    if rule == "exact_residual":
        assert tw.residual.all()
    grule = "exact" if rule.startswith("exact") else rule
    tested, worst_mismatch, per_bin = 0, 0.0, {}
    for b in range(ci.B):
        picks = near_boundary_uniforms(tw.w[b], tw.Z[b], BINS, 8, rng)
        if not picks:
            continue
        m = len(picks)
        u = _rep(u0, b, m)
        u[:, ci.K] = [p[0] for p in picks]
        xb = _rep(x, b, m)
        g_len, g_tok = _gpu(grule, ci, b, xb, u, **kw)
        o = _oracle(grule, ci, b, xb, u, **kw)
        assert (g_len == n[b]).all() and (o.accept_len == n[b]).all()
        for i, (uu, dist, want) in enumerate(picks):
            got = int(g_tok[i, n[b]])
            key = f"{10.0 ** np.floor(np.log10(abs(dist))):.0e}"
            per_bin[key] = per_bin.get(key, 0) + 1
            tested += 1
            if abs(dist) >= SAMPLE_CHECK:
                assert got == want, (f"{rule} {name} request {b}: u*Z - boundary = {dist:.3e} Z, "
                                     f"gpu {got} want {want}")
            elif got != want:
                worst_mismatch = max(worst_mismatch, abs(dist))
            if o.flag[i] < 0:
                assert int(o.tokens[i, n[b]]) == got
    print(f"MEASURED terminal window {rule} {name}: {tested} draws by decade of distance "
          f"{dict(sorted(per_bin.items()))}; largest distance decided differently from the "
          f"extended-precision CDF {worst_mismatch:.2e}", flush=True)
    assert tested >= 30


@pytest.mark.parametrize("name", ["exact_b32_k5_rows", "large_b64_k8_rows", "small_f32"])
def test_sampler_draw_window(name):
    """The draft sampler: one draw per draft row, u next to its CDF boundaries."""
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    ci = _workload(name)
    print(f"sampler window {name}", flush=True)
    rows = ci.draft.reshape(-1, ci.V)[:8]
    tw = oracle.terminal_weights("sampler", rows, ci.dtype)
    tested, worst_mismatch = 0, 0.0
    for r_ in range(rows.shape[0]):
        picks = near_boundary_uniforms(tw.w[r_], tw.Z[r_], BINS, 8, rng)
        if not picks:
            continue
        X = _rep(rows, r_, len(picks))
        u = np.array([p[0] for p in picks], np.float32)
        s = sv.spec_sample_drafts(dev_logits(X, ci.dtype), dev(u))
        torch.cuda.synchronize()
        got = s.tokens.cpu().numpy()
        o = oracle.sample(X, u, ci.dtype)
        for i, (uu, dist, want) in enumerate(picks):
            tested += 1
            if abs(dist) >= SAMPLE_CHECK:
                assert got[i] == want, f"sampler {name} row {r_}: {dist:.3e}"
            elif got[i] != want:
                worst_mismatch = max(worst_mismatch, abs(dist))
            if not o.flag[i]:
                assert o.tokens[i] == got[i]
    print(f"MEASURED sampler window {name}: {tested} draws; largest distance decided differently "
          f"{worst_mismatch:.2e}", flush=True)
    assert tested >= 30
