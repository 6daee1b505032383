"""The oracle's exact rule against its closed form, and the oracle's terminal
draw against an extended-precision inverse CDF.

spec-decode README, "Provably exact": accepting draft x with probability
min(1, p/q) and otherwise drawing from normalize(relu(p - q)) emits tokens
whose law is p exactly.  Here every term of that identity is read from the
oracle's own outputs (accept decisions, emitted tokens and behaviour
log-probs), so a mistake anywhere in the oracle's exact rule -- the ratio, the
min, the residual, its normalizer, the (1 - r) factor of mu, the inverse-CDF
order -- breaks the identity.  The expected side, p, is torch's float64
softmax of the same logits.

None of these tests calls the HIP library.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import BINS, U_REJECT, near_boundary_uniforms

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def softmax64(a):
    return torch.softmax(torch.from_numpy(np.asarray(a, np.float64)), dim=-1).numpy()


def _pairs(rng, P, V):
    """P random target/draft logit row pairs (float32) at vocabulary V: target
    scale in [0.3, 3], draft noise in [0.05, 2]; a third of the drafts get a
    near-zero probability somewhere (a logit 30 below)."""
    ts = rng.uniform(0.3, 3.0, size=(P, 1)).astype(np.float32)
    dn = rng.uniform(0.05, 2.0, size=(P, 1)).astype(np.float32)
    t = (rng.standard_normal((P, V), dtype=np.float32) * ts).astype(np.float32)
    d = (t + rng.standard_normal((P, V), dtype=np.float32) * dn).astype(np.float32)
    low = rng.random(P) < 1 / 3
    d[low, rng.integers(0, V, size=low.sum())] -= np.float32(30.0)
    return t, d


def _induced(V, P, rng):
    """For P random pairs at vocabulary V: induced(t) = sum_x q(x) mu(t|x), with
    mu(t|x) read from oracle.exact (K = 1).  Returns (induced, p, mu row sums)
    over the pairs whose every outcome a float32 uniform can reach."""
    t, d = _pairs(rng, P, V)
    T = np.stack([t, t], 1)           # [P][2][V]: row 0 is tested, row 1 unused
    D = d[:, None, :]                 # [P][1][V]
    # accept branch: u_0 = 0 accepts x whenever p(x) > 0; mu(x|x) = min(1, p/q)
    xs = np.tile(np.arange(V, dtype=np.int32), P)[:, None]
    pi = np.repeat(np.arange(P), V)
    u = np.zeros((P * V, 2), np.float32)
    u[:, 1] = 0.5
    ra = oracle.exact(T[pi], D[pi], xs, u, "f32", eps_accept=0.0, eps_sample=0.0)
    assert (ra.accept_len == 1).all()
    a = np.exp(ra.behavior_logprob[:, 0]).reshape(P, V)
    # the residual the rejection branch inverts (independent of x)
    tw = oracle.terminal_weights("exact", T, "f32", np.zeros(P, np.int32), D)
    keep = np.ones(P, bool)
    for i in range(P):
        rel = tw.w[i] / tw.Z[i]
        # outcomes a float32 uniform cannot isolate: an acceptance probability
        # in (1 - 1e-6, 1), or a residual interval narrower than 1e-6
        if ((a[i] < 1.0) & (a[i] > 1.0 - 1e-6)).any() or ((rel > 0) & (rel < 1e-6)).any():
            keep[i] = False
        if not tw.residual[i]:
            keep[i] = False  # p == q on this row: nothing is ever rejected
    reqs, meta = [], []
    for i in np.flatnonzero(keep):
        c = np.cumsum(tw.w[i])
        lo = np.concatenate([[0.0], c[:-1]])
        for tt in np.flatnonzero(tw.w[i] > 0):
            mid = np.float32(0.5 * (lo[tt] + c[tt]) / tw.Z[i])
            assert lo[tt] < float(mid) * tw.Z[i] < c[tt]
            for x in np.flatnonzero(a[i] < 1.0):
                reqs.append((i, x, mid))
                meta.append((i, x, tt))
    ri = np.array([r[0] for r in reqs])
    rx = np.array([[r[1]] for r in reqs], np.int32)
    ru = np.array([[U_REJECT, r[2]] for r in reqs], np.float32)
    rr = oracle.exact(T[ri], D[ri], rx, ru, "f32", eps_accept=0.0, eps_sample=0.0)
    assert (rr.accept_len == 0).all()
    mt = np.array([m[2] for m in meta])
    assert (rr.tokens[:, 0] == mt).all(), "the midpoint of t's interval must emit t"
    mu_rej = np.exp(rr.behavior_logprob[:, 0])
    q = softmax64(d)
    p = softmax64(t)
    induced = q * a                   # accepted draft x emits x
    rowsum = a.copy()
    for (i, x, tt), m in zip(meta, mu_rej):
        induced[i, tt] += q[i, x] * m
        rowsum[i, x] += m
    return induced[keep], p[keep], rowsum[keep], int(keep.sum())


def test_oracle_exact_mu_marginalises_to_target_on_random_pairs():
    """sum_x q(x) mu(t|x) = p(t) to 1e-12 on >= 5000 random (p, q) pairs
    (V = 2..64, then 256 and 512), and sum_t mu(t|x) = 1 for every x.  The
    page prints 2.21e-16 for the induced-vs-target distance of its sampler."""
    rng = np.random.default_rng(2024)
    n, worst, worst_sum = 0, 0.0, 0.0
    for V in list(range(2, 65)) + [256, 512]:
        P = 2 if V > 64 else 90
        ind, p, rs, k = _induced(V, P, rng)
        n += k
        worst = max(worst, float(np.abs(ind - p).max()))
        worst_sum = max(worst_sum, float(np.abs(rs - 1.0).max()))
    assert n >= 5000, n
    assert worst <= GOLD["spec_decode_verify"]["bound"], worst
    assert worst_sum <= 1e-12, worst_sum


def test_closed_form_identity_in_numpy():
    """The identity itself, in numpy and without the oracle: q*min(1, p/q) +
    (1 - sum min(p, q)) * relu(p - q)/sum relu(p - q) = p on 5000 random pairs
    (the test above is the one that pins the oracle)."""
    rng = np.random.default_rng(11)
    worst, n = 0.0, 0
    for V in list(range(2, 65)) + [1000]:
        for _ in range(80 if V < 1000 else 40):
            p = rng.dirichlet(np.full(V, rng.uniform(0.05, 2.0)))
            q = rng.dirichlet(np.full(V, rng.uniform(0.05, 2.0)))
            acc = np.minimum(p, q)
            res = np.maximum(p - q, 0.0)
            induced = acc + ((1.0 - acc.sum()) * res / res.sum() if res.sum() > 0 else 0.0)
            worst = max(worst, 0.5 * np.abs(induced - p).sum())
            n += 1
    assert n >= 5000 and worst <= 1e-12, worst


# ---------------------------------------------------------------- the export
def test_terminal_weights_match_numpy():
    """oracle.terminal_weights against numpy in extended precision: relu(p - q)
    (or p) of the rejected row for the exact rule, p_n for the target rule, and
    exp(l - max) for the sampler, each to 1e-15 relative to its sum."""
    rng = np.random.default_rng(77)
    ci = synth.chain_inputs(6, 4, 5003, "bf16", seed=78, useed=79)
    n = np.array([0, 1, 2, 3, 4, 2], np.int32)
    tw = oracle.terminal_weights("exact", ci.target, "bf16", n, ci.draft)
    T = synth.widen(ci.target, "bf16").astype(np.longdouble)
    D = synth.widen(ci.draft, "bf16").astype(np.longdouble)

    def sm(r):
        e = np.exp(r - r.max())
        return e / e.sum()

    for b in range(6):
        p = sm(T[b, n[b]])
        if n[b] < 4:
            w = np.maximum(p - sm(D[b, n[b]]), 0)
            assert tw.residual[b] == 1
        else:
            w = p
            assert tw.residual[b] == 0
        np.testing.assert_allclose(tw.w[b], w.astype(np.float64), rtol=0, atol=1e-15 * float(w.sum()))
        assert abs(tw.Z[b] - float(w.sum())) <= 1e-14 * float(w.sum())
    tt = oracle.terminal_weights("target", ci.target, "bf16", n)
    for b in range(6):
        p = sm(T[b, n[b]])
        np.testing.assert_allclose(tt.w[b], p.astype(np.float64), rtol=0, atol=1e-15)
    rows = ci.draft.reshape(-1, ci.V)[:7]
    ts = oracle.terminal_weights("sampler", rows, "bf16")
    R = synth.widen(rows, "bf16").astype(np.longdouble)
    for r in range(7):
        e = np.exp(R[r] - R[r].max())
        np.testing.assert_allclose(ts.w[r], e.astype(np.float64), rtol=1e-15, atol=0)
    x = rng.integers(0, 7)
    assert ts.Z[x] == pytest.approx(float(np.exp(R[x] - R[x].max()).sum()), rel=1e-13)


# ------------------------------------------- inverse CDF at full vocabulary
def test_oracle_inverse_cdf_precision_at_full_vocab():
    """At V = 128256 the oracle's draw agrees with the extended-precision
    inverse CDF whenever u*Z lies at least 1e-13*Z from a boundary: the
    oracle's own rounding (a sequential fp64 running sum over 128k terms) stays
    two orders below the near-tie window used for terminal draws.  Residual,
    bonus and draft-sampler rows of the exact B=32 workload."""
    rng = np.random.default_rng(91)
    ci = synth.exact_b32_k5()
    sub = slice(0, 3)
    T, Dr, x = ci.target[sub], ci.draft[sub], ci.tokens[sub]
    # two residual rows (the first drafts whose ratio r < 1 lets a uniform
    # reject them) and a bonus row
    r0 = oracle.exact(T, Dr, x, np.zeros((3, 6), np.float32), "bf16")
    assert (r0.accept_len == 5).all()
    rej = np.exp(r0.behavior_logprob[:, :5]) < 0.999
    n = np.array([np.flatnonzero(rej[0])[0], np.flatnonzero(rej[1])[-1], 5], np.int32)
    tw = oracle.terminal_weights("exact", T, "bf16", n, Dr)
    checked = 0
    for b in range(3):
        picks = near_boundary_uniforms(tw.w[b], tw.Z[b], BINS, 12, rng)
        m = len(picks)
        u = np.zeros((m, 6), np.float32)
        u[:, n[b]] = U_REJECT if n[b] < 5 else 0.0
        u[:, 5] = [p[0] for p in picks]
        r = oracle.exact(np.repeat(T[b:b + 1], m, 0), np.repeat(Dr[b:b + 1], m, 0),
                         np.repeat(x[b:b + 1], m, 0), u, "bf16", eps_sample=0.0)
        assert (r.accept_len == n[b]).all()
        for (uu, dist, want), tok in zip(picks, r.tokens[:, n[b]]):
            if abs(dist) >= 1e-13:
                assert tok == want, (b, uu, dist)
                checked += 1
    rows = Dr.reshape(-1, ci.V)[:2]
    ts = oracle.terminal_weights("sampler", rows, "bf16")
    for r_ in range(2):
        picks = near_boundary_uniforms(ts.w[r_], ts.Z[r_], BINS, 12, rng)
        u = np.array([p[0] for p in picks], np.float32)
        s = oracle.sample(np.repeat(rows[r_:r_ + 1], len(u), 0), u, "bf16", eps_sample=0.0)
        for (uu, dist, want), tok in zip(picks, s.tokens):
            if abs(dist) >= 1e-13:
                assert tok == want, (r_, uu, dist)
                checked += 1
    assert checked >= 100, checked
