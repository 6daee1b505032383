"""Parity at scale: enough decisions to show the near-tie budget, not just
assert it.

Each workload runs many rounds against the fp64 oracle, reusing a few seeded
logit sets with fresh uniforms every round (and, for the B=32 exact workload,
fresh draft tokens drawn from the draft softmax every round).  Every round is
compared element by element (tokens and accepted counts bit-exact outside
flagged near-ties, log-probs within 1e-4); the flagged near-ties of all rounds
of a workload are pooled and must stay strictly under 1e-4 of the pooled
decisions (mini-sglang PR #134, "Accuracy Tests": the speculative path must
reproduce the reference outputs; spec: near-ties counted and kept under
1e-4 of decisions).

Sizes: B=32 K=5 V=128256 exact, 300 rounds (six logit sets x 50); B=64 K=8
V=151936 exact and relaxed, 60 rounds each (three sets x 20); B=8 greedy,
100 rounds (five sets x 20 token draws); the draft sampler on the 160 draft
rows of the B=32 workload, 320 uniform draws each (51,200 draws).
"""
import numpy as np
import pytest
import torch

import draft_verification_row_amd as sv
import oracle
import synth
from parity import NEAR_TIE_BUDGET, Tally, compare_chain, dev, dev_logits

pytestmark = pytest.mark.gpu

POOL = {}


def _pool(key):
    return POOL.setdefault(key, Tally())


def _report(key, t, extra=""):
    print(f"SCALE {key}: requests {t.requests} decisions {t.decisions} flagged {t.flagged} "
          f"({t.flagged / max(t.decisions, 1):.2e} of decisions){extra}", flush=True)


def _budget(key, min_decisions):
    t = POOL.get(key)
    assert t is not None, f"{key}: its rounds did not run"
    _report(key + " (pooled)", t)
    assert t.decisions >= min_decisions, t
    assert t.flagged < NEAR_TIE_BUDGET * t.decisions, t


# ------------------------------------------------------------ B=32 exact
@pytest.mark.parametrize("s", range(6))
def test_exact_b32_k5_rounds(s):
    """50 rounds on logit set s: fresh draft tokens and uniforms each round."""
    ci = synth.exact_b32_k5(rnd=s)
    print(f"exact B=32 set {s}", flush=True)
    T, D = dev_logits(ci.target, "bf16"), dev_logits(ci.draft, "bf16")
    rng = np.random.default_rng([3, 1000 + s])
    tally, acc = Tally(), []
    for r in range(50):
        x = ci.tokens if r == 0 else synth.redraw_draft_tokens(ci.draft, "bf16", rng)
        u = ci.uniforms if r == 0 else rng.random((ci.B, ci.K + 1), dtype=np.float32)
        res = sv.spec_verify_exact(T, D, dev(x), dev(u))
        torch.cuda.synchronize()
        o = oracle.exact(ci.target, ci.draft, x, u, "bf16")
        tally.add(compare_chain(res, o, what=f"exact B=32 set {s} round {r}"))
        acc.append(o.accept_len.mean())
    _pool("exact_b32_k5").add(tally)
    _report(f"exact_b32_k5 set {s}", tally, f" mean accepted {np.mean(acc):.3f}")


def test_exact_b32_k5_budget():
    _budget("exact_b32_k5", 35000)


# ------------------------------------------------- B=64 exact and relaxed
@pytest.mark.parametrize("s", range(3))
def test_large_b64_k8_rounds(s):
    """20 rounds of the exact and the relaxed rule on logit set s."""
    ci = synth.large_b64_k8(rnd=s)
    print(f"B=64 K=8 set {s}", flush=True)
    T, D, x = dev_logits(ci.target, "bf16"), dev_logits(ci.draft, "bf16"), dev(ci.tokens)
    rng = np.random.default_rng([5, 1000 + s])
    te, tr = Tally(), Tally()
    for r in range(20):
        u = ci.uniforms if r == 0 else rng.random((ci.B, ci.K + 1), dtype=np.float32)
        ud = dev(u)
        re_ = sv.spec_verify_exact(T, D, x, ud)
        rr = sv.spec_verify_relaxed(T, x, ud, ci.tau, ci.top_k)
        torch.cuda.synchronize()
        oe = oracle.exact(ci.target, ci.draft, ci.tokens, u, "bf16")
        orl = oracle.relaxed(ci.target, ci.tokens, u, "bf16", ci.tau, ci.top_k)
        te.add(compare_chain(re_, oe, what=f"exact B=64 set {s} round {r}"))
        tr.add(compare_chain(rr, orl, what=f"relaxed B=64 set {s} round {r}"))
    _pool("large_b64_k8 exact").add(te)
    _pool("large_b64_k8 relaxed").add(tr)
    _report(f"large_b64_k8 exact set {s}", te)
    _report(f"large_b64_k8 relaxed set {s}", tr)


def test_large_b64_k8_budget():
    _budget("large_b64_k8 exact", 12000)
    _budget("large_b64_k8 relaxed", 7000)


# ---------------------------------------------------------- B=8 greedy
@pytest.mark.parametrize("s", range(5))
def test_greedy_b8_rounds(s):
    """20 token draws on logit set s, each with its own accepted length j_b per
    request (the workload's construction), and the oracle agreeing with it."""
    base = synth.greedy_chain_b8(rnd=s)
    print(f"greedy B=8 set {s}", flush=True)
    T = dev_logits(base.target, "bf16")
    tw = synth.bf16_to_f32(base.target)
    g = np.argmax(tw, -1)
    below = [[np.flatnonzero(tw[b, j] < tw[b, j].max()) for j in range(base.K)] for b in range(base.B)]
    rng = np.random.default_rng([2, 1000 + s])
    for r in range(20):
        jb = rng.integers(0, base.K + 1, size=base.B)
        x = rng.integers(0, base.V, size=(base.B, base.K)).astype(np.int32)
        for b in range(base.B):
            x[b, :jb[b]] = g[b, :jb[b]]
            if jb[b] < base.K:
                x[b, jb[b]] = below[b][jb[b]][rng.integers(0, below[b][jb[b]].size)]
        o = oracle.greedy(base.target, x, "bf16")
        np.testing.assert_array_equal(o.accept_len, jb)
        for lp in (True, False):
            res = sv.spec_verify_greedy(T, dev(x), logprobs=lp)
            torch.cuda.synchronize()
            compare_chain(res, o, logprobs=lp, what=f"greedy B=8 set {s} round {r} logprobs={lp}")


# ------------------------------------------------------- draft sampler
@pytest.mark.parametrize("s", range(4))
def test_sampler_draws(s):
    """80 uniform sets over the 160 draft rows of B=32 logit set s: 12,800
    draws per set, 51,200 in all."""
    ci = synth.exact_b32_k5(rnd=s)
    print(f"sampler set {s}", flush=True)
    rows = ci.draft.reshape(-1, ci.V)
    X = dev_logits(rows, "bf16")
    rng = np.random.default_rng([203, s])
    t = Tally()
    worst = 0.0
    for r in range(80):
        u = rng.random(rows.shape[0], dtype=np.float32)
        res = sv.spec_sample_drafts(X, dev(u))
        torch.cuda.synchronize()
        o = oracle.sample(rows, u, "bf16")
        tok, lq = res.tokens.cpu().numpy(), res.logprob.cpu().numpy()
        ok = o.flag == 0
        bad = np.flatnonzero((tok != o.tokens) & ok)
        assert bad.size == 0, f"sampler set {s} round {r}: unflagged mismatches at rows {bad[:5]}"
        if ok.any():
            worst = max(worst, float(np.abs(lq - o.logq)[ok].max()))
        t.add(Tally(requests=rows.shape[0], decisions=rows.shape[0], flagged=int(o.flag.sum())))
    assert worst < 1e-4, worst
    _pool("sampler").add(t)
    _report(f"sampler set {s}", t, f" max |dlogq| {worst:.2e}")


def test_sampler_budget():
    _budget("sampler", 50000)
