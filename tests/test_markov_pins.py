"""Pins of the multi-round driver (oracle.speculative_generate) against facts
fixed by the mathematics, not by another implementation:

* the emitted sequence is a sample of the target Markov chain (the
  spec-decode README's "Provably exact": the output is distributed as
  target-only sampling), so per state the emitted transitions follow the
  target's next-token distribution (chi-square);
* the accepted drafts of a round have the closed-form mean E_K(s):
  E_0 = 0, E_k(s) = sum_x min(p(x|s), q(x|s)) * (1 + E_{k-1}(x)), since the
  first draft x is proposed with q(x|s) and kept with min(1, p/q).

Expected values come from fp64 softmax of the stored tables only.
"""
import numpy as np
import pytest
from scipy import stats

import oracle
import synth


def softmax64(t, dtype):
    w = synth.widen(t, dtype).astype(np.float64)
    w = np.exp(w - w.max(-1, keepdims=True))
    return w / w.sum(-1, keepdims=True)


def transition_counts(start, emitted, accept_len, V):
    rounds, B, _ = emitted.shape
    C = np.zeros((V, V), np.int64)
    for b in range(B):
        seq = [int(start[b])]
        for r in range(rounds):
            seq += [int(t) for t in emitted[r, b, : accept_len[r, b] + 1]]
        np.add.at(C, (np.array(seq[:-1]), np.array(seq[1:])), 1)
    return C


def chi2_pvalue(C, P):
    stat, df = 0.0, 0
    for s in range(P.shape[0]):
        n = C[s].sum()
        if n == 0:
            continue
        e = n * P[s]
        keep = e > 0
        stat += ((C[s][keep] - e[keep]) ** 2 / e[keep]).sum()
        df += keep.sum() - 1
    return stats.chi2.sf(stat, df)


def expected_accepts(P, Q, K):
    A = np.minimum(P, Q)
    E = np.zeros(P.shape[0])
    for _ in range(K):
        E = A @ (1.0 + E)
    return E


def test_emitted_transitions_follow_the_target_chain():
    m = synth.markov_inputs(6, 512, 3, 30, "bf16", seed=11)
    tr = oracle.speculative_generate(m.target, m.draft, m.start, m.u_draft, m.u_verify, "bf16")
    assert (tr.flag_round < 0).all()
    C = transition_counts(m.start, tr.emitted, tr.accept_len, m.V)
    assert C.sum() > 30000
    P = softmax64(m.target, "bf16")
    assert chi2_pvalue(C, P) > 1e-4
    # the draft chain is a different law: the same counts reject it
    assert chi2_pvalue(C, softmax64(m.draft, "bf16")) < 1e-6


def test_first_round_accepts_match_the_closed_form_mean():
    K = 3
    m = synth.markov_inputs(6, 20000, K, 1, "bf16", seed=12)
    tr = oracle.speculative_generate(m.target, m.draft, m.start, m.u_draft, m.u_verify, "bf16")
    E = expected_accepts(softmax64(m.target, "bf16"), softmax64(m.draft, "bf16"), K)
    d = tr.accept_len[0] - E[m.start]
    assert abs(d.mean()) < 4 * d.std() / np.sqrt(d.size)
    assert 0 < E.min() and E.max() < K


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rounds_chain_through_the_last_emitted_token(dtype):
    """Each round emits accepted + 1 tokens, -1 after them, and its drafts start
    where the previous round's output ended (re-run of round r alone from that
    token reproduces it)."""
    m = synth.markov_inputs(40, 16, 4, 6, dtype, seed=13)
    tr = oracle.speculative_generate(m.target, m.draft, m.start, m.u_draft, m.u_verify, dtype)
    B = m.B
    for r in range(m.rounds):
        n = tr.accept_len[r]
        for b in range(B):
            assert (tr.emitted[r, b, : n[b] + 1] >= 0).all()
            assert (tr.emitted[r, b, n[b] + 1:] == -1).all()
    last = tr.emitted[2, np.arange(B), tr.accept_len[2]]
    again = oracle.speculative_generate(m.target, m.draft, last, m.u_draft[3:4], m.u_verify[3:4], dtype)
    np.testing.assert_array_equal(again.emitted[0], tr.emitted[3])
