"""The multi-round driver on the GPU (spec_sample_drafts + spec_verify_exact
through the C ABI) against the oracle's driver on the same uniforms, and its
emitted transitions against the target chain."""
import numpy as np
import pytest
import torch

import draft_verification_row_amd.markov as mk
import oracle
import synth
from parity import dev, dev_logits
from test_markov_pins import chi2_pvalue, softmax64, transition_counts

pytestmark = pytest.mark.gpu


def _run(m):
    tr = mk.generate_speculative(dev_logits(m.target, m.dtype), dev_logits(m.draft, m.dtype),
                                 dev(m.start), dev(m.u_draft), dev(m.u_verify))
    torch.cuda.synchronize()
    return tr.emitted.cpu().numpy(), tr.accept_len.cpu().numpy()


@pytest.mark.parametrize("V,B,K,rounds,dtype", [
    (32, 64, 4, 40, "bf16"),     # the README example's vocabulary and k
    (4096, 32, 4, 20, "bf16"),
    (100, 48, 2, 30, "f32"),
    (7, 16, 8, 10, "bf16"),
])
def test_driver_matches_the_oracle_driver(V, B, K, rounds, dtype):
    print(f"markov driver V={V} B={B} K={K} rounds={rounds} {dtype}", flush=True)
    m = synth.markov_inputs(V, B, K, rounds, dtype, seed=V + K)
    o = oracle.speculative_generate(m.target, m.draft, m.start, m.u_draft, m.u_verify, dtype)
    em, ln = _run(m)
    flagged = 0
    for b in range(B):
        f = int(o.flag_round[b])
        upto = rounds if f < 0 else f  # rounds before a flagged near tie must agree exactly
        flagged += f >= 0
        np.testing.assert_array_equal(ln[:upto, b], o.accept_len[:upto, b])
        np.testing.assert_array_equal(em[:upto, b], o.emitted[:upto, b])
    assert flagged <= 1


def test_driver_transitions_follow_the_target_chain():
    m = synth.markov_inputs(6, 512, 3, 30, "bf16", seed=21)
    em, ln = _run(m)
    C = transition_counts(m.start, em, ln, m.V)
    assert chi2_pvalue(C, softmax64(m.target, "bf16")) > 1e-4
    stats = mk.trace_stats(ln, m.K)
    assert stats["tokens"] == int(C.sum())
    assert 1.0 <= stats["tokens_per_target_pass"] <= m.K + 1


def test_graph_replays_match_the_eager_driver():
    """SpeculativeGraph: each replay, with new start tokens and uniforms
    copied in and eager driver runs between the replays, equals the eager
    driver on the same inputs bit for bit."""
    V, B, K, rounds = 512, 16, 3, 12
    m = synth.markov_inputs(V, B, K, rounds, "bf16", seed=31)
    other = synth.markov_inputs(V, B, K, rounds, "bf16", seed=32)
    P, Q = dev_logits(m.target, "bf16"), dev_logits(m.draft, "bf16")
    inputs = [(dev(m.start), dev(m.u_draft), dev(m.u_verify)),
              (dev(other.start), dev(other.u_draft), dev(other.u_verify))]
    eager = []
    for st, ud, uv in inputs:
        tr = mk.generate_speculative(P, Q, st, ud, uv)
        eager.append((tr.emitted.clone(), tr.accept_len.clone()))
    torch.cuda.synchronize()
    g = mk.SpeculativeGraph(P, Q, B, K, rounds)
    for rep, i in enumerate([0, 1, 0]):
        print(f"graph replay {rep} inputs {i}", flush=True)
        tr = g.run(*inputs[i])
        torch.cuda.synchronize()
        assert torch.equal(tr.emitted, eager[i][0]), f"replay {rep}"
        assert torch.equal(tr.accept_len, eager[i][1]), f"replay {rep}"
        # eager work between replays, on the other tables
        mk.generate_speculative(dev_logits(other.target, "bf16"), dev_logits(other.draft, "bf16"),
                                *inputs[1 - i])
        torch.cuda.synchronize()
