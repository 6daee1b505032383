"""GPU parity of the power acceptance rule (spec_verify_power) against the
fp64 oracle (nanospec README, acceptance rules: accept with probability
min(1, p/rest)^alpha, read with rest = q; y ~ p_n after a rejection)."""
import numpy as np
import pytest
import torch

import draft_verification_row_amd as sv
import oracle
import synth

from parity import NEAR_TIE_BUDGET, compare_chain, dev, dev_logits

pytestmark = pytest.mark.gpu


def _power(ci, alpha, **kw):
    r = sv.spec_verify_power(dev_logits(ci.target, ci.dtype), dev_logits(ci.draft, ci.dtype),
                             dev(ci.tokens), dev(ci.uniforms), alpha, **kw)
    torch.cuda.synchronize()
    return r


def _check(ci, alpha, what):
    o = oracle.power(ci.target, ci.draft, ci.tokens, ci.uniforms, ci.dtype, alpha)
    t = compare_chain(_power(ci, alpha), o, what=what)
    return t, o


@pytest.mark.parametrize("alpha", [0.5, 1.0, 2.0])
def test_power_b32(alpha):
    """The benchmark batch, B=32 K=5 V=128256 bf16, at three exponents."""
    t, o = _check(synth.exact_b32_k5(), alpha, f"power B=32 alpha={alpha}")
    assert t.flagged <= NEAR_TIE_BUDGET * max(t.decisions, 1) + 3


def test_power_b64():
    t, o = _check(synth.large_b64_k8(), 0.7, "power B=64")
    assert t.flagged <= NEAR_TIE_BUDGET * max(t.decisions, 1) + 3


def test_power_alpha_zero_accepts_all():
    ci = synth.chain_inputs(16, 4, 5000, "bf16", seed=91, useed=92)
    r = _power(ci, 0.0)
    assert (r.accept_len.cpu().numpy() == 4).all()
    _check(ci, 0.0, "alpha 0")


def test_power_alpha_one_accepts_as_exact():
    """alpha = 1: the accepted prefixes equal the exact rule's."""
    ci = synth.chain_inputs(32, 5, 20000, "bf16", seed=93, useed=94)
    p = _power(ci, 1.0)
    e = sv.spec_verify_exact(dev_logits(ci.target, "bf16"), dev_logits(ci.draft, "bf16"),
                             dev(ci.tokens), dev(ci.uniforms))
    torch.cuda.synchronize()
    assert torch.equal(p.accept_len, e.accept_len)


def test_power_small_fp32_many_requests():
    ci = synth.tiny_exact_v32()
    _check(ci, 1.5, "power tiny V=32")


@pytest.mark.parametrize("B,K,V,dtype", [(3, 1, 1, "f32"), (5, 3, 7, "bf16"), (2, 5, 8193, "bf16"),
                                         (4, 4, 1000, "f32"), (1, 5, 128257, "bf16")])
def test_power_ragged(B, K, V, dtype):
    ci = synth.chain_inputs(B, K, V, dtype, seed=B * 31 + V, useed=K + 7)
    _check(ci, 0.8, f"power ragged {B},{K},{V},{dtype}")


def test_power_out_of_range_tokens():
    ci = synth.chain_inputs(6, 4, 3000, "bf16", seed=95, useed=96)
    ci.tokens = ci.tokens.copy()
    ci.tokens[0, 0] = -3
    ci.tokens[2, 1] = 3000
    _check(ci, 1.3, "power oor")
    assert _power(ci, 1.3).status.cpu().numpy()[0] == 1
