"""GPU parity of the draft-token sampler (spec_sample_drafts) against the fp64
oracle: one inverse-CDF draw per row at the row's uniform, and its log-prob
(spec-decode README, "How it works": the draft samples its tokens from q)."""
import numpy as np
import pytest
import torch

import draft_verification_row_amd as sv
import oracle
import synth

from parity import LOGPROB_TOL, dev_logits

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _compare(x, u, dtype, what, max_flags=None):
    """Tokens bit-exact and log-probs within LOGPROB_TOL on every row the
    oracle does not flag as near a CDF boundary; flags strictly under 1e-4 of
    the draws (none below 1e4 draws)."""
    o = oracle.sample(x, u, dtype)
    r = sv.spec_sample_drafts(dev_logits(x, dtype), _dev(u))
    torch.cuda.synchronize()
    tok = r.tokens.cpu().numpy()
    lq = r.logprob.cpu().numpy()
    st = r.status.cpu().numpy()
    ok = o.flag == 0
    assert (st == 0).all(), what
    bad = np.flatnonzero((tok != o.tokens) & ok)
    assert bad.size == 0, f"{what}: {bad.size} unflagged token mismatches, first at {bad[:5]}"
    d = np.abs(lq - o.logq)[ok]
    assert d.size == 0 or d.max() < LOGPROB_TOL, f"{what}: logprob diff {d.max()}"
    if max_flags is not None:
        assert o.flag.sum() <= max_flags, f"{what}: {o.flag.sum()} near-boundary flags"
    else:
        assert o.flag.sum() < 1e-4 * o.flag.size, f"{what}: {o.flag.sum()} near-boundary flags"
    return tok


def test_sampler_b32_draft_rows():
    """The benchmark batch's draft logits, [32][5][128256] bf16, one draw per row."""
    ci = synth.exact_b32_k5()
    u = np.random.default_rng(203).random(ci.tokens.shape, dtype=np.float32)
    _compare(ci.draft, u, "bf16", "B=32 draft rows")


def test_sampler_b64_draft_rows():
    ci = synth.large_b64_k8()
    u = np.random.default_rng(205).random(ci.tokens.shape, dtype=np.float32)
    _compare(ci.draft, u, "bf16", "B=64 draft rows")


def test_sampler_small_fp32_many_rows():
    """The tiny exact workload's shape: V=32 fp32, 1000 x 4 rows."""
    ci = synth.tiny_exact_v32()
    u = np.random.default_rng(201).random(ci.tokens.shape, dtype=np.float32)
    _compare(ci.draft, u, "f32", "tiny V=32 draft rows")


@pytest.mark.parametrize("V", [1, 2, 7, 8, 4095, 4097, 8193, 128257])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sampler_ragged_vocab(V, dtype):
    rng = np.random.default_rng(V * 7 + len(dtype))
    x32 = (3.0 * rng.standard_normal((3, 5, V))).astype(np.float32)
    x = synth.bf16_rne(x32) if dtype == "bf16" else x32
    u = rng.random((3, 5), dtype=np.float32)
    _compare(x, u, dtype, f"ragged V={V} {dtype}")


def test_sampler_grid_law():
    """A midpoint grid of 4000 uniforms over one V=8 row: bit-exact with the
    oracle, whose law on this grid is pinned to softmax within 1/4000."""
    x = np.array([0.5, -1.0, 2.0, 0.0, 1.25, -3.0, 0.75, 1.0], np.float32)
    M = 4000
    X = np.broadcast_to(x, (M, 8)).copy()
    u = ((np.arange(M) + 0.5) / M).astype(np.float32)
    _compare(X, u, "f32", "grid law", max_flags=0)


def test_sampler_masked_and_misaligned():
    rng = np.random.default_rng(207)
    x = (2.0 * rng.standard_normal((40, 3001))).astype(np.float32)
    x[:, 100:1500] = -np.inf
    u = rng.random(40, dtype=np.float32)
    tok = _compare(x, u, "f32", "masked")
    assert not ((tok >= 100) & (tok < 1500)).any()
    # a contiguous view that starts off the 16-byte grid takes the element path
    flat = torch.zeros(40 * 3001 + 1, dtype=torch.float32, device="cuda")
    view = flat[1:].view(40, 3001)
    view.copy_(torch.from_numpy(x).cuda())
    assert view.is_contiguous() and view.data_ptr() % 16 != 0
    r = sv.spec_sample_drafts(view, _dev(u))
    torch.cuda.synchronize()
    assert (r.tokens.cpu().numpy() == tok).all()


def test_sampler_deterministic():
    ci = synth.chain_inputs(8, 3, 20000, "bf16", seed=211, useed=212)
    X = dev_logits(ci.draft, "bf16")
    u = _dev(np.random.default_rng(213).random((8, 3), dtype=np.float32))
    a = sv.spec_sample_drafts(X, u)
    b = sv.spec_sample_drafts(X, u)
    torch.cuda.synchronize()
    assert torch.equal(a.tokens, b.tokens) and torch.equal(a.logprob, b.logprob)
