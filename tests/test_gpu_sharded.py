"""Vocabulary-sharded verification (spec_shard_* through the C ABI) on one GPU.

The G shards of a call run one after another on the same device and share
the gathered buffers, so the pipeline's result must equal the unsharded
oracle's on the full logits, to the same parity rule as the unsharded entry
points.  With G = 1 the sharded steps compute exactly what the unsharded call
does, so those results must match it bit for bit.
"""
import numpy as np
import pytest
import torch

import draft_verification_row_amd as sv
import draft_verification_row_amd.sharded as sh
import oracle
import synth
from parity import Tally, compare_chain, compare_tree, dev, dev_logits

pytestmark = pytest.mark.gpu


def _split(a: torch.Tensor, G: int):
    Vs = a.shape[-1] // G
    return [a[:, :, s * Vs:(s + 1) * Vs].contiguous() for s in range(G)]


def _exact_sharded(ci, G, **kw):
    T = _split(dev_logits(ci.target, ci.dtype), G)
    D = _split(dev_logits(ci.draft, ci.dtype), G)
    r = sh.verify_exact_sharded(T, D, dev(ci.tokens), dev(ci.uniforms), **kw)
    torch.cuda.synchronize()
    return r


def _greedy_sharded(ci, G, **kw):
    r = sh.verify_greedy_sharded(_split(dev_logits(ci.target, ci.dtype), G), dev(ci.tokens), **kw)
    torch.cuda.synchronize()
    return r


def _tree_sharded(ti, G, **kw):
    r = sh.verify_tree_sharded(_split(dev_logits(ti.target, ti.dtype), G), dev(ti.node_tok),
                               dev(ti.parents), dev(ti.num_nodes), **kw)
    torch.cuda.synchronize()
    return r


def _check_owner(res, G, V):
    """The reported owner is the shard whose columns hold the terminal token."""
    r, own = res
    n = r.accept_len.cpu().numpy()
    tok = r.tokens.cpu().numpy()
    y = tok[np.arange(len(n)), n]
    np.testing.assert_array_equal(own.cpu().numpy(), y // (V // G))


# ------------------------------------------------------------------ exact
def test_exact_b32_eight_shards():
    """B=32, K=5, V=128256 bf16 split over 8 shards of 16032 columns."""
    print("sharded exact B=32 g8", flush=True)
    ci = synth.exact_b32_k5()
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16")
    res = _exact_sharded(ci, 8)
    t = compare_chain(res.result, o, what="sharded exact B=32 g8")
    assert t.within_budget(), t
    _check_owner(res, 8, ci.V)


@pytest.mark.parametrize("B,K,V,G,dtype", [
    (6, 5, 20000, 4, "bf16"),      # 5000 columns per shard: two chunks, ragged
    (5, 3, 3 * 3001, 3, "bf16"),   # odd shard width: element path
    (4, 2, 12288, 2, "f32"),
    (3, 4, 128256, 16, "bf16"),    # 16 shards of 8016 columns
    (7, 1, 1000, 8, "bf16"),       # shards far smaller than one chunk
    (2, 6, 262144, 64, "f32"),     # the widest split: one tile and one chunk per shard
])
def test_exact_sharded_shapes(B, K, V, G, dtype):
    print(f"sharded exact B={B} K={K} V={V} G={G} {dtype}", flush=True)
    ci = synth.chain_inputs(B, K, V, dtype, seed=3000 + G, useed=4000 + V % 997)
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, dtype)
    res = _exact_sharded(ci, G)
    compare_chain(res.result, o, what=f"sharded exact {B},{K},{V},{G}")
    _check_owner(res, G, V)


def test_exact_one_shard_is_the_unsharded_call():
    ci = synth.chain_inputs(8, 5, 40000, "bf16", seed=91, useed=92)
    T, D = dev_logits(ci.target, "bf16"), dev_logits(ci.draft, "bf16")
    x, u = dev(ci.tokens), dev(ci.uniforms)
    a = sv.spec_verify_exact(T, D, x, u)
    b = sh.verify_exact_sharded([T], [D], x, u).result
    torch.cuda.synchronize()
    for f in ("tokens", "accept_len", "target_logprob", "behavior_logprob", "status"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


def test_exact_sharded_malformed_tokens():
    ci = synth.chain_inputs(4, 4, 8000, "bf16", seed=93, useed=94)
    ci.tokens = ci.tokens.copy()
    ci.tokens[1, 0] = ci.V          # first draft outside the vocabulary
    ci.tokens[2, 2] = -3
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16")
    res = _exact_sharded(ci, 4)
    compare_chain(res.result, o, what="sharded malformed")
    assert res.result.status.cpu().numpy()[1] == 1


def test_exact_sharded_reuses_buffers_across_calls():
    """Two calls in a row (the second smaller) give the oracle's results."""
    for (B, K, V, seed) in [(16, 5, 64000, 95), (3, 2, 16000, 96)]:
        ci = synth.chain_inputs(B, K, V, "bf16", seed=seed, useed=seed + 1)
        o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16")
        compare_chain(_exact_sharded(ci, 8).result, o, what=f"sharded reuse {B},{K},{V}")


# ----------------------------------------------------------------- greedy
@pytest.mark.parametrize("G", [1, 2, 8])
def test_greedy_b8_sharded(G):
    print(f"sharded greedy B=8 G={G}", flush=True)
    ci = synth.greedy_chain_b8()
    o = oracle.greedy(ci.target, ci.tokens, "bf16")
    np.testing.assert_array_equal(o.accept_len, ci.expected_accept_len)
    compare_chain(_greedy_sharded(ci, G), o, what=f"sharded greedy G={G}")
    r = _greedy_sharded(ci, G, logprobs=False)
    compare_chain(r, o, logprobs=False, what=f"sharded greedy G={G} no-logprob")


def test_greedy_sharded_ties_across_shards():
    """Equal maxima in different shards: the lowest vocabulary index wins."""
    B, K, V, G = 4, 3, 4096, 4
    rng = np.random.default_rng(97)
    t = synth.bf16_rne(rng.standard_normal((B, K + 1, V), dtype=np.float32))
    top = synth.bf16_rne(np.array([8.0], np.float32))[0]
    for b in range(B):
        for r in range(K + 1):
            cols = rng.choice(V, size=3, replace=False)
            t[b, r, cols] = top
    g = np.argmax(synth.bf16_to_f32(t), -1)
    x = g[:, :K].astype(np.int32).copy()
    x[1, 1] = (x[1, 1] + 1) % V
    ci = synth.ChainInputs("ties", "bf16", B, K, V, t, None, x,
                           np.zeros((B, K + 1), np.float32))
    o = oracle.greedy(ci.target, ci.tokens, "bf16")
    compare_chain(_greedy_sharded(ci, G), o, what="sharded ties")


def test_greedy_one_shard_is_the_unsharded_call():
    ci = synth.chain_inputs(8, 5, 30011, "bf16", seed=98, useed=99, with_draft=False)
    T, x = dev_logits(ci.target, "bf16"), dev(ci.tokens)
    a = sv.spec_verify_greedy(T, x)
    b = sh.verify_greedy_sharded([T], x)
    torch.cuda.synchronize()
    for f in ("tokens", "accept_len", "target_logprob", "behavior_logprob", "status"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    # without log-probs the unsharded stream reads 8 KiB tiles, the shard's
    # 16 KiB: the argmax (exact) and so every output still agree
    a = sv.spec_verify_greedy(T, x, logprobs=False)
    b = sh.verify_greedy_sharded([T], x, logprobs=False)
    torch.cuda.synchronize()
    for f in ("tokens", "accept_len", "status"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


# ------------------------------------------------------------------- tree
@pytest.mark.parametrize("G", [1, 8])
def test_tree_b8_sharded(G):
    print(f"sharded tree B=8 G={G}", flush=True)
    ti = synth.tree_b8_n61()
    o = oracle.tree(ti.target, ti.node_tok, ti.parents, "bf16", num_nodes=ti.num_nodes)
    compare_tree(_tree_sharded(ti, G), o, what=f"sharded tree G={G}")
    compare_tree(_tree_sharded(ti, G, logprobs=False), o, logprobs=False,
                 what=f"sharded tree G={G} no-logprob")


def test_tree_sharded_partial_counts_and_bad_parents():
    ti = synth.tree_inputs(B=6, V=3000, seed=75)
    ti.num_nodes = np.array([61, 1, 2, 30, 60, 17], np.int32)
    ti.parents = ti.parents.copy()
    ti.parents[3, 5] = 40
    ti.node_tok = ti.node_tok.copy()
    ti.node_tok[4, 7] = 10 ** 6
    o = oracle.tree(ti.target, ti.node_tok, ti.parents, "bf16", num_nodes=ti.num_nodes)
    compare_tree(_tree_sharded(ti, 4), o, what="sharded tree edge")


# ------------------------------------------------------------------ power
@pytest.mark.parametrize("alpha", [0.5, 2.0])
def test_power_b32_eight_shards(alpha):
    print(f"sharded power B=32 g8 alpha={alpha}", flush=True)
    ci = synth.exact_b32_k5()
    o = oracle.power(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16", alpha)
    T = _split(dev_logits(ci.target, "bf16"), 8)
    D = _split(dev_logits(ci.draft, "bf16"), 8)
    res = sh.verify_power_sharded(T, D, dev(ci.tokens), dev(ci.uniforms), alpha)
    torch.cuda.synchronize()
    t = compare_chain(res.result, o, what=f"sharded power {alpha}")
    assert t.within_budget(), t
    _check_owner(res, 8, ci.V)


def test_power_one_shard_is_the_unsharded_call():
    ci = synth.chain_inputs(8, 5, 30000, "bf16", seed=101, useed=102)
    T, D = dev_logits(ci.target, "bf16"), dev_logits(ci.draft, "bf16")
    x, u = dev(ci.tokens), dev(ci.uniforms)
    a = sv.spec_verify_power(T, D, x, u, 0.7)
    b = sh.verify_power_sharded([T], [D], x, u, 0.7).result
    torch.cuda.synchronize()
    for f in ("tokens", "accept_len", "target_logprob", "behavior_logprob", "status"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


def test_power_sharded_ragged_fp32():
    ci = synth.chain_inputs(5, 3, 3 * 2999, "f32", seed=103, useed=104)
    o = oracle.power(ci.target, ci.draft, ci.tokens, ci.uniforms, "f32", 1.5)
    res = _pq_power(ci, 3, 1.5)
    compare_chain(res.result, o, what="sharded power fp32 ragged")


def _pq_power(ci, G, alpha):
    T = _split(dev_logits(ci.target, ci.dtype), G)
    D = _split(dev_logits(ci.draft, ci.dtype), G)
    r = sh.verify_power_sharded(T, D, dev(ci.tokens), dev(ci.uniforms), alpha)
    torch.cuda.synchronize()
    return r


# ---------------------------------------------------------------- relaxed
def _relaxed_sharded(ci, G):
    T = _split(dev_logits(ci.target, ci.dtype), G)
    r = sh.verify_relaxed_sharded(T, dev(ci.tokens), dev(ci.uniforms), ci.tau, ci.top_k)
    torch.cuda.synchronize()
    return r


def test_relaxed_b64_eight_shards():
    """B=64, K=8, V=151936 bf16 over 8 shards of 18992 columns."""
    print("sharded relaxed B=64 g8", flush=True)
    ci = synth.large_b64_k8()
    o = oracle.relaxed(ci.target, ci.tokens, ci.uniforms, "bf16", ci.tau, ci.top_k)
    res = _relaxed_sharded(ci, 8)
    t = compare_chain(res.result, o, what="sharded relaxed B=64")
    assert t.within_budget(), t
    _check_owner(res, 8, ci.V)


@pytest.mark.parametrize("tau,k,G", [(2.0, 0, 4), (-1.0, 0, 4), (2.0, 1, 5), (0.05, 2, 2),
                                     (0.5, 10, 8)])
def test_relaxed_sharded_special_cases(tau, k, G):
    """Reject-all, accept-all, greedy-like, and rank tests whose top-k members
    lie in other shards than the drafted token."""
    ci = synth.chain_inputs(16, 6, 20000, "bf16", seed=61, useed=62, d_noise=0.3)
    ci.tau, ci.top_k = tau, k
    o = oracle.relaxed(ci.target, ci.tokens, ci.uniforms, "bf16", tau, k)
    compare_chain(_relaxed_sharded(ci, G).result, o, what=f"sharded relaxed tau={tau} k={k} G={G}")


def test_relaxed_one_shard_is_the_unsharded_call():
    ci = synth.chain_inputs(8, 5, 30000, "bf16", seed=105, useed=106)
    T, x, u = dev_logits(ci.target, "bf16"), dev(ci.tokens), dev(ci.uniforms)
    a = sv.spec_verify_relaxed(T, x, u, 0.1, 4)
    b = sh.verify_relaxed_sharded([T], x, u, 0.1, 4).result
    torch.cuda.synchronize()
    for f in ("tokens", "accept_len", "target_logprob", "behavior_logprob", "status"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


def test_relaxed_sharded_malformed_and_fp32():
    ci = synth.chain_inputs(5, 4, 4 * 1501, "f32", seed=107, useed=108)
    ci.tokens = ci.tokens.copy()
    ci.tokens[2, 0] = ci.V + 5
    o = oracle.relaxed(ci.target, ci.tokens, ci.uniforms, "f32", ci.tau, ci.top_k)
    compare_chain(_relaxed_sharded(ci, 4).result, o, what="sharded relaxed fp32 malformed")
