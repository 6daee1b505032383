"""The seeded generators: bf16 rounding, draft-token law, tree shape, determinism."""
import numpy as np
import torch

import synth


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30], np.float32)])
    ours = synth.bf16_rne(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = synth.bf16_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_gumbel_max_tokens_follow_softmax():
    rng = np.random.default_rng(2)
    logits = np.array([1.0, 0.0, -1.0, 2.0, 0.5])
    n = 200000
    x = synth.gumbel_max_tokens(np.broadcast_to(logits, (n, 5)).copy(), rng)
    freq = np.bincount(x, minlength=5) / n
    p = np.exp(logits) / np.exp(logits).sum()
    assert np.abs(freq - p).max() < 5 * np.sqrt(p * (1 - p) / n).max()


def test_chain_inputs_deterministic_and_shaped():
    a = synth.chain_inputs(3, 5, 1000, "bf16", seed=9, useed=10)
    b = synth.chain_inputs(3, 5, 1000, "bf16", seed=9, useed=10)
    np.testing.assert_array_equal(a.target, b.target)
    np.testing.assert_array_equal(a.tokens, b.tokens)
    assert a.target.shape == (3, 6, 1000) and a.draft.shape == (3, 5, 1000)
    assert a.uniforms.shape == (3, 6) and a.uniforms.dtype == np.float32
    assert ((a.uniforms >= 0) & (a.uniforms < 1)).all()
    assert a.tokens.dtype == np.int32 and ((a.tokens >= 0) & (a.tokens < 1000)).all()
    c = synth.chain_inputs(3, 5, 1000, "bf16", seed=9, useed=10, rnd=1)
    assert not np.array_equal(a.target, c.target)


def test_tiny_exact_shapes():
    ci = synth.tiny_exact_v32(rounds=1000)
    assert ci.target.shape == (1000, 5, 32) and ci.target.dtype == np.float32
    assert ci.draft.shape == (1000, 4, 32)
    np.testing.assert_array_equal(
        ci.uniforms, np.random.default_rng(0).random((1000, 1, 5), dtype=np.float32).reshape(1000, 5))


def test_tree_shape_properties():
    rng = np.random.default_rng(3)
    for _ in range(20):
        par, rank = synth.make_tree(rng)
        assert par.shape == (61,) and par[0] == -1
        assert all(0 <= par[i] < i for i in range(1, 61))
        depth = np.zeros(61, int)
        for i in range(1, 61):
            depth[i] = depth[par[i]] + 1
        assert depth.max() <= 5
        assert (depth == 1).sum() == 4
        # at most topk children per parent
        assert np.bincount(par[1:], minlength=61).max() <= 4


def test_tree_inputs_sibling_tokens_distinct():
    ti = synth.tree_inputs(B=3, V=500, seed=7)
    for b in range(ti.B):
        kids = {}
        for i in range(1, ti.N):
            kids.setdefault(int(ti.parents[b, i]), []).append(int(ti.node_tok[b, i]))
        for toks in kids.values():
            assert len(toks) == len(set(toks))


def test_greedy_b8_construction_facts():
    ci = synth.greedy_chain_b8(V=2000)
    g = np.argmax(synth.bf16_to_f32(ci.target), -1)
    for b in range(ci.B):
        j = int(ci.expected_accept_len[b])
        assert list(ci.tokens[b, :j]) == list(g[b, :j])
        if j < ci.K:
            row = synth.bf16_to_f32(ci.target[b, j])
            assert row[ci.tokens[b, j]] < row.max()
