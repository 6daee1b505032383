"""Pins of the fp64 oracle to facts other than itself.

Each test ties one oracle function to something the pages or mathematics fix:
hand-worked examples (tests/golden), closed forms, library routines the C
oracle does not call (numpy argmax / searchsorted, torch log_softmax), special
cases that reduce to another rule, and brute-force enumeration on tiny inputs.
None of these tests calls the HIP library.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def softmax64(a):
    t = torch.from_numpy(np.asarray(a, dtype=np.float64))
    return torch.softmax(t, dim=-1).numpy()


def log_softmax64(a):
    t = torch.from_numpy(np.asarray(a, dtype=np.float64))
    return torch.log_softmax(t, dim=-1).numpy()


def logs32(p):
    return np.log(np.asarray(p, dtype=np.float64)).astype(np.float32)


# ---------------------------------------------------------------------------
# hand-worked examples (tests/golden/worked_examples.json)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", GOLD["exact"], ids=lambda c: c["why"][:30])
def test_exact_worked_examples(orc, case):
    T = logs32(case["p"])[None]
    D = logs32(case["q"])[None]
    x = np.array([case["x"]], np.int32)
    u = np.array([case["u"]], np.float32)
    r = orc.exact(T, D, x, u, "f32")
    L = case["accept_len"] + 1
    assert r.accept_len[0] == case["accept_len"]
    assert list(r.tokens[0, :L]) == case["tokens"]
    np.testing.assert_allclose(r.target_logprob[0, :L], case["target_logprob"], atol=1e-6)
    np.testing.assert_allclose(r.behavior_logprob[0, :L], case["behavior_logprob"], atol=1e-6)
    assert r.flag[0] == -1


def _rows_with_argmax(argmaxes, V, rng):
    rows = rng.uniform(-1.0, 1.0, size=(len(argmaxes), V)).astype(np.float32)
    for i, a in enumerate(argmaxes):
        rows[i, a] = 5.0
    return rows


@pytest.mark.parametrize("case", GOLD["greedy"], ids=lambda c: c["why"][:30])
def test_greedy_worked_examples(orc, case):
    rng = np.random.default_rng(5)
    T = _rows_with_argmax(case["argmax_rows"], case["V"], rng)[None]
    r = orc.greedy(T, np.array([case["x"]], np.int32), "f32")
    assert r.accept_len[0] == case["accept_len"]
    assert list(r.tokens[0, : case["accept_len"] + 1]) == case["tokens"]


@pytest.mark.parametrize("case", GOLD["relaxed"], ids=lambda c: c["why"][:30])
def test_relaxed_worked_examples(orc, case):
    T = logs32(case["p"])[None]
    r = orc.relaxed(T, np.array([case["x"]], np.int32), np.array([case["u"]], np.float32), "f32",
                    case["tau"], case["top_k"])
    L = case["accept_len"] + 1
    assert r.accept_len[0] == case["accept_len"]
    assert list(r.tokens[0, :L]) == case["tokens"]
    np.testing.assert_allclose(r.target_logprob[0, :L], case["target_logprob"], atol=1e-6)
    np.testing.assert_allclose(r.behavior_logprob[0, :L], case["behavior_logprob"], atol=1e-6)


@pytest.mark.parametrize("case", GOLD["tree"], ids=lambda c: c["why"][:30])
def test_tree_worked_examples(orc, case):
    rng = np.random.default_rng(6)
    T = _rows_with_argmax(case["argmax_rows"], case["V"], rng)[None]
    r = orc.tree(T, np.array([case["node_tokens"]], np.int32), np.array([case["parents"]], np.int32),
                 "f32")
    d = case["accept_len"]
    assert r.accept_len[0] == d
    assert list(r.path[0, :d]) == case["path"]
    assert list(r.tokens[0, : d + 1]) == case["tokens"]


# ---------------------------------------------------------------------------
# greedy scenarios (mini-sglang PR #134, "Accuracy Tests")
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K", [1, 2, 5, 8])
def test_greedy_scenarios(orc, K):
    """all-correct + bonus, all-reject, every interior partial accept, K = 1."""
    rng = np.random.default_rng(100 + K)
    V = 50
    g = rng.integers(0, V, size=K + 1)
    T = _rows_with_argmax(g, V, rng)
    for n in range(K + 1):                     # n accepted drafts
        x = g[:K].copy()
        if n < K:
            x[n] = (g[n] + 1 + rng.integers(0, V - 1)) % V
        r = orc.greedy(T[None], x[None].astype(np.int32), "f32")
        assert r.accept_len[0] == n
        assert list(r.tokens[0, :n]) == list(g[:n])
        assert r.tokens[0, n] == g[n]            # bonus = argmax of the first unmatched row
        assert (r.tokens[0, n + 1:] == -1).all()
        np.testing.assert_array_equal(r.behavior_logprob[0], 0.0)


def test_greedy_b8_construction(orc):
    ci = synth.greedy_chain_b8(V=4099)
    r = orc.greedy(ci.target, ci.tokens, "bf16")
    np.testing.assert_array_equal(r.accept_len, ci.expected_accept_len)
    np.testing.assert_array_equal(r.tokens[np.arange(ci.B), r.accept_len], ci.extra["expected_bonus"])


def test_greedy_out_of_range_draft(orc):
    rng = np.random.default_rng(3)
    T = _rows_with_argmax([1, 2, 3], 10, rng)[None]
    r = orc.greedy(T, np.array([[1, 99]], np.int32), "f32")
    assert r.accept_len[0] == 1 and r.status[0] == 1 and r.tokens[0, 1] == 2


# ---------------------------------------------------------------------------
# argmax ties and log-probs against library routines
# ---------------------------------------------------------------------------
def test_argmax_lowest_index_among_ties(orc):
    rng = np.random.default_rng(7)
    # bf16 values from a tiny set: ties at the max are the rule, not the exception
    vals = rng.integers(-4, 5, size=(64, 300)).astype(np.float32)
    h = synth.bf16_rne(vals)
    M, g, S = orc.row_stats(h, "bf16")
    np.testing.assert_array_equal(g, np.argmax(vals, axis=-1))
    np.testing.assert_array_equal(M, vals.max(-1))
    # bf16 3*N(0,1) rows at V = 128256: about 5% of rows tie at the max
    t = synth.bf16_rne(3.0 * np.random.default_rng(8).standard_normal((40, 128256), dtype=np.float32))
    M, g, S = orc.row_stats(t, "bf16")
    np.testing.assert_array_equal(g, np.argmax(synth.bf16_to_f32(t), axis=-1))


def test_logprobs_match_torch_log_softmax(orc):
    ci = synth.chain_inputs(6, 4, 3001, "bf16", seed=21, useed=22)
    T64 = synth.widen(ci.target, "bf16")
    ls = log_softmax64(T64)
    r = orc.greedy(ci.target, ci.tokens, "bf16")
    for b in range(ci.B):
        for i in range(r.accept_len[b] + 1):
            assert abs(r.target_logprob[b, i] - ls[b, i, r.tokens[b, i]]) < 1e-12
    re = orc.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16")
    for b in range(ci.B):
        for i in range(re.accept_len[b] + 1):
            assert abs(re.target_logprob[b, i] - ls[b, i, re.tokens[b, i]]) < 1e-12
    _, _, S = orc.row_stats(ci.target, "bf16")
    M = T64.max(-1)
    np.testing.assert_allclose(np.log(S) + M, torch.logsumexp(torch.from_numpy(T64), -1).numpy(),
                               rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# inverse CDF against numpy.searchsorted (relaxed special case: tau > 1, k = 0)
# ---------------------------------------------------------------------------
def test_relaxed_reject_all_is_inverse_cdf_of_p0(orc):
    ci = synth.chain_inputs(400, 3, 777, "f32", seed=31, useed=32, t_scale=2.0, with_draft=False)
    r = orc.relaxed(ci.target, ci.tokens, ci.uniforms, "f32", tau=2.0, top_k=0)
    assert (r.accept_len == 0).all()
    P = softmax64(synth.widen(ci.target, "f32")[:, 0, :])
    checked = 0
    for b in range(ci.B):
        c = np.cumsum(P[b])
        y = int(np.searchsorted(c, float(ci.uniforms[b, -1]) * c[-1], side="right"))
        if r.flag[b] == 0:
            continue
        assert r.tokens[b, 0] == y
        assert abs(r.behavior_logprob[b, 0] - math.log(P[b, y])) < 1e-12
        checked += 1
    assert checked >= 395


def test_relaxed_accept_all_samples_last_row(orc):
    ci = synth.chain_inputs(200, 4, 500, "f32", seed=33, useed=34, with_draft=False)
    r = orc.relaxed(ci.target, ci.tokens, ci.uniforms, "f32", tau=-1.0, top_k=0)
    assert (r.accept_len == 4).all()
    np.testing.assert_array_equal(r.tokens[:, :4], ci.tokens)
    np.testing.assert_array_equal(r.behavior_logprob[:, :4], 0.0)   # mu = 1 on accepted drafts
    P = softmax64(synth.widen(ci.target, "f32")[:, 4, :])
    for b in range(ci.B):
        c = np.cumsum(P[b])
        if r.flag[b] < 0:
            assert r.tokens[b, 4] == np.searchsorted(c, float(ci.uniforms[b, 4]) * c[-1], "right")


def test_relaxed_topk1_equals_greedy_on_tie_free_rows(orc):
    ci = synth.chain_inputs(100, 5, 1000, "f32", seed=35, useed=36, with_draft=False)
    T = synth.widen(ci.target, "f32")
    g = np.argmax(T, -1)
    rng = np.random.default_rng(37)
    x = g[:, :5].copy()
    flip = rng.random(x.shape) < 0.3
    x[flip] = (x[flip] + 1) % 1000
    x = x.astype(np.int32)
    rr = orc.relaxed(ci.target, x, ci.uniforms, "f32", tau=2.0, top_k=1)
    rg = orc.greedy(ci.target, x, "f32")
    np.testing.assert_array_equal(rr.accept_len, rg.accept_len)
    for b in range(ci.B):
        n = rr.accept_len[b]
        np.testing.assert_array_equal(rr.tokens[b, :n], rg.tokens[b, :n])


def test_relaxed_rank_threshold_against_numpy_count(orc):
    """c = #{t : l_t > l_x}; with tau > 1, accepted iff c < k (ties share a rank)."""
    rng = np.random.default_rng(38)
    V = 64
    for trial in range(50):
        row = rng.integers(-3, 4, size=V).astype(np.float32)   # many ties
        x = int(rng.integers(0, V))
        c = int((row > row[x]).sum())
        T = np.stack([row, row])[None]
        for k in (c, c + 1):
            r = orc.relaxed(T, np.array([[x]], np.int32), np.array([[0.5, 0.5]], np.float32),
                            "f32", tau=2.0, top_k=k)
            assert r.accept_len[0] == (1 if c < k else 0)


# ---------------------------------------------------------------------------
# brute force at V <= 8: the exact sampler's emitted-token law equals p
# ---------------------------------------------------------------------------
def _grid(M):
    return ((np.arange(M) + 0.5) / M).astype(np.float32)


@pytest.mark.parametrize("V,seed", [(2, 1), (4, 2), (6, 3), (8, 4)])
def test_exact_brute_force_first_token_law(orc, V, seed):
    """K = 1: enumerate x (weight q(x)) and a midpoint grid of (u0, u1).

    The law of the first emitted token must equal p_0 up to the grid's
    resolution, and the oracle's behaviour probability mu(t|x) must equal the
    grid frequency of t given x (spec-decode README, "Provably exact":
    the emitted distribution equals the target's; nanospec README: mu is the
    probability the sampler emitted the token).
    """
    rng = np.random.default_rng(seed)
    M = 256
    T = (rng.standard_normal((2, V)) * 1.5).astype(np.float32)
    Dq = (T[:1] + rng.standard_normal((1, V)) * 1.0).astype(np.float32)
    p = softmax64(T[0].astype(np.float64))
    q = softmax64(Dq[0].astype(np.float64))
    g = _grid(M)
    U0, U1 = np.meshgrid(g, g, indexing="ij")
    n = M * M
    law = np.zeros(V)
    for x in range(V):
        Tb = np.broadcast_to(T, (n, 2, V))
        Db = np.broadcast_to(Dq, (n, 1, V))
        xb = np.full((n, 1), x, np.int32)
        u = np.stack([U0.ravel(), U1.ravel()], axis=1)
        r = orc.exact(Tb, Db, xb, u, "f32", eps_sample=0.0, eps_accept=0.0)
        t0 = r.tokens[:, 0]
        freq = np.bincount(t0, minlength=V) / n
        law += q[x] * freq
        # mu(t|x) reported for each outcome == empirical frequency of t given x
        for t in np.unique(t0):
            mu = np.exp(r.behavior_logprob[t0 == t, 0])
            assert np.ptp(mu) < 1e-12
            assert abs(mu[0] - freq[t]) <= 2.5 * (V + 1) / M
    np.testing.assert_allclose(law, p, atol=2.5 * (V + 1) / M)


def test_exact_brute_force_second_position_law(orc):
    """K = 2 with x0 always accepted (p0(x0) >= q0(x0)): the conditional law of
    the second emitted token equals p_1 (every emitted token is a first token
    relative to its own prefix; spec-decode README, "Provably exact")."""
    rng = np.random.default_rng(9)
    V, M = 5, 256
    T = (rng.standard_normal((3, V)) * 1.5).astype(np.float32)
    Dq = (T[:2] + rng.standard_normal((2, V))).astype(np.float32)
    p0 = softmax64(T[0].astype(np.float64))
    q0 = softmax64(Dq[0].astype(np.float64))
    x0 = int(np.argmax(p0 / q0))
    assert p0[x0] >= q0[x0]
    p1 = softmax64(T[1].astype(np.float64))
    q1 = softmax64(Dq[1].astype(np.float64))
    g = _grid(M)
    U1, U2 = np.meshgrid(g, g, indexing="ij")
    n = M * M
    law = np.zeros(V)
    for x1 in range(V):
        u = np.stack([np.full(n, 0.5, np.float32), U1.ravel(), U2.ravel()], axis=1)
        xb = np.tile(np.array([[x0, x1]], np.int32), (n, 1))
        r = orc.exact(np.broadcast_to(T, (n, 3, V)), np.broadcast_to(Dq, (n, 2, V)), xb, u, "f32",
                      eps_sample=0.0, eps_accept=0.0)
        assert (r.accept_len >= 1).all()
        law += q1[x1] * np.bincount(r.tokens[:, 1], minlength=V) / n
    np.testing.assert_allclose(law, p1, atol=2.5 * (V + 1) / M)


def test_exact_mu_sums_to_one_and_marginalises_to_p(orc):
    """For each draft x: sum_t mu(t|x) = 1; and sum_x q(x) mu(t|x) = p(t), with
    mu read from the oracle's outputs at u values that land in each outcome."""
    rng = np.random.default_rng(12)
    V = 6
    T = (rng.standard_normal((2, V)) * 2).astype(np.float32)
    Dq = (T[:1] + rng.standard_normal((1, V)) * 0.8).astype(np.float32)
    p = softmax64(T[0].astype(np.float64))
    q = softmax64(Dq[0].astype(np.float64))
    M = 512
    g = _grid(M)
    marg = np.zeros(V)
    for x in range(V):
        u = np.stack([np.repeat(g, M), np.tile(g, M)], axis=1)
        n = u.shape[0]
        r = orc.exact(np.broadcast_to(T, (n, 2, V)), np.broadcast_to(Dq, (n, 1, V)),
                      np.full((n, 1), x, np.int32), u, "f32")
        mu = {}
        for t, lb in zip(r.tokens[:, 0], r.behavior_logprob[:, 0]):
            mu.setdefault(int(t), math.exp(lb))
        assert abs(sum(mu.values()) - 1.0) < 1e-12
        for t, m in mu.items():
            marg[t] += q[x] * m
    np.testing.assert_allclose(marg, p, atol=1e-12)


def test_exact_identical_draft_accepts_everything(orc):
    """q == p gives r == 1 for every draft, so u < 1 always accepts."""
    ci = synth.chain_inputs(50, 4, 300, "f32", seed=41, useed=42)
    r = orc.exact(ci.target, ci.target[:, :4, :], ci.tokens, ci.uniforms, "f32")
    assert (r.accept_len == 4).all()
    np.testing.assert_allclose(r.behavior_logprob[:, :4], 0.0, atol=1e-12)


def test_exact_tiny_acceptance_rate_matches_tv(orc):
    """Mean acceptance of test j equals 1 - TV(p_j, q_j) in expectation; checked
    on the tiny exact workload (1000 rounds) within a binomial 5-sigma band."""
    ci = synth.tiny_exact_v32()
    r = orc.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "f32")
    P = softmax64(synth.widen(ci.target, "f32")[:, 0, :])
    Q = softmax64(synth.widen(ci.draft, "f32")[:, 0, :])
    alpha = 1.0 - 0.5 * np.abs(P - Q).sum(-1)
    acc0 = (r.accept_len >= 1).astype(np.float64)
    sd = math.sqrt((alpha * (1 - alpha)).sum())
    assert abs(acc0.sum() - alpha.sum()) < 5 * sd


# ---------------------------------------------------------------------------
# tree: reductions and brute force
# ---------------------------------------------------------------------------
def test_tree_chain_equals_greedy(orc):
    ci = synth.chain_inputs(20, 6, 2000, "bf16", seed=51, useed=52, with_draft=False)
    g = np.argmax(synth.widen(ci.target, "bf16"), -1)
    rng = np.random.default_rng(53)
    x = g[:, :6].copy()
    x[rng.random(x.shape) < 0.25] = 7
    x = x.astype(np.int32)
    N = 7
    parents = np.tile(np.arange(-1, N - 1, dtype=np.int32), (ci.B, 1))
    node_tok = np.concatenate([np.zeros((ci.B, 1), np.int32), x], axis=1)
    rt = orc.tree(ci.target, node_tok, parents, "bf16")
    rg = orc.greedy(ci.target, x, "bf16")
    np.testing.assert_array_equal(rt.accept_len, rg.accept_len)
    for b in range(ci.B):
        n = rg.accept_len[b]
        np.testing.assert_array_equal(rt.tokens[b, : n + 1], rg.tokens[b, : n + 1])
        np.testing.assert_allclose(rt.target_logprob[b, : n + 1], rg.target_logprob[b, : n + 1],
                                   atol=1e-12)


def test_tree_star_accepts_at_most_one(orc):
    rng = np.random.default_rng(54)
    B, N, V = 30, 9, 40
    T = (rng.standard_normal((B, N, V)) * 3).astype(np.float32)
    g0 = np.argmax(T[:, 0, :], -1)
    parents = np.zeros((B, N), np.int32)
    parents[:, 0] = -1
    node_tok = rng.integers(0, V, size=(B, N)).astype(np.int32)
    node_tok[::2, 3] = g0[::2]
    r = orc.tree(T, node_tok, parents, "f32")
    assert (r.accept_len <= 1).all()
    assert (r.accept_len[::2] == 1).all()


def _brute_tree(Tw, node_tok, parents, nb):
    g = np.argmax(Tw, -1)
    best = (0, 0)   # (depth, -index)
    best_path = []
    for e in range(1, nb):
        path, v, ok = [], e, True
        while v != 0:
            p = parents[v]
            if node_tok[v] != g[p]:
                ok = False
                break
            path.append(v)
            v = p
        if ok and (len(path), -e) > best:
            best, best_path = (len(path), -e), path[::-1]
    end = best_path[-1] if best_path else 0
    return best_path, int(g[end])


def test_tree_brute_force_all_root_paths(orc):
    """Random trees with duplicate sibling tokens allowed; num_nodes < N on some
    requests.  The oracle's path equals the deepest all-matching root path
    found by enumerating every node (ties -> lowest end index)."""
    rng = np.random.default_rng(55)
    B, N, V = 60, 24, 6
    T = rng.integers(-2, 3, size=(B, N, V)).astype(np.float32)   # ties in rows
    parents = np.zeros((B, N), np.int32)
    parents[:, 0] = -1
    for i in range(1, N):
        parents[:, i] = rng.integers(0, i, size=B)
    node_tok = rng.integers(0, 2, size=(B, N)).astype(np.int32)
    g = np.argmax(T, -1)
    # bias tokens towards the parent argmax so that deep paths exist
    for b in range(B):
        for i in range(1, N):
            if rng.random() < 0.6:
                node_tok[b, i] = g[b, parents[b, i]]
    num_nodes = rng.integers(1, N + 1, size=B).astype(np.int32)
    r = orc.tree(T, node_tok, parents, "f32", num_nodes=num_nodes)
    for b in range(B):
        path, bonus = _brute_tree(T[b], node_tok[b], parents[b], int(num_nodes[b]))
        d = len(path)
        assert r.accept_len[b] == d
        assert list(r.path[b, :d]) == path
        assert list(r.tokens[b, :d]) == [int(node_tok[b, v]) for v in path]
        assert r.tokens[b, d] == bonus


def test_tree_b8_construction(orc):
    ti = synth.tree_inputs(B=4, V=3001, seed=4)
    r = orc.tree(ti.target, ti.node_tok, ti.parents, "bf16", num_nodes=ti.num_nodes)
    for b in range(ti.B):
        d = len(ti.expected_path[b])
        assert r.accept_len[b] == d
        assert list(r.path[b, :d]) == ti.expected_path[b]
        assert r.tokens[b, d] == ti.expected_bonus[b]


def test_tree_bad_parent_sets_status(orc):
    rng = np.random.default_rng(56)
    T = rng.standard_normal((1, 4, 10)).astype(np.float32)
    g = np.argmax(T[0], -1)
    parents = np.array([[-1, 0, 5, 1]], np.int32)          # node 2's parent is not < 2
    node_tok = np.array([[0, g[0], g[0], g[1]]], np.int32)
    r = orc.tree(T, node_tok, parents, "f32")
    assert r.status[0] == 1
    assert r.accept_len[0] == 2 and list(r.path[0, :2]) == [1, 3]


# ------------------------------------------------------------ draft sampler
# The proposal step before verification: one draw per draft row from
# q = softmax(row) (spec-decode README, "How it works"), by inverse CDF at a
# caller uniform.
def test_sampler_matches_searchsorted(orc):
    """A library routine on the fp64 softmax: searchsorted(cumsum(w), u*Z,
    'right') is the smallest t whose inclusive prefix exceeds u*Z."""
    rng = np.random.default_rng(71)
    for dtype, V in (("f32", 97), ("bf16", 3000), ("f32", 1)):
        x32 = (3.0 * rng.standard_normal((6, 4, V))).astype(np.float32)
        x = synth.bf16_rne(x32) if dtype == "bf16" else x32
        u = rng.random((6, 4), dtype=np.float32)
        r = orc.sample(x, u, dtype)
        xw = synth.widen(x, dtype)
        for idx in np.ndindex(6, 4):
            w = np.exp(xw[idx] - xw[idx].max())
            c = np.cumsum(w)
            want = min(int(np.searchsorted(c, float(u[idx]) * c[-1], side="right")), V - 1)
            if not r.flag[idx]:
                assert r.tokens[idx] == want, (dtype, idx)
        np.testing.assert_allclose(r.logq, log_softmax64(xw)[np.arange(6)[:, None], np.arange(4)[None, :],
                                                           r.tokens], rtol=0, atol=1e-12)


def test_sampler_law_on_a_grid(orc):
    """Brute force: over a midpoint grid of M uniforms the frequency of each
    token is its probability to within 1/M (each CDF boundary moves at most
    one grid point)."""
    rng = np.random.default_rng(72)
    M = 4000
    for V in (2, 5, 8):
        x = (2.0 * rng.standard_normal(V)).astype(np.float32)
        u = ((np.arange(M) + 0.5) / M).astype(np.float32)
        r = orc.sample(np.broadcast_to(x, (M, V)).copy(), u, "f32")
        freq = np.bincount(r.tokens, minlength=V) / M
        p = softmax64(x.astype(np.float64))
        assert np.abs(freq - p).max() <= 1.0 / M + 1e-12, (V, freq, p)


def test_sampler_special_cases(orc):
    """A row with one finite logit always yields that token (log q = 0); a row
    of equal logits yields floor(u*V) away from the multiples of 1/V."""
    V = 16
    x = np.full((5, V), -np.inf, np.float32)
    x[np.arange(5), [0, 3, 7, 12, 15]] = np.array([1.5, -2.0, 0.0, 40.0, -7.25], np.float32)
    u = np.array([0.0, 0.3, 0.5, 0.9, 0.999], np.float32)
    r = orc.sample(x, u, "f32")
    assert list(r.tokens) == [0, 3, 7, 12, 15]
    assert np.all(r.logq == 0.0)
    e = np.zeros((7, 10), np.float32)
    u = np.array([0.01, 0.17, 0.35, 0.52, 0.66, 0.81, 0.97], np.float32)
    r = orc.sample(e, u, "f32")
    assert list(r.tokens) == [int(math.floor(float(v) * 10)) for v in u]
    np.testing.assert_allclose(r.logq, -math.log(10.0), rtol=0, atol=1e-15)


# ---------------------------------------------------------------- power rule
# nanospec README, acceptance-rule paragraph: accept with probability
# min(1, p/rest)^alpha.  Reading: rest = q; after a rejection y ~ p_n.
def test_power_alpha_one_accepts_like_exact(orc):
    """alpha = 1 gives min(1, p/q): the exact rule's acceptance tests."""
    ci = synth.chain_inputs(64, 4, 300, "f32", seed=81, useed=82)
    pw = orc.power(ci.target, ci.draft, ci.tokens, ci.uniforms, "f32", 1.0)
    ex = orc.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "f32")
    assert (pw.accept_len == ex.accept_len).all()
    for b in range(64):
        n = int(pw.accept_len[b])
        assert (pw.tokens[b, :n] == ex.tokens[b, :n]).all()
        np.testing.assert_allclose(pw.behavior_logprob[b, :n], ex.behavior_logprob[b, :n], atol=1e-12)


def test_power_alpha_zero_accepts_everything(orc):
    """alpha = 0 makes every acceptance probability 1: all K drafts, then the
    bonus drawn from p_K as by the relaxed rule with tau <= 0."""
    ci = synth.chain_inputs(32, 3, 200, "f32", seed=83, useed=84)
    pw = orc.power(ci.target, ci.draft, ci.tokens, ci.uniforms, "f32", 0.0)
    rx = orc.relaxed(ci.target, ci.tokens, ci.uniforms, "f32", tau=-1.0, top_k=0)
    assert (pw.accept_len == 3).all()
    assert (pw.tokens == rx.tokens).all()
    np.testing.assert_allclose(pw.target_logprob, rx.target_logprob, atol=1e-12)
    assert (pw.behavior_logprob[:, :3] == 0).all()


@pytest.mark.parametrize("alpha", [0.5, 2.0])
def test_power_first_token_law_brute_force(orc, alpha):
    """K = 1, V = 5: enumerate the draft token x (weight q(x)) and a midpoint
    grid of (u_0, u_1).  The first emitted token's law is
    q(t) a(t) + p(t) (1 - sum_x q(x) a(x)), with a = min(1, p/q)^alpha, and the
    accept rate given x is a(x); both to within the grid's breakpoints."""
    rng = np.random.default_rng(85)
    V, M = 5, 160
    t_log = rng.standard_normal(V).astype(np.float32)
    d_log = (t_log + 0.8 * rng.standard_normal(V)).astype(np.float32)
    p = softmax64(t_log.astype(np.float64))
    q = softmax64(d_log.astype(np.float64))
    a = np.minimum(1.0, (p / q) ** alpha)
    g = (np.arange(M) + 0.5) / M
    u0, u1 = np.meshgrid(g, g, indexing="ij")
    U = np.stack([u0.ravel(), u1.ravel()], 1).astype(np.float32)
    B = U.shape[0]
    T = np.broadcast_to(t_log, (B, 2, V)).copy()
    D = np.broadcast_to(d_log, (B, 1, V)).copy()
    law = np.zeros(V)
    for x in range(V):
        r = orc.power(T, D, np.full((B, 1), x, np.int32), U, "f32", alpha)
        first = r.tokens[:, 0]
        law += q[x] * np.bincount(first, minlength=V) / B
        acc = (r.accept_len == 1).mean()
        assert abs(acc - a[x]) <= 1.0 / M + 1e-12, (x, acc, a[x])
        rej = r.accept_len == 0
        # after a rejection the token follows p
        np.testing.assert_allclose(np.bincount(first[rej], minlength=V) / B, (1 - acc) * p,
                                   atol=(V + 1) / M)
    want = q * a + p * (1.0 - np.sum(q * a))
    assert np.abs(law - want).max() <= (V + 1) / M, (law, want)
