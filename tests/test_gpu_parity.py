"""Parity of the HIP library (through the C ABI) with the fp64 oracle.

Every test here runs on an MI355X.  Inputs come from the seeded generators in
``synth``; expected values come only from ``oracle``.
"""
import numpy as np
import pytest
import torch

import draft_verification_row_amd as sv
import oracle
import synth
from parity import Tally, compare_chain, compare_tree, dev, dev_logits

pytestmark = pytest.mark.gpu


def _exact(ci, **kw):
    T = dev_logits(ci.target, ci.dtype)
    D = dev_logits(ci.draft, ci.dtype)
    r = sv.spec_verify_exact(T, D, dev(ci.tokens), dev(ci.uniforms), **kw)
    torch.cuda.synchronize()
    return r


def _greedy(ci, **kw):
    r = sv.spec_verify_greedy(dev_logits(ci.target, ci.dtype), dev(ci.tokens), **kw)
    torch.cuda.synchronize()
    return r


def _relaxed(ci, **kw):
    r = sv.spec_verify_relaxed(dev_logits(ci.target, ci.dtype), dev(ci.tokens), dev(ci.uniforms),
                               ci.tau, ci.top_k, **kw)
    torch.cuda.synchronize()
    return r


def _tree(ti, **kw):
    r = sv.spec_verify_tree(dev_logits(ti.target, ti.dtype), dev(ti.node_tok), dev(ti.parents),
                            dev(ti.num_nodes), **kw)
    torch.cuda.synchronize()
    return r


# ------------------------------------------------------------------ greedy
@pytest.mark.parametrize("rnd", range(6))
def test_greedy_b8_full_size(rnd):
    """B=8, K=5, V=128256 bf16; the accepted length equals the construction."""
    ci = synth.greedy_chain_b8(rnd=rnd)
    print(f"greedy B=8 round {rnd}", flush=True)
    o = oracle.greedy(ci.target, ci.tokens, "bf16")
    np.testing.assert_array_equal(o.accept_len, ci.expected_accept_len)
    compare_chain(_greedy(ci), o, what=f"greedy B=8 r{rnd}")
    r = _greedy(ci, logprobs=False)
    assert r.target_logprob is None
    compare_chain(r, o, logprobs=False, what=f"greedy B=8 r{rnd} no-logprob")


def test_greedy_b32_k5():
    ci = synth.exact_b32_k5()
    o = oracle.greedy(ci.target, ci.tokens, "bf16")
    compare_chain(_greedy(ci), o, what="greedy B=32")


@pytest.mark.parametrize("K", [1, 2, 5, 8, 63])
def test_greedy_scenarios(K):
    """all-correct + bonus, all-reject and every interior partial accept."""
    rng = np.random.default_rng(200 + K)
    V = 3001
    B = K + 1
    t = synth.bf16_rne(3.0 * rng.standard_normal((B, K + 1, V), dtype=np.float32))
    g = np.argmax(synth.bf16_to_f32(t), -1)
    x = g[:, :K].copy()
    for n in range(K):  # request n rejects at position n; request K accepts all
        x[n, n] = (g[n, n] + 1 + rng.integers(0, V - 1)) % V
        while synth.bf16_to_f32(t[n, n])[x[n, n]] == synth.bf16_to_f32(t[n, n]).max():
            x[n, n] = (x[n, n] + 1) % V
    ci = synth.ChainInputs("scen", "bf16", B, K, V, t, None, x.astype(np.int32),
                           np.zeros((B, K + 1), np.float32))
    o = oracle.greedy(ci.target, ci.tokens, "bf16")
    np.testing.assert_array_equal(o.accept_len, np.arange(K + 1))
    compare_chain(_greedy(ci), o, what=f"scenarios K={K}")


# ------------------------------------------------------------------- exact
def test_exact_tiny_v32_batched():
    """1000 rounds of B=1, K=4, V=32 fp32, run as one B=1000 call."""
    ci = synth.tiny_exact_v32()
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "f32")
    t = compare_chain(_exact(ci), o, what="tiny exact batched")
    assert t.within_budget(), t
    og = oracle.greedy(ci.target, ci.tokens, "f32")
    compare_chain(_greedy(ci), og, what="tiny greedy")


def test_exact_tiny_v32_single_requests():
    """The same 1000 rounds as individual B=1 calls."""
    ci = synth.tiny_exact_v32()
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "f32")
    tot = Tally()
    for r in range(1000):
        sub = synth.ChainInputs("tiny_exact_v32", "f32", 1, 4, 32, ci.target[r:r + 1], ci.draft[r:r + 1],
                                ci.tokens[r:r + 1], ci.uniforms[r:r + 1])
        osub = oracle.OracleResult(*(getattr(o, f)[r:r + 1] for f in
                                     ("tokens", "accept_len", "target_logprob",
                                      "behavior_logprob", "status", "flag", "decisions")))
        tot.add(compare_chain(_exact(sub), osub, what=f"tiny exact round {r}"))
    assert tot.within_budget(), tot


@pytest.mark.parametrize("rnd", range(4))
def test_exact_b32_full_size(rnd):
    """B=32, K=5, V=128256 bf16 -- the benchmarked configuration."""
    print(f"exact B=32 round {rnd}", flush=True)
    ci = synth.exact_b32_k5(rnd=rnd)
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16")
    t = compare_chain(_exact(ci), o, what=f"exact B=32 r{rnd}")
    assert t.within_budget(), t


def test_exact_b64_full_size():
    print("exact B=64 K=8", flush=True)
    ci = synth.large_b64_k8()
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16")
    t = compare_chain(_exact(ci), o, what="exact B=64")
    assert t.within_budget(), t


# ----------------------------------------------------------------- relaxed
def test_relaxed_b64_full_size():
    print("relaxed B=64 K=8", flush=True)
    ci = synth.large_b64_k8()
    o = oracle.relaxed(ci.target, ci.tokens, ci.uniforms, "bf16", ci.tau, ci.top_k)
    t = compare_chain(_relaxed(ci), o, what="relaxed B=64")
    assert t.within_budget(), t


@pytest.mark.parametrize("tau,k", [(2.0, 0), (-1.0, 0), (2.0, 1), (0.05, 2), (0.5, 10)])
def test_relaxed_special_cases(tau, k):
    ci = synth.chain_inputs(16, 6, 20000, "bf16", seed=61, useed=62, d_noise=0.3)
    ci.tau, ci.top_k = tau, k
    o = oracle.relaxed(ci.target, ci.tokens, ci.uniforms, "bf16", tau, k)
    compare_chain(_relaxed(ci), o, what=f"relaxed tau={tau} k={k}")


# -------------------------------------------------------------------- tree
@pytest.mark.parametrize("rnd", range(3))
def test_tree_b8_n61_full_size(rnd):
    print(f"tree B=8 N=61 round {rnd}", flush=True)
    ti = synth.tree_b8_n61(rnd=rnd)
    o = oracle.tree(ti.target, ti.node_tok, ti.parents, "bf16", num_nodes=ti.num_nodes)
    for b in range(ti.B):
        assert list(o.path[b, : o.accept_len[b]]) == ti.expected_path[b]
    compare_tree(_tree(ti), o, what=f"tree B=8 r{rnd}")
    r = _tree(ti, logprobs=False)
    compare_tree(r, o, logprobs=False, what=f"tree B=8 r{rnd} no-logprob")


def test_tree_chain_equals_greedy_on_gpu():
    ci = synth.chain_inputs(8, 7, 5003, "bf16", seed=71, useed=72, with_draft=False)
    g = np.argmax(synth.bf16_to_f32(ci.target), -1)
    x = g[:, :7].copy()
    x[np.random.default_rng(73).random(x.shape) < 0.3] = 11
    ci.tokens = x.astype(np.int32)
    N = 8
    ti = synth.TreeInputs("chain", "bf16", 8, N, 5003, ci.target,
                          np.concatenate([np.zeros((8, 1), np.int32), ci.tokens], 1),
                          np.tile(np.arange(-1, N - 1, dtype=np.int32), (8, 1)),
                          np.full(8, N, np.int32))
    rt = _tree(ti)
    rg = _greedy(ci)
    ln = rg.accept_len.cpu().numpy()
    np.testing.assert_array_equal(rt.accept_len.cpu().numpy(), ln)
    tt, gt = rt.tokens.cpu().numpy(), rg.tokens.cpu().numpy()
    for b in range(8):
        np.testing.assert_array_equal(tt[b, : ln[b] + 1], gt[b, : ln[b] + 1])


@pytest.mark.parametrize("shape", ["chain64", "broom", "random", "bushy_ties"])
def test_tree_deep_and_irregular_shapes(shape):
    """Trees up to the 64-node limit: a full chain (depth 63), a long handle
    with a fan of leaves, random parents, and many equal-depth leaves (ties go
    to the lowest node index).  Tokens match the parent's argmax 90% of the
    time, so accepted paths run deep."""
    print(f"tree shape {shape}", flush=True)
    B, N, V = 6, 64, 3001
    rng = np.random.default_rng({"chain64": 81, "broom": 82, "random": 83, "bushy_ties": 84}[shape])
    par = np.full((B, N), -1, np.int32)
    for i in range(1, N):
        if shape == "chain64":
            par[:, i] = i - 1
        elif shape == "broom":
            par[:, i] = i - 1 if i < 40 else 39
        elif shape == "random":
            par[:, i] = rng.integers(max(0, i - 4), i, size=B)
        else:
            par[:, i] = (i - 1) // 3
    target = synth.bf16_rne(3.0 * rng.standard_normal((B, N, V), dtype=np.float32))
    g = np.argmax(synth.bf16_to_f32(target), -1)
    tok = np.zeros((B, N), np.int32)
    for b in range(B):
        for i in range(1, N):
            p = par[b, i]
            tok[b, i] = g[b, p] if rng.random() < 0.9 else (g[b, p] + 1 + rng.integers(V - 1)) % V
    nn = np.full(B, N, np.int32)
    nn[-1] = 37
    ti = synth.TreeInputs(shape, "bf16", B, N, V, target, tok, par, nn)
    o = oracle.tree(ti.target, ti.node_tok, ti.parents, "bf16", num_nodes=ti.num_nodes)
    if shape == "chain64":
        assert o.accept_len.max() >= 5
    compare_tree(_tree(ti), o, what=f"tree {shape}")


def test_tree_partial_node_counts_and_bad_parents():
    ti = synth.tree_inputs(B=6, V=3001, seed=75)
    ti.num_nodes = np.array([61, 1, 2, 30, 60, 17], np.int32)
    ti.parents = ti.parents.copy()
    ti.parents[3, 5] = 40     # not < 5: malformed
    ti.node_tok = ti.node_tok.copy()
    ti.node_tok[4, 7] = 10 ** 6  # out of vocabulary: malformed
    o = oracle.tree(ti.target, ti.node_tok, ti.parents, "bf16", num_nodes=ti.num_nodes)
    assert o.status[3] == 1 and o.status[4] == 1
    compare_tree(_tree(ti), o, what="tree edge")


# ------------------------------------------------------------- edge cases
@pytest.mark.parametrize("B,K,V,dtype", [
    (3, 1, 1, "bf16"), (3, 2, 2, "f32"), (5, 3, 7, "bf16"), (4, 4, 1000, "f32"),
    (2, 5, 8191, "bf16"), (2, 5, 8193, "bf16"), (3, 3, 16385, "f32"), (2, 63, 300, "bf16"),
    (40, 2, 2051, "bf16"), (1, 5, 128257, "bf16"),
])
def test_exact_greedy_relaxed_ragged_shapes(B, K, V, dtype):
    """Sizes spanning several chunks with a ragged tail, odd V (element path),
    V = 1, and the largest K."""
    print(f"ragged B={B} K={K} V={V} {dtype}", flush=True)
    ci = synth.chain_inputs(B, K, V, dtype, seed=1000 + V, useed=2000 + K)
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, dtype)
    compare_chain(_exact(ci), o, what=f"exact {B},{K},{V}")
    og = oracle.greedy(ci.target, ci.tokens, dtype)
    compare_chain(_greedy(ci), og, what=f"greedy {B},{K},{V}")
    orl = oracle.relaxed(ci.target, ci.tokens, ci.uniforms, dtype, 0.1, 4)
    ci.tau, ci.top_k = 0.1, 4
    compare_chain(_relaxed(ci), orl, what=f"relaxed {B},{K},{V}")


@pytest.mark.parametrize("B,K,V", [(32, 3, 131072), (33, 3, 131072), (32, 2, 129025), (33, 2, 129025)])
def test_sweep_chunking_boundary(B, K, V):
    """The exact, power and relaxed launches sum the terminal rows in 2048-token
    sweep chunks while B * ceil(V / 2048) <= 2048 (the chip's resident
    workgroups beside the streamers) and in 4096-token chunks above: B = 32
    and 33 sit on either side of it, and V = 129025 leaves a one-token last
    chunk."""
    print(f"sweep boundary B={B} K={K} V={V}", flush=True)
    ci = synth.chain_inputs(B, K, V, "bf16", seed=3100 + B, useed=3200 + V % 97)
    compare_chain(_exact(ci), oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16"),
                  what=f"exact {B},{K},{V}")
    T, D = dev_logits(ci.target, "bf16"), dev_logits(ci.draft, "bf16")
    r = sv.spec_verify_power(T, D, dev(ci.tokens), dev(ci.uniforms), 0.5)
    torch.cuda.synchronize()
    compare_chain(r, oracle.power(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16", 0.5),
                  what=f"power {B},{K},{V}")
    ci.tau, ci.top_k = 0.1, 4
    compare_chain(_relaxed(ci), oracle.relaxed(ci.target, ci.tokens, ci.uniforms, "bf16", 0.1, 4),
                  what=f"relaxed {B},{K},{V}")


def test_misaligned_rows_take_element_path():
    """A view starting one element into an allocation is not 16-byte aligned."""
    ci = synth.chain_inputs(3, 4, 4096, "bf16", seed=81, useed=82)
    big = np.zeros(ci.target.size + 1, np.uint16)
    big[1:] = ci.target.ravel()
    T = dev_logits(big, "bf16")[1:].view(ci.target.shape)
    bigd = np.zeros(ci.draft.size + 1, np.uint16)
    bigd[1:] = ci.draft.ravel()
    D = dev_logits(bigd, "bf16")[1:].view(ci.draft.shape)
    assert T.data_ptr() % 16 != 0
    r = sv.spec_verify_exact(T, D, dev(ci.tokens), dev(ci.uniforms))
    torch.cuda.synchronize()
    compare_chain(r, oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16"),
                  what="misaligned")
    og = oracle.greedy(ci.target, ci.tokens, "bf16")
    for lp in (True, False):  # 16 KiB and 8 KiB tiles
        g = sv.spec_verify_greedy(T, dev(ci.tokens), logprobs=lp)
        torch.cuda.synchronize()
        compare_chain(g, og, logprobs=lp, what=f"misaligned greedy logprobs={lp}")
    # the relaxed rule reads each drafted token's logit as the 4-byte word that
    # holds it; here rows start 2 bytes past a word boundary
    rr = sv.spec_verify_relaxed(T, dev(ci.tokens), dev(ci.uniforms), 0.05, 3)
    torch.cuda.synchronize()
    compare_chain(rr, oracle.relaxed(ci.target, ci.tokens, ci.uniforms, "bf16", 0.05, 3),
                  what="misaligned relaxed")


def test_out_of_range_draft_tokens_set_status():
    ci = synth.chain_inputs(6, 4, 5000, "bf16", seed=83, useed=84)
    ci.tokens = ci.tokens.copy()
    ci.tokens[0, 0] = -1
    ci.tokens[1, 2] = 5000
    ci.tokens[2, 3] = 2 ** 30
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16")
    r = _exact(ci)
    compare_chain(r, o, what="oor exact")
    assert r.status.cpu().numpy()[0] == 1
    og = oracle.greedy(ci.target, ci.tokens, "bf16")
    compare_chain(_greedy(ci), og, what="oor greedy")


def test_masked_vocabulary_minus_inf():
    """-inf logits have probability zero and are never emitted."""
    ci = synth.chain_inputs(8, 3, 4000, "f32", seed=85, useed=86)
    t = ci.target.copy()
    d = ci.draft.copy()
    t[:, :, 1000:2000] = -np.inf
    d[:, :, 1500:2500] = -np.inf
    ci.target, ci.draft = t, d
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "f32")
    r = _exact(ci)
    compare_chain(r, o, what="masked")
    toks = r.tokens.cpu().numpy()
    assert not ((toks >= 1000) & (toks < 2000)).any()


def test_bitwise_determinism():
    ci = synth.chain_inputs(16, 5, 50000, "bf16", seed=87, useed=88)
    a = _exact(ci)
    b = _exact(ci)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_workspace_reuse_across_shapes():
    """One zero-filled workspace serves calls of several rules and shapes in
    turn, and every call leaves it zero-filled again (the single-launch rules
    read zero as "not yet published")."""
    nb = sv.spec_verify_workspace_bytes(64, 17, 151936)
    ws = torch.zeros(nb, dtype=torch.uint8, device="cuda")
    for (B, K, V) in [(4, 3, 5000), (32, 5, 20000), (2, 8, 3000), (32, 5, 20000)]:
        ci = synth.chain_inputs(B, K, V, "bf16", seed=B * 7 + K, useed=V)
        T, D = dev_logits(ci.target, "bf16"), dev_logits(ci.draft, "bf16")
        r = sv.spec_verify_exact(T, D, dev(ci.tokens), dev(ci.uniforms), workspace=ws)
        g = sv.spec_verify_greedy(T, dev(ci.tokens), workspace=ws)
        torch.cuda.synchronize()
        compare_chain(r, oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16"),
                      what=f"reuse exact {B},{K},{V}")
        compare_chain(g, oracle.greedy(ci.target, ci.tokens, "bf16"), what=f"reuse greedy {B}")
        assert int(ws.count_nonzero()) == 0, f"workspace left dirty after B={B} K={K} V={V}"
    # the tree rule's single launch on the same workspace, partial node counts
    ti = synth.tree_inputs(B=6, V=3001, seed=76)
    ti.num_nodes = np.array([61, 1, 2, 30, 60, 17], np.int32)
    for logprobs in (False, True):
        r = sv.spec_verify_tree(dev_logits(ti.target, "bf16"), dev(ti.node_tok), dev(ti.parents),
                                dev(ti.num_nodes), logprobs=logprobs, workspace=ws)
        torch.cuda.synchronize()
        compare_tree(r, oracle.tree(ti.target, ti.node_tok, ti.parents, "bf16", num_nodes=ti.num_nodes),
                     logprobs=logprobs, what=f"reuse tree logprobs={logprobs}")
        assert int(ws.count_nonzero()) == 0, f"workspace left dirty after the tree (logprobs={logprobs})"


# --------------------------------------------------------- statistical pin
def test_first_token_histogram_matches_target():
    """Fixed logits at V=32 and many uniforms: the law of the first emitted
    token equals p_0 (spec-decode README, "Provably exact": empirical output
    frequencies match target-only sampling).  This pins the GPU path without
    the oracle."""
    rng = np.random.default_rng(91)
    V, K, n = 32, 2, 400000
    t = (2.0 * rng.standard_normal((K + 1, V))).astype(np.float32)
    d = (t[:K] + 0.7 * rng.standard_normal((K, V))).astype(np.float32)
    q0 = np.exp(d[0].astype(np.float64) - d[0].max()); q0 /= q0.sum()
    p0 = np.exp(t[0].astype(np.float64) - t[0].max()); p0 /= p0.sum()
    x = np.stack([rng.choice(V, size=n, p=q0)] +
                 [rng.integers(0, V, size=n) for _ in range(K - 1)], 1).astype(np.int32)
    u = rng.random((n, K + 1), dtype=np.float32)
    m = 50000  # requests per call (the library takes at most 65536)
    T = torch.from_numpy(np.broadcast_to(t, (m, K + 1, V)).copy()).cuda()
    D = torch.from_numpy(np.broadcast_to(d, (m, K, V)).copy()).cuda()
    obs = np.zeros(V, np.int64)
    for s in range(0, n, m):
        r = sv.spec_verify_exact(T, D, dev(x[s:s + m]), dev(u[s:s + m]))
        torch.cuda.synchronize()
        obs += np.bincount(r.tokens[:, 0].cpu().numpy(), minlength=V)
    exp = p0 * n
    chi2 = ((obs - exp) ** 2 / exp).sum()
    # chi-square with 31 degrees of freedom: P(chi2 > 70) < 1e-4
    assert chi2 < 70, chi2


def test_read_ceiling_kernel_runs_on_odd_sizes():
    """The benchmarking read kernel reads any multiple of 16 bytes and writes
    one word per 16 KiB; its ragged last tile stays inside the buffer."""
    import ctypes
    lib = sv.load_library()
    for nbytes in (16, 16384, 16400, 3 * 16384 + 48):
        buf = torch.full((nbytes,), 7, dtype=torch.uint8, device="cuda")
        words = lib.spec_read_ceiling_out_words(nbytes)
        assert words == (nbytes + 16383) // 16384
        out = torch.full((words + 1,), -1, dtype=torch.int32, device="cuda")
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert lib.spec_read_ceiling(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                     ctypes.c_void_p(out.data_ptr()), st) == 0
        torch.cuda.synchronize()
        assert int(out[words]) == -1  # nothing written past the last word


def test_graph_capture_replays_match_eager():
    """Calls captured in a HIP graph (every rule and the draft sampler): every
    replay equals the eager result bit for bit, with other eager calls
    (reusing the same workspace) between the replays."""
    ci = synth.chain_inputs(16, 5, 50000, "bf16", seed=111, useed=112)
    T, D = dev_logits(ci.target, "bf16"), dev_logits(ci.draft, "bf16")
    x, u = dev(ci.tokens), dev(ci.uniforms)
    B, K, V = ci.B, ci.K, ci.V
    ws = torch.zeros(sv.spec_verify_workspace_bytes(B, 2 * K + 1, V), dtype=torch.uint8,
                     device="cuda")
    ws_s = torch.zeros(sv.spec_sample_workspace_bytes(B * K, V), dtype=torch.uint8, device="cuda")
    ud = u[:, :K].contiguous()
    ti = synth.tree_inputs(B=4, V=50000, seed=115)
    Tt, tok_t, par_t, nn_t = dev_logits(ti.target, "bf16"), dev(ti.node_tok), dev(ti.parents), dev(ti.num_nodes)
    ws_t = torch.zeros(sv.spec_verify_workspace_bytes(ti.B, ti.N, ti.V), dtype=torch.uint8, device="cuda")

    def calls():
        return (sv.spec_verify_exact(T, D, x, u, workspace=ws),
                sv.spec_verify_greedy(T, x, workspace=ws),
                sv.spec_verify_greedy(T, x, logprobs=False, workspace=ws),  # 8 KiB tiles
                sv.spec_verify_relaxed(T, x, u, 0.1, 4, workspace=ws),
                sv.spec_verify_power(T, D, x, u, 0.5, workspace=ws),
                sv.spec_verify_tree(Tt, tok_t, par_t, nn_t, workspace=ws_t),
                sv.spec_sample_drafts(D, ud, workspace=ws_s))

    eager = [[t.clone() for t in r if t is not None] for r in calls()]
    torch.cuda.synchronize()
    other = synth.chain_inputs(16, 5, 50000, "bf16", seed=113, useed=114)
    T2, x2 = dev_logits(other.target, "bf16"), dev(other.tokens)
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        captured = calls()
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for r_eager, r_cap in zip(eager, captured):
            for a, b in zip(r_eager, [t for t in r_cap if t is not None]):
                assert torch.equal(a, b), f"replay {rep}"
        sv.spec_verify_greedy(T2, x2, workspace=ws)  # eager work on the same workspace
        sv.spec_verify_exact(T2, dev_logits(other.draft, "bf16"), x2, dev(other.uniforms),
                             workspace=ws)
        torch.cuda.synchronize()


def test_concurrent_calls_on_two_streams():
    """Calls on two streams (default priority) with their own workspaces run
    concurrently: an exact call on one, an exact and a greedy call on the
    other, five rounds without a synchronization between the streams; every
    result equals the oracle's."""
    a = synth.chain_inputs(32, 5, 128256, "bf16", seed=131, useed=132)
    b = synth.chain_inputs(24, 4, 100003, "bf16", seed=133, useed=134)
    Ta, Da, xa, ua = dev_logits(a.target, "bf16"), dev_logits(a.draft, "bf16"), dev(a.tokens), dev(a.uniforms)
    Tb, Db, xb, ub = dev_logits(b.target, "bf16"), dev_logits(b.draft, "bf16"), dev(b.tokens), dev(b.uniforms)
    ws_a = torch.zeros(sv.spec_verify_workspace_bytes(32, 11, 128256), dtype=torch.uint8, device="cuda")
    ws_b = torch.zeros(sv.spec_verify_workspace_bytes(24, 9, 100003), dtype=torch.uint8, device="cuda")
    ws_g = torch.zeros(sv.spec_verify_workspace_bytes(24, 5, 100003), dtype=torch.uint8, device="cuda")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    res = []
    for rnd in range(5):
        print(f"concurrent round {rnd}", flush=True)
        with torch.cuda.stream(sa):
            ra = sv.spec_verify_exact(Ta, Da, xa, ua, workspace=ws_a)
        with torch.cuda.stream(sb):
            rb = sv.spec_verify_exact(Tb, Db, xb, ub, workspace=ws_b)
            rg = sv.spec_verify_greedy(Tb, xb, workspace=ws_g)
        res.append((ra, rb, rg))
    torch.cuda.synchronize()
    oa = oracle.exact(a.target, a.draft, a.tokens, a.uniforms, "bf16")
    ob = oracle.exact(b.target, b.draft, b.tokens, b.uniforms, "bf16")
    og = oracle.greedy(b.target, b.tokens, "bf16")
    for rnd, (ra, rb, rg) in enumerate(res):
        compare_chain(ra, oa, what=f"stream a, round {rnd}")
        compare_chain(rb, ob, what=f"stream b exact, round {rnd}")
        compare_chain(rg, og, what=f"stream b greedy, round {rnd}")
    for ws in (ws_a, ws_b, ws_g):
        assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_largest_vocabulary(dtype):
    """V = 262144: in fp32 a row has 64 tile records and 64 pass-2 chunks, so
    the fold and the chunk scan use every lane of a wave."""
    print(f"largest vocabulary {dtype}", flush=True)
    ci = synth.chain_inputs(2, 3, 262144, dtype, seed=121, useed=122)
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, dtype)
    compare_chain(_exact(ci), o, what=f"exact V max {dtype}")
    og = oracle.greedy(ci.target, ci.tokens, dtype)
    compare_chain(_greedy(ci), og, what=f"greedy V max {dtype}")
    # bf16 without log-probs: 8 KiB tiles, 64 tile records a row (one per lane)
    compare_chain(_greedy(ci, logprobs=False), og, logprobs=False, what=f"greedy V max {dtype} no-logprob")
    ci.tau, ci.top_k = 0.1, 4
    compare_chain(_relaxed(ci), oracle.relaxed(ci.target, ci.tokens, ci.uniforms, dtype, 0.1, 4),
                  what=f"relaxed V max {dtype}")
    po = oracle.power(ci.target, ci.draft, ci.tokens, ci.uniforms, dtype, 0.5)
    pr = sv.spec_verify_power(dev_logits(ci.target, dtype), dev_logits(ci.draft, dtype),
                              dev(ci.tokens), dev(ci.uniforms), 0.5)
    torch.cuda.synchronize()
    compare_chain(pr, po, what=f"power V max {dtype}")
    s = sv.spec_sample_drafts(dev_logits(ci.draft, dtype), dev(ci.uniforms[:, :3].copy()))
    os_ = oracle.sample(ci.draft, ci.uniforms[:, :3].copy(), dtype)
    ok = os_.flag == 0
    np.testing.assert_array_equal(s.tokens.cpu().numpy()[ok], os_.tokens[ok])


def test_largest_batch():
    """B = 65536 requests (the library's limit), K = 1, V = 40."""
    print("largest batch", flush=True)
    ci = synth.chain_inputs(65536, 1, 40, "bf16", seed=123, useed=124)
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16")
    t = compare_chain(_exact(ci), o, what="exact B max")
    assert t.within_budget(), t
    compare_chain(_greedy(ci), oracle.greedy(ci.target, ci.tokens, "bf16"), what="greedy B max")
    rows = ci.draft.reshape(65536, 40)
    u = ci.uniforms[:, 0].copy()
    s = sv.spec_sample_drafts(dev_logits(rows, "bf16"), dev(u))
    os_ = oracle.sample(rows, u, "bf16")
    ok = os_.flag == 0
    np.testing.assert_array_equal(s.tokens.cpu().numpy()[ok], os_.tokens[ok])
