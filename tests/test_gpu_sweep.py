"""A seeded sweep of shapes and value scales through every rule, against the
fp64 oracle.  Vocabulary sizes sit at and around the streaming tile (16 KiB:
8192 bf16 or 4096 fp32 tokens) and pass-2 chunk (4096 tokens) boundaries, or
are small and odd (the element path), or random; batch sizes, draft counts,
trees, logit scales (flat to peaked) and draft noise are drawn per case.
"""
import numpy as np
import pytest
import torch

import draft_verification_row_amd as sv
import oracle
import synth
from parity import LOGPROB_TOL, Tally, compare_chain, compare_tree, dev, dev_logits

pytestmark = pytest.mark.gpu

EDGE_V = [1, 2, 3, 8, 9, 255, 4095, 4096, 4097, 8191, 8192, 8193, 12287, 12289, 16384, 16385,
          24576, 32769]


def _chain_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        V = int(rng.choice(EDGE_V)) if rng.random() < 0.7 else int(rng.integers(10, 40000))
        out.append(dict(i=i, B=int(rng.integers(1, 9)), K=int(rng.integers(1, 11)), V=V,
                        dtype="bf16" if rng.random() < 0.7 else "f32",
                        scale=float(rng.choice([0.3, 3.0, 12.0])),
                        noise=float(rng.choice([0.1, 0.5, 2.0])),
                        tau=float(rng.choice([0.02, 0.1, 0.5])), top_k=int(rng.integers(0, 6)),
                        alpha=float(rng.choice([0.25, 0.5, 1.0, 3.0]))))
    return out


def _tree_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        depth, topk = int(rng.integers(1, 7)), int(rng.integers(1, 5))
        cand = topk + (depth - 1) * topk * topk
        V = int(rng.choice([64, 4095, 8193, 16385])) if rng.random() < 0.6 else int(rng.integers(64, 40000))
        out.append(dict(i=i, B=int(rng.integers(1, 7)), V=V, depth=depth, topk=topk,
                        keep=int(rng.integers(1, min(63, cand) + 1)),
                        dtype="bf16" if rng.random() < 0.7 else "f32",
                        scale=float(rng.choice([0.3, 3.0, 12.0])),
                        p_match=float(rng.choice([0.3, 0.7, 1.0]))))
    return out


CHAIN = _chain_cases(40, 4242)
TREE = _tree_cases(16, 4343)
# 2048-token sweep chunks (aligned bf16 rows): V at and around their
# boundaries, a multiple of 8 so the rows take the 16-byte path
CHAIN += [dict(i=100 + j, B=B, K=K, V=V, dtype="bf16", scale=sc, noise=nz, tau=0.1, top_k=3, alpha=0.5)
          for j, (B, K, V, sc, nz) in enumerate([(3, 4, 2040, 3.0, 0.5), (5, 2, 2048, 0.3, 2.0),
                                                 (4, 6, 2056, 12.0, 0.1), (2, 3, 6136, 3.0, 2.0),
                                                 (6, 5, 6144, 3.0, 0.5), (3, 8, 6152, 0.3, 0.5)])]


def _sync(r):
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("c", CHAIN, ids=lambda c: f"{c['i']}-B{c['B']}-K{c['K']}-V{c['V']}-{c['dtype']}")
def test_chain_rules_sweep(c):
    """Exact, greedy (with and without log-probs), relaxed and power on one
    batch, and the draft sampler on its draft rows."""
    print(f"sweep {c}", flush=True)
    B, K, V, dt = c["B"], c["K"], c["V"], c["dtype"]
    ci = synth.chain_inputs(B, K, V, dt, seed=5000 + c["i"], useed=6000 + c["i"],
                            t_scale=c["scale"], d_noise=c["noise"])
    T, D = dev_logits(ci.target, dt), dev_logits(ci.draft, dt)
    x, u = dev(ci.tokens), dev(ci.uniforms)
    what = f"case {c['i']}"
    t = Tally()
    t.add(compare_chain(_sync(sv.spec_verify_exact(T, D, x, u)),
                        oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, dt),
                        what=f"{what} exact"))
    og = oracle.greedy(ci.target, ci.tokens, dt)
    t.add(compare_chain(_sync(sv.spec_verify_greedy(T, x)), og, what=f"{what} greedy"))
    # without log-probs the bf16 stream reads 8 KiB tiles
    t.add(compare_chain(_sync(sv.spec_verify_greedy(T, x, logprobs=False)), og, logprobs=False,
                        what=f"{what} greedy no-logprob"))
    t.add(compare_chain(_sync(sv.spec_verify_relaxed(T, x, u, c["tau"], c["top_k"])),
                        oracle.relaxed(ci.target, ci.tokens, ci.uniforms, dt, c["tau"], c["top_k"]),
                        what=f"{what} relaxed"))
    t.add(compare_chain(_sync(sv.spec_verify_power(T, D, x, u, c["alpha"])),
                        oracle.power(ci.target, ci.draft, ci.tokens, ci.uniforms, dt, c["alpha"]),
                        what=f"{what} power"))
    assert t.flagged <= 2, f"{what}: {t.flagged} flagged near ties in {t.decisions} decisions"
    # the sampler on the draft rows
    us = np.random.default_rng(7000 + c["i"]).random((B, K), dtype=np.float32)
    o = oracle.sample(ci.draft, us, dt)
    r = _sync(sv.spec_sample_drafts(D, dev(us)))
    ok = o.flag == 0
    tok, lq = r.tokens.cpu().numpy(), r.logprob.cpu().numpy()
    assert (r.status.cpu().numpy() == 0).all(), what
    assert ((tok == o.tokens) | ~ok).all(), f"{what} sampler tokens"
    assert not ok.any() or np.abs(lq - o.logq)[ok].max() < LOGPROB_TOL, f"{what} sampler logq"
    assert o.flag.sum() <= 1, what


@pytest.mark.parametrize("c", TREE, ids=lambda c: f"{c['i']}-B{c['B']}-N{c['keep'] + 1}-V{c['V']}-{c['dtype']}")
def test_tree_sweep(c):
    print(f"tree sweep {c}", flush=True)
    ti = synth.tree_inputs(B=c["B"], V=c["V"], dtype=c["dtype"], seed=8000 + c["i"],
                           depth=c["depth"], topk=c["topk"], keep=c["keep"],
                           p_match=c["p_match"], t_scale=c["scale"])
    r = _sync(sv.spec_verify_tree(dev_logits(ti.target, ti.dtype), dev(ti.node_tok),
                                  dev(ti.parents), dev(ti.num_nodes)))
    o = oracle.tree(ti.target, ti.node_tok, ti.parents, ti.dtype, ti.num_nodes)
    compare_tree(r, o, what=f"tree case {c['i']}")
    for b in range(ti.B):  # and the construction's own path
        assert int(o.accept_len[b]) == len(ti.expected_path[b])
