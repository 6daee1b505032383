"""The timeout path of the single-launch calls, forced from the host.

With the bound of the kernels' waits set to 0 (spec_set_spin_limit), a wait
that does not find its data on the first poll gives up at once and its
request reports status 2; every kernel still ends (the bound only shortens
the kernels' own bounded waits: nothing faults, traps or hangs).  A request
that reports 0 or 1 has completed every step, so it must equal the oracle's.
With the default bound restored and a fresh zero-filled workspace, every
request must equal the oracle's again: a timed-out call leaves its own
workspace possibly dirty, and nothing else.
"""
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import draft_verification_row_amd as sv
import oracle
import synth
from parity import compare_chain, compare_tree, dev, dev_logits

pytestmark = pytest.mark.gpu

ALPHA = 0.5
TAU, TOP_K = 0.1, 4


@pytest.fixture
def zero_spin_limit():
    sv.spec_set_spin_limit(0)
    try:
        yield
    finally:
        sv.spec_set_spin_limit(-1)


@pytest.fixture(params=[0, 4])
def small_spin_limit(request):
    """0: every wait that is not already satisfied gives up; 4: a few polling
    rounds, so that some requests complete and some do not."""
    sv.spec_set_spin_limit(request.param)
    try:
        yield request.param
    finally:
        sv.spec_set_spin_limit(-1)


def _keep(res, keep):
    k = torch.from_numpy(keep).to(res.tokens.device)
    return SimpleNamespace(tokens=res.tokens[k], accept_len=res.accept_len[k], status=res.status[k],
                           target_logprob=None if res.target_logprob is None else res.target_logprob[k],
                           behavior_logprob=None if res.behavior_logprob is None else res.behavior_logprob[k])


def _keep_oracle(o, keep):
    return SimpleNamespace(tokens=o.tokens[keep], accept_len=o.accept_len[keep], status=o.status[keep],
                           target_logprob=o.target_logprob[keep], behavior_logprob=o.behavior_logprob[keep],
                           decisions=o.decisions[keep], flag=o.flag[keep])


def _chain_cases(ci):
    T, D = dev_logits(ci.target, "bf16"), dev_logits(ci.draft, "bf16")
    x, u = dev(ci.tokens), dev(ci.uniforms)
    B, K, V = ci.B, ci.K, ci.V
    return [
        ("exact", 2 * K + 1, lambda ws: sv.spec_verify_exact(T, D, x, u, workspace=ws),
         lambda: oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16"), True),
        ("power", 2 * K + 1, lambda ws: sv.spec_verify_power(T, D, x, u, ALPHA, workspace=ws),
         lambda: oracle.power(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16", ALPHA), True),
        ("relaxed", K + 1, lambda ws: sv.spec_verify_relaxed(T, x, u, TAU, TOP_K, workspace=ws),
         lambda: oracle.relaxed(ci.target, ci.tokens, ci.uniforms, "bf16", TAU, TOP_K), True),
        ("greedy", K + 1, lambda ws: sv.spec_verify_greedy(T, x, logprobs=False, workspace=ws),
         lambda: oracle.greedy(ci.target, ci.tokens, "bf16"), False),
    ]


def test_chain_rules_time_out_cleanly(small_spin_limit):
    """B=32, K=5, V=128256 bf16 at a small bound: every status in {0, 1, 2};
    the requests that did not time out equal the oracle's."""
    ci = synth.exact_b32_k5()
    B, V = ci.B, ci.V
    timed_out = {}
    for name, rows, call, orc, lp in _chain_cases(ci):
        ws = torch.zeros(sv.spec_verify_workspace_bytes(B, rows, V), dtype=torch.uint8, device="cuda")
        r = call(ws)
        torch.cuda.synchronize()
        st = r.status.cpu().numpy()
        assert set(np.unique(st).tolist()) <= {0, 1, 2}, (name, st)
        keep = st != 2
        timed_out[name] = int((~keep).sum())
        if keep.any():
            compare_chain(_keep(r, keep), _keep_oracle(orc(), keep), logprobs=lp,
                          what=f"{name}, zero spin limit")
        del ws
    print(f"spin limit {small_spin_limit}: requests timed out per rule:", timed_out, flush=True)


def test_sampler_times_out_cleanly(zero_spin_limit):
    """The draft sampler on the 160 draft rows of the same batch: status 0 or
    2 per row; rows that did not time out equal the oracle's draws."""
    ci = synth.exact_b32_k5()
    rows = ci.draft.reshape(-1, ci.V)
    u = np.random.default_rng(17).random(rows.shape[0], dtype=np.float32)
    ws = torch.zeros(sv.spec_sample_workspace_bytes(rows.shape[0], ci.V), dtype=torch.uint8, device="cuda")
    r = sv.spec_sample_drafts(dev_logits(rows, "bf16"), dev(u), workspace=ws)
    torch.cuda.synchronize()
    st = r.status.cpu().numpy()
    assert set(np.unique(st).tolist()) <= {0, 2}, st
    o = oracle.sample(rows, u, "bf16")
    keep = (st == 0) & (o.flag < 0)
    assert (r.tokens.cpu().numpy()[keep] == o.tokens[keep]).all()


def test_tree_times_out_cleanly(zero_spin_limit):
    """The tree rule (B=8, 61 nodes, V=128256): status in {0, 1, 2}; requests
    that did not time out equal the oracle's."""
    ti = synth.tree_b8_n61()
    ws = torch.zeros(sv.spec_verify_workspace_bytes(ti.B, ti.N, ti.V), dtype=torch.uint8, device="cuda")
    r = sv.spec_verify_tree(dev_logits(ti.target, "bf16"), dev(ti.node_tok), dev(ti.parents),
                            dev(ti.num_nodes), workspace=ws)
    torch.cuda.synchronize()
    st = r.status.cpu().numpy()
    assert set(np.unique(st).tolist()) <= {0, 1, 2}, st
    keep = st != 2
    o = oracle.tree(ti.target, ti.node_tok, ti.parents, "bf16", num_nodes=ti.num_nodes)
    k = torch.from_numpy(keep).cuda()
    sub = SimpleNamespace(path_nodes=r.path_nodes[k], tokens=r.tokens[k], accept_len=r.accept_len[k],
                          status=r.status[k], target_logprob=r.target_logprob[k],
                          behavior_logprob=r.behavior_logprob[k])
    osub = SimpleNamespace(path=o.path[keep], tokens=o.tokens[keep], accept_len=o.accept_len[keep],
                           status=o.status[keep], target_logprob=o.target_logprob[keep])
    compare_tree(sub, osub, what="tree, zero spin limit")
    print("tree requests timed out:", int((~keep).sum()), flush=True)


def test_default_limit_restored_after_timeouts():
    """After calls at a zero bound, the default bound and a fresh workspace
    give results equal to the oracle's for every request and row."""
    ci = synth.exact_b32_k5()
    sv.spec_set_spin_limit(0)
    try:
        for name, rows, call, _, _ in _chain_cases(ci):
            ws = torch.zeros(sv.spec_verify_workspace_bytes(ci.B, rows, ci.V), dtype=torch.uint8, device="cuda")
            call(ws)
        torch.cuda.synchronize()
    finally:
        sv.spec_set_spin_limit(-1)
    for name, rows, call, orc, lp in _chain_cases(ci):
        ws = torch.zeros(sv.spec_verify_workspace_bytes(ci.B, rows, ci.V), dtype=torch.uint8, device="cuda")
        r = call(ws)
        torch.cuda.synchronize()
        assert (r.status.cpu().numpy() != 2).all(), name
        compare_chain(r, orc(), logprobs=lp, what=f"{name}, default spin limit")
        assert int(ws.count_nonzero()) == 0, f"{name} left its workspace dirty"
