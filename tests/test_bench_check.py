"""The benchmark's check of its timed outputs against the oracle (host logic,
no GPU): outputs equal to the oracle's count no mismatch, and each kind of
planted difference (a token, an accepted count, a log-prob beyond 1e-4, a
sampled token) counts exactly one."""
import os
import sys

import numpy as np
import torch

import oracle
import synth

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _chain_outputs(o, with_lp=True):
    d = {"tok": torch.from_numpy(o.tokens.copy()), "ln": torch.from_numpy(o.accept_len.copy()),
         "st": torch.from_numpy(o.status.copy())}
    if with_lp:
        d["tlp"] = torch.from_numpy(o.target_logprob.astype(np.float32))
        d["blp"] = torch.from_numpy(o.behavior_logprob.astype(np.float32))
    return d


def _first_unflagged(o):
    return int(np.flatnonzero(o.flag < 0)[0])


def test_exact_outputs_equal_to_the_oracle_have_no_mismatch():
    ci = synth.tiny_exact_v32()
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, ci.dtype)
    r = bench.check_outputs("exact", [_chain_outputs(o), _chain_outputs(o)], o)
    assert r["mismatched_requests"] == 0 and r["calls_checked"] == 2
    assert r["max_abs_dlogprob"] < 1e-6
    assert r["decisions_per_call"] == int(o.decisions.sum())
    assert abs(r["mean_accept_len"] - o.accept_len.mean()) < 1e-12


def test_planted_differences_count_once_each():
    ci = synth.tiny_exact_v32()
    o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, ci.dtype)
    b = _first_unflagged(o)
    n = int(o.accept_len[b])
    for plant in ("token", "length", "logprob"):
        out = _chain_outputs(o)
        if plant == "token":
            out["tok"][b, n] = (out["tok"][b, n] + 1) % ci.V
        elif plant == "length":
            out["ln"][b] = (n + 1) % (ci.K + 1)
        else:
            out["tlp"][b, 0] += 2e-4
        r = bench.check_outputs("exact", [out], o)
        assert r["mismatched_requests"] == 1, plant


def test_greedy_outputs_without_logprobs():
    ci = synth.tiny_exact_v32()
    o = oracle.greedy(ci.target, ci.tokens, ci.dtype)
    r = bench.check_outputs("greedy", [_chain_outputs(o, with_lp=False)], o)
    assert r["mismatched_requests"] == 0


def test_sampler_rows():
    ci = synth.tiny_exact_v32()
    u = np.random.default_rng(5).random(ci.tokens.shape, dtype=np.float32)
    o = oracle.sample(ci.draft, u, ci.dtype)
    out = {"tok": torch.from_numpy(o.tokens.copy()), "lq": torch.from_numpy(o.logq.astype(np.float32)),
           "st": torch.zeros(o.tokens.shape, dtype=torch.int32)}
    assert bench.check_outputs("sample", [out], o)["mismatched_rows"] == 0
    i = np.unravel_index(int(np.flatnonzero(o.flag.ravel() == 0)[0]), o.flag.shape)
    out["tok"][i] = (out["tok"][i] + 1) % ci.V
    assert bench.check_outputs("sample", [out], o)["mismatched_rows"] == 1


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU: --gpus 2 exits with status 2 and a message,
    before touching any device."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=root, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
    assert not r.stdout.strip().startswith("{")  # no benchmark line
