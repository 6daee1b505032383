"""The allocation-free exact call (spec_verify_exact_noalloc) against the
workspace entry point it is a variant of (spec_verify_exact), through the C
ABI: two calls in a row on the same device, the second with a smaller input,
each bit-identical to spec_verify_exact on the same inputs and within the
parity rule of the fp64 oracle.  The second call reuses the static scratch
array the first one filled, so stale contents must not matter; nor may the
words a call that timed out (status 2) left behind."""
import ctypes

import numpy as np
import pytest
import torch

import draft_verification_row_amd as sv
import oracle
import synth
from parity import compare_chain, dev, dev_logits

pytestmark = pytest.mark.gpu


def _noalloc(lib, T, D, x, u, logprobs=True):
    B, L, V = T.shape
    K = L - 1
    tok = torch.full((B, L), -7, dtype=torch.int32, device=T.device)
    ln = torch.full((B,), -7, dtype=torch.int32, device=T.device)
    st = torch.full((B,), -7, dtype=torch.int32, device=T.device)
    tlp = torch.full((B, L), 7.0, dtype=torch.float32, device=T.device) if logprobs else None
    blp = torch.full((B, L), 7.0, dtype=torch.float32, device=T.device) if logprobs else None
    p = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    code = 1 if T.dtype == torch.bfloat16 else 0
    rc = lib.spec_verify_exact_noalloc(p(T), p(D), code, p(x), p(u), B, K, V, p(tok), p(ln),
                                       p(tlp), p(blp), p(st), stream)
    assert rc == 0, lib.spec_status_string(rc)
    return sv.VerifyResult(tok, ln, tlp, blp, st)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_call_twice_then_smaller(dtype):
    lib = sv.load_library()
    shapes = [(32, 5, 128256), (5, 3, 4099)] if dtype == "bf16" else [(8, 5, 40000), (3, 2, 1000)]
    for i, (B, K, V) in enumerate(shapes):
        print(f"no-alloc exact {dtype} call {i}: B={B} K={K} V={V}", flush=True)
        ci = synth.chain_inputs(B, K, V, dtype, seed=900 + i, useed=950 + i)
        T, D = dev_logits(ci.target, dtype), dev_logits(ci.draft, dtype)
        x, u = dev(ci.tokens), dev(ci.uniforms)
        got = _noalloc(lib, T, D, x, u)
        want = sv.spec_verify_exact(T, D, x, u)
        torch.cuda.synchronize()
        for a, b, name in zip(got, want, want._fields):
            assert torch.equal(a, b), f"{name} differs from spec_verify_exact on call {i}"
        o = oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, dtype)
        compare_chain(got, o, what=f"no-alloc exact {dtype} call {i}")
    # without log-probs, after the larger calls
    ci = synth.chain_inputs(2, 4, 3001, dtype, seed=990, useed=991)
    T, D = dev_logits(ci.target, dtype), dev_logits(ci.draft, dtype)
    got = _noalloc(lib, T, D, dev(ci.tokens), dev(ci.uniforms), logprobs=False)
    torch.cuda.synchronize()
    compare_chain(got, oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, dtype),
                  logprobs=False, what="no-alloc exact without log-probs")


def test_noalloc_after_a_timed_out_call():
    """A call at a zero wait bound may leave published words in the shared
    array; the next call at the default bound zeroes what it uses first and
    must equal spec_verify_exact and the oracle."""
    lib = sv.load_library()
    ci = synth.exact_b32_k5()
    T, D = dev_logits(ci.target, "bf16"), dev_logits(ci.draft, "bf16")
    x, u = dev(ci.tokens), dev(ci.uniforms)
    sv.spec_set_spin_limit(0)
    try:
        first = _noalloc(lib, T, D, x, u)
        torch.cuda.synchronize()
    finally:
        sv.spec_set_spin_limit(-1)
    print("requests timed out at a zero bound:", int((first.status == 2).sum()), flush=True)
    got = _noalloc(lib, T, D, x, u)
    want = sv.spec_verify_exact(T, D, x, u)
    torch.cuda.synchronize()
    for a, b, name in zip(got, want, want._fields):
        assert torch.equal(a, b), f"{name} differs from spec_verify_exact after a timed-out call"
    compare_chain(got, oracle.exact(ci.target, ci.draft, ci.tokens, ci.uniforms, "bf16"),
                  what="no-alloc exact after a timed-out call")


def test_noalloc_captured_in_a_graph():
    """The allocation-free call captured into a HIP graph: each replay, with
    eager allocation-free calls on other inputs in between (which leave their
    own words in the shared static array), equals the eager result."""
    lib = sv.load_library()
    ci = synth.exact_b32_k5()
    T, D = dev_logits(ci.target, "bf16"), dev_logits(ci.draft, "bf16")
    x, u = dev(ci.tokens), dev(ci.uniforms)
    eager = [t.clone() for t in _noalloc(lib, T, D, x, u)]
    other = synth.chain_inputs(8, 3, 50000, "bf16", seed=991, useed=992)
    To, Do = dev_logits(other.target, "bf16"), dev_logits(other.draft, "bf16")
    xo, uo = dev(other.tokens), dev(other.uniforms)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        captured = _noalloc(lib, T, D, x, u)
    for rep in range(3):
        print(f"no-alloc graph replay {rep}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        for a, b, name in zip(eager, captured, sv.VerifyResult._fields):
            assert torch.equal(a, b), f"{name} differs on replay {rep}"
        _noalloc(lib, To, Do, xo, uo)  # eager work on the same static array
        torch.cuda.synchronize()


def test_noalloc_rejects_calls_beyond_the_scratch_array():
    lib = sv.load_library()
    T = torch.zeros((1, 6, 16), dtype=torch.bfloat16, device="cuda")
    p = ctypes.c_void_p(T.data_ptr())
    # 4096 requests x 11 rows at V = 128256 need far more than 4 MiB
    rc = lib.spec_verify_exact_noalloc(p, p, 1, p, p, 4096, 5, 128256, p, p, None, None, p, None)
    assert rc == 5  # SPEC_ESCRATCH, nothing enqueued
    assert np.isfinite(float(T.float().sum()))
